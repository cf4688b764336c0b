// Fused all-reduce + residual add + RMSNorm over rows of W bf16 rank buffers.
//
// Sources (web pages; cited by tag and section):
//   [TRIAR] "用 Triton + Symmetric Memory 写一个 AllReduce + RMSNorm 融合算子"
//           (riverclouds.net)
//   [SGLv1] "SGLang Custom AllReduce v1 线程模型和工作原理细节" (todaynews.cc)
//
// One workgroup owns one row ([TRIAR] "overall design": the row statistic must
// stay local, so a row is never split across workgroups).  Each lane loads
// its packs of the W inputs, the residual and the weight up front (all loads
// independent and in flight together), forms h in fp32 registers, writes
// residual_out, and contributes sum(h^2) to a DPP wavefront reduction; the
// wavefront sums meet in LDS.  h never leaves registers between the sum and
// the normalisation.  Traffic per row is (W + 3) * N * 2 bytes; a single row
// is latency-bound (one launch, one HBM round trip), many rows stream.
#include "device.h"
#include "launch.h"

namespace ar {

// Lamport data-as-flag reading ([TRIAR] "Option 2: Lamport"): the inputs are
// the W slots of this rank's comm buffer, filled by the ranks' pushes; a
// 16-byte chunk is ready once none of its four words is the sentinel (two
// bf16 -0.0, which a scrubbed push can never write).  After use, the slots
// of the previous call's region are reset to the sentinel.
constexpr uint32_t kLamportSentinel = 0x80008000u;

template <int W>
struct LamportArgs {
    u32x4 *reset[W];       // slot bases of the region to refill with the sentinel
    uint32_t max_spins;    // bound on re-reads of a chunk still holding a sentinel
    uint32_t *bad;         // (slot, chunk) units never ready; NULL: not counted
    // one-launch form only: this rank's rows and slot `rank` of the region in
    // use in every rank's buffer
    const u32x4 *x_self;
    u32x4 *push[W];
    int rank;
};

__device__ __forceinline__ bool has_sentinel(u32x4 v)
{
    return v.x == kLamportSentinel || v.y == kLamportSentinel ||
           v.z == kLamportSentinel || v.w == kLamportSentinel;
}

// NT lanes per row, each lane owning PPL packs: packs t, t + NT, ... so a
// wavefront's loads of one pack index are 1 KiB contiguous.
template <int W, int NT, int PPL, bool LAMPORT, bool PUSH>
__global__ __launch_bounds__(NT) void fused_rmsnorm_kernel(
    InTable<W> in, const u32x4 *residual, const u32x4 *weight,
    u32x4 *residual_out, u32x4 *norm_out, int packs_per_row, float n_cols,
    float eps, LamportArgs<W> la)
{
    constexpr int kWaves = NT / 64;
    const int t = threadIdx.x;
    const int64_t row0 = (int64_t)blockIdx.x * packs_per_row;

    u32x4 xv[PPL][W], rv[PPL], wv[PPL];
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
        const int idx = t + p * NT;
        if (idx < packs_per_row) {
            u32x4 own = {0u, 0u, 0u, 0u};
            if (PUSH) {
                // one-launch Lamport call: push this rank's scrubbed pack to
                // every rank's buffer and keep it for the own slot
                own = scrub_negative_zero(ld_stream(la.x_self + row0 + idx));
#pragma unroll
                for (int q = 0; q < W; ++q)
                    st_stream(la.push[q] + row0 + idx, own);
            }
#pragma unroll
            for (int r = 0; r < W; ++r)
                xv[p][r] = (PUSH && r == la.rank) ? own : in.p[r][row0 + idx];
            rv[p] = residual[row0 + idx];
            wv[p] = weight[idx];
        }
    }
    if (LAMPORT) {
        uint32_t bad = 0;
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
            const int idx = t + p * NT;
            if (idx < packs_per_row) {
#pragma unroll
                for (int r = 0; r < W; ++r) {
                    bool ok = (PUSH && r == la.rank) || !has_sentinel(xv[p][r]);
                    for (uint32_t s = 0; !ok && s < la.max_spins; ++s) {
                        xv[p][r] = reload16(in.p[r] + row0 + idx);
                        ok = !has_sentinel(xv[p][r]);
                    }
                    bad += ok ? 0u : 1u;
                }
            }
        }
        if (bad && la.bad)
            atomicAdd(la.bad, bad);
    }

    // a = sum over ranks in order 0..W-1 starting from rank 0's value, then
    // h = a + residual, all in fp32 ([TRIAR] "what this operator computes";
    // the all-reduce part is [SGLv1]'s one-stage sum).
    float h[PPL][8];
    float ss = 0.0f;
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
        const int idx = t + p * NT;
        if (idx < packs_per_row) {
            float acc[8], tmp[8];
            widen8(xv[p][0], acc);
#pragma unroll
            for (int r = 1; r < W; ++r) {
                widen8(xv[p][r], tmp);
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    acc[k] = acc[k] + tmp[k];
            }
            widen8(rv[p], tmp);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                h[p][k] = acc[k] + tmp[k];
                ss += h[p][k] * h[p][k];
            }
            residual_out[row0 + idx] = narrow8(h[p]);
        }
    }

    // Row sum of h^2: wavefront via DPP, then the kWaves partials via LDS.
    ss = wave_sum(ss);
    if (kWaves > 1) {
        __shared__ float part[kWaves];
        if ((t & 63) == 0)
            part[t >> 6] = ss;
        __syncthreads();
        ss = part[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            ss += part[w];
    }
    const float rms = rsqrtf(ss / n_cols + eps);

#pragma unroll
    for (int p = 0; p < PPL; ++p) {
        const int idx = t + p * NT;
        if (idx < packs_per_row) {
            float wf[8], y[8];
            widen8(wv[p], wf);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                y[k] = (h[p][k] * rms) * wf[k];
            norm_out[row0 + idx] = narrow8(y);
            if (LAMPORT) {
                const u32x4 sent = {kLamportSentinel, kLamportSentinel, kLamportSentinel,
                                    kLamportSentinel};
#pragma unroll
                for (int r = 0; r < W; ++r)
                    st_stream(la.reset[r] + row0 + idx, sent);
            }
        }
    }
}

template <int W, int NT, int PPL, bool LAMPORT, bool PUSH>
static hipError_t launch_fused_shape(const InTable<W> &in, const void *residual,
                                     const void *weight, void *residual_out,
                                     void *norm_out, int64_t M, int64_t N,
                                     float eps, const LamportArgs<W> &la, hipStream_t s)
{
    fused_rmsnorm_kernel<W, NT, PPL, LAMPORT, PUSH><<<dim3((unsigned)M), dim3(NT), 0, s>>>(
        in, static_cast<const u32x4 *>(residual), static_cast<const u32x4 *>(weight),
        static_cast<u32x4 *>(residual_out), static_cast<u32x4 *>(norm_out),
        (int)(N / 8), (float)N, eps, la);
    return hipGetLastError();
}

// Row shape: up to 64 packs (N <= 512) one wavefront with one pack per lane;
// up to 256 packs (N <= 2048) four wavefronts; beyond that 256 or 512 lanes
// with 2..4 packs each (N <= 16384).
template <int W, bool LAMPORT, bool PUSH>
static hipError_t launch_fused_w(const InTable<W> &in, const void *residual,
                                 const void *weight, void *residual_out,
                                 void *norm_out, int64_t M, int64_t N, float eps,
                                 const LamportArgs<W> &la, hipStream_t s)
{
    const int64_t packs = N / 8;
    if (packs <= 64)
        return launch_fused_shape<W, 64, 1, LAMPORT, PUSH>(in, residual, weight, residual_out, norm_out, M, N, eps, la, s);
    if (packs <= 256)
        return launch_fused_shape<W, 256, 1, LAMPORT, PUSH>(in, residual, weight, residual_out, norm_out, M, N, eps, la, s);
    if (packs <= 512)
        return launch_fused_shape<W, 256, 2, LAMPORT, PUSH>(in, residual, weight, residual_out, norm_out, M, N, eps, la, s);
    if (packs <= 1024)
        return launch_fused_shape<W, 256, 4, LAMPORT, PUSH>(in, residual, weight, residual_out, norm_out, M, N, eps, la, s);
    return launch_fused_shape<W, 512, 4, LAMPORT, PUSH>(in, residual, weight, residual_out, norm_out, M, N, eps, la, s);
}

template <int W>
static hipError_t launch_plain_w(const void *const *inputs, const void *residual,
                                 const void *weight, void *residual_out, void *norm_out,
                                 int64_t M, int64_t N, float eps, hipStream_t s)
{
    InTable<W> in;
    for (int r = 0; r < W; ++r)
        in.p[r] = static_cast<const u32x4 *>(inputs[r]);
    LamportArgs<W> la{};
    return launch_fused_w<W, false, false>(in, residual, weight, residual_out, norm_out, M, N, eps,
                                    la, s);
}

// The comm buffer is u32 words [3 regions][W slots][M][N / 2], i.e. each
// slot has the layout of a bf16 [M, N] matrix.
// With x_self (the one-launch call) this rank's rows are also pushed into
// slot `rank` of the region in use of every buffer in `comms`; `comm` is
// then comms[rank].
template <int W>
static hipError_t launch_lamport_w(void *comm, const void *residual, const void *weight,
                                   void *residual_out, void *norm_out, int64_t M, int64_t N,
                                   float eps, uint32_t flag, uint32_t max_spins,
                                   uint32_t *bad, const void *x_self, int rank,
                                   void *const *comms, hipStream_t s)
{
    u32x4 *base = static_cast<u32x4 *>(comm);
    const int64_t chunks = M * N / 8;
    const int64_t use = flag % 3u, reset = (flag + 2u) % 3u;
    InTable<W> in;
    LamportArgs<W> la{};
    for (int r = 0; r < W; ++r) {
        in.p[r] = base + (use * W + r) * chunks;
        la.reset[r] = base + (reset * W + r) * chunks;
    }
    la.max_spins = max_spins;
    la.bad = bad;
    if (!x_self)
        return launch_fused_w<W, true, false>(in, residual, weight, residual_out, norm_out, M,
                                              N, eps, la, s);
    la.x_self = static_cast<const u32x4 *>(x_self);
    la.rank = rank;
    for (int q = 0; q < W; ++q)
        la.push[q] = static_cast<u32x4 *>(comms[q]) + (use * W + rank) * chunks;
    return launch_fused_w<W, true, true>(in, residual, weight, residual_out, norm_out, M, N,
                                         eps, la, s);
}

hipError_t launch_fused_rmsnorm(const void *const *inputs, int W,
                                const void *residual, const void *weight,
                                void *residual_out, void *norm_out, int64_t M,
                                int64_t N, float eps, hipStream_t s)
{
    switch (W) {
    case 2: return launch_plain_w<2>(inputs, residual, weight, residual_out, norm_out, M, N, eps, s);
    case 3: return launch_plain_w<3>(inputs, residual, weight, residual_out, norm_out, M, N, eps, s);
    case 4: return launch_plain_w<4>(inputs, residual, weight, residual_out, norm_out, M, N, eps, s);
    case 5: return launch_plain_w<5>(inputs, residual, weight, residual_out, norm_out, M, N, eps, s);
    case 6: return launch_plain_w<6>(inputs, residual, weight, residual_out, norm_out, M, N, eps, s);
    case 7: return launch_plain_w<7>(inputs, residual, weight, residual_out, norm_out, M, N, eps, s);
    case 8: return launch_plain_w<8>(inputs, residual, weight, residual_out, norm_out, M, N, eps, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_lamport_fused(void *comm, int W, const void *residual,
                                const void *weight, void *residual_out, void *norm_out,
                                int64_t M, int64_t N, float eps, uint32_t flag,
                                uint32_t max_spins, uint32_t *bad, const void *x_self,
                                int rank, void *const *comms, hipStream_t s)
{
    switch (W) {
#define AR_LAMPORT_CASE(w)                                                              \
    case w:                                                                             \
        return launch_lamport_w<w>(comm, residual, weight, residual_out, norm_out, M, N, \
                                   eps, flag, max_spins, bad, x_self, rank, comms, s);
    AR_LAMPORT_CASE(2)
    AR_LAMPORT_CASE(3)
    AR_LAMPORT_CASE(4)
    AR_LAMPORT_CASE(5)
    AR_LAMPORT_CASE(6)
    AR_LAMPORT_CASE(7)
    AR_LAMPORT_CASE(8)
#undef AR_LAMPORT_CASE
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ar
