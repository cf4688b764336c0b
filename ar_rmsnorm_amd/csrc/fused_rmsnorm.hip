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
// bf16 -0.0, which a scrubbed push can never write).  Each call also resets
// the slots of the previous call's region to the sentinel; that region is
// neither read nor pushed to by the call, so the reset goes out together
// with the first loads.
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

// One row's arithmetic, shared by the one-shot and two-shot kernels.
// a = sum over the W inputs in table order starting from the first one's
// value, then h = a + residual, all in fp32 ([TRIAR] "what this operator
// computes"; the all-reduce part is [SGLv1]'s one-stage sum).  Returns the
// lane's sum of h^2; lanes past the row's end hold no packs and return 0.
template <int W, int NT, int PPL>
__device__ __forceinline__ float sum_residual(const u32x4 (&xv)[PPL][W], const u32x4 (&rv)[PPL],
                                              int t, int packs_per_row, float (&h)[PPL][8])
{
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
        }
    }
    return ss;
}

// Sum of the lanes' partials over the workgroup: DPP within each wavefront,
// then the wavefront sums through LDS.  Every lane gets the result.
template <int NT>
__device__ __forceinline__ float row_sum(float ss)
{
    constexpr int kWaves = NT / 64;
    ss = wave_sum(ss);
    if (kWaves > 1) {
        __shared__ float part[kWaves];
        if ((threadIdx.x & 63) == 0)
            part[threadIdx.x >> 6] = ss;
        __syncthreads();
        ss = part[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            ss += part[w];
    }
    return ss;
}

// (h * rms) * weight, rounded once to bf16.
__device__ __forceinline__ u32x4 normalize8(const float (&h)[8], float rms, u32x4 w)
{
    float wf[8], y[8];
    widen8(w, wf);
#pragma unroll
    for (int k = 0; k < 8; ++k)
        y[k] = (h[k] * rms) * wf[k];
    return narrow8(y);
}

// One row for one workgroup.  NT lanes per row, each lane owning PPL packs:
// packs t, t + NT, ... so a wavefront's loads of one pack index are 1 KiB
// contiguous.
// With COHERENT_PUSH the push stores are system-coherent, for readers in
// the same launch; otherwise they stream, for readers in later launches.
template <int W, int NT, int PPL, bool LAMPORT, bool PUSH, bool COHERENT_PUSH = false>
__device__ __forceinline__ void fused_row(
    const InTable<W> &in, const u32x4 *residual, const u32x4 *weight,
    u32x4 *residual_out, u32x4 *norm_out, int packs_per_row, float n_cols,
    float eps, const LamportArgs<W> &la, int64_t row)
{
    const int t = threadIdx.x;
    const int64_t row0 = row * packs_per_row;

    // Every load of the row is issued before any store, so the one-launch
    // call's push (which needs its own pack first) does not delay the reads
    // of the peer slots; those are slots other than `rank` of this rank's
    // buffer, never a push target.
    u32x4 xv[PPL][W], rv[PPL], wv[PPL], own[PPL];
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
        const int idx = t + p * NT;
        own[p] = u32x4{0u, 0u, 0u, 0u};
        if (idx < packs_per_row) {
            if (PUSH)
                own[p] = ld_stream(la.x_self + row0 + idx);
#pragma unroll
            for (int r = 0; r < W; ++r)
                xv[p][r] = (PUSH && r == la.rank) ? u32x4{0u, 0u, 0u, 0u} : in.p[r][row0 + idx];
            rv[p] = residual[row0 + idx];
            wv[p] = weight[idx];
        }
    }
    if (PUSH) {
        // one-launch Lamport call: push this rank's scrubbed packs to every
        // rank's buffer and keep them for the own slot
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
            const int idx = t + p * NT;
            if (idx < packs_per_row) {
                own[p] = scrub_negative_zero(own[p]);
#pragma unroll
                for (int q = 0; q < W; ++q) {
                    if (COHERENT_PUSH)
                        store16_coherent(la.push[q] + row0, idx, packs_per_row, own[p]);
                    else
                        st_stream(la.push[q] + row0 + idx, own[p]);
                }
#pragma unroll
                for (int r = 0; r < W; ++r)
                    if (r == la.rank)
                        xv[p][r] = own[p];
            }
        }
    }
    if (LAMPORT) {
        // the previous call's region is neither read nor pushed to by this
        // call, so its sentinel goes out now, while the loads are in flight
        const u32x4 sent = {kLamportSentinel, kLamportSentinel, kLamportSentinel,
                            kLamportSentinel};
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
            const int idx = t + p * NT;
            if (idx < packs_per_row) {
#pragma unroll
                for (int r = 0; r < W; ++r)
                    st_stream(la.reset[r] + row0 + idx, sent);
            }
        }
        // Chunks that still hold the sentinel are re-read, all of a lane's
        // together, with system-coherent loads, a bounded number of times.
        // The own slot of the one-launch form holds the scrubbed push, which
        // is never the sentinel.
        auto missing = [&](int p, int r) {
            return t + p * NT < packs_per_row && has_sentinel(xv[p][r]);
        };
        bool all = true;
#pragma unroll
        for (int p = 0; p < PPL; ++p)
#pragma unroll
            for (int r = 0; r < W; ++r)
                all = all && !missing(p, r);
        if (!all) {
            for (uint32_t s = 0; s < la.max_spins; ++s) {
                asm volatile("" ::: "memory");   // reload on every spin
#pragma unroll
                for (int p = 0; p < PPL; ++p)
#pragma unroll
                    for (int r = 0; r < W; ++r)
                        if (missing(p, r))
                            xv[p][r] = load16_coherent(in.p[r] + row0, t + p * NT,
                                                       packs_per_row);
                all = true;
#pragma unroll
                for (int p = 0; p < PPL; ++p)
#pragma unroll
                    for (int r = 0; r < W; ++r)
                        all = all && !missing(p, r);
                if (all)
                    break;
            }
            uint32_t bad = 0;
#pragma unroll
            for (int p = 0; p < PPL; ++p)
#pragma unroll
                for (int r = 0; r < W; ++r)
                    bad += missing(p, r) ? 1u : 0u;
            if (bad && la.bad)
                atomicAdd(la.bad, bad);
        }
    }

    float h[PPL][8];
    const float ss = sum_residual<W, NT, PPL>(xv, rv, t, packs_per_row, h);
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
        const int idx = t + p * NT;
        if (idx < packs_per_row)
            residual_out[row0 + idx] = narrow8(h[p]);
    }
    const float rms = rsqrtf(row_sum<NT>(ss) / n_cols + eps);

#pragma unroll
    for (int p = 0; p < PPL; ++p) {
        const int idx = t + p * NT;
        if (idx < packs_per_row) {
            norm_out[row0 + idx] = normalize8(h[p], rms, wv[p]);
        }
    }
}

// One workgroup per row.
template <int W, int NT, int PPL, bool LAMPORT, bool PUSH>
__global__ __launch_bounds__(NT) void fused_rmsnorm_kernel(
    InTable<W> in, const u32x4 *residual, const u32x4 *weight,
    u32x4 *residual_out, u32x4 *norm_out, int packs_per_row, float n_cols,
    float eps, LamportArgs<W> la)
{
    fused_row<W, NT, PPL, LAMPORT, PUSH>(in, residual, weight, residual_out, norm_out,
                                         packs_per_row, n_cols, eps, la, blockIdx.x);
}

// The Lamport exchange of all W ranks in one launch, as W GPUs run it at the
// same time ([TRIAR] "Option 2: Lamport"): workgroup (row m, rank r) runs
// rank r's one-launch program on row m -- push row m of x[r] into slot r of
// the region in use of every comm buffer, wait for the W - 1 peer slots of
// row m in comm[r], reduce, add the residual, normalise into rank r's
// outputs, and reset row m of the previous region of comm[r].  The peers'
// pushes land while the reader polls, so the re-read path runs.  The
// workgroups of one row sit on different XCDs, whose L2 caches are not
// coherent with each other inside a launch, so the pushes are
// system-coherent stores and the re-reads system-coherent loads.  Every
// workgroup of the launch is resident at once (checked by the host), so
// every push is made and every wait ends.
template <int W>
struct LamportAllArgs {
    const u32x4 *x[W];            // rank r's rows
    u32x4 *comm[W];               // rank r's comm buffer
    u32x4 *residual_out[W];
    u32x4 *norm_out[W];
    int64_t chunks;               // 16-byte chunks of one slot (M * N / 8)
    int use, reset;               // regions of this call and of the previous one
    uint32_t max_spins;
    uint32_t *bad;
};

template <int W, int NT, int PPL>
__global__ __launch_bounds__(NT) void lamport_all_ranks_kernel(
    const u32x4 *residual, const u32x4 *weight, int packs_per_row, float n_cols, float eps,
    LamportAllArgs<W> a)
{
    const int rank = blockIdx.y;
    InTable<W> in;
    LamportArgs<W> la;
#pragma unroll
    for (int r = 0; r < W; ++r) {
        in.p[r] = a.comm[rank] + ((int64_t)a.use * W + r) * a.chunks;
        la.reset[r] = a.comm[rank] + ((int64_t)a.reset * W + r) * a.chunks;
        la.push[r] = a.comm[r] + ((int64_t)a.use * W + rank) * a.chunks;
    }
    la.max_spins = a.max_spins;
    la.bad = a.bad;
    la.x_self = a.x[rank];
    la.rank = rank;
    fused_row<W, NT, PPL, true, true, true>(in, residual, weight, a.residual_out[rank],
                                            a.norm_out[rank], packs_per_row, n_cols, eps, la,
                                            blockIdx.x);
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

// Row shape: one pack per lane up to 1,024 packs (N <= 8192): one wavefront
// up to N = 512, then 256, 512 or 1,024 lanes; two packs per lane on 1,024
// lanes beyond (N <= 16384).  More lanes per row measured faster than more
// packs per lane from N = 4096 on: 2.58 -> 2.21 us at M = 1, N = 4096 and
// 26.4 -> 24.0 us at M = 1024, N = 8192 against 256 lanes with 2 or 4 packs.
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
        return launch_fused_shape<W, 512, 1, LAMPORT, PUSH>(in, residual, weight, residual_out, norm_out, M, N, eps, la, s);
    if (packs <= 1024)
        return launch_fused_shape<W, 1024, 1, LAMPORT, PUSH>(in, residual, weight, residual_out, norm_out, M, N, eps, la, s);
    return launch_fused_shape<W, 1024, 2, LAMPORT, PUSH>(in, residual, weight, residual_out, norm_out, M, N, eps, la, s);
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
    // the region of this call and the one before it (the caller keeps flag
    // below a multiple of 3, so the sequence of regions never repeats one)
    const int64_t use = flag % 3u, reset = (use + 2) % 3;
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

template <int W, int NT, int PPL>
static hipError_t launch_all_ranks_shape(const void *const *xs, void *const *comms,
                                         const void *residual, const void *weight,
                                         void *const *residual_outs, void *const *norm_outs,
                                         int64_t M, int64_t N, float eps, uint32_t flag,
                                         uint32_t max_spins, uint32_t *bad, bool check_only,
                                         int *resident, hipStream_t s)
{
    const void *fn = reinterpret_cast<const void *>(&lamport_all_ranks_kernel<W, NT, PPL>);
    if (check_only) {
        int dev = 0, cus = 0, per_cu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess)
            e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NT, 0);
        *resident = e == hipSuccess ? cus * per_cu : 0;
        return e;
    }
    LamportAllArgs<W> a{};
    for (int r = 0; r < W; ++r) {
        a.x[r] = static_cast<const u32x4 *>(xs[r]);
        a.comm[r] = static_cast<u32x4 *>(comms[r]);
        a.residual_out[r] = static_cast<u32x4 *>(residual_outs[r]);
        a.norm_out[r] = static_cast<u32x4 *>(norm_outs[r]);
    }
    a.chunks = M * N / 8;
    a.use = (int)(flag % 3u);
    a.reset = (a.use + 2) % 3;
    a.max_spins = max_spins;
    a.bad = bad;
    lamport_all_ranks_kernel<W, NT, PPL><<<dim3((unsigned)M, (unsigned)W), dim3(NT), 0, s>>>(
        static_cast<const u32x4 *>(residual), static_cast<const u32x4 *>(weight), (int)(N / 8),
        (float)N, eps, a);
    return hipGetLastError();
}

template <int W>
static hipError_t launch_all_ranks_w(const void *const *xs, void *const *comms,
                                     const void *residual, const void *weight,
                                     void *const *residual_outs, void *const *norm_outs,
                                     int64_t M, int64_t N, float eps, uint32_t flag,
                                     uint32_t max_spins, uint32_t *bad, bool check_only,
                                     int *resident, hipStream_t s)
{
    const int64_t packs = N / 8;
#define AR_ALL_RANKS(NT, PPL)                                                             \
    return launch_all_ranks_shape<W, NT, PPL>(xs, comms, residual, weight, residual_outs, \
                                              norm_outs, M, N, eps, flag, max_spins, bad,  \
                                              check_only, resident, s)
    if (packs <= 64)
        AR_ALL_RANKS(64, 1);
    if (packs <= 256)
        AR_ALL_RANKS(256, 1);
    if (packs <= 512)
        AR_ALL_RANKS(512, 1);
    if (packs <= 1024)
        AR_ALL_RANKS(1024, 1);
    AR_ALL_RANKS(1024, 2);
#undef AR_ALL_RANKS
}

hipError_t launch_lamport_all_ranks(const void *const *xs, void *const *comms, int W,
                                    const void *residual, const void *weight,
                                    void *const *residual_outs, void *const *norm_outs,
                                    int64_t M, int64_t N, float eps, uint32_t flag,
                                    uint32_t max_spins, uint32_t *bad, bool check_only,
                                    int *resident, hipStream_t s)
{
    switch (W) {
#define AR_ALL_CASE(w)                                                                     \
    case w:                                                                                \
        return launch_all_ranks_w<w>(xs, comms, residual, weight, residual_outs, norm_outs, \
                                     M, N, eps, flag, max_spins, bad, check_only, resident, s);
    AR_ALL_CASE(2)
    AR_ALL_CASE(3)
    AR_ALL_CASE(4)
    AR_ALL_CASE(5)
    AR_ALL_CASE(6)
    AR_ALL_CASE(7)
    AR_ALL_CASE(8)
#undef AR_ALL_CASE
    default: return hipErrorInvalidValue;
    }
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

// Two-shot fused form, as run by one rank: [SGLv1]'s two-stage structure on
// rows.  part = M / W rows per shard, the last shard also taking the
// remainder; tmps[s] stages shard s as residual_out rows followed by norm_out
// rows ([2][part + rem][N] bf16).  One-dimensional grid:
//   blocks [0, rs_rows) (RS): one row of this rank's shard each, inputs in
//       `in` order (the owner's rotation); both outputs go to tmps[rank] and,
//       with AG, straight to residual_out / norm_out (each workgroup gathers
//       the rows it computed, so no barrier is needed inside the launch);
//   the remaining blocks (AG): part + rem per shard, copying row j of shard
//       g = (rank + i) mod W from tmps[g], for i = 1..W-1 after an RS, or
//       i = 0..W-1 for a gather alone.
template <int W, int NT, int PPL, bool RS, bool AG>
__global__ __launch_bounds__(NT) void fused_2stage_kernel(
    InTable<W> in, const u32x4 *residual, const u32x4 *weight, u32x4 *residual_out,
    u32x4 *norm_out, OutTable<W> tmps, int rank, int64_t part, int64_t rem,
    int packs_per_row, float n_cols, float eps, uint32_t rs_rows)
{
    const uint32_t b = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t cap = part + rem;
    const int64_t packs = packs_per_row;
    if (RS && b < rs_rows) {
        const int64_t row0 = ((int64_t)rank * part + b) * packs;
        u32x4 *stage_res = tmps.p[rank] + (int64_t)b * packs;
        u32x4 *stage_norm = tmps.p[rank] + (cap + b) * packs;
        u32x4 xv[PPL][W], rv[PPL], wv[PPL];
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
            const int idx = t + p * NT;
            if (idx < packs_per_row) {
#pragma unroll
                for (int r = 0; r < W; ++r)
                    xv[p][r] = in.p[r][row0 + idx];
                rv[p] = residual[row0 + idx];
                wv[p] = weight[idx];
            }
        }
        float h[PPL][8];
        const float ss = sum_residual<W, NT, PPL>(xv, rv, t, packs_per_row, h);
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
            const int idx = t + p * NT;
            if (idx < packs_per_row) {
                const u32x4 ro = narrow8(h[p]);
                st_stream(stage_res + idx, ro);
                if (AG)
                    st_stream(residual_out + row0 + idx, ro);
            }
        }
        const float rms = rsqrtf(row_sum<NT>(ss) / n_cols + eps);
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
            const int idx = t + p * NT;
            if (idx < packs_per_row) {
                const u32x4 no = normalize8(h[p], rms, wv[p]);
                st_stream(stage_norm + idx, no);
                if (AG)
                    st_stream(norm_out + row0 + idx, no);
            }
        }
        return;
    }
    if (!AG)
        return;
    const uint32_t k = RS ? b - rs_rows : b;
    const int i = (RS ? 1 : 0) + (int)(k / cap);
    const int64_t j = k % cap;
    int g = rank + i;
    if (g >= W)
        g -= W;
    const int64_t rows_g = part + (g == W - 1 ? rem : 0);
    if (j >= rows_g)
        return;
    const int64_t row0 = ((int64_t)g * part + j) * packs;
    const u32x4 *src_res = tmps.p[g] + j * packs;
    const u32x4 *src_norm = tmps.p[g] + (cap + j) * packs;
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
        const int idx = t + p * NT;
        if (idx < packs_per_row) {
            st_stream(residual_out + row0 + idx, src_res[idx]);
            st_stream(norm_out + row0 + idx, src_norm[idx]);
        }
    }
}

template <int W, int NT, int PPL, bool RS, bool AG>
static hipError_t launch_2stage_shape(const InTable<W> &in, const OutTable<W> &tmps,
                                      int rank, const void *residual, const void *weight,
                                      void *residual_out, void *norm_out, int64_t M,
                                      int64_t N, float eps, hipStream_t s)
{
    const int64_t part = M / W, rem = M % W, cap = part + rem;
    const int64_t rs_rows = RS ? part + (rank == W - 1 ? rem : 0) : 0;
    const int64_t blocks = rs_rows + (AG ? (RS ? W - 1 : W) * cap : 0);
    if (blocks == 0)
        return hipSuccess;
    fused_2stage_kernel<W, NT, PPL, RS, AG><<<dim3((unsigned)blocks), dim3(NT), 0, s>>>(
        in, static_cast<const u32x4 *>(residual), static_cast<const u32x4 *>(weight),
        static_cast<u32x4 *>(residual_out), static_cast<u32x4 *>(norm_out), tmps, rank, part,
        rem, (int)(N / 8), (float)N, eps, (uint32_t)rs_rows);
    return hipGetLastError();
}

template <int W, bool RS, bool AG>
static hipError_t launch_2stage_mode(const InTable<W> &in, const OutTable<W> &tmps, int rank,
                                     const void *residual, const void *weight,
                                     void *residual_out, void *norm_out, int64_t M, int64_t N,
                                     float eps, hipStream_t s)
{
    const int64_t packs = N / 8;
#define AR_2SHOT(NT, PPL)                                                                   \
    return launch_2stage_shape<W, NT, PPL, RS, AG>(in, tmps, rank, residual, weight,        \
                                                   residual_out, norm_out, M, N, eps, s)
    if (packs <= 64)
        AR_2SHOT(64, 1);
    if (packs <= 256)
        AR_2SHOT(256, 1);
    if (packs <= 512)
        AR_2SHOT(512, 1);
    if (packs <= 1024)
        AR_2SHOT(1024, 1);
    AR_2SHOT(1024, 2);
#undef AR_2SHOT
}

template <int W>
static hipError_t launch_2stage_w(const void *const *inputs, const int *order,
                                  void *const *tmps, int rank, const void *residual,
                                  const void *weight, void *residual_out, void *norm_out,
                                  int64_t M, int64_t N, float eps, bool rs, bool ag,
                                  hipStream_t s)
{
    InTable<W> in;
    OutTable<W> tp;
    for (int r = 0; r < W; ++r) {
        in.p[r] = static_cast<const u32x4 *>(inputs[order[r]]);
        tp.p[r] = static_cast<u32x4 *>(tmps[r]);
    }
    if (rs && ag)
        return launch_2stage_mode<W, true, true>(in, tp, rank, residual, weight, residual_out,
                                                 norm_out, M, N, eps, s);
    if (rs)
        return launch_2stage_mode<W, true, false>(in, tp, rank, residual, weight, residual_out,
                                                  norm_out, M, N, eps, s);
    return launch_2stage_mode<W, false, true>(in, tp, rank, residual, weight, residual_out,
                                              norm_out, M, N, eps, s);
}

hipError_t launch_fused_2stage(const void *const *inputs, const int *order,
                               void *const *tmps, int W, int rank, const void *residual,
                               const void *weight, void *residual_out, void *norm_out,
                               int64_t M, int64_t N, float eps, bool rs, bool ag, hipStream_t s)
{
    switch (W) {
#define AR_2SHOT_CASE(w)                                                                  \
    case w:                                                                               \
        return launch_2stage_w<w>(inputs, order, tmps, rank, residual, weight, residual_out, \
                                  norm_out, M, N, eps, rs, ag, s);
    AR_2SHOT_CASE(2)
    AR_2SHOT_CASE(3)
    AR_2SHOT_CASE(4)
    AR_2SHOT_CASE(5)
    AR_2SHOT_CASE(6)
    AR_2SHOT_CASE(7)
    AR_2SHOT_CASE(8)
#undef AR_2SHOT_CASE
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ar
