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

// NT lanes per row, each lane owning PPL packs: packs t, t + NT, ... so a
// wavefront's loads of one pack index are 1 KiB contiguous.
template <int W, int NT, int PPL>
__global__ __launch_bounds__(NT) void fused_rmsnorm_kernel(
    InTable<W> in, const u32x4 *residual, const u32x4 *weight,
    u32x4 *residual_out, u32x4 *norm_out, int packs_per_row, float n_cols,
    float eps)
{
    constexpr int kWaves = NT / 64;
    const int t = threadIdx.x;
    const int64_t row0 = (int64_t)blockIdx.x * packs_per_row;

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
        }
    }
}

template <int W, int NT, int PPL>
static hipError_t launch_fused_shape(const InTable<W> &in, const void *residual,
                                     const void *weight, void *residual_out,
                                     void *norm_out, int64_t M, int64_t N,
                                     float eps, hipStream_t s)
{
    fused_rmsnorm_kernel<W, NT, PPL><<<dim3((unsigned)M), dim3(NT), 0, s>>>(
        in, static_cast<const u32x4 *>(residual), static_cast<const u32x4 *>(weight),
        static_cast<u32x4 *>(residual_out), static_cast<u32x4 *>(norm_out),
        (int)(N / 8), (float)N, eps);
    return hipGetLastError();
}

// Row shape: up to 64 packs (N <= 512) one wavefront with one pack per lane;
// up to 256 packs (N <= 2048) four wavefronts; beyond that 256 lanes with
// 2..8 packs each (N <= 16384).
template <int W>
static hipError_t launch_fused_w(const void *const *inputs, const void *residual,
                                 const void *weight, void *residual_out,
                                 void *norm_out, int64_t M, int64_t N, float eps,
                                 hipStream_t s)
{
    InTable<W> in;
    for (int r = 0; r < W; ++r)
        in.p[r] = static_cast<const u32x4 *>(inputs[r]);
    const int64_t packs = N / 8;
    if (packs <= 64)
        return launch_fused_shape<W, 64, 1>(in, residual, weight, residual_out, norm_out, M, N, eps, s);
    if (packs <= 256)
        return launch_fused_shape<W, 256, 1>(in, residual, weight, residual_out, norm_out, M, N, eps, s);
    if (packs <= 512)
        return launch_fused_shape<W, 256, 2>(in, residual, weight, residual_out, norm_out, M, N, eps, s);
    if (packs <= 1024)
        return launch_fused_shape<W, 256, 4>(in, residual, weight, residual_out, norm_out, M, N, eps, s);
    return launch_fused_shape<W, 512, 4>(in, residual, weight, residual_out, norm_out, M, N, eps, s);
}

hipError_t launch_fused_rmsnorm(const void *const *inputs, int W,
                                const void *residual, const void *weight,
                                void *residual_out, void *norm_out, int64_t M,
                                int64_t N, float eps, hipStream_t s)
{
    switch (W) {
    case 2: return launch_fused_w<2>(inputs, residual, weight, residual_out, norm_out, M, N, eps, s);
    case 3: return launch_fused_w<3>(inputs, residual, weight, residual_out, norm_out, M, N, eps, s);
    case 4: return launch_fused_w<4>(inputs, residual, weight, residual_out, norm_out, M, N, eps, s);
    case 5: return launch_fused_w<5>(inputs, residual, weight, residual_out, norm_out, M, N, eps, s);
    case 6: return launch_fused_w<6>(inputs, residual, weight, residual_out, norm_out, M, N, eps, s);
    case 7: return launch_fused_w<7>(inputs, residual, weight, residual_out, norm_out, M, N, eps, s);
    case 8: return launch_fused_w<8>(inputs, residual, weight, residual_out, norm_out, M, N, eps, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ar
