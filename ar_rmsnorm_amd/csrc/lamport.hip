// Lamport data-as-flag wire for the fused one-shot: the push (scrub, pack,
// store into every rank's comm buffer) and the sentinel fill.  The reader is
// the Lamport form of the fused kernel (fused_rmsnorm.hip).
//
// Source (web page; cited by tag and section):
//   [TRIAR] "用 Triton + Symmetric Memory 写一个 AllReduce + RMSNorm 融合算子"
//           (riverclouds.net), "Option 2: Lamport"
//
// A u32 word holds two bf16 with element 2j in the low half, which is the
// memory layout of the bf16 row itself, so a pushed slot is the row with
// every -0.0 (0x8000) turned into +0.0: then no word can equal the sentinel
// 0x80008000 that marks "not written yet".  Both kernels are streams of
// 16-byte packs, bound by HBM bandwidth.
#include "device.h"
#include "launch.h"

namespace ar {

constexpr int kLamportThreads = 256;
constexpr uint32_t kSentinel = 0x80008000u;

template <int W>
__global__ __launch_bounds__(kLamportThreads) void lamport_push_kernel(
    const u32x4 *x, int64_t packs, OutTable<W> slots)
{
    const int64_t i = (int64_t)blockIdx.x * kLamportThreads + threadIdx.x;
    if (i >= packs)
        return;
    const u32x4 v = scrub_negative_zero(ld_stream(x + i));
#pragma unroll
    for (int p = 0; p < W; ++p)
        st_stream(slots.p[p] + i, v);
}

// Grid-stride fill: the whole buffer holds three regions, so the grid is
// capped and each lane covers every gridDim.x * threads-th chunk.
__global__ __launch_bounds__(kLamportThreads) void lamport_fill_kernel(u32x4 *comm,
                                                                       int64_t chunks)
{
    const int64_t stride = (int64_t)gridDim.x * kLamportThreads;
    for (int64_t i = (int64_t)blockIdx.x * kLamportThreads + threadIdx.x; i < chunks;
         i += stride)
        st_stream(comm + i, u32x4{kSentinel, kSentinel, kSentinel, kSentinel});
}

hipError_t launch_lamport_fill(void *comm, int64_t chunks, hipStream_t s)
{
    constexpr int64_t kMaxBlocks = 1 << 20;
    int64_t blocks = (chunks + kLamportThreads - 1) / kLamportThreads;
    if (blocks > kMaxBlocks)
        blocks = kMaxBlocks;
    lamport_fill_kernel<<<dim3((unsigned)blocks), kLamportThreads, 0, s>>>(
        static_cast<u32x4 *>(comm), chunks);
    return hipGetLastError();
}

// Slot `rank` of region flag mod 3 in each of the W comm buffers
// (u32 words [3][W][M][N / 2]).
template <int W>
static hipError_t launch_push_w(const void *x, int rank, void *const *comms, int64_t M,
                                int64_t N, uint32_t flag, hipStream_t s)
{
    const int64_t chunks = M * N / 8;
    const int64_t region = flag % 3u;
    OutTable<W> slots;
    for (int p = 0; p < W; ++p)
        slots.p[p] = static_cast<u32x4 *>(comms[p]) + (region * W + rank) * chunks;
    const int64_t blocks = (chunks + kLamportThreads - 1) / kLamportThreads;
    lamport_push_kernel<W><<<dim3((unsigned)blocks), kLamportThreads, 0, s>>>(
        static_cast<const u32x4 *>(x), chunks, slots);
    return hipGetLastError();
}

hipError_t launch_lamport_push(const void *x, int W, int rank, void *const *comms,
                               int64_t M, int64_t N, uint32_t flag, hipStream_t s)
{
    switch (W) {
    case 2: return launch_push_w<2>(x, rank, comms, M, N, flag, s);
    case 3: return launch_push_w<3>(x, rank, comms, M, N, flag, s);
    case 4: return launch_push_w<4>(x, rank, comms, M, N, flag, s);
    case 5: return launch_push_w<5>(x, rank, comms, M, N, flag, s);
    case 6: return launch_push_w<6>(x, rank, comms, M, N, flag, s);
    case 7: return launch_push_w<7>(x, rank, comms, M, N, flag, s);
    case 8: return launch_push_w<8>(x, rank, comms, M, N, flag, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ar
