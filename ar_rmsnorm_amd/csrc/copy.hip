// Plain 16-byte copy: the achievable-copy reference the measurements put
// beside the reduce and wire kernels.  It is not an operation of the method;
// it shows what a kernel that only reads and writes each byte once reaches
// on this device, with the same access pattern as the reduce kernels (one
// dwordx4 nontemporal load and store per lane, 256 lanes per workgroup, one
// workgroup per 4 KiB, so large copies launch many thousands of workgroups
// across the 256 CUs).
#include "device.h"
#include "launch.h"

namespace ar {

constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void copy_kernel(const u32x4 *src, u32x4 *dst,
                                                           int64_t packs)
{
    const int64_t i = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x;
    if (i < packs)
        st_stream(dst + i, ld_stream(src + i));
}

hipError_t launch_copy(const void *src, void *dst, int64_t packs, hipStream_t s)
{
    const int64_t blocks = (packs + kCopyThreads - 1) / kCopyThreads;
    copy_kernel<<<dim3((unsigned)blocks), dim3(kCopyThreads), 0, s>>>(
        static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), packs);
    return hipGetLastError();
}

}  // namespace ar
