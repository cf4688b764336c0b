// Device-side building blocks shared by the libar kernels (gfx950 only).
//
// Sources (web pages; cited by tag and section):
//   [SGLv1] "SGLang Custom AllReduce v1 线程模型和工作原理细节" (todaynews.cc)
//   [JITAR] "0-custom-all-reduce" (obnotes-4iw.pages.dev, sglang jit_kernel)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ar {

// 16 bytes = one "pack" of 8 bf16 or 4 fp32: the unit every lane moves with
// one dwordx4 load or store ([SGLv1] "thread model: 16 bytes per unit";
// [JITAR] section 1).  The _a4/_a8 forms only promise 4/8-byte alignment;
// gfx950 global memory accepts dwordx4 at dword alignment.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4_a8 __attribute__((ext_vector_type(4), aligned(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Streaming accesses for data touched exactly once per launch (the rank
// buffers, staging shards, wire FIFOs and outputs): the nontemporal hint
// sets the nt cache policy on gfx950 so these streams do not displace other
// lines in L2 / Infinity Cache and their writes drain during the kernel
// rather than at its end.
__device__ __forceinline__ u32x4 ld_stream(const u32x4 *p)
{
    return __builtin_nontemporal_load(p);
}
__device__ __forceinline__ void st_stream(u32x4 *p, u32x4 v)
{
    __builtin_nontemporal_store(v, p);
}
// Forms for addresses that are only 4-byte aligned (fp32 payloads): the cast
// to the aligned(4) vector types keeps that alignment visible to the compiler.
__device__ __forceinline__ u32x4 ld4_stream_a4(const uint32_t *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_a4 *>(p));
}
__device__ __forceinline__ u32x2 ld2_stream_a4(const uint32_t *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2_a4 *>(p));
}
__device__ __forceinline__ void st4_stream_a4(uint32_t *p, u32x4 v)
{
    __builtin_nontemporal_store(u32x4_a4(v), reinterpret_cast<u32x4_a4 *>(p));
}
__device__ __forceinline__ void st2_stream_a4(uint32_t *p, u32x2 v)
{
    __builtin_nontemporal_store(u32x2_a4(v), reinterpret_cast<u32x2_a4 *>(p));
}

// Lamport push: clear every bf16 half equal to -0.0 (0x8000), so that no
// u32 word of two bf16 can equal the sentinel 0x80008000.
__device__ __forceinline__ u32x4 scrub_negative_zero(u32x4 v)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t w = v[k];
        const uint32_t lo = (w & 0xFFFFu) == 0x8000u ? 0xFFFFu : 0u;
        const uint32_t hi = (w & 0xFFFF0000u) == 0x80000000u ? 0xFFFF0000u : 0u;
        v[k] = w & ~(lo | hi);
    }
    return v;
}

// Re-read one 16-byte chunk past the caches (a real load on every spin of a
// bounded flag wait).
__device__ __forceinline__ u32x4 reload16(const u32x4 *p)
{
    return *reinterpret_cast<const volatile u32x4 *>(p);
}

// System-coherent (sc0 sc1) load of 16-byte chunk idx of a row of `count`
// chunks whose base is the same for the whole workgroup (the buffer
// descriptor lives in scalar registers).  Unlike a volatile access, which on
// gfx950 waits for its own completion, several of these can be in flight at
// once; a poll loop needs a compiler barrier per spin so that it reloads.
__device__ __forceinline__ u32x4 load16_coherent(const u32x4 *row, int idx, int count)
{
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4 *>(row), 0, count * 16, 0x00020000 /* 32-bit data format */);
    return __builtin_amdgcn_raw_buffer_load_b128(r, idx * 16, 0, 1 | 16 /* sc0 | sc1 */);
}

// System-coherent (sc0 sc1) store of 16-byte chunk idx of a row of `count`
// chunks: acknowledged only once visible to every XCD, so a reader in
// another workgroup of the same launch (possibly on another XCD, whose L2 is
// not coherent with the writer's) sees it with system-coherent loads.
__device__ __forceinline__ void store16_coherent(u32x4 *row, int idx, int count, u32x4 v)
{
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        row, 0, count * 16, 0x00020000 /* 32-bit data format */);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, idx * 16, 0, 1 | 16 /* sc0 | sc1 */);
}

// Kernel-argument pointer tables, passed by value so no device-side
// indirection is needed (the W pointers land in SGPRs).
template <int W>
struct InTable {
    const u32x4 *p[W];
};
template <int W>
struct OutTable {
    u32x4 *p[W];
};

// bf16 -> fp32 is exact: the bf16 bits are the upper half of the fp32.
// Element 2k of a pack is the low half of dword k (little-endian).
__device__ __forceinline__ void widen8(u32x4 v, float f[8])
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f[2 * k] = __uint_as_float(v[k] << 16);
        f[2 * k + 1] = __uint_as_float(v[k] & 0xFFFF0000u);
    }
}

// fp32 pair -> bf16 pair with gfx950's v_cvt_pk_bf16_f32: one rounding to
// nearest, ties to even (the default rounding mode), denormals kept.
__device__ __forceinline__ uint32_t narrow2(float lo, float hi)
{
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ u32x4 narrow8(const float f[8])
{
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        r[k] = narrow2(f[2 * k], f[2 * k + 1]);
    return r;
}

// Sum over the 64 lanes of a wavefront with DPP moves, result in every lane.
// quad_perm swaps (xor 1, xor 2) and row rotations (4, 8) leave each row of
// 16 lanes holding its row sum; row_bcast:15 and row_bcast:31 then fold the
// four rows into lane 63, which readlane broadcasts.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_mov(float v)
{
    // Lanes of rows outside ROW_MASK receive 0 (the "old" operand).
    return __int_as_float(__builtin_amdgcn_update_dpp(
        0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_mov<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v += dpp_mov<0x124, 0xF>(v);  // row_ror:4
    v += dpp_mov<0x128, 0xF>(v);  // row_ror:8
    v += dpp_mov<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_mov<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

}  // namespace ar
