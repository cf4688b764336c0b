// LL and LL128 wire formats: encode a fp32 payload into a FIFO of flagged
// lines, and decode + reduce W such FIFOs with flag validation.
//
// Source (web page; cited by tag and section):
//   [NCCL14] "NCCL 专家课程 14：Simple、LL、LL128 的线格式、同步与真实性能边界"
//            (blog.cptz.space)
//
// Geometry ([NCCL14] "prerequisite mental model", "how LL publishes and waits
// for flags"): a FIFO is a ring of 8 steps of step_lines lines; line i of a
// call belongs to step k = first_step + i / step_lines, sits at line
// (k mod 8) * step_lines + i mod step_lines, and is ready when its flag
// equals k + 1.
//
// All four kernels are streams (LL moves 16 wire bytes per 8 payload bytes,
// LL128 128 per 120), so they are bound by HBM bandwidth.  Every lane moves
// 16-byte chunks: LL gives a lane one whole line; the LL128 decoder gives
// eight lanes one 128-byte line, lane 7 of each group holding the line's last
// payload word and its flag word (the flag-lane arrangement of [NCCL14]
// "LL128's warp-level ready check"); the LL128 encoder gives sixteen lanes
// two lines so that its payload loads stay 16-byte aligned.  Where payload
// addresses are only 4- or 8-byte aligned (the decoder's 120-byte output
// spans, sources at a 4/8/12-byte offset) gfx950's dwordx4 accesses at dword
// alignment are used directly; no staging through LDS is needed
// ([NCCL14] "why LL128 alignment matters" stages misaligned sources through
// shared memory on its hardware).
#include "device.h"
#include "launch.h"

namespace ar {

constexpr int kWireThreads = 256;

// Write-through stores (sc0 sc1): the line goes to memory with the store, so
// the kernel ends with no dirty L2 lines of it to write back.  Measured per
// kernel against the nontemporal stores, 16 Mi values, W=4: the LL decoder's
// output stores gain (98.1 -> 94.4 us from cold HBM); the LL128 encoder's
// FIFO stores gain when its source is still in the Infinity Cache (23.4 ->
// 19.5 us) and are even from cold HBM (23.7 -> 23.3 us).  The LL128 decoder
// (58 -> 62 us), the reduce kernels and the LL encoder lose or do not gain,
// so they keep nontemporal stores.  These are the last memory operations of
// their kernels, so nothing waits on them inside the kernel.
__device__ __forceinline__ void st16_through(u32x4 *p, u32x4 v)
{
    asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void st8_through(uint32_t *p, u32x2 v)
{
    asm volatile("global_store_dwordx2 %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
}
// The LL decoder runs 128-lane workgroups: against 256 lanes, 95.9 instead of
// 101 us for W=4 FIFOs of 16 Mi values in separate allocations, 1% faster
// with the FIFOs carved from one allocation; 64 and 512 lanes no better.
constexpr int kLLDecodeThreads = 128;

struct StepPos {
    uint64_t step;   // k
    uint64_t line;   // position in the FIFO, in lines
};

__device__ __forceinline__ StepPos step_pos(uint32_t i, uint32_t step_lines,
                                            uint64_t first_step)
{
    const uint32_t q = i / step_lines;
    const uint32_t r = i - q * step_lines;
    const uint64_t k = first_step + q;
    return {k, (k & 7u) * (uint64_t)step_lines + r};
}

// ---------------------------------------------------------------------------
// LL ([NCCL14] "LL's 16-byte FIFO line"): {data lo32, flag, data hi32, flag}
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kWireThreads) void ll_pack_kernel(
    const uint32_t *src, int64_t n, u32x4 *fifo, uint32_t lines,
    uint32_t step_lines, uint64_t first_step)
{
    const uint32_t i = blockIdx.x * kWireThreads + threadIdx.x;
    if (i >= lines)
        return;
    const int64_t e = 2 * (int64_t)i;
    uint32_t lo, hi;
    if (e + 1 < n) {
        // a plain load: measured faster than a streaming one for these
        // 8-byte source reads, while the 16-byte FIFO stores stream
        const u32x2 d = *reinterpret_cast<const u32x2_a4 *>(src + e);
        lo = d.x;
        hi = d.y;
    } else {           // last line of an odd count: zero padding
        lo = src[e];
        hi = 0;
    }
    const StepPos sp = step_pos(i, step_lines, first_step);
    const uint32_t flag = (uint32_t)(sp.step + 1);
    st_stream(fifo + sp.line, u32x4{lo, flag, hi, flag});
}

template <int W>
__global__ __launch_bounds__(kLLDecodeThreads) void ll_unpack_reduce_kernel(
    InTable<W> fifos, float *out, int64_t n, uint32_t lines, uint32_t step_lines,
    uint64_t first_step, uint32_t max_spins, uint32_t *bad_lines)
{
    const uint32_t i = blockIdx.x * kLLDecodeThreads + threadIdx.x;
    if (i >= lines)
        return;
    const StepPos sp = step_pos(i, step_lines, first_step);
    const uint32_t flag = (uint32_t)(sp.step + 1);
    u32x4 v[W];
#pragma unroll
    for (int r = 0; r < W; ++r)
        v[r] = ld_stream(fifos.p[r] + sp.line);
    // Both flags must match ([NCCL14] "how LL publishes and waits for
    // flags"); otherwise re-read, a bounded number of times.
    uint32_t bad = 0;
#pragma unroll
    for (int r = 0; r < W; ++r) {
        bool ok = v[r].y == flag && v[r].w == flag;
        for (uint32_t s = 0; !ok && s < max_spins; ++s) {
            v[r] = reload16(&fifos.p[r][sp.line]);
            ok = v[r].y == flag && v[r].w == flag;
        }
        bad += ok ? 0u : 1u;
    }
    float a0 = __uint_as_float(v[0].x), a1 = __uint_as_float(v[0].z);
#pragma unroll
    for (int r = 1; r < W; ++r) {
        a0 = a0 + __uint_as_float(v[r].x);
        a1 = a1 + __uint_as_float(v[r].z);
    }
    const int64_t e = 2 * (int64_t)i;
    if (e + 1 < n) {
        st8_through(reinterpret_cast<uint32_t *>(out + e),
                    u32x2{__float_as_uint(a0), __float_as_uint(a1)});
    } else {
        out[e] = a0;
    }
    if (bad && bad_lines)
        atomicAdd(bad_lines, bad);
}

// ---------------------------------------------------------------------------
// LL128 ([NCCL14] "LL128's 128-byte line"): 15 payload u64 + 1 flag u64.
// Wire chunk j (16 bytes) of a line: payload fp32 words 30l + 4j .. +3 for
// j < 7; chunk 7 holds words 28, 29 and the flag.
//
// Encode: sixteen lanes (one DPP row) build two consecutive lines from their
// 240-byte payload span.  Lane c < 15 loads the c-th 16-byte chunk of the
// span, so every payload load is a whole, aligned dwordx4 (when src is
// 16-byte aligned).  Line A's chunks are those loads as they are; line B
// starts 8 bytes into chunk 7, so its chunk j is the high half of span chunk
// 7 + j (held by the lane to the left, fetched with DPP row_shr:1) followed
// by the low half of span chunk 8 + j.  Lanes 7 and 15 put the flags in.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kWireThreads) void ll128_pack_kernel(
    const uint32_t *src, int64_t n, u32x4 *fifo, uint32_t lines,
    uint32_t step_lines, uint64_t first_step)
{
    const uint64_t t = (uint64_t)blockIdx.x * kWireThreads + threadIdx.x;
    const uint32_t pair = (uint32_t)(t >> 4);
    const int c = (int)(t & 15);
    const uint32_t la = 2 * pair, lb = la + 1;
    const bool live = la < lines;          // the same for all 16 lanes of a pair
    const int64_t e0 = 60 * (int64_t)pair + 4 * c;
    u32x4 d = {0u, 0u, 0u, 0u};
    if (live && c < 15) {
        if (e0 + 3 < n) {
            d = ld4_stream_a4(src + e0);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                d[k] = e0 + k < n ? src[e0 + k] : 0u;
        }
    }
    // Every lane takes part in the row shift; lane 0 of a row receives 0.
    const uint32_t hz = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)d.z, 0x111, 0xF, 0xF, false);
    const uint32_t hw = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)d.w, 0x111, 0xF, 0xF, false);
    if (!live || (c >= 8 && lb >= lines))
        return;
    const uint32_t line = c < 8 ? la : lb;
    const StepPos sp = step_pos(line, step_lines, first_step);
    const uint64_t flag = sp.step + 1;
    u32x4 o;
    if (c < 7)
        o = d;
    else if (c == 7)
        o = u32x4{d.x, d.y, (uint32_t)flag, (uint32_t)(flag >> 32)};
    else if (c < 15)
        o = u32x4{hz, hw, d.x, d.y};
    else
        o = u32x4{hz, hw, (uint32_t)flag, (uint32_t)(flag >> 32)};
    st16_through(fifo + sp.line * 8 + (c & 7), o);
}

// Decode: eight lanes per line, lane j owning wire chunk j (an aligned
// dwordx4 load from each FIFO); lane 7 also holds the flag.
template <int W>
__global__ __launch_bounds__(kWireThreads) void ll128_unpack_reduce_kernel(
    InTable<W> fifos, float *out, int64_t n, uint32_t lines, uint32_t step_lines,
    uint64_t first_step, uint32_t max_spins, uint32_t *bad_lines)
{
    const uint64_t t = (uint64_t)blockIdx.x * kWireThreads + threadIdx.x;
    const uint32_t l = (uint32_t)(t >> 3);
    const int j = (int)(t & 7);
    const int lane = threadIdx.x & 63;
    // Every lane stays to the end: the readiness vote below is wavefront-wide.
    const bool live = l < lines;
    StepPos sp{0, 0};
    u32x4 v[W];
    if (live) {
        sp = step_pos(l, step_lines, first_step);
#pragma unroll
        for (int r = 0; r < W; ++r)
            v[r] = ld_stream(fifos.p[r] + sp.line * 8 + j);
    }
    const uint64_t flag = sp.step + 1;
    const uint32_t flo = (uint32_t)flag, fhi = (uint32_t)(flag >> 32);
    // The flag lane of each line checks the flag word; a ballot tells the
    // other 7 lanes of that line whether to re-read their chunk too
    // ([NCCL14] "LL128's warp-level ready check").  Bounded by max_spins.
    uint32_t bad = 0;
#pragma unroll
    for (int r = 0; r < W; ++r) {
        bool ok = !live || j != 7 || (v[r].z == flo && v[r].w == fhi);
        uint64_t mask = __ballot(!ok);
        for (uint32_t s = 0; mask != 0 && s < max_spins; ++s) {
            if (live && ((mask >> (lane | 7)) & 1u))
                v[r] = reload16(&fifos.p[r][sp.line * 8 + j]);
            ok = !live || j != 7 || (v[r].z == flo && v[r].w == fhi);
            mask = __ballot(!ok);
        }
        bad += ok ? 0u : 1u;
    }
    if (!live)
        return;
    const int nv = j < 7 ? 4 : 2;
    float a[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        a[c] = __uint_as_float(v[0][c]);
#pragma unroll
    for (int r = 1; r < W; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            a[c] = a[c] + __uint_as_float(v[r][c]);
    const int64_t e0 = 30 * (int64_t)l + 4 * j;
    if (e0 + nv <= n) {
        if (nv == 4)
            st4_stream_a4(reinterpret_cast<uint32_t *>(out + e0),
                          u32x4{__float_as_uint(a[0]), __float_as_uint(a[1]),
                                __float_as_uint(a[2]), __float_as_uint(a[3])});
        else
            st2_stream_a4(reinterpret_cast<uint32_t *>(out + e0),
                          u32x2{__float_as_uint(a[0]), __float_as_uint(a[1])});
    } else {
        for (int c = 0; c < nv; ++c)
            if (e0 + c < n)
                out[e0 + c] = a[c];
    }
    if (bad && bad_lines)
        atomicAdd(bad_lines, bad);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static unsigned blocks_for(uint64_t threads)
{
    return (unsigned)((threads + kWireThreads - 1) / kWireThreads);
}

hipError_t launch_ll_pack(const float *src, int64_t n, void *fifo,
                          int64_t step_lines, uint64_t first_step, hipStream_t s)
{
    const uint32_t lines = (uint32_t)((n + 1) / 2);
    ll_pack_kernel<<<blocks_for(lines), kWireThreads, 0, s>>>(
        reinterpret_cast<const uint32_t *>(src), n, static_cast<u32x4 *>(fifo),
        lines, (uint32_t)step_lines, first_step);
    return hipGetLastError();
}

hipError_t launch_ll128_pack(const float *src, int64_t n, void *fifo,
                             int64_t step_lines, uint64_t first_step,
                             hipStream_t s)
{
    const uint32_t lines = (uint32_t)((n + 29) / 30);
    const uint64_t pairs = ((uint64_t)lines + 1) / 2;
    ll128_pack_kernel<<<blocks_for(pairs * 16), kWireThreads, 0, s>>>(
        reinterpret_cast<const uint32_t *>(src), n, static_cast<u32x4 *>(fifo),
        lines, (uint32_t)step_lines, first_step);
    return hipGetLastError();
}

template <int W, bool LL128>
static hipError_t launch_unpack_w(const void *const *fifos, float *out, int64_t n,
                                  int64_t step_lines, uint64_t first_step,
                                  uint32_t max_spins, uint32_t *bad, hipStream_t s)
{
    InTable<W> t;
    for (int r = 0; r < W; ++r)
        t.p[r] = static_cast<const u32x4 *>(fifos[r]);
    if (LL128) {
        const uint32_t lines = (uint32_t)((n + 29) / 30);
        ll128_unpack_reduce_kernel<W><<<blocks_for((uint64_t)lines * 8), kWireThreads, 0, s>>>(
            t, out, n, lines, (uint32_t)step_lines, first_step, max_spins, bad);
    } else {
        const uint32_t lines = (uint32_t)((n + 1) / 2);
        ll_unpack_reduce_kernel<W><<<(unsigned)(((uint64_t)lines + kLLDecodeThreads - 1) /
                                                kLLDecodeThreads),
                                     kLLDecodeThreads, 0, s>>>(
            t, out, n, lines, (uint32_t)step_lines, first_step, max_spins, bad);
    }
    return hipGetLastError();
}

template <bool LL128>
static hipError_t launch_unpack(const void *const *fifos, int W, float *out,
                                int64_t n, int64_t step_lines, uint64_t first_step,
                                uint32_t max_spins, uint32_t *bad, hipStream_t s)
{
    switch (W) {
    case 1: return launch_unpack_w<1, LL128>(fifos, out, n, step_lines, first_step, max_spins, bad, s);
    case 2: return launch_unpack_w<2, LL128>(fifos, out, n, step_lines, first_step, max_spins, bad, s);
    case 3: return launch_unpack_w<3, LL128>(fifos, out, n, step_lines, first_step, max_spins, bad, s);
    case 4: return launch_unpack_w<4, LL128>(fifos, out, n, step_lines, first_step, max_spins, bad, s);
    case 5: return launch_unpack_w<5, LL128>(fifos, out, n, step_lines, first_step, max_spins, bad, s);
    case 6: return launch_unpack_w<6, LL128>(fifos, out, n, step_lines, first_step, max_spins, bad, s);
    case 7: return launch_unpack_w<7, LL128>(fifos, out, n, step_lines, first_step, max_spins, bad, s);
    case 8: return launch_unpack_w<8, LL128>(fifos, out, n, step_lines, first_step, max_spins, bad, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_ll_unpack_reduce(const void *const *fifos, int W, float *out,
                                   int64_t n, int64_t step_lines,
                                   uint64_t first_step, uint32_t max_spins,
                                   uint32_t *bad_lines, hipStream_t s)
{
    return launch_unpack<false>(fifos, W, out, n, step_lines, first_step, max_spins,
                                bad_lines, s);
}

hipError_t launch_ll128_unpack_reduce(const void *const *fifos, int W,
                                      float *out, int64_t n, int64_t step_lines,
                                      uint64_t first_step, uint32_t max_spins,
                                      uint32_t *bad_lines, hipStream_t s)
{
    return launch_unpack<true>(fifos, W, out, n, step_lines, first_step, max_spins,
                               bad_lines, s);
}

}  // namespace ar
