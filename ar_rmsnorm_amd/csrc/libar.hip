// C entry points of libar: argument validation, then one kernel launch on the
// caller's stream.  Every check runs before anything is enqueued, so a call
// that returns an error code has touched no buffer.  See include/libar.h for
// the contract of each entry point.
#include "../../include/libar.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "index_map.h"
#include "launch.h"
#include "stream_plan.h"

#define LIBAR_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local int g_last_hip_error = 0;

ar_status_t from_hip(hipError_t e)
{
    if (e == hipSuccess)
        return AR_OK;
    g_last_hip_error = (int)e;
    return AR_ERR_HIP;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Do the byte ranges [a, a + na) and [b, b + nb) share a byte?
bool overlaps(const void *a, int64_t na, const void *b, int64_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na > 0 && nb > 0 && x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// Overlap that is not exact identity of the two ranges.
bool overlaps_partially(const void *a, const void *b, int64_t nbytes)
{
    return a != b && overlaps(a, nbytes, b, nbytes);
}

constexpr int64_t kMaxLines = (int64_t)1 << 31;
constexpr int64_t kMaxElems = (int64_t)1 << 40;   // keeps every grid in range

}  // namespace

LIBAR_EXPORT const char *ar_status_str(ar_status_t status)
{
    switch (status) {
    case AR_OK: return "ok";
    case AR_ERR_NULL: return "a required pointer is NULL";
    case AR_ERR_ARG: return "invalid size, flag or buffer aliasing";
    case AR_ERR_ALIGN: return "pointer not aligned as required";
    case AR_ERR_WORLD: return "number of rank buffers W out of range";
    case AR_ERR_CAPACITY:
        return "payload does not fit the 8 steps of the FIFO or the library's staging "
               "array, or the streaming workgroups cannot all be resident at once";
    case AR_ERR_HIP: return "HIP runtime rejected the launch";
    default: return "unknown status";
    }
}

LIBAR_EXPORT int ar_last_hip_error(void) { return g_last_hip_error; }

// ---------------------------------------------------------------------------
LIBAR_EXPORT ar_status_t ar_reduce_1stage(const void *const *inputs, int W, void *out,
                                          int64_t n, ar_stream_t stream)
{
    if (!inputs || !out)
        return AR_ERR_NULL;
    if (W < 2 || W > AR_MAX_WORLD)
        return AR_ERR_WORLD;
    for (int r = 0; r < W; ++r)
        if (!inputs[r])
            return AR_ERR_NULL;
    if (n < 0 || n % 8 != 0 || n > kMaxElems)
        return AR_ERR_ARG;
    if (!aligned(out, 16))
        return AR_ERR_ALIGN;
    for (int r = 0; r < W; ++r)
        if (!aligned(inputs[r], 16))
            return AR_ERR_ALIGN;
    for (int r = 0; r < W; ++r)
        if (overlaps_partially(out, inputs[r], 2 * n))
            return AR_ERR_ARG;
    if (n == 0)
        return AR_OK;
    return from_hip(ar::launch_reduce_1stage(inputs, W, out, n / 8,
                                             static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
LIBAR_EXPORT ar_status_t ar_reduce_2stage(const void *const *inputs, void *const *tmps,
                                          int W, int rank, void *out, int64_t n,
                                          unsigned flags, ar_stream_t stream)
{
    if (!inputs || !tmps)
        return AR_ERR_NULL;
    if (W < 2 || W > AR_MAX_WORLD)
        return AR_ERR_WORLD;
    if (flags & ~(AR_STAGE_RS | AR_STAGE_AG | AR_ORDER_RANK))
        return AR_ERR_ARG;
    if ((flags & (AR_STAGE_RS | AR_STAGE_AG)) == 0)
        flags |= AR_STAGE_RS | AR_STAGE_AG;
    const bool rs = flags & AR_STAGE_RS, ag = flags & AR_STAGE_AG;
    for (int r = 0; r < W; ++r)
        if (!inputs[r] || !tmps[r])
            return AR_ERR_NULL;
    if (ag && !out)
        return AR_ERR_NULL;
    if (rank < 0 || rank >= W || n < 0 || n % 8 != 0 || n > kMaxElems)
        return AR_ERR_ARG;
    for (int r = 0; r < W; ++r)
        if (!aligned(inputs[r], 16) || !aligned(tmps[r], 16))
            return AR_ERR_ALIGN;
    if (ag && !aligned(out, 16))
        return AR_ERR_ALIGN;
    const int64_t packs = n / 8;
    const int64_t tmp_bytes = (packs / W + packs % W) * 16;
    for (int r = 0; r < W; ++r) {
        if (ag && (overlaps(out, 2 * n, inputs[r], 2 * n) ||
                   overlaps(out, 2 * n, tmps[r], tmp_bytes)))
            return AR_ERR_ARG;
        if (rs && overlaps(tmps[rank], tmp_bytes, inputs[r], 2 * n))
            return AR_ERR_ARG;
        if (rs && ag && r != rank && overlaps(tmps[rank], tmp_bytes, tmps[r], tmp_bytes))
            return AR_ERR_ARG;
    }
    if (n == 0)
        return AR_OK;
    // The owner's summation order: its own buffer first, then the next ranks
    // round the ring, or plain rank order on request.
    int order[AR_MAX_WORLD];
    for (int i = 0; i < W; ++i)
        order[i] = (flags & AR_ORDER_RANK) ? i : (rank + i) % W;
    return from_hip(ar::launch_reduce_2stage(inputs, order, tmps, W, rank, out, packs,
                                             rs, ag, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// Two-stage reduce with library-owned staging.  The W staging shards live in
// `scratch`, one array per device for the life of the process.  In host code
// the array's name is only a stand-in for the symbol: its device address is
// looked up once per device with hipGetSymbolAddress and kept in
// g_scratch_ptr, and only that address reaches a kernel.
// ---------------------------------------------------------------------------
namespace {

static __device__ __align__(256) uint8_t scratch[AR_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, looked up on the first call on
// that device.  Concurrent first calls may both look it up; they store the
// same address.
hipError_t scratch_address(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace

LIBAR_EXPORT ar_status_t ar_reduce_2stage_noalloc(const void *const *inputs, int W, int rank,
                                                  void *out, int64_t n, unsigned flags,
                                                  ar_stream_t stream)
{
    if (!inputs)
        return AR_ERR_NULL;
    if (W < 2 || W > AR_MAX_WORLD)
        return AR_ERR_WORLD;
    if (flags & ~(AR_STAGE_RS | AR_STAGE_AG | AR_ORDER_RANK))
        return AR_ERR_ARG;
    if ((flags & (AR_STAGE_RS | AR_STAGE_AG)) == 0)
        flags |= AR_STAGE_RS | AR_STAGE_AG;
    const bool rs = flags & AR_STAGE_RS, ag = flags & AR_STAGE_AG;
    for (int r = 0; r < W; ++r)
        if (!inputs[r])
            return AR_ERR_NULL;
    if (ag && !out)
        return AR_ERR_NULL;
    if (rank < 0 || rank >= W || n < 0 || n % 8 != 0 || n > kMaxElems)
        return AR_ERR_ARG;
    const int64_t packs = n / 8;
    const int64_t cap_bytes = (packs / W + packs % W) * 16;   // one shard's staging
    if (cap_bytes * W > (int64_t)AR_SCRATCH_BYTES)
        return AR_ERR_CAPACITY;
    for (int r = 0; r < W; ++r)
        if (!aligned(inputs[r], 16))
            return AR_ERR_ALIGN;
    if (ag && !aligned(out, 16))
        return AR_ERR_ALIGN;
    if (ag)
        for (int r = 0; r < W; ++r)
            if (overlaps(out, 2 * n, inputs[r], 2 * n))
                return AR_ERR_ARG;
    if (n == 0)
        return AR_OK;
    void *base = nullptr;
    const hipError_t e = scratch_address(&base);
    if (e != hipSuccess)
        return from_hip(e);
    void *tmps[AR_MAX_WORLD];
    for (int s = 0; s < W; ++s)
        tmps[s] = static_cast<uint8_t *>(base) + (int64_t)s * cap_bytes;
    int order[AR_MAX_WORLD];
    for (int i = 0; i < W; ++i)
        order[i] = (flags & AR_ORDER_RANK) ? i : (rank + i) % W;
    return from_hip(ar::launch_reduce_2stage(inputs, order, tmps, W, rank, out, packs, rs, ag,
                                             static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
LIBAR_EXPORT ar_status_t ar_fused_residual_rmsnorm(const void *const *inputs, int W,
                                                   const void *residual, const void *weight,
                                                   void *residual_out, void *norm_out,
                                                   int64_t M, int64_t N, float eps,
                                                   ar_stream_t stream)
{
    if (!inputs || !residual || !weight || !residual_out || !norm_out)
        return AR_ERR_NULL;
    if (W < 2 || W > AR_MAX_WORLD)
        return AR_ERR_WORLD;
    for (int r = 0; r < W; ++r)
        if (!inputs[r])
            return AR_ERR_NULL;
    if (M < 0 || N < 8 || N > AR_FUSED_MAX_N || N % 8 != 0 || M > 0x7FFFFFFF)
        return AR_ERR_ARG;
    if (!(eps >= 0.0f) || eps > 3.0e38f)   // rejects NaN, negatives and inf
        return AR_ERR_ARG;
    if (!aligned(residual, 16) || !aligned(weight, 16) || !aligned(residual_out, 16) ||
        !aligned(norm_out, 16))
        return AR_ERR_ALIGN;
    for (int r = 0; r < W; ++r)
        if (!aligned(inputs[r], 16))
            return AR_ERR_ALIGN;
    const int64_t mat = 2 * M * N, vec = 2 * N;
    if (overlaps_partially(residual_out, residual, mat) ||
        overlaps(residual_out, mat, weight, vec) ||
        overlaps(norm_out, mat, residual, mat) || overlaps(norm_out, mat, weight, vec) ||
        overlaps(norm_out, mat, residual_out, mat))
        return AR_ERR_ARG;
    for (int r = 0; r < W; ++r)
        if (overlaps(norm_out, mat, inputs[r], mat) ||
            overlaps(residual_out, mat, inputs[r], mat))
            return AR_ERR_ARG;
    if (M == 0)
        return AR_OK;
    return from_hip(ar::launch_fused_rmsnorm(inputs, W, residual, weight, residual_out,
                                             norm_out, M, N, eps,
                                             static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
LIBAR_EXPORT ar_status_t ar_fused_residual_rmsnorm_2stage(
    const void *const *inputs, void *const *tmps, int W, int rank, const void *residual,
    const void *weight, void *residual_out, void *norm_out, int64_t M, int64_t N, float eps,
    unsigned flags, ar_stream_t stream)
{
    if (!inputs || !tmps || !residual || !weight)
        return AR_ERR_NULL;
    if (W < 2 || W > AR_MAX_WORLD)
        return AR_ERR_WORLD;
    if (flags & ~(AR_STAGE_RS | AR_STAGE_AG | AR_ORDER_RANK))
        return AR_ERR_ARG;
    if ((flags & (AR_STAGE_RS | AR_STAGE_AG)) == 0)
        flags |= AR_STAGE_RS | AR_STAGE_AG;
    const bool rs = flags & AR_STAGE_RS, ag = flags & AR_STAGE_AG;
    for (int r = 0; r < W; ++r)
        if (!inputs[r] || !tmps[r])
            return AR_ERR_NULL;
    if (ag && (!residual_out || !norm_out))
        return AR_ERR_NULL;
    if (rank < 0 || rank >= W || M < 0 || M > 0x7FFFFFFF || N < 8 || N > AR_FUSED_MAX_N ||
        N % 8 != 0 || !(eps >= 0.0f) || eps > 3.0e38f)
        return AR_ERR_ARG;
    if (!aligned(residual, 16) || !aligned(weight, 16) ||
        (ag && (!aligned(residual_out, 16) || !aligned(norm_out, 16))))
        return AR_ERR_ALIGN;
    for (int r = 0; r < W; ++r)
        if (!aligned(inputs[r], 16) || !aligned(tmps[r], 16))
            return AR_ERR_ALIGN;
    const int64_t mat = 2 * M * N, vec = 2 * N;
    const int64_t tmp_bytes = 2 * (M / W + M % W) * N * 2;
    for (int r = 0; r < W; ++r) {
        if (rs && (overlaps(tmps[rank], tmp_bytes, inputs[r], mat) ||
                   (r != rank && overlaps(tmps[rank], tmp_bytes, tmps[r], tmp_bytes))))
            return AR_ERR_ARG;
        if (ag && (overlaps(residual_out, mat, inputs[r], mat) ||
                   overlaps(residual_out, mat, tmps[r], tmp_bytes) ||
                   overlaps(norm_out, mat, inputs[r], mat) ||
                   overlaps(norm_out, mat, tmps[r], tmp_bytes)))
            return AR_ERR_ARG;
    }
    if (rs && (overlaps(tmps[rank], tmp_bytes, residual, mat) ||
               overlaps(tmps[rank], tmp_bytes, weight, vec)))
        return AR_ERR_ARG;
    if (ag && (overlaps_partially(residual_out, residual, mat) ||
               overlaps(residual_out, mat, weight, vec) || overlaps(norm_out, mat, residual, mat) ||
               overlaps(norm_out, mat, weight, vec) || overlaps(norm_out, mat, residual_out, mat)))
        return AR_ERR_ARG;
    if (M == 0)
        return AR_OK;
    int order[AR_MAX_WORLD];
    for (int i = 0; i < W; ++i)
        order[i] = (flags & AR_ORDER_RANK) ? i : (rank + i) % W;
    return from_hip(ar::launch_fused_2stage(inputs, order, tmps, W, rank, residual, weight,
                                            residual_out, norm_out, M, N, eps, rs, ag,
                                            static_cast<hipStream_t>(stream)));
}

// One-GPU choice between the fused forms.  Per rank the one-shot call reads
// W input rows and the residual and writes two outputs for every row: W + 3
// rows of traffic per row.  The two-shot call does that only for its M / W
// own rows (plus staging them) and copies two staged rows for every other
// row: about 4 + 5 / W rows per row, fewer from W = 3 on, and its per-row
// latency chain is one row's loads, not W rows'.  Timed for one rank on one
// MI355X (cold buffers, N = 2048 and 8192, M from W to 2048 rows), the
// two-shot call was faster at every M >= W for W = 4 and W = 8, by 6-60 %;
// for W = 2 the two forms were within 3 % either way, and the one-shot call
// is kept (it needs no staging and, on several GPUs, no second exchange).
// With M < W one owner would take every row, which saves nothing.
LIBAR_EXPORT int ar_fused_prefers_two_shot(int W, int64_t M, int64_t N)
{
    if (W < 2 || W > AR_MAX_WORLD || M < 0 || M > 0x7FFFFFFF || N < 8 ||
        N > AR_FUSED_MAX_N || N % 8 != 0)
        return -1;
    return (W >= 3 && M >= W) ? 1 : 0;
}

// ---------------------------------------------------------------------------
// Lamport data-as-flag fused one-shot
// ---------------------------------------------------------------------------
namespace {

bool fused_shape_ok(int64_t M, int64_t N)
{
    return M >= 0 && M <= 0x7FFFFFFF && N >= 8 && N <= AR_FUSED_MAX_N && N % 8 == 0 &&
           M * N <= kMaxElems;
}

}  // namespace

LIBAR_EXPORT uint32_t ar_lamport_next_flag(uint32_t flag)
{
    return flag + 1u >= AR_LAMPORT_FLAG_PERIOD ? 0u : flag + 1u;
}

LIBAR_EXPORT int64_t ar_lamport_comm_bytes(int W, int64_t M, int64_t N)
{
    if (W < 2 || W > AR_MAX_WORLD || !fused_shape_ok(M, N))
        return 0;
    return 3 * (int64_t)W * M * N * 2;
}

LIBAR_EXPORT ar_status_t ar_lamport_fill(void *comm, int W, int64_t M, int64_t N,
                                         ar_stream_t stream)
{
    if (!comm)
        return AR_ERR_NULL;
    if (W < 2 || W > AR_MAX_WORLD)
        return AR_ERR_WORLD;
    if (!fused_shape_ok(M, N))
        return AR_ERR_ARG;
    if (!aligned(comm, 16))
        return AR_ERR_ALIGN;
    if (M == 0)
        return AR_OK;
    return from_hip(ar::launch_lamport_fill(comm, ar_lamport_comm_bytes(W, M, N) / 16,
                                            static_cast<hipStream_t>(stream)));
}

LIBAR_EXPORT ar_status_t ar_lamport_push(const void *x, int W, int rank, void *const *comms,
                                         int64_t M, int64_t N, uint32_t flag,
                                         ar_stream_t stream)
{
    if (!x || !comms)
        return AR_ERR_NULL;
    if (W < 2 || W > AR_MAX_WORLD)
        return AR_ERR_WORLD;
    for (int p = 0; p < W; ++p)
        if (!comms[p])
            return AR_ERR_NULL;
    if (rank < 0 || rank >= W || !fused_shape_ok(M, N) || flag >= AR_LAMPORT_FLAG_PERIOD)
        return AR_ERR_ARG;
    if (!aligned(x, 16))
        return AR_ERR_ALIGN;
    for (int p = 0; p < W; ++p)
        if (!aligned(comms[p], 16))
            return AR_ERR_ALIGN;
    const int64_t cb = ar_lamport_comm_bytes(W, M, N);
    for (int p = 0; p < W; ++p) {
        if (overlaps(x, 2 * M * N, comms[p], cb))
            return AR_ERR_ARG;
        for (int q = 0; q < p; ++q)
            if (overlaps(comms[p], cb, comms[q], cb))
                return AR_ERR_ARG;
    }
    if (M == 0)
        return AR_OK;
    return from_hip(ar::launch_lamport_push(x, W, rank, comms, M, N, flag,
                                            static_cast<hipStream_t>(stream)));
}

LIBAR_EXPORT ar_status_t ar_lamport_fused_residual_rmsnorm(
    void *comm, int W, const void *residual, const void *weight, void *residual_out,
    void *norm_out, int64_t M, int64_t N, float eps, uint32_t flag, uint32_t max_spins,
    uint32_t *bad_chunks, ar_stream_t stream)
{
    if (!comm || !residual || !weight || !residual_out || !norm_out)
        return AR_ERR_NULL;
    if (W < 2 || W > AR_MAX_WORLD)
        return AR_ERR_WORLD;
    if (!fused_shape_ok(M, N) || max_spins > AR_MAX_SPINS || flag >= AR_LAMPORT_FLAG_PERIOD)
        return AR_ERR_ARG;
    if (!(eps >= 0.0f) || eps > 3.0e38f)
        return AR_ERR_ARG;
    if (!aligned(comm, 16) || !aligned(residual, 16) || !aligned(weight, 16) ||
        !aligned(residual_out, 16) || !aligned(norm_out, 16) ||
        (bad_chunks && !aligned(bad_chunks, 4)))
        return AR_ERR_ALIGN;
    const int64_t mat = 2 * M * N, vec = 2 * N, cb = ar_lamport_comm_bytes(W, M, N);
    if (overlaps_partially(residual_out, residual, mat) ||
        overlaps(residual_out, mat, weight, vec) || overlaps(residual_out, mat, comm, cb) ||
        overlaps(norm_out, mat, residual, mat) || overlaps(norm_out, mat, weight, vec) ||
        overlaps(norm_out, mat, residual_out, mat) || overlaps(norm_out, mat, comm, cb) ||
        overlaps(residual, mat, comm, cb) || overlaps(weight, vec, comm, cb))
        return AR_ERR_ARG;
    if (bad_chunks && (overlaps(bad_chunks, 4, comm, cb) || overlaps(bad_chunks, 4, norm_out, mat) ||
                       overlaps(bad_chunks, 4, residual_out, mat)))
        return AR_ERR_ARG;
    if (M == 0)
        return AR_OK;
    return from_hip(ar::launch_lamport_fused(comm, W, residual, weight, residual_out, norm_out,
                                             M, N, eps, flag, max_spins, bad_chunks, nullptr, 0,
                                             nullptr, static_cast<hipStream_t>(stream)));
}

LIBAR_EXPORT ar_status_t ar_lamport_oneshot_residual_rmsnorm(
    const void *x, int rank, void *const *comms, int W, const void *residual,
    const void *weight, void *residual_out, void *norm_out, int64_t M, int64_t N, float eps,
    uint32_t flag, uint32_t max_spins, uint32_t *bad_chunks, ar_stream_t stream)
{
    if (!x || !comms)
        return AR_ERR_NULL;
    if (W < 2 || W > AR_MAX_WORLD)
        return AR_ERR_WORLD;
    for (int p = 0; p < W; ++p)
        if (!comms[p])
            return AR_ERR_NULL;
    if (rank < 0 || rank >= W)
        return AR_ERR_ARG;
    // the reader's checks, on this rank's own buffer
    if (!residual || !weight || !residual_out || !norm_out)
        return AR_ERR_NULL;
    if (!fused_shape_ok(M, N) || max_spins > AR_MAX_SPINS || !(eps >= 0.0f) || eps > 3.0e38f ||
        flag >= AR_LAMPORT_FLAG_PERIOD)
        return AR_ERR_ARG;
    if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(weight, 16) ||
        !aligned(residual_out, 16) || !aligned(norm_out, 16) ||
        (bad_chunks && !aligned(bad_chunks, 4)))
        return AR_ERR_ALIGN;
    for (int p = 0; p < W; ++p)
        if (!aligned(comms[p], 16))
            return AR_ERR_ALIGN;
    const int64_t mat = 2 * M * N, vec = 2 * N, cb = ar_lamport_comm_bytes(W, M, N);
    if (overlaps_partially(residual_out, residual, mat) ||
        overlaps(residual_out, mat, weight, vec) || overlaps(norm_out, mat, residual, mat) ||
        overlaps(norm_out, mat, weight, vec) || overlaps(norm_out, mat, residual_out, mat) ||
        overlaps(x, mat, residual_out, mat) || overlaps(x, mat, norm_out, mat))
        return AR_ERR_ARG;
    for (int p = 0; p < W; ++p) {
        const void *c = comms[p];
        if (overlaps(c, cb, x, mat) || overlaps(c, cb, residual, mat) ||
            overlaps(c, cb, weight, vec) || overlaps(c, cb, residual_out, mat) ||
            overlaps(c, cb, norm_out, mat) || (bad_chunks && overlaps(c, cb, bad_chunks, 4)))
            return AR_ERR_ARG;
        for (int q = 0; q < p; ++q)
            if (overlaps(c, cb, comms[q], cb))
                return AR_ERR_ARG;
    }
    if (bad_chunks && (overlaps(bad_chunks, 4, norm_out, mat) ||
                       overlaps(bad_chunks, 4, residual_out, mat)))
        return AR_ERR_ARG;
    if (M == 0)
        return AR_OK;
    return from_hip(ar::launch_lamport_fused(comms[rank], W, residual, weight, residual_out,
                                             norm_out, M, N, eps, flag, max_spins, bad_chunks,
                                             x, rank, comms, static_cast<hipStream_t>(stream)));
}

LIBAR_EXPORT ar_status_t ar_lamport_all_ranks_residual_rmsnorm(
    const void *const *xs, void *const *comms, int W, const void *residual, const void *weight,
    void *const *residual_outs, void *const *norm_outs, int64_t M, int64_t N, float eps,
    uint32_t flag, uint32_t max_spins, uint32_t *bad_chunks, ar_stream_t stream)
{
    if (!xs || !comms || !residual || !weight || !residual_outs || !norm_outs)
        return AR_ERR_NULL;
    if (W < 2 || W > AR_MAX_WORLD)
        return AR_ERR_WORLD;
    for (int r = 0; r < W; ++r)
        if (!xs[r] || !comms[r] || !residual_outs[r] || !norm_outs[r])
            return AR_ERR_NULL;
    if (!fused_shape_ok(M, N) || max_spins > AR_MAX_SPINS || !(eps >= 0.0f) || eps > 3.0e38f ||
        flag >= AR_LAMPORT_FLAG_PERIOD)
        return AR_ERR_ARG;
    if (!aligned(residual, 16) || !aligned(weight, 16) || (bad_chunks && !aligned(bad_chunks, 4)))
        return AR_ERR_ALIGN;
    for (int r = 0; r < W; ++r)
        if (!aligned(xs[r], 16) || !aligned(comms[r], 16) || !aligned(residual_outs[r], 16) ||
            !aligned(norm_outs[r], 16))
            return AR_ERR_ALIGN;
    const int64_t mat = 2 * M * N, vec = 2 * N, cb = ar_lamport_comm_bytes(W, M, N);
    // every rank reads the shared residual and weight while the others write
    // their outputs, so no output may overlap any input or another output
    for (int r = 0; r < W; ++r) {
        const void *outs[2] = {residual_outs[r], norm_outs[r]};
        for (const void *o : outs) {
            if (overlaps(o, mat, residual, mat) || overlaps(o, mat, weight, vec) ||
                (bad_chunks && overlaps(o, mat, bad_chunks, 4)))
                return AR_ERR_ARG;
            for (int q = 0; q < W; ++q)
                if (overlaps(o, mat, xs[q], mat) || overlaps(o, mat, comms[q], cb))
                    return AR_ERR_ARG;
        }
        if (overlaps(residual_outs[r], mat, norm_outs[r], mat))
            return AR_ERR_ARG;
        for (int q = 0; q < r; ++q)
            if (overlaps(residual_outs[r], mat, residual_outs[q], mat) ||
                overlaps(residual_outs[r], mat, norm_outs[q], mat) ||
                overlaps(norm_outs[r], mat, residual_outs[q], mat) ||
                overlaps(norm_outs[r], mat, norm_outs[q], mat))
                return AR_ERR_ARG;
        const void *c = comms[r];
        if (overlaps(c, cb, residual, mat) || overlaps(c, cb, weight, vec) ||
            (bad_chunks && overlaps(c, cb, bad_chunks, 4)))
            return AR_ERR_ARG;
        for (int q = 0; q < W; ++q)
            if (overlaps(c, cb, xs[q], mat) || (q < r && overlaps(c, cb, comms[q], cb)))
                return AR_ERR_ARG;
    }
    if (M == 0)
        return AR_OK;
    int resident = 0;
    hipError_t e = ar::launch_lamport_all_ranks(xs, comms, W, residual, weight, residual_outs,
                                                norm_outs, M, N, eps, flag, max_spins,
                                                bad_chunks, true, &resident, nullptr);
    if (e != hipSuccess)
        return from_hip(e);
    if ((int64_t)resident < M * W)
        return AR_ERR_CAPACITY;
    return from_hip(ar::launch_lamport_all_ranks(xs, comms, W, residual, weight, residual_outs,
                                                 norm_outs, M, N, eps, flag, max_spins,
                                                 bad_chunks, false, nullptr,
                                                 static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// wire formats
// ---------------------------------------------------------------------------
LIBAR_EXPORT int64_t ll_lines(int64_t n)
{
    return n > 0 && n <= kMaxElems ? (4 * n + 7) / 8 : 0;
}
LIBAR_EXPORT int64_t ll128_lines(int64_t n)
{
    return n > 0 && n <= kMaxElems ? (4 * n + 119) / 120 : 0;
}
LIBAR_EXPORT int64_t ll_fifo_bytes(int64_t step_lines)
{
    return step_lines > 0 && step_lines <= kMaxLines / AR_FIFO_STEPS
               ? AR_FIFO_STEPS * step_lines * 16 : 0;
}
LIBAR_EXPORT int64_t ll128_fifo_bytes(int64_t step_lines)
{
    return step_lines > 0 && step_lines <= kMaxLines / AR_FIFO_STEPS
               ? AR_FIFO_STEPS * step_lines * 128 : 0;
}
LIBAR_EXPORT int64_t ll_default_step_lines(void) { return 4096; }
LIBAR_EXPORT int64_t ll128_default_step_lines(void) { return 4800; }

namespace {

// Checks common to the pack entry points.
ar_status_t check_pack(const float *src, int64_t n, void *fifo, int64_t step_lines,
                       int64_t lines, int64_t line_bytes)
{
    if (!src || !fifo)
        return AR_ERR_NULL;
    if (n < 0 || n > kMaxElems || step_lines < 1 || step_lines > kMaxLines / AR_FIFO_STEPS)
        return AR_ERR_ARG;
    if (lines > AR_FIFO_STEPS * step_lines)
        return AR_ERR_CAPACITY;
    if (!aligned(src, 4) || !aligned(fifo, line_bytes == 16 ? 16 : 128))
        return AR_ERR_ALIGN;
    if (overlaps(src, 4 * n, fifo, AR_FIFO_STEPS * step_lines * line_bytes))
        return AR_ERR_ARG;
    return AR_OK;
}

ar_status_t check_unpack(const void *const *fifos, int W, float *out, int64_t n,
                         int64_t step_lines, int64_t lines, int64_t line_bytes,
                         uint32_t max_spins, uint32_t *bad_lines)
{
    if (!fifos || !out)
        return AR_ERR_NULL;
    if (W < 1 || W > AR_MAX_WORLD)
        return AR_ERR_WORLD;
    for (int r = 0; r < W; ++r)
        if (!fifos[r])
            return AR_ERR_NULL;
    if (n < 0 || n > kMaxElems || step_lines < 1 || step_lines > kMaxLines / AR_FIFO_STEPS ||
        max_spins > AR_MAX_SPINS)
        return AR_ERR_ARG;
    if (lines > AR_FIFO_STEPS * step_lines)
        return AR_ERR_CAPACITY;
    if (!aligned(out, 4) || (bad_lines && !aligned(bad_lines, 4)))
        return AR_ERR_ALIGN;
    for (int r = 0; r < W; ++r)
        if (!aligned(fifos[r], line_bytes == 16 ? 16 : 128))
            return AR_ERR_ALIGN;
    const int64_t fifo_bytes = AR_FIFO_STEPS * step_lines * line_bytes;
    for (int r = 0; r < W; ++r)
        if (overlaps(out, 4 * n, fifos[r], fifo_bytes) ||
            (bad_lines && overlaps(bad_lines, 4, fifos[r], fifo_bytes)))
            return AR_ERR_ARG;
    if (bad_lines && overlaps(bad_lines, 4, out, 4 * n))
        return AR_ERR_ARG;
    return AR_OK;
}

}  // namespace

LIBAR_EXPORT ar_status_t ll_pack(const float *src, int64_t n, void *fifo,
                                 int64_t step_lines, uint64_t first_step,
                                 ar_stream_t stream)
{
    const ar_status_t st = check_pack(src, n, fifo, step_lines, ll_lines(n), 16);
    if (st != AR_OK || n == 0)
        return st;
    return from_hip(ar::launch_ll_pack(src, n, fifo, step_lines, first_step,
                                       static_cast<hipStream_t>(stream)));
}

LIBAR_EXPORT ar_status_t ll128_pack(const float *src, int64_t n, void *fifo,
                                    int64_t step_lines, uint64_t first_step,
                                    ar_stream_t stream)
{
    const ar_status_t st = check_pack(src, n, fifo, step_lines, ll128_lines(n), 128);
    if (st != AR_OK || n == 0)
        return st;
    return from_hip(ar::launch_ll128_pack(src, n, fifo, step_lines, first_step,
                                          static_cast<hipStream_t>(stream)));
}

LIBAR_EXPORT ar_status_t ll_unpack_reduce(const void *const *fifos, int W, float *out,
                                          int64_t n, int64_t step_lines,
                                          uint64_t first_step, uint32_t max_spins,
                                          uint32_t *bad_lines, ar_stream_t stream)
{
    const ar_status_t st = check_unpack(fifos, W, out, n, step_lines, ll_lines(n), 16,
                                        max_spins, bad_lines);
    if (st != AR_OK || n == 0)
        return st;
    return from_hip(ar::launch_ll_unpack_reduce(fifos, W, out, n, step_lines, first_step,
                                                max_spins, bad_lines,
                                                static_cast<hipStream_t>(stream)));
}

LIBAR_EXPORT ar_status_t ll128_unpack_reduce(const void *const *fifos, int W, float *out,
                                             int64_t n, int64_t step_lines,
                                             uint64_t first_step, uint32_t max_spins,
                                             uint32_t *bad_lines, ar_stream_t stream)
{
    const ar_status_t st = check_unpack(fifos, W, out, n, step_lines, ll128_lines(n), 128,
                                        max_spins, bad_lines);
    if (st != AR_OK || n == 0)
        return st;
    return from_hip(ar::launch_ll128_unpack_reduce(fifos, W, out, n, step_lines,
                                                   first_step, max_spins, bad_lines,
                                                   static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// plain copy (the achievable-copy reference of the measurements)
// ---------------------------------------------------------------------------
LIBAR_EXPORT ar_status_t ar_copy(const void *src, void *dst, int64_t nbytes,
                                 ar_stream_t stream)
{
    if (!src || !dst)
        return AR_ERR_NULL;
    if (nbytes < 0 || nbytes % 16 != 0 || nbytes > ((int64_t)1 << 44))
        return AR_ERR_ARG;
    if (!aligned(src, 16) || !aligned(dst, 16))
        return AR_ERR_ALIGN;
    if (overlaps(src, nbytes, dst, nbytes))
        return AR_ERR_ARG;
    if (nbytes == 0)
        return AR_OK;
    return from_hip(ar::launch_copy(src, dst, nbytes / 16, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// streaming through 8-step FIFOs
// ---------------------------------------------------------------------------
LIBAR_EXPORT int64_t ar_fifo_step_wire_bytes(int proto, int64_t step_bytes)
{
    const int64_t unit = proto == AR_PROTO_LL ? 8 : proto == AR_PROTO_LL128 ? 120 : 16;
    if (proto < AR_PROTO_LL || proto > AR_PROTO_SIMPLE || step_bytes < unit ||
        step_bytes > ((int64_t)1 << 30) || step_bytes % unit != 0)
        return 0;
    if (proto == AR_PROTO_LL)
        return step_bytes / 8 * 16;
    if (proto == AR_PROTO_LL128)
        return step_bytes / 120 * 128;
    return step_bytes;
}

LIBAR_EXPORT int64_t ar_fifo_steps_per_channel(int64_t n, int64_t step_bytes, int channels)
{
    if (n <= 0 || n > kMaxElems || step_bytes <= 0 || channels < 1)
        return 0;
    return ar::fifo_steps_per_channel(n, step_bytes, channels);
}

static_assert(ar::kFifoMaxPairs == AR_FIFO_MAX_PAIRS, "pairs per channel");
static_assert(AR_PROTO_LL == 0 && AR_PROTO_LL128 == 1 && AR_PROTO_SIMPLE == 2,
              "protocol numbers of the streaming plan");

LIBAR_EXPORT int64_t ar_fifo_counter_words(int channels)
{
    return channels < 1 || channels > AR_FIFO_MAX_CHANNELS
               ? 0 : 2 * (int64_t)channels * AR_FIFO_MAX_PAIRS + 2;
}

namespace {

// Workgroups of the streaming kernel the device can hold at once, per
// (device, protocol, local addend, geometry), looked up once.
int resident_workgroups(int proto, bool local, bool wide, int *workgroups)
{
    constexpr int kDevices = 64;
    static std::atomic<int> cache[kDevices][3][2][2];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return (int)e;
    if (dev >= 0 && dev < kDevices) {
        const int c = cache[dev][proto][local][wide].load(std::memory_order_relaxed);
        if (c > 0) {
            *workgroups = c;
            return 0;
        }
    }
    e = ar::fifo_stream_resident_workgroups(proto, local, wide, workgroups);
    if (e == hipSuccess && dev >= 0 && dev < kDevices)
        cache[dev][proto][local][wide].store(*workgroups, std::memory_order_relaxed);
    return (int)e;
}

// Geometry and pairs (ar::fifo_plan_pairs, ar::fifo_plan_wide) from the
// workgroups of each size the device holds at once.  A pair's slice of a
// full step is at least 512 items, and a channel gets one pair per 2,048
// items it carries in the call: extra pairs only add workgroups when there
// is little to move (32 channels, LL: an 8 KiB message took 7.5 us with four
// pairs against 5.1 us with one, a 512 KiB one 8.2 against 6.4 us, while a
// 16 MiB one took 140 against 195 us).  1,024-lane workgroups take as many
// pairs as fit, unless that leaves one pair per channel (or none) where
// 512-lane ones fit at least two.  Measured on 16 Mi fp32 at NCCL's steps:
// at 128 channels two narrow pairs beat one wide pair (LL 86 against 99 us,
// LL128 67 against 71 us), at 32 channels four wide pairs beat eight narrow
// ones (LL 147 against 154 us, with batches inside one step).  LL with
// batches of whole steps also takes the 512-lane form where it gives at
// least twice the pairs and every channel carries 32 steps or more: 16 Mi
// fp32 at 64 channels 101 -> 83 us, at 48 channels 107 -> 94 us, at 32
// channels 95 -> 92 us; with fewer steps per channel (4 Mi over 32
// channels) the wider form stays faster (32 against 36 us).  Arguments
// already checked; n >= 1.
ar_status_t fifo_plan(int proto, bool local, int64_t n, int channels, int64_t step_bytes,
                      bool *wide, int *pairs)
{
    int wide_res = 0, narrow_res = 0;
    int he = resident_workgroups(proto, local, true, &wide_res);
    if (he == 0)
        he = resident_workgroups(proto, local, false, &narrow_res);
    if (he != 0)
        return from_hip((hipError_t)he);
    const int wide_pairs = ar::fifo_plan_pairs(proto, step_bytes, n, channels, wide_res);
    const int narrow_pairs = ar::fifo_plan_pairs(proto, step_bytes, n, channels, narrow_res);
    *wide = ar::fifo_plan_wide(proto, wide_pairs, narrow_pairs,
                               ar::fifo_steps_per_channel(n, step_bytes, channels));
    *pairs = *wide ? wide_pairs : narrow_pairs;
    return *pairs < 1 ? AR_ERR_CAPACITY : AR_OK;
}

}  // namespace

LIBAR_EXPORT ar_status_t ar_fifo_plan(int proto, int64_t n, int channels, int64_t step_bytes,
                                      int with_local, int *lanes, int *pairs, int *batch_steps)
{
    if (lanes)
        *lanes = 0;
    if (pairs)
        *pairs = 0;
    if (batch_steps)
        *batch_steps = 0;
    if (ar_fifo_step_wire_bytes(proto, step_bytes) == 0 || n < 0 || n > kMaxElems ||
        channels < 1 || channels > AR_FIFO_MAX_CHANNELS)
        return AR_ERR_ARG;
    if (n == 0)
        return AR_OK;
    bool wide = false;
    int p = 0;
    const ar_status_t ps = fifo_plan(proto, with_local != 0, n, channels, step_bytes, &wide, &p);
    if (ps != AR_OK)
        return ps;
    if (lanes)
        *lanes = wide ? 1024 : 512;
    if (pairs)
        *pairs = p;
    if (batch_steps)
        *batch_steps = ar::fifo_plan_batch_steps(proto, step_bytes, n, channels, p);
    return AR_OK;
}

LIBAR_EXPORT ar_status_t ar_fifo_stream(int proto, const float *src, const float *local,
                                        float *out, int64_t n, void *fifo, uint64_t *counters,
                                        int channels, int64_t step_bytes, uint64_t first_step,
                                        uint32_t max_spins, uint32_t *errors,
                                        ar_stream_t stream)
{
    if (!src || !out || !fifo || !counters || !errors)
        return AR_ERR_NULL;
    const int64_t wire = ar_fifo_step_wire_bytes(proto, step_bytes);
    if (wire == 0 || n < 0 || n > kMaxElems || channels < 1 || channels > AR_FIFO_MAX_CHANNELS ||
        max_spins > AR_MAX_SPINS)
        return AR_ERR_ARG;
    if (!aligned(src, 4) || !aligned(out, 4) || (local && !aligned(local, 4)) ||
        !aligned(fifo, proto == AR_PROTO_LL128 ? 128 : 16) || !aligned(counters, 8) ||
        !aligned(errors, 4))
        return AR_ERR_ALIGN;
    const int64_t fifo_bytes = (int64_t)channels * AR_FIFO_STEPS * wire;
    const int64_t cnt_bytes = ar_fifo_counter_words(channels) * 8;
    const int64_t nb = 4 * n;
    const void *ro[2] = {src, local};   // read-only inputs
    for (const void *r : ro) {
        if (!r)
            continue;
        if (overlaps(fifo, fifo_bytes, r, nb) || overlaps(counters, cnt_bytes, r, nb) ||
            overlaps(errors, 4, r, nb))
            return AR_ERR_ARG;
    }
    if (overlaps(out, nb, src, nb) || (local && overlaps_partially(out, local, nb)) ||
        overlaps(out, nb, fifo, fifo_bytes) || overlaps(out, nb, counters, cnt_bytes) ||
        overlaps(out, nb, errors, 4) || overlaps(fifo, fifo_bytes, counters, cnt_bytes) ||
        overlaps(fifo, fifo_bytes, errors, 4) || overlaps(counters, cnt_bytes, errors, 4))
        return AR_ERR_ARG;
    if (n == 0)
        return AR_OK;
    bool wide = false;
    int pairs = 0;
    const ar_status_t ps = fifo_plan(proto, local != nullptr, n, channels, step_bytes, &wide,
                                     &pairs);
    if (ps != AR_OK)
        return ps;
    return from_hip(ar::launch_fifo_stream(proto, src, local, out, n, fifo, counters, channels,
                                           step_bytes, wire, first_step,
                                           first_step == AR_FIFO_CONTINUE, max_spins, errors,
                                           wide, pairs, static_cast<hipStream_t>(stream)));
}
