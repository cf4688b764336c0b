// Streaming a payload through 8-step FIFOs on one device: producer and
// consumer workgroups run concurrently in one launch, each channel with its
// own 8-slot ring and one or more producer/consumer pairs.
//
// Source (web page; cited by tag and section):
//   [NCCL14] "NCCL 专家课程 14：Simple、LL、LL128 的线格式、同步与真实性能边界"
//            (blog.cptz.space): "prerequisite mental model" (an 8-step ring;
//            the sender never overwrites a step the receiver has not
//            consumed, the receiver never consumes a step before it is
//            ready), "how LL publishes and waits for flags", "LL128's 128-byte
//            line", "LL128's warp-level ready check", "how Simple
//            synchronizes".
//
// Protocols (payload per step = step_bytes):
//   LL      16-byte lines {lo, flag, hi, flag}; each line is written in one
//           16-byte access, so a line is ready once both flags are k + 1.
//   LL128   128-byte lines, 120 payload bytes + a 64-bit flag.  gfx950 does
//           not promise that a line written by eight lanes becomes visible
//           as a whole, so the producer makes the order explicit per batch
//           of 4,096 chunks (512 lines): every line of the batch goes out
//           whole, flag included, except that the batch's first line
//           carries a zero flag word; then a wait until those stores are
//           acknowledged and a barrier; then the first line's flag.  The
//           consumer waits for that flag (after which every byte of the
//           batch, every other line's flag included, is visible), then
//           reads every line and checks every line's flag, re-reading the
//           flag chunk of a line whose flag has not arrived yet.
//   Simple  raw payload; the producer publishes a tail step once the step's
//           data is acknowledged, and the consumer waits for it.
// For every protocol the consumer publishes a head step (the next step it
// will consume) after each step, and the producer reuses slot k mod 8 only
// once head >= k - 7.
//
// Pairs per channel.  A channel's steps may be shared by P producer/consumer
// workgroup pairs: pair g owns the same contiguous slice of every step
// (items [g * span, (g + 1) * span), span a whole number of LL128 line pairs),
// in the same 8-slot ring, with its own head and tail counters.  Producer g
// writes only its slice of a slot and consumer g reads only that slice, so a
// pair is a complete FIFO of its own and the pairs of a channel need no
// common counter.  More pairs keep more CUs busy when there are few channels,
// and shorten each pair's part of a step when a channel carries only one.
// The host picks P so that every full step gives every pair a slice; only a
// channel's last step, if partial, can leave a pair without one.
//
// Memory-level parallelism: every lane issues a batch of loads (source words,
// ring chunks, local addends) before it checks or stores any of them, items
// not yet ready are re-polled together, and the consumer releases a slot
// before it stores the step's last batch, so a step costs a few memory round
// trips rather than one per line.
//
// Step numbering persists in device memory between calls, as NCCL keeps a
// connection's step across launches: the counters end with {next first step,
// finished consumers}, and the last consumer of a launch to finish advances
// the stored first step by the call's steps per channel.  A call that asks
// for the stored step starts from it, which keeps a captured graph
// replayable.
//
// Ordering without cache maintenance.  Producer and consumer may sit on
// different XCDs, whose L2 caches are not coherent with each other, so every
// ring and counter access is system-coherent (sc0 sc1): a load reads the
// coherent copy and a store is acknowledged only once it is visible there.
// With that, "data before flag" needs no L2 write-back: a wavefront waits
// for its own stores (vmcnt(0)), the workgroup meets at a barrier, and only
// then is the flag, tail or head written.  A reader orders its later loads
// after a flag simply by issuing them after the flag's value came back.
// Counters are relaxed atomics, and each side caches the last value it saw
// of the other's counter, as NCCL caches a peer's step.  Every wait is
// bounded by max_spins and also ends as soon as any wait of the launch has
// failed (errors[0] != 0), so the launch always drains; its outputs are then
// unspecified.
#include "device.h"
#include "index_map.h"
#include "launch.h"
#include "stream_plan.h"

namespace ar {

// A batch is kPerBatch items of one step.  Two launch geometries cover it:
// 1,024 lanes with 4 items in flight each when the device holds 2 x channels
// such workgroups at once, else 512 lanes with 8 each (two workgroups per CU,
// up to 256 channels).  The wider one hides more of each batch's round trips.
constexpr int64_t kPerBatch = kFifoPerBatch;
constexpr int kWideThreads = 1024;
constexpr int kNarrowThreads = 512;
template <int T>
constexpr int kBatchOf = (int)(kPerBatch / T);   // items in flight per lane
constexpr uint32_t kAbortCheck = 16;   // spins between looks at the error count
constexpr int kMaxPairs = kFifoMaxPairs;      // producer/consumer pairs per channel
constexpr int kMaxBatchSteps = kFifoMaxBatchSteps;   // LL: whole steps per batch

struct StreamArgs {
    const uint32_t *src;    // n fp32 payload values (as words)
    const float *local;     // n fp32 added to the received payload, or NULL
    float *out;             // n fp32
    int64_t n;
    uint8_t *fifo;          // channels x 8 slots x wire bytes
    uint64_t *head;         // per pair: next ring step its consumer needs
    uint64_t *tail;         // per pair (Simple): ring steps published
    uint64_t *state;        // {next first step, finished consumers}
    uint32_t *errors;       // [0]: failed waits
    int64_t step_bytes;     // payload bytes per step
    int64_t wire_bytes;     // ring bytes per step
    int64_t total_steps;    // T = ceil(4n / step_bytes)
    int64_t steps_per_channel;
    int channels;
    int pairs;              // producer/consumer pairs per channel
    int64_t span;           // items of a full step per pair (fifo_span)
    int batch_steps;        // LL: whole steps per batch (fifo_batch_steps), else 1
    int from_state;         // the first step comes from state[0]
    uint64_t first_step;
    uint32_t max_spins;
};

// Ring accesses are buffer loads and stores with the system-coherent cache
// policy (sc0 sc1).  They are deliberately not volatile: on gfx950 every
// volatile access waits for its own completion before the next one issues,
// while these let a lane keep a whole batch in flight.  A descriptor covers
// one ring slot (at most 2^31 bytes), so every offset fits in 32 bits, and
// the hardware range check drops anything outside the slot.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kSysCoherent = 1 | 16;       // cache-policy bits sc0 | sc1
constexpr int kRsrcWord3 = 0x00020000;     // descriptor word 3: 32-bit data format
__device__ __forceinline__ Rsrc slot_rsrc(uint8_t *slot, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(slot, 0, (int)(uint32_t)bytes, kRsrcWord3);
}
__device__ __forceinline__ void store16_sys(Rsrc r, uint32_t off, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kSysCoherent);
}
__device__ __forceinline__ void store8_sys(Rsrc r, uint32_t off, u32x2 v)
{
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kSysCoherent);
}
__device__ __forceinline__ void store4_sys(Rsrc r, uint32_t off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, kSysCoherent);
}
__device__ __forceinline__ u32x4 load16_sys(Rsrc r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kSysCoherent);
}
__device__ __forceinline__ u32x2 load8_sys(Rsrc r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kSysCoherent);
}
// A compiler-only barrier at the top of every spin, so that a poll loop
// issues its loads again instead of reusing the values of the last spin.
__device__ __forceinline__ void respin()
{
    asm volatile("" ::: "memory");
}
// A value every lane holds alike, made visibly uniform to the compiler (so
// descriptors and branches built from it stay scalar).
__device__ __forceinline__ uint64_t uniform64(uint64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (uint64_t)hi << 32 | lo;
}
__device__ __forceinline__ uint64_t load_counter(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void store_counter(uint64_t *p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ bool aborted(const uint32_t *errors)
{
    return __hip_atomic_load(errors, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}
// The wavefront's loads have returned and its stores are acknowledged: an
// explicit wait.  A workgroup-scope release fence is not enough here: on
// gfx950 it emits no wait for vector memory (the waves of a workgroup share
// one CU), so the stores of a batch could still be in flight when the flags
// that publish them go out.  System-coherent (sc0 sc1) stores are
// acknowledged once they are visible at that scope, so no L2 write-back is
// needed.  The memory clobber keeps the compiler from moving memory
// accesses across the wait.
__device__ __forceinline__ void drain_memory()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Per-workgroup LDS slots for broadcasting lane 0's results.
struct Shared {
    int verdict;
    uint64_t value;
};

// Lane 0 waits (bounded) until poll() returns a value v with ready(v); the
// verdict and v reach the whole workgroup through LDS.  Returns false if the
// launch must stop.  Callers call it uniformly.
template <typename Poll, typename Ready>
__device__ bool wait_lane0(const StreamArgs &a, Shared *sh, uint64_t *seen, Poll poll,
                           Ready ready)
{
    if (threadIdx.x == 0) {
        uint64_t v = poll();
        bool ok = ready(v);
        for (uint32_t s = 0; !ok && s < a.max_spins; ++s) {
            respin();
            if (s % kAbortCheck == 0 && aborted(a.errors))
                break;
            v = poll();
            ok = ready(v);
        }
        if (!ok)
            atomicAdd(a.errors, 1u);
        sh->verdict = ok ? 1 : 0;
        sh->value = v;
    }
    __syncthreads();
    const bool go = __builtin_amdgcn_readfirstlane(sh->verdict) != 0;
    if (seen)
        *seen = uniform64(sh->value);
    __syncthreads();   // the slots are reused by the next wait
    return go;
}

// Wait until *counter >= need, skipping the poll when the last value seen
// already satisfies it.
__device__ bool wait_counter(const StreamArgs &a, Shared *sh, const uint64_t *counter,
                             uint64_t need, uint64_t *seen)
{
    if (*seen >= need)
        return true;
    return wait_lane0(
        a, sh, seen, [&] { return load_counter(counter); }, [&](uint64_t v) { return v >= need; });
}

// ---------------------------------------------------------------------------
// Payload access: source words past n read as zero; only out[0, n) is
// written and only local[0, n) is read.
__device__ __forceinline__ uint32_t word_at(const StreamArgs &a, int64_t w)
{
    return w < a.n ? a.src[w] : 0u;
}
__device__ __forceinline__ u32x2 pair_at(const StreamArgs &a, int64_t w)
{
    if (w + 2 <= a.n)
        return ld2_stream_a4(a.src + w);
    return u32x2{word_at(a, w), word_at(a, w + 1)};
}
__device__ __forceinline__ u32x4 quad_at(const StreamArgs &a, int64_t w)
{
    if (w + 4 <= a.n)
        return ld4_stream_a4(a.src + w);
    return u32x4{word_at(a, w), word_at(a, w + 1), word_at(a, w + 2), word_at(a, w + 3)};
}

// The local addend of words [w, w + cnt) (cnt is 2 or 4), zero past n.
__device__ __forceinline__ u32x4 local_at(const StreamArgs &a, int64_t w, int cnt)
{
    const uint32_t *l = reinterpret_cast<const uint32_t *>(a.local);
    if (cnt == 4 && w + 4 <= a.n)
        return ld4_stream_a4(l + w);
    if (cnt == 2 && w + 2 <= a.n) {
        const u32x2 v = ld2_stream_a4(l + w);
        return u32x4{v.x, v.y, 0u, 0u};
    }
    u32x4 r = {0u, 0u, 0u, 0u};
    for (int e = 0; e < cnt; ++e)
        if (w + e < a.n)
            r[e] = l[w + e];
    return r;
}

// out[w + e] = v[e], or local[w + e] + v[e] in fp32, for e < cnt, w + e < n.
template <bool LOCAL>
__device__ __forceinline__ void deliver(const StreamArgs &a, int64_t w, int cnt, u32x4 v,
                                        u32x4 lv)
{
    if (LOCAL) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = __float_as_uint(__uint_as_float(lv[e]) + __uint_as_float(v[e]));
    }
    uint32_t *o = reinterpret_cast<uint32_t *>(a.out);
    if (cnt == 4 && w + 4 <= a.n) {
        st4_stream_a4(o + w, v);
    } else if (cnt == 2 && w + 2 <= a.n) {
        st2_stream_a4(o + w, u32x2{v.x, v.y});
    } else {
        for (int e = 0; e < cnt; ++e)
            if (w + e < a.n)
                o[w + e] = v[e];
    }
}

// ---------------------------------------------------------------------------
// Steps and batches.  Items are LL lines, LL128 line chunks or Simple
// 16-byte chunks.  With T lanes a batch is kBatchOf<T> items per lane: items
// base + u * T + threadIdx.x, u < kBatchOf<T>.
//
// LL128 item q is chunk q % 8 of line q / 8 (chunks 0..6 carry 16 payload
// bytes, chunk 7 carries 8 payload bytes and then the flag).  Sixteen
// consecutive items, one DPP row, cover a pair of lines, whose 240 payload
// bytes are 15 aligned 16-byte payload chunks: lane c < 15 of the row moves
// payload chunk c with one whole dwordx4 load or store, and the 8-byte shift
// between the second line's chunks and the payload chunks is done across
// lanes with DPP row shifts.
struct Step {
    Rsrc slot;        // the step's ring slot
    int64_t w0;       // first payload word
    int64_t words;    // payload words
    int64_t lo;       // the pair's slice of the step's items: [lo, items)
    int64_t items;
    uint64_t k;       // ring step
};

// Items of a step of `len` payload bytes (`words` words).
template <int PROTO>
__device__ __forceinline__ int64_t items_of(int64_t len, int64_t words)
{
    return PROTO == 0 ? (len + 7) / 8 : PROTO == 1 ? (len + 119) / 120 * 8 : (words + 3) / 4;
}

// The slice of pair `pair` in a step of `total` items (fifo_slice: the same
// region of every ring slot, cut from a full step, so a partial last step
// keeps the regions of the full steps that used its slot before).  The span
// comes from the host, which computed it with fifo_span.
__device__ __forceinline__ void slice_of(const StreamArgs &a, int64_t total, int pair,
                                         int64_t *lo, int64_t *hi)
{
    fifo_slice_at(a.span, total, pair, lo, hi);
}

template <int PROTO>
__device__ __forceinline__ Step step_at(const StreamArgs &a, uint8_t *ring, int64_t s0,
                                        uint64_t first, int64_t j, int pair)
{
    Step g;
    g.k = first + (uint64_t)j;
    g.slot = slot_rsrc(ring + (int64_t)(g.k % 8u) * a.wire_bytes, a.wire_bytes);
    const int64_t b0 = (s0 + j) * a.step_bytes;
    const int64_t left = 4 * a.n - b0;
    const int64_t len = left < a.step_bytes ? left : a.step_bytes;
    g.w0 = b0 / 4;
    g.words = len / 4;
    slice_of(a, items_of<PROTO>(len, g.words), pair, &g.lo, &g.items);
    return g;
}

// A batch: local step j, first item base.
struct Cursor {
    int64_t j, base;
    Step g;
};

// The pair's first batch; false when it has nothing to move (its slice of
// the channel's only step is empty).
template <int PROTO>
__device__ __forceinline__ bool start(const StreamArgs &a, uint8_t *ring, int64_t s0,
                                      uint64_t first, int64_t steps, int pair, Cursor *cur)
{
    if (steps <= 0)
        return false;
    cur->j = 0;
    cur->g = step_at<PROTO>(a, ring, s0, first, 0, pair);
    cur->base = cur->g.lo;
    return cur->g.lo < cur->g.items;
}

// The batch after cur; false past the pair's last batch (an empty slice can
// only be that of the channel's last step).
template <int PROTO>
__device__ __forceinline__ bool advance(const StreamArgs &a, uint8_t *ring, int64_t s0,
                                        uint64_t first, int64_t steps, int pair,
                                        const Cursor &cur, Cursor *nxt)
{
    nxt->j = cur.j;
    nxt->base = cur.base + kPerBatch;
    nxt->g = cur.g;
    if (nxt->base >= cur.g.items) {
        nxt->j = cur.j + 1;
        if (nxt->j < steps) {
            nxt->g = step_at<PROTO>(a, ring, s0, first, nxt->j, pair);
            nxt->base = nxt->g.lo;
            if (nxt->g.lo >= nxt->g.items)
                nxt->j = steps;
        }
    }
    return nxt->j < steps;
}

// Payload words of LL or Simple item i of a step and how many of them there
// are (LL128 items go through the line-pair helpers below).
template <int PROTO>
__device__ __forceinline__ int64_t item_word(const Step &g, int64_t i)
{
    return PROTO == 0 ? g.w0 + 2 * i : g.w0 + 4 * i;
}
template <int PROTO>
__device__ __forceinline__ int item_count(const Step &g, int64_t i)
{
    if (PROTO == 0)
        return 2;
    const int64_t rem = g.words - 4 * i;
    return rem < 4 ? (int)rem : 4;
}
template <int PROTO>
__device__ __forceinline__ uint32_t ring_offset(int64_t i)
{
    return (uint32_t)(PROTO == 1 ? 128 * (i >> 3) + 16 * (i & 7) : 16 * i);
}

// Source words of a batch (zero for items past the step).
// Payload word of lane c's 16-byte payload chunk in the LL128 line pair
// holding item q.
__device__ __forceinline__ int64_t pair_chunk_word(const Step &g, int64_t q)
{
    return g.w0 + 60 * (q >> 4) + 4 * (q & 15);
}

template <int T, int PROTO>
__device__ __forceinline__ void load_src(const StreamArgs &a, const Step &g, int64_t base,
                                         u32x4 d[kBatchOf<T>])
{
#pragma unroll
    for (int u = 0; u < kBatchOf<T>; ++u) {
        const int64_t i = base + (int64_t)u * T + threadIdx.x;
        d[u] = u32x4{0u, 0u, 0u, 0u};
        if constexpr (PROTO == 1) {
            // payload chunk i % 16 of the pair (lane 15 has none); words past
            // the step belong to lines this step does not write
            if (i < g.items && (i & 15) < 15)
                d[u] = quad_at(a, pair_chunk_word(g, i));
        } else if (i < g.items) {
            const int64_t w = item_word<PROTO>(g, i);
            if (item_count<PROTO>(g, i) == 2) {
                const u32x2 p = pair_at(a, w);
                d[u] = u32x4{p.x, p.y, 0u, 0u};
            } else {
                d[u] = quad_at(a, w);
            }
        }
    }
}

template <int CTRL>
__device__ __forceinline__ uint32_t row_shift(uint32_t v)
{
    // lanes whose source lies outside their row of 16 receive 0
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kRowShr1 = 0x111;   // lane c receives lane c - 1
constexpr int kRowShl1 = 0x101;   // lane c receives lane c + 1

template <int T, int PROTO>
__device__ __forceinline__ void store_ring(const Step &g, int64_t base, const u32x4 d[kBatchOf<T>])
{
#pragma unroll
    for (int u = 0; u < kBatchOf<T>; ++u) {
        const int64_t i = base + (int64_t)u * T + threadIdx.x;
        // LL128: the second line's chunk c - 8 is the high half of payload
        // chunk c - 1 and the low half of payload chunk c (every lane takes
        // part in the shift)
        uint32_t hz = 0u, hw = 0u;
        if (PROTO == 1) {
            hz = row_shift<kRowShr1>(d[u].z);
            hw = row_shift<kRowShr1>(d[u].w);
        }
        if (i >= g.items)
            continue;
        const uint32_t p = ring_offset<PROTO>(i);
        if (PROTO == 0) {
            const uint32_t f = (uint32_t)(g.k + 1);
            store16_sys(g.slot, p, u32x4{d[u].x, f, d[u].y, f});
        } else if (PROTO == 1) {
            // every line goes out whole, chunk 7 with the step's flag, except
            // the batch's first line (chunk 7 of the row's line A), whose flag
            // word is zero (no step's flag is 0) until the batch is
            // acknowledged
            const int c = (int)(i & 15);
            const uint64_t f = g.k + 1;
            const bool first_line = (i >> 3) == (base >> 3);
            const uint32_t flo = first_line ? 0u : (uint32_t)f;
            const uint32_t fhi = first_line ? 0u : (uint32_t)(f >> 32);
            store16_sys(g.slot, p, c < 7    ? d[u]
                           : c == 7 ? u32x4{d[u].x, d[u].y, flo, fhi}
                           : c < 15 ? u32x4{hz, hw, d[u].x, d[u].y}
                                    : u32x4{hz, hw, (uint32_t)f, (uint32_t)(f >> 32)});
        } else if (4 * i + 4 <= g.words) {
            store16_sys(g.slot, p, d[u]);
        } else {
            for (int e = 0; e < 4; ++e)
                if (4 * i + e < g.words)
                    store4_sys(g.slot, p + 4 * e, d[u][e]);
        }
    }
}

template <int T, int PROTO>
__device__ __forceinline__ void load_ring(const Step &g, int64_t base, u32x4 v[kBatchOf<T>])
{
#pragma unroll
    for (int u = 0; u < kBatchOf<T>; ++u) {
        const int64_t i = base + (int64_t)u * T + threadIdx.x;
        v[u] = i < g.items ? load16_sys(g.slot, ring_offset<PROTO>(i)) : u32x4{0u, 0u, 0u, 0u};
    }
}

// LL128 delivery: lane c < 15 of a line pair owns payload chunk c; the step's
// payload words past the last line of the step are not written.
__device__ __forceinline__ int pair_chunk_count(const Step &g, int64_t q)
{
    const int64_t rem = g.words - (60 * (q >> 4) + 4 * (q & 15));
    return (q & 15) == 15 || rem <= 0 ? 0 : rem < 4 ? (int)rem : 4;
}

template <int T, int PROTO, bool LOCAL>
__device__ __forceinline__ void load_local(const StreamArgs &a, const Step &g, int64_t base,
                                           u32x4 lv[kBatchOf<T>])
{
#pragma unroll
    for (int u = 0; u < kBatchOf<T>; ++u) {
        const int64_t i = base + (int64_t)u * T + threadIdx.x;
        lv[u] = u32x4{0u, 0u, 0u, 0u};
        if (!LOCAL || i >= g.items)
            continue;
        if constexpr (PROTO == 1) {
            if (pair_chunk_count(g, i) > 0)
                lv[u] = local_at(a, pair_chunk_word(g, i), 4);
        } else {
            lv[u] = local_at(a, item_word<PROTO>(g, i), item_count<PROTO>(g, i));
        }
    }
}

template <int T, int PROTO, bool LOCAL>
__device__ __forceinline__ void deliver_batch(const StreamArgs &a, const Step &g, int64_t base,
                                              const u32x4 v[kBatchOf<T>], const u32x4 lv[kBatchOf<T>])
{
#pragma unroll
    for (int u = 0; u < kBatchOf<T>; ++u) {
        const int64_t i = base + (int64_t)u * T + threadIdx.x;
        if constexpr (PROTO == 1) {
            // payload chunk c: line A's chunk c (c < 7); line A's chunk 7
            // data then line B's chunk 0 low half (c == 7); line B's chunk
            // c - 8 high half then chunk c - 7 low half (8 <= c < 15)
            const uint32_t nx = row_shift<kRowShl1>(v[u].x);
            const uint32_t ny = row_shift<kRowShl1>(v[u].y);
            if (i >= g.items)
                continue;
            const int c = (int)(i & 15);
            const int cnt = pair_chunk_count(g, i);
            if (cnt == 0)
                continue;
            const u32x4 x = c < 7 ? v[u] : c == 7 ? u32x4{v[u].x, v[u].y, nx, ny}
                                                  : u32x4{v[u].z, v[u].w, nx, ny};
            deliver<LOCAL>(a, pair_chunk_word(g, i), cnt, x, lv[u]);
        } else {
            if (i >= g.items)
                continue;
            const u32x4 x = PROTO == 0 ? u32x4{v[u].x, v[u].z, 0u, 0u} : v[u];
            deliver<LOCAL>(a, item_word<PROTO>(g, i), item_count<PROTO>(g, i), x, lv[u]);
        }
    }
}

// The batch's loads have returned (their registers are read by an empty
// asm statement, so the compiler waits for exactly these loads).
template <int T>
__device__ __forceinline__ void loads_returned(const u32x4 v[kBatchOf<T>])
{
#pragma unroll
    for (int u = 0; u < kBatchOf<T>; ++u)
        asm volatile("" ::"v"(v[u]));
}

// ---------------------------------------------------------------------------
// Producer: the batches of the channel's steps in order, each batch's source
// loads issued before the previous batch's ring stores.
// Pair `pair` of channel c; its counters are head[p] and tail[p].
template <int T, int PROTO>
__device__ void produce(const StreamArgs &a, int c, int pair, int p, int64_t s0, int64_t steps,
                        uint64_t first, Shared *sh)
{
    uint8_t *ring = a.fifo + (int64_t)c * 8 * a.wire_bytes;
    uint64_t head_seen = first;      // the consumer has taken every step before `first`
    Cursor cur;
    if (!start<PROTO>(a, ring, s0, first, steps, pair, &cur))
        return;
    u32x4 d[kBatchOf<T>];
    load_src<T, PROTO>(a, cur.g, cur.base, d);
    for (;;) {
        Cursor nxt;
        const bool more = advance<PROTO>(a, ring, s0, first, steps, pair, cur, &nxt);
        u32x4 nd[kBatchOf<T>];
        if (more)
            load_src<T, PROTO>(a, nxt.g, nxt.base, nd);
        if (cur.base == cur.g.lo && cur.j >= 8 &&
            !wait_counter(a, sh, a.head + p, cur.g.k - 7, &head_seen))
            return;
        store_ring<T, PROTO>(cur.g, cur.base, d);
        if (PROTO == 1) {
            // every line of the batch, flags included, is acknowledged
            // before the flag of its first line
            drain_memory();
            __syncthreads();
            const uint64_t f = cur.g.k + 1;
            if (threadIdx.x == 0)
                store8_sys(cur.g.slot, (uint32_t)(128 * (cur.base / 8) + 120),
                           u32x2{(uint32_t)f, (uint32_t)(f >> 32)});
        }
        if (PROTO == 2 && nxt.j != cur.j) {
            // the step's data is acknowledged before its tail
            drain_memory();
            __syncthreads();
            if (threadIdx.x == 0)
                store_counter(a.tail + p, cur.g.k + 1);
        }
        if (!more)
            return;
        cur = nxt;
#pragma unroll
        for (int u = 0; u < kBatchOf<T>; ++u)
            d[u] = nd[u];
    }
}

// ---------------------------------------------------------------------------
// Consumer side.  A step is closed once every lane's loads of it have
// returned: the workgroup agrees on success and lane 0 publishes head = k + 1,
// before the step's last batch is delivered from registers.  A failed wait
// is counted where it happens.  Returns false once the launch must stop.
__device__ bool close_step(const StreamArgs &a, int p, uint64_t k, bool failed)
{
    const bool any_failed = __syncthreads_or(failed ? 1 : 0) != 0;
    if (threadIdx.x == 0 && !any_failed)
        store_counter(a.head + p, k + 1);
    return !any_failed;
}

// Wait until every item of a batch is valid(u, item) (bounded; gives up early once
// any wait of the launch has failed).  While items are missing, one lane of
// the wavefront (the first still waiting) polls the earliest of its missing
// items, since the producer stores a lane's items in that order and the
// producer's lanes write together; a miss backs off briefly.  Once that item
// is valid, every waiting lane reads its missing items again.  One poll per
// wavefront instead of one per lane keeps the polls from adding traffic.
template <int T, bool BY_SLOT = false, typename Offset, typename Valid>
__device__ bool poll_batch(const StreamArgs &a, u32x4 v[kBatchOf<T>], bool ok[kBatchOf<T>], Rsrc slot,
                           Offset off, Valid valid)
{
    bool all = true;
#pragma unroll
    for (int u = 0; u < kBatchOf<T>; ++u)
        all = all && ok[u];
    for (uint32_t s = 0; !all && s < a.max_spins; ++s) {
        respin();
        if (s % kAbortCheck == 0 && aborted(a.errors))
            break;
        // the polling lane looks at its earliest missing item
        const int first = __builtin_amdgcn_readfirstlane((int)threadIdx.x);
        int hit = 0;
        if constexpr (BY_SLOT) {
            // callbacks that read per-slot arrays are called with constant
            // slots only, so those arrays stay in registers
            if ((int)threadIdx.x == first) {
                uint32_t o = 0;
                int lead = -1;
#pragma unroll
                for (int u = kBatchOf<T> - 1; u >= 0; --u) {
                    if (!ok[u]) {
                        o = off(u);
                        lead = u;
                    }
                }
                const u32x4 x = load16_sys(slot, o);
                bool h = false;
#pragma unroll
                for (int u = 0; u < kBatchOf<T>; ++u)
                    if (u == lead)
                        h = valid(u, x);
                hit = h ? 1 : 0;
            }
        } else {
            int lead = 0;
#pragma unroll
            for (int u = kBatchOf<T> - 1; u >= 0; --u)
                if (!ok[u])
                    lead = u;
            if ((int)threadIdx.x == first)
                hit = valid(lead, load16_sys(slot, off(lead))) ? 1 : 0;
        }
        if (!__builtin_amdgcn_readfirstlane(hit)) {
            __builtin_amdgcn_s_sleep(1);
            continue;
        }
#pragma unroll
        for (int u = 0; u < kBatchOf<T>; ++u)
            if (!ok[u])
                v[u] = load16_sys(slot, off(u));
        all = true;
#pragma unroll
        for (int u = 0; u < kBatchOf<T>; ++u) {
            ok[u] = ok[u] || valid(u, v[u]);
            all = all && ok[u];
        }
    }
    if (!all)
        atomicAdd(a.errors, 1u);
    return all;
}

// LL: every line validates itself, so the next batch (also of the next step)
// is loaded before this batch is delivered; lines not yet written are
// re-polled.
template <int T, bool LOCAL>
__device__ void consume_ll(const StreamArgs &a, int c, int pair, int p, int64_t s0, int64_t steps,
                           uint64_t first)
{
    uint8_t *ring = a.fifo + (int64_t)c * 8 * a.wire_bytes;
    Cursor cur;
    if (!start<0>(a, ring, s0, first, steps, pair, &cur))
        return;
    u32x4 v[kBatchOf<T>], lv[kBatchOf<T>];
    load_ring<T, 0>(cur.g, cur.base, v);
    load_local<T, 0, LOCAL>(a, cur.g, cur.base, lv);
    bool failed = false;
    for (;;) {
        const uint32_t flag = (uint32_t)(cur.g.k + 1);
        const int64_t i0 = cur.base + threadIdx.x;
        auto valid = [&](u32x4 x) { return x.y == flag && x.w == flag; };
        bool ok[kBatchOf<T>];
        bool ahead = true;       // every line was there on the first look
#pragma unroll
        for (int u = 0; u < kBatchOf<T>; ++u) {
            ok[u] = i0 + (int64_t)u * T >= cur.g.items || valid(v[u]);
            ahead = ahead && ok[u];
        }
        if (!failed)
            failed = !poll_batch<T>(
                a, v, ok, cur.g.slot,
                [&](int u) { return (uint32_t)(16 * (i0 + (int64_t)u * T)); },
                [&](int, u32x4 x) { return valid(x); });
        Cursor nxt;
        const bool more = advance<0>(a, ring, s0, first, steps, pair, cur, &nxt);
        loads_returned<T>(v);
        if (nxt.j != cur.j && !close_step(a, p, cur.g.k, failed))
            return;
        // With the producer ahead, the next batch is loaded before this one
        // is delivered; a lane that had to wait delivers first, so that its
        // next look does not find lines not yet written.
        u32x4 nv[kBatchOf<T>], nlv[kBatchOf<T>];
        if (more && ahead) {
            load_ring<T, 0>(nxt.g, nxt.base, nv);
            load_local<T, 0, LOCAL>(a, nxt.g, nxt.base, nlv);
        }
        if (!failed)
            deliver_batch<T, 0, LOCAL>(a, cur.g, cur.base, v, lv);
        if (more && !ahead) {
            load_ring<T, 0>(nxt.g, nxt.base, nv);
            load_local<T, 0, LOCAL>(a, nxt.g, nxt.base, nlv);
        }
        if (!more)
            return;
        cur = nxt;
#pragma unroll
        for (int u = 0; u < kBatchOf<T>; ++u) {
            v[u] = nv[u];
            lv[u] = nlv[u];
        }
    }
}

// ---------------------------------------------------------------------------
// LL with whole steps per batch.  With several pairs per channel a pair's
// slice of NCCL's 32 KiB LL step is 512-2,048 lines, half a batch or less,
// so a batch kept inside one step left lanes one or a few lines in flight
// per round trip.  When the host sets batch_steps S > 1, a batch is S
// consecutive whole steps of the pair instead: lane slot v = u * T + lane
// carries line v mod L of the batch's step v / L (fifo_batch_slot; L is the
// pair's slice of a full step), the same slot every batch.  LL lines
// validate themselves, so the protocol is unchanged: the producer waits for
// the head that frees the slot of the batch's last step (with S <= 4 it can
// work a batch ahead of its consumer), the consumer re-polls missing lines
// and publishes the head once per batch.  A batch's lines lie in several
// ring slots, so these paths address the channel's whole ring through one
// descriptor (the host sets S > 1 only for rings under 2 GiB).
template <int T>
struct LLSteps {
    Rsrc ring;                      // the channel's 8 slots
    int64_t lo;                     // first line of the pair's slice
    uint32_t len_full, len_last;    // lines of the pair's slice of a full step and of
                                    // the channel's last step
    int64_t last;                   // local index of the channel's last step
    int64_t steps;                  // steps that give the pair a slice
    uint32_t slot[kBatchOf<T>];     // per lane slot: step within the batch << 16 | line
                                    // within the slice (a slice is under 2^16 lines
                                    // whenever a batch takes two steps or more)
};

// False when the pair has nothing to move (no steps, or its slice of the
// channel's only step is empty).
template <int T>
__device__ __forceinline__ bool ll_steps_setup(const StreamArgs &a, int c, int pair, int64_t s0,
                                               int64_t steps, LLSteps<T> *m)
{
    m->ring = slot_rsrc(a.fifo + (int64_t)c * 8 * a.wire_bytes, 8 * a.wire_bytes);
    int64_t hi_full = 0;
    fifo_slice_at(a.span, a.step_bytes / 8, pair, &m->lo, &hi_full);
    const int64_t len = hi_full - m->lo;
    m->len_full = len > 0 ? (uint32_t)len : 0u;
    m->len_last = 0;
    m->last = steps - 1;
    m->steps = steps;
    if (steps > 0) {
        const int64_t left = 4 * a.n - (s0 + steps - 1) * a.step_bytes;
        const int64_t bytes = left < a.step_bytes ? left : a.step_bytes;
        int64_t lo_last = 0, hi_last = 0;
        fifo_slice_at(a.span, items_of<0>(bytes, bytes / 4), pair, &lo_last, &hi_last);
        if (hi_last > lo_last)
            m->len_last = (uint32_t)(hi_last - lo_last);   // lo_last == lo then
        else
            m->steps = steps - 1;   // only a channel's last step can leave a pair no slice
    }
    if (len <= 0)
        m->steps = 0;
#pragma unroll
    for (int u = 0; u < kBatchOf<T>; ++u) {
        int step = kMaxBatchSteps;
        uint32_t line = 0;
        if (len > 0)
            fifo_batch_slot((uint32_t)(u * T) + threadIdx.x, (uint32_t)len, &step, &line);
        m->slot[u] = (uint32_t)(step < kMaxBatchSteps ? step : kMaxBatchSteps) << 16 | line;
    }
    return m->steps > 0;
}

// One batch, the same for every lane: what the lane slots need from it.
struct LLBatch {
    int n_in;          // steps in the batch
    int dj_last;       // the channel's last step as a step of the batch, or -1
    uint32_t k0;       // low 32 bits of the batch's first ring step
    int64_t word0;     // payload word of line lo of the batch's first step
};
template <int T>
__device__ __forceinline__ LLBatch ll_batch(const StreamArgs &a, const LLSteps<T> &m, int64_t s0,
                                            uint64_t first, int64_t j0)
{
    LLBatch b;
    b.n_in = m.steps - j0 < a.batch_steps ? (int)(m.steps - j0) : a.batch_steps;
    b.dj_last = m.last - j0 < b.n_in ? (int)(m.last - j0) : -1;
    b.k0 = (uint32_t)(first + (uint64_t)j0);
    b.word0 = (s0 + j0) * (a.step_bytes / 4) + 2 * m.lo;
    return b;
}
template <int T>
__device__ __forceinline__ bool ll_has(const LLSteps<T> &m, const LLBatch &b, int u)
{
    const int dj = (int)(m.slot[u] >> 16);
    const uint32_t line = m.slot[u] & 0xFFFFu;
    return dj < b.n_in && line < (dj == b.dj_last ? m.len_last : m.len_full);
}
// Lane parts in 32 bits: a step is at most 2^30 bytes and dj <= 3.
template <int T>
__device__ __forceinline__ int64_t ll_word(const StreamArgs &a, const LLSteps<T> &m,
                                           const LLBatch &b, int u)
{
    return b.word0 + (int64_t)((m.slot[u] >> 16) * (uint32_t)(a.step_bytes / 4) +
                               2u * (m.slot[u] & 0xFFFFu));
}
template <int T>
__device__ __forceinline__ uint32_t ll_off(const StreamArgs &a, const LLSteps<T> &m,
                                           const LLBatch &b, int u)
{
    return ((b.k0 + (m.slot[u] >> 16)) & 7u) * (uint32_t)a.wire_bytes +
           16u * ((uint32_t)m.lo + (m.slot[u] & 0xFFFFu));
}
template <int T>
__device__ __forceinline__ uint32_t ll_flag(const LLSteps<T> &m, const LLBatch &b, int u)
{
    return b.k0 + (m.slot[u] >> 16) + 1u;
}

template <int T>
__device__ __forceinline__ void ll_steps_load_src(const StreamArgs &a, const LLSteps<T> &m,
                                                  const LLBatch &b, u32x4 d[kBatchOf<T>])
{
#pragma unroll
    for (int u = 0; u < kBatchOf<T>; ++u) {
        d[u] = u32x4{0u, 0u, 0u, 0u};
        if (ll_has(m, b, u)) {
            const u32x2 p = pair_at(a, ll_word(a, m, b, u));
            d[u] = u32x4{p.x, p.y, 0u, 0u};
        }
    }
}

template <int T, bool LOCAL>
__device__ __forceinline__ void ll_steps_load(const StreamArgs &a, const LLSteps<T> &m,
                                              const LLBatch &b, u32x4 v[kBatchOf<T>],
                                              u32x4 lv[kBatchOf<T>])
{
#pragma unroll
    for (int u = 0; u < kBatchOf<T>; ++u) {
        const bool has = ll_has(m, b, u);
        v[u] = has ? load16_sys(m.ring, ll_off(a, m, b, u)) : u32x4{0u, 0u, 0u, 0u};
        lv[u] = LOCAL && has ? local_at(a, ll_word(a, m, b, u), 2) : u32x4{0u, 0u, 0u, 0u};
    }
}

template <int T>
__device__ void produce_ll_steps(const StreamArgs &a, int c, int pair, int p, int64_t s0,
                                 int64_t steps, uint64_t first, Shared *sh)
{
    LLSteps<T> m;
    if (!ll_steps_setup<T>(a, c, pair, s0, steps, &m))
        return;
    const int S = a.batch_steps;
    uint64_t head_seen = first;      // the consumer has taken every step before `first`
    LLBatch b = ll_batch<T>(a, m, s0, first, 0);
    u32x4 d[kBatchOf<T>];
    ll_steps_load_src<T>(a, m, b, d);
    for (int64_t j0 = 0;; j0 += S) {
        const int64_t nj = j0 + S;
        const bool more = nj < m.steps;
        const LLBatch nb = ll_batch<T>(a, m, s0, first, nj);
        u32x4 nd[kBatchOf<T>];
        if (more)
            ll_steps_load_src<T>(a, m, nb, nd);
        const int64_t jl = j0 + b.n_in - 1;   // the batch's last step
        if (jl >= 8 && !wait_counter(a, sh, a.head + p, first + (uint64_t)jl - 7, &head_seen))
            return;
#pragma unroll
        for (int u = 0; u < kBatchOf<T>; ++u) {
            if (!ll_has(m, b, u))
                continue;
            const uint32_t f = ll_flag(m, b, u);
            store16_sys(m.ring, ll_off(a, m, b, u), u32x4{d[u].x, f, d[u].y, f});
        }
        if (!more)
            return;
        b = nb;
#pragma unroll
        for (int u = 0; u < kBatchOf<T>; ++u)
            d[u] = nd[u];
    }
}

// Before a consumer's first batch.  Its producer starts in the same launch
// at the same moment, so a first look at the batch would find its lines not
// yet written and read them all twice.  Instead the first lane of each
// wavefront polls the wavefront's last line slot of the batch (the last the
// producer's wavefront stores) until it holds the batch's flags, then the
// wavefront reads the batch (bounded; a batch whose last slot carries no
// line, or a wait that runs out, goes on to the usual validation).
template <int T>
__device__ __forceinline__ void ll_await_last_line(const StreamArgs &a, const LLSteps<T> &m,
                                                   const LLBatch &b)
{
    constexpr int u = kBatchOf<T> - 1;
    const bool has = ll_has(m, b, u);
    const uint32_t off = ll_off(a, m, b, u), f = ll_flag(m, b, u);
    const int lead = __builtin_amdgcn_readfirstlane((int)threadIdx.x);
    for (uint32_t s = 0; s < a.max_spins; ++s) {
        respin();
        int hit = 1;
        if ((int)threadIdx.x == lead && has) {
            const u32x4 x = load16_sys(m.ring, off);
            hit = x.y == f && x.w == f ? 1 : 0;
        }
        if (__builtin_amdgcn_readfirstlane(hit))
            break;
        if (s % kAbortCheck == 0 && aborted(a.errors))
            break;
        __builtin_amdgcn_s_sleep(1);
    }
}

template <int T, bool LOCAL>
__device__ void consume_ll_steps(const StreamArgs &a, int c, int pair, int p, int64_t s0,
                                 int64_t steps, uint64_t first)
{
    LLSteps<T> m;
    if (!ll_steps_setup<T>(a, c, pair, s0, steps, &m))
        return;
    const int S = a.batch_steps;
    LLBatch b = ll_batch<T>(a, m, s0, first, 0);
    u32x4 v[kBatchOf<T>], lv[kBatchOf<T>];
    ll_await_last_line<T>(a, m, b);
    ll_steps_load<T, LOCAL>(a, m, b, v, lv);
    bool failed = false;
    for (int64_t j0 = 0;; j0 += S) {
        auto valid = [&](int u, u32x4 x) {
            const uint32_t f = ll_flag(m, b, u);
            return x.y == f && x.w == f;
        };
        bool ok[kBatchOf<T>];
        bool ahead = true;       // every line was there on the first look
#pragma unroll
        for (int u = 0; u < kBatchOf<T>; ++u) {
            ok[u] = !ll_has(m, b, u) || valid(u, v[u]);
            ahead = ahead && ok[u];
        }
        if (!failed)
            failed = !poll_batch<T, true>(
                a, v, ok, m.ring, [&](int u) { return ll_off(a, m, b, u); }, valid);
        const int64_t nj = j0 + S;
        const bool more = nj < m.steps;
        loads_returned<T>(v);
        if (!close_step(a, p, first + (uint64_t)(j0 + b.n_in - 1), failed))
            return;
        const LLBatch nb = ll_batch<T>(a, m, s0, first, nj);
        // With the producer ahead, 1,024-lane workgroups load the next
        // batch before delivering this one; 512-lane ones (twice the lines
        // per lane) always deliver first, which keeps them in their
        // registers.
        const bool load_first = T == kWideThreads && ahead;
        u32x4 nv[kBatchOf<T>], nlv[kBatchOf<T>];
        if (more && load_first)
            ll_steps_load<T, LOCAL>(a, m, nb, nv, nlv);
        if (!failed) {
#pragma unroll
            for (int u = 0; u < kBatchOf<T>; ++u)
                if (ll_has(m, b, u))
                    deliver<LOCAL>(a, ll_word(a, m, b, u), 2, u32x4{v[u].x, v[u].z, 0u, 0u},
                                   lv[u]);
        }
        if (more && !load_first)
            ll_steps_load<T, LOCAL>(a, m, nb, nv, nlv);
        if (!more)
            return;
        b = nb;
#pragma unroll
        for (int u = 0; u < kBatchOf<T>; ++u) {
            v[u] = nv[u];
            lv[u] = nlv[u];
        }
    }
}

// Lane 0 waits for a 64-bit flag, starting from a value it read earlier.
__device__ bool wait_flag64(const StreamArgs &a, Shared *sh, Rsrc slot, uint32_t off,
                            uint64_t want, uint64_t pre)
{
    bool first = true;
    return wait_lane0(
        a, sh, nullptr,
        [&] {
            if (first) {
                first = false;
                return pre;
            }
            const u32x2 f = load8_sys(slot, off);
            return (uint64_t)f.x | ((uint64_t)f.y << 32);
        },
        [&](uint64_t f) { return f == want; });
}
__device__ __forceinline__ uint64_t read_flag64(Rsrc slot, uint32_t off)
{
    const u32x2 f = load8_sys(slot, off);
    return (uint64_t)f.x | ((uint64_t)f.y << 32);
}

// LL128: a batch's data was acknowledged before any of its flags, so once
// the flag of the batch's first line is seen the whole batch is read, each
// line's flag checked, and chunk 7 of lines whose flag has not arrived yet
// re-read.  Lane 0 reads the next batch's first flag together with this
// batch's data, and the next batch is loaded before this one is delivered.
template <int T, bool LOCAL>
__device__ void consume_ll128(const StreamArgs &a, int c, int pair, int p, int64_t s0,
                              int64_t steps, uint64_t first, Shared *sh)
{
    uint8_t *ring = a.fifo + (int64_t)c * 8 * a.wire_bytes;
    auto flag_at = [](int64_t base) { return (uint32_t)(128 * (base >> 3) + 120); };
    Cursor cur;
    if (!start<1>(a, ring, s0, first, steps, pair, &cur))
        return;
    uint64_t pre = threadIdx.x == 0 ? read_flag64(cur.g.slot, flag_at(cur.base)) : 0;
    if (!wait_flag64(a, sh, cur.g.slot, flag_at(cur.base), cur.g.k + 1, pre))
        return;
    u32x4 v[kBatchOf<T>], lv[kBatchOf<T>];
    load_ring<T, 1>(cur.g, cur.base, v);
    load_local<T, 1, LOCAL>(a, cur.g, cur.base, lv);
    bool failed = false;
    for (;;) {
        Cursor nxt;
        const bool more = advance<1>(a, ring, s0, first, steps, pair, cur, &nxt);
        if (threadIdx.x == 0 && more)
            pre = read_flag64(nxt.g.slot, flag_at(nxt.base));
        const uint64_t flag = cur.g.k + 1;
        const uint32_t flo = (uint32_t)flag, fhi = (uint32_t)(flag >> 32);
        const int64_t q0 = cur.base + threadIdx.x;
        auto valid = [&](u32x4 x) { return x.z == flo && x.w == fhi; };
        bool ok[kBatchOf<T>];
#pragma unroll
        for (int u = 0; u < kBatchOf<T>; ++u) {
            const int64_t q = q0 + (int64_t)u * T;
            ok[u] = q >= cur.g.items || (q & 7) != 7 || valid(v[u]);
        }
        // only flag chunks can be missing; a re-read takes the line's chunk 7
        if (!failed)
            failed = !poll_batch<T>(
                a, v, ok, cur.g.slot,
                [&](int u) {
                    const int64_t q = q0 + (int64_t)u * T;
                    return (uint32_t)(128 * (q >> 3) + 112);
                },
                [&](int, u32x4 x) { return valid(x); });
        loads_returned<T>(v);
        if (nxt.j != cur.j && !close_step(a, p, cur.g.k, failed))
            return;
        if (more && !wait_flag64(a, sh, nxt.g.slot, flag_at(nxt.base), nxt.g.k + 1, pre))
            return;
        u32x4 nv[kBatchOf<T>], nlv[kBatchOf<T>];
        if (more) {
            load_ring<T, 1>(nxt.g, nxt.base, nv);
            load_local<T, 1, LOCAL>(a, nxt.g, nxt.base, nlv);
        }
        if (!failed)
            deliver_batch<T, 1, LOCAL>(a, cur.g, cur.base, v, lv);
        if (!more)
            return;
        cur = nxt;
#pragma unroll
        for (int u = 0; u < kBatchOf<T>; ++u) {
            v[u] = nv[u];
            lv[u] = nlv[u];
        }
    }
}

// Simple: a step is read only after its tail; within a step (and across a
// step boundary when the tail already covers the next step) the next batch
// is loaded before this one is delivered.
template <int T, bool LOCAL>
__device__ void consume_simple(const StreamArgs &a, int c, int pair, int p, int64_t s0,
                               int64_t steps, uint64_t first, Shared *sh)
{
    uint8_t *ring = a.fifo + (int64_t)c * 8 * a.wire_bytes;
    uint64_t tail_seen = first;      // the producer has written every step before `first`
    Cursor cur;
    if (!start<2>(a, ring, s0, first, steps, pair, &cur))
        return;
    if (!wait_counter(a, sh, a.tail + p, cur.g.k + 1, &tail_seen))
        return;
    u32x4 v[kBatchOf<T>], lv[kBatchOf<T>];
    load_ring<T, 2>(cur.g, cur.base, v);
    load_local<T, 2, LOCAL>(a, cur.g, cur.base, lv);
    for (;;) {
        Cursor nxt;
        const bool more = advance<2>(a, ring, s0, first, steps, pair, cur, &nxt);
        loads_returned<T>(v);
        if (nxt.j != cur.j && !close_step(a, p, cur.g.k, false))
            return;
        if (more && nxt.j != cur.j &&
            !wait_counter(a, sh, a.tail + p, nxt.g.k + 1, &tail_seen))
            return;
        u32x4 nv[kBatchOf<T>], nlv[kBatchOf<T>];
        if (more) {
            load_ring<T, 2>(nxt.g, nxt.base, nv);
            load_local<T, 2, LOCAL>(a, nxt.g, nxt.base, nlv);
        }
        deliver_batch<T, 2, LOCAL>(a, cur.g, cur.base, v, lv);
        if (!more)
            return;
        cur = nxt;
#pragma unroll
        for (int u = 0; u < kBatchOf<T>; ++u) {
            v[u] = nv[u];
            lv[u] = nlv[u];
        }
    }
}

// Blocks [0, channels * pairs) produce, the next channels * pairs consume;
// block q of either half is pair q mod pairs of channel q / pairs.  Without
// a local addend the kernel keeps to 128 VGPRs (4 wavefronts per SIMD), so
// two workgroups fit on a CU and up to 256 channels can run at once; with one
// it has two wavefronts per SIMD.  STEPS (LL only) selects the whole-step
// batch paths, a kernel of its own so that the one-step-batch kernel keeps
// its registers and code.
template <int T, int PROTO, bool LOCAL, bool STEPS = false>
__global__ __launch_bounds__(T, T == kWideThreads || !LOCAL ? 4 : 2) void stream_kernel(StreamArgs a)
{
    __shared__ Shared sh;
    const int b = blockIdx.x;
    const int pairs_total = a.channels * a.pairs;
    const bool producer = b < pairs_total;
    const int p = producer ? b : b - pairs_total;
    const int c = p / a.pairs, pair = p % a.pairs;
    // Every block reads the stored first step before its channel moves, and
    // the last consumer advances it only after every step of every channel
    // has been written and read; a channel with no steps may read either
    // value and uses neither.
    if (threadIdx.x == 0)
        sh.value = a.from_state ? __hip_atomic_load(a.state, __ATOMIC_ACQUIRE,
                                                    __HIP_MEMORY_SCOPE_AGENT)
                                : a.first_step;
    __syncthreads();
    const uint64_t first = uniform64(sh.value);
    __syncthreads();
    const int64_t s0 = (int64_t)c * a.total_steps / a.channels;
    const int64_t s1 = (int64_t)(c + 1) * a.total_steps / a.channels;
    if (producer) {
        if constexpr (PROTO == 0 && STEPS)
            produce_ll_steps<T>(a, c, pair, p, s0, s1 - s0, first, &sh);
        else
            produce<T, PROTO>(a, c, pair, p, s0, s1 - s0, first, &sh);
        return;
    }
    if constexpr (PROTO == 0 && STEPS)
        consume_ll_steps<T, LOCAL>(a, c, pair, p, s0, s1 - s0, first);
    else if constexpr (PROTO == 0)
        consume_ll<T, LOCAL>(a, c, pair, p, s0, s1 - s0, first);
    else if (PROTO == 1)
        consume_ll128<T, LOCAL>(a, c, pair, p, s0, s1 - s0, first, &sh);
    else
        consume_simple<T, LOCAL>(a, c, pair, p, s0, s1 - s0, first, &sh);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint64_t done = __hip_atomic_fetch_add(a.state + 1, (uint64_t)1, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done == (uint64_t)pairs_total - 1) {
            __hip_atomic_store(a.state + 1, (uint64_t)0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.state, first + (uint64_t)a.steps_per_channel, __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int T>
static const void *stream_fn_t(int proto, bool local, bool steps)
{
    if (proto == 0 && steps)
        return local ? reinterpret_cast<const void *>(&stream_kernel<T, 0, true, true>)
                     : reinterpret_cast<const void *>(&stream_kernel<T, 0, false, true>);
    if (local)
        return proto == 0   ? reinterpret_cast<const void *>(&stream_kernel<T, 0, true>)
               : proto == 1 ? reinterpret_cast<const void *>(&stream_kernel<T, 1, true>)
                            : reinterpret_cast<const void *>(&stream_kernel<T, 2, true>);
    return proto == 0   ? reinterpret_cast<const void *>(&stream_kernel<T, 0, false>)
           : proto == 1 ? reinterpret_cast<const void *>(&stream_kernel<T, 1, false>)
                        : reinterpret_cast<const void *>(&stream_kernel<T, 2, false>);
}

static const void *stream_fn(int proto, bool local, bool wide, bool steps)
{
    return wide ? stream_fn_t<kWideThreads>(proto, local, steps)
                : stream_fn_t<kNarrowThreads>(proto, local, steps);
}

// Workgroups of the kernel the call may launch that fit on the device at
// once; for LL the smaller count of its two kernels, since the pair count
// that depends on it also decides which of them runs.
hipError_t fifo_stream_resident_workgroups(int proto, bool local, bool wide, int *workgroups)
{
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int lanes = wide ? kWideThreads : kNarrowThreads;
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stream_fn(proto, local, wide, false),
                                                         lanes, 0);
    if (e == hipSuccess && proto == 0) {
        int steps_per_cu = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&steps_per_cu,
                                                         stream_fn(proto, local, wide, true), lanes, 0);
        if (steps_per_cu < per_cu)
            per_cu = steps_per_cu;
    }
    *workgroups = e == hipSuccess ? cus * per_cu : 0;
    return e;
}

hipError_t launch_fifo_stream(int proto, const float *src, const float *local, float *out,
                              int64_t n, void *fifo, uint64_t *counters, int channels,
                              int64_t step_bytes, int64_t wire_bytes, uint64_t first_step,
                              bool from_state, uint32_t max_spins, uint32_t *errors,
                              bool wide, int pairs, hipStream_t s)
{
    StreamArgs a;
    a.src = reinterpret_cast<const uint32_t *>(src);
    a.local = local;
    a.out = out;
    a.n = n;
    a.fifo = static_cast<uint8_t *>(fifo);
    a.head = counters;
    a.tail = counters + (int64_t)channels * kMaxPairs;
    a.state = counters + 2 * (int64_t)channels * kMaxPairs;
    a.errors = errors;
    a.step_bytes = step_bytes;
    a.wire_bytes = wire_bytes;
    a.total_steps = (4 * n + step_bytes - 1) / step_bytes;
    a.steps_per_channel = (a.total_steps + channels - 1) / channels;
    a.channels = channels;
    a.pairs = pairs;
    a.span = fifo_span(fifo_full_items(proto, step_bytes), proto == 1 ? 16 : 1, pairs);
    a.batch_steps = fifo_plan_batch_steps(proto, step_bytes, n, channels, pairs);
    a.from_state = from_state ? 1 : 0;
    a.first_step = first_step;
    a.max_spins = max_spins;
    void *args[] = {&a};
    return hipLaunchKernel(stream_fn(proto, local != nullptr, wide, a.batch_steps > 1),
                           dim3(2 * channels * pairs),
                           dim3(wide ? kWideThreads : kNarrowThreads), args, 0, s);
}

}  // namespace ar
