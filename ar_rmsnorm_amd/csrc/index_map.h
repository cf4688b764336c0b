// Index maps as plain C++17 constexpr functions: the block and lane map of
// the two-stage reduce, and the slices that the producer/consumer pairs of a
// streaming channel own.  HIP device code may call constexpr functions, so
// the kernels use exactly these; the host can compile them with any C++17
// compiler, so every (block, lane) of a launch and every slice of a ring can
// be enumerated and checked on a CPU.  No HIP header is needed here.
//
// Source (web page; cited by tag and section):
//   [SGLv1] "SGLang Custom AllReduce v1 线程模型和工作原理细节" (todaynews.cc),
//           "2stage: sharding, rotation, and why no exit barrier"
//
// The message is P packs of 16 bytes; part = P / W; shard s covers packs
// [s * part, s * part + part), the last shard also the P mod W remainder.
// The launch is one-dimensional:
//   reduce blocks [0, rs_blocks): lane t of block b reduces packs
//     idx = b * threads * rpl + c * threads + t, c < rpl, of this rank's
//     shard (idx < own), reading pack rank * part + idx of every input,
//     writing pack idx of tmps[rank] and, when the gather runs in the same
//     launch, the same pack of out;
//   copy blocks: cp_blocks per shard copied (W - 1 shards after a reduce, the
//     W shards for a gather alone); block k of them copies shard
//     g = (rank + i) mod W, i = (reduce ? 1 : 0) + k / cp_blocks, lane t
//     taking packs idx0 + c * threads, c < cpl, idx0 = (k mod cp_blocks) *
//     threads * cpl + t, those below the shard's size: tmps[g][idx] ->
//     out[g * part + idx].
#pragma once

#include <stdint.h>

namespace ar {

struct TwoStageGrid {
    int64_t part;        // packs per shard (the last one has rem more)
    int64_t rem;         // P mod W
    int64_t own;         // packs of this rank's shard
    int64_t cap;         // part + rem: packs a staging buffer must hold
    int64_t rs_blocks;   // reduce blocks (0 without the reduce stage)
    int64_t cp_blocks;   // copy blocks per gathered shard
    int64_t blocks;      // the whole grid
};

constexpr TwoStageGrid two_stage_grid(int W, int rank, int64_t packs, bool rs, bool ag,
                                      int threads, int rpl, int cpl)
{
    TwoStageGrid g{};
    g.part = packs / W;
    g.rem = packs % W;
    g.own = g.part + (rank == W - 1 ? g.rem : 0);
    g.cap = g.part + g.rem;
    const int64_t per_rs_block = (int64_t)threads * rpl;
    g.rs_blocks = rs ? (g.own + per_rs_block - 1) / per_rs_block : 0;
    const int64_t per_block = (int64_t)threads * cpl;
    g.cp_blocks = (g.cap + per_block - 1) / per_block;
    g.blocks = g.rs_blocks + (ag ? (int64_t)(rs ? W - 1 : W) * g.cp_blocks : 0);
    return g;
}

// What one lane does for its c-th pack (c < rpl in a reduce block, c < cpl
// in a copy block).
struct TwoStageLane {
    int kind;            // 0: nothing, 1: reduce, 2: copy
    int shard;           // copy: the shard g read from tmps[g]
    int64_t read;        // reduce: pack of every input; copy: pack of tmps[g]
    int64_t tmp;         // reduce: pack written in tmps[rank]
    int64_t out;         // pack written in out (reduce with a gather, copy)
};

constexpr TwoStageLane two_stage_lane(const TwoStageGrid &g, int W, int rank, bool rs,
                                      int threads, int rpl, int cpl, int64_t b, int t, int c)
{
    TwoStageLane l{};
    if (rs && b < g.rs_blocks) {
        const int64_t idx = b * threads * rpl + (int64_t)c * threads + t;
        if (c < rpl && idx < g.own) {
            l.kind = 1;
            l.read = (int64_t)rank * g.part + idx;
            l.tmp = idx;
            l.out = (int64_t)rank * g.part + idx;
        }
        return l;
    }
    if (c >= cpl)
        return l;
    // block numbers fit 32 bits (a grid is at most 2^32 - 1 blocks), and
    // 32-bit division is far cheaper on the GPU than 64-bit
    const uint32_t k = (uint32_t)(rs ? b - g.rs_blocks : b);
    const uint32_t per_shard = (uint32_t)g.cp_blocks;
    const int i = (rs ? 1 : 0) + (int)(k / per_shard);
    const int64_t idx = (int64_t)(k % per_shard) * threads * cpl + (int64_t)c * threads + t;
    int s = rank + i;
    if (s >= W)
        s -= W;
    const int64_t size = g.part + (s == W - 1 ? g.rem : 0);
    if (idx < size) {
        l.kind = 2;
        l.shard = s;
        l.read = idx;
        l.out = (int64_t)s * g.part + idx;
    }
    return l;
}

// ---------------------------------------------------------------------------
// Streaming: a channel's steps may be shared by `pairs` producer/consumer
// pairs.  Pair g owns the same region of every ring slot: items
// [g * span, (g + 1) * span) of a full step of `full` items, span being
// ceil(full / pairs) rounded up to whole `unit`s (16 items = one LL128 line
// pair).  In a step of `total` <= full items (only the last step of a
// payload can be shorter) the slice is that region cut to [0, total), so it
// may be empty for the later pairs.
constexpr int64_t fifo_span(int64_t full, int64_t unit, int pairs)
{
    return ((full + pairs - 1) / pairs + unit - 1) / unit * unit;
}

// Pair `pair`'s slice of a step of `total` items, given the span.
constexpr void fifo_slice_at(int64_t span, int64_t total, int pair, int64_t *lo, int64_t *hi)
{
    const int64_t start = (int64_t)pair * span;
    *lo = start < total ? start : total;
    *hi = *lo + span < total ? *lo + span : total;
}

constexpr void fifo_slice(int64_t full, int64_t total, int64_t unit, int pairs, int pair,
                          int64_t *lo, int64_t *hi)
{
    fifo_slice_at(fifo_span(full, unit, pairs), total, pair, lo, hi);
}

// Steps per batch on the LL path.  A batch holds per_batch lines; when a
// pair's slice of a full step (span lines) is half a batch or less, a batch
// takes that many whole consecutive steps instead, at most max_steps, so
// that every lane keeps several lines in flight; 1 otherwise.  A producer
// waits for the head that frees the last slot of its batch, so it can work
// a batch ahead of its consumer in the 8-step ring only while 2 * S <= 8.
constexpr int fifo_batch_steps(int64_t span, int64_t per_batch, int max_steps)
{
    if (span <= 0)
        return 1;
    const int64_t s = per_batch / span;
    return s < 2 ? 1 : s > max_steps ? max_steps : (int)s;
}

// Lane slot v (u * lanes + lane) of a batch of whole steps whose slices are
// len lines long: the slot carries line `line` of the pair's slice of the
// batch's step `step` (no line when step is past the batch).  The same slot
// every batch; 32-bit division, once per workgroup.
constexpr void fifo_batch_slot(uint32_t v, uint32_t len, int *step, uint32_t *line)
{
    *step = (int)(v / len);
    *line = v % len;
}

// Pairs per channel when `resident` workgroups fit on the device at once: as
// many as fit (two workgroups per pair), at most max_pairs, and no more than
// leave every pair a slice of a full step of at least min_slice items (one
// pair always).  0 when not even one pair per channel fits.
constexpr int fifo_pairs_for(int64_t full, int64_t unit, int channels, int resident,
                             int max_pairs, int64_t min_slice)
{
    int g = resident / (2 * channels);
    if (g > max_pairs)
        g = max_pairs;
    for (; g > 1; --g) {
        int64_t lo = 0, hi = 0;
        fifo_slice(full, full, unit, g, g - 1, &lo, &hi);
        if (hi - lo >= min_slice)
            break;
    }
    return g;
}

}  // namespace ar
