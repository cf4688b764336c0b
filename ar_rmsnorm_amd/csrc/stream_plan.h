// The launch plan of a streaming call as plain C++17 constexpr functions:
// the steps of the busiest channel, the producer/consumer pairs a channel
// gets, the workgroup size, and the whole LL steps a batch takes.  The host
// library evaluates them with the device's occupancy (how many workgroups of
// each size it holds at once), the streaming kernel takes its batch
// constants from here, and g++ evaluates them in tests/fifo_slice_check.cpp
// for the occupancy of one MI355X.  Protocols: 0 LL, 1 LL128, 2 Simple.
#pragma once

#include <stdint.h>

#include "index_map.h"

namespace ar {

constexpr int kFifoMaxPairs = 8;             // pairs a channel can have; a head and a tail each
constexpr int64_t kFifoPerBatch = 4096;      // items a workgroup keeps in flight in one batch
constexpr int kFifoMaxBatchSteps = 4;        // LL: whole steps per batch, 2 * 4 <= 8 ring slots
constexpr int64_t kFifoMinSlice = 512;       // items of a full step every pair gets at least
constexpr int64_t kFifoItemsPerPair = 2048;  // payload items a channel carries per pair
constexpr int64_t kFifoNarrowSteps = 32;     // LL: steps per channel from which 512-lane pairs
                                             // may be taken over fewer 1,024-lane ones

// Items of a full step: LL lines, LL128 16-byte chunks (8 per line), Simple
// 16-byte chunks.
constexpr int64_t fifo_full_items(int proto, int64_t step_bytes)
{
    return proto == 0 ? step_bytes / 8 : proto == 1 ? step_bytes / 120 * 8 : step_bytes / 16;
}

// Steps the busiest channel carries: the T = ceil(4n / step_bytes) steps of
// the payload dealt to the channels in contiguous runs.
constexpr int64_t fifo_steps_per_channel(int64_t n, int64_t step_bytes, int channels)
{
    const int64_t total = (4 * n + step_bytes - 1) / step_bytes;
    return (total + channels - 1) / channels;
}

// Pairs per channel when `resident` workgroups of one size fit on the device
// at once (fifo_pairs_for): as many as fit, at most kFifoMaxPairs and at
// most one per kFifoItemsPerPair payload items of the busiest channel (at
// least one), none with a slice of a full step under kFifoMinSlice items
// (LL128 slices are whole line pairs).  0 when not one pair per channel fits.
constexpr int fifo_plan_pairs(int proto, int64_t step_bytes, int64_t n, int channels,
                              int resident)
{
    int64_t bytes = fifo_steps_per_channel(n, step_bytes, channels) * step_bytes;
    if (bytes > 4 * n)
        bytes = 4 * n;
    const int64_t per_item = proto == 0 ? 8 : proto == 1 ? 15 : 16;   // payload bytes
    int64_t by_work = bytes / per_item / kFifoItemsPerPair;
    if (by_work < 1)
        by_work = 1;
    const int most = by_work < kFifoMaxPairs ? (int)by_work : kFifoMaxPairs;
    return fifo_pairs_for(fifo_full_items(proto, step_bytes), proto == 1 ? 16 : 1, channels,
                          resident, most, kFifoMinSlice);
}

// True for 1,024-lane workgroups, given the pairs each size allows: the
// wider form unless it leaves one pair per channel (or none) where 512-lane
// workgroups allow two or more; LL also takes the 512-lane form where it
// gives at least twice the pairs and every channel carries kFifoNarrowSteps
// steps or more.
constexpr bool fifo_plan_wide(int proto, int wide_pairs, int narrow_pairs,
                              int64_t steps_per_channel)
{
    if (proto == 0 && narrow_pairs >= 2 && narrow_pairs >= 2 * wide_pairs &&
        steps_per_channel >= kFifoNarrowSteps)
        return false;
    return wide_pairs >= 2 || (wide_pairs == 1 && narrow_pairs < 2);
}

// Whole steps per LL batch (fifo_batch_steps) for a call of `pairs` pairs
// per channel; 1 for the other protocols, for channels of one step (where
// whole-step batches do not pay), and for rings of 2 GiB or more (one buffer
// descriptor addresses a batch's slots).
constexpr int fifo_plan_batch_steps(int proto, int64_t step_bytes, int64_t n, int channels,
                                    int pairs)
{
    if (proto != 0 || n <= 0 || channels < 1 || pairs < 1)
        return 1;
    const int64_t wire_bytes = step_bytes / 8 * 16;
    if (fifo_steps_per_channel(n, step_bytes, channels) < 2 || 8 * wire_bytes > (int64_t)INT32_MAX)
        return 1;
    return fifo_batch_steps(fifo_span(fifo_full_items(proto, step_bytes), 1, pairs),
                            kFifoPerBatch, kFifoMaxBatchSteps);
}

}  // namespace ar
