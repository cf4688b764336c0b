// One-stage and two-stage reduce of W bf16 rank buffers on one GPU.
//
// Sources (web pages; cited by tag and section):
//   [SGLv1] "SGLang Custom AllReduce v1 线程模型和工作原理细节" (todaynews.cc)
//   [JITAR] "0-custom-all-reduce" (obnotes-4iw.pages.dev, sglang jit_kernel)
//
// Both forms are pure streams over 16-byte packs: every byte is read once and
// written once, with ~1 fp32 add per 2 bytes, so they are bound by HBM
// bandwidth (8 TB/s on MI355X), not by the vector ALUs, and there is no
// contraction to put on the matrix cores.  All their accesses are streaming
// (nontemporal); on cold data that is worth ~20% at these sizes.  The launch
// shape differs from the pages' (512 threads x at most 36 blocks, tuned for
// NVLink-era parts): here
// one 256-lane workgroup covers 256 consecutive packs and the grid grows
// with the message, so an 8 MB x 8 reduce fills all 256 CUs with thousands
// of wavefronts, each lane keeping its W loads in flight at once.
#include "device.h"
#include "index_map.h"
#include "launch.h"

namespace ar {

constexpr int kReduceThreads = 256;

// Sum of the W packs of one 16-byte column, in table order, rounded once
// ([SGLv1] "1stage: full kernel and timeline": fp32 accumulation starting
// from the first buffer's value; [JITAR] section 4).
template <int W>
__device__ __forceinline__ u32x4 reduce_column(const u32x4 (&v)[W])
{
    float acc[8];
    widen8(v[0], acc);
#pragma unroll
    for (int r = 1; r < W; ++r) {
        float t[8];
        widen8(v[r], t);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            acc[k] = acc[k] + t[k];
    }
    return narrow8(acc);
}

// out[i] = bf16(sum_r in[r][i]) for every pack i.  out may be one of the
// inputs: each lane loads all W packs of column i before storing column i.
template <int W>
__global__ __launch_bounds__(kReduceThreads) void reduce_1stage_kernel(
    InTable<W> in, u32x4 *out, int64_t packs)
{
    const int64_t i = (int64_t)blockIdx.x * kReduceThreads + threadIdx.x;
    if (i >= packs)
        return;
    u32x4 v[W];
#pragma unroll
    for (int r = 0; r < W; ++r)
        v[r] = ld_stream(in.p[r] + i);
    st_stream(out + i, reduce_column<W>(v));
}

// Two-stage reduce for one rank ([SGLv1] "2stage: sharding, rotation, and
// why no exit barrier").  One-dimensional grid, reduce blocks first; which
// packs a lane touches is two_stage_lane() (index_map.h), the same function
// the host-side checks enumerate:
//   reduce blocks (RS): this rank's shard, inputs in `in` order (the owner's
//       rotation), stored to tmps[rank] and, with AG, to out.  The value goes
//       from registers to out and each lane gathers exactly the packs it
//       reduced (the pages' same-thread mapping), so no barrier is needed
//       inside the launch.
//   copy blocks (AG): CPL packs per lane of the other shards (of every shard
//       for a gather alone), tmps[g] -> out.
// A reduce lane takes RPL packs, all of their W loads issued before any sum.
// The gather reads use plain loads and everything else streams: on cold
// data that measured fastest among the cache-policy combinations.
template <int W, bool RS, bool AG, int T, int RPL, int CPL>
__global__ __launch_bounds__(T) void reduce_2stage_kernel(
    InTable<W> in, OutTable<W> tmps, int rank, u32x4 *out, TwoStageGrid grid)
{
    const int64_t b = blockIdx.x;
    const int t = threadIdx.x;
    if (RS && b < grid.rs_blocks) {
        TwoStageLane l[RPL];
        u32x4 v[RPL][W];
#pragma unroll
        for (int c = 0; c < RPL; ++c) {
            l[c] = two_stage_lane(grid, W, rank, RS, T, RPL, CPL, b, t, c);
            if (l[c].kind == 1) {
#pragma unroll
                for (int r = 0; r < W; ++r)
                    v[c][r] = ld_stream(in.p[r] + l[c].read);
            }
        }
#pragma unroll
        for (int c = 0; c < RPL; ++c) {
            if (l[c].kind != 1)
                continue;
            const u32x4 s = reduce_column<W>(v[c]);
            st_stream(tmps.p[rank] + l[c].tmp, s);
            if (AG)
                st_stream(out + l[c].out, s);
        }
        return;
    }
    if (!AG)
        return;
    TwoStageLane l[CPL];
    u32x4 v[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        l[c] = two_stage_lane(grid, W, rank, RS, T, RPL, CPL, b, t, c);
        if (l[c].kind == 2)
            v[c] = tmps.p[l[c].shard][l[c].read];
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        if (l[c].kind == 2)
            st_stream(out + l[c].out, v[c]);
}

template <int W>
static hipError_t launch_1stage_w(const void *const *inputs, void *out,
                                  int64_t packs, hipStream_t s)
{
    InTable<W> t;
    for (int r = 0; r < W; ++r)
        t.p[r] = static_cast<const u32x4 *>(inputs[r]);
    const int64_t blocks = (packs + kReduceThreads - 1) / kReduceThreads;
    reduce_1stage_kernel<W><<<dim3((unsigned)blocks), dim3(kReduceThreads), 0, s>>>(
        t, static_cast<u32x4 *>(out), packs);
    return hipGetLastError();
}

hipError_t launch_reduce_1stage(const void *const *inputs, int W, void *out,
                                int64_t packs, hipStream_t s)
{
    switch (W) {
    case 2: return launch_1stage_w<2>(inputs, out, packs, s);
    case 3: return launch_1stage_w<3>(inputs, out, packs, s);
    case 4: return launch_1stage_w<4>(inputs, out, packs, s);
    case 5: return launch_1stage_w<5>(inputs, out, packs, s);
    case 6: return launch_1stage_w<6>(inputs, out, packs, s);
    case 7: return launch_1stage_w<7>(inputs, out, packs, s);
    case 8: return launch_1stage_w<8>(inputs, out, packs, s);
    default: return hipErrorInvalidValue;
    }
}

template <int W, bool RS, bool AG, int T, int RPL, int CPL>
static hipError_t launch_2stage_shape(const InTable<W> &in, const OutTable<W> &tmps,
                                      int rank, void *out, int64_t packs, hipStream_t s)
{
    const TwoStageGrid g = two_stage_grid(W, rank, packs, RS, AG, T, RPL, CPL);
    if (g.blocks == 0)
        return hipSuccess;
    reduce_2stage_kernel<W, RS, AG, T, RPL, CPL><<<dim3((unsigned)g.blocks), dim3(T), 0, s>>>(
        in, tmps, rank, static_cast<u32x4 *>(out), g);
    return hipGetLastError();
}

// 256 lanes, one pack per reduce lane and two per gather lane.  Timed at the
// 8 MB cap (W = 8, cold buffers, back to back), this beat every other shape
// tried: 5.10 us against 5.22 us with one gather pack per lane; four gather
// packs, two reduce packs, and 128-, 512- or 1,024-lane workgroups were all
// slower (5.8-7.2 us).
template <int W, bool RS, bool AG>
static hipError_t launch_2stage_mode(const InTable<W> &in, const OutTable<W> &tmps,
                                     int rank, void *out, int64_t packs, hipStream_t s)
{
    return launch_2stage_shape<W, RS, AG, kReduceThreads, 1, 2>(in, tmps, rank, out, packs, s);
}

template <int W>
static hipError_t launch_2stage_w(const void *const *inputs, const int *order,
                                  void *const *tmps, int rank, void *out,
                                  int64_t packs, bool rs, bool ag, hipStream_t s)
{
    InTable<W> in;
    OutTable<W> tp;
    for (int r = 0; r < W; ++r) {
        in.p[r] = static_cast<const u32x4 *>(inputs[order[r]]);
        tp.p[r] = static_cast<u32x4 *>(tmps[r]);
    }
    if (rs && ag)
        return launch_2stage_mode<W, true, true>(in, tp, rank, out, packs, s);
    if (rs)
        return launch_2stage_mode<W, true, false>(in, tp, rank, out, packs, s);
    return launch_2stage_mode<W, false, true>(in, tp, rank, out, packs, s);
}

hipError_t launch_reduce_2stage(const void *const *inputs, const int *order,
                                void *const *tmps, int W, int rank, void *out,
                                int64_t packs, bool rs, bool ag, hipStream_t s)
{
    switch (W) {
    case 2: return launch_2stage_w<2>(inputs, order, tmps, rank, out, packs, rs, ag, s);
    case 3: return launch_2stage_w<3>(inputs, order, tmps, rank, out, packs, rs, ag, s);
    case 4: return launch_2stage_w<4>(inputs, order, tmps, rank, out, packs, rs, ag, s);
    case 5: return launch_2stage_w<5>(inputs, order, tmps, rank, out, packs, rs, ag, s);
    case 6: return launch_2stage_w<6>(inputs, order, tmps, rank, out, packs, rs, ag, s);
    case 7: return launch_2stage_w<7>(inputs, order, tmps, rank, out, packs, rs, ag, s);
    case 8: return launch_2stage_w<8>(inputs, order, tmps, rank, out, packs, rs, ag, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ar
