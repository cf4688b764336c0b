// Kernel launchers behind the C ABI (internal C++ interface of libar).
// Each launcher assumes its arguments were validated by the C entry point
// and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ar {

hipError_t launch_reduce_1stage(const void *const *inputs, int W, void *out,
                                int64_t packs, hipStream_t s);

// order[i] = index of the input summed i-th; tmps absolute per shard owner.
hipError_t launch_reduce_2stage(const void *const *inputs, const int *order,
                                void *const *tmps, int W, int rank, void *out,
                                int64_t packs, bool rs, bool ag, hipStream_t s);

hipError_t launch_fused_rmsnorm(const void *const *inputs, int W,
                                const void *residual, const void *weight,
                                void *residual_out, void *norm_out, int64_t M,
                                int64_t N, float eps, hipStream_t s);

// order[i] = index of the input summed i-th; tmps absolute per shard owner.
hipError_t launch_fused_2stage(const void *const *inputs, const int *order,
                               void *const *tmps, int W, int rank, const void *residual,
                               const void *weight, void *residual_out, void *norm_out,
                               int64_t M, int64_t N, float eps, bool rs, bool ag,
                               hipStream_t s);

hipError_t launch_lamport_fill(void *comm, int64_t chunks, hipStream_t s);
hipError_t launch_lamport_push(const void *x, int W, int rank, void *const *comms,
                               int64_t M, int64_t N, uint32_t flag, hipStream_t s);
// x_self == NULL: reader only; otherwise also push x_self as rank `rank`
// into every buffer of `comms` in the same launch (comm == comms[rank]).
hipError_t launch_lamport_fused(void *comm, int W, const void *residual,
                                const void *weight, void *residual_out, void *norm_out,
                                int64_t M, int64_t N, float eps, uint32_t flag,
                                uint32_t max_spins, uint32_t *bad, const void *x_self,
                                int rank, void *const *comms, hipStream_t s);

// The Lamport exchange of all W ranks in one launch (M x W workgroups).
// With check_only nothing is launched: *resident receives how many of its
// workgroups the current device holds at once.
hipError_t launch_lamport_all_ranks(const void *const *xs, void *const *comms, int W,
                                    const void *residual, const void *weight,
                                    void *const *residual_outs, void *const *norm_outs,
                                    int64_t M, int64_t N, float eps, uint32_t flag,
                                    uint32_t max_spins, uint32_t *bad, bool check_only,
                                    int *resident, hipStream_t s);

// One launch of 2 * channels * pairs workgroups (producers, then consumers),
// all of which the caller has checked can be resident at once in the chosen
// geometry (wide: 1,024 lanes per workgroup, else 512).
hipError_t launch_fifo_stream(int proto, const float *src, const float *local, float *out,
                              int64_t n, void *fifo, uint64_t *counters, int channels,
                              int64_t step_bytes, int64_t wire_bytes, uint64_t first_step,
                              bool from_state, uint32_t max_spins, uint32_t *errors,
                              bool wide, int pairs, hipStream_t s);
// Workgroups of the streaming kernel, in the given geometry, that the current
// device holds at once.
hipError_t fifo_stream_resident_workgroups(int proto, bool local, bool wide, int *workgroups);

// dst[0 .. 16 * packs) = src[0 .. 16 * packs)
hipError_t launch_copy(const void *src, void *dst, int64_t packs, hipStream_t s);

hipError_t launch_ll_pack(const float *src, int64_t n, void *fifo,
                          int64_t step_lines, uint64_t first_step, hipStream_t s);
hipError_t launch_ll_unpack_reduce(const void *const *fifos, int W, float *out,
                                   int64_t n, int64_t step_lines,
                                   uint64_t first_step, uint32_t max_spins,
                                   uint32_t *bad_lines, hipStream_t s);
hipError_t launch_ll128_pack(const float *src, int64_t n, void *fifo,
                             int64_t step_lines, uint64_t first_step,
                             hipStream_t s);
hipError_t launch_ll128_unpack_reduce(const void *const *fifos, int W,
                                      float *out, int64_t n, int64_t step_lines,
                                      uint64_t first_step, uint32_t max_spins,
                                      uint32_t *bad_lines, hipStream_t s);

}  // namespace ar
