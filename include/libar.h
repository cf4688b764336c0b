/*
 * libar — the per-GPU reduction at the heart of a custom all-reduce, for
 * AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes only.
 *
 * All W "peer" rank buffers are ordinary device buffers of one GPU; nothing
 * here talks to another GPU.  The operations follow these pages (cited by tag
 * and section below):
 *   [SGLv1]  "SGLang Custom AllReduce v1 线程模型和工作原理细节" (todaynews.cc)
 *   [NCCL14] "NCCL 专家课程 14：Simple、LL、LL128 的线格式、同步与真实性能边界"
 *            (blog.cptz.space)
 *   [JITAR]  "0-custom-all-reduce" (obnotes-4iw.pages.dev, sglang jit_kernel)
 *   [TRIAR]  "用 Triton + Symmetric Memory 写一个 AllReduce + RMSNorm 融合算子"
 *            (riverclouds.net)
 *
 * Conventions shared by every entry point
 *   Ownership  The caller owns every buffer, except the staging array of
 *              ar_reduce_2stage_noalloc, which is static device memory of
 *              the library.  The library never allocates, frees or
 *              synchronizes.
 *   State      No call depends on an earlier call except through the
 *              caller's buffers (and, for ar_reduce_2stage_noalloc, that
 *              staging array).  The library keeps two things of its own:
 *              a thread-local copy of the last HIP error, and, per device,
 *              how many streaming workgroups (ar_fifo_stream) the device
 *              holds at once.  The latter is looked up once per (device,
 *              protocol, geometry) with the HIP occupancy API and stored in
 *              a process-wide table of atomics: concurrent first calls may
 *              each look it up and store the same value; it is only read
 *              afterwards.  ar_reduce_2stage_noalloc also keeps, per
 *              device, the address of its staging array, looked up once
 *              the same way.
 *   Pointers   Data pointers are device pointers.  Pointer tables (inputs,
 *              tmps, fifos) are HOST arrays of W device pointers; they are
 *              read during the call and copied into the kernel arguments, so
 *              the table may be reused as soon as the call returns.
 *   Streams    Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *              stream) and the call returns without waiting.
 *   Errors     Argument errors are detected before anything is enqueued and
 *              leave every buffer untouched.  AR_ERR_HIP means a launch was
 *              rejected by the HIP runtime; ar_last_hip_error() gives its
 *              hipError_t code.
 *   Sizes      Counts are elements (bf16 for the reduce forms, fp32 for the
 *              wire formats).  A count of 0 is valid and enqueues nothing.
 *   bf16       Raw bfloat16 bit patterns (upper half of an IEEE binary32).
 *              Sums are formed in fp32 and rounded once to bf16, to nearest,
 *              ties to even; fp32 denormals are kept ([JITAR] section 4).
 */
#ifndef LIBAR_H
#define LIBAR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *ar_stream_t;
typedef int ar_status_t;

#define AR_OK 0
#define AR_ERR_NULL 1      /* a required pointer is NULL */
#define AR_ERR_ARG 2       /* a size, flag or aliasing rule is violated */
#define AR_ERR_ALIGN 3     /* a pointer lacks the required alignment */
#define AR_ERR_WORLD 4     /* W outside the supported range */
#define AR_ERR_CAPACITY 5  /* the payload does not fit the FIFO's 8 steps or
                              (ar_reduce_2stage_noalloc) the staging array, or
                              (ar_fifo_stream) its workgroups cannot all be
                              resident at once */
#define AR_ERR_HIP 6       /* the HIP runtime rejected a launch */

#define AR_MAX_WORLD 8          /* W <= 8 rank buffers */
#define AR_FUSED_MAX_N 16384    /* longest row of the fused form */
#define AR_MAX_SPINS 65536u     /* bound on flag re-reads per line */
#define AR_FIFO_STEPS 8         /* slots in a wire FIFO ring */

/* Flags of ar_reduce_2stage and ar_fused_residual_rmsnorm_2stage. */
#define AR_STAGE_RS 1u     /* run the reduce-scatter of this rank's shard */
#define AR_STAGE_AG 2u     /* run the all-gather into out */
#define AR_ORDER_RANK 4u   /* sum 0..W-1 instead of the owner's rotation */

/* Short English text for a status code (static storage). */
const char *ar_status_str(ar_status_t status);

/* hipError_t of the last failed launch on the calling thread (0 if none). */
int ar_last_hip_error(void);

/*
 * One-stage reduce ([SGLv1] "1stage: full kernel and timeline"; [JITAR]
 * sections 1-5).  For every element j:
 *     acc = fp32(inputs[0][j]); acc += fp32(inputs[r][j]) for r = 1..W-1;
 *     out[j] = bf16(acc)
 * in this order, so the result is the same bits on every rank.  Each lane
 * moves whole 16-byte packs (8 bf16).
 *   inputs  host table of W device pointers, each to n bf16
 *   W       2 <= W <= 8                                 else AR_ERR_WORLD
 *   out     n bf16; may be one of the inputs (in place), must not partially
 *           overlap any input                            else AR_ERR_ARG
 *   n       multiple of 8 (whole 16-byte packs), >= 0   else AR_ERR_ARG
 *   every data pointer 16-byte aligned                   else AR_ERR_ALIGN
 */
ar_status_t ar_reduce_1stage(const void *const *inputs, int W, void *out,
                             int64_t n, ar_stream_t stream);

/*
 * Two-stage reduce = reduce-scatter + all-gather, as run by one rank
 * ([SGLv1] "2stage: sharding, rotation, and why no exit barrier").
 * The message is P = n/8 packs; part = P / W; shard s is packs
 * [s*part, (s+1)*part), the last shard also taking the P mod W remainder.
 *   RS: tmps[rank][q] = bf16(sum of inputs[(rank+i) mod W][s*part*8 + q],
 *       i = 0..W-1, in that rotated order) for the elements q of shard rank.
 *       With AR_ORDER_RANK the order is 0..W-1.
 *   AG: out[s*part*8 + q] = tmps[s][q] for every shard s.
 * On one GPU the peers' shards are whatever tmps[s != rank] hold: run the
 * RS stage for every other rank first (flags = AR_STAGE_RS).  With both
 * stages, this rank's shard goes from registers to both tmps[rank] and out,
 * each lane gathering the same packs it reduced (the pages' same-thread
 * mapping), so no barrier is needed inside the launch.
 *   inputs  host table of W device pointers, each to n bf16
 *   tmps    host table of W device pointers, each to at least
 *           (part + P mod W) * 8 bf16
 *   W       2 <= W <= 8                                 else AR_ERR_WORLD
 *   rank    0 <= rank < W                                else AR_ERR_ARG
 *   out     n bf16 (may be NULL when AG is not run); must not overlap any
 *           input or tmp buffer                          else AR_ERR_ARG
 *   n       multiple of 8, >= 0                          else AR_ERR_ARG
 *   flags   AR_STAGE_RS | AR_STAGE_AG | AR_ORDER_RANK; no stage bit means
 *           both stages; other bits                      -> AR_ERR_ARG
 *   every data pointer 16-byte aligned                   else AR_ERR_ALIGN
 */
ar_status_t ar_reduce_2stage(const void *const *inputs, void *const *tmps,
                             int W, int rank, void *out, int64_t n,
                             unsigned flags, ar_stream_t stream);

/*
 * Two-stage reduce that allocates nothing and takes no staging buffers, for
 * callers that cannot allocate device memory (code being captured into a
 * HIP graph, tight serving loops, harnesses that forbid hipMalloc).  Same
 * operation and arguments as ar_reduce_2stage, except that the W staging
 * shards live in a library-owned device array of AR_SCRATCH_BYTES bytes
 * (one per GPU, held until the process ends): shard s at byte offset
 * s * (part + P mod W) * 16.  A call with AR_STAGE_RS leaves its shard there
 * for later calls, as the tmps buffers of ar_reduce_2stage would hold it.
 * Every call on one GPU uses that GPU's one array, so calls that overlap in
 * time on one GPU (other streams, other threads) race: order them on one
 * stream.  No call allocates or frees memory.
 *   W * (part + P mod W) * 16 <= AR_SCRATCH_BYTES        else AR_ERR_CAPACITY
 *   (every message up to 8 MiB, 4,194,304 bf16, fits for any W)
 *   other arguments and errors as ar_reduce_2stage
 */
#define AR_SCRATCH_BYTES ((8u << 20) + 4096u)

ar_status_t ar_reduce_2stage_noalloc(const void *const *inputs, int W, int rank,
                                     void *out, int64_t n, unsigned flags,
                                     ar_stream_t stream);

/*
 * Fused all-reduce + residual add + RMSNorm ([TRIAR] "what this operator
 * computes" and "overall design").  For every row m and column j:
 *     a    = one-stage sum of inputs[r][m, j] (fp32, order 0..W-1)
 *     h    = a + fp32(residual[m, j])               (fp32)
 *     residual_out[m, j] = bf16(h)
 *     rms  = 1 / sqrt(sum_j h^2 / N + eps)          (fp32, per row)
 *     norm_out[m, j] = bf16((h * rms) * fp32(weight[j]))
 * One workgroup owns a whole row, so h stays in registers between the sum
 * and the norm.  residual_out is bit-exact; norm_out matches the exact value
 * to within 2 bf16 ulp.
 *   inputs       host table of W device pointers, each to bf16 [M, N]
 *                row-major
 *   W            2 <= W <= 8                            else AR_ERR_WORLD
 *   residual     bf16 [M, N]
 *   weight       bf16 [N]
 *   residual_out bf16 [M, N]; may equal residual (in place)
 *   norm_out     bf16 [M, N]; must not overlap any other buffer
 *   M >= 0; 8 <= N <= 16384 and N multiple of 8; eps finite and >= 0
 *                                                       else AR_ERR_ARG
 *   every data pointer 16-byte aligned                   else AR_ERR_ALIGN
 */
ar_status_t ar_fused_residual_rmsnorm(const void *const *inputs, int W,
                                      const void *residual, const void *weight,
                                      void *residual_out, void *norm_out,
                                      int64_t M, int64_t N, float eps,
                                      ar_stream_t stream);

/*
 * Two-shot fused all-reduce + residual + RMSNorm, as run by one rank: the
 * two-stage structure of [SGLv1] "2stage: sharding, rotation, and why no
 * exit barrier" applied to rows, so that each row is normalised by one owner
 * ([TRIAR] "overall design" keeps a row whole).  part = M / W rows per
 * shard; shard s is rows [s*part, (s+1)*part), the last shard also taking the
 * M mod W remainder.
 *   RS: the rows of shard `rank` get the fused operator (as
 *       ar_fused_residual_rmsnorm), the W inputs summed in the owner's
 *       rotated order rank, rank+1, ..., rank-1 (AR_ORDER_RANK: 0..W-1, which
 *       gives exactly the one-shot result); tmps[rank] receives the shard's
 *       residual_out rows followed by its norm_out rows.
 *   AG: residual_out and norm_out receive every shard's rows from tmps[s].
 * On one GPU the peers' shards are whatever tmps[s != rank] hold: run the
 * RS stage for every other rank first (flags = AR_STAGE_RS).  With both
 * stages this rank's rows go from registers to both tmps[rank] and the
 * outputs, so no barrier is needed inside the launch.
 *   inputs, W, residual, weight, M, N, eps  as ar_fused_residual_rmsnorm
 *   tmps     host table of W device pointers, each to at least
 *            2 * (part + M mod W) * N bf16, 16-byte aligned
 *   rank     0 <= rank < W                               else AR_ERR_ARG
 *   residual_out, norm_out  bf16 [M, N] (may be NULL when AG is not run);
 *            residual_out may equal residual; no other overlap with an
 *            input, a tmp buffer or each other             else AR_ERR_ARG
 *   flags    AR_STAGE_RS | AR_STAGE_AG | AR_ORDER_RANK; no stage bit means
 *            both stages                                  else AR_ERR_ARG
 */
ar_status_t ar_fused_residual_rmsnorm_2stage(const void *const *inputs,
                                             void *const *tmps, int W, int rank,
                                             const void *residual,
                                             const void *weight,
                                             void *residual_out, void *norm_out,
                                             int64_t M, int64_t N, float eps,
                                             unsigned flags, ar_stream_t stream);

/*
 * Which fused form to call on one GPU ([SGLv1] "Algorithm switching and
 * admission limits" chooses between its one-stage and two-stage kernels from
 * W and the message size, with thresholds its authors measured on NVLink-era
 * parts; [TRIAR] "overall design" keeps the one-shot form for small batches).
 * Returns 1 when ar_fused_residual_rmsnorm_2stage is expected to finish a
 * rank's M x N call sooner than ar_fused_residual_rmsnorm on one MI355X, 0
 * when the one-shot call is, and -1 for arguments either call rejects.  The
 * thresholds come from timing both calls for one rank on one MI355X (cold
 * buffers); on several GPUs the two-shot form also pays an exchange between
 * its stages, which this one-GPU choice does not include.
 */
int ar_fused_prefers_two_shot(int W, int64_t M, int64_t N);

/*
 * Lamport data-as-flag form of the fused one-shot ([TRIAR] "Option 2:
 * Lamport").  Each rank owns a comm buffer of u32 words
 * [3 regions][W slots][M][N / 2] (ar_lamport_comm_bytes), filled with the
 * sentinel 0x80008000 (two bf16 -0.0) before first use (ar_lamport_fill).
 * A call with counter `flag` uses region flag mod 3.  The page advances the
 * flag by one per launch; here it must stay below AR_LAMPORT_FLAG_PERIOD
 * (3 * 2^30, a multiple of 3) and the next call's flag is
 * ar_lamport_next_flag(flag), which wraps to 0 after PERIOD - 1.  Because
 * the period is a multiple of 3, the region sequence 0, 1, 2, 0, ... runs on
 * unbroken across the wrap (a 32-bit counter wrapping at 2^32 would use
 * region 0 twice in a row).  Flags at or above the period -> AR_ERR_ARG.
 *   push   rank r writes its bf16 [M, N] rows into slot r of that region of
 *          every rank's buffer, as u32 words of two bf16 (element 2j in the
 *          low half) with every -0.0 turned into +0.0, so no word can equal
 *          the sentinel;
 *   fused  rank p waits until no word of its region holds the sentinel (at
 *          most max_spins re-reads per 16-byte chunk, never a hang), sums the
 *          W slots in slot order 0..W-1 in fp32 and applies the residual add
 *          and RMSNorm exactly as ar_fused_residual_rmsnorm; it then refills
 *          region ((flag mod 3) + 2) mod 3, the previous call's region, with
 *          the sentinel.  Every peer finished writing that region before the
 *          previous call could complete, and writes it again only two calls
 *          later, so three regions make the buffer reusable without a barrier.
 * On one GPU the W comm buffers are ordinary device buffers and the pushes
 * are separate launches ahead of the fused call.
 */

#define AR_LAMPORT_FLAG_PERIOD 0xC0000000u   /* 3 * 2^30 */

/* The flag of the call after `flag`: (flag + 1) mod AR_LAMPORT_FLAG_PERIOD
 * (flags at or above the period give 0). */
uint32_t ar_lamport_next_flag(uint32_t flag);

/* Bytes of one rank's comm buffer: 3 * W * M * N * 2 (0 for invalid sizes). */
int64_t ar_lamport_comm_bytes(int W, int64_t M, int64_t N);

/*
 * Fill a comm buffer (all three regions) with the sentinel.
 *   comm   ar_lamport_comm_bytes(W, M, N) bytes, 16-byte aligned
 *   W, M, N as for ar_lamport_push
 */
ar_status_t ar_lamport_fill(void *comm, int W, int64_t M, int64_t N,
                            ar_stream_t stream);

/*
 * Push this rank's rows into slot `rank` of region flag mod 3 of every comm
 * buffer.
 *   x      bf16 [M, N] row-major, 16-byte aligned; must not overlap a buffer
 *   comms  host table of the W ranks' comm buffers (16-byte aligned)
 *   W      2 <= W <= 8                                  else AR_ERR_WORLD
 *   rank   0 <= rank < W; 0 <= M < 2^31, M * N <= 2^40; 8 <= N <= 16384,
 *          N multiple of 8; flag < AR_LAMPORT_FLAG_PERIOD
 *                                                       else AR_ERR_ARG
 */
ar_status_t ar_lamport_push(const void *x, int W, int rank, void *const *comms,
                            int64_t M, int64_t N, uint32_t flag,
                            ar_stream_t stream);

/*
 * Read this rank's comm buffer (region flag mod 3), reduce, add the residual,
 * normalise, and reset region ((flag mod 3) + 2) mod 3 to the sentinel.
 *   flag          < AR_LAMPORT_FLAG_PERIOD               else AR_ERR_ARG
 *   comm          this rank's comm buffer (16-byte aligned)
 *   residual, weight, residual_out, norm_out, M, N, eps
 *                 as ar_fused_residual_rmsnorm; no output may overlap comm
 *   max_spins     <= AR_MAX_SPINS                       else AR_ERR_ARG
 *   bad_chunks    device u32 (4-byte aligned) the caller zeroes; the library
 *                 adds the number of (slot, 16-byte chunk) units still holding
 *                 a sentinel after max_spins re-reads (their outputs are
 *                 unspecified).  NULL: not counted.
 */
ar_status_t ar_lamport_fused_residual_rmsnorm(void *comm, int W,
                                              const void *residual,
                                              const void *weight,
                                              void *residual_out, void *norm_out,
                                              int64_t M, int64_t N, float eps,
                                              uint32_t flag, uint32_t max_spins,
                                              uint32_t *bad_chunks,
                                              ar_stream_t stream);

/*
 * The whole Lamport call of one rank in one launch, as the page's program
 * does it: push x as rank `rank` into every buffer of `comms` (as
 * ar_lamport_push), then read comms[rank] (as
 * ar_lamport_fused_residual_rmsnorm).  The own slot is taken from registers;
 * only the W - 1 peer slots are polled.  Arguments and errors are those of
 * the two calls; x must not overlap an output or a comm buffer.
 */
ar_status_t ar_lamport_oneshot_residual_rmsnorm(const void *x, int rank,
                                                void *const *comms, int W,
                                                const void *residual,
                                                const void *weight,
                                                void *residual_out, void *norm_out,
                                                int64_t M, int64_t N, float eps,
                                                uint32_t flag, uint32_t max_spins,
                                                uint32_t *bad_chunks,
                                                ar_stream_t stream);

/*
 * The Lamport exchange of all W ranks in one launch, as W GPUs would run
 * their one-launch calls at the same time: for every rank r and row m, one
 * workgroup runs ar_lamport_oneshot_residual_rmsnorm's program for rank r
 * on row m (push row m of xs[r] into every buffer of comms, wait for the
 * W - 1 peer slots of row m in comms[r], reduce, add the residual,
 * normalise into residual_outs[r] and norm_outs[r], reset row m of the
 * previous region of comms[r]).  The peers' pushes land while a reader
 * polls, so this is the call that exercises the re-read path on one GPU.
 * All ranks share one residual and one weight (in tensor parallelism every
 * rank holds the same residual stream), and every rank's outputs equal what
 * ar_lamport_fused_residual_rmsnorm gives after all W pushes.
 *   xs, comms, residual_outs, norm_outs  host tables of W device pointers
 *            (bf16 [M, N] rows, comm buffers, outputs), 16-byte aligned
 *   flag, max_spins, bad_chunks, M, N, eps  as the one-launch call
 *   no output may overlap any input, buffer or other output   else AR_ERR_ARG
 *   the M * W workgroups must all be resident on the device at once (a
 *   waiting workgroup must never hold back a push): AR_ERR_CAPACITY when the
 *   device cannot hold them (M * W above about 2,000 on MI355X at N = 2048)
 */
ar_status_t ar_lamport_all_ranks_residual_rmsnorm(const void *const *xs, void *const *comms,
                                                  int W, const void *residual,
                                                  const void *weight,
                                                  void *const *residual_outs,
                                                  void *const *norm_outs, int64_t M, int64_t N,
                                                  float eps, uint32_t flag, uint32_t max_spins,
                                                  uint32_t *bad_chunks, ar_stream_t stream);

/*
 * LL wire format ([NCCL14] "LL's 16-byte FIFO line", "How LL publishes and
 * waits for flags", "Prerequisite mental model").
 * A FIFO is a ring of 8 steps of step_lines 16-byte lines.  The payload
 * (the 4n bytes of n fp32 values, zero-padded to a multiple of 8) is cut
 * into 8-byte pieces; piece i becomes the line
 *     { u32 bytes[8i..8i+4), u32 flag, u32 bytes[8i+4..8i+8), u32 flag }
 * of step k = first_step + i / step_lines, stored at line
 * (k mod 8) * step_lines + (i mod step_lines), with flag = (uint32)(k + 1).
 * FIFO lines not covered by the payload are left untouched.
 *   src         n fp32, 4-byte aligned (any offset)      else AR_ERR_ALIGN
 *   n           0 <= n <= 2^40                           else AR_ERR_ARG
 *   fifo        ll_fifo_bytes(step_lines) bytes, 16-byte aligned
 *   step_lines  1 <= step_lines <= 2^28                  else AR_ERR_ARG
 *               ll_lines(n) <= 8 * step_lines            else AR_ERR_CAPACITY
 */
ar_status_t ll_pack(const float *src, int64_t n, void *fifo, int64_t step_lines,
                    uint64_t first_step, ar_stream_t stream);

/*
 * LL decode + reduce.  For each line and each FIFO r (in order 0..W-1) the
 * line is accepted only when both flags equal (uint32)(k + 1); otherwise it
 * is re-read up to max_spins times (a bounded wait, never a hang) and, if
 * still not accepted, counted as bad.  Element e (line e / 2, half e mod 2)
 * of the output is the fp32 sum over FIFOs in order 0..W-1 starting from
 * FIFO 0's value.  out[e] is unspecified where a line was bad in any FIFO.
 *   fifos       host table of W device pointers (16-byte aligned)
 *   W           1 <= W <= 8                               else AR_ERR_WORLD
 *   out         n fp32, 4-byte aligned; only out[0..n) is written
 *   n, step_lines  as ll_pack
 *   max_spins   <= AR_MAX_SPINS                           else AR_ERR_ARG
 *   bad_lines   device u32 (4-byte aligned) the caller zeroes; the library
 *               adds the number of bad (FIFO, line) pairs.  NULL: not counted.
 */
ar_status_t ll_unpack_reduce(const void *const *fifos, int W, float *out,
                             int64_t n, int64_t step_lines, uint64_t first_step,
                             uint32_t max_spins, uint32_t *bad_lines,
                             ar_stream_t stream);

/*
 * LL128 wire format ([NCCL14] "LL128's 128-byte line", "LL128's warp-level
 * ready check", "Why LL128 alignment matters").  A 128-byte line is 16 u64
 * words: words 0..14 carry payload bytes [120l, 120l + 120) in order (zero
 * past the end), word 15 carries the flag (uint64)(k + 1).  Steps, slots and
 * placement as for LL with 128-byte lines.  src may sit at any 4-byte offset.
 *   fifo        ll128_fifo_bytes(step_lines) bytes, 128-byte aligned
 *   other arguments and errors as ll_pack
 */
ar_status_t ll128_pack(const float *src, int64_t n, void *fifo,
                       int64_t step_lines, uint64_t first_step,
                       ar_stream_t stream);

/*
 * LL128 decode + reduce: a line is accepted when its flag word equals
 * (uint64)(k + 1); re-reads, bad-line counting and the reduction are as for
 * ll_unpack_reduce, with 30 fp32 values per line.
 */
ar_status_t ll128_unpack_reduce(const void *const *fifos, int W, float *out,
                                int64_t n, int64_t step_lines,
                                uint64_t first_step, uint32_t max_spins,
                                uint32_t *bad_lines, ar_stream_t stream);

/*
 * Streaming through 8-step FIFOs on one device ([NCCL14] "prerequisite
 * mental model": a ring of 8 steps; the sender never overwrites a step the
 * receiver has not consumed and the receiver never consumes a step before it
 * is ready; "how LL publishes and waits for flags", "LL128's warp-level
 * ready check", "how Simple synchronizes").  The 4n payload bytes are cut
 * into steps of step_bytes payload bytes; the T = ceil(4n / step_bytes)
 * steps are dealt to `channels` channels in contiguous runs (channel c takes
 * steps [c*T/channels, (c+1)*T/channels)).  Each channel has an 8-slot ring
 * and one or more producer/consumer workgroup pairs that run concurrently in
 * one launch; with P pairs, pair g owns the same contiguous slice of every
 * step (items [g*span, (g+1)*span), whole LL128 line pairs) and keeps its own
 * head and tail.  The library picks P: as many pairs as the device holds at
 * once, up to AR_FIFO_MAX_PAIRS, at most one per 2,048 items a channel
 * carries in the call, and no more than leave every pair a slice of at
 * least 512 items of a full step.  Local step j of a channel is ring step
 * k = first + j, in slot k mod 8:
 *   AR_PROTO_LL      16-byte lines of 8 payload bytes + two 32-bit flags
 *                    (k + 1), ready when both flags match
 *   AR_PROTO_LL128   128-byte lines of 120 payload bytes + a 64-bit flag
 *                    (k + 1); per batch of 512 lines the producer writes
 *                    every line whole with its flag, except a zero flag in
 *                    the batch's first line, waits until those stores are
 *                    acknowledged, then writes the first line's flag; the
 *                    consumer waits for that flag, then reads every line and
 *                    checks its flag
 *   AR_PROTO_SIMPLE  raw payload; ready when the channel's tail counter
 *                    reaches k + 1
 * After each step a pair's consumer sets the pair's head counter to k + 1
 * (on the LL path where a batch spans S <= 4 whole steps, once per batch,
 * to its last step's k + 1); its producer reuses its slice of slot k mod 8
 * only once head >= k - 7.  A step writes only
 * the lines (or bytes) that carry payload.  The consumer delivers
 * out[e] = src[e], or local[e] + src[e] in fp32 when local is given.
 *   proto       AR_PROTO_LL / AR_PROTO_LL128 / AR_PROTO_SIMPLE
 *   step_bytes  payload bytes per step: a multiple of 8 / 120 / 16, at most
 *               2^30 (NCCL's defaults: 32768 / 576000 / 524288)
 *   fifo        channels * 8 * ar_fifo_step_wire_bytes(proto, step_bytes)
 *               bytes, 16-byte aligned (128 for LL128)
 *   counters    ar_fifo_counter_words(channels) u64, 8-byte aligned: the
 *               heads (channels * AR_FIFO_MAX_PAIRS), the tails (as many),
 *               then {stored first step, finished consumers}.  Zero fifo
 *               and counters together before the first call on them.
 *   channels    1..AR_FIFO_MAX_CHANNELS
 *   first_step  the first ring step of every channel, or AR_FIFO_CONTINUE
 *               for the stored first step.  Each call ends by storing
 *               first + ar_fifo_steps_per_channel(n, step_bytes, channels),
 *               so calls with AR_FIFO_CONTINUE (also from a replayed graph)
 *               keep flags and counters growing.  Explicit values must not
 *               go below the stored step on fifo/counters in use.
 *   max_spins   bound on every wait (<= AR_MAX_SPINS); a wait that runs out
 *               adds 1 to errors[0] and makes every other wait of the launch
 *               give up, so the launch always ends
 *   errors      device u32 the caller zeroes; non-zero afterwards means out
 *               is unspecified and fifo/counters must be zeroed before reuse
 *   src, local, out  n fp32, 4-byte aligned; out may equal local, no other
 *               overlap among the buffers                 else AR_ERR_ARG
 * The 2 * channels * P workgroups must be resident together.  They have
 * 1,024 lanes, or 512 when the device holds two or more pairs per channel
 * of those but only one of the wider ones (for LL also when the 512-lane
 * form gives at least twice the pairs and every channel carries 32 steps
 * or more; ar_fifo_plan reports the choice); AR_ERR_CAPACITY if it cannot hold
 * one pair per channel in either form (with local, more than 128 channels
 * on MI355X).  Work from other streams that holds
 * compute units while a call runs can delay a consumer or producer; the
 * bounded waits then end the launch with errors[0] != 0.
 */
#define AR_PROTO_LL 0
#define AR_PROTO_LL128 1
#define AR_PROTO_SIMPLE 2
#define AR_FIFO_MAX_CHANNELS 256
#define AR_FIFO_MAX_PAIRS 8           /* producer/consumer pairs per channel */
#define AR_FIFO_CONTINUE UINT64_MAX

ar_status_t ar_fifo_stream(int proto, const float *src, const float *local,
                           float *out, int64_t n, void *fifo, uint64_t *counters,
                           int channels, int64_t step_bytes, uint64_t first_step,
                           uint32_t max_spins, uint32_t *errors,
                           ar_stream_t stream);

/* u64 words of the counters of `channels` channels:
 * 2 * channels * AR_FIFO_MAX_PAIRS + 2 (0 if channels is out of range). */
int64_t ar_fifo_counter_words(int channels);

/* Ring bytes per step for a protocol (0 if step_bytes is not valid). */
int64_t ar_fifo_step_wire_bytes(int proto, int64_t step_bytes);

/* Ring steps a call advances every channel's numbering by:
 * ceil(ceil(4n / step_bytes) / channels) (0 for invalid arguments). */
int64_t ar_fifo_steps_per_channel(int64_t n, int64_t step_bytes, int channels);

/* The launch shape ar_fifo_stream picks for these arguments on the current
 * device, without launching anything: *lanes = lanes per workgroup (1,024
 * or 512), *pairs = producer/consumer pairs per channel (P above),
 * *batch_steps = whole ring steps an LL batch spans (1 when batches stay
 * inside one step, and for LL128 and Simple).  Any output may be NULL; all
 * are set to 0 first, and stay 0 for n = 0 (no launch).  with_local != 0
 * plans for a call with a local addend.  Not an operation of the pages: it
 * reports the one-device choices ([NCCL14] "prerequisite mental model"
 * fixes the ring and steps, not how workgroups share them).
 *   AR_ERR_ARG       proto, step_bytes, n or channels as ar_fifo_stream
 *   AR_ERR_CAPACITY  not one pair per channel fits
 *   AR_ERR_HIP       the device could not be queried */
ar_status_t ar_fifo_plan(int proto, int64_t n, int channels, int64_t step_bytes,
                         int with_local, int *lanes, int *pairs, int *batch_steps);

/*
 * Plain device copy, dst[0 .. nbytes) = src[0 .. nbytes), one 16-byte load
 * and store per lane.  Not an operation of the pages: it is the
 * achievable-copy reference that the measurements report beside the reduce
 * and wire kernels (what a kernel moving each byte once reaches here).
 *   src, dst  device pointers, 16-byte aligned            else AR_ERR_ALIGN
 *   nbytes    multiple of 16, 0 <= nbytes <= 2^44; the two ranges must not
 *             overlap                                     else AR_ERR_ARG
 */
ar_status_t ar_copy(const void *src, void *dst, int64_t nbytes, ar_stream_t stream);

/* Geometry helpers ([NCCL14] "Default buffers and effective data per
 * step": the default buffers give 4096 LL lines and 4800 LL128 lines per
 * step).  Arguments outside what the entry points accept (n < 1 or
 * n > 2^40 values, step_lines < 1 or step_lines > 2^28) give 0. */
int64_t ll_lines(int64_t n);                  /* ceil(4n / 8)   */
int64_t ll128_lines(int64_t n);               /* ceil(4n / 120) */
int64_t ll_fifo_bytes(int64_t step_lines);    /* 8 * step_lines * 16  */
int64_t ll128_fifo_bytes(int64_t step_lines); /* 8 * step_lines * 128 */
int64_t ll_default_step_lines(void);          /* 4096 */
int64_t ll128_default_step_lines(void);       /* 4800 */

#ifdef __cplusplus
}
#endif

#endif /* LIBAR_H */
