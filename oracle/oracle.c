/*
 * Plain, slow CPU oracle for the per-GPU reduction of a custom all-reduce.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link, load or call this file.  Only the
 * tests, the smoke check and the CPU-baseline leg of the bench use it.  It
 * shares no code, header, table or helper with the HIP path.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 *        (x86-64 SSE arithmetic: every float operation is one IEEE-754
 *        binary32 operation rounded to nearest-even; no excess precision,
 *        no fused multiply-add).
 *
 * Sources (web pages; cited by tag and section):
 *   [SGLv1]  "SGLang Custom AllReduce v1 线程模型和工作原理细节" (todaynews.cc)
 *   [NCCL14] "NCCL 专家课程 14：Simple、LL、LL128 的线格式、同步与真实性能边界"
 *            (blog.cptz.space)
 *   [JITAR]  "0-custom-all-reduce" (obnotes-4iw.pages.dev, sglang jit_kernel)
 *   [TRIAR]  "用 Triton + Symmetric Memory 写一个 AllReduce + RMSNorm 融合算子"
 *            (riverclouds.net)
 *
 * Pins (the tests that tie each function to something other than itself):
 *   orc_bf16_rne        torch CPU float32->bfloat16 (a library RNE) over every
 *                       low half-word of 256 high half-words; hand cases.
 *   orc_bf16_from_f64   exact rational brute force on random doubles.
 *   orc_reduce_1stage   closed forms (ones -> W, r+1 -> W(W+1)/2, all -0.0),
 *                       W=2 exact-sum special case, an order-revealing case
 *                       whose rank-order result is derived by hand.
 *   orc_reduce_2stage   partition numbers printed on [SGLv1], W=2 equality
 *                       with 1stage, hand-derived rotated-order case.
 *   orc_fused_...       constant rows (closed form incl. eps), W-1 zero
 *                       inputs reduce to torch's rms_norm (library routine),
 *                       power-of-two scale invariance with eps = 0.
 *   orc_ll_* / ll128_*  hand-written golden wire bytes (tests/golden), the
 *                       buffer/step constants printed on [NCCL14], round trip,
 *                       exact bad-line counts for planted corruptions.
 *   orc_lamport_*       hand-packed words, exhaustive check that no packed
 *                       word equals the sentinel, a hand-derived W=2 region
 *                       example, equality with the (pinned) fused operator
 *                       when no input is -0.0, exact missing-push counts.
 *   orc_fused_2stage*   row partition numbers, equality with the one-shot
 *                       fused operator for W=2 or rank order, a hand-derived
 *                       rotated case.
 *   orc_fifo_*          payload delivered bit for bit, one lap equal to the
 *                       (pinned) packers, the last-lap ring contents and the
 *                       channel split derived by hand, [NCCL14]'s step table.
 * No function here is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------------
 * bf16 <-> fp32.
 * [JITAR] section 4 "sum (reduce_impl)": inputs are widened to fp32, summed,
 * and the result is narrowed once with round-to-nearest.  The pages do not
 * cover NaN/Inf/denormals; IEEE round-to-nearest-even with denormals kept and
 * NaN made quiet (sign kept) is the reading taken here.
 * ------------------------------------------------------------------------- */

/* A bf16 value is the top half of the fp32 with the same bits, so widening
 * is exact. */
float orc_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round an fp32 to the nearest bf16, ties to even.  The 16 dropped bits are
 * compared with one half-unit: adding 0x7FFF plus the lowest kept bit carries
 * into the kept part exactly when the dropped part is above half, or equal to
 * half with an odd kept part.  Overflow carries into the exponent and gives
 * the infinity of the same sign. */
uint16_t orc_bf16_rne(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN, sign kept */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Round a double straight to the nearest bf16, ties to even (no detour via
 * fp32, so no double rounding).  bf16 keeps 8 significant bits; below the
 * smallest normal (2^-126) its spacing stays 2^-133. */
uint16_t orc_bf16_from_f64(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(x);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);                /* a = m * 2^e with m in [0.5, 1) */
    int qexp = e - 8;            /* spacing of the 8-bit significand */
    if (qexp < -133)
        qexp = -133;
    double q = nearbyint(ldexp(a, -qexp)); /* ties to even (default mode) */
    double r = ldexp(q, qexp);             /* at most 8 significant bits */
    if (r > 3.3895313892515355e38)         /* above the largest bf16 */
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)r;                    /* exact */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

/* ---------------------------------------------------------------------------
 * One-stage reduce.
 * [SGLv1] section "1stage: full kernel and timeline": every element is the
 * fp32 sum of the W rank buffers taken in the fixed order 0..W-1, starting
 * from rank 0's value (not from zero), then narrowed once to bf16.  The same
 * order on every rank makes every rank's output bit-identical.
 * [JITAR] section 4 gives the same sum but starts from +0.0; the two differ
 * only when all W inputs are -0.0.  The [SGLv1] start is taken.
 * ------------------------------------------------------------------------- */
void orc_reduce_1stage(const uint16_t *const *x, int W, uint16_t *out, int64_t n)
{
    for (int64_t j = 0; j < n; ++j) {
        float acc = orc_bf16_to_f32(x[0][j]);
        for (int r = 1; r < W; ++r)
            acc = acc + orc_bf16_to_f32(x[r][j]);
        out[j] = orc_bf16_rne(acc);
    }
}

/* ---------------------------------------------------------------------------
 * Two-stage reduce = reduce-scatter + all-gather.
 * [SGLv1] section "2stage: sharding, rotation, and why no exit barrier":
 * the message is cut into 16-byte packs (8 bf16); part = packs / W; shard s
 * covers packs [s*part, (s+1)*part), except that the last shard also takes
 * the remainder.  The owner of shard s sums it in the rotated order
 * s, s+1, ..., s-1 (mod W) and rounds once; the all-gather copies the W
 * shards into place, so every rank ends with the same bits.
 * rank_order != 0 selects the 0..W-1 order of the one-stage form instead.
 * ------------------------------------------------------------------------- */

/* Pack range [*first, *last) of shard s. */
void orc_shard_range(int64_t n, int W, int s, int64_t *first, int64_t *last)
{
    int64_t packs = n / 8;
    int64_t part = packs / W;
    *first = (int64_t)s * part;
    *last = (s == W - 1) ? packs : *first + part;
}

/* Reduce-scatter of shard s into tmp (tmp[0] is the shard's first element). */
void orc_reduce_scatter(const uint16_t *const *x, int W, int s, uint16_t *tmp,
                        int64_t n, int rank_order)
{
    int64_t p0, p1;
    orc_shard_range(n, W, s, &p0, &p1);
    for (int64_t j = p0 * 8; j < p1 * 8; ++j) {
        int first = rank_order ? 0 : s;
        float acc = orc_bf16_to_f32(x[first][j]);
        for (int i = 1; i < W; ++i) {
            int r = rank_order ? i : (s + i) % W;
            acc = acc + orc_bf16_to_f32(x[r][j]);
        }
        tmp[j - p0 * 8] = orc_bf16_rne(acc);
    }
}

/* All-gather: shard s is copied from its owner's staging buffer tmps[s] to
 * its place in out. */
void orc_all_gather(const uint16_t *const *tmps, int W, uint16_t *out, int64_t n)
{
    for (int s = 0; s < W; ++s) {
        int64_t p0, p1;
        orc_shard_range(n, W, s, &p0, &p1);
        for (int64_t j = p0 * 8; j < p1 * 8; ++j)
            out[j] = tmps[s][j - p0 * 8];
    }
}

/* Full two-stage result: every shard reduced by its owner into its staging
 * buffer, then gathered.  The result does not depend on which rank gathers
 * it.  Returns -1 if the staging buffers cannot be allocated. */
int orc_reduce_2stage(const uint16_t *const *x, int W, uint16_t *out,
                      int64_t n, int rank_order)
{
    uint16_t *tmps[8] = {0};
    for (int s = 0; s < W; ++s) {
        int64_t p0, p1;
        orc_shard_range(n, W, s, &p0, &p1);
        tmps[s] = (uint16_t *)malloc((size_t)((p1 - p0) * 8 + 1) * sizeof(uint16_t));
        if (!tmps[s]) {
            for (int t = 0; t < s; ++t)
                free(tmps[t]);
            return -1;
        }
        orc_reduce_scatter(x, W, s, tmps[s], n, rank_order);
    }
    orc_all_gather((const uint16_t *const *)tmps, W, out, n);
    for (int s = 0; s < W; ++s)
        free(tmps[s]);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Fused all-reduce + residual + RMSNorm.
 * [TRIAR] section "what this operator computes": ar = sum over ranks of x;
 * h = ar + residual (this is residual_out); rms = rsqrt(mean(h^2) + eps);
 * out = (h * rms) * weight.  Section "overall design": one row at a time,
 * fp32 accumulation, the sum kept in registers for the norm, so the norm
 * uses the fp32 h, not the bf16-rounded residual_out.
 * The all-reduce part is the [SGLv1] one-stage sum (rank order, start at
 * rank 0).  h is an fp32 add, so residual_out is exact.  The statistics and
 * the scaling are done here in double; norm_exact receives the unrounded
 * double product and norm_out its bf16 rounding.
 * ------------------------------------------------------------------------- */
void orc_fused_residual_rmsnorm(const uint16_t *const *x, int W,
                                const uint16_t *residual, const uint16_t *weight,
                                uint16_t *residual_out, uint16_t *norm_out,
                                double *norm_exact, int64_t M, int64_t N,
                                double eps, float *h_scratch)
{
    for (int64_t m = 0; m < M; ++m) {
        const int64_t row = m * N;
        double ss = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            float a = orc_bf16_to_f32(x[0][row + j]);
            for (int r = 1; r < W; ++r)
                a = a + orc_bf16_to_f32(x[r][row + j]);
            float h = a + orc_bf16_to_f32(residual[row + j]);
            h_scratch[j] = h;
            residual_out[row + j] = orc_bf16_rne(h);
            ss += (double)h * (double)h;
        }
        double rms = 1.0 / sqrt(ss / (double)N + eps);
        for (int64_t j = 0; j < N; ++j) {
            double y = ((double)h_scratch[j] * rms) * (double)orc_bf16_to_f32(weight[j]);
            if (norm_exact)
                norm_exact[row + j] = y;
            norm_out[row + j] = orc_bf16_from_f64(y);
        }
    }
}

/* ---------------------------------------------------------------------------
 * FIFO geometry shared by LL and LL128.
 * [NCCL14] section "prerequisite mental model": the connection buffer is a
 * ring of 8 steps.  Section "how LL publishes and waits for flags": a step's
 * lines start at (step mod 8) * step_lines and the flag that marks a line of
 * step k as ready is the value k + 1 (NCCL_LL_FLAG's body is not shown; it
 * is read as plain truncation to the flag width).
 * Line i of a call belongs to step first_step + i / step_lines.
 * ------------------------------------------------------------------------- */
static int64_t wire_index(int64_t i, int64_t step_lines, uint64_t first_step,
                          uint64_t *step)
{
    uint64_t k = first_step + (uint64_t)(i / step_lines);
    *step = k;
    return (int64_t)(k % 8u) * step_lines + i % step_lines;
}

static uint32_t get_u32le(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
           ((uint32_t)p[3] << 24);
}

static void put_u32le(uint8_t *p, uint32_t v)
{
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
    p[2] = (uint8_t)(v >> 16);
    p[3] = (uint8_t)(v >> 24);
}

static void put_u64le(uint8_t *p, uint64_t v)
{
    put_u32le(p, (uint32_t)v);
    put_u32le(p + 4, (uint32_t)(v >> 32));
}

static uint64_t get_u64le(const uint8_t *p)
{
    return (uint64_t)get_u32le(p) | ((uint64_t)get_u32le(p + 4) << 32);
}

/* Payload byte b of a message of nbytes bytes, zero past the end. */
static uint8_t payload_byte(const uint8_t *src, int64_t nbytes, int64_t b)
{
    return b < nbytes ? src[b] : 0;
}

/* ---------------------------------------------------------------------------
 * LL wire format.
 * [NCCL14] section "LL's 16-byte FIFO line": a 16-byte line carries 8 bytes
 * of data as two 32-bit halves, each followed by a 32-bit flag, in the order
 * data1, flag1, data2, flag2.  Section "how LL publishes and waits for
 * flags": the sender writes {low 32 bits, flag, high 32 bits, flag}; the
 * receiver accepts the line only when both flags equal the expected value
 * and rebuilds the 8 bytes as data1 + (data2 << 32).
 * ------------------------------------------------------------------------- */
int64_t orc_ll_lines(int64_t n) { return (4 * n + 7) / 8; }

/* Encode n fp32 values (given as their 4n bytes, any alignment) into the
 * FIFO.  Bytes of the FIFO outside the written lines are left untouched. */
void orc_ll_pack(const uint8_t *src, int64_t n, uint8_t *fifo,
                 int64_t step_lines, uint64_t first_step)
{
    const int64_t nbytes = 4 * n, lines = orc_ll_lines(n);
    for (int64_t i = 0; i < lines; ++i) {
        uint8_t data[8];
        for (int b = 0; b < 8; ++b)
            data[b] = payload_byte(src, nbytes, 8 * i + b);
        uint64_t k;
        uint8_t *line = fifo + 16 * wire_index(i, step_lines, first_step, &k);
        uint32_t flag = (uint32_t)(k + 1);
        put_u32le(line + 0, get_u32le(data));     /* data1 */
        put_u32le(line + 4, flag);                /* flag1 */
        put_u32le(line + 8, get_u32le(data + 4)); /* data2 */
        put_u32le(line + 12, flag);               /* flag2 */
    }
}

/* Decode W FIFOs and add them element by element in FIFO order 0..W-1
 * (fp32, starting from FIFO 0's value).  A (FIFO, line) pair whose two flags
 * are not both the expected value is counted as bad; valid[e] (if given) is
 * set to 0 for elements of a line that is bad in any FIFO, else 1, and out[e]
 * is then left unspecified.  Returns the number of bad (FIFO, line) pairs.
 * There is no concurrent writer here, so one read of each line is final. */
int64_t orc_ll_unpack_reduce(const uint8_t *const *fifos, int W, float *out,
                             uint8_t *valid, int64_t n, int64_t step_lines,
                             uint64_t first_step)
{
    int64_t bad = 0;
    const int64_t lines = orc_ll_lines(n);
    for (int64_t i = 0; i < lines; ++i) {
        uint64_t k;
        int64_t w = wire_index(i, step_lines, first_step, &k);
        uint32_t expect = (uint32_t)(k + 1);
        float acc[2] = {0.0f, 0.0f};
        int ok_all = 1;
        for (int r = 0; r < W; ++r) {
            const uint8_t *line = fifos[r] + 16 * w;
            uint32_t d1 = get_u32le(line + 0), f1 = get_u32le(line + 4);
            uint32_t d2 = get_u32le(line + 8), f2 = get_u32le(line + 12);
            if (f1 != expect || f2 != expect) {
                ++bad;
                ok_all = 0;
            }
            uint64_t v = (uint64_t)d1 + ((uint64_t)d2 << 32);
            for (int h = 0; h < 2; ++h) {
                uint32_t bits = (uint32_t)(v >> (32 * h));
                float f;
                memcpy(&f, &bits, 4);
                acc[h] = (r == 0) ? f : acc[h] + f;
            }
        }
        for (int h = 0; h < 2; ++h) {
            int64_t e = 2 * i + h;
            if (e < n) {
                out[e] = acc[h];
                if (valid)
                    valid[e] = (uint8_t)ok_all;
            }
        }
    }
    return bad;
}

/* ---------------------------------------------------------------------------
 * LL128 wire format.
 * [NCCL14] section "LL128's 128-byte line": a 128-byte line is 16 u64 words,
 * 15 of data and 1 flag (120 of 128 bytes carry payload).  Section "LL128's
 * warp-level ready check": the receiver validates a line by its flag word
 * against the expected step + 1 (64-bit).  NCCL spreads a line's 16-byte
 * chunks over threads in its own order; with no NCCL peer to talk to, the
 * plain reading is taken: bytes 120l .. 120l+119 of the payload in words
 * 0..14 in order, the flag in word 15.
 * ------------------------------------------------------------------------- */
int64_t orc_ll128_lines(int64_t n) { return (4 * n + 119) / 120; }

void orc_ll128_pack(const uint8_t *src, int64_t n, uint8_t *fifo,
                    int64_t step_lines, uint64_t first_step)
{
    const int64_t nbytes = 4 * n, lines = orc_ll128_lines(n);
    for (int64_t l = 0; l < lines; ++l) {
        uint64_t k;
        uint8_t *line = fifo + 128 * wire_index(l, step_lines, first_step, &k);
        for (int b = 0; b < 120; ++b)
            line[b] = payload_byte(src, nbytes, 120 * l + b);
        put_u64le(line + 120, k + 1);
    }
}

int64_t orc_ll128_unpack_reduce(const uint8_t *const *fifos, int W, float *out,
                                uint8_t *valid, int64_t n, int64_t step_lines,
                                uint64_t first_step)
{
    int64_t bad = 0;
    const int64_t lines = orc_ll128_lines(n);
    for (int64_t l = 0; l < lines; ++l) {
        uint64_t k;
        int64_t w = wire_index(l, step_lines, first_step, &k);
        int ok_all = 1;
        float acc[30];
        for (int r = 0; r < W; ++r) {
            const uint8_t *line = fifos[r] + 128 * w;
            if (get_u64le(line + 120) != k + 1) {
                ++bad;
                ok_all = 0;
            }
            for (int q = 0; q < 30; ++q) {
                uint32_t bits = get_u32le(line + 4 * q);
                float f;
                memcpy(&f, &bits, 4);
                acc[q] = (r == 0) ? f : acc[q] + f;
            }
        }
        for (int q = 0; q < 30; ++q) {
            int64_t e = 30 * l + q;
            if (e < n) {
                out[e] = acc[q];
                if (valid)
                    valid[e] = (uint8_t)ok_all;
            }
        }
    }
    return bad;
}

/* Element-wise array forms of the two roundings, for callers that hold whole
 * arrays. */
void orc_bf16_rne_array(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_rne(x[i]);
}

void orc_bf16_from_f64_array(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_from_f64(x[i]);
}

/* ---------------------------------------------------------------------------
 * Lamport data-as-flag wire for the fused one-shot.
 * [TRIAR] "Option 2: Lamport": each rank pushes its bf16 row to every peer
 * as u32 words holding two bf16 (element 2j in the low half).  Before
 * packing, a bf16 -0.0 (0x8000) is scrubbed to +0.0, so no word can equal
 * the sentinel 0x80008000 (two -0.0) that fills an empty comm buffer; a
 * reader polls until no word is the sentinel.  The buffer is used in three
 * regions selected by flag mod 3, the flag growing by one per launch.
 * Layout read here: comm[region][slot r][row m][word j], region = flag % 3,
 * slot = the pushing rank.  After reading region flag % 3 the reader resets
 * the region before it, (region + 2) % 3 (the region of the previous call),
 * to the sentinel: every peer finished writing it before the previous call
 * could complete, and peers write it again only two calls later.
 * Reading taken for the counter's width: a 32-bit flag wraps at
 * ORC_LAMPORT_FLAG_PERIOD = 3 * 2^30, a multiple of 3, so that "one more per
 * launch" keeps the region sequence 0, 1, 2, 0, ... across the wrap; flags at
 * or above the period are not valid and the functions below refuse them
 * (push: nothing written; reader: returns -1, nothing written).
 * ------------------------------------------------------------------------- */
#define ORC_LAMPORT_SENTINEL 0x80008000u
#define ORC_LAMPORT_FLAG_PERIOD 0xC0000000u

uint32_t orc_lamport_next_flag(uint32_t flag)
{
    return flag + 1u >= ORC_LAMPORT_FLAG_PERIOD ? 0u : flag + 1u;
}

uint32_t orc_lamport_pack(uint16_t lo, uint16_t hi)
{
    if (lo == 0x8000u)
        lo = 0;
    if (hi == 0x8000u)
        hi = 0;
    return (uint32_t)lo | ((uint32_t)hi << 16);
}

/* Rank `rank` pushes its [M, N] row block into every rank's comm buffer. */
void orc_lamport_push(const uint16_t *x, int W, int rank, uint32_t *const *comms,
                      int64_t M, int64_t N, uint32_t flag)
{
    if (flag >= ORC_LAMPORT_FLAG_PERIOD)
        return;
    const int64_t words = M * N / 2;
    const int64_t region = (int64_t)(flag % 3u);
    for (int p = 0; p < W; ++p) {
        uint32_t *slot = comms[p] + (region * W + rank) * words;
        for (int64_t q = 0; q < words; ++q)
            slot[q] = orc_lamport_pack(x[2 * q], x[2 * q + 1]);
    }
}

/* Reader side for one rank: returns the number of (slot, 16-byte chunk)
 * units that still hold a sentinel word (their outputs are unspecified).
 * The reduction and the norm are the fused operator above, applied to the
 * unpacked slots in slot order 0..W-1. */
int64_t orc_lamport_fused_residual_rmsnorm(uint32_t *comm, int W,
                                           const uint16_t *residual,
                                           const uint16_t *weight,
                                           uint16_t *residual_out,
                                           uint16_t *norm_out, double *norm_exact,
                                           int64_t M, int64_t N, double eps,
                                           uint32_t flag)
{
    if (flag >= ORC_LAMPORT_FLAG_PERIOD)
        return -1;
    const int64_t words = M * N / 2;
    const int64_t region = (int64_t)(flag % 3u);
    int64_t bad = 0;
    uint16_t *xs[8] = {0};
    for (int r = 0; r < W; ++r) {
        const uint32_t *slot = comm + (region * W + r) * words;
        xs[r] = (uint16_t *)malloc((size_t)(M * N) * sizeof(uint16_t));
        for (int64_t q = 0; q < words; ++q) {
            xs[r][2 * q] = (uint16_t)(slot[q] & 0xFFFFu);
            xs[r][2 * q + 1] = (uint16_t)(slot[q] >> 16);
        }
        for (int64_t c = 0; c < words / 4; ++c) {
            int any = 0;
            for (int k = 0; k < 4; ++k)
                any |= slot[4 * c + k] == ORC_LAMPORT_SENTINEL;
            bad += any;
        }
    }
    float *h = (float *)malloc((size_t)N * sizeof(float));
    orc_fused_residual_rmsnorm((const uint16_t *const *)xs, W, residual, weight,
                               residual_out, norm_out, norm_exact, M, N, eps, h);
    free(h);
    for (int r = 0; r < W; ++r)
        free(xs[r]);
    const int64_t stale = (region + 2) % 3;
    for (int64_t q = 0; q < (int64_t)W * words; ++q)
        comm[stale * W * words + q] = ORC_LAMPORT_SENTINEL;
    return bad;
}

/* ---------------------------------------------------------------------------
 * Two-shot fused all-reduce + residual + RMSNorm: the two-stage structure of
 * [SGLv1] "2stage: sharding, rotation, and why no exit barrier" applied to
 * rows, so that each row's statistic stays with one owner ([TRIAR] "overall
 * design" keeps a row whole).  Rows are cut into W shards: part = M / W,
 * shard s = rows [s*part, (s+1)*part), the last shard also taking the
 * remainder.  The owner of shard s applies the fused operator to its rows,
 * summing in the rotated order s, s+1, ..., s-1 (rank_order != 0: 0..W-1),
 * and stages residual_out and norm_out rows; the gather copies every shard's
 * rows into place.
 * ------------------------------------------------------------------------- */
void orc_row_shard_range(int64_t M, int W, int s, int64_t *first, int64_t *last)
{
    int64_t part = M / W;
    *first = (int64_t)s * part;
    *last = (s == W - 1) ? M : *first + part;
}

/* Owner s's reduce-scatter: stage[0 .. rows*N) = residual_out rows,
 * stage[rows*N .. 2*rows*N) = norm_out rows, norm_exact (optional) likewise
 * for its rows only. */
void orc_fused_2stage_scatter(const uint16_t *const *x, int W, int s,
                              const uint16_t *residual, const uint16_t *weight,
                              uint16_t *stage, double *norm_exact, int64_t M,
                              int64_t N, double eps, int rank_order)
{
    int64_t m0, m1;
    orc_row_shard_range(M, W, s, &m0, &m1);
    const int64_t rows = m1 - m0;
    if (rows == 0)
        return;
    const uint16_t *xs[8];
    for (int i = 0; i < W; ++i)
        xs[i] = x[rank_order ? i : (s + i) % W] + m0 * N;
    float *h = (float *)malloc((size_t)N * sizeof(float));
    orc_fused_residual_rmsnorm(xs, W, residual + m0 * N, weight, stage, stage + rows * N,
                               norm_exact, rows, N, eps, h);
    free(h);
}

/* The whole two-shot result (every shard staged by its owner, then
 * gathered); the same for every rank. */
void orc_fused_2stage(const uint16_t *const *x, int W, const uint16_t *residual,
                      const uint16_t *weight, uint16_t *residual_out,
                      uint16_t *norm_out, double *norm_exact, int64_t M, int64_t N,
                      double eps, int rank_order)
{
    for (int s = 0; s < W; ++s) {
        int64_t m0, m1;
        orc_row_shard_range(M, W, s, &m0, &m1);
        const int64_t rows = m1 - m0;
        uint16_t *stage = (uint16_t *)malloc((size_t)(2 * rows * N + 1) * sizeof(uint16_t));
        orc_fused_2stage_scatter(x, W, s, residual, weight, stage,
                                 norm_exact ? norm_exact + m0 * N : NULL, M, N, eps,
                                 rank_order);
        for (int64_t q = 0; q < rows * N; ++q) {
            residual_out[m0 * N + q] = stage[q];
            norm_out[m0 * N + q] = stage[rows * N + q];
        }
        free(stage);
    }
}

/* ---------------------------------------------------------------------------
 * Streaming through an 8-step FIFO ([NCCL14] "prerequisite mental model":
 * a ring of NCCL_STEPS = 8 steps, the sender never overwriting a step the
 * receiver has not consumed; "how LL publishes and waits for flags", "LL128's
 * 128-byte line", "how Simple synchronizes").  The payload (4n bytes) is cut
 * into steps of step_bytes payload bytes; the T steps are dealt to
 * `channels` channels in contiguous runs (channel c takes steps
 * [c*T/G, (c+1)*T/G)), each channel owning its own 8-slot ring.  Local step
 * j of a channel is ring step k = first_step + j, stored in slot k mod 8 of
 * that channel's ring:
 *   LL     step_bytes/8 lines of 16 bytes (as orc_ll_pack, flag = k + 1)
 *   LL128  step_bytes/120 lines of 128 bytes (as orc_ll128_pack)
 *   Simple step_bytes raw payload bytes (readiness is a separate counter)
 * A step writes only the lines (LL, LL128) or bytes (Simple) that carry
 * payload, so the last step of a message may be partial; padding bytes of a
 * partial line are zero.  The receiver delivers out[e] = src[e], or
 * local[e] + src[e] (fp32) when a local buffer is given.  Every step is written into its slot in order, so
 * the ring ends holding the last lap of each channel: that final state is
 * what this function leaves in `fifo`.
 * proto: 0 = LL, 1 = LL128, 2 = Simple.
 * ------------------------------------------------------------------------- */
int64_t orc_fifo_step_wire_bytes(int proto, int64_t step_bytes)
{
    if (proto == 0)
        return step_bytes / 8 * 16;
    if (proto == 1)
        return step_bytes / 120 * 128;
    return step_bytes;
}

int64_t orc_fifo_total_steps(int64_t n, int64_t step_bytes)
{
    return (4 * n + step_bytes - 1) / step_bytes;
}

void orc_fifo_stream(int proto, const uint8_t *src, const float *local, float *out,
                     int64_t n, uint8_t *fifo, int channels, int64_t step_bytes,
                     uint64_t first_step)
{
    const int64_t nbytes = 4 * n;
    const int64_t T = orc_fifo_total_steps(n, step_bytes);
    const int64_t wire = orc_fifo_step_wire_bytes(proto, step_bytes);
    for (int c = 0; c < channels; ++c) {
        const int64_t s0 = (int64_t)c * T / channels, s1 = (int64_t)(c + 1) * T / channels;
        uint8_t *ring = fifo + (int64_t)c * 8 * wire;
        for (int64_t g = s0; g < s1; ++g) {
            const uint64_t k = first_step + (uint64_t)(g - s0);
            uint8_t *slot = ring + (int64_t)(k % 8u) * wire;
            const int64_t b0 = g * step_bytes;
            const int64_t len = nbytes - b0 < step_bytes ? nbytes - b0 : step_bytes;
            if (proto == 0) {
                for (int64_t i = 0; i < (len + 7) / 8; ++i) {
                    uint8_t d[8];
                    for (int b = 0; b < 8; ++b)
                        d[b] = payload_byte(src, nbytes, b0 + 8 * i + b);
                    put_u32le(slot + 16 * i + 0, get_u32le(d));
                    put_u32le(slot + 16 * i + 4, (uint32_t)(k + 1));
                    put_u32le(slot + 16 * i + 8, get_u32le(d + 4));
                    put_u32le(slot + 16 * i + 12, (uint32_t)(k + 1));
                }
            } else if (proto == 1) {
                for (int64_t l = 0; l < (len + 119) / 120; ++l) {
                    for (int b = 0; b < 120; ++b)
                        slot[128 * l + b] = payload_byte(src, nbytes, b0 + 120 * l + b);
                    put_u64le(slot + 128 * l + 120, k + 1);
                }
            } else {
                for (int64_t b = 0; b < len; ++b)
                    slot[b] = src[b0 + b];
            }
        }
    }
    for (int64_t e = 0; e < n; ++e) {
        float v;
        memcpy(&v, src + 4 * e, 4);
        out[e] = local ? local[e] + v : v;
    }
}
