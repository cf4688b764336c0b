// Host-side check of the streaming slices (built with g++ by
// tests/test_index_map.py): for every pair count the slices that
// fifo_slice() -- the function the kernel calls -- gives the pairs of a
// channel must cut every step into disjoint, unit-aligned pieces that cover
// it exactly, each pair keeping the same region of the ring slot in every
// step, and fifo_pairs_for() -- the host's choice -- must fit the device and
// leave every pair a slice of a full step.  The launch plan of
// stream_plan.h is evaluated too: on the shapes the measurements and the
// GPU tests use, with the occupancy of one 256-CU MI355X (one 1,024-lane or
// two 512-lane streaming workgroups per CU), and over a grid of calls for
// the properties every plan must have.
#include <cstdio>
#include <vector>

#include "../ar_rmsnorm_amd/csrc/index_map.h"
#include "../ar_rmsnorm_amd/csrc/stream_plan.h"

static long g_fail = 0;
#define CHECK(c, ...)                                              \
    do {                                                           \
        if (!(c)) {                                                \
            if (g_fail < 20) {                                     \
                std::printf("FAIL full=%lld unit=%lld pairs=%d: ", \
                            (long long)full, (long long)unit, pairs); \
                std::printf(__VA_ARGS__);                          \
                std::printf("\n");                                 \
            }                                                      \
            ++g_fail;                                              \
        }                                                          \
    } while (0)

static void check(int64_t full, int64_t unit, int pairs)
{
    std::vector<int64_t> flo(pairs), fhi(pairs);
    for (int g = 0; g < pairs; ++g)
        ar::fifo_slice(full, full, unit, pairs, g, &flo[g], &fhi[g]);
    // totals: every count up to 600, then a spread up to full
    std::vector<int64_t> totals;
    for (int64_t t = 0; t <= full && t <= 600; ++t)
        totals.push_back(t);
    for (int64_t t = 601; t < full; t += full / 97 + 1)
        totals.push_back(t);
    totals.push_back(full);
    for (int64_t total : totals) {
        int64_t next = 0;
        for (int g = 0; g < pairs; ++g) {
            int64_t lo = -1, hi = -1;
            ar::fifo_slice(full, total, unit, pairs, g, &lo, &hi);
            CHECK(lo == next, "total %lld pair %d starts at %lld, expected %lld", (long long)total,
                  g, (long long)lo, (long long)next);
            CHECK(lo <= hi && hi <= total, "total %lld pair %d: [%lld, %lld)", (long long)total, g,
                  (long long)lo, (long long)hi);
            CHECK(lo == total || lo % unit == 0, "pair %d not unit-aligned", g);
            CHECK(lo == hi || (lo >= flo[g] && hi <= fhi[g]),
                  "total %lld pair %d leaves its region of the slot", (long long)total, g);
            next = hi;
        }
        CHECK(next == total, "total %lld covered up to %lld", (long long)total, (long long)next);
    }
}

// Batches of whole steps (the LL path with fifo_batch_steps() > 1): over a
// channel of `steps` steps whose last one has last_total lines, every line
// of every pair's slice of every step is carried by exactly one lane slot
// (fifo_batch_slot(), as the kernel computes it) of exactly one batch, no
// slot carries a line outside its step's slice, a batch's lines fit its
// 4,096 lane slots, and the batch stays within half the 8-step ring.
static void check_batches(int64_t full, int pairs, int64_t last_total, int64_t steps)
{
    const int64_t unit = 1;
    const int64_t span = ar::fifo_span(full, 1, pairs);
    const int S = ar::fifo_batch_steps(span, ar::kFifoPerBatch, ar::kFifoMaxBatchSteps);
    CHECK(S >= 1 && S <= ar::kFifoMaxBatchSteps && 2 * S <= 8, "batch of %d steps", S);
    if (S == 1)
        return;
    for (int g = 0; g < pairs; ++g) {
        int64_t lo = 0, hi_full = 0, lo_last = 0, hi_last = 0;
        ar::fifo_slice_at(span, full, g, &lo, &hi_full);
        ar::fifo_slice_at(span, last_total, g, &lo_last, &hi_last);
        const int64_t len = hi_full - lo;
        if (len <= 0)
            continue;                       // the host never leaves a pair without a slice
        CHECK(S * len <= ar::kFifoPerBatch, "pair %d: %d steps of %lld lines exceed a batch",
              g, S, (long long)len);
        int64_t eff = steps;
        if (hi_last <= lo_last)
            --eff;
        std::vector<std::vector<int>> seen(steps, std::vector<int>(full, 0));
        for (int64_t j0 = 0; j0 < eff; j0 += S) {
            const int n_in = eff - j0 < S ? (int)(eff - j0) : S;
            for (uint32_t v = 0; v < (uint32_t)ar::kFifoPerBatch; ++v) {
                int step = 0;
                uint32_t line = 0;
                ar::fifo_batch_slot(v, (uint32_t)len, &step, &line);
                if (step >= n_in)
                    continue;
                const int64_t j = j0 + step;
                const int64_t hi = j == steps - 1 ? hi_last : hi_full;
                const int64_t i = lo + (int64_t)line;
                if (i >= hi)
                    continue;
                CHECK(i >= lo && i < full, "pair %d step %lld line %lld outside", g,
                      (long long)j, (long long)i);
                if (i >= 0 && i < full)
                    ++seen[j][i];
            }
        }
        for (int64_t j = 0; j < steps; ++j) {
            const int64_t a = j == steps - 1 ? lo_last : lo, b = j == steps - 1 ? hi_last : hi_full;
            for (int64_t i = 0; i < full; ++i) {
                const int want = i >= a && i < b ? 1 : 0;
                CHECK(seen[j][i] == want, "pair %d step %lld line %lld carried %d times",
                      g, (long long)j, (long long)i, seen[j][i]);
            }
        }
    }
}

// The plan of one call as the host library makes it (libar.hip fifo_plan
// and ar_fifo_plan): lanes, pairs per channel, whole steps per LL batch.
struct Plan {
    int lanes, pairs, steps;
};
constexpr int kWideResident = 256, kNarrowResident = 512;   // one MI355X

static Plan plan_of(int proto, int64_t n, int channels, int64_t step_bytes)
{
    const int wp = ar::fifo_plan_pairs(proto, step_bytes, n, channels, kWideResident);
    const int np = ar::fifo_plan_pairs(proto, step_bytes, n, channels, kNarrowResident);
    const bool wide =
        ar::fifo_plan_wide(proto, wp, np, ar::fifo_steps_per_channel(n, step_bytes, channels));
    const int pairs = wide ? wp : np;
    return {wide ? 1024 : 512, pairs,
            ar::fifo_plan_batch_steps(proto, step_bytes, n, channels, pairs)};
}

static long check_plans()
{
    const int64_t full = 0, unit = 0;   // for CHECK's message
    const int pairs = 0;
    long cases = 0;
    // the bench rows and the GPU tests' cases: protocol, n, channels, step, plan
    struct Want {
        int proto;
        int64_t n;
        int channels;
        int64_t step;
        Plan plan;
    };
    const int64_t mi16 = 1 << 24;
    const Want want[] = {
        {0, mi16, 32, 32768, {512, 8, 4}},      {0, mi16, 128, 32768, {512, 2, 2}},
        {1, mi16, 32, 576000, {1024, 4, 1}},    {1, mi16, 128, 576000, {512, 2, 1}},
        {2, mi16, 32, 524288, {1024, 4, 1}},    {2, mi16, 128, 524288, {512, 2, 1}},
        {0, 2048, 32, 32768, {1024, 1, 1}},     {0, 1 << 22, 32, 32768, {1024, 4, 4}},
        {0, mi16, 64, 32768, {512, 4, 4}},      {0, 48 * 33 * 8192 + 11, 48, 32768, {512, 5, 4}},
        {0, 16 * 3 * 8192 + 5, 16, 32768, {1024, 8, 4}},
        {0, 32 * 3 * 10240 + 7, 32, 40960, {1024, 4, 3}},
        {0, 64 * 2 * 8192 + 3, 64, 32768, {1024, 2, 2}},
        {0, 128 * 2 * 8192, 128, 32768, {512, 2, 2}},
    };
    for (const Want &w : want) {
        const Plan p = plan_of(w.proto, w.n, w.channels, w.step);
        CHECK(p.lanes == w.plan.lanes && p.pairs == w.plan.pairs && p.steps == w.plan.steps,
              "proto %d n %lld channels %d step %lld: plan (%d, %d, %d), expected (%d, %d, %d)",
              w.proto, (long long)w.n, w.channels, (long long)w.step, p.lanes, p.pairs, p.steps,
              w.plan.lanes, w.plan.pairs, w.plan.steps);
        ++cases;
    }
    // every call of a grid: the workgroups fit, every pair has a slice of a
    // full step, and an LL batch of whole steps fits its lane slots and
    // leaves the producer a batch of room in the ring
    for (int proto = 0; proto < 3; ++proto) {
        const int64_t unit_bytes = proto == 0 ? 8 : proto == 1 ? 120 : 16;
        for (int64_t step : {unit_bytes, 64 * unit_bytes, 1000 * unit_bytes, (int64_t)32768,
                             (int64_t)576000, (int64_t)524288}) {
            if (step % unit_bytes != 0)
                continue;
            for (int channels : {1, 2, 7, 32, 48, 64, 100, 128, 200, 256}) {
                for (int64_t n : {(int64_t)1, (int64_t)2048, (int64_t)100003, (int64_t)1 << 20,
                                  (int64_t)1 << 24, (int64_t)3 << 26}) {
                    const Plan p = plan_of(proto, n, channels, step);
                    const int res = p.lanes == 1024 ? kWideResident : kNarrowResident;
                    CHECK(p.pairs >= 1 && p.pairs <= ar::kFifoMaxPairs,
                          "proto %d n %lld channels %d step %lld: %d pairs", proto,
                          (long long)n, channels, (long long)step, p.pairs);
                    CHECK(2 * channels * p.pairs <= res, "proto %d channels %d: does not fit",
                          proto, channels);
                    const int64_t items = ar::fifo_full_items(proto, step);
                    int64_t lo = 0, hi = 0;
                    ar::fifo_slice(items, items, proto == 1 ? 16 : 1, p.pairs, p.pairs - 1, &lo,
                                   &hi);
                    CHECK(lo < hi, "proto %d channels %d: the last pair has no slice", proto,
                          channels);
                    CHECK(p.steps >= 1 && p.steps <= ar::kFifoMaxBatchSteps &&
                              (proto == 0 || p.steps == 1),
                          "proto %d: %d steps per batch", proto, p.steps);
                    if (p.steps > 1) {
                        const int64_t span = ar::fifo_span(items, 1, p.pairs);
                        CHECK(p.steps * span <= ar::kFifoPerBatch,
                              "n %lld channels %d: %d steps of %lld lines exceed a batch",
                              (long long)n, channels, p.steps, (long long)span);
                        CHECK(ar::fifo_steps_per_channel(n, step, channels) >= 2,
                              "batches of whole steps on channels of one step");
                    }
                    ++cases;
                }
            }
        }
    }
    return cases;
}

int main()
{
    long cases = 0;
    const int64_t fulls[] = {1, 2, 3, 7, 8, 16, 24, 31, 32, 100, 127, 256, 1000, 2048, 2160,
                             4096, 4800 * 8, 32768, 69906 * 8, 131072 / 16, 1 << 20};
    for (int64_t unit : {1, 16}) {
        for (int64_t full : fulls) {
            if (unit == 16 && full % 8 != 0)
                continue;                       // LL128 steps are whole lines
            for (int pairs = 1; pairs <= 8; ++pairs) {
                check(full, unit, pairs);
                ++cases;
            }
            for (int64_t min_slice : {1, 512})
            for (int channels : {1, 2, 3, 32, 100, 128, 200, 256}) {
                for (int resident : {0, 1, 2, 255, 256, 511, 512, 2048}) {
                    const int pairs = ar::fifo_pairs_for(full, unit, channels, resident, 8,
                                                         min_slice);
                    const int pairs_ = pairs;
                    {
                        const int pairs = pairs_;
                        CHECK(pairs >= 0 && pairs <= 8, "pairs %d", pairs);
                        CHECK((pairs >= 1) == (resident >= 2 * channels),
                              "channels %d resident %d gave %d pairs", channels, resident, pairs);
                        CHECK(2 * channels * pairs <= resident || pairs == 0, "does not fit");
                        if (pairs >= 1) {
                            int64_t lo = 0, hi = 0;
                            ar::fifo_slice(full, full, unit, pairs, pairs - 1, &lo, &hi);
                            CHECK(lo < hi, "last pair has no slice of a full step");
                            CHECK(pairs == 1 || hi - lo >= min_slice, "slice under the minimum");
                        }
                    }
                    ++cases;
                }
            }
        }
    }
    for (int64_t full : {600, 1000, 1024, 2048, 2049, 4096, 8192, 16384}) {
        for (int pairs = 1; pairs <= 8; ++pairs) {
            for (int64_t steps : {1, 2, 3, 4, 5, 7, 8, 9, 13, 16}) {
                for (int64_t last : {full, full - 1, full / 2, (int64_t)1, full * 3 / 4 + 1}) {
                    check_batches(full, pairs, last, steps);
                    ++cases;
                }
            }
        }
    }
    cases += check_plans();
    std::printf("%ld cases checked, %ld failures\n", cases, g_fail);
    return g_fail == 0 ? 0 : 1;
}
