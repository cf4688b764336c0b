// Host-side check of the streaming slices (built with g++ by
// tests/test_index_map.py): for every pair count the slices that
// fifo_slice() -- the function the kernel calls -- gives the pairs of a
// channel must cut every step into disjoint, unit-aligned pieces that cover
// it exactly, each pair keeping the same region of the ring slot in every
// step, and fifo_pairs_for() -- the host's choice -- must fit the device and
// leave every pair a slice of a full step.
#include <cstdio>
#include <vector>

#include "../ar_rmsnorm_amd/csrc/index_map.h"

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
    const int S = ar::fifo_batch_steps(span, 4096, 4);
    CHECK(S >= 1 && S <= 4, "batch of %d steps", S);
    if (S == 1)
        return;
    for (int g = 0; g < pairs; ++g) {
        int64_t lo = 0, hi_full = 0, lo_last = 0, hi_last = 0;
        ar::fifo_slice_at(span, full, g, &lo, &hi_full);
        ar::fifo_slice_at(span, last_total, g, &lo_last, &hi_last);
        const int64_t len = hi_full - lo;
        if (len <= 0)
            continue;                       // the host never leaves a pair without a slice
        CHECK(S * len <= 4096, "pair %d: %d steps of %lld lines exceed a batch", g, S,
              (long long)len);
        int64_t eff = steps;
        if (hi_last <= lo_last)
            --eff;
        std::vector<std::vector<int>> seen(steps, std::vector<int>(full, 0));
        for (int64_t j0 = 0; j0 < eff; j0 += S) {
            const int n_in = eff - j0 < S ? (int)(eff - j0) : S;
            for (uint32_t v = 0; v < 4096; ++v) {
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
    std::printf("%ld cases checked, %ld failures\n", cases, g_fail);
    return g_fail == 0 ? 0 : 1;
}
