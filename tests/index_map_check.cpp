// Host-side enumeration of the two-stage reduce's launches (built with g++
// by tests/test_index_map.py).  For every (block, lane, pack) of a launch it
// asks two_stage_lane() -- the function the kernel itself calls -- what the
// lane touches, and checks that every read and write falls inside its
// buffer, that the reduce lanes keep the same-thread mapping, and that each
// output and staging pack is written exactly once.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../ar_rmsnorm_amd/csrc/index_map.h"

using ar::TwoStageGrid;
using ar::TwoStageLane;

static long g_failures = 0;

#define CHECK(cond, ...)                                           \
    do {                                                           \
        if (!(cond)) {                                             \
            if (g_failures < 20) {                                 \
                std::printf("FAIL W=%d P=%lld rank=%d rs=%d ag=%d threads=%d rpl=%d cpl=%d: ", \
                            W, (long long)P, rank, (int)rs, (int)ag, threads, rpl, cpl); \
                std::printf(__VA_ARGS__);                          \
                std::printf("\n");                                 \
            }                                                      \
            ++g_failures;                                          \
        }                                                          \
    } while (0)

// One launch of one rank.  Buffers: W inputs of P packs, W staging buffers of
// cap packs (the header's minimum), out of P packs.
static void check_launch(int W, long long P, int rank, bool rs, bool ag, int threads, int rpl,
                         int cpl)
{
    const TwoStageGrid g = ar::two_stage_grid(W, rank, P, rs, ag, threads, rpl, cpl);
    CHECK(g.blocks >= 0 && g.blocks < (1LL << 32), "grid of %lld blocks", (long long)g.blocks);
    CHECK(g.cap == g.part + g.rem && g.part == P / W && g.rem == P % W, "partition");
    std::vector<unsigned char> out_writes((size_t)P, 0), tmp_writes((size_t)g.cap, 0);
    for (long long b = 0; b < g.blocks; ++b) {
        for (int t = 0; t < threads; ++t) {
            for (int c = 0; c < (rpl > cpl ? rpl : cpl); ++c) {
                const TwoStageLane l =
                    ar::two_stage_lane(g, W, rank, rs, threads, rpl, cpl, b, t, c);
                if (l.kind == 0)
                    continue;
                if (l.kind == 1) {
                    CHECK(rs && b < g.rs_blocks && c < rpl, "reduce lane outside the reduce blocks");
                    CHECK(l.read >= 0 && l.read < P, "input pack %lld of %lld", (long long)l.read, P);
                    CHECK(l.tmp >= 0 && l.tmp < g.own && g.own <= g.cap,
                          "staging pack %lld of %lld", (long long)l.tmp, (long long)g.cap);
                    CHECK(l.read == (long long)rank * g.part + l.tmp, "reduce read is not its shard pack");
                    if (l.tmp >= 0 && l.tmp < g.cap)
                        ++tmp_writes[(size_t)l.tmp];
                    if (ag) {
                        CHECK(l.out == l.read, "same-thread mapping broken");
                        if (l.out >= 0 && l.out < P)
                            ++out_writes[(size_t)l.out];
                    }
                } else {
                    CHECK(ag && !(rs && b < g.rs_blocks) && c < cpl,
                          "copy lane outside the copy blocks");
                    CHECK(l.shard >= 0 && l.shard < W, "shard %d", l.shard);
                    CHECK(!(rs && l.shard == rank), "own shard copied after the reduce");
                    const long long size = g.part + (l.shard == W - 1 ? g.rem : 0);
                    CHECK(l.read >= 0 && l.read < size && size <= g.cap,
                          "staging pack %lld of shard %d (size %lld)", (long long)l.read, l.shard, size);
                    CHECK(l.out == (long long)l.shard * g.part + l.read, "copy destination");
                    CHECK(l.out >= 0 && l.out < P, "out pack %lld of %lld", (long long)l.out, P);
                    if (l.out >= 0 && l.out < P)
                        ++out_writes[(size_t)l.out];
                }
            }
        }
    }
    for (long long q = 0; q < P; ++q)
        CHECK(out_writes[(size_t)q] == (ag ? 1 : 0), "out pack %lld written %d times", q,
              (int)out_writes[(size_t)q]);
    for (long long q = 0; q < g.cap; ++q)
        CHECK(tmp_writes[(size_t)q] == ((rs && q < g.own) ? 1 : 0),
              "staging pack %lld written %d times", q, (int)tmp_writes[(size_t)q]);
}

int main(int argc, char **argv)
{
    // argv: threads, then any number of "W P" pairs; every rank, every stage
    // combination, 1 and 2 packs per reduce lane and 1, 2 and 4 packs per
    // copy lane are checked for each.
    if (argc < 4 || (argc - 2) % 2 != 0) {
        std::printf("usage: %s threads W P [W P ...]\n", argv[0]);
        return 2;
    }
    const int threads = std::atoi(argv[1]);
    long launches = 0;
    for (int a = 2; a + 1 < argc; a += 2) {
        const int W = std::atoi(argv[a]);
        const long long P = std::atoll(argv[a + 1]);
        for (int rank = 0; rank < W; ++rank)
            for (int mode = 0; mode < 3; ++mode)
                for (int rpl : {1, 2})
                    for (int cpl : {1, 2, 4}) {
                        const bool rs = mode != 1, ag = mode != 0;
                        check_launch(W, P, rank, rs, ag, threads, rpl, cpl);
                        ++launches;
                    }
    }
    std::printf("%ld launches checked, %ld failures\n", launches, g_failures);
    return g_failures == 0 ? 0 : 1;
}
