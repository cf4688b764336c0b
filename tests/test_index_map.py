"""CPU enumeration of the two-stage reduce's launches.

The kernel decides which packs a lane reads and writes with the constexpr
functions of ar_rmsnorm_amd/csrc/index_map.h.  tests/index_map_check.cpp
compiles those same functions with g++ and walks every (block, lane, pack)
of a launch: every input, staging and output access must fall inside the
buffer sizes the header requires, reduce lanes must gather the packs they
reduced, and every output and staging pack must be written exactly once.

Cases: the message size of the 8 MB cap (W = 8, 4,194,304 bf16 = 524,288
packs) for every rank as reduce-scatter alone, all-gather alone and both, with
1 and 2 packs per reduce lane and 1, 2 and 4 per copy lane, on 256- and
512-lane workgroups -- including the stage-only launches a bench
row ran back to back over 23 buffer sets (the sets differ only in their
addresses, not in any index) -- and every W from 2 to 8 with pack counts that
leave remainders, down to fewer packs than ranks.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def map_walk(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("imap") / "index_map_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-o", exe,
                    os.path.join(HERE, "index_map_check.cpp")], check=True)
    return exe


def run(exe, *args):
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


@pytest.mark.parametrize("threads", [256, 512])
def test_cap_message_every_rank_and_stage(map_walk, threads):
    out = run(map_walk, threads, 8, 524_288)
    assert "144 launches checked, 0 failures" in out     # 8 ranks x 3 stages x 6 widths


@pytest.mark.parametrize("W", range(2, 9))
def test_ragged_sizes_every_world_size(map_walk, W):
    sizes = [0, 1, W - 1, W, W + 1, 255 * W + W - 1, 256 * W, 257 * W + 1, 1024 * W + 3,
             8 * (8 * 300 + 5), 65_536 * W + W - 1]
    args = []
    for P in sizes:
        args += [W, P]
    out = run(map_walk, 256, *args)
    assert f"{len(sizes) * W * 18} launches checked, 0 failures" in out


def test_the_map_walk_catches_a_planted_out_of_range_map(map_walk, tmp_path):
    """Plant an off-by-one in a copy of the map (the last shard's remainder
    given to every shard) and make sure the enumeration reports it."""
    src = open(os.path.join(HERE, "..", "ar_rmsnorm_amd", "csrc", "index_map.h")).read()
    old = "const int64_t size = g.part + (s == W - 1 ? g.rem : 0);"
    assert src.count(old) == 1
    bad_dir = tmp_path / "ar_rmsnorm_amd" / "csrc"
    bad_dir.mkdir(parents=True)
    (bad_dir / "index_map.h").write_text(src.replace(old, "const int64_t size = g.part + g.rem;"))
    tests_dir = tmp_path / "tests"
    tests_dir.mkdir()
    shutil.copy(os.path.join(HERE, "index_map_check.cpp"), tests_dir)
    exe = str(tmp_path / "bad_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-o", exe,
                    str(tests_dir / "index_map_check.cpp")], check=True)
    r = subprocess.run([exe, "256", "8", str(8 * 100 + 5)], capture_output=True, text=True)
    assert r.returncode == 1 and "FAIL" in r.stdout


def test_streaming_slices_cover_every_step(tmp_path):
    """tests/fifo_slice_check.cpp compiles the slice functions the streaming
    kernel and the host's pair choice use, and checks that the pairs of a
    channel cut every step (full, or a shorter last step) into disjoint,
    aligned pieces that cover it, each pair staying in its region of the
    ring slot, and that the chosen pair count fits the device; and that the
    launch plan gives the shapes the measurements and GPU tests use on one
    MI355X and, over a grid of calls, fits and leaves every pair a slice."""
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "fifo_slice_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-o", exe,
                    os.path.join(HERE, "fifo_slice_check.cpp")], check=True)
    out = run(exe)
    assert out.endswith("0 failures\n"), out


@pytest.mark.parametrize("header,old,new", [
    # a batch of whole steps one step too long for the ring window
    ("index_map.h", "return s < 2 ? 1 : s > max_steps ? max_steps : (int)s;",
     "return s < 2 ? 1 : s > max_steps ? max_steps + 1 : (int)s + 1;"),
    # the step of a lane slot changing one slot early
    ("index_map.h", "*step = (int)(v / len);", "*step = (int)((v + 1) / len);"),
    # LL's 512-lane form from one step more per channel than the rule says
    ("stream_plan.h", "steps_per_channel >= kFifoNarrowSteps)",
     "steps_per_channel > kFifoNarrowSteps)"),
    # a pair per 2,048 payload bytes instead of 2,048 items
    ("stream_plan.h", "int64_t by_work = bytes / per_item / kFifoItemsPerPair;",
     "int64_t by_work = bytes / kFifoItemsPerPair;"),
    # whole-step batches on channels that carry a single step
    ("stream_plan.h", "if (fifo_steps_per_channel(n, step_bytes, channels) < 2 ||",
     "if (fifo_steps_per_channel(n, step_bytes, channels) < 1 ||"),
])
def test_the_slice_check_catches_planted_batch_and_plan_mistakes(tmp_path, header, old, new):
    """Plant a mistake in a copy of the batch-of-steps functions or of the
    launch plan and make sure tests/fifo_slice_check.cpp reports it."""
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    csrc = os.path.join(HERE, "..", "ar_rmsnorm_amd", "csrc")
    bad_dir = tmp_path / "ar_rmsnorm_amd" / "csrc"
    bad_dir.mkdir(parents=True)
    for name in ("index_map.h", "stream_plan.h"):
        src = open(os.path.join(csrc, name)).read()
        if name == header:
            assert src.count(old) == 1
            src = src.replace(old, new)
        (bad_dir / name).write_text(src)
    tests_dir = tmp_path / "tests"
    tests_dir.mkdir()
    shutil.copy(os.path.join(HERE, "fifo_slice_check.cpp"), tests_dir)
    exe = str(tmp_path / "bad_slice_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-o", exe,
                    str(tests_dir / "fifo_slice_check.cpp")], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 1 and "FAIL" in r.stdout
