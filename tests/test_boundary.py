"""The C-ABI library loads, exports every symbol include/libar.h declares, and
its host-side logic (geometry helpers, argument checks) behaves as the header
says.  No test here launches a kernel.

The argument-error cases pass fake device addresses and rely on each check
returning before anything is enqueued; to make sure no stray launch can ever
reach a GPU with such addresses, this module only runs where no GPU is
visible.  The same rejections with real device buffers are in the GPU tests.
"""
import os
import re

import pytest
import torch

from ar_rmsnorm_amd import libar as ar

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "libar.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\([^;{]*\)\s*;", text)))


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(ar.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ar.raw()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_geometry_helpers_match_printed_buffer_table():
    # LL: 524288-byte default buffer / 8 steps / 16 B lines = 4096 lines, 32768
    # payload bytes per step; LL128: 4915200 / 8 / 128 = 4800 lines, 576000 B.
    assert ar.ll_default_step_lines() == 4096
    assert ar.ll128_default_step_lines() == 4800
    assert ar.ll_fifo_bytes(4096) == 524288
    assert ar.ll128_fifo_bytes(4800) == 4915200
    assert ar.ll_lines(32768 // 4) == 4096
    assert ar.ll128_lines(576000 // 4) == 4800
    assert ar.ll_lines(16_777_216) == 8_388_608
    assert ar.ll_lines(16_777_229) == 8_388_615
    assert ar.ll128_lines(16_777_216) == 559_241
    assert ar.ll128_fifo_bytes(69_906) // 8 * 8 == 71_583_744
    assert ar.ll128_lines(16_777_216) * 128 == 71_582_848
    assert (ar.ll_lines(0), ar.ll_lines(-3), ar.ll_fifo_bytes(0)) == (0, 0, 0)


def test_status_strings():
    for s in range(7):
        assert ar.status_str(s)
    assert ar.status_str(0) == "ok"
    assert ar.status_str(99) == "unknown status"


# --------------------------------------------------------------------------
# argument errors with fake addresses (never dereferenced)
# --------------------------------------------------------------------------
gpu_visible = torch.cuda.is_available()
cpu_only = pytest.mark.skipif(gpu_visible, reason="fake-address error paths run only "
                              "where no GPU can receive a launch")

A = 0x7F0000000000          # 16-byte (and 128-byte) aligned fake addresses
B = A + (1 << 30)
C = A + (2 << 30)
D = A + (3 << 30)
E = A + (4 << 30)
F = A + (5 << 30)


def st(fn, *args):
    """Status of a call with fake addresses: the binding's own buffer checks
    are off, so the C ABI's validation is what answers."""
    try:
        with ar.checks_disabled():
            fn(*args)
    except ar.ArError as e:
        return e.status
    return ar.AR_OK


@cpu_only
def test_reduce_1stage_argument_errors():
    f = ar.ar_reduce_1stage
    assert st(f, [A], B, 8, 0) == ar.AR_ERR_WORLD
    assert st(f, [A] * 9, B, 8, 0) == ar.AR_ERR_WORLD
    assert st(f, [A, None], B, 8, 0) == ar.AR_ERR_NULL
    assert st(f, [A, B], None, 8, 0) == ar.AR_ERR_NULL
    assert st(f, [A, B], C, 12, 0) == ar.AR_ERR_ARG
    assert st(f, [A, B], C, -8, 0) == ar.AR_ERR_ARG
    assert st(f, [A, B + 8], C, 8, 0) == ar.AR_ERR_ALIGN
    assert st(f, [A, B], C + 4, 8, 0) == ar.AR_ERR_ALIGN
    assert st(f, [A, B], A + 16, 64, 0) == ar.AR_ERR_ARG      # partial overlap
    assert st(f, [A, B], C, 0, 0) == ar.AR_OK                 # empty: no launch


@cpu_only
def test_reduce_2stage_argument_errors():
    f = ar.ar_reduce_2stage
    ins, tms = [A, B], [C, D]
    assert st(f, [A], [C], 0, E, 0, 8, 0) == ar.AR_ERR_WORLD
    assert st(f, ins, tms, 2, E, 0, 8, 0) == ar.AR_ERR_ARG     # rank out of range
    assert st(f, ins, tms, -1, E, 0, 8, 0) == ar.AR_ERR_ARG
    assert st(f, ins, tms, 0, E, 8, 8, 0) == ar.AR_ERR_ARG     # unknown flag bit
    assert st(f, ins, tms, 0, None, 0, 8, 0) == ar.AR_ERR_NULL  # AG needs out
    assert st(f, ins, [C, None], 0, E, 0, 8, 0) == ar.AR_ERR_NULL
    assert st(f, ins, tms, 0, E, 0, 9, 0) == ar.AR_ERR_ARG
    assert st(f, ins, [C, D + 4], 0, E, 0, 8, 0) == ar.AR_ERR_ALIGN
    assert st(f, ins, tms, 0, A, 0, 64, 0) == ar.AR_ERR_ARG    # out aliases input
    assert st(f, ins, tms, 0, D, 0, 64, 0) == ar.AR_ERR_ARG    # out aliases tmp
    assert st(f, ins, [A, D], 0, E, ar.AR_STAGE_RS, 64, 0) == ar.AR_ERR_ARG
    assert st(f, ins, [C, C], 0, E, 0, 64, 0) == ar.AR_ERR_ARG  # own tmp = peer tmp
    assert st(f, ins, tms, 0, E, 0, 0, 0) == ar.AR_OK


@cpu_only
def test_fused_argument_errors():
    f = ar.ar_fused_residual_rmsnorm
    ins = [A, B]
    assert st(f, [A], C, D, E, F, 1e-6, 1, 2048, 0) == ar.AR_ERR_WORLD
    assert st(f, ins, None, D, E, F, 1e-6, 1, 2048, 0) == ar.AR_ERR_NULL
    assert st(f, ins, C, D, E, F, 1e-6, 1, 2044, 0) == ar.AR_ERR_ARG
    assert st(f, ins, C, D, E, F, 1e-6, 1, 16392, 0) == ar.AR_ERR_ARG
    assert st(f, ins, C, D, E, F, 1e-6, -1, 2048, 0) == ar.AR_ERR_ARG
    assert st(f, ins, C, D, E, F, float("nan"), 1, 2048, 0) == ar.AR_ERR_ARG
    assert st(f, ins, C, D, E, F, -1.0, 1, 2048, 0) == ar.AR_ERR_ARG
    assert st(f, ins, C, D + 2, E, F, 1e-6, 1, 2048, 0) == ar.AR_ERR_ALIGN
    assert st(f, ins, C, D, E, A, 1e-6, 1, 2048, 0) == ar.AR_ERR_ARG   # norm_out = input
    assert st(f, ins, C, D, E, E, 1e-6, 1, 2048, 0) == ar.AR_ERR_ARG   # norm = res_out
    assert st(f, ins, C, D, C + 16, F, 1e-6, 1, 2048, 0) == ar.AR_ERR_ARG
    assert st(f, ins, C, D, C, F, 1e-6, 0, 2048, 0) == ar.AR_OK        # in place, M=0


@cpu_only
def test_wire_argument_errors():
    assert st(ar.ll_pack, A, B, 0, 0, 9, 0) == ar.AR_ERR_ARG            # step_lines 0
    assert st(ar.ll_pack, A, B, 1, 0, 17, 0) == ar.AR_ERR_CAPACITY      # 9 lines > 8
    assert st(ar.ll_pack, A + 2, B, 1, 0, 8, 0) == ar.AR_ERR_ALIGN
    assert st(ar.ll_pack, B + 4, B, 1, 0, 8, 0) == ar.AR_ERR_ARG        # src in fifo
    assert st(ar.ll_pack, A + 4, B + 8, 1, 0, 8, 0) == ar.AR_ERR_ALIGN
    assert st(ar.ll128_pack, A, B + 64, 1, 0, 8, 0) == ar.AR_ERR_ALIGN  # 128 B lines
    assert st(ar.ll128_pack, A, B, 1, 0, 241, 0) == ar.AR_ERR_CAPACITY
    assert st(ar.ll_pack, None, B, 1, 0, 8, 0) == ar.AR_ERR_NULL
    assert st(ar.ll_pack, A, B, 1, 0, 0, 0) == ar.AR_OK
    u = ar.ll_unpack_reduce
    assert st(u, [], C, 1, 0, 0, None, 8, 0) == ar.AR_ERR_WORLD
    assert st(u, [A] * 9, C, 1, 0, 0, None, 8, 0) == ar.AR_ERR_WORLD
    assert st(u, [A, None], C, 1, 0, 0, None, 8, 0) == ar.AR_ERR_NULL
    assert st(u, [A], C, 1, 0, ar.AR_MAX_SPINS + 1, None, 8, 0) == ar.AR_ERR_ARG
    assert st(u, [A], C, 1, 0, 0, None, 17, 0) == ar.AR_ERR_CAPACITY
    assert st(u, [A], C + 2, 1, 0, 0, None, 8, 0) == ar.AR_ERR_ALIGN
    assert st(u, [A], C, 1, 0, 0, D + 2, 8, 0) == ar.AR_ERR_ALIGN
    assert st(u, [A], A + 16, 1, 0, 0, None, 8, 0) == ar.AR_ERR_ARG     # out in fifo
    assert st(u, [A], C, 1, 0, 0, C + 4, 8, 0) == ar.AR_ERR_ARG         # counter in out
    assert st(ar.ll128_unpack_reduce, [A + 16], C, 1, 0, 0, None, 8, 0) == ar.AR_ERR_ALIGN
    assert st(u, [A], C, 1, 0, 0, None, 0, 0) == ar.AR_OK


def test_stream_geometry_helpers():
    # NCCL's default steps: LL 32768 payload bytes in 4096 16-byte lines, LL128
    # 576000 in 4800 128-byte lines, Simple 524288 raw
    assert ar.ar_fifo_step_wire_bytes(ar.AR_PROTO_LL, 32768) == 65536
    assert ar.ar_fifo_step_wire_bytes(ar.AR_PROTO_LL128, 576000) == 4800 * 128
    assert ar.ar_fifo_step_wire_bytes(ar.AR_PROTO_SIMPLE, 524288) == 524288
    for proto, bad in ((ar.AR_PROTO_LL, 12), (ar.AR_PROTO_LL128, 1000),
                       (ar.AR_PROTO_SIMPLE, 24), (3, 1024), (ar.AR_PROTO_LL, 0),
                       (ar.AR_PROTO_LL, (1 << 30) + 8)):
        assert ar.ar_fifo_step_wire_bytes(proto, bad) == 0
    # 16 Mi fp32 at 32 KiB steps: 2048 steps; 13 more values need one more
    assert ar.ar_fifo_steps_per_channel(16_777_216, 32768, 32) == 64
    assert ar.ar_fifo_steps_per_channel(16_777_229, 32768, 32) == 65
    assert ar.ar_fifo_steps_per_channel(2048, 32768, 32) == 1
    assert ar.ar_fifo_steps_per_channel(0, 32768, 4) == 0
    # a head and a tail per pair (up to 8 pairs per channel), then two state words
    assert [ar.ar_fifo_counter_words(c) for c in (0, 1, 256, 257)] == [0, 18, 4098, 0]
    assert ar.AR_FIFO_CONTINUE == (1 << 64) - 1


@cpu_only
def test_stream_argument_errors():
    f = ar.ar_fifo_stream
    LL, LL128 = ar.AR_PROTO_LL, ar.AR_PROTO_LL128
    assert st(f, LL, None, B, C, D, 2, 1024, 0, 8, E, None, 8, 0) == ar.AR_ERR_NULL
    assert st(f, LL, A, B, C, D, 2, 1024, 0, 8, None, None, 8, 0) == ar.AR_ERR_NULL
    assert st(f, LL, A, B, C, D, 0, 1024, 0, 8, E, None, 8, 0) == ar.AR_ERR_ARG
    assert st(f, LL, A, B, C, D, 257, 1024, 0, 8, E, None, 8, 0) == ar.AR_ERR_ARG
    assert st(f, LL, A, B, C, D, 2, 1020, 0, 8, E, None, 8, 0) == ar.AR_ERR_ARG
    assert st(f, LL, A, B, C, D, 2, 1024, 0, ar.AR_MAX_SPINS + 1, E, None, 8, 0) == ar.AR_ERR_ARG
    assert st(f, LL, A + 2, B, C, D, 2, 1024, 0, 8, E, None, 8, 0) == ar.AR_ERR_ALIGN
    assert st(f, LL128, A, B, C + 64, D, 2, 1200, 0, 8, E, None, 8, 0) == ar.AR_ERR_ALIGN
    assert st(f, LL, A, B, C, D + 4, 2, 1024, 0, 8, E, None, 8, 0) == ar.AR_ERR_ALIGN
    assert st(f, LL, A, A + 16, C, D, 2, 1024, 0, 8, E, None, 8, 0) == ar.AR_ERR_ARG
    assert st(f, LL, A, B, C, D, 2, 1024, 0, 8, E, B + 4, 8, 0) == ar.AR_ERR_ARG   # local partial
    assert st(f, LL, A, B, C, C + 64, 2, 1024, 0, 8, E, None, 8, 0) == ar.AR_ERR_ARG  # counters
    # the two state words follow the 2 * channels * 8 heads and tails
    words = 2 * 2 * ar.AR_FIFO_MAX_PAIRS + 2
    assert st(f, LL, A, B, C, D, 2, 1024, 0, 8, D + 8 * words - 8, None, 8, 0) == ar.AR_ERR_ARG
    assert st(f, LL, A, B, C, D, 2, 1024, 0, 8, D + 8 * words, None, 0, 0) == ar.AR_OK
    assert st(f, LL, A, B, C, D, 2, 1024, 0, 8, E, None, 0, 0) == ar.AR_OK       # n = 0


@cpu_only
def test_stream_plan_argument_errors():
    """ar_fifo_plan refuses what ar_fifo_stream refuses before asking the
    device anything, and plans nothing for an empty call."""
    f = ar.ar_fifo_plan
    LL = ar.AR_PROTO_LL
    for args in ((3, 1024, 2, 1024), (LL, 1024, 0, 1024), (LL, 1024, 257, 1024),
                 (LL, 1024, 2, 1020), (LL, -1, 2, 1024), (ar.AR_PROTO_LL128, 1024, 2, 1000)):
        assert st(f, *args) == ar.AR_ERR_ARG, args
    assert f(LL, 0, 2, 1024) == (0, 0, 0)
    # the outputs are optional
    assert ar._lib.ar_fifo_plan(LL, 0, 2, 1024, 0, None, None, None) == ar.AR_OK


def test_size_limits_of_the_wire_helpers():
    big = (1 << 62) + 3                     # 4n would not fit in 64 bits
    assert ar.ll_lines(1 << 40) == (1 << 39) and ar.ll_lines((1 << 40) + 1) == 0
    assert ar.ll_lines(big) == 0 and ar.ll128_lines(big) == 0
    assert ar.ll_fifo_bytes(1 << 28) == (1 << 35) and ar.ll_fifo_bytes((1 << 28) + 1) == 0
    assert ar.ll128_fifo_bytes(1 << 62) == 0
    assert ar.ar_fifo_steps_per_channel(big, 32768, 4) == 0


@cpu_only
def test_wire_calls_reject_sizes_past_the_limit():
    big = (1 << 62) + 3
    assert st(ar.ll_pack, A, B, 1, 0, big, 0) == ar.AR_ERR_ARG
    assert st(ar.ll128_pack, A, B, 1, 0, (1 << 40) + 30, 0) == ar.AR_ERR_ARG
    assert st(ar.ll_unpack_reduce, [A], C, 1, 0, 0, None, big, 0) == ar.AR_ERR_ARG
    assert st(ar.ll128_unpack_reduce, [A], C, 1, 0, 0, None, big, 0) == ar.AR_ERR_ARG
    assert st(ar.ll_pack, A, B, (1 << 28) + 1, 0, 8, 0) == ar.AR_ERR_ARG


def test_lamport_shape_limits():
    assert ar.ar_lamport_comm_bytes(4, 1 << 26, 16384) == 3 * 4 * (1 << 40) * 2
    assert ar.ar_lamport_comm_bytes(4, (1 << 26) + 1, 16384) == 0     # M * N > 2^40
    assert ar.ar_lamport_comm_bytes(4, 1 << 31, 8) == 0               # M >= 2^31


# --------------------------------------------------------------------------
# the binding's own checks, the Lamport flag period, the copy reference and
# the one-GPU fused-form choice
# --------------------------------------------------------------------------
def test_binding_refuses_host_tensors_and_integer_addresses():
    """With its checks on (the default) the binding passes only contiguous
    GPU tensors: a host tensor or a bare integer address is refused with
    AR_ERR_ARG before the C ABI is called."""
    host = torch.zeros(64, dtype=torch.int16)
    with pytest.raises(ar.ArError) as e:
        ar.ar_reduce_1stage([host, host], host, stream=0)
    assert e.value.status == ar.AR_ERR_ARG and "not on a GPU" in str(e.value)
    with pytest.raises(ar.ArError) as e:
        ar.ar_reduce_1stage([A, B], C, 8, 0)
    assert e.value.status == ar.AR_ERR_ARG and "torch tensor" in str(e.value)
    with pytest.raises(ar.ArError) as e:
        ar.ll_pack(torch.zeros(8), A, 1, stream=0)
    assert e.value.status == ar.AR_ERR_ARG


def test_lamport_next_flag_wraps_at_a_multiple_of_three():
    P = ar.AR_LAMPORT_FLAG_PERIOD
    assert P == 3 << 30
    assert ar.ar_lamport_next_flag(0) == 1
    assert ar.ar_lamport_next_flag(P - 2) == P - 1
    assert ar.ar_lamport_next_flag(P - 1) == 0
    assert ar.ar_lamport_next_flag(0xFFFFFFFF) == 0
    f, regions = P - 3, []
    for _ in range(6):
        regions.append(f % 3)
        f = ar.ar_lamport_next_flag(f)
    assert regions == [0, 1, 2, 0, 1, 2]
    with pytest.raises(ar.ArError):
        ar.ar_lamport_next_flag(1 << 32)


@cpu_only
def test_lamport_flags_at_or_past_the_period_are_rejected():
    P = ar.AR_LAMPORT_FLAG_PERIOD
    W, M, N = 2, 1, 8
    for flag in (P, P + 1, 0xFFFFFFFF):
        assert st(ar.ar_lamport_push, A, 0, [B, C], flag, M, N, 0) == ar.AR_ERR_ARG
        assert st(ar.ar_lamport_fused_residual_rmsnorm, B, W, D, E, F, F + 4096, 1e-6, flag,
                  0, None, M, N, 0) == ar.AR_ERR_ARG
        assert st(ar.ar_lamport_oneshot_residual_rmsnorm, A, 0, [B, C], D, E, F, F + 4096,
                  1e-6, flag, 0, None, M, N, 0) == ar.AR_ERR_ARG
    # the last valid flag reaches the launch (rejected by the runtime here)
    assert st(ar.ar_lamport_push, A, 0, [B, C], P - 1, M, N, 0) == ar.AR_ERR_HIP


@cpu_only
def test_copy_argument_errors():
    f = ar.ar_copy
    assert st(f, None, B, 16, 0) == ar.AR_ERR_NULL
    assert st(f, A, None, 16, 0) == ar.AR_ERR_NULL
    assert st(f, A, B, 8, 0) == ar.AR_ERR_ARG                 # not whole 16-byte packs
    assert st(f, A, B, -16, 0) == ar.AR_ERR_ARG
    assert st(f, A, B, (1 << 44) + 16, 0) == ar.AR_ERR_ARG
    assert st(f, A + 4, B, 16, 0) == ar.AR_ERR_ALIGN
    assert st(f, A, B + 8, 16, 0) == ar.AR_ERR_ALIGN
    assert st(f, A, A + 16, 32, 0) == ar.AR_ERR_ARG           # overlapping ranges
    assert st(f, A, B, 0, 0) == ar.AR_OK                      # nothing to launch
    assert st(f, A, B, 16, 0) == ar.AR_ERR_HIP                # reaches the launch


def test_fused_form_choice():
    f = ar.ar_fused_prefers_two_shot
    assert f(1, 16, 2048) == -1 and f(9, 16, 2048) == -1
    assert f(4, -1, 2048) == -1 and f(4, 16, 2049) == -1 and f(4, 16, 16392) == -1
    # W = 2: the two-shot form moves more bytes than the one-shot form
    assert all(f(2, M, N) == 0 for M in (1, 16, 1024, 8192) for N in (2048, 8192))
    # fewer rows than ranks: one owner would take every row
    assert f(8, 7, 2048) == 0 and f(4, 3, 8192) == 0
    for W in (3, 4, 8):
        assert f(W, 1, 2048) == 0
        assert all(f(W, M, N) == 1 for M in (W, 16, 128, 2048, 8192) for N in (2048, 8192))


@cpu_only
def test_reduce_2stage_noalloc_argument_errors():
    f = ar.ar_reduce_2stage_noalloc
    W = 8
    ins = [A + i * (1 << 26) for i in range(W)]
    assert st(f, ins[:1], 0, B, 0, 8, 0) == ar.AR_ERR_WORLD
    assert st(f, ins[:-1] + [None], 0, B, 0, 8, 0) == ar.AR_ERR_NULL
    assert st(f, ins, 0, None, 0, 8, 0) == ar.AR_ERR_NULL            # gather needs out
    assert st(f, ins, 8, B, 0, 8, 0) == ar.AR_ERR_ARG                # rank out of range
    assert st(f, ins, 0, B, 8, 8, 0) == ar.AR_ERR_ARG                # unknown flag bit
    assert st(f, ins, 0, B, 0, 12, 0) == ar.AR_ERR_ARG               # not whole packs
    assert st(f, ins[:-1] + [A + 8], 0, B, 0, 8, 0) == ar.AR_ERR_ALIGN
    assert st(f, ins, 0, A, 0, 8, 0) == ar.AR_ERR_ARG                # out overlaps an input
    # the 8 MiB cap message fits the staging array for every W; one more pack
    # per shard than the array holds does not
    assert st(f, ins, 0, B, 0, 4_194_304, 0) == ar.AR_ERR_HIP        # reaches the launch
    for w in range(2, 9):
        assert st(f, ins[:w], 0, B, 0, 4_194_304 + 8 * (w - 1), 0) == ar.AR_ERR_HIP
    big = 8 * ((ar.AR_SCRATCH_BYTES // 16 // W + 1) * W)
    assert st(f, ins, 0, B, 0, big, 0) == ar.AR_ERR_CAPACITY
    assert st(f, ins, 0, None, ar.AR_STAGE_RS, 0, 0) == ar.AR_OK     # nothing to launch


@cpu_only
def test_lamport_all_ranks_argument_errors():
    f = ar.ar_lamport_all_ranks_residual_rmsnorm
    W, M, N = 4, 2, 64
    mat = 2 * M * N
    G = 1 << 24                                   # spacing of the fake buffers
    xs = [A + i * G for i in range(W)]
    comms = [B + i * G for i in range(W)]
    ros = [C + i * G for i in range(W)]
    nos = [D + i * G for i in range(W)]
    res, wt = E, F

    def call(xs=xs, comms=comms, ros=ros, nos=nos, res=res, wt=wt, flag=0, spins=0, M=M, N=N,
             eps=1e-6):
        return st(f, xs, comms, res, wt, ros, nos, eps, flag, spins, None, M, N, 0)

    assert call() == ar.AR_ERR_HIP                       # valid: reaches the device
    assert call(M=0) == ar.AR_OK
    assert call(xs=xs[:1], comms=comms[:1], ros=ros[:1], nos=nos[:1]) == ar.AR_ERR_WORLD
    assert call(xs=xs[:-1] + [None]) == ar.AR_ERR_NULL
    assert call(nos=nos[:-1] + [None]) == ar.AR_ERR_NULL
    assert call(flag=ar.AR_LAMPORT_FLAG_PERIOD) == ar.AR_ERR_ARG
    assert call(spins=ar.AR_MAX_SPINS + 1) == ar.AR_ERR_ARG
    assert call(N=12) == ar.AR_ERR_ARG
    assert call(eps=-1.0) == ar.AR_ERR_ARG
    assert call(ros=ros[:-1] + [C + 3 * G + 8]) == ar.AR_ERR_ALIGN
    assert call(ros=ros[:-1] + [res]) == ar.AR_ERR_ARG            # output on the residual
    assert call(nos=nos[:-1] + [ros[0]]) == ar.AR_ERR_ARG         # two outputs overlap
    assert call(ros=ros[:-1] + [xs[1] + mat // 2]) == ar.AR_ERR_ARG  # output inside an input
    assert call(comms=comms[:-1] + [comms[0]]) == ar.AR_ERR_ARG   # shared comm buffer
    assert call(xs=xs[:-1] + [comms[2]]) == ar.AR_ERR_ARG         # input inside a comm buffer
