"""GPU parity of the two-shot fused all-reduce + residual + RMSNorm against
the oracle: every rank's reduce-scatter of its row shard, then each rank's
gather; residual_out and the staged shards bit-exact, norm_out within the
fused tolerance."""
import numpy as np
import pytest
import torch

import oracle as orc
from ar_rmsnorm_amd import libar as ar
from ar_rmsnorm_amd import synth
from tests.util import dev_u16, host_u16, norm_within_tolerance

pytestmark = pytest.mark.gpu


def sync():
    torch.cuda.synchronize()


def run_all_ranks(xs, res, w, eps, device, extra=0, in_place=False):
    W = len(xs)
    M, N = res.shape
    cap = M // W + M % W
    d = [dev_u16(x, device) for x in xs]
    dr, dw = dev_u16(res, device), dev_u16(w, device)
    tmps = [torch.full((2 * cap * N + 64,), 0x3C3C, dtype=torch.int16, device=device)
            for _ in range(W)]
    for r in range(1, W):
        ar.ar_fused_residual_rmsnorm_2stage(d, tmps, r, dr, dw, None, None, eps,
                                            flags=ar.AR_STAGE_RS | extra)
    outs = []
    for r in range(W):
        ro = dev_u16(res, device) if in_place else torch.full((M, N), 0x1111, dtype=torch.int16,
                                                               device=device)
        no = torch.full((M * N + 64,), 0x5A5A, dtype=torch.int16, device=device)
        flags = extra if r == 0 else ar.AR_STAGE_AG | extra
        # in place: this rank's residual is its residual_out buffer
        ar.ar_fused_residual_rmsnorm_2stage(d, tmps, r, ro if in_place else dr, dw, ro, no, eps,
                                            flags=flags, M=M, N=N)
        outs.append((ro, no))
    sync()
    res_out = []
    for ro, no in outs:
        hn = host_u16(no)
        assert np.all(hn[M * N:] == 0x5A5A), "norm_out written past M*N"
        res_out.append((host_u16(ro).reshape(M, N), hn[:M * N].reshape(M, N)))
    ht = [host_u16(t) for t in tmps]
    for s in range(W):
        assert np.all(ht[s][2 * cap * N:] == 0x3C3C), "tmp written past its capacity"
    return res_out, ht


def check(xs, res, w, eps, device, rank_order=False, in_place=False):
    W = len(xs)
    M, N = res.shape
    cap = M // W + M % W
    outs, ht = run_all_ranks(xs, res, w, eps, device,
                             ar.AR_ORDER_RANK if rank_order else 0, in_place)
    wro, wno, exact = orc.fused_2stage(xs, res, w, eps, rank_order)
    for r, (ro, no) in enumerate(outs):
        assert np.array_equal(ro, wro), f"residual_out rank {r}"
        ok, _ = norm_within_tolerance(no, exact)
        assert ok.all(), f"norm_out rank {r}"
    for s in range(W):
        m0, m1 = orc.row_shard_range(M, W, s)
        sro, sno, sne = orc.fused_2stage_scatter(xs, s, res, w, eps, rank_order)
        rows = m1 - m0
        assert np.array_equal(ht[s][:rows * N].reshape(rows, N), sro), f"staged res {s}"
        got = ht[s][cap * N:(cap + rows) * N].reshape(rows, N)
        ok, _ = norm_within_tolerance(got, sne)
        assert ok.all(), f"staged norm {s}"
    return outs


@pytest.mark.parametrize("M", [1, 16, 128])
def test_fused_2stage_workloads(gpu, M):
    xs, res, w = synth.fused(M)
    check(xs, res, w, synth.FUSED["eps"], gpu)


@pytest.mark.parametrize("W,M,N", [(2, 7, 8), (3, 3 * 5 + 2, 512), (8, 8 * 3 + 7, 1000),
                                   (4, 4 * 4 + 3, 4096), (8, 11, 16384), (5, 3, 2056)])
def test_fused_2stage_shapes(gpu, W, M, N):
    xs, res, w = synth.fused_inputs(W, M, N, [99, W, M, N])
    check(xs, res, w, 1e-6, gpu)


@pytest.mark.parametrize("case", range(8))
def test_fused_2stage_seeded_random_shapes(gpu, case):
    """Seeded random W (2..8), M (1..60, so M < W and remainders occur) and
    N (any multiple of 8 up to 16,384)."""
    rng = np.random.default_rng([87, case])
    W, M, N = int(rng.integers(2, 9)), int(rng.integers(1, 61)), 8 * int(rng.integers(1, 2049))
    xs, res, w = synth.fused_inputs(W, M, N, [88, case])
    check(xs, res, w, 1e-6, gpu)


def test_fused_2stage_rank_order_matches_one_shot_kernel(gpu):
    """In rank order the two-shot rows come from the same arithmetic as the
    one-shot kernel: both outputs are bit-identical to it."""
    W, M, N = 4, 4 * 8 + 3, 2048
    xs, res, w = synth.fused_inputs(W, M, N, [100])
    outs = check(xs, res, w, 1e-6, gpu, rank_order=True)
    d = [dev_u16(x, gpu) for x in xs]
    dr, dw = dev_u16(res, gpu), dev_u16(w, gpu)
    ro, no = torch.empty_like(dr), torch.empty_like(dr)
    ar.ar_fused_residual_rmsnorm(d, dr, dw, ro, no, 1e-6)
    sync()
    for r_ro, r_no in outs:
        assert np.array_equal(r_ro, host_u16(ro)) and np.array_equal(r_no, host_u16(no))


def test_fused_2stage_in_place(gpu):
    xs, res, w = synth.fused_inputs(4, 4 * 6 + 1, 1024, [101])
    check(xs, res, w, 1e-6, gpu, in_place=True)


def test_fused_2stage_rotation_hand_case(gpu):
    M, N = 4, 64
    xs = [np.full((M, N), v, np.uint16) for v in (0x3F80, 0x4B80, 0x3F80, 0xCB80)]
    res = np.zeros((M, N), np.uint16)
    w = np.full(N, 0x3F80, np.uint16)
    outs = check(xs, res, w, 1e-6, gpu)
    ro, no = outs[1]
    assert list(orc.bf16_to_f32(ro[:, 0])) == [0.0, 1.0, 2.0, 2.0]
    assert list(orc.bf16_to_f32(no[:, 0])) == [0.0, 1.0, 1.0, 1.0]


def test_fused_large_m_row_configuration(gpu):
    """The large-M shape the bench times (W=4, M=2048, N=8192): the two-shot
    form for every rank, and the one-shot form, against the oracle."""
    W, M, N = synth.FUSED["W"], 2048, 8192
    xs, res, w = synth.fused_inputs(W, M, N, [1000 + synth.FUSED["id"], M, N])
    eps = synth.FUSED["eps"]
    check(xs, res, w, eps, gpu)
    d = [dev_u16(x, gpu) for x in xs]
    dr, dw = dev_u16(res, gpu), dev_u16(w, gpu)
    ro, no = torch.empty_like(dr), torch.empty_like(dr)
    ar.ar_fused_residual_rmsnorm(d, dr, dw, ro, no, eps)
    sync()
    wro, _, exact = orc.fused_residual_rmsnorm(xs, res, w, eps)
    assert np.array_equal(host_u16(ro), wro)
    ok, _ = norm_within_tolerance(host_u16(no), exact)
    assert ok.all()
