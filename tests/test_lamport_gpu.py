"""GPU parity of the Lamport data-as-flag fused one-shot against the oracle.

All ranks' comm buffers live on the one GPU: every rank pushes (separate
launches), then each rank runs the fused reader.  The pushed comm-buffer
bytes, residual_out and the reset of the previous region are bit-exact; the
norm is within the fused tolerance.  Flag waits are bounded (max_spins), so
a missing push ends in a counted, not a hung, wait.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from ar_rmsnorm_amd import libar as ar
from ar_rmsnorm_amd import synth
from tests.util import dev_u16, host_u16, norm_within_tolerance

pytestmark = pytest.mark.gpu

SENT = orc.LAMPORT_SENTINEL


def sync():
    torch.cuda.synchronize()


def comm_words(W, M, N):
    return ar.ar_lamport_comm_bytes(W, M, N) // 4


def new_comms(W, M, N, device):
    comms = [torch.empty(comm_words(W, M, N), dtype=torch.int32, device=device)
             for _ in range(W)]
    for c in comms:
        ar.ar_lamport_fill(c, W, M, N)
    return comms


def host_words(t):
    return t.cpu().numpy().view(np.uint32)


def run_call(xs, res, w, comms, hcomms, flag, device, eps=1e-6, max_spins=0,
             skip_rank=None):
    """One call: pushes of every rank (GPU and oracle), then every rank's
    reader; returns the per-rank GPU outputs and bad counts, checked."""
    W = len(xs)
    M, N = res.shape
    dx = [dev_u16(x, device) for x in xs]
    for r in range(W):
        if r == skip_rank:
            continue
        ar.ar_lamport_push(dx[r], r, comms, flag)
        orc.lamport_push(xs[r], r, hcomms, flag)
    sync()
    for p in range(W):
        assert np.array_equal(host_words(comms[p]), hcomms[p]), f"push bytes, rank {p}"
    dr, dw = dev_u16(res, device), dev_u16(w, device)
    results = []
    for p in range(W):
        ro = torch.empty_like(dr)
        no = torch.empty_like(dr)
        bad = torch.zeros(1, dtype=torch.int32, device=device)
        ar.ar_lamport_fused_residual_rmsnorm(comms[p], W, dr, dw, ro, no, eps, flag,
                                             max_spins, bad)
        sync()
        wro, wno, exact, wbad = orc.lamport_fused_residual_rmsnorm(hcomms[p], W, res, w, eps,
                                                                   flag)
        assert int(bad.item()) == wbad
        assert np.array_equal(host_words(comms[p]), hcomms[p]), f"reset region, rank {p}"
        if wbad == 0:
            assert np.array_equal(host_u16(ro), wro), "residual_out not bit-exact"
            ok, _ = norm_within_tolerance(host_u16(no), exact)
            assert ok.all(), "norm_out outside tolerance"
        results.append((host_u16(ro), host_u16(no), int(bad.item())))
    return results


@pytest.mark.parametrize("M", [1, 16, 128])
def test_lamport_workloads(gpu, M):
    xs, res, w = synth.fused(M)
    W, N = len(xs), res.shape[1]
    comms = new_comms(W, M, N, gpu)
    hcomms = [orc.lamport_comm(W, M, N) for _ in range(W)]
    sync()
    for c in comms:
        assert np.all(host_words(c) == SENT)
    out = run_call(xs, res, w, comms, hcomms, 0, gpu)
    # same numbers as the plain fused operator on these inputs (no -0.0)
    wro, wno, _ = orc.fused_residual_rmsnorm(xs, res, w, synth.FUSED["eps"])
    for ro, no, bad in out:
        assert bad == 0 and np.array_equal(ro, wro)


@pytest.mark.parametrize("W,M,N", [(2, 3, 8), (8, 2, 512), (3, 5, 1000), (5, 2, 4096),
                                   (8, 1, 16384), (6, 4, 2056)])
def test_lamport_shapes(gpu, W, M, N):
    xs, res, w = synth.fused_inputs(W, M, N, [93, W, M, N])
    comms = new_comms(W, M, N, gpu)
    hcomms = [orc.lamport_comm(W, M, N) for _ in range(W)]
    run_call(xs, res, w, comms, hcomms, 5, gpu)


def test_lamport_triple_buffer_over_calls(gpu):
    W, M, N = 4, 3, 256
    comms = new_comms(W, M, N, gpu)
    hcomms = [orc.lamport_comm(W, M, N) for _ in range(W)]
    words = M * N // 2
    for f in range(7):
        sync()
        for c in comms:
            reg = host_words(c).reshape(3, W * words)[f % 3]
            assert np.all(reg == SENT), f"region {f % 3} not clear before call {f}"
        xs, res, w = synth.fused_inputs(W, M, N, [94, f])
        run_call(xs, res, w, comms, hcomms, f, gpu)


def test_lamport_negative_zero_scrub(gpu):
    W, M, N = 4, 2, 64
    xs = [np.full((M, N), 0x8000, np.uint16) for _ in range(W)]
    res = np.full((M, N), 0x8000, np.uint16)
    w = np.full(N, 0x3F80, np.uint16)
    comms = new_comms(W, M, N, gpu)
    hcomms = [orc.lamport_comm(W, M, N) for _ in range(W)]
    out = run_call(xs, res, w, comms, hcomms, 1, gpu)
    for ro, _, bad in out:
        assert bad == 0 and np.all(ro == 0)


def test_lamport_missing_push_is_counted_not_hung(gpu):
    W, M, N = 3, 2, 512
    xs, res, w = synth.fused_inputs(W, M, N, [95])
    comms = new_comms(W, M, N, gpu)
    hcomms = [orc.lamport_comm(W, M, N) for _ in range(W)]
    out = run_call(xs, res, w, comms, hcomms, 2, gpu, max_spins=4, skip_rank=1)
    for _, _, bad in out:
        assert bad == M * N // 8


def test_lamport_argument_errors_with_device_buffers(gpu):
    W, M, N = 2, 1, 64
    comms = new_comms(W, M, N, gpu)
    x = torch.zeros((M, N), dtype=torch.int16, device=gpu)
    with pytest.raises(ar.ArError) as e:
        ar.ar_lamport_push(x, 2, comms, 0)
    assert e.value.status == ar.AR_ERR_ARG
    with pytest.raises(ar.ArError) as e:
        ar.ar_lamport_push(comms[0][:M * N // 2].view(torch.int16).view(M, N), 0, comms, 0)
    assert e.value.status == ar.AR_ERR_ARG
    r = torch.zeros((M, N), dtype=torch.int16, device=gpu)
    wt = torch.zeros(N, dtype=torch.int16, device=gpu)
    with pytest.raises(ar.ArError) as e:
        ar.ar_lamport_fused_residual_rmsnorm(comms[0], W, r, wt, r, comms[1][:M * N // 2]
                                             .view(torch.int16), 1e-6, 0, ar.AR_MAX_SPINS + 1)
    assert e.value.status == ar.AR_ERR_ARG
    with pytest.raises(ar.ArError) as e:
        ar.ar_lamport_fused_residual_rmsnorm(comms[0], W, r, wt, r, comms[0][:M * N // 2]
                                             .view(torch.int16), 1e-6, 0)
    assert e.value.status == ar.AR_ERR_ARG        # norm_out inside the comm buffer
    sync()


def _random_shapes(seed, count):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(2, 9)), int(rng.integers(1, 9)), 8 * int(rng.integers(1, 2049)))
            for _ in range(count)]


@pytest.mark.parametrize("W,M,N", [(4, 1, 2048), (4, 128, 2048), (2, 3, 8), (8, 2, 16384),
                                   (3, 5, 1000)] + _random_shapes(97, 5))
def test_lamport_oneshot_call(gpu, W, M, N):
    """One rank (a different one each call) makes the one-launch call after
    the other ranks pushed; then the others read.  Everything matches the
    oracle's pushes and readers bit for bit (norm within tolerance)."""
    comms = new_comms(W, M, N, gpu)
    hcomms = [orc.lamport_comm(W, M, N) for _ in range(W)]
    for f in range(4):
        xs, res, w = synth.fused_inputs(W, M, N, [96, W, M, N, f])
        me = f % W
        dx = [dev_u16(x, gpu) for x in xs]
        dr, dw = dev_u16(res, gpu), dev_u16(w, gpu)
        for r in range(W):
            orc.lamport_push(xs[r], r, hcomms, f)
            if r != me:
                ar.ar_lamport_push(dx[r], r, comms, f)
        ro, no = torch.empty_like(dr), torch.empty_like(dr)
        bad = torch.zeros(1, dtype=torch.int32, device=gpu)
        ar.ar_lamport_oneshot_residual_rmsnorm(dx[me], me, comms, dr, dw, ro, no, 1e-6, f,
                                               0, bad)
        sync()
        wro, wno, exact, wbad = orc.lamport_fused_residual_rmsnorm(hcomms[me], W, res, w,
                                                                   1e-6, f)
        assert int(bad.item()) == wbad == 0
        assert np.array_equal(host_u16(ro), wro)
        ok, _ = norm_within_tolerance(host_u16(no), exact)
        assert ok.all()
        for p in range(W):                       # the in-kernel push landed everywhere
            assert np.array_equal(host_words(comms[p]), hcomms[p]), (f, p)
        for p in range(W):
            if p == me:
                continue
            ro2, no2 = torch.empty_like(dr), torch.empty_like(dr)
            ar.ar_lamport_fused_residual_rmsnorm(comms[p], W, dr, dw, ro2, no2, 1e-6, f, 0, bad)
            sync()
            orc.lamport_fused_residual_rmsnorm(hcomms[p], W, res, w, 1e-6, f)
            assert int(bad.item()) == 0
            assert np.array_equal(host_u16(ro2), wro)
            assert np.array_equal(host_words(comms[p]), hcomms[p])


def test_lamport_flag_sequence_across_the_wrap(gpu):
    """Calls with flags P - 4 .. P - 1, 0 .. 2 (P = AR_LAMPORT_FLAG_PERIOD),
    each advanced with ar_lamport_next_flag: every call finds its region all
    sentinel before its pushes and matches the oracle's call sequence."""
    W, M, N = 3, 2, 64
    comms = new_comms(W, M, N, gpu)
    hcomms = [orc.lamport_comm(W, M, N) for _ in range(W)]
    words = M * N // 2
    f = ar.AR_LAMPORT_FLAG_PERIOD - 4
    for call in range(7):
        sync()
        for c in comms:
            reg = host_words(c).reshape(3, W * words)[f % 3]
            assert np.all(reg == SENT), f"region {f % 3} not clear before flag {f}"
        xs, res, w = synth.fused_inputs(W, M, N, [95, call])
        run_call(xs, res, w, comms, hcomms, f, gpu)
        f = ar.ar_lamport_next_flag(f)
    assert f == 3


def test_lamport_flag_past_the_period_is_refused(gpu):
    W, M, N = 2, 1, 64
    comms = new_comms(W, M, N, gpu)
    x = torch.zeros((M, N), dtype=torch.int16, device=gpu)
    sync()
    before = [host_words(c).copy() for c in comms]
    with pytest.raises(ar.ArError) as e:
        ar.ar_lamport_push(x, 0, comms, ar.AR_LAMPORT_FLAG_PERIOD)
    assert e.value.status == ar.AR_ERR_ARG
    sync()
    for c, b in zip(comms, before):
        assert np.array_equal(host_words(c), b)


def run_all_ranks(xs, res, w, comms, hcomms, flag, device, eps=1e-6):
    """One all-ranks launch (every rank pushes and reads at once), checked
    against the oracle's pushes of every rank followed by every reader."""
    W = len(xs)
    dx = [dev_u16(x, device) for x in xs]
    dr, dw = dev_u16(res, device), dev_u16(w, device)
    ros = [torch.empty_like(dr) for _ in range(W)]
    nos = [torch.empty_like(dr) for _ in range(W)]
    bad = torch.zeros(1, dtype=torch.int32, device=device)
    ar.ar_lamport_all_ranks_residual_rmsnorm(dx, comms, dr, dw, ros, nos, eps, flag,
                                             ar.AR_MAX_SPINS, bad)
    sync()
    assert int(bad.item()) == 0, "a peer slot never arrived"
    for r in range(W):
        orc.lamport_push(xs[r], r, hcomms, flag)
    for p in range(W):
        wro, _, exact, wbad = orc.lamport_fused_residual_rmsnorm(hcomms[p], W, res, w, eps, flag)
        assert wbad == 0
        assert np.array_equal(host_u16(ros[p]), wro), f"residual_out, rank {p}"
        ok, _ = norm_within_tolerance(host_u16(nos[p]), exact)
        assert ok.all(), f"norm_out, rank {p}"
    for p in range(W):
        assert np.array_equal(host_words(comms[p]), hcomms[p]), f"comm buffer of rank {p}"


@pytest.mark.parametrize("W,M,N", [(4, 1, 2048), (4, 16, 2048), (4, 128, 2048), (2, 3, 8),
                                   (8, 5, 1000), (3, 7, 16384)])
def test_lamport_all_ranks_in_one_launch(gpu, W, M, N):
    """All ranks' one-launch programs in one launch, over consecutive flags:
    each rank's reader polls peer slots that other workgroups of the same
    launch are pushing, and every rank's outputs and buffer match the
    oracle's call sequence."""
    comms = new_comms(W, M, N, gpu)
    hcomms = [orc.lamport_comm(W, M, N) for _ in range(W)]
    for f in range(4):
        xs, res, w = synth.fused_inputs(W, M, N, [98, W, M, N, f])
        run_all_ranks(xs, res, w, comms, hcomms, f, gpu)


def test_lamport_all_ranks_graph_replays(gpu):
    """The all-ranks launch captured for flags 0..5 and replayed three times
    (with eager work between): every replay leaves outputs equal to the
    eager launch's and no chunk missing."""
    W, M, N, eps = 4, 16, 2048, 1e-6
    xs, res, w = synth.fused_inputs(W, M, N, [99])
    dx = [dev_u16(x, gpu) for x in xs]
    dr, dw = dev_u16(res, gpu), dev_u16(w, gpu)
    comms = new_comms(W, M, N, gpu)
    ros = [torch.empty_like(dr) for _ in range(W)]
    nos = [torch.empty_like(dr) for _ in range(W)]
    bad = torch.zeros(1, dtype=torch.int32, device=gpu)
    calls = [lambda f=f: ar.ar_lamport_all_ranks_residual_rmsnorm(
        dx, comms, dr, dw, ros, nos, eps, f, ar.AR_MAX_SPINS, bad) for f in range(6)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(s)
    sync()
    want = [(host_u16(a), host_u16(b)) for a, b in zip(ros, nos)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    for rep in range(3):
        for t in ros + nos:
            t.zero_()
        sync()
        g.replay()
        sync()
        assert int(bad.item()) == 0, f"replay {rep}: a slot never arrived"
        for p in range(W):
            assert np.array_equal(host_u16(ros[p]), want[p][0]), (rep, p)
            assert np.array_equal(host_u16(nos[p]), want[p][1]), (rep, p)


def test_lamport_all_ranks_refuses_what_cannot_be_resident(gpu):
    W, M, N = 8, 4096, 2048
    x = torch.zeros((M, N), dtype=torch.int16, device=gpu)
    comms = [torch.empty(ar.ar_lamport_comm_bytes(W, M, N) // 4, dtype=torch.int32, device=gpu)
             for _ in range(W)]
    outs = [torch.empty_like(x) for _ in range(2 * W)]
    with pytest.raises(ar.ArError) as e:
        ar.ar_lamport_all_ranks_residual_rmsnorm([x] * W, comms, x.clone(), x[0].clone(),
                                                 outs[:W], outs[W:], 1e-6, 0)
    assert e.value.status == ar.AR_ERR_CAPACITY
