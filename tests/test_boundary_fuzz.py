"""Seeded random checks of the C ABI's argument validation (CPU only).

Each case starts from a random valid call (random W, sizes, flags and fake,
never dereferenced device addresses far apart) and breaks exactly one rule
stated in include/libar.h, or none.  The library must return the status the
header gives for that rule; a call that breaks nothing must reach the launch,
which on a machine without a GPU the HIP runtime rejects (AR_ERR_HIP), or
return AR_OK without launching when its size is zero.
"""
import numpy as np
import pytest
import torch

from ar_rmsnorm_amd import libar as ar

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="fake addresses only where no GPU can take a launch")

BASE = 1 << 44          # fake device addresses: slots 2^40 bytes apart
SLOT = 1 << 40
MAX_ELEMS = 1 << 40


def addr(i: int) -> int:
    return BASE + i * SLOT


def status(fn, *args, **kw):
    kw.setdefault("stream", 0)       # the null stream: no torch device needed
    try:
        with ar.checks_disabled():   # fake addresses: the C ABI's checks answer
            fn(*args, **kw)
    except ar.ArError as e:
        return e.status
    return ar.AR_OK


def launched(n: int) -> int:
    """Status of a valid call: AR_OK when nothing is launched, else the
    runtime's rejection of the launch on a machine without a GPU."""
    return ar.AR_OK if n == 0 else ar.AR_ERR_HIP


CASES = 300


@pytest.mark.parametrize("seed", range(4))
def test_reduce_1stage_single_violations(seed):
    g = np.random.default_rng([500, seed])
    for _ in range(CASES):
        W = int(g.integers(2, 9))
        n = 8 * int(g.integers(0, 1 << 20))
        ins = [addr(i) for i in range(W)]
        out = addr(W)
        want = launched(n)
        kind = int(g.integers(0, 8))
        if kind == 1:
            ins = [addr(i) for i in range(int(g.choice([1, 9, 10])))]
            want = ar.AR_ERR_WORLD
        elif kind == 2:
            ins[int(g.integers(0, W))] = None
            want = ar.AR_ERR_NULL
        elif kind == 3:
            out = None
            want = ar.AR_ERR_NULL
        elif kind == 4:
            n = int(g.choice([n + int(g.integers(1, 8)), -8, MAX_ELEMS + 8]))
            want = ar.AR_ERR_ARG
        elif kind == 5:
            r = int(g.integers(0, W + 1))
            bump = int(g.choice([2, 4, 8]))
            if r == W:
                out += bump
            else:
                ins[r] += bump
            want = ar.AR_ERR_ALIGN
        elif kind == 6 and n >= 16:
            r = int(g.integers(0, W))
            out = ins[r] + 16 * int(g.integers(1, n // 8))     # partial overlap
            want = ar.AR_ERR_ARG
        elif kind == 7:
            out = ins[int(g.integers(0, W))]                   # in place: allowed
        assert status(ar.ar_reduce_1stage, ins, out, n) == want, (kind, W, n)


@pytest.mark.parametrize("seed", range(4))
def test_reduce_2stage_single_violations(seed):
    g = np.random.default_rng([501, seed])
    for _ in range(CASES):
        W = int(g.integers(2, 9))
        P = int(g.integers(0, 1 << 18))
        n = 8 * P
        rank = int(g.integers(0, W))
        flags = int(g.choice([0, ar.AR_STAGE_RS, ar.AR_STAGE_AG,
                              ar.AR_STAGE_RS | ar.AR_STAGE_AG])) | \
            int(g.choice([0, ar.AR_ORDER_RANK]))
        stages = flags & 3 or 3
        rs, ag = bool(stages & 1), bool(stages & 2)
        ins = [addr(i) for i in range(W)]
        tms = [addr(8 + i) for i in range(W)]
        out = addr(16)
        tmp_bytes = (P // W + P % W) * 16
        want = launched(n)
        kind = int(g.integers(0, 10))
        if kind == 1:
            flags |= 8 << int(g.integers(0, 8))
            want = ar.AR_ERR_ARG
        elif kind == 2:
            tms[int(g.integers(0, W))] = None
            want = ar.AR_ERR_NULL
        elif kind == 3 and ag:
            out = None
            want = ar.AR_ERR_NULL
        elif kind == 4:
            rank = int(g.choice([-1, W, W + 3]))
            want = ar.AR_ERR_ARG
        elif kind == 5:
            n = int(g.choice([n + 4, -8, MAX_ELEMS + 8]))
            want = ar.AR_ERR_ARG
        elif kind == 6:
            tms[int(g.integers(0, W))] += int(g.choice([2, 4, 8]))
            want = ar.AR_ERR_ALIGN
        elif kind == 7 and ag and n > 0:
            out = ins[int(g.integers(0, W))] + 16 * int(g.integers(0, P))
            want = ar.AR_ERR_ARG
        elif kind == 8 and rs and n > 0:
            tms[rank] = ins[int(g.integers(0, W))] + 16 * int(g.integers(0, P))
            want = ar.AR_ERR_ARG
        elif kind == 9 and rs and ag and n > 0 and tmp_bytes > 0:
            peer = (rank + 1 + int(g.integers(0, W - 1))) % W
            tms[rank] = tms[peer] + 16 * int(g.integers(0, tmp_bytes // 16))
            want = ar.AR_ERR_ARG
        elif kind == 0 and not ag:
            out = None                                         # allowed without AG
        assert status(ar.ar_reduce_2stage, ins, tms, rank, out, flags, n) == want, \
            (kind, W, n, rank, flags)


@pytest.mark.parametrize("seed", range(4))
def test_fused_single_violations(seed):
    g = np.random.default_rng([502, seed])
    for _ in range(CASES):
        W = int(g.integers(2, 9))
        M = int(g.integers(0, 4096))
        N = 8 * int(g.integers(1, 2049))
        eps = float(g.choice([0.0, 1e-6, 1e-5]))
        ins = [addr(i) for i in range(W)]
        res, w, ro, no = addr(8), addr(9), addr(10), addr(11)
        want = launched(M)
        kind = int(g.integers(0, 9))
        if kind == 1:
            res = None
            want = ar.AR_ERR_NULL
        elif kind == 2:
            N = int(g.choice([N + 4, 0, 16392, 16384 + 8 * int(g.integers(1, 100))]))
            want = ar.AR_ERR_ARG
        elif kind == 3:
            M = -1
            want = ar.AR_ERR_ARG
        elif kind == 4:
            eps = float(g.choice([-1e-6, float("nan"), float("inf")]))
            want = ar.AR_ERR_ARG
        elif kind == 5:
            no += int(g.choice([2, 4, 8]))
            want = ar.AR_ERR_ALIGN
        elif kind == 6 and M > 0:
            no = ins[int(g.integers(0, W))]
            want = ar.AR_ERR_ARG
        elif kind == 7 and M > 0:
            no = ro
            want = ar.AR_ERR_ARG
        elif kind == 8:
            ro = res                                           # in place: allowed
        assert status(ar.ar_fused_residual_rmsnorm, ins, res, w, ro, no, eps, M, N) == want, \
            (kind, W, M, N, eps)


@pytest.mark.parametrize("fmt", ["ll", "ll128"])
@pytest.mark.parametrize("seed", range(3))
def test_wire_single_violations(fmt, seed):
    g = np.random.default_rng([503, seed, fmt == "ll128"])
    line = 16 if fmt == "ll" else 128
    lines_of = ar.ll_lines if fmt == "ll" else ar.ll128_lines
    pack = ar.ll_pack if fmt == "ll" else ar.ll128_pack
    unpack = ar.ll_unpack_reduce if fmt == "ll" else ar.ll128_unpack_reduce
    for _ in range(CASES):
        n = int(g.integers(0, 1 << 22))
        L = lines_of(n)
        sl = max(1, -(-L // 8) + int(g.integers(0, 3)))
        W = int(g.integers(1, 9))
        src, fifo, out, bad = addr(0) + 4 * int(g.integers(0, 4)), addr(1), addr(2), addr(3)
        fifos = [addr(4 + i) for i in range(W)]
        spins = int(g.integers(0, ar.AR_MAX_SPINS + 1))
        want_p = want_u = launched(n)
        kind = int(g.integers(0, 8))
        if kind == 1:
            sl = 0
            want_p = want_u = ar.AR_ERR_ARG
        elif kind == 2 and L > 8:
            sl = (L - 1) // 8            # 8 steps hold fewer than L lines
            want_p = want_u = ar.AR_ERR_CAPACITY
        elif kind == 3:
            src += 2
            fifo += int(g.choice([4, 8])) if fmt == "ll" else int(g.choice([16, 64]))
            fifos[int(g.integers(0, W))] = fifo
            want_p = want_u = ar.AR_ERR_ALIGN
        elif kind == 4 and n > 0:
            fifo = src - 4 * (src % 16 // 4) + 16 * line  # inside the source (aligned)
            if fifo < src + 4 * n:
                want_p = ar.AR_ERR_ARG
            out = fifos[0] + 4 * int(g.integers(0, 8 * sl * line // 4))
            out -= out % 4
            want_u = ar.AR_ERR_ARG
        elif kind == 5:
            spins = ar.AR_MAX_SPINS + 1 + int(g.integers(0, 100))
            want_u = ar.AR_ERR_ARG
        elif kind == 6:
            fifos = [addr(4 + i) for i in range(int(g.choice([0, 9])))]
            want_u = ar.AR_ERR_WORLD
        elif kind == 7:
            bad = out + 4 * int(g.integers(0, max(1, n)))
            if n > 0:
                want_u = ar.AR_ERR_ARG
        assert status(pack, src, fifo, sl, 0, n=n) == want_p, ("pack", kind, n, sl)
        assert status(unpack, fifos, out, sl, 0, spins, bad, n=n) == want_u, \
            ("unpack", kind, n, sl, W)


@pytest.mark.parametrize("seed", range(3))
def test_fused_2stage_single_violations(seed):
    g = np.random.default_rng([504, seed])
    for _ in range(CASES):
        W = int(g.integers(2, 9))
        M = int(g.integers(0, 2048))
        N = 8 * int(g.integers(1, 2049))
        rank = int(g.integers(0, W))
        flags = int(g.choice([0, ar.AR_STAGE_RS, ar.AR_STAGE_AG])) | \
            int(g.choice([0, ar.AR_ORDER_RANK]))
        stages = flags & 3 or 3
        rs, ag = bool(stages & 1), bool(stages & 2)
        ins = [addr(i) for i in range(W)]
        tms = [addr(8 + i) for i in range(W)]
        res, w, ro, no = addr(16), addr(17), addr(18), addr(19)
        tmp_bytes = 2 * (M // W + M % W) * N * 2
        want = launched(M)
        kind = int(g.integers(0, 9))
        if kind == 1:
            tms[int(g.integers(0, W))] = None
            want = ar.AR_ERR_NULL
        elif kind == 2 and ag:
            no = None
            want = ar.AR_ERR_NULL
        elif kind == 3:
            rank = int(g.choice([-1, W]))
            want = ar.AR_ERR_ARG
        elif kind == 4:
            N = int(g.choice([N + 2, 16392]))
            want = ar.AR_ERR_ARG
        elif kind == 5:
            flags |= 16
            want = ar.AR_ERR_ARG
        elif kind == 6:
            tms[int(g.integers(0, W))] += 8
            want = ar.AR_ERR_ALIGN
        elif kind == 7 and rs and M > 0:
            tms[rank] = ins[int(g.integers(0, W))]
            want = ar.AR_ERR_ARG
        elif kind == 8 and ag and M > 0 and tmp_bytes > 0:
            ro = tms[int(g.integers(0, W))] + 16 * int(g.integers(0, tmp_bytes // 16))
            want = ar.AR_ERR_ARG
        assert status(ar.ar_fused_residual_rmsnorm_2stage, ins, tms, rank, res, w, ro, no,
                      1e-6, flags, M, N) == want, (kind, W, M, N, rank, flags)


@pytest.mark.parametrize("seed", range(3))
def test_lamport_single_violations(seed):
    g = np.random.default_rng([505, seed])
    for _ in range(CASES):
        W = int(g.integers(2, 9))
        M = int(g.integers(0, 1024))
        N = 8 * int(g.integers(1, 2049))
        rank = int(g.integers(0, W))
        x = addr(0)
        comms = [addr(1 + i) for i in range(W)]
        res, w, ro, no, bad = addr(10), addr(11), addr(12), addr(13), addr(14)
        spins = int(g.integers(0, ar.AR_MAX_SPINS + 1))
        cb = ar.ar_lamport_comm_bytes(W, M, N)
        assert cb == 3 * W * M * N * 2
        want_push = want_read = want_one = launched(M)
        kind = int(g.integers(0, 8))
        if kind == 1:
            comms[int(g.integers(0, W))] = None
            want_push = want_one = ar.AR_ERR_NULL
        elif kind == 2:
            N = N + 4
            want_push = want_read = want_one = ar.AR_ERR_ARG
        elif kind == 3:
            rank = int(g.choice([-1, W]))
            want_push = want_one = ar.AR_ERR_ARG
        elif kind == 4:
            spins = ar.AR_MAX_SPINS + 1
            want_read = want_one = ar.AR_ERR_ARG
        elif kind == 5:
            bad += 2
            want_read = want_one = ar.AR_ERR_ALIGN
        elif kind == 6 and M > 0:
            q = int(g.integers(1, W))
            comms[q] = comms[0] + 16 * int(g.integers(0, cb // 16))   # two buffers overlap
            want_push = want_one = ar.AR_ERR_ARG
        elif kind == 7 and M > 0:
            no = comms[rank] + 16 * int(g.integers(0, cb // 16))      # output inside comm
            want_read = want_one = ar.AR_ERR_ARG
        own = comms[rank] if 0 <= rank < W else comms[0]
        if own is not None:
            assert status(ar.ar_lamport_fused_residual_rmsnorm, own, W, res, w, ro, no,
                          1e-6, 1, spins, bad, M, N) == want_read, ("read", kind, W, M, N)
        assert status(ar.ar_lamport_push, x, rank, comms, 1, M, N) == want_push, \
            ("push", kind, W, M, N, rank)
        assert status(ar.ar_lamport_oneshot_residual_rmsnorm, x, rank, comms, res, w, ro, no,
                      1e-6, 1, spins, bad, M, N) == want_one, ("oneshot", kind, W, M, N, rank)


@pytest.mark.parametrize("seed", range(3))
def test_stream_single_violations(seed):
    g = np.random.default_rng([506, seed])
    units = {ar.AR_PROTO_LL: 8, ar.AR_PROTO_LL128: 120, ar.AR_PROTO_SIMPLE: 16}
    for _ in range(CASES):
        proto = int(g.integers(0, 3))
        n = int(g.integers(0, 1 << 22))
        step = units[proto] * int(g.integers(1, 5000))
        channels = int(g.integers(1, ar.AR_FIFO_MAX_CHANNELS + 1))
        src, out, fifo, cnt, err = addr(0), addr(1), addr(2), addr(3), addr(4)
        local = addr(5) if g.integers(0, 2) else None
        spins = int(g.integers(0, ar.AR_MAX_SPINS + 1))
        want = launched(n)
        kind = int(g.integers(0, 9))
        if kind == 1:
            err = None
            want = ar.AR_ERR_NULL
        elif kind == 2:
            step = units[proto] * int(g.integers(1, 100)) + int(g.integers(1, units[proto]))
            want = ar.AR_ERR_ARG
        elif kind == 3:
            channels = int(g.choice([0, ar.AR_FIFO_MAX_CHANNELS + 1]))
            want = ar.AR_ERR_ARG
        elif kind == 4:
            spins = ar.AR_MAX_SPINS + 1
            want = ar.AR_ERR_ARG
        elif kind == 5:
            cnt += 4
            want = ar.AR_ERR_ALIGN
        elif kind == 6:
            fifo += 64 if proto == ar.AR_PROTO_LL128 else 8
            want = ar.AR_ERR_ALIGN
        elif kind == 7 and n > 0:
            out = src + 4 * int(g.integers(0, n))
            want = ar.AR_ERR_ARG
        elif kind == 8 and n > 0:
            cnt = fifo                                              # counters in the ring
            want = ar.AR_ERR_ARG
        assert status(ar.ar_fifo_stream, proto, src, out, fifo, cnt, channels, step, 0, spins,
                      err, local, n=n) == want, (kind, proto, n, step, channels)
