"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties an oracle function to a value the pages print, a closed form
derived by hand, a special case that reduces to a library routine, an
invariant, or exact brute force on tiny inputs.  The cases are chosen so that
a plausible slip (wrong rounding tie, dropped term, wrong summation order or
start, wrong shard bound, transposed word, off-by-one slot) fails at least one.

Sources: [SGLv1] "SGLang Custom AllReduce v1 thread model" (todaynews.cc);
[NCCL14] "NCCL expert course 14: Simple, LL, LL128 wire formats"
(blog.cptz.space); [JITAR] "0-custom-all-reduce" (obnotes-4iw.pages.dev);
[TRIAR] "Triton + Symmetric Memory fused AllReduce + RMSNorm" (riverclouds.net).
"""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as orc
from ar_rmsnorm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

BF16_ONE = 0x3F80
BF16_2P24 = 0x4B80       # 2^24
BF16_M2P24 = 0xCB80      # -2^24


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def bf16_value(b: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", b << 16))[0])


# ---------------------------------------------------------------------------
# bf16 rounding  ([JITAR] section 4: widen to fp32, narrow once, nearest)
# ---------------------------------------------------------------------------
def test_bf16_rne_matches_torch_cast_exhaustively_on_low_halves():
    """fp32 -> bf16 must equal torch's CPU cast (an IEEE round-to-nearest-even
    library routine) on every low half-word under 263 high half-words."""
    his = sorted(set(range(0, 65536, 257)) |
                 {0x0000, 0x0080, 0x3F80, 0x7F7F, 0x7F80, 0x7FC0, 0x8000, 0xFF80})
    lo = np.arange(65536, dtype=np.uint32)
    bits = (np.array(his, np.uint32)[:, None] << 16 | lo[None, :]).reshape(-1)
    x = bits.view(np.float32)
    got = orc.bf16_rne(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    # NaN stays NaN (exponent all ones, nonzero fraction) and keeps its sign.
    g = got[nan]
    assert np.all((g & 0x7F80) == 0x7F80) and np.all((g & 0x7F) != 0)
    assert np.array_equal(g >> 15, (bits[nan] >> 31).astype(np.uint16))


@pytest.mark.parametrize("bits,want", [
    (0x3F808000, 0x3F80),   # exact tie, even kept part -> stays
    (0x3F818000, 0x3F82),   # exact tie, odd kept part -> rounds up to even
    (0x3F808001, 0x3F81),   # just above the tie
    (0x3F807FFF, 0x3F80),   # just below the tie
    (0x7F7FFFFF, 0x7F80),   # overflow to +inf
    (0xFF7FFFFF, 0xFF80),   # overflow to -inf
    (0x807FFFFF, 0x8080),   # largest negative denormal rounds to -min normal
    (0x00008000, 0x0000),   # tie at the bottom, even -> zero
    (0x00018000, 0x0002),   # denormal tie, odd -> up
    (0x7F800000, 0x7F80),   # +inf
    (0x80000000, 0x8000),   # -0.0 kept
])
def test_bf16_rne_hand_cases(bits, want):
    x = np.array([bits], np.uint32).view(np.float32)
    assert int(orc.bf16_rne(x)[0]) == want


def _nearest_even_check(x: Fraction, b: int):
    """b is the correct round-to-nearest-even bf16 of x (exact rationals)."""
    sign = -1 if x < 0 else 1
    assert (b >> 15) == (1 if sign < 0 else 0)
    mag = b & 0x7FFF
    ax = abs(x)
    maxf = bf16_value(0x7F7F)
    if mag == 0x7F80:
        # overflow: x lies at or beyond the midpoint of max and 2^128
        assert ax >= (maxf + Fraction(2) ** 128) / 2
        return
    v = bf16_value(mag)
    d = abs(ax - v)
    for nb in (mag - 1, mag + 1):
        if nb < 0 or nb >= 0x7F80:
            continue
        dn = abs(ax - bf16_value(nb))
        assert d <= dn
        if d == dn:                        # tie: the kept code is even
            assert mag % 2 == 0


def test_bf16_from_f64_is_nearest_even_by_exact_brute_force():
    g = np.random.default_rng(7)
    xs = []
    for _ in range(3000):
        m = g.uniform(1.0, 2.0)
        e = int(g.integers(-140, 129))
        xs.append(math.ldexp(m, e) * (1 if g.random() < 0.5 else -1))
    # exact ties and near-ties: bf16 midpoints, and a hair either side
    for _ in range(1000):
        b = int(g.integers(0x0001, 0x7F7F))
        mid = (bf16_value(b) + bf16_value(b + 1)) / 2
        xs += [float(mid), math.nextafter(float(mid), 0), math.nextafter(float(mid), math.inf)]
    xs += [3.3961e38, 3.3958e38, -3.4e38, 1e-45, 9.2e-41, 2.0 ** -133, 2.0 ** -134,
           3 * 2.0 ** -135]
    got = orc.bf16_from_f64(np.array(xs))
    for x, b in zip(xs, got):
        _nearest_even_check(Fraction(x), int(b))


def test_bf16_from_f64_agrees_with_fp32_rounding_on_floats():
    g = np.random.default_rng(8)
    bits = g.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(orc.bf16_from_f64(x.astype(np.float64)), orc.bf16_rne(x))


# ---------------------------------------------------------------------------
# one-stage reduce  ([SGLv1] "1stage: full kernel and timeline")
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("W", range(2, 9))
def test_1stage_closed_forms(W):
    n = 64
    ones = [np.full(n, BF16_ONE, np.uint16) for _ in range(W)]
    assert np.all(orc.bf16_to_f32(orc.reduce_1stage(ones)) == W)
    # x_r = r + 1  ->  W (W + 1) / 2 exactly
    xs = [np.full(n, f32_bits(r + 1.0) >> 16, np.uint16) for r in range(W)]
    assert np.all(orc.bf16_to_f32(orc.reduce_1stage(xs)) == W * (W + 1) // 2)
    # all -0.0 -> -0.0: the sum starts from rank 0's value, not from +0.0
    negz = [np.full(n, 0x8000, np.uint16) for _ in range(W)]
    assert np.all(orc.reduce_1stage(negz) == 0x8000)
    # one +0.0 among -0.0 -> +0.0
    mixed = negz[:-1] + [np.zeros(n, np.uint16)]
    assert np.all(orc.reduce_1stage(mixed) == 0x0000)


def test_1stage_rank_order_is_revealed_by_absorption():
    """x = (1, 2^24, 1, -2^24): in fp32, 1 + 2^24 is a tie that rounds back to
    2^24, so the rank-order sum ((1 + 2^24) + 1) - 2^24 is 0.  A tree order
    (1 + 2^24) + (1 - 2^24) gives 1 and the reverse order gives 2."""
    vals = [BF16_ONE, BF16_2P24, BF16_ONE, BF16_M2P24]
    xs = [np.full(16, v, np.uint16) for v in vals]
    assert np.all(orc.reduce_1stage(xs) == 0x0000)
    assert np.all(orc.bf16_to_f32(orc.reduce_1stage(xs[::-1])) == 2.0)


def test_1stage_w2_equals_rounded_exact_sum():
    """For two bf16 values whose exponents differ by at most 15 the fp32 sum
    is exact, so the result is the exact sum rounded once; torch's CPU cast
    (float64 -> float32 exact here, then RNE to bf16) supplies the rounding."""
    g = np.random.default_rng(11)
    x0 = orc.bf16_rne(g.standard_normal(50_000).astype(np.float32))
    x1 = orc.bf16_rne((g.standard_normal(50_000) * 10.0 ** g.integers(-3, 4, 50_000))
                      .astype(np.float32))
    a, b = orc.bf16_to_f32(x0).astype(np.float64), orc.bf16_to_f32(x1).astype(np.float64)
    ea = np.frexp(a)[1]
    eb = np.frexp(b)[1]
    keep = (np.abs(ea - eb) <= 15) & (a != 0) & (b != 0)
    exact = torch.from_numpy((a + b)[keep])
    want = exact.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.reduce_1stage([x0, x1])[keep]
    assert keep.sum() > 40_000
    assert np.array_equal(got, want)


def test_1stage_error_within_bound_of_exact_sum():
    """The fp32 chain of W-1 adds then one bf16 rounding is within
    (W-1) * 2^-24 * sum|x| + half a bf16 ulp of the exact sum."""
    g = np.random.default_rng(12)
    W, n = 8, 20_000
    xs = [orc.bf16_rne(g.standard_normal(n).astype(np.float32)) for _ in range(W)]
    got = orc.bf16_to_f32(orc.reduce_1stage(xs)).astype(np.float64)
    vals = np.stack([orc.bf16_to_f32(x).astype(np.float64) for x in xs])
    exact = vals.sum(0)                     # float64 sum of 8 bf16: exact
    bound = (W - 1) * 2.0 ** -24 * np.abs(vals).sum(0) * 1.0001
    half_ulp = np.abs(exact + bound) * 2.0 ** -8
    assert np.all(np.abs(got - exact) <= bound + half_ulp + 1e-45)


# ---------------------------------------------------------------------------
# two-stage reduce  ([SGLv1] "2stage: sharding, rotation, no exit barrier")
# ---------------------------------------------------------------------------
def test_2stage_partition_numbers_printed_on_the_page():
    # 512 KB of bf16 at W=8: 32768 packs, part = 4096 ([SGLv1] worked example)
    n = 512 * 1024 // 2
    assert orc.shard_range(n, 8, 0) == (0, 4096)
    assert orc.shard_range(n, 8, 7) == (7 * 4096, 32768)
    # the 8 MB cap: 524288 packs, part = 65536
    assert orc.shard_range(4_194_304, 8, 3) == (3 * 65536, 4 * 65536)
    # remainder goes to the last shard: 45 packs over 8 -> part 5, last 10
    assert orc.shard_range(45 * 8, 8, 6) == (30, 35)
    assert orc.shard_range(45 * 8, 8, 7) == (35, 45)
    # fewer packs than shards: everything is the last shard's
    assert orc.shard_range(3 * 8, 4, 0) == (0, 0)
    assert orc.shard_range(3 * 8, 4, 3) == (0, 3)


def test_2stage_rotated_order_hand_derived():
    """x = (1, 2^24, 1, -2^24) at every element, W=4, 4 packs (one per shard).
    Owner s sums from x_s onwards:
      s=0: ((1 + 2^24) + 1) - 2^24 = 0
      s=1: ((2^24 + 1) - 2^24) + 1 = 1
      s=2: ((1 - 2^24) + 1) + 2^24 = 2
      s=3: ((-2^24 + 1) + 2^24) + 1 = 2
    and with the rank order every shard is 0."""
    vals = [BF16_ONE, BF16_2P24, BF16_ONE, BF16_M2P24]
    xs = [np.full(32, v, np.uint16) for v in vals]
    got = orc.bf16_to_f32(orc.reduce_2stage(xs)).reshape(4, 8)
    assert np.array_equal(got, np.repeat(np.array([[0.0], [1.0], [2.0], [2.0]]), 8, 1))
    assert np.all(orc.reduce_2stage(xs, rank_order=True) == 0)
    # the scatter/gather pieces compose to the same result
    tmps = [orc.reduce_scatter(xs, s) for s in range(4)]
    assert [t.size for t in tmps] == [8, 8, 8, 8]
    assert np.array_equal(orc.all_gather(tmps, 32), orc.reduce_2stage(xs))


@pytest.mark.parametrize("P", [5, 45, 64, 1027])
def test_2stage_w2_equals_1stage(P):
    """With two ranks the rotated order is x0+x1 or x1+x0, equal by fp32
    commutativity, so the two-stage result is the one-stage result."""
    g = np.random.default_rng(P)
    xs = [orc.bf16_rne(g.standard_normal(P * 8).astype(np.float32)) for _ in range(2)]
    assert np.array_equal(orc.reduce_2stage(xs), orc.reduce_1stage(xs))


@pytest.mark.parametrize("W", [3, 4, 8])
def test_2stage_rank_order_flag_equals_1stage_and_ones(W):
    g = np.random.default_rng(W)
    xs = [orc.bf16_rne(g.standard_normal(45 * 8).astype(np.float32)) for _ in range(W)]
    assert np.array_equal(orc.reduce_2stage(xs, rank_order=True), orc.reduce_1stage(xs))
    ones = [np.full(45 * 8, BF16_ONE, np.uint16) for _ in range(W)]
    assert np.all(orc.bf16_to_f32(orc.reduce_2stage(ones)) == W)


# ---------------------------------------------------------------------------
# fused all-reduce + residual + RMSNorm  ([TRIAR] "what this operator computes")
# ---------------------------------------------------------------------------
def _fused(xs, res, w, eps=1e-6):
    return orc.fused_residual_rmsnorm(xs, res, w, eps)


@pytest.mark.parametrize("c,W", [(1.0, 4), (-1.0, 4), (3.0, 2), (0.25, 8)])
def test_fused_constant_row_returns_weight(c, W):
    """h = c at every position: rms = 1/sqrt(c^2 + eps), (h*rms) differs from
    sign(c) by ~eps/(2c^2) << half a bf16 ulp, so norm_out = sign(c) * w."""
    M, N = 3, 2048
    g = np.random.default_rng(5)
    w = orc.bf16_rne(g.normal(1.0, 0.1, N).astype(np.float32))
    xs = [np.full((M, N), f32_bits(c) >> 16, np.uint16)] + \
         [np.zeros((M, N), np.uint16) for _ in range(W - 1)]
    res = np.zeros((M, N), np.uint16)
    ro, no, ne = _fused(xs, res, w)
    assert np.all(ro == (f32_bits(c) >> 16))
    want = w if c > 0 else (w ^ 0x8000)
    assert np.array_equal(no, np.broadcast_to(want, (M, N)))


def test_fused_all_ones_w4():
    M, N, W = 2, 1024, 4
    w = orc.bf16_rne(np.linspace(0.5, 1.5, N).astype(np.float32))
    xs = [np.full((M, N), BF16_ONE, np.uint16) for _ in range(W)]
    res = np.zeros((M, N), np.uint16)
    ro, no, _ = _fused(xs, res, w)
    assert np.all(orc.bf16_to_f32(ro) == 4.0)
    assert np.array_equal(no, np.broadcast_to(w, (M, N)))


@pytest.mark.parametrize("c", [2.0 ** -12, 2.0 ** -10, 1e-3])
def test_fused_constant_row_where_eps_matters(c):
    """Closed form y = c / sqrt(c^2 + eps) * w_j; at these c, eps is 1..16x
    c^2, so a dropped or misplaced eps changes the value visibly."""
    M, N, W, eps = 1, 256, 2, 1e-6
    cb = orc.bf16_rne(np.array([c], np.float32))[0]
    cv = float(orc.bf16_to_f32(np.array([cb]))[0])
    w = orc.bf16_rne(np.linspace(-2, 2, N).astype(np.float32))
    xs = [np.full((M, N), cb, np.uint16), np.zeros((M, N), np.uint16)]
    _, no, ne = _fused(xs, np.zeros((M, N), np.uint16), w, eps)
    want = cv / math.sqrt(cv * cv + eps) * orc.bf16_to_f32(w).astype(np.float64)
    assert np.allclose(ne[0], want, rtol=1e-13, atol=0)


def test_fused_reduces_to_torch_rms_norm_when_peers_are_zero():
    """With x_1..x_{W-1} = 0 the all-reduce is x_0 exactly, so the operator is
    h = fp32(x_0 + residual) followed by torch's rms_norm (library routine)."""
    W, M, N, eps = 4, 16, 2048, 1e-6
    g = np.random.default_rng(21)
    x0 = orc.bf16_rne(g.standard_normal((M, N)).astype(np.float32))
    res = orc.bf16_rne(g.standard_normal((M, N)).astype(np.float32))
    w = orc.bf16_rne(g.normal(1.0, 0.1, N).astype(np.float32))
    xs = [x0] + [np.zeros((M, N), np.uint16) for _ in range(W - 1)]
    ro, no, ne = _fused(xs, res, w, eps)
    h = torch.from_numpy(orc.bf16_to_f32(x0)) + torch.from_numpy(orc.bf16_to_f32(res))
    want_ro = h.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ro, want_ro)
    wt = torch.from_numpy(orc.bf16_to_f32(w)).double()
    want = torch.nn.functional.rms_norm(h.double(), (N,), wt, eps).numpy()
    assert np.allclose(ne, want, rtol=1e-12, atol=1e-300)
    # norm_out is the nearest bf16 of the exact value
    assert np.array_equal(no, orc.bf16_from_f64(ne))


def test_fused_power_of_two_scale_invariance_eps0():
    """Scaling x and residual by 2^k scales residual_out by 2^k exactly and,
    with eps = 0, leaves norm_out unchanged."""
    W, M, N = 4, 4, 512
    g = np.random.default_rng(22)
    xs = [orc.bf16_rne(g.standard_normal((M, N)).astype(np.float32)) for _ in range(W)]
    res = orc.bf16_rne(g.standard_normal((M, N)).astype(np.float32))
    w = orc.bf16_rne(g.normal(1.0, 0.1, N).astype(np.float32))
    ro, no, _ = _fused(xs, res, w, 0.0)
    k = 5
    sc = lambda a: np.where((a & 0x7F80) != 0, a + (k << 7), a).astype(np.uint16)  # noqa: E731
    ro2, no2, _ = _fused([sc(x) for x in xs], sc(res), w, 0.0)
    r1, r2 = orc.bf16_to_f32(ro), orc.bf16_to_f32(ro2)
    assert np.array_equal(r2, r1 * np.float32(2 ** k))
    assert np.array_equal(no2, no)


def test_fused_residual_out_equals_1stage_plus_residual():
    """residual_out is the one-stage sum (kept in fp32) plus the residual: for
    a zero residual it is the one-stage result exactly."""
    W, M, N = 4, 8, 2048
    g = np.random.default_rng(23)
    xs = [orc.bf16_rne(g.standard_normal((M, N)).astype(np.float32)) for _ in range(W)]
    ro, _, _ = _fused(xs, np.zeros((M, N), np.uint16),
                      np.full(N, BF16_ONE, np.uint16))
    assert np.array_equal(ro.reshape(-1), orc.reduce_1stage([x.reshape(-1) for x in xs]))


# ---------------------------------------------------------------------------
# LL / LL128 wire formats ([NCCL14])
# ---------------------------------------------------------------------------
def _read_golden(name):
    meta, rows = {}, {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0].isdigit():
                rows[int(parts[0])] = [int(p, 16) for p in parts[1:]]
            else:
                meta[parts[0]] = parts[1:]
    return meta, rows


def test_ll_pack_golden_bytes():
    meta, rows = _read_golden("ll_pack_n5.txt")
    src = np.array([float(v) for v in meta["payload_f32"]], np.float32)
    fifo = np.full(8 * 16, 0xEE, np.uint8)
    orc.ll_pack(src, fifo, int(meta["step_lines"][0]), int(meta["first_step"][0]))
    words = fifo.view("<u4").reshape(8, 4)
    for i in range(8):
        assert list(words[i]) == rows[i], i


def test_ll128_pack_golden_bytes():
    meta, rows = _read_golden("ll128_pack_n31.txt")
    a, b = (int(v) for v in meta["payload_f32_range"])
    src = np.arange(a, b + 1, dtype=np.float32)
    fifo = np.full(8 * 128, 0xEE, np.uint8)
    orc.ll128_pack(src, fifo, int(meta["step_lines"][0]), int(meta["first_step"][0]))
    words = fifo.view("<u4").reshape(8, 32)
    for i in range(8):
        assert list(words[i]) == rows[i], i


def test_wire_geometry_matches_printed_buffer_table():
    """[NCCL14] "default buffers and effective data per step": LL 524288 B
    wire buffer -> 65536 B per step -> 32768 data B; LL128 4915200 B ->
    614400 B per step -> 576000 data B; payload efficiency 8/16 and 120/128."""
    ll_step_lines = 524288 // 8 // 16
    ll128_step_lines = 4915200 // 8 // 128
    assert (ll_step_lines, ll128_step_lines) == (4096, 4800)
    # a step's worth of data fills exactly one step's worth of lines
    assert orc.ll_lines(32768 // 4) == ll_step_lines
    assert orc.ll128_lines(576000 // 4) == ll128_step_lines
    assert orc.ll_lines(32768 // 4 + 1) == ll_step_lines + 1
    assert orc.ll128_lines(576000 // 4 + 1) == ll128_step_lines + 1
    # efficiency measured on the packed bytes: flags and data of one step
    n = 32768 // 4
    fifo = np.zeros(8 * ll_step_lines * 16, np.uint8)
    orc.ll_pack(np.ones(n, np.float32), fifo, ll_step_lines)
    used = fifo[: ll_step_lines * 16].view("<u4").reshape(-1, 4)
    assert np.all(used[:, 1] == 1) and np.all(used[:, 3] == 1)
    assert Fraction(n * 4, ll_step_lines * 16) == Fraction(8, 16)
    n = 576000 // 4
    fifo = np.zeros(8 * ll128_step_lines * 128, np.uint8)
    orc.ll128_pack(np.ones(n, np.float32), fifo, ll128_step_lines)
    used = fifo[: ll128_step_lines * 128].view("<u8").reshape(-1, 16)
    assert np.all(used[:, 15] == 1)
    assert Fraction(n * 4, ll128_step_lines * 128) == Fraction(120, 128)


@pytest.mark.parametrize("fmt", ["ll", "ll128"])
@pytest.mark.parametrize("n,step_lines,first_step", [
    (1, 1, 0), (2, 1, 5), (29, 1, 0), (30, 2, 3), (31, 1, 7), (1000, 200, 0),
    (1013, 127, 9), (4096, 512, 2 ** 32 - 3)])
def test_round_trip_single_fifo(fmt, n, step_lines, first_step):
    pack = orc.ll_pack if fmt == "ll" else orc.ll128_pack
    unpack = orc.ll_unpack_reduce if fmt == "ll" else orc.ll128_unpack_reduce
    lines = (orc.ll_lines if fmt == "ll" else orc.ll128_lines)(n)
    size = 16 if fmt == "ll" else 128
    step_lines = max(step_lines, -(-lines // 8))   # one call spans <= 8 steps
    g = np.random.default_rng(n)
    src = g.standard_normal(n).astype(np.float32)
    src[::7] = -0.0
    fifo = np.zeros(8 * step_lines * size, np.uint8)
    pack(src, fifo, step_lines, first_step)
    out, valid, bad = unpack([fifo], n, step_lines, first_step)
    assert bad == 0 and valid.all()
    assert np.array_equal(out.view(np.uint32), src.view(np.uint32))


@pytest.mark.parametrize("fmt", ["ll", "ll128"])
def test_decode_reduce_small_integers_and_order(fmt):
    pack = orc.ll_pack if fmt == "ll" else orc.ll128_pack
    unpack = orc.ll_unpack_reduce if fmt == "ll" else orc.ll128_unpack_reduce
    size = 16 if fmt == "ll" else 128
    n, sl = 301, 64
    g = np.random.default_rng(3)
    x = g.integers(-100, 100, n).astype(np.float32)
    W = 4
    fifos = []
    for _ in range(W):
        f = np.zeros(8 * sl * size, np.uint8)
        pack(x, f, sl)
        fifos.append(f)
    out, valid, bad = unpack(fifos, n, sl)
    assert bad == 0 and np.array_equal(out, W * x)
    # FIFO order: (1, 2^24, 1, -2^24) sums to 0 in order 0..3 (see 1stage)
    vals = [1.0, 2.0 ** 24, 1.0, -(2.0 ** 24)]
    fifos = []
    for v in vals:
        f = np.zeros(8 * sl * size, np.uint8)
        pack(np.full(n, v, np.float32), f, sl)
        fifos.append(f)
    out, _, _ = unpack(fifos, n, sl)
    assert np.all(out == 0.0)
    out, _, _ = unpack(fifos[::-1], n, sl)
    assert np.all(out == 2.0)


@pytest.mark.parametrize("fmt", ["ll", "ll128"])
def test_decode_counts_planted_corruption(fmt):
    """[NCCL14]: a line is ready only when its flag(s) equal step + 1; LL needs
    both flags.  Bad (FIFO, line) pairs are counted exactly."""
    pack = orc.ll_pack if fmt == "ll" else orc.ll128_pack
    unpack = orc.ll_unpack_reduce if fmt == "ll" else orc.ll128_unpack_reduce
    nlines = orc.ll_lines if fmt == "ll" else orc.ll128_lines
    size = 16 if fmt == "ll" else 128
    per_line = 2 if fmt == "ll" else 30
    n, sl, W = 997, 80, 3
    L = nlines(n)
    assert L <= 8 * sl
    g = np.random.default_rng(4)
    fifos = []
    for _ in range(W):
        f = np.zeros(8 * sl * size, np.uint8)
        pack(g.standard_normal(n).astype(np.float32), f, sl, 1)
        fifos.append(f)
    # one flag word wrong in FIFO 1, line 5 (LL: flag2 only; flag1 stays right)
    bad_fifo = [f.copy() for f in fifos]
    wire5 = ((1 + 5 // sl) % 8) * sl + 5 % sl     # where logical line 5 sits
    if fmt == "ll":
        bad_fifo[1][wire5 * 16 + 12] ^= 0x01
    else:
        bad_fifo[1][wire5 * 128 + 120] ^= 0x01
    out, valid, bad = unpack(bad_fifo, n, sl, 1)
    assert bad == 1
    assert not valid[5 * per_line:6 * per_line].any()
    assert valid[:5 * per_line].all() and valid[6 * per_line:].all()
    # a stale round: expected flags one lap (8 steps) ahead -> all bad
    _, valid, bad = unpack(fifos, n, sl, 1 + 8)
    assert bad == W * L and not valid.any()
    # a zeroed FIFO never validates (flags are step + 1 >= 1)
    zeros = [np.zeros_like(f) for f in fifos]
    _, _, bad = unpack(zeros, n, sl, 0)
    assert bad == W * L


@pytest.mark.parametrize("fmt", ["ll", "ll128"])
@pytest.mark.parametrize("offset", [4, 8, 12])
def test_pack_from_unaligned_source_gives_same_wire(fmt, offset):
    pack = orc.ll_pack if fmt == "ll" else orc.ll128_pack
    size = 16 if fmt == "ll" else 128
    n, sl = 1013, 200
    g = np.random.default_rng(offset)
    x = g.standard_normal(n).astype(np.float32)
    raw = np.zeros(4 * n + 64, np.uint8)
    base = (-raw.ctypes.data) % 16
    view = raw[base + offset: base + offset + 4 * n].view(np.float32)
    view[:] = x
    assert view.ctypes.data % 16 == offset
    a = np.zeros(8 * sl * size, np.uint8)
    b = np.zeros(8 * sl * size, np.uint8)
    pack(x, a, sl)
    pack(view, b, sl)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# Lamport data-as-flag wire ([TRIAR] "Option 2: Lamport")
# ---------------------------------------------------------------------------
SENT = orc.LAMPORT_SENTINEL


@pytest.mark.parametrize("lo,hi,want", [
    (0x3F80, 0x4000, 0x40003F80),   # element 2j in the low half
    (0x8000, 0x3F80, 0x3F800000),   # -0.0 scrubbed to +0.0 (low)
    (0x3F80, 0x8000, 0x00003F80),   # -0.0 scrubbed to +0.0 (high)
    (0x8000, 0x8000, 0x00000000),   # two -0.0: not the sentinel
    (0x8001, 0xFF80, 0xFF808001),   # other negatives untouched
    (0x0000, 0x7FC0, 0x7FC00000),
])
def test_lamport_pack_hand_cases(lo, hi, want):
    assert orc.lamport_pack(lo, hi) == want


def test_lamport_pack_never_produces_the_sentinel():
    """Exhaustive over every bf16 paired with -0.0 on either side: only a
    -0.0/-0.0 pair could form 0x80008000, and scrubbing removes it."""
    v = np.arange(65536, dtype=np.uint16)
    for pair in (np.stack([v, np.full_like(v, 0x8000)], 1),
                 np.stack([np.full_like(v, 0x8000), v], 1)):
        x = pair.reshape(1, -1)
        comm = orc.lamport_comm(1, 1, x.shape[1])
        orc.lamport_push(x, 0, [comm], 0)
        words = comm[: x.shape[1] // 2]
        assert not np.any(words == SENT)
        lo, hi = (words & 0xFFFF).astype(np.uint16), (words >> 16).astype(np.uint16)
        want = np.where(pair == 0x8000, 0, pair).astype(np.uint16)
        assert np.array_equal(lo, want[:, 0]) and np.array_equal(hi, want[:, 1])


def test_lamport_regions_hand_example():
    """W=2, M=1, N=8: a slot is 4 words, a region 2 slots (8 words).  Flag 4
    uses region 4 % 3 = 1 (words 8..15: slot 0 at 8, slot 1 at 12) and the
    reader then resets region (4 + 2) % 3 = 0 (words 0..7)."""
    x0 = np.array([[0x3F80, 0x4000, 0x4040, 0x4080, 0x40A0, 0x40C0, 0x40E0, 0x4100]],
                  np.uint16)                                  # 1..8
    x1 = np.array([[0x3F80] * 8], np.uint16)                  # 1.0
    comms = [np.full(3 * 2 * 4, 0x11111111, np.uint32) for _ in range(2)]
    orc.lamport_push(x0, 0, comms, 4)
    orc.lamport_push(x1, 1, comms, 4)
    for c in comms:
        assert list(c[8:12]) == [0x40003F80, 0x40804040, 0x40C040A0, 0x410040E0]
        assert list(c[12:16]) == [0x3F803F80] * 4
        assert np.all(c[0:8] == 0x11111111) and np.all(c[16:24] == 0x11111111)
    res = np.zeros((1, 8), np.uint16)
    w = np.full(8, 0x3F80, np.uint16)
    ro, no, ne, bad = orc.lamport_fused_residual_rmsnorm(comms[0], 2, res, w, 1e-6, 4)
    assert bad == 0
    assert list(orc.bf16_to_f32(ro[0])) == [2, 3, 4, 5, 6, 7, 8, 9]
    assert np.all(comms[0][0:8] == SENT)                      # region 0 reset
    assert np.all(comms[0][16:24] == 0x11111111)              # region 2 untouched
    assert list(comms[0][12:16]) == [0x3F803F80] * 4          # region 1 kept


def test_lamport_fused_equals_the_fused_operator():
    """Without -0.0 inputs the Lamport path computes exactly the fused
    operator (already pinned above) on the pushed rows."""
    W, M, N, eps = 4, 16, 2048, 1e-6
    xs, res, w = synth.fused_inputs(W, M, N, [90])
    for x in xs:
        assert not np.any(x == 0x8000)
    comms = [orc.lamport_comm(W, M, N) for _ in range(W)]
    for r, x in enumerate(xs):
        orc.lamport_push(x, r, comms, 7)
    want = orc.fused_residual_rmsnorm(xs, res, w, eps)
    for p in range(W):
        ro, no, ne, bad = orc.lamport_fused_residual_rmsnorm(comms[p], W, res, w, eps, 7)
        assert bad == 0
        assert np.array_equal(ro, want[0]) and np.array_equal(no, want[1])
        assert np.array_equal(ne, want[2])


def test_lamport_scrub_changes_the_sign_of_an_all_negative_zero_sum():
    """All inputs and the residual -0.0: the fused operator gives -0.0 for
    residual_out, the Lamport path +0.0 (its inputs were scrubbed)."""
    W, M, N = 2, 1, 16
    xs = [np.full((M, N), 0x8000, np.uint16) for _ in range(W)]
    res = np.full((M, N), 0x8000, np.uint16)
    w = np.full(N, 0x3F80, np.uint16)
    assert np.all(orc.fused_residual_rmsnorm(xs, res, w, 1e-6)[0] == 0x8000)
    comms = [orc.lamport_comm(W, M, N) for _ in range(W)]
    for r, x in enumerate(xs):
        orc.lamport_push(x, r, comms, 0)
    ro, _, _, bad = orc.lamport_fused_residual_rmsnorm(comms[0], W, res, w, 1e-6, 0)
    assert bad == 0 and np.all(ro == 0x0000)


def test_lamport_counts_missing_pushes():
    W, M, N = 3, 2, 64
    xs, res, w = synth.fused_inputs(W, M, N, [91])
    comms = [orc.lamport_comm(W, M, N) for _ in range(W)]
    orc.lamport_push(xs[0], 0, comms, 2)        # rank 1 never pushes
    orc.lamport_push(xs[2], 2, comms, 2)
    *_, bad = orc.lamport_fused_residual_rmsnorm(comms[0], W, res, w, 1e-6, 2)
    assert bad == M * N // 8                    # every chunk of slot 1


def test_lamport_triple_buffer_invariant_over_calls():
    """Before the pushes of call f, region f % 3 of every buffer is all
    sentinel: it was reset by call f - 2 and untouched by call f - 1."""
    W, M, N = 3, 2, 32
    comms = [orc.lamport_comm(W, M, N) for _ in range(W)]
    words = M * N // 2
    for f in range(7):
        xs, res, w = synth.fused_inputs(W, M, N, [92, f])
        for c in comms:
            reg = c.reshape(3, W * words)[f % 3]
            assert np.all(reg == SENT), f
        for r, x in enumerate(xs):
            orc.lamport_push(x, r, comms, f)
        want = orc.fused_residual_rmsnorm(xs, res, w, 1e-6)
        for p in range(W):
            ro, no, _, bad = orc.lamport_fused_residual_rmsnorm(comms[p], W, res, w, 1e-6, f)
            assert bad == 0 and np.array_equal(ro, want[0]) and np.array_equal(no, want[1])


def test_lamport_flag_sequence_across_the_wrap():
    """[TRIAR] "Option 2: Lamport": region = flag % 3 and the flag grows by one
    per launch.  The counter wraps at 3 * 2^30, a multiple of 3, so the
    region sequence runs on across the wrap (2, 0, 1, 2, ...) and every
    call still finds its region all sentinel before its pushes.  A plain
    32-bit wrap would give region 0 twice in a row (2^32 - 1 = 0 mod 3)."""
    P = orc.LAMPORT_FLAG_PERIOD
    assert P == 3 << 30 and P % 3 == 0
    assert (2 ** 32 - 1) % 3 == 0 % 3          # the collision a 2^32 wrap has
    assert orc.lamport_next_flag(P - 1) == 0
    assert orc.lamport_next_flag(P - 2) == P - 1
    assert orc.lamport_next_flag(5) == 6
    W, M, N = 2, 1, 16
    words = M * N // 2
    comms = [orc.lamport_comm(W, M, N) for _ in range(W)]
    f = P - 4
    regions = []
    for call in range(8):
        xs, res, w = synth.fused_inputs(W, M, N, [93, call])
        regions.append(f % 3)
        for c in comms:
            assert np.all(c.reshape(3, W * words)[f % 3] == SENT), (call, f)
        for r, x in enumerate(xs):
            orc.lamport_push(x, r, comms, f)
        want = orc.fused_residual_rmsnorm(xs, res, w, 1e-6)
        for p in range(W):
            ro, no, _, bad = orc.lamport_fused_residual_rmsnorm(comms[p], W, res, w, 1e-6, f)
            assert bad == 0 and np.array_equal(ro, want[0]) and np.array_equal(no, want[1])
        f = orc.lamport_next_flag(f)
    assert regions == [2, 0, 1, 2, 0, 1, 2, 0]          # flags P-4 .. P-1, 0 .. 3


def test_lamport_flags_past_the_period_are_refused():
    """A flag at or above the period is not a valid counter value: the push
    writes nothing and the reader returns -1 without touching the buffer."""
    W, M, N = 2, 1, 8
    xs, res, w = synth.fused_inputs(W, M, N, [94])
    comm = orc.lamport_comm(W, M, N)
    before = comm.copy()
    lib = orc.lib()
    lib.orc_lamport_push(orc._ptr(np.ascontiguousarray(xs[0])), 1, 0,
                         orc._ptr_table([comm]), M, N, orc.LAMPORT_FLAG_PERIOD)
    assert np.array_equal(comm, before)
    ro = np.empty((M, N), np.uint16)
    no = np.empty((M, N), np.uint16)
    ne = np.empty((M, N), np.float64)
    got = lib.orc_lamport_fused_residual_rmsnorm(
        orc._ptr(comm), W, orc._ptr(np.ascontiguousarray(res)), orc._ptr(np.ascontiguousarray(w)),
        orc._ptr(ro), orc._ptr(no), orc._ptr(ne), M, N, 1e-6, 0xFFFFFFFF)
    assert got == -1 and np.array_equal(comm, before)
    with pytest.raises(ValueError):
        orc.lamport_push(xs[0], 0, [comm, comm.copy()], orc.LAMPORT_FLAG_PERIOD)


# ---------------------------------------------------------------------------
# two-shot fused (rows sharded as [SGLv1]'s two-stage form, [TRIAR] operator)
# ---------------------------------------------------------------------------
def test_fused_2stage_row_partition():
    assert orc.row_shard_range(128, 4, 0) == (0, 32)
    assert orc.row_shard_range(128, 4, 3) == (96, 128)
    assert orc.row_shard_range(4 * 10 + 3, 4, 2) == (20, 30)
    assert orc.row_shard_range(4 * 10 + 3, 4, 3) == (30, 43)
    assert orc.row_shard_range(3, 8, 0) == (0, 0)
    assert orc.row_shard_range(3, 8, 7) == (0, 3)


@pytest.mark.parametrize("W,M", [(2, 7), (2, 128), (4, 16), (8, 11), (3, 2)])
def test_fused_2stage_equals_one_shot_when_order_agrees(W, M):
    """W=2: the rotated order is x0+x1 or x1+x0, equal by commutativity; with
    the rank-order flag every W gives the one-shot fused result exactly."""
    N = 512
    xs, res, w = synth.fused_inputs(W, M, N, [97, W, M])
    one = orc.fused_residual_rmsnorm(xs, res, w, 1e-6)
    two = orc.fused_2stage(xs, res, w, 1e-6, rank_order=True)
    for a, b in zip(one, two):
        assert np.array_equal(a, b)
    if W == 2:
        rot = orc.fused_2stage(xs, res, w, 1e-6)
        for a, b in zip(one, rot):
            assert np.array_equal(a, b)


def test_fused_2stage_rotation_hand_case():
    """x = (1, 2^24, 1, -2^24) at every position, W=4, M=4 (one row per
    shard), residual 0, weight 1: the owners' sums are 0, 1, 2, 2 (as in the
    two-stage reduce), and the normalised rows are 0, 1, 1, 1."""
    M, N = 4, 64
    vals = [0x3F80, 0x4B80, 0x3F80, 0xCB80]
    xs = [np.full((M, N), v, np.uint16) for v in vals]
    res = np.zeros((M, N), np.uint16)
    w = np.full(N, 0x3F80, np.uint16)
    ro, no, _ = orc.fused_2stage(xs, res, w, 1e-6)
    assert list(orc.bf16_to_f32(ro[:, 0])) == [0.0, 1.0, 2.0, 2.0]
    assert list(orc.bf16_to_f32(no[:, 0])) == [0.0, 1.0, 1.0, 1.0]
    assert np.all(ro == ro[:, :1]) and np.all(no == no[:, :1])


def test_fused_2stage_staged_shards_are_the_gathered_rows():
    W, M, N = 4, 4 * 5 + 3, 256
    xs, res, w = synth.fused_inputs(W, M, N, [98])
    ro, no, ne = orc.fused_2stage(xs, res, w, 1e-6)
    for s in range(W):
        m0, m1 = orc.row_shard_range(M, W, s)
        sro, sno, sne = orc.fused_2stage_scatter(xs, s, res, w, 1e-6)
        assert np.array_equal(sro, ro[m0:m1]) and np.array_equal(sno, no[m0:m1])
        assert np.array_equal(sne, ne[m0:m1])


# ---------------------------------------------------------------------------
# streaming through the 8-step FIFO ([NCCL14] "prerequisite mental model")
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("proto,step", [(orc.PROTO_LL, 256), (orc.PROTO_LL128, 240),
                                        (orc.PROTO_SIMPLE, 256)])
def test_fifo_stream_delivers_the_payload(proto, step):
    g = np.random.default_rng(proto)
    src = g.standard_normal(1000 + proto).astype(np.float32)
    out, _ = orc.fifo_stream(proto, src, 3, step)
    assert np.array_equal(out.view(np.uint32), src.view(np.uint32))
    out, _ = orc.fifo_stream(proto, src, 3, step, local=src)
    assert np.array_equal(out, 2 * src)                      # doubling is exact


@pytest.mark.parametrize("first", [0, 5])
def test_fifo_stream_within_one_lap_is_the_packers(first):
    """One channel, at most 8 steps: the ring is exactly what the (pinned)
    LL / LL128 packers produce with step_lines = step_bytes / 8 or / 120."""
    g = np.random.default_rng(first)
    src = g.standard_normal(7 * 60 + 11).astype(np.float32)      # 1724 payload bytes
    _, ring = orc.fifo_stream(orc.PROTO_LL, src, 1, 256, first)
    want = np.zeros(8 * 32 * 16, np.uint8)
    orc.ll_pack(src, want, 32, first)
    assert np.array_equal(ring, want)
    _, ring = orc.fifo_stream(orc.PROTO_LL128, src, 1, 240, first)
    want = np.zeros(8 * 2 * 128, np.uint8)
    orc.ll128_pack(src, want, 2, first)
    assert np.array_equal(ring, want)


def test_fifo_stream_ring_keeps_the_last_lap():
    """13 steps of 256 payload bytes through one ring (the last one partial):
    the ring is the first lap (steps 0..7) overwritten by steps 8..12, each
    slot holding the latest step with its index mod 8, and slot 4 keeping
    step 4's lines past the end of the partial step 12."""
    g = np.random.default_rng(3)
    src = g.standard_normal(13 * 64 - 7).astype(np.float32)
    _, ring = orc.fifo_stream(orc.PROTO_LL, src, 1, 256)
    want = np.zeros(8 * 32 * 16, np.uint8)
    orc.ll_pack(src[:8 * 64], want, 32, 0)
    orc.ll_pack(src[8 * 64:], want, 32, 8)
    assert np.array_equal(ring, want)
    _, ring = orc.fifo_stream(orc.PROTO_SIMPLE, src, 1, 256)
    raw = src.view(np.uint8)
    for k in range(5, 13):
        part = raw[k * 256:(k + 1) * 256]            # the last step is partial
        assert np.array_equal(ring[(k % 8) * 256:(k % 8) * 256 + part.size], part)
    # past the partial step 12, slot 4 still holds step 4's bytes
    cut = raw.size - 12 * 256
    assert np.array_equal(ring[4 * 256 + cut:5 * 256], raw[4 * 256 + cut:5 * 256])


def test_fifo_stream_channel_split():
    """T = 10 steps over 4 channels: channel c takes steps [c*10/4, (c+1)*10/4)
    = [0,2), [2,5), [5,7), [7,10), each numbered from first_step in its ring."""
    step = 256
    src = np.arange(10 * 64, dtype=np.float32)
    _, ring = orc.fifo_stream(orc.PROTO_SIMPLE, src, 4, step, first_step=3)
    raw = src.view(np.uint8)
    for c, (s0, s1) in enumerate([(0, 2), (2, 5), (5, 7), (7, 10)]):
        base = c * 8 * step
        for j, gstep in enumerate(range(s0, s1)):
            slot = (3 + j) % 8
            assert np.array_equal(ring[base + slot * step: base + (slot + 1) * step],
                                  raw[gstep * step:(gstep + 1) * step]), (c, j)
    assert orc.fifo_total_steps(10 * 64, step) == 10
    assert orc.fifo_step_wire_bytes(orc.PROTO_LL, 32768) == 65536
    assert orc.fifo_step_wire_bytes(orc.PROTO_LL128, 576000) == 614400
