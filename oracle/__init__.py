"""Python face of the CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``ar_rmsnorm_amd``) never imports it, and this package never imports the
product path; the only module both sides use is the seeded input generator
``ar_rmsnorm_amd.synth``, which holds none of the method's arithmetic.

Every function here is a thin ctypes marshaller around one C routine of the
oracle, which cites the passage of the pages it follows.  Arrays are numpy:
bf16 tensors are carried as ``uint16`` bit patterns, fp32 as ``float32``, wire
FIFOs and raw payloads as ``uint8`` byte arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

# Strict IEEE binary32 on x86-64 SSE: no contraction into FMA, no fast-math.
CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
          "-fno-fast-math", "-fPIC", "-shared"]


def build() -> str:
    """Compile ``liboracle.so`` with gcc (always recompiles)."""
    cmd = ["gcc", *CFLAGS, "-o", LIB + ".tmp", SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64


def lib():
    """Load the oracle library, building it first if it is not there.  The
    environment variable ORACLE_LIB names another build of oracle.c to load
    instead (the sanitizer test uses it)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB", LIB)
        if path == LIB and not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(path)
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_bf16_rne.argtypes = [ctypes.c_float]
        L.orc_bf16_rne.restype = ctypes.c_uint16
        L.orc_bf16_from_f64.argtypes = [ctypes.c_double]
        L.orc_bf16_from_f64.restype = ctypes.c_uint16
        L.orc_bf16_rne_array.argtypes = [_p, _p, _i64]
        L.orc_bf16_from_f64_array.argtypes = [_p, _p, _i64]
        L.orc_reduce_1stage.argtypes = [_p, ctypes.c_int, _p, _i64]
        L.orc_shard_range.argtypes = [_i64, ctypes.c_int, ctypes.c_int,
                                      ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
        L.orc_reduce_scatter.argtypes = [_p, ctypes.c_int, ctypes.c_int, _p, _i64,
                                         ctypes.c_int]
        L.orc_all_gather.argtypes = [_p, ctypes.c_int, _p, _i64]
        L.orc_reduce_2stage.argtypes = [_p, ctypes.c_int, _p, _i64, ctypes.c_int]
        L.orc_reduce_2stage.restype = ctypes.c_int
        L.orc_fused_residual_rmsnorm.argtypes = [_p, ctypes.c_int, _p, _p, _p, _p,
                                                 _p, _i64, _i64, ctypes.c_double, _p]
        for name in ("orc_ll_lines", "orc_ll128_lines"):
            getattr(L, name).argtypes = [_i64]
            getattr(L, name).restype = _i64
        for name in ("orc_ll_pack", "orc_ll128_pack"):
            getattr(L, name).argtypes = [_p, _i64, _p, _i64, _u64]
        L.orc_row_shard_range.argtypes = [_i64, ctypes.c_int, ctypes.c_int,
                                          ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
        L.orc_fused_2stage_scatter.argtypes = [_p, ctypes.c_int, ctypes.c_int, _p, _p, _p, _p,
                                               _i64, _i64, ctypes.c_double, ctypes.c_int]
        L.orc_fused_2stage.argtypes = [_p, ctypes.c_int, _p, _p, _p, _p, _p, _i64, _i64,
                                       ctypes.c_double, ctypes.c_int]
        L.orc_fifo_step_wire_bytes.argtypes = [ctypes.c_int, _i64]
        L.orc_fifo_step_wire_bytes.restype = _i64
        L.orc_fifo_total_steps.argtypes = [_i64, _i64]
        L.orc_fifo_total_steps.restype = _i64
        L.orc_fifo_stream.argtypes = [ctypes.c_int, _p, _p, _p, _i64, _p, ctypes.c_int, _i64,
                                      _u64]
        L.orc_lamport_pack.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
        L.orc_lamport_pack.restype = ctypes.c_uint32
        L.orc_lamport_next_flag.argtypes = [ctypes.c_uint32]
        L.orc_lamport_next_flag.restype = ctypes.c_uint32
        L.orc_lamport_push.argtypes = [_p, ctypes.c_int, ctypes.c_int, _p, _i64, _i64,
                                       ctypes.c_uint32]
        L.orc_lamport_fused_residual_rmsnorm.argtypes = [_p, ctypes.c_int, _p, _p, _p, _p, _p,
                                                         _i64, _i64, ctypes.c_double,
                                                         ctypes.c_uint32]
        L.orc_lamport_fused_residual_rmsnorm.restype = _i64
        for name in ("orc_ll_unpack_reduce", "orc_ll128_unpack_reduce"):
            getattr(L, name).argtypes = [_p, ctypes.c_int, _p, _p, _i64, _i64, _u64]
            getattr(L, name).restype = _i64
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _ptr_table(arrays) -> ctypes.Array:
    return (ctypes.c_void_p * len(arrays))(*[_ptr(a) for a in arrays])


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


# --------------------------------------------------------------------------
# bf16 <-> fp32
# --------------------------------------------------------------------------
def bf16_to_f32(b) -> np.ndarray:
    """Exact widening: the bf16 bits become the top half of an fp32."""
    b = _u16(b)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_rne(x) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (oracle C routine)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_bf16_rne_array(_ptr(x), _ptr(out), x.size)
    return out


def bf16_from_f64(x) -> np.ndarray:
    """float64 -> bf16 bits, rounded once to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().orc_bf16_from_f64_array(_ptr(x), _ptr(out), x.size)
    return out


# --------------------------------------------------------------------------
# reduce forms
# --------------------------------------------------------------------------
def reduce_1stage(xs) -> np.ndarray:
    xs = [_u16(x).reshape(-1) for x in xs]
    n = xs[0].size
    out = np.empty(n, np.uint16)
    lib().orc_reduce_1stage(_ptr_table(xs), len(xs), _ptr(out), n)
    return out


def shard_range(n: int, W: int, s: int):
    """Pack range [first, last) owned by shard s."""
    a, b = _i64(), _i64()
    lib().orc_shard_range(n, W, s, ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def reduce_scatter(xs, s: int, rank_order: bool = False) -> np.ndarray:
    xs = [_u16(x).reshape(-1) for x in xs]
    n, W = xs[0].size, len(xs)
    p0, p1 = shard_range(n, W, s)
    tmp = np.empty((p1 - p0) * 8, np.uint16)
    lib().orc_reduce_scatter(_ptr_table(xs), W, s, _ptr(tmp), n, int(rank_order))
    return tmp


def all_gather(tmps, n: int) -> np.ndarray:
    tmps = [_u16(t).reshape(-1) for t in tmps]
    out = np.empty(n, np.uint16)
    lib().orc_all_gather(_ptr_table(tmps), len(tmps), _ptr(out), n)
    return out


def reduce_2stage(xs, rank_order: bool = False) -> np.ndarray:
    xs = [_u16(x).reshape(-1) for x in xs]
    n = xs[0].size
    out = np.empty(n, np.uint16)
    rc = lib().orc_reduce_2stage(_ptr_table(xs), len(xs), _ptr(out), n, int(rank_order))
    if rc != 0:
        raise MemoryError("oracle two-stage staging allocation failed")
    return out


def fused_residual_rmsnorm(xs, residual, weight, eps: float):
    """Returns (residual_out bf16, norm_out bf16, norm_exact float64)."""
    residual = _u16(residual)
    M, N = residual.shape
    xs = [_u16(x).reshape(M, N) for x in xs]
    weight = _u16(weight).reshape(N)
    res_out = np.empty((M, N), np.uint16)
    norm_out = np.empty((M, N), np.uint16)
    norm_exact = np.empty((M, N), np.float64)
    h = np.empty(N, np.float32)
    lib().orc_fused_residual_rmsnorm(_ptr_table(xs), len(xs), _ptr(residual), _ptr(weight),
                                     _ptr(res_out), _ptr(norm_out), _ptr(norm_exact),
                                     M, N, float(eps), _ptr(h))
    return res_out, norm_out, norm_exact


def row_shard_range(M: int, W: int, s: int):
    """Row range [first, last) owned by shard s of the two-shot fused form."""
    a, b = _i64(), _i64()
    lib().orc_row_shard_range(M, W, s, ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def fused_2stage_scatter(xs, s: int, residual, weight, eps: float, rank_order: bool = False):
    """Owner s's staged rows: (residual_out rows, norm_out rows, norm_exact)."""
    residual = _u16(residual)
    M, N = residual.shape
    xs = [_u16(x).reshape(M, N) for x in xs]
    weight = _u16(weight).reshape(N)
    m0, m1 = row_shard_range(M, len(xs), s)
    rows = m1 - m0
    stage = np.empty(2 * rows * N + 1, np.uint16)
    exact = np.empty(rows * N + 1, np.float64)
    lib().orc_fused_2stage_scatter(_ptr_table(xs), len(xs), s, _ptr(residual), _ptr(weight),
                                   _ptr(stage), _ptr(exact), M, N, float(eps), int(rank_order))
    return (stage[:rows * N].reshape(rows, N), stage[rows * N:2 * rows * N].reshape(rows, N),
            exact[:rows * N].reshape(rows, N))


def fused_2stage(xs, residual, weight, eps: float, rank_order: bool = False):
    """Two-shot fused result: (residual_out, norm_out, norm_exact)."""
    residual = _u16(residual)
    M, N = residual.shape
    xs = [_u16(x).reshape(M, N) for x in xs]
    weight = _u16(weight).reshape(N)
    ro = np.empty((M, N), np.uint16)
    no = np.empty((M, N), np.uint16)
    ne = np.empty((M, N), np.float64)
    lib().orc_fused_2stage(_ptr_table(xs), len(xs), _ptr(residual), _ptr(weight), _ptr(ro),
                           _ptr(no), _ptr(ne), M, N, float(eps), int(rank_order))
    return ro, no, ne


# --------------------------------------------------------------------------
# LL / LL128 wire formats
# --------------------------------------------------------------------------
def ll_lines(n: int) -> int:
    return lib().orc_ll_lines(n)


def ll128_lines(n: int) -> int:
    return lib().orc_ll128_lines(n)


def _payload_bytes(src) -> np.ndarray:
    src = np.ascontiguousarray(src)
    return src.view(np.uint8).reshape(-1)


def _check_fifo(fifo: np.ndarray, lines: int, step_lines: int, line_bytes: int):
    assert fifo.dtype == np.uint8 and fifo.flags.c_contiguous
    if lines > 8 * step_lines:
        raise ValueError("one call spans at most 8 steps of step_lines lines")
    if fifo.size < 8 * step_lines * line_bytes:
        raise ValueError("FIFO smaller than 8 steps")


def ll_pack(src, fifo: np.ndarray, step_lines: int, first_step: int = 0) -> None:
    """Encode fp32 ``src`` into the uint8 ``fifo`` in place."""
    b = _payload_bytes(src)
    _check_fifo(fifo, ll_lines(b.size // 4), step_lines, 16)
    lib().orc_ll_pack(_ptr(b), b.size // 4, _ptr(fifo), step_lines, first_step)


def ll128_pack(src, fifo: np.ndarray, step_lines: int, first_step: int = 0) -> None:
    b = _payload_bytes(src)
    _check_fifo(fifo, ll128_lines(b.size // 4), step_lines, 128)
    lib().orc_ll128_pack(_ptr(b), b.size // 4, _ptr(fifo), step_lines, first_step)


def _unpack(fn, fifos, n, step_lines, first_step):
    fifos = [np.ascontiguousarray(f, dtype=np.uint8) for f in fifos]
    out = np.empty(n, np.float32)
    valid = np.empty(n, np.uint8)
    bad = fn(_ptr_table(fifos), len(fifos), _ptr(out), _ptr(valid), n, step_lines,
             first_step)
    return out, valid.astype(bool), int(bad)


def ll_unpack_reduce(fifos, n: int, step_lines: int, first_step: int = 0):
    """Returns (out fp32, valid mask, bad (FIFO, line) count)."""
    return _unpack(lib().orc_ll_unpack_reduce, fifos, n, step_lines, first_step)


def ll128_unpack_reduce(fifos, n: int, step_lines: int, first_step: int = 0):
    return _unpack(lib().orc_ll128_unpack_reduce, fifos, n, step_lines, first_step)


# --------------------------------------------------------------------------
# Lamport data-as-flag wire for the fused one-shot
# --------------------------------------------------------------------------
LAMPORT_SENTINEL = 0x80008000
LAMPORT_FLAG_PERIOD = 0xC0000000      # 3 * 2^30: the 32-bit flag wraps here


def lamport_next_flag(flag: int) -> int:
    return int(lib().orc_lamport_next_flag(flag))


def lamport_comm(W: int, M: int, N: int) -> np.ndarray:
    """A comm buffer of one rank, filled with the sentinel: u32 words
    [3 regions][W slots][M][N / 2]."""
    return np.full(3 * W * M * N // 2, LAMPORT_SENTINEL, np.uint32)


def lamport_pack(lo: int, hi: int) -> int:
    return int(lib().orc_lamport_pack(lo, hi))


def lamport_push(x, rank: int, comms, flag: int) -> None:
    """Rank `rank` pushes bf16 [M, N] x into the comm buffers of all W ranks
    (in place); `comms` lists those W buffers, so W = len(comms)."""
    x = _u16(x)
    M, N = x.shape
    for c in comms:
        assert c.dtype == np.uint32 and c.flags.c_contiguous
    if not 0 <= flag < LAMPORT_FLAG_PERIOD:
        raise ValueError(f"Lamport flag {flag} outside [0, 3 * 2^30)")
    lib().orc_lamport_push(_ptr(x), len(comms), rank, _ptr_table(comms), M, N, flag)


def lamport_fused_residual_rmsnorm(comm, W: int, residual, weight, eps: float, flag: int):
    """Reader side for one rank; returns (residual_out, norm_out, norm_exact,
    bad_chunks).  Resets region (flag % 3 + 2) % 3 of `comm` in place."""
    if not 0 <= flag < LAMPORT_FLAG_PERIOD:
        raise ValueError(f"Lamport flag {flag} outside [0, 3 * 2^30)")
    residual = _u16(residual)
    M, N = residual.shape
    weight = _u16(weight).reshape(N)
    assert comm.dtype == np.uint32 and comm.flags.c_contiguous
    res_out = np.empty((M, N), np.uint16)
    norm_out = np.empty((M, N), np.uint16)
    norm_exact = np.empty((M, N), np.float64)
    bad = lib().orc_lamport_fused_residual_rmsnorm(
        _ptr(comm), W, _ptr(residual), _ptr(weight), _ptr(res_out), _ptr(norm_out),
        _ptr(norm_exact), M, N, float(eps), flag)
    return res_out, norm_out, norm_exact, int(bad)


# --------------------------------------------------------------------------
# streaming through an 8-step FIFO (LL = 0, LL128 = 1, Simple = 2)
# --------------------------------------------------------------------------
PROTO_LL, PROTO_LL128, PROTO_SIMPLE = 0, 1, 2


def fifo_step_wire_bytes(proto: int, step_bytes: int) -> int:
    return lib().orc_fifo_step_wire_bytes(proto, step_bytes)


def fifo_total_steps(n: int, step_bytes: int) -> int:
    return lib().orc_fifo_total_steps(n, step_bytes)


def fifo_stream(proto: int, src, channels: int, step_bytes: int, first_step: int = 0,
                local=None, fifo=None):
    """Returns (out, fifo): the delivered payload and the rings' final bytes
    (written over `fifo` if given, else over a zeroed buffer)."""
    src = np.ascontiguousarray(src, dtype=np.float32)
    n = src.size
    wire = fifo_step_wire_bytes(proto, step_bytes)
    if fifo is None:
        fifo = np.zeros(channels * 8 * wire, np.uint8)
    assert fifo.dtype == np.uint8 and fifo.size >= channels * 8 * wire
    out = np.empty(n, np.float32)
    loc = None if local is None else np.ascontiguousarray(local, dtype=np.float32)
    lib().orc_fifo_stream(proto, _ptr(src), None if loc is None else _ptr(loc), _ptr(out), n,
                          _ptr(fifo), channels, step_bytes, first_step)
    return out, fifo
