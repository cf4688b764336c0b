"""ctypes binding of libar (include/libar.h), same names as the C ABI.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libar.so``.  Tensors are torch device tensors (torch supplies
device memory and streams); bf16 tensors are ``torch.bfloat16`` or raw
``torch.int16``/``torch.uint16`` bit patterns.  Each call enqueues on
``stream`` (default: torch's current stream) and returns without waiting.
A non-zero status raises ``ArError``.

Before each call the binding checks what the C ABI cannot: every buffer is a
contiguous tensor on a GPU, of the element size the header gives (2 bytes
for bf16, 4 for fp32) and at least the byte extent the call touches.  A
failed check raises ``ArError`` with ``AR_ERR_ARG`` and nothing is enqueued.
Raw integer addresses are refused, since nothing would keep their memory
alive.  ``checks_disabled()`` turns the checks off (and admits integer
addresses) for tests of the C ABI's own validation that use fake addresses.

Importing this module loads ``libar.so`` and fails loudly if it was not
built (``python -m ar_rmsnorm_amd.build``): there is no fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Sequence

import torch

from .build import LIB

if not os.path.exists(LIB):
    raise ImportError(f"libar.so not built at {LIB}; run `python -m ar_rmsnorm_amd.build`")

_lib = ctypes.CDLL(LIB)

AR_OK, AR_ERR_NULL, AR_ERR_ARG, AR_ERR_ALIGN, AR_ERR_WORLD, AR_ERR_CAPACITY, AR_ERR_HIP = range(7)
AR_STAGE_RS, AR_STAGE_AG, AR_ORDER_RANK = 1, 2, 4
AR_MAX_WORLD, AR_FUSED_MAX_N, AR_MAX_SPINS, AR_FIFO_STEPS = 8, 16384, 65536, 8
AR_LAMPORT_FLAG_PERIOD = 0xC0000000
AR_SCRATCH_BYTES = (8 << 20) + 4096

EXPORTS = (
    "ar_status_str", "ar_last_hip_error", "ar_reduce_1stage", "ar_reduce_2stage",
    "ar_fused_residual_rmsnorm", "ar_fused_residual_rmsnorm_2stage", "ar_lamport_comm_bytes", "ar_lamport_fill",
    "ar_lamport_push", "ar_lamport_fused_residual_rmsnorm",
    "ar_lamport_oneshot_residual_rmsnorm", "ll_pack", "ll_unpack_reduce", "ll128_pack",
    "ll128_unpack_reduce", "ll_lines", "ll128_lines", "ll_fifo_bytes",
    "ll128_fifo_bytes", "ll_default_step_lines", "ll128_default_step_lines",
    "ar_fifo_stream", "ar_fifo_step_wire_bytes", "ar_fifo_steps_per_channel", "ar_fifo_plan",
    "ar_fifo_counter_words", "ar_lamport_next_flag", "ar_fused_prefers_two_shot", "ar_copy",
    "ar_reduce_2stage_noalloc", "ar_lamport_all_ranks_residual_rmsnorm",
)
AR_PROTO_LL, AR_PROTO_LL128, AR_PROTO_SIMPLE = 0, 1, 2
AR_FIFO_MAX_CHANNELS = 256
AR_FIFO_MAX_PAIRS = 8
AR_FIFO_CONTINUE = (1 << 64) - 1

_vp, _i64, _u64, _u32, _int = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                               ctypes.c_uint32, ctypes.c_int)
_pp = ctypes.POINTER(ctypes.c_void_p)

_lib.ar_status_str.argtypes = [_int]
_lib.ar_status_str.restype = ctypes.c_char_p
_lib.ar_last_hip_error.argtypes = []
_lib.ar_last_hip_error.restype = _int
_lib.ar_reduce_1stage.argtypes = [_pp, _int, _vp, _i64, _vp]
_lib.ar_reduce_2stage.argtypes = [_pp, _pp, _int, _int, _vp, _i64, ctypes.c_uint, _vp]
_lib.ar_reduce_2stage_noalloc.argtypes = [_pp, _int, _int, _vp, _i64, ctypes.c_uint, _vp]
_lib.ar_reduce_2stage_noalloc.restype = _int
_lib.ar_fused_residual_rmsnorm.argtypes = [_pp, _int, _vp, _vp, _vp, _vp, _i64, _i64,
                                           ctypes.c_float, _vp]
_lib.ar_fused_residual_rmsnorm_2stage.argtypes = [_pp, _pp, _int, _int, _vp, _vp, _vp, _vp,
                                                  _i64, _i64, ctypes.c_float, ctypes.c_uint,
                                                  _vp]
_lib.ar_lamport_comm_bytes.argtypes = [_int, _i64, _i64]
_lib.ar_lamport_comm_bytes.restype = _i64
_lib.ar_lamport_next_flag.argtypes = [_u32]
_lib.ar_lamport_next_flag.restype = _u32
_lib.ar_fused_prefers_two_shot.argtypes = [_int, _i64, _i64]
_lib.ar_fused_prefers_two_shot.restype = _int
_lib.ar_copy.argtypes = [_vp, _vp, _i64, _vp]
_lib.ar_copy.restype = _int
_lib.ar_lamport_fill.argtypes = [_vp, _int, _i64, _i64, _vp]
_lib.ar_lamport_push.argtypes = [_vp, _int, _int, _pp, _i64, _i64, _u32, _vp]
_lib.ar_lamport_fused_residual_rmsnorm.argtypes = [_vp, _int, _vp, _vp, _vp, _vp, _i64, _i64,
                                                   ctypes.c_float, _u32, _u32, _vp, _vp]
_lib.ar_lamport_oneshot_residual_rmsnorm.argtypes = [_vp, _int, _pp, _int, _vp, _vp, _vp, _vp,
                                                     _i64, _i64, ctypes.c_float, _u32, _u32,
                                                     _vp, _vp]
_lib.ar_lamport_all_ranks_residual_rmsnorm.argtypes = [_pp, _pp, _int, _vp, _vp, _pp, _pp, _i64,
                                                       _i64, ctypes.c_float, _u32, _u32, _vp,
                                                       _vp]
_lib.ar_lamport_all_ranks_residual_rmsnorm.restype = _int
for _n in ("ll_pack", "ll128_pack"):
    getattr(_lib, _n).argtypes = [_vp, _i64, _vp, _i64, _u64, _vp]
for _n in ("ll_unpack_reduce", "ll128_unpack_reduce"):
    getattr(_lib, _n).argtypes = [_pp, _int, _vp, _i64, _i64, _u64, _u32, _vp, _vp]
for _n in ("ar_reduce_1stage", "ar_reduce_2stage", "ar_fused_residual_rmsnorm",
           "ar_fused_residual_rmsnorm_2stage",
           "ar_lamport_fill", "ar_lamport_push", "ar_lamport_fused_residual_rmsnorm",
           "ar_lamport_oneshot_residual_rmsnorm", "ll_pack",
           "ll128_pack", "ll_unpack_reduce", "ll128_unpack_reduce"):
    getattr(_lib, _n).restype = _int
for _n in ("ll_lines", "ll128_lines", "ll_fifo_bytes", "ll128_fifo_bytes"):
    getattr(_lib, _n).argtypes = [_i64]
    getattr(_lib, _n).restype = _i64
for _n in ("ll_default_step_lines", "ll128_default_step_lines"):
    getattr(_lib, _n).argtypes = []
    getattr(_lib, _n).restype = _i64


_lib.ar_fifo_stream.argtypes = [_int, _vp, _vp, _vp, _i64, _vp, _vp, _int, _i64, _u64, _u32,
                                _vp, _vp]
_lib.ar_fifo_stream.restype = _int
_lib.ar_fifo_step_wire_bytes.argtypes = [_int, _i64]
_lib.ar_fifo_step_wire_bytes.restype = _i64
_lib.ar_fifo_steps_per_channel.argtypes = [_i64, _i64, _int]
_lib.ar_fifo_steps_per_channel.restype = _i64
_pint = ctypes.POINTER(ctypes.c_int)
_lib.ar_fifo_plan.argtypes = [_int, _i64, _int, _i64, _int, _pint, _pint, _pint]
_lib.ar_fifo_plan.restype = _int
_lib.ar_fifo_counter_words.argtypes = [_int]
_lib.ar_fifo_counter_words.restype = _i64


class ArError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        msg = _lib.ar_status_str(status).decode()
        if status == AR_ERR_HIP:
            msg += f" (hipError_t {_lib.ar_last_hip_error()})"
        if detail:
            msg += f" ({detail})"
        super().__init__(f"{where}: status {status}: {msg}")


def _check(status: int, where: str) -> None:
    if status != AR_OK:
        raise ArError(status, where)


_checks = True


@contextlib.contextmanager
def checks_disabled():
    """Skip the binding's buffer checks and admit integer addresses (for tests
    of the C ABI's own argument validation with fake, never used addresses)."""
    global _checks
    saved, _checks = _checks, False
    try:
        yield
    finally:
        _checks = saved


BF16, F32, U32, ANY = 2, 4, 4, 0   # element sizes a buffer argument must have (0: any)


def _addr(x, nbytes: int = 0, esize: int = ANY, what: str = "buffer",
          where: str = "libar") -> Optional[int]:
    """Device address of tensor x (None for NULL), after checking that x is a
    contiguous GPU tensor of element size `esize` holding >= nbytes bytes."""
    if x is None:
        return None
    if not _checks:
        return x if isinstance(x, int) else x.data_ptr()
    if not isinstance(x, torch.Tensor):
        raise ArError(AR_ERR_ARG, where, f"{what} must be a torch tensor, not {type(x).__name__}")
    if not x.is_cuda:
        raise ArError(AR_ERR_ARG, where, f"{what} is not on a GPU")
    if not x.is_contiguous():
        raise ArError(AR_ERR_ARG, where, f"{what} is not contiguous")
    if esize and x.element_size() != esize:
        raise ArError(AR_ERR_ARG, where,
                      f"{what} has {x.element_size()}-byte elements, {esize} expected")
    have = x.numel() * x.element_size()
    if have < nbytes:
        raise ArError(AR_ERR_ARG, where, f"{what} holds {have} bytes, the call touches {nbytes}")
    return x.data_ptr()


def _table(xs, nbytes: int = 0, esize: int = ANY, what: str = "buffer",
           where: str = "libar") -> ctypes.Array:
    return (ctypes.c_void_p * len(xs))(*[_addr(x, nbytes, esize, f"{what}[{i}]", where)
                                         for i, x in enumerate(xs)])


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _numel(x, n: Optional[int]) -> int:
    return x.numel() if n is None else n


# ---------------------------------------------------------------------------
def ar_reduce_1stage(inputs: Sequence, out, n: Optional[int] = None, stream=None) -> None:
    """out = bf16(sum in fp32 of the W inputs, rank order 0..W-1)."""
    w = "ar_reduce_1stage"
    n = _numel(inputs[0], n)
    _check(_lib.ar_reduce_1stage(_table(inputs, 2 * n, BF16, "inputs", w), len(inputs),
                                 _addr(out, 2 * n, BF16, "out", w), n, _stream(stream)), w)


def ar_reduce_2stage(inputs: Sequence, tmps: Sequence, rank: int, out,
                     flags: int = 0, n: Optional[int] = None, stream=None) -> None:
    """Reduce-scatter of this rank's shard into tmps[rank], then all-gather
    of all W shards into out (flags select the stages and the order)."""
    w = "ar_reduce_2stage"
    n = _numel(inputs[0], n)
    P, W = n // 8, max(len(inputs), 1)
    tmp_bytes = (P // W + P % W) * 16
    _check(_lib.ar_reduce_2stage(_table(inputs, 2 * n, BF16, "inputs", w),
                                 _table(tmps, tmp_bytes, BF16, "tmps", w), len(inputs), rank,
                                 _addr(out, 2 * n, BF16, "out", w), n, flags, _stream(stream)),
           w)


def ar_reduce_2stage_noalloc(inputs: Sequence, rank: int, out, flags: int = 0,
                             n: Optional[int] = None, stream=None) -> None:
    """ar_reduce_2stage with the staging shards in the library's own device
    array (AR_SCRATCH_BYTES per GPU): nothing is allocated.  Calls on one
    GPU share that array, so they must not overlap in time."""
    w = "ar_reduce_2stage_noalloc"
    n = _numel(inputs[0], n)
    _check(_lib.ar_reduce_2stage_noalloc(_table(inputs, 2 * n, BF16, "inputs", w), len(inputs),
                                         rank, _addr(out, 2 * n, BF16, "out", w), n, flags,
                                         _stream(stream)), w)


def ar_fused_residual_rmsnorm(inputs: Sequence, residual, weight, residual_out, norm_out,
                              eps: float, M: Optional[int] = None, N: Optional[int] = None,
                              stream=None) -> None:
    """residual_out = sum(inputs) + residual; norm_out = RMSNorm(residual_out)."""
    w = "ar_fused_residual_rmsnorm"
    if M is None or N is None:
        M, N = residual.shape
    mat = 2 * M * N
    _check(_lib.ar_fused_residual_rmsnorm(_table(inputs, mat, BF16, "inputs", w), len(inputs),
                                          _addr(residual, mat, BF16, "residual", w),
                                          _addr(weight, 2 * N, BF16, "weight", w),
                                          _addr(residual_out, mat, BF16, "residual_out", w),
                                          _addr(norm_out, mat, BF16, "norm_out", w), M, N,
                                          float(eps), _stream(stream)), w)


def ar_fused_residual_rmsnorm_2stage(inputs: Sequence, tmps: Sequence, rank: int, residual,
                                     weight, residual_out, norm_out, eps: float,
                                     flags: int = 0, M: Optional[int] = None,
                                     N: Optional[int] = None, stream=None) -> None:
    """Two-shot fused form for one rank: the fused operator on this rank's
    row shard (staged in tmps[rank]), then the gather of every shard."""
    w = "ar_fused_residual_rmsnorm_2stage"
    if M is None or N is None:
        M, N = residual.shape
    mat, W = 2 * M * N, max(len(inputs), 1)
    tmp_bytes = 2 * (M // W + M % W) * N * 2
    _check(_lib.ar_fused_residual_rmsnorm_2stage(
        _table(inputs, mat, BF16, "inputs", w), _table(tmps, tmp_bytes, BF16, "tmps", w),
        len(inputs), rank, _addr(residual, mat, BF16, "residual", w),
        _addr(weight, 2 * N, BF16, "weight", w),
        _addr(residual_out, mat, BF16, "residual_out", w),
        _addr(norm_out, mat, BF16, "norm_out", w), M, N, float(eps), flags, _stream(stream)), w)


def ar_fused_prefers_two_shot(W: int, M: int, N: int) -> int:
    """1 if the two-shot fused call is the faster form for this shape on one
    GPU, 0 if the one-shot call is, -1 for invalid arguments."""
    return _lib.ar_fused_prefers_two_shot(W, M, N)


def ar_lamport_comm_bytes(W: int, M: int, N: int) -> int:
    return _lib.ar_lamport_comm_bytes(W, M, N)


def ar_lamport_next_flag(flag: int) -> int:
    """The flag of the next call: (flag + 1) mod AR_LAMPORT_FLAG_PERIOD."""
    return _lib.ar_lamport_next_flag(_flag(flag, "ar_lamport_next_flag"))


def _flag(flag: int, where: str) -> int:
    # the C ABI takes a uint32; a Python int outside it would be truncated
    if not 0 <= flag <= 0xFFFFFFFF:
        raise ArError(AR_ERR_ARG, where, f"flag {flag} does not fit 32 bits")
    return flag


def ar_lamport_fill(comm, W: int, M: int, N: int, stream=None) -> None:
    """Fill a comm buffer with the sentinel (all three regions)."""
    w = "ar_lamport_fill"
    _check(_lib.ar_lamport_fill(_addr(comm, _lib.ar_lamport_comm_bytes(W, M, N), ANY, "comm", w),
                                W, M, N, _stream(stream)), w)


def ar_lamport_push(x, rank: int, comms: Sequence, flag: int, M: Optional[int] = None,
                    N: Optional[int] = None, stream=None) -> None:
    """Push bf16 [M, N] rows of `rank` into slot `rank` of region flag % 3 of
    the W comm buffers (W = len(comms))."""
    w = "ar_lamport_push"
    if M is None or N is None:
        M, N = x.shape
    cb = _lib.ar_lamport_comm_bytes(len(comms), M, N)
    _check(_lib.ar_lamport_push(_addr(x, 2 * M * N, BF16, "x", w), len(comms), rank,
                                _table(comms, cb, ANY, "comms", w), M, N, _flag(flag, w),
                                _stream(stream)), w)


def ar_lamport_fused_residual_rmsnorm(comm, W: int, residual, weight, residual_out,
                                      norm_out, eps: float, flag: int, max_spins: int = 0,
                                      bad_chunks=None, M: Optional[int] = None,
                                      N: Optional[int] = None, stream=None) -> None:
    """Reduce the W slots of region flag % 3 of `comm`, add the residual,
    normalise; then reset the previous call's region to the sentinel."""
    w = "ar_lamport_fused_residual_rmsnorm"
    if M is None or N is None:
        M, N = residual.shape
    mat = 2 * M * N
    _check(_lib.ar_lamport_fused_residual_rmsnorm(
        _addr(comm, _lib.ar_lamport_comm_bytes(W, M, N), ANY, "comm", w), W,
        _addr(residual, mat, BF16, "residual", w), _addr(weight, 2 * N, BF16, "weight", w),
        _addr(residual_out, mat, BF16, "residual_out", w),
        _addr(norm_out, mat, BF16, "norm_out", w), M, N, float(eps), _flag(flag, w), max_spins,
        _addr(bad_chunks, 4, U32, "bad_chunks", w), _stream(stream)), w)


def ar_lamport_oneshot_residual_rmsnorm(x, rank: int, comms: Sequence, residual, weight,
                                        residual_out, norm_out, eps: float, flag: int,
                                        max_spins: int = 0, bad_chunks=None,
                                        M: Optional[int] = None, N: Optional[int] = None,
                                        stream=None) -> None:
    """One launch: push x as `rank` into the W comm buffers, then reduce
    comms[rank], add the residual and normalise (W = len(comms))."""
    w = "ar_lamport_oneshot_residual_rmsnorm"
    if M is None or N is None:
        M, N = residual.shape
    mat = 2 * M * N
    cb = _lib.ar_lamport_comm_bytes(len(comms), M, N)
    _check(_lib.ar_lamport_oneshot_residual_rmsnorm(
        _addr(x, mat, BF16, "x", w), rank, _table(comms, cb, ANY, "comms", w), len(comms),
        _addr(residual, mat, BF16, "residual", w), _addr(weight, 2 * N, BF16, "weight", w),
        _addr(residual_out, mat, BF16, "residual_out", w),
        _addr(norm_out, mat, BF16, "norm_out", w), M, N, float(eps), _flag(flag, w), max_spins,
        _addr(bad_chunks, 4, U32, "bad_chunks", w), _stream(stream)), w)


def ar_lamport_all_ranks_residual_rmsnorm(xs: Sequence, comms: Sequence, residual, weight,
                                          residual_outs: Sequence, norm_outs: Sequence,
                                          eps: float, flag: int, max_spins: int = AR_MAX_SPINS,
                                          bad_chunks=None, M: Optional[int] = None,
                                          N: Optional[int] = None, stream=None) -> None:
    """Every rank's one-launch Lamport call in one launch (W = len(xs)):
    rank r pushes xs[r] and reads comms[r] into residual_outs[r], norm_outs[r]."""
    w = "ar_lamport_all_ranks_residual_rmsnorm"
    if M is None or N is None:
        M, N = residual.shape
    mat = 2 * M * N
    cb = _lib.ar_lamport_comm_bytes(len(xs), M, N)
    _check(_lib.ar_lamport_all_ranks_residual_rmsnorm(
        _table(xs, mat, BF16, "xs", w), _table(comms, cb, ANY, "comms", w), len(xs),
        _addr(residual, mat, BF16, "residual", w), _addr(weight, 2 * N, BF16, "weight", w),
        _table(residual_outs, mat, BF16, "residual_outs", w),
        _table(norm_outs, mat, BF16, "norm_outs", w), M, N, float(eps), _flag(flag, w),
        max_spins, _addr(bad_chunks, 4, U32, "bad_chunks", w), _stream(stream)), w)


def ll_pack(src, fifo, step_lines: int, first_step: int = 0, n: Optional[int] = None,
            stream=None) -> None:
    w = "ll_pack"
    n = _numel(src, n)
    _check(_lib.ll_pack(_addr(src, 4 * n, F32, "src", w), n,
                        _addr(fifo, _lib.ll_fifo_bytes(step_lines), ANY, "fifo", w),
                        step_lines, first_step, _stream(stream)), w)


def ll128_pack(src, fifo, step_lines: int, first_step: int = 0, n: Optional[int] = None,
               stream=None) -> None:
    w = "ll128_pack"
    n = _numel(src, n)
    _check(_lib.ll128_pack(_addr(src, 4 * n, F32, "src", w), n,
                           _addr(fifo, _lib.ll128_fifo_bytes(step_lines), ANY, "fifo", w),
                           step_lines, first_step, _stream(stream)), w)


def ll_unpack_reduce(fifos: Sequence, out, step_lines: int, first_step: int = 0,
                     max_spins: int = 0, bad_lines=None, n: Optional[int] = None,
                     stream=None) -> None:
    w = "ll_unpack_reduce"
    n = _numel(out, n)
    _check(_lib.ll_unpack_reduce(_table(fifos, _lib.ll_fifo_bytes(step_lines), ANY, "fifos", w),
                                 len(fifos), _addr(out, 4 * n, F32, "out", w), n, step_lines,
                                 first_step, max_spins, _addr(bad_lines, 4, U32, "bad_lines", w),
                                 _stream(stream)), w)


def ll128_unpack_reduce(fifos: Sequence, out, step_lines: int, first_step: int = 0,
                        max_spins: int = 0, bad_lines=None, n: Optional[int] = None,
                        stream=None) -> None:
    w = "ll128_unpack_reduce"
    n = _numel(out, n)
    _check(_lib.ll128_unpack_reduce(
        _table(fifos, _lib.ll128_fifo_bytes(step_lines), ANY, "fifos", w), len(fifos),
        _addr(out, 4 * n, F32, "out", w), n, step_lines, first_step, max_spins,
        _addr(bad_lines, 4, U32, "bad_lines", w), _stream(stream)), w)


def ll_lines(n: int) -> int:
    return _lib.ll_lines(n)


def ll128_lines(n: int) -> int:
    return _lib.ll128_lines(n)


def ll_fifo_bytes(step_lines: int) -> int:
    return _lib.ll_fifo_bytes(step_lines)


def ll128_fifo_bytes(step_lines: int) -> int:
    return _lib.ll128_fifo_bytes(step_lines)


def ll_default_step_lines() -> int:
    return _lib.ll_default_step_lines()


def ll128_default_step_lines() -> int:
    return _lib.ll128_default_step_lines()


def ar_fifo_step_wire_bytes(proto: int, step_bytes: int) -> int:
    return _lib.ar_fifo_step_wire_bytes(proto, step_bytes)


def ar_fifo_steps_per_channel(n: int, step_bytes: int, channels: int) -> int:
    return _lib.ar_fifo_steps_per_channel(n, step_bytes, channels)


def ar_fifo_plan(proto: int, n: int, channels: int, step_bytes: int,
                 with_local: bool = False):
    """(lanes per workgroup, pairs per channel, whole steps per LL batch)
    that ar_fifo_stream picks for these arguments on the current device."""
    lanes, pairs, steps = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check(_lib.ar_fifo_plan(proto, n, channels, step_bytes, 1 if with_local else 0,
                             ctypes.byref(lanes), ctypes.byref(pairs), ctypes.byref(steps)),
           "ar_fifo_plan")
    return lanes.value, pairs.value, steps.value


def ar_fifo_counter_words(channels: int) -> int:
    return _lib.ar_fifo_counter_words(channels)


def ar_fifo_stream(proto: int, src, out, fifo, counters, channels: int, step_bytes: int,
                   first_step: int = 0, max_spins: int = AR_MAX_SPINS, errors=None,
                   local=None, n: Optional[int] = None, stream=None) -> None:
    """Stream src through `channels` 8-slot rings (one launch of producer and
    consumer workgroups) into out (= src, or local + src).  first_step may be
    AR_FIFO_CONTINUE: start from the step stored in counters by the last call."""
    w = "ar_fifo_stream"
    n = _numel(src, n)
    ring = channels * AR_FIFO_STEPS * _lib.ar_fifo_step_wire_bytes(proto, step_bytes)
    _check(_lib.ar_fifo_stream(proto, _addr(src, 4 * n, F32, "src", w),
                               _addr(local, 4 * n, F32, "local", w),
                               _addr(out, 4 * n, F32, "out", w), n,
                               _addr(fifo, ring, ANY, "fifo", w),
                               _addr(counters, 8 * _lib.ar_fifo_counter_words(channels), ANY,
                                     "counters", w), channels, step_bytes, first_step,
                               max_spins, _addr(errors, 4, U32, "errors", w), _stream(stream)),
           w)


def ar_copy(src, dst, nbytes: Optional[int] = None, stream=None) -> None:
    """dst[0..nbytes) = src[0..nbytes) with the plain 16-byte copy kernel
    (the achievable-copy reference of the measurements)."""
    w = "ar_copy"
    if nbytes is None:
        nbytes = src.numel() * src.element_size()
    _check(_lib.ar_copy(_addr(src, nbytes, ANY, "src", w), _addr(dst, nbytes, ANY, "dst", w),
                        nbytes, _stream(stream)), w)


def status_str(status: int) -> str:
    return _lib.ar_status_str(status).decode()


def raw():
    """The underlying ctypes library (for the export and error-path tests)."""
    return _lib
