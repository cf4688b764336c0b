"""ctypes binding of libar (include/libar.h), same names as the C ABI.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libar.so``.  Tensors are torch device tensors (torch supplies
device memory and streams); bf16 tensors are ``torch.bfloat16`` or raw
``torch.int16``/``torch.uint16`` bit patterns.  Each call enqueues on
``stream`` (default: torch's current stream) and returns without waiting.
A non-zero status raises ``ArError``.

Importing this module loads ``libar.so`` and fails loudly if it was not
built (``python -m ar_rmsnorm_amd.build``): there is no fallback path.
"""
from __future__ import annotations

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

EXPORTS = (
    "ar_status_str", "ar_last_hip_error", "ar_reduce_1stage", "ar_reduce_2stage",
    "ar_fused_residual_rmsnorm", "ar_fused_residual_rmsnorm_2stage", "ar_lamport_comm_bytes", "ar_lamport_fill",
    "ar_lamport_push", "ar_lamport_fused_residual_rmsnorm",
    "ar_lamport_oneshot_residual_rmsnorm", "ll_pack", "ll_unpack_reduce", "ll128_pack",
    "ll128_unpack_reduce", "ll_lines", "ll128_lines", "ll_fifo_bytes",
    "ll128_fifo_bytes", "ll_default_step_lines", "ll128_default_step_lines",
    "ar_fifo_stream", "ar_fifo_step_wire_bytes", "ar_fifo_steps_per_channel",
    "ar_fifo_counter_words",
)
AR_PROTO_LL, AR_PROTO_LL128, AR_PROTO_SIMPLE = 0, 1, 2
AR_FIFO_MAX_CHANNELS = 256
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
_lib.ar_fused_residual_rmsnorm.argtypes = [_pp, _int, _vp, _vp, _vp, _vp, _i64, _i64,
                                           ctypes.c_float, _vp]
_lib.ar_fused_residual_rmsnorm_2stage.argtypes = [_pp, _pp, _int, _int, _vp, _vp, _vp, _vp,
                                                  _i64, _i64, ctypes.c_float, ctypes.c_uint,
                                                  _vp]
_lib.ar_lamport_comm_bytes.argtypes = [_int, _i64, _i64]
_lib.ar_lamport_comm_bytes.restype = _i64
_lib.ar_lamport_fill.argtypes = [_vp, _int, _i64, _i64, _vp]
_lib.ar_lamport_push.argtypes = [_vp, _int, _int, _pp, _i64, _i64, _u32, _vp]
_lib.ar_lamport_fused_residual_rmsnorm.argtypes = [_vp, _int, _vp, _vp, _vp, _vp, _i64, _i64,
                                                   ctypes.c_float, _u32, _u32, _vp, _vp]
_lib.ar_lamport_oneshot_residual_rmsnorm.argtypes = [_vp, _int, _pp, _int, _vp, _vp, _vp, _vp,
                                                     _i64, _i64, ctypes.c_float, _u32, _u32,
                                                     _vp, _vp]
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
_lib.ar_fifo_counter_words.argtypes = [_int]
_lib.ar_fifo_counter_words.restype = _i64


class ArError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.ar_status_str(status).decode()
        if status == AR_ERR_HIP:
            msg += f" (hipError_t {_lib.ar_last_hip_error()})"
        super().__init__(f"{where}: status {status}: {msg}")


def _check(status: int, where: str) -> None:
    if status != AR_OK:
        raise ArError(status, where)


def _addr(x) -> Optional[int]:
    """Device address of a tensor, or an int address, or None for NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _table(xs) -> ctypes.Array:
    return (ctypes.c_void_p * len(xs))(*[_addr(x) for x in xs])


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
    _check(_lib.ar_reduce_1stage(_table(inputs), len(inputs), _addr(out),
                                 _numel(inputs[0], n), _stream(stream)),
           "ar_reduce_1stage")


def ar_reduce_2stage(inputs: Sequence, tmps: Sequence, rank: int, out,
                     flags: int = 0, n: Optional[int] = None, stream=None) -> None:
    """Reduce-scatter of this rank's shard into tmps[rank], then all-gather
    of all W shards into out (flags select the stages and the order)."""
    _check(_lib.ar_reduce_2stage(_table(inputs), _table(tmps), len(inputs), rank,
                                 _addr(out), _numel(inputs[0], n), flags, _stream(stream)),
           "ar_reduce_2stage")


def ar_fused_residual_rmsnorm(inputs: Sequence, residual, weight, residual_out, norm_out,
                              eps: float, M: Optional[int] = None, N: Optional[int] = None,
                              stream=None) -> None:
    """residual_out = sum(inputs) + residual; norm_out = RMSNorm(residual_out)."""
    if M is None or N is None:
        M, N = residual.shape
    _check(_lib.ar_fused_residual_rmsnorm(_table(inputs), len(inputs), _addr(residual),
                                          _addr(weight), _addr(residual_out),
                                          _addr(norm_out), M, N, float(eps),
                                          _stream(stream)),
           "ar_fused_residual_rmsnorm")


def ar_fused_residual_rmsnorm_2stage(inputs: Sequence, tmps: Sequence, rank: int, residual,
                                     weight, residual_out, norm_out, eps: float,
                                     flags: int = 0, M: Optional[int] = None,
                                     N: Optional[int] = None, stream=None) -> None:
    """Two-shot fused form for one rank: the fused operator on this rank's
    row shard (staged in tmps[rank]), then the gather of every shard."""
    if M is None or N is None:
        M, N = residual.shape
    _check(_lib.ar_fused_residual_rmsnorm_2stage(
        _table(inputs), _table(tmps), len(inputs), rank, _addr(residual), _addr(weight),
        _addr(residual_out), _addr(norm_out), M, N, float(eps), flags, _stream(stream)),
        "ar_fused_residual_rmsnorm_2stage")


def ar_lamport_comm_bytes(W: int, M: int, N: int) -> int:
    return _lib.ar_lamport_comm_bytes(W, M, N)


def ar_lamport_fill(comm, W: int, M: int, N: int, stream=None) -> None:
    """Fill a comm buffer with the sentinel (all three regions)."""
    _check(_lib.ar_lamport_fill(_addr(comm), W, M, N, _stream(stream)), "ar_lamport_fill")


def ar_lamport_push(x, rank: int, comms: Sequence, flag: int, M: Optional[int] = None,
                    N: Optional[int] = None, stream=None) -> None:
    """Push bf16 [M, N] rows of `rank` into slot `rank` of region flag % 3 of
    the W comm buffers (W = len(comms))."""
    if M is None or N is None:
        M, N = x.shape
    _check(_lib.ar_lamport_push(_addr(x), len(comms), rank, _table(comms), M, N,
                                flag & 0xFFFFFFFF, _stream(stream)), "ar_lamport_push")


def ar_lamport_fused_residual_rmsnorm(comm, W: int, residual, weight, residual_out,
                                      norm_out, eps: float, flag: int, max_spins: int = 0,
                                      bad_chunks=None, M: Optional[int] = None,
                                      N: Optional[int] = None, stream=None) -> None:
    """Reduce the W slots of region flag % 3 of `comm`, add the residual,
    normalise; then reset region (flag + 2) % 3 to the sentinel."""
    if M is None or N is None:
        M, N = residual.shape
    _check(_lib.ar_lamport_fused_residual_rmsnorm(
        _addr(comm), W, _addr(residual), _addr(weight), _addr(residual_out), _addr(norm_out),
        M, N, float(eps), flag & 0xFFFFFFFF, max_spins, _addr(bad_chunks), _stream(stream)),
        "ar_lamport_fused_residual_rmsnorm")


def ar_lamport_oneshot_residual_rmsnorm(x, rank: int, comms: Sequence, residual, weight,
                                        residual_out, norm_out, eps: float, flag: int,
                                        max_spins: int = 0, bad_chunks=None,
                                        M: Optional[int] = None, N: Optional[int] = None,
                                        stream=None) -> None:
    """One launch: push x as `rank` into the W comm buffers, then reduce
    comms[rank], add the residual and normalise (W = len(comms))."""
    if M is None or N is None:
        M, N = residual.shape
    _check(_lib.ar_lamport_oneshot_residual_rmsnorm(
        _addr(x), rank, _table(comms), len(comms), _addr(residual), _addr(weight),
        _addr(residual_out), _addr(norm_out), M, N, float(eps), flag & 0xFFFFFFFF, max_spins,
        _addr(bad_chunks), _stream(stream)), "ar_lamport_oneshot_residual_rmsnorm")


def ll_pack(src, fifo, step_lines: int, first_step: int = 0, n: Optional[int] = None,
            stream=None) -> None:
    _check(_lib.ll_pack(_addr(src), _numel(src, n), _addr(fifo), step_lines, first_step,
                        _stream(stream)), "ll_pack")


def ll128_pack(src, fifo, step_lines: int, first_step: int = 0, n: Optional[int] = None,
               stream=None) -> None:
    _check(_lib.ll128_pack(_addr(src), _numel(src, n), _addr(fifo), step_lines, first_step,
                           _stream(stream)), "ll128_pack")


def ll_unpack_reduce(fifos: Sequence, out, step_lines: int, first_step: int = 0,
                     max_spins: int = 0, bad_lines=None, n: Optional[int] = None,
                     stream=None) -> None:
    _check(_lib.ll_unpack_reduce(_table(fifos), len(fifos), _addr(out), _numel(out, n),
                                 step_lines, first_step, max_spins, _addr(bad_lines),
                                 _stream(stream)), "ll_unpack_reduce")


def ll128_unpack_reduce(fifos: Sequence, out, step_lines: int, first_step: int = 0,
                        max_spins: int = 0, bad_lines=None, n: Optional[int] = None,
                        stream=None) -> None:
    _check(_lib.ll128_unpack_reduce(_table(fifos), len(fifos), _addr(out), _numel(out, n),
                                    step_lines, first_step, max_spins, _addr(bad_lines),
                                    _stream(stream)), "ll128_unpack_reduce")


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


def ar_fifo_counter_words(channels: int) -> int:
    return _lib.ar_fifo_counter_words(channels)


def ar_fifo_stream(proto: int, src, out, fifo, counters, channels: int, step_bytes: int,
                   first_step: int = 0, max_spins: int = AR_MAX_SPINS, errors=None,
                   local=None, n: Optional[int] = None, stream=None) -> None:
    """Stream src through `channels` 8-slot rings (one launch of producer and
    consumer workgroups) into out (= src, or local + src).  first_step may be
    AR_FIFO_CONTINUE: start from the step stored in counters by the last call."""
    _check(_lib.ar_fifo_stream(proto, _addr(src), _addr(local), _addr(out), _numel(src, n),
                               _addr(fifo), _addr(counters), channels, step_bytes, first_step,
                               max_spins, _addr(errors), _stream(stream)), "ar_fifo_stream")


def status_str(status: int) -> str:
    return _lib.ar_status_str(status).decode()


def raw():
    """The underlying ctypes library (for the export and error-path tests)."""
    return _lib
