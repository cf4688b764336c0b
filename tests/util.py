"""Helpers shared by the tests: host <-> device moves and the fused-norm
tolerance.  No arithmetic of the method lives here."""
import numpy as np
import torch


def dev_u16(a: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit patterns -> int16 device tensor holding the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def dev_f32(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def dev_u8(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v|: 2^(floor(log2|v|) - 7), and 2^-133 in
    the denormal range."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.exp2(e - 7.0)


def norm_within_tolerance(got_bits: np.ndarray, exact: np.ndarray):
    """The fused norm_out bar: |gpu - exact| <= 2 bf16 ulp of the exact value,
    or <= 1e-2 absolute.  Returns (ok mask, max error in ulp)."""
    got = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(got - exact)
    ulp = bf16_ulp(exact)
    ok = (err <= 2.0 * ulp) | (err <= 1e-2)
    return ok, float(np.max(err / ulp)) if err.size else 0.0
