"""Seeded synthetic inputs for the tests, the smoke check and the bench.

This module holds none of the method's arithmetic: it only draws random
numbers and stores them as bf16 or fp32.  Both the HIP path's tests and the
oracle are fed from here, so they always see the same bytes.

Shapes and distributions follow the workloads the method is run on:
  * one-shot reduce, W=2 rank buffers of 8192 bf16 ~ N(0, 1)
  * one-shot reduce at the decode shape, W=8 buffers of 1 x 8192 bf16 ~ N(0, 1)
  * fused all-reduce + residual + RMSNorm, W=4, rows [M, 2048] with
    M in {1, 16, 128}; x and residual ~ N(0, 1), weight ~ N(1, 0.1), eps 1e-6
  * two-stage reduce at the 8 MB message cap, W=8 buffers of 4,194,304 bf16
    ~ U(-1, 1)
  * LL / LL128 wire formats, W=4 fp32 payloads of 16,777,216 values ~ N(0, 1),
    and the same plus a 13-value tail
Each workload has its own seed sequence ``[1000 + id, ...]``; the W rank
buffers are drawn first, in rank order, then residual, then weight.

bf16 values are made by drawing fp32 and converting with torch's CPU cast
(plain input preparation, not part of what is tested).
"""
from __future__ import annotations

import numpy as np
import torch

REDUCE_SMALL = dict(id=1, W=2, n=8192)
REDUCE_DECODE = dict(id=2, W=8, n=8192)
FUSED = dict(id=3, W=4, N=2048, Ms=(1, 16, 128), eps=1e-6)
REDUCE_CAP = dict(id=4, W=8, n=4_194_304)
WIRE = dict(id=5, W=4, n=16_777_216, tail=13)


def rng(*seed) -> np.random.Generator:
    return np.random.default_rng(list(seed))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(g: np.random.Generator, shape, mean=0.0, std=1.0) -> np.ndarray:
    return to_bf16_bits(g.normal(mean, std, size=shape).astype(np.float32))


def uniform_bf16(g: np.random.Generator, shape, lo=-1.0, hi=1.0) -> np.ndarray:
    return to_bf16_bits(g.uniform(lo, hi, size=shape).astype(np.float32))


def reduce_inputs(W: int, n: int, seed, dist: str = "normal"):
    """W rank buffers of n bf16 values (uint16 bits), drawn in rank order."""
    g = rng(*seed) if isinstance(seed, (list, tuple)) else rng(seed)
    draw = normal_bf16 if dist == "normal" else uniform_bf16
    return [draw(g, n) for _ in range(W)]


def fused_inputs(W: int, M: int, N: int, seed):
    """(xs, residual, weight): W bf16 [M, N] buffers, bf16 [M, N] residual
    ~ N(0, 1), bf16 [N] weight ~ N(1, 0.1)."""
    g = rng(*seed) if isinstance(seed, (list, tuple)) else rng(seed)
    xs = [normal_bf16(g, (M, N)) for _ in range(W)]
    residual = normal_bf16(g, (M, N))
    weight = normal_bf16(g, N, 1.0, 0.1)
    return xs, residual, weight


def wire_payloads(W: int, n: int, seed):
    """W fp32 payloads of n values ~ N(0, 1)."""
    g = rng(*seed) if isinstance(seed, (list, tuple)) else rng(seed)
    return [g.standard_normal(n, dtype=np.float32) for _ in range(W)]


# The workloads as (inputs, description) makers, seeded as described above.
def reduce_small():
    c = REDUCE_SMALL
    return reduce_inputs(c["W"], c["n"], [1000 + c["id"]])


def reduce_decode():
    c = REDUCE_DECODE
    return reduce_inputs(c["W"], c["n"], [1000 + c["id"]])


def fused(M: int):
    c = FUSED
    return fused_inputs(c["W"], M, c["N"], [1000 + c["id"], M])


def reduce_cap():
    c = REDUCE_CAP
    return reduce_inputs(c["W"], c["n"], [1000 + c["id"]], dist="uniform")


def wire(n: int):
    c = WIRE
    return wire_payloads(c["W"], n, [1000 + c["id"], n])
