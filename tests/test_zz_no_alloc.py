"""The allocation-free two-stage reduce against the entry point it mirrors.

ar_reduce_2stage_noalloc keeps the W staging shards in the library's own
device array instead of caller buffers.  For every rank of a message, the
peers' reduce-scatters go first (as on several GPUs), then the rank's
reduce-scatter + all-gather; the output must equal, bit for bit, what
ar_reduce_2stage gives on the same inputs with caller-owned staging buffers
and the oracle.  Two calls in a row, the second with a smaller message, so
the array holds the first call's shards when the second starts.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from ar_rmsnorm_amd import libar as ar
from ar_rmsnorm_amd import synth
from tests.util import dev_u16, host_u16

pytestmark = pytest.mark.gpu


def with_caller_staging(d, rank, n):
    W, P = len(d), n // 8
    tmps = [torch.empty((P // W + P % W) * 8, dtype=torch.int16, device=d[0].device)
            for _ in range(W)]
    for r in range(W):
        if r != rank:
            ar.ar_reduce_2stage(d, tmps, r, None, flags=ar.AR_STAGE_RS)
    out = torch.empty(n, dtype=torch.int16, device=d[0].device)
    ar.ar_reduce_2stage(d, tmps, rank, out)
    return out


def with_library_staging(d, rank, n):
    W = len(d)
    for r in range(W):
        if r != rank:
            ar.ar_reduce_2stage_noalloc(d, r, None, flags=ar.AR_STAGE_RS)
    out = torch.full((n,), 0x7FC1, dtype=torch.int16, device=d[0].device)
    ar.ar_reduce_2stage_noalloc(d, rank, out)
    return out


@pytest.mark.parametrize("W", [8, 3])
def test_noalloc_matches_the_entry_point_it_mirrors(gpu, W):
    # the 8 MB cap message first, then a smaller one with a remainder
    for n, seed in ((4_194_304, 1), (8 * (W * 1000 + W - 1), 2)):
        xs = synth.reduce_inputs(W, n, [97, W, seed], dist="uniform")
        d = [dev_u16(x, gpu) for x in xs]
        want = orc.reduce_2stage(xs)
        for rank in (0, W - 1):
            ref = with_caller_staging(d, rank, n)
            got = with_library_staging(d, rank, n)
            torch.cuda.synchronize()
            assert np.array_equal(host_u16(got), host_u16(ref)), (W, n, rank)
            assert np.array_equal(host_u16(got), want), (W, n, rank)


def test_noalloc_refuses_messages_past_its_array(gpu):
    W = 8
    n = 8 * (((ar.AR_SCRATCH_BYTES // 16) // W + 1) * W)
    d = [torch.zeros(n, dtype=torch.int16, device=gpu) for _ in range(W)]
    out = torch.zeros(n, dtype=torch.int16, device=gpu)
    with pytest.raises(ar.ArError) as e:
        ar.ar_reduce_2stage_noalloc(d, 0, out)
    assert e.value.status == ar.AR_ERR_CAPACITY
