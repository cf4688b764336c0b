"""The binding's own buffer checks with real device tensors, and the plain
copy kernel that the measurements use as their achievable-copy reference.

A buffer that is too small, strided, of the wrong element size or on the
host is refused with AR_ERR_ARG before anything is enqueued, so the output
is left as it was.
"""
import numpy as np
import pytest
import torch

from ar_rmsnorm_amd import libar as ar

pytestmark = pytest.mark.gpu


def refused(fn, *args, **kw):
    with pytest.raises(ar.ArError) as e:
        fn(*args, **kw)
    assert e.value.status == ar.AR_ERR_ARG
    return str(e.value)


def test_short_strided_mistyped_and_host_buffers_are_refused(gpu):
    W, n = 4, 4096
    ins = [torch.randint(-100, 100, (n,), dtype=torch.int16, device=gpu) for _ in range(W)]
    out = torch.full((n,), 7, dtype=torch.int16, device=gpu)
    assert "touches" in refused(ar.ar_reduce_1stage, ins, out[: n - 8], n)
    assert "touches" in refused(ar.ar_reduce_1stage, [ins[0][:8]] + ins[1:], out, n)
    wide = torch.zeros((n, 2), dtype=torch.int16, device=gpu)
    assert "contiguous" in refused(ar.ar_reduce_1stage, ins, wide[:, 0])
    assert "element" in refused(ar.ar_reduce_1stage, [x.float() for x in ins], out)
    assert "not on a GPU" in refused(ar.ar_reduce_1stage, ins, out.cpu())
    assert "torch tensor" in refused(ar.ar_reduce_1stage, ins, out.data_ptr(), n)
    P = n // 8
    tmps = [torch.empty((P // W + P % W) * 8, dtype=torch.int16, device=gpu)
            for _ in range(W)]
    assert "tmps" in refused(ar.ar_reduce_2stage, ins, tmps[:-1] + [tmps[0][:-8]], 0, out)
    fifo = torch.zeros(ar.ll_fifo_bytes(64) - 16, dtype=torch.uint8, device=gpu)
    src = torch.zeros(256, dtype=torch.float32, device=gpu)
    assert "fifo" in refused(ar.ll_pack, src, fifo, 64)
    torch.cuda.synchronize()
    assert torch.all(out == 7), "a refused call wrote its output"


def test_refused_wire_and_stream_extents(gpu):
    src = torch.zeros(1000, dtype=torch.float32, device=gpu)
    out = torch.zeros(999, dtype=torch.float32, device=gpu)
    fifos = [torch.zeros(ar.ll128_fifo_bytes(2), dtype=torch.uint8, device=gpu)]
    refused(ar.ll128_unpack_reduce, fifos, out, 2, n=1000)
    ch, step = 2, 1024
    ring = torch.zeros(ch * 8 * ar.ar_fifo_step_wire_bytes(ar.AR_PROTO_LL, step) - 16,
                       dtype=torch.uint8, device=gpu)
    cnt = torch.zeros(ar.ar_fifo_counter_words(ch), dtype=torch.int64, device=gpu)
    errs = torch.zeros(1, dtype=torch.int32, device=gpu)
    assert "fifo" in refused(ar.ar_fifo_stream, ar.AR_PROTO_LL, src, src.clone(), ring, cnt, ch,
                             step, errors=errs)


@pytest.mark.parametrize("nbytes", [16, 4096, 4096 + 16 * 13, 12 << 20])
def test_copy_is_exact(gpu, nbytes):
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    host = torch.randint(0, 256, (nbytes + 64,), dtype=torch.uint8, generator=g)
    src = host[:nbytes].to(gpu)
    dst = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device=gpu)
    ar.ar_copy(src, dst, nbytes)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    assert np.array_equal(got[:nbytes], host[:nbytes].numpy())
    assert np.all(got[nbytes:] == 0xA5), "copy wrote past its end"
