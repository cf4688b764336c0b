"""GPU parity of streaming through 8-step FIFOs (producer and consumer
workgroups concurrent in one launch) against the oracle: the
delivered payload and the rings' final bytes are bit-exact, and no wait
times out.  Every wait in the kernel is bounded; the abort test forces the
give-up path from the host (the error count set before the launch)."""
import numpy as np
import pytest
import torch

import oracle as orc
from ar_rmsnorm_amd import libar as ar
from ar_rmsnorm_amd import synth

pytestmark = pytest.mark.gpu

PROTOS = {"ll": ar.AR_PROTO_LL, "ll128": ar.AR_PROTO_LL128, "simple": ar.AR_PROTO_SIMPLE}


def sync():
    torch.cuda.synchronize()


class Fifo:
    """One set of rings and counters, with the oracle's copy of the rings and
    the first step the next call starts from."""

    def __init__(self, proto, step, channels, device):
        self.proto, self.step, self.channels, self.device = proto, step, channels, device
        wire = ar.ar_fifo_step_wire_bytes(proto, step)
        assert wire > 0
        self.fifo = torch.zeros(channels * 8 * wire, dtype=torch.uint8, device=device)
        self.counters = torch.zeros(ar.ar_fifo_counter_words(channels), dtype=torch.int64,
                                    device=device)
        self.errors = torch.zeros(1, dtype=torch.int32, device=device)
        self.host = np.zeros(channels * 8 * wire, np.uint8)
        self.first = 0

    def launch(self, d, out, n, dl=None, cont=False, max_spins=ar.AR_MAX_SPINS):
        ar.ar_fifo_stream(self.proto, d, out, self.fifo, self.counters, self.channels, self.step,
                          ar.AR_FIFO_CONTINUE if cont else self.first, max_spins, self.errors,
                          local=dl, n=n)

    def check(self, src, out, local=None):
        """Compare a finished call with the oracle and advance the step."""
        n = src.size
        got = out.cpu().numpy()
        assert np.all(got[n:] == 777.0), "wrote past n"
        want, self.host = orc.fifo_stream(self.proto, src, self.channels, self.step, self.first,
                                          local=local, fifo=self.host)
        assert int(self.errors.item()) == 0, "a wait timed out"
        assert np.array_equal(got[:n].view(np.uint32), want.view(np.uint32)), "payload"
        assert np.array_equal(self.fifo.cpu().numpy(), self.host), "ring bytes"
        self.first += ar.ar_fifo_steps_per_channel(n, self.step, self.channels)
        state = self.counters.cpu().numpy()[-2:]
        assert state[0] == self.first and state[1] == 0, "stored step"

    def run(self, src, local=None, cont=False, max_spins=ar.AR_MAX_SPINS):
        n = src.size
        d = torch.from_numpy(src).to(self.device)
        dl = None if local is None else torch.from_numpy(local).to(self.device)
        out = torch.full((n + 16,), 777.0, dtype=torch.float32, device=self.device)
        self.launch(d, out, n, dl, cont, max_spins)
        sync()
        self.check(src, out, local)


@pytest.mark.parametrize("name,step", [("ll", 1024), ("ll128", 1200), ("ll128", 840),
                                       ("simple", 1024)])
@pytest.mark.parametrize("channels", [1, 4, 16])
def test_stream_many_laps(gpu, name, step, channels):
    """About 20 steps per channel (2.5 laps of the ring) and a ragged tail."""
    n = channels * 20 * step // 4 + 13
    src = synth.wire_payloads(1, n, [102, channels, step])[0]
    Fifo(PROTOS[name], step, channels, gpu).run(src)


@pytest.mark.parametrize("name,step,channels", [("ll", 32768, 16), ("ll128", 576000, 4),
                                                ("simple", 524288, 4)])
def test_stream_nccl_default_steps_wire_workload(gpu, name, step, channels):
    """The wire workload (16 Mi + 13 fp32) at NCCL's default step sizes."""
    n = synth.WIRE["n"] + synth.WIRE["tail"]
    src = synth.wire(n)[0]
    Fifo(PROTOS[name], step, channels, gpu).run(src)


@pytest.mark.parametrize("name,step,channels", [("ll", 32768, 32), ("ll128", 576000, 32),
                                                ("simple", 524288, 32), ("ll", 32768, 128),
                                                ("ll128", 576000, 128), ("simple", 524288, 128),
                                                ("ll", 32768, 256)])
def test_stream_bench_configurations(gpu, name, step, channels):
    """The channel counts the bench times, on the wire workload's payload,
    twice in a row from the stored step."""
    n = synth.WIRE["n"]
    src = synth.wire(n)[0]
    f = Fifo(PROTOS[name], step, channels, gpu)
    f.run(src, cont=True)
    f.run(src, cont=True)


@pytest.mark.parametrize("name,step,channels", [("ll", 32768, 32), ("ll", 32768, 128),
                                                ("ll128", 576000, 32), ("ll128", 576000, 128),
                                                ("simple", 524288, 32),
                                                ("simple", 524288, 128)])
def test_stream_bench_configurations_over_many_calls(gpu, name, step, channels):
    """The bench rows' configurations over 100 calls each, as the bench runs
    them (back to back on one set of rings, each call from the stored step):
    a graph of 20 calls, each into its own output, replayed 5 times with the
    outputs cleared in between; every call must deliver the oracle's payload
    bit for bit with no failed wait."""
    proto, n, calls = PROTOS[name], synth.WIRE["n"], 20
    src = synth.wire(n)[0]
    want, _ = orc.fifo_stream(proto, src, channels, step, 0)
    want = torch.from_numpy(want).to(gpu).view(torch.int32)
    f = Fifo(proto, step, channels, gpu)
    d = torch.from_numpy(src).to(gpu)
    outs = [torch.zeros(n, dtype=torch.float32, device=gpu) for _ in range(calls)]
    f.launch(d, outs[0], n, cont=True)      # warm-up call outside the graph
    sync()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for o in outs:
            f.launch(d, o, n, cont=True)
    torch.cuda.current_stream().wait_stream(s)
    sync()
    for r in range(5):
        for o in outs:
            o.zero_()
        sync()
        g.replay()
        sync()
        assert int(f.errors.item()) == 0, f"replay {r}: a wait timed out"
        bad = [i for i, o in enumerate(outs) if not torch.equal(o.view(torch.int32), want)]
        assert not bad, f"replay {r}: calls {bad} delivered wrong payload"
    del g


def test_stream_plans_of_the_bench_rows(gpu):
    """The launch shapes the bench rows run with (lanes, pairs per channel,
    whole steps per LL batch) on a 256-CU MI355X: 32 channels take four
    1,024-lane pairs, except LL, whose 64 steps per channel take eight
    512-lane pairs; 128 channels two 512-lane pairs; LL spans 4 and 2 steps
    per batch there, one-step messages stay in one step."""
    n = synth.WIRE["n"]
    want = {("ll", 32): (512, 8, 4), ("ll", 128): (512, 2, 2),
            ("ll128", 32): (1024, 4, 1), ("ll128", 128): (512, 2, 1),
            ("simple", 32): (1024, 4, 1), ("simple", 128): (512, 2, 1)}
    steps = {"ll": 32768, "ll128": 576000, "simple": 524288}
    for (name, ch), plan in want.items():
        assert ar.ar_fifo_plan(PROTOS[name], n, ch, steps[name]) == plan, (name, ch)
    # 8 KiB over 32 channels at the 32 KiB step: one step on one channel,
    # one pair, one step per batch
    assert ar.ar_fifo_plan(ar.AR_PROTO_LL, 2048, 32, 32768) == (1024, 1, 1)
    # 4 Mi fp32 over 32 channels: 16 steps a channel keep the wider form
    assert ar.ar_fifo_plan(ar.AR_PROTO_LL, 1 << 22, 32, 32768) == (1024, 4, 4)
    # 16 Mi fp32 over 64 channels: 32 steps a channel, four 512-lane pairs
    assert ar.ar_fifo_plan(ar.AR_PROTO_LL, 1 << 24, 64, 32768) == (512, 4, 4)


@pytest.mark.parametrize("name,step", [("ll", 1024), ("ll128", 1200), ("simple", 1024)])
def test_stream_256_channels(gpu, name, step):
    """256 channels need two workgroups per CU: the 512-lane geometry where
    the 1,024-lane one does not fit twice, with three steps per channel and a
    ragged tail, called twice from the stored step."""
    n = 256 * 3 * step // 4 - 3
    src = synth.wire_payloads(1, n, [107, step])[0]
    f = Fifo(PROTOS[name], step, 256, gpu)
    f.run(src, cont=True)
    f.run(src, cont=True)


def test_stream_workgroups_that_cannot_be_resident_are_refused(gpu):
    """256 channels need 512 resident workgroups; where a variant cannot
    have them the call is refused before anything runs, else it is exact."""
    n, step, ch = 256 * 2 * 1200 // 4, 1200, 256
    src, local = synth.wire_payloads(2, n, [106])
    f = Fifo(ar.AR_PROTO_LL128, step, ch, gpu)
    d, dl = torch.from_numpy(src).to(gpu), torch.from_numpy(local).to(gpu)
    out = torch.full((n + 16,), 777.0, dtype=torch.float32, device=gpu)
    try:
        f.launch(d, out, n, dl)
    except ar.ArError as e:
        assert e.status == ar.AR_ERR_CAPACITY
        sync()
        assert np.all(f.counters.cpu().numpy() == 0) and np.all(out.cpu().numpy() == 777.0)
        return
    sync()
    f.check(src, out, local)


@pytest.mark.parametrize("name,step", [("ll", 2048), ("ll128", 2400), ("ll128", 1080),
                                       ("simple", 2048)])
def test_stream_reduce_with_local_and_consecutive_calls(gpu, name, step):
    """Calls on one set of rings: explicit first steps, then the stored one."""
    f = Fifo(PROTOS[name], step, 8, gpu)
    for call in range(4):
        n = 8 * 13 * step // 4 + 7 * call + 1
        src, local = synth.wire_payloads(2, n, [103, call])
        f.run(src, local=local if call != 1 else None, cont=call >= 2)


@pytest.mark.parametrize("name,step,channels", [("ll", 1024, 3), ("ll128", 1200, 4),
                                                ("simple", 2048, 5)])
def test_stream_graph_replays_continue(gpu, name, step, channels):
    """A captured call with the stored first step, replayed: every replay
    runs a fresh range of ring steps (flags never repeat) and matches the
    oracle, with eager calls between replays."""
    f = Fifo(PROTOS[name], step, channels, gpu)
    n = channels * 11 * step // 4 + 5
    src = synth.wire_payloads(1, n, [104, channels])[0]
    d = torch.from_numpy(src).to(gpu)
    out = torch.full((n + 16,), 777.0, dtype=torch.float32, device=gpu)
    f.launch(d, out, n, cont=True)
    sync()
    f.check(src, out)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        f.launch(d, out, n, cont=True)
    torch.cuda.current_stream().wait_stream(s)
    sync()
    for r in range(3):
        out[:n].zero_()
        sync()
        g.replay()
        sync()
        f.check(src, out)
        other = synth.wire_payloads(1, n - r, [105, r])[0]      # eager call between replays
        f.run(other, cont=True)
    del g


@pytest.mark.parametrize("with_local", [False, True])
@pytest.mark.parametrize("name,step", [("ll", 32768), ("ll128", 120000), ("simple", 65536)])
def test_stream_producers_and_consumers_on_different_xcds(gpu, name, step, with_local):
    """Workgroups go round-robin to the 8 XCDs, whose L2 caches are not
    coherent with each other; with 100 channels a channel's producer (block
    c) and consumer (block 100 + c) sit on different XCDs.  Twenty-four
    calls in a row are captured in a graph, each into its own output, and
    the graph is replayed twice: every call must deliver the oracle's
    payload with no failed wait.  Data published before its stores were
    acknowledged showed up here as a few stale lines in about one call in
    a hundred."""
    proto, ch, n, calls = PROTOS[name], 100, 4 * 1024 * 1024 + 5, 24
    src, local = synth.wire_payloads(2, n, [108, step])
    if not with_local:
        local = None
    want, _ = orc.fifo_stream(proto, src, ch, step, 0, local=local)
    want = torch.from_numpy(want).to(gpu)
    f = Fifo(proto, step, ch, gpu)
    d = torch.from_numpy(src).to(gpu)
    dl = None if local is None else torch.from_numpy(local).to(gpu)
    outs = [torch.zeros(n, dtype=torch.float32, device=gpu) for _ in range(calls)]
    f.launch(d, outs[0], n, dl, cont=True)      # warm-up call outside the graph
    sync()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for o in outs:
            f.launch(d, o, n, dl, cont=True)
    torch.cuda.current_stream().wait_stream(s)
    sync()
    for r in range(2):
        for o in outs:
            o.zero_()
        sync()
        g.replay()
        sync()
        assert int(f.errors.item()) == 0, "a wait timed out"
        bad = [i for i, o in enumerate(outs) if not torch.equal(o.view(torch.int32),
                                                                 want.view(torch.int32))]
        assert not bad, f"replay {r}: calls {bad} delivered wrong payload"
    del g


# LL configurations whose pairs get slices of at most half a batch, so the
# library runs them as batches of S whole steps, with the reasoning that
# picks each case (the host takes as many pairs as fit, at most one per
# 2,048 lines a channel carries, none with a slice under 512 lines):
#   16 channels, 32 KiB steps (4,096 lines), 3 steps a channel and a
#     20-byte last step: 8 pairs of 512 lines, S = 4 on 1,024-lane
#     workgroups; the last step gives only pair 0 a slice
#   32 channels, 40 KiB steps, 3 steps a channel and 28 bytes more: 4 pairs
#     (all that fit) of 1,280 lines, S = 3
#   64 channels, 32 KiB steps, 2 steps a channel and 12 bytes more: 2 pairs
#     of 2,048 lines on 1,024-lane workgroups, S = 2
#   128 channels, 32 KiB steps, 2 steps a channel: one 1,024-lane pair fits
#     per channel, two 512-lane ones do: S = 2 on 512-lane workgroups
#   48 channels, 32 KiB steps, 33 steps a channel and a 44-byte step more
#     (channel 47 carries 34): two 1,024-lane pairs fit per channel, five
#     512-lane ones do, and with 32 steps or more a channel LL takes the
#     narrow form: 5 pairs of 820 lines (the last 816), S = 4; the short
#     step gives only pair 0 a slice
# Each runs twice on the same rings (the second call from the stored step),
# with and without a local addend where the addend still leaves S > 1.
# (channels, step, n, with_local, the plan: lanes, pairs, steps per batch)
WHOLE_STEP_CASES = [
    (16, 32768, 16 * 3 * 8192 + 5, True, (1024, 8, 4)),
    (32, 40960, 32 * 3 * 10240 + 7, True, (1024, 4, 3)),
    (64, 32768, 64 * 2 * 8192 + 3, False, (1024, 2, 2)),
    (128, 32768, 128 * 2 * 8192, False, (512, 2, 2)),
    (48, 32768, 48 * 33 * 8192 + 11, False, (512, 5, 4)),
]


@pytest.mark.parametrize("channels,step,n,with_local,plan", WHOLE_STEP_CASES)
def test_stream_ll_batches_of_whole_steps(gpu, channels, step, n, with_local, plan):
    assert ar.ar_fifo_plan(ar.AR_PROTO_LL, n, channels, step) == plan
    if with_local:
        assert ar.ar_fifo_plan(ar.AR_PROTO_LL, n, channels, step, with_local=True) == plan
    f = Fifo(ar.AR_PROTO_LL, step, channels, gpu)
    for call in range(2):
        src, local = synth.wire_payloads(2, n, [111, channels, call])
        f.run(src, cont=call == 1)
        if with_local:
            f.run(src, local=local, cont=True)


@pytest.mark.parametrize("case", range(12))
def test_stream_seeded_random_configurations(gpu, case):
    """Seeded random protocol, channel count (1..200), step size, payload
    length (from a few values to ~3 steps per channel, so channels without a
    step, partial last steps and single-step channels all occur), local
    addend or not (up to 128 channels, all a 256-CU device holds with one),
    and first step (explicit, then the stored one): two calls
    on one set of rings, each checked against the oracle, ring bytes
    included."""
    rng = np.random.default_rng([109, case])
    name = ["ll", "ll128", "simple"][case % 3]
    unit = {"ll": 8, "ll128": 120, "simple": 16}[name]
    step = unit * int(rng.integers(1, 400))
    channels = int(rng.integers(1, 201))
    f = Fifo(PROTOS[name], step, channels, gpu)
    f.first = int(rng.integers(0, 1 << 20))
    for call in range(2):
        n = int(rng.integers(1, 3 * channels * step // 4 + 2))
        src, local = synth.wire_payloads(2, n, [110, case, call])
        # with a local addend one workgroup fits per CU: at most 128 channels
        with_local = channels <= 128 and bool(rng.integers(0, 2))
        f.run(src, local=local if with_local else None, cont=call == 1)


def test_stream_aborted_launch_ends(gpu):
    """The error count is set before the launch, so every wait gives up at
    once: the launch must end (outputs unspecified)."""
    proto, step, channels = ar.AR_PROTO_LL, 1024, 8
    n = channels * 40 * step // 4
    f = Fifo(proto, step, channels, gpu)
    f.errors.fill_(1)
    src = torch.zeros(n, dtype=torch.float32, device=gpu)
    out = torch.empty_like(src)
    ar.ar_fifo_stream(proto, src, out, f.fifo, f.counters, channels, step, 0, 64, f.errors)
    sync()
    for p in (ar.AR_PROTO_LL128, ar.AR_PROTO_SIMPLE):
        g = Fifo(p, 1200 if p == ar.AR_PROTO_LL128 else 1024, channels, gpu)
        g.errors.fill_(1)
        ar.ar_fifo_stream(p, src, out, g.fifo, g.counters, channels, g.step, 0, 64, g.errors)
    sync()
    assert int(f.errors.item()) >= 1


def test_stream_argument_errors(gpu):
    f = Fifo(ar.AR_PROTO_LL128, 1200, 2, gpu)
    src = torch.zeros(1000, dtype=torch.float32, device=gpu)
    out = torch.zeros(1000, dtype=torch.float32, device=gpu)
    for bad_step in (1000, 0, 119):
        with pytest.raises(ar.ArError) as e:
            ar.ar_fifo_stream(ar.AR_PROTO_LL128, src, out, f.fifo, f.counters, 2, bad_step, 0,
                              100, f.errors)
        assert e.value.status == ar.AR_ERR_ARG
    with pytest.raises(ar.ArError) as e:
        ar.ar_fifo_stream(ar.AR_PROTO_LL128, src, out, f.fifo, f.counters, 0, 1200, 0, 100,
                          f.errors)
    assert e.value.status == ar.AR_ERR_ARG
    with pytest.raises(ar.ArError) as e:
        ar.ar_fifo_stream(3, src, out, f.fifo, f.counters, 2, 1200, 0, 100, f.errors)
    assert e.value.status == ar.AR_ERR_ARG
    with pytest.raises(ar.ArError) as e:
        ar.ar_fifo_stream(ar.AR_PROTO_LL128, src, src, f.fifo, f.counters, 2, 1200, 0, 100,
                          f.errors)
    assert e.value.status == ar.AR_ERR_ARG      # out overlaps src
    with pytest.raises(ar.ArError) as e:
        ar.ar_fifo_stream(ar.AR_PROTO_LL128, src, out, f.fifo, f.counters, 2, 1200, 0, 100,
                          out[:1].view(torch.int32))
    assert e.value.status == ar.AR_ERR_ARG      # errors inside out
    sync()
