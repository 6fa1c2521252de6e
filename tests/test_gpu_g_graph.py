"""GPU: fused calls captured into a HIP graph (the way the bench times them) give, on every
replay, the bits the same calls give when launched eagerly.  Replays are separated by eager
work and synchronizations, and each replay is checked (a captured library call that only
the first replay gets right would fail here)."""
import numpy as np
import pytest
import torch

import synth
from helpers import Packed, dev_bits, host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from decode_linear_amd import build
    build.ensure_built()


def _replays_match(calls, outs):
    eager = []
    for f in calls:
        f()
    torch.cuda.synchronize()
    eager = [host_bits(o).copy() for o in outs]
    for o in outs:
        o.zero_()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in calls:
            f()
    for r in range(3):
        for o in outs:
            o.zero_()
        calls[0]()                      # eager work between replays
        torch.cuda.synchronize()
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert np.array_equal(host_bits(o), eager[i]), f"replay {r}, output {i}"


def test_graph_replay_gateup_and_linear():
    from decode_linear_amd import qlin_gateup_swiglu, qlin_linear
    gc = synth.random_gateup(7001, 4, 4096, 1024, 4)
    gq, uq = Packed(gc.gate, 4), Packed(gc.up, 4)
    xg = dev_bits(gc.x, synth.BF16)
    lc = synth.random_case(7002, 4, 2048, 512, 8, ln=True, act=1, x_mean=3.0)
    lq = Packed(lc.w_f32, 8)
    xl = dev_bits(lc.x, synth.BF16)
    ln = (dev_bits(lc.gamma, synth.BF16), dev_bits(lc.beta, synth.BF16), lc.eps)
    y1 = torch.empty((4, 1024), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((4, 512), dtype=torch.bfloat16, device="cuda")
    y3 = torch.empty((4, 1024), dtype=torch.float32, device="cuda")
    calls = [lambda: qlin_gateup_swiglu(xg, gq.q, uq.q, out=y1),
             lambda: qlin_linear(xl, lq.q, ln=ln, act=1, out=y2),
             lambda: qlin_gateup_swiglu(xg, gq.q, uq.q, out=y3)]
    _replays_match(calls, [y1, y2, y3])


def test_graph_replay_stream_read():
    from decode_linear_amd import qlin_stream_read
    buf = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    part = torch.zeros(1024, dtype=torch.int32, device="cuda")
    _replays_match([lambda: qlin_stream_read(buf, part)], [part])
