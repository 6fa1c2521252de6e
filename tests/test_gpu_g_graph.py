"""GPU: calls of every compute entry point (fused linear, gate/up, MLP, attend, sample,
quantized-KV decode, streaming read) captured into a HIP graph (the way the bench times
them) give, on every replay, the bits the same calls give when launched eagerly.  Replays are separated by eager
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


def test_graph_replay_mlp():
    # the long-K down projection (K = I = 8192 > the streaming windows) with the residual
    from decode_linear_amd import qlin_mlp
    c = synth.random_mlp(7003, 4, 1024, 8192, 512, 4, res=True)
    gq, uq, dq = (Packed(a, 4) for a in (c.gate, c.up, c.down))
    x, res = dev_bits(c.x, synth.BF16), dev_bits(c.res, synth.BF16)
    h = torch.empty((4, 8192), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((4, 512), dtype=torch.bfloat16, device="cuda")
    _replays_match([lambda: qlin_mlp(x, gq.q, uq.q, dq.q, residual=res, h=h, out=y)], [h, y])


def test_graph_replay_attend():
    from decode_linear_amd import qlin_attend
    c = synth.attend_workload()
    qkv, kv = dev_bits(c.qkv, c.dtype), dev_bits(c.kv, c.dtype)
    out = torch.empty((c.T, c.H * c.HD), dtype=torch.bfloat16, device="cuda")
    kv_out = torch.empty((2, c.H, c.P + c.T, c.HD), dtype=torch.bfloat16, device="cuda")
    _replays_match([lambda: qlin_attend(qkv, kv, c.H, c.HD, out=out, kv_out=kv_out)], [out, kv_out])


def test_graph_replay_sample():
    from decode_linear_amd import qlin_sample
    c = synth.sample_workload()
    lg = dev_bits(c.logits, c.logit_dtype)
    g = torch.from_numpy(c.gumbel).cuda()
    tb, pre = dev_bits(c.table, c.emb_dtype), dev_bits(c.prefix, c.emb_dtype)
    out = torch.empty((c.prefix.shape[0] + 1, c.D), dtype=torch.bfloat16, device="cuda")
    code = torch.empty(1, dtype=torch.int32, device="cuda")
    _replays_match([lambda: qlin_sample(lg, g, 1, tb, pre, 1.0 / 0.9, 64, out=out, code=code)], [out, code])


def test_graph_replay_kvq_decode():
    from decode_linear_amd import qlin_kvq_decode
    from decode_linear_amd.qlin import lib
    c = synth.kvq_case(7004, 4, 2, 5000, 128, 64, 4)
    q = dev_bits(c.q, c.q_dtype)

    def cache(t):
        return (torch.from_numpy(t[0].view(np.int32)).cuda(), dev_bits(t[1], c.sb_dtype), dev_bits(t[2], c.sb_dtype))
    k, v = cache(c.k), cache(c.v)
    ws = torch.empty(int(lib().qlin_kvq_decode_workspace(c.H, c.N, c.D)) // 4, dtype=torch.float32, device="cuda")
    out = torch.empty((c.H, c.D), dtype=torch.bfloat16, device="cuda")
    _replays_match([lambda: qlin_kvq_decode(q, k, v, c.KV, c.GS, c.bits, out=out, workspace=ws)], [out])
