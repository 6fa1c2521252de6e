"""A fresh process whose FIRST call of each library entry point happens inside a HIP graph
capture (torch.cuda.graph): no lazy set-up of the library (device queries, the static
scratch's address, kernel loading) may break the capture or be left out of the graph.
The graph is then replayed three times, with unrelated eager work and a refill of every
output between replays, and each replay must equal the same calls made eagerly, bit for
bit.  Inputs are random tensors of the library's formats (no oracle involved: the parity
of each call is checked elsewhere; this checks capture)."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r'''
import sys
import torch
import decode_linear_amd as q

torch.cuda.init()
dev = torch.device("cuda:0")
g = torch.Generator(device=dev).manual_seed(1234)

def rnd(shape, dtype, sd=1.0, mean=0.0):
    return (torch.randn(shape, generator=g, device=dev) * sd + mean).to(dtype)

def weight(N, K, bits):
    words = torch.randint(-2**31, 2**31 - 1, (N, K * bits // 32), dtype=torch.int32, device=dev, generator=g)
    s = (torch.rand((N, K // 64), device=dev, generator=g) * 0.002 + 0.0005).half()
    b = (torch.randn((N, K // 64), device=dev, generator=g) * 0.01).half()
    return q.QWeight(bits, N, K, words, s, b)

bf = torch.bfloat16
x4 = rnd((4, 1024), bf)
W4, W8 = weight(256, 1024, 4), weight(256, 1024, 8)
gam, bet = rnd((1024,), bf, 0.1, 1.0), rnd((1024,), bf, 0.1)
Gt, Up, Dn = weight(512, 1024, 4), weight(512, 1024, 4), weight(1024, 512, 4)
res = rnd((4, 1024), bf)
qkv = rnd((8, 3 * 4 * 64), bf)
kv = rnd((2, 4, 16, 64), bf)
logits = rnd((1024,), torch.float32, 2.0)
gumbel = -torch.log(-torch.log(torch.rand((1, 1024), device=dev, generator=g).clamp(1e-6, 1 - 1e-6)))
table = rnd((1, 1024, 256), bf)
prefix = rnd((3, 256), bf)
H, KV, N, D = 8, 4, 700, 128
qh = rnd((H, D), bf)
kc = torch.randint(-2**31, 2**31 - 1, (KV, N, D * 4 // 32), dtype=torch.int32, device=dev, generator=g)
vc = torch.randint(-2**31, 2**31 - 1, (KV, N, D * 4 // 32), dtype=torch.int32, device=dev, generator=g)
ks, kb = (torch.rand((KV, N, D // 64), device=dev, generator=g) * 0.02).to(bf), rnd((KV, N, D // 64), bf, 0.05)
vs, vb = (torch.rand((KV, N, D // 64), device=dev, generator=g) * 0.02).to(bf), rnd((KV, N, D // 64), bf, 0.05)
ws = torch.empty(q.qlin.lib().qlin_kvq_decode_workspace(H, N, D) // 4, dtype=torch.float32, device=dev)
torch.cuda.synchronize()

def outputs():
    return dict(
        lin4=torch.empty((4, 256), dtype=torch.float32, device=dev),
        lin8ln=torch.empty((4, 256), dtype=bf, device=dev),
        gen=torch.empty((4, 256), dtype=torch.float32, device=dev),
        gu=torch.empty((4, 512), dtype=bf, device=dev),
        mlp_h=torch.empty((4, 512), dtype=bf, device=dev),
        mlp_y=torch.empty((4, 1024), dtype=bf, device=dev),
        att=torch.empty((8, 256), dtype=bf, device=dev),
        att_kv=torch.empty((2, 4, 24, 64), dtype=bf, device=dev),
        code=torch.empty((1,), dtype=torch.int32, device=dev),
        smp=torch.empty((4, 256), dtype=bf, device=dev),
        kvq=torch.empty((H, D), dtype=torch.float32, device=dev),
        kvq0=torch.empty((H, D), dtype=bf, device=dev),
    )

def calls(o):
    q.qlin_linear(x4, W4, out=o["lin4"])
    q.qlin_linear(x4, W8, ln=(gam, bet, 1e-5), act=q.QLIN_ACT_GELU, out=o["lin8ln"])
    prev = q.qlin_set_path(1)
    q.qlin_linear(x4, W4, residual=None, out=o["gen"])
    q.qlin_set_path(prev)
    q.qlin_gateup_swiglu(x4, Gt, Up, out=o["gu"])
    q.qlin_mlp(x4, Gt, Up, Dn, residual=res, h=o["mlp_h"], out=o["mlp_y"])
    q.qlin_attend(qkv, kv, 4, 64, out=o["att"], kv_out=o["att_kv"])
    q.qlin_sample(logits, gumbel, 0, table, prefix, 1.0, 64, out=o["smp"], code=o["code"])
    q.qlin_kvq_decode((qh), (kc, ks, kb), (vc, vs, vb), KV, 64, 4, out=o["kvq"], workspace=ws)
    q.qlin_kvq_decode_noalloc(qh, (kc, ks, kb), (vc, vs, vb), KV, 64, 4, o["kvq0"])

for i in range(9):
    assert q.qlin_dispatch_count(i) == 0, "a library kernel ran before the capture"
og = outputs()
graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph):
    calls(og)
counts = [q.qlin_dispatch_count(i) for i in range(9)]
print("captured; dispatch counts", counts, flush=True)

oe = outputs()
calls(oe)
torch.cuda.synchronize()

def bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)

for rep in range(3):
    for t in og.values():
        t.view(torch.uint8).fill_(0xA5)
    _ = (x4.float() * 3).sum().item()
    graph.replay()
    torch.cuda.synchronize()
    for name in og:
        assert torch.equal(bits(og[name]), bits(oe[name])), f"replay {rep}: {name} differs from the eager call"
    print(f"replay {rep} matches eager", flush=True)
print("capture-first ok", flush=True)
'''


def test_first_calls_inside_capture_in_fresh_process():
    env = dict(os.environ)
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    print("starting fresh process: first library calls inside graph capture", flush=True)
    r = subprocess.run([sys.executable, "-u", "-c", SCRIPT], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    print(r.stdout[-4000:])
    print(r.stderr[-4000:])
    assert r.returncode == 0, f"child exited {r.returncode}"
    assert "capture-first ok" in r.stdout
