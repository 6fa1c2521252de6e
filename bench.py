"""Benchmark of the decode-time fused quantized linear on one MI355X.

Metric: weight-stream HBM GB/s (and % of the 8 TB/s MI355X peak) and us per fused call.
The headline workload is the largest single call, the 4-bit SwiGLU gate+up projection
(M=4 rows, K=4096, N=14336 per projection, affine group 64, fp16 scale/bias).  One
"step" is one qlin_gateup_swiglu call over one batch of synthetic input.

Weight bytes per call are the algorithmic weight stream: codes + scales + biases of both
projections, each byte read once (activations and outputs are reported separately).
Weights rotate over enough copies to total >= 1 GiB, so the 256 MB Infinity Cache cannot
serve them; everything is resident in HBM before the timed region.  The timed steps are
captured into one HIP graph (after eager warmup steps and one untimed replay) and replayed
several times, each replay bracketed by HIP events on the stream the graph runs on, with
device synchronization on both sides: that is the GPU time of the calls, without the
~10 us of host work a Python call costs.  The headline value is the median over the
replays; p10 / median / p90 are reported with it (us_per_call_stats).  Also reported: the
same steps launched eagerly from Python (us_per_call_eager) and on one weight set that
stays cache-resident (us_per_call_warm).

read_ceiling: the library's plain streaming read (qlin_stream_read_config, 16-byte loads
and nothing else) over the same number of bytes, rotated and timed the same way, the best
of a small sweep of launches (grid, loads in flight, non-temporal or not): the rate a pure
read of that size reaches on this device.

Also reported: the headline workload at one shard's shape of an 8-way split along N (1792
rows per projection), the other workloads (plain fp16 linear, LN+GELU 8-bit, LN+residual
8-bit with 32 rows), the 124-pass LN+linear chain (hipGraph replay vs eager launches), the
whole MLP around the headline projection (qlin_mlp: gate/up then down with the residual),
one attend pass, one sampling step (qlin_sample), one quantized-KV decode attention step
(qlin_kvq_decode), and a CPU baseline: the fp64 oracle timed on the host on a bounded
sample of the workload, on one thread and on every host core (the core count and CPU model
are reported).

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--no-cpu] [--only-main]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
ROTATE_BYTES = 1 << 30         # weights rotate over at least this many bytes
METRIC = "weight-stream HBM GB/s and % of MI355X peak; µs per fused linear call"


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only-main", action="store_true", help="time only the headline workload")
    ap.add_argument("--only", default="", help="comma-separated labels of the secondary workloads to time "
                    "(swiglu-shard8, linear-config-1..3, chain, mlp, attend, sample, kvq); default all")
    ap.add_argument("--path", type=int, default=0, choices=(0, 1, 2),
                    help="kernel family for the quantized calls (qlin_set_path): 0 the library's choice, "
                    "1 the general kernel, 2 the vector-ALU kernel where it applies (for A/B runs)")
    ap.add_argument("--path-ab", action="store_true",
                    help="instead: time the SwiGLU (4-bit, K=4096, N=14336) and LN+GELU (8-bit, K=2048, "
                    "N=8192) calls at T = 1..4 on each kernel family (qlin_set_path 0, 2, 1) and exit")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target wall time of the CPU baseline")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="instead: run a plain device copy of this many bytes (counter calibration) and exit")
    return ap.parse_args()


def _torch():
    import torch
    return torch


def _time_calls(fn, n_copies, steps, warmup):
    """Run fn(i) for warmup then timed steps (i cycles over the weight copies); returns
    total ms of the timed steps from events on the current stream."""
    torch = _torch()
    for i in range(warmup):
        fn(i % n_copies)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn((warmup + i) % n_copies)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end)


def _time_graph(fn, n_copies, steps, warmup, replays=1):
    """Warmup calls eagerly, then exactly `steps` calls (cycling over the weight copies)
    captured into one HIP graph; one untimed replay uploads it, then `replays` timed replays
    run the steps back to back, each bracketed by events on the stream the graph runs on.
    Returns the ms of each timed replay (GPU time of the calls, without per-call host
    overhead)."""
    torch = _torch()
    for i in range(warmup):
        fn(i % n_copies)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn((warmup + i) % n_copies)
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(replays):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        g.replay()
        end.record()
        torch.cuda.synchronize()
        out.append(start.elapsed_time(end))
    del g
    return out


def _stats(us_list):
    """p10 / median / p90 of per-call microseconds over the replays."""
    a = np.sort(np.asarray(us_list, dtype=np.float64))
    return dict(p10=round(float(np.quantile(a, 0.1)), 3), median=round(float(np.median(a)), 3),
                p90=round(float(np.quantile(a, 0.9)), 3), replays=int(a.size))


# (blocks of 512 threads, loads in flight per thread, non-temporal): the launches of the
# plain streaming read the ceiling takes the best of
READ_SWEEP = [(256, 4, True), (256, 4, False), (512, 4, True), (256, 8, True), (1024, 8, True), (1024, 16, False),
              (1024, 16, True)]


def read_ceiling(nbytes, steps, warmup):
    """The device's streaming-read rate over nbytes: the best of a small sweep of launches of
    the library's plain 16-byte read (qlin_stream_read_config: no work beyond the loads),
    rotated over >= 1 GiB of buffers and timed like the fused calls.  The ceiling depends on
    the size (the launch's fixed cost weighs more on small reads): it is reported for this
    size only."""
    from decode_linear_amd import qlin_stream_read_config
    torch = _torch()
    nbytes = -(-nbytes // 16) * 16
    n_copies = max(2, -(-ROTATE_BYTES // nbytes))
    bufs = [torch.full((nbytes // 4,), i + 1, dtype=torch.int32, device="cuda") for i in range(n_copies)]
    part = torch.zeros(1024, dtype=torch.int32, device="cuda")
    sweep = []
    for blocks, unroll, nt in READ_SWEEP:
        ms = _time_graph(lambda i: qlin_stream_read_config(bufs[i], blocks, unroll, nt, part), n_copies, steps, warmup,
                         replays=3)
        us = min(ms) * 1e3 / steps
        sweep.append(dict(blocks=blocks, unroll=unroll, nontemporal=nt, us=round(us, 3)))
    best = min(sweep, key=lambda r: r["us"])
    del bufs
    return dict(bytes=nbytes, copies=n_copies, us=best["us"], gbs=nbytes / (best["us"] * 1e-6) / 1e9,
                best=best, sweep=sweep)


def _rotated(make, nbytes):
    """Enough independent copies of a weight set to total >= ROTATE_BYTES."""
    n = max(2, -(-ROTATE_BYTES // nbytes))
    first = make()
    return [first] + [tuple(w.clone() for w in first) if isinstance(first, tuple) else first.clone()
                      for _ in range(n - 1)]


def _clone_q(q):
    from decode_linear_amd import QWeight
    return QWeight(q.bits, q.N, q.K, q.data.clone(), None if q.scales is None else q.scales.clone(),
                   None if q.biases is None else q.biases.clone())


def _dev(bits_arr, dtype):
    torch = _torch()
    import synth
    if dtype == synth.F32:
        return torch.from_numpy(np.ascontiguousarray(bits_arr, np.float32)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(bits_arr, np.uint16).view(np.int16))
    return t.view(torch.float16 if dtype == synth.F16 else torch.bfloat16).cuda()


def _pack(w_f32, bits):
    from decode_linear_amd import qlin_pack_affine
    torch = _torch()
    wd = torch.from_numpy(w_f32).cuda()
    q = qlin_pack_affine(wd, bits)
    del wd
    return q


def bench_swiglu(steps, warmup, n_override=None, replays=7):
    """The headline workload (or its N cut to one shard's rows per projection): cold (weights
    rotated over >= 1 GiB) p10/median/p90 over graph replays, eager, and warm (one weight
    set, MALL-resident)."""
    import synth
    from decode_linear_amd import qlin_gateup_swiglu
    torch = _torch()
    case = synth.workload(4, scale_n=n_override)
    g0, u0 = _pack(case.gate, 4), _pack(case.up, 4)
    del case.gate, case.up
    wbytes = g0.nbytes + u0.nbytes
    n_copies = max(2, -(-ROTATE_BYTES // wbytes))
    weights = [(g0, u0)] + [(_clone_q(g0), _clone_q(u0)) for _ in range(n_copies - 1)]
    x = _dev(case.x, case.x_dtype)
    y = torch.empty((case.T, case.N), dtype=torch.bfloat16, device="cuda")

    def step(i):
        g, u = weights[i]
        qlin_gateup_swiglu(x, g, u, out=y)

    per = [ms * 1e3 / steps for ms in _time_graph(step, n_copies, steps, warmup, replays=replays)]
    st = _stats(per)
    us_eager = _time_calls(step, n_copies, steps, warmup) * 1e3 / steps
    warm = [ms * 1e3 / steps for ms in _time_graph(step, 1, steps, warmup, replays=3)]
    other = case.x.size * 2 + y.numel() * 2
    name = case.name if n_override is None else f"{case.name}-shard{14336 // case.N}"
    return dict(name=name, T=case.T, K=case.K, N=case.N, bits=4, weight_bytes=wbytes, other_bytes=other,
                copies=n_copies, us=st["median"], us_stats=st, gbs=wbytes / (st["median"] * 1e-6) / 1e9,
                us_eager=us_eager, us_warm=round(float(np.median(warm)), 3))


def bench_linear(c, steps, warmup):
    import synth
    from decode_linear_amd import QWeight, qlin_linear
    torch = _torch()
    case = synth.workload(c)
    if case.bits == 16:
        q0 = QWeight(16, case.N, case.K, _dev(case.w_dense, case.w_dtype))
    else:
        q0 = _pack(case.w_f32, case.bits)
    wbytes = q0.nbytes
    n_copies = max(2, -(-ROTATE_BYTES // wbytes))
    weights = [q0] + [_clone_q(q0) for _ in range(n_copies - 1)]
    x = _dev(case.x, case.x_dtype)
    ln = None if case.gamma is None else (_dev(case.gamma, case.x_dtype), _dev(case.beta, case.x_dtype), case.eps)
    res = None if case.res is None else _dev(case.res, case.x_dtype)
    y = torch.empty((case.T, case.N), dtype=torch.float16 if case.y_dtype == synth.F16 else torch.bfloat16,
                    device="cuda")

    def step(i):
        qlin_linear(x, weights[i], ln=ln, act=case.act, residual=res, out=y)

    st = _stats([ms * 1e3 / steps for ms in _time_graph(step, n_copies, steps, warmup, replays=5)])
    us = st["median"]
    us_eager = _time_calls(step, n_copies, steps, warmup) * 1e3 / steps
    us_warm = float(np.median([ms * 1e3 / steps for ms in _time_graph(step, 1, steps, warmup, replays=3)]))
    return dict(name=case.name, T=case.T, K=case.K, N=case.N, bits=case.bits, weight_bytes=wbytes, copies=n_copies,
                us=us, us_stats=st, gbs=wbytes / (us * 1e-6) / 1e9, us_eager=us_eager, us_warm=us_warm)


def bench_mlp(steps, warmup):
    """The MLP around the headline workload (qlin_mlp: gate/up 4-bit K=4096 I=14336, then the
    4-bit down projection Hout=4096 with the residual), weights rotated like the others."""
    import synth
    from decode_linear_amd import qlin_mlp
    torch = _torch()
    case = synth.mlp_workload()
    g0, u0, d0 = _pack(case.gate, 4), _pack(case.up, 4), _pack(case.down, 4)
    del case.gate, case.up, case.down
    wbytes = g0.nbytes + u0.nbytes + d0.nbytes
    n_copies = max(2, -(-ROTATE_BYTES // wbytes))
    weights = [(g0, u0, d0)] + [tuple(_clone_q(q) for q in (g0, u0, d0)) for _ in range(n_copies - 1)]
    x = _dev(case.x, case.x_dtype)
    res = _dev(case.res, case.x_dtype)
    h = torch.empty((case.T, case.I), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((case.T, case.Hout), dtype=torch.bfloat16, device="cuda")

    def step(i):
        qlin_mlp(x, *weights[i], residual=res, h=h, out=y)

    st = _stats([ms * 1e3 / steps for ms in _time_graph(step, n_copies, steps, warmup, replays=5)])
    us = st["median"]
    us_eager = _time_calls(step, n_copies, steps, warmup) * 1e3 / steps
    return dict(name=case.name, T=case.T, K=case.K, I=case.I, Hout=case.Hout, bits=4, weight_bytes=wbytes,
                copies=n_copies, dispatches=2, us=us, us_stats=st, gbs=wbytes / (us * 1e-6) / 1e9, us_eager=us_eager)


def bench_attend(steps, warmup):
    """One attend pass of the depth decoder's band (16 heads of 64, 24 cached + 8 new
    positions, bf16): ~300 KB per call, so it is bound by latency and stays cache-resident;
    bytes are qkv + cache read, extended cache + output written."""
    import synth
    from decode_linear_amd import qlin_attend
    torch = _torch()
    case = synth.attend_workload()
    qkv, kv = _dev(case.qkv, case.dtype), _dev(case.kv, case.dtype)
    D = case.H * case.HD
    out = torch.empty((case.T, D), dtype=torch.bfloat16, device="cuda")
    kv_out = torch.empty((2, case.H, case.P + case.T, case.HD), dtype=torch.bfloat16, device="cuda")

    def step(i):
        qlin_attend(qkv, kv, case.H, case.HD, out=out, kv_out=kv_out)

    us = _time_graph(step, 1, steps, warmup)[0] * 1e3 / steps
    nbytes = (qkv.numel() + kv.numel() + kv_out.numel() + out.numel()) * 2
    return dict(name=case.name, H=case.H, HD=case.HD, P=case.P, T=case.T, bytes=nbytes, us=us,
                gbs=nbytes / (us * 1e-6) / 1e9, bound="latency")


def bench_sample(steps, warmup):
    """One sampling step of the depth decoder (qlin_sample: 2048 bf16 logits, top-64,
    Gumbel-max, a 1024-wide bf16 embedding row appended to a 16-row prefix): latency-bound,
    cache-resident; bytes are logits, noise row, prefix and table row read, rows written."""
    import synth
    from decode_linear_amd import qlin_sample
    torch = _torch()
    case = synth.sample_workload()
    lg = _dev(case.logits, case.logit_dtype)
    g = torch.from_numpy(case.gumbel).cuda()
    tb = _dev(case.table, case.emb_dtype)
    pre = _dev(case.prefix, case.emb_dtype)
    n_prev = case.prefix.shape[0]
    out = torch.empty((n_prev + 1, case.D), dtype=torch.bfloat16, device="cuda")
    code = torch.empty(1, dtype=torch.int32, device="cuda")

    def step(i):
        qlin_sample(lg, g, 1, tb, pre, 1.0 / 0.9, 64, out=out, code=code)

    us = _time_graph(step, 1, steps, warmup)[0] * 1e3 / steps
    nbytes = case.n * (2 + 4) + (2 * n_prev + 2) * case.D * 2 + 4
    return dict(name=case.name, n=case.n, D=case.D, n_prev=n_prev, top_k=64, bytes=nbytes, us=us,
                gbs=nbytes / (us * 1e-6) / 1e9, bound="latency")


def bench_kvq(steps, warmup):
    """One decode step of attention over a quantized K/V cache (qlin_kvq_decode: 16 query
    heads on 8 KV heads, head_dim 256, 8192 rows, 4-bit groups of 64), the cache rotated over
    >= 1 GiB of copies; bytes are the cache (codes, scales, biases of K and V, read once
    each), q and the output."""
    import synth
    from decode_linear_amd import qlin_kvq_decode
    torch = _torch()
    c = synth.kvq_workload()
    q = _dev(c.q, c.q_dtype)

    def dev_cache(t):
        return (torch.from_numpy(t[0].view(np.int32)).cuda(), _dev(t[1], c.sb_dtype), _dev(t[2], c.sb_dtype))
    k0, v0 = dev_cache(c.k), dev_cache(c.v)
    cache_bytes = sum(t.numel() * t.element_size() for t in k0 + v0)
    n_copies = max(2, -(-ROTATE_BYTES // cache_bytes))
    caches = [(k0, v0)] + [(tuple(t.clone() for t in k0), tuple(t.clone() for t in v0)) for _ in range(n_copies - 1)]
    out = torch.empty((c.H, c.D), dtype=torch.bfloat16, device="cuda")
    from decode_linear_amd.qlin import lib
    ws = torch.empty(int(lib().qlin_kvq_decode_workspace(c.H, c.N, c.D)) // 4, dtype=torch.float32, device="cuda")

    def step(i):
        qlin_kvq_decode(q, caches[i][0], caches[i][1], c.KV, c.GS, c.bits, out=out, workspace=ws)

    us = _time_graph(step, n_copies, steps, warmup)[0] * 1e3 / steps
    nbytes = cache_bytes + 2 * c.H * c.D * 2
    return dict(name=c.name, H=c.H, KV=c.KV, N=c.N, D=c.D, bits=c.bits, group=c.GS, cache_bytes=cache_bytes,
                copies=n_copies, dispatches=2, us=us, gbs=nbytes / (us * 1e-6) / 1e9)


def bench_chain(replays, warmup):
    """124 dependent LN + linear passes (8-bit, K=N=1024, T = 1 + p mod 8): graph replay
    and eager launches, rotated over >= 1 GiB of chain copies."""
    import synth
    from decode_linear_amd import QlinChain, qlin_linear
    torch = _torch()
    P = synth.CHAIN_PASSES
    B0 = _dev(synth.chain_buffers(), synth.BF16)
    base = []
    for p in range(P):
        w, g, b = synth.chain_pass(p)
        base.append((_pack(w, 8), _dev(g, synth.BF16), _dev(b, synth.BF16)))
    chain_bytes = sum(q.nbytes for q, _, _ in base)
    n_copies = max(2, -(-ROTATE_BYTES // chain_bytes))
    copies = [base] + [[(_clone_q(q), g, b) for q, g, b in base] for _ in range(n_copies - 1)]
    bufs = [B0.clone() for _ in range(n_copies)]
    chains = []
    for cp, B in zip(copies, bufs):
        ps = [dict(x=B[p, :synth.chain_T(p)], T=synth.chain_T(p), w=q, ln=(g, b, 1e-5), y=B[p + 1, :synth.chain_T(p)])
              for p, (q, g, b) in enumerate(cp)]
        chains.append(QlinChain(ps, torch.bfloat16, torch.bfloat16))
    ms_graph = _time_calls(lambda i: chains[i].launch(), n_copies, replays, warmup)

    def eager(i):
        B = bufs[i]
        for p, (q, g, b) in enumerate(copies[i]):
            T = synth.chain_T(p)
            qlin_linear(B[p, :T], q, ln=(g, b, 1e-5), out=B[p + 1, :T])

    ms_eager = _time_calls(eager, n_copies, max(1, replays // 2), max(1, warmup // 2))
    for ch in chains:
        ch.close()
    us_graph = ms_graph * 1e3 / replays / P
    us_eager = ms_eager * 1e3 / max(1, replays // 2) / P
    per_pass = chain_bytes / P
    return dict(name="chain-124-ln-q8-K1024-N1024", passes=P, weight_bytes_per_pass=per_pass, copies=n_copies,
                us_per_pass_graph=us_graph, us_per_pass_eager=us_eager,
                us_per_frame_graph=us_graph * P, gbs_graph=per_pass / (us_graph * 1e-6) / 1e9)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(target_s):
    """The oracle (plain fp64 C++, untuned) on the host: the SwiGLU workload restricted to
    its first Ns output rows per projection, called repeatedly on one thread and then from
    one thread per host core until about target_s seconds of wall time in all; reported in
    weight GB/s of that sample (the all-core rate is the value)."""
    import oracle
    import synth
    case = synth.workload(4, scale_n=1024)      # same distributions; N cut to the sample
    gw = oracle.pack_affine(case.gate, 4)
    uw = oracle.pack_affine(case.up, 4)
    Ns, K = case.N, case.K
    wbytes = 2 * (Ns * K // 2 + 2 * Ns * (K // 64) * 2)
    t0 = time.time()
    oracle.gateup(case.x, case.x_dtype, 4, gw[:3], uw[:3])
    one = time.time() - t0

    def run(threads, seconds):
        per_thread = max(1, int(seconds / max(one, 1e-3) / 1.2 / (1 if threads == 1 else 1)))
        done = [0] * threads

        def work(k):
            for _ in range(per_thread):
                oracle.gateup(case.x, case.x_dtype, 4, gw[:3], uw[:3])
                done[k] += 1
        t0 = time.time()
        ts = [threading.Thread(target=work, args=(k,)) for k in range(threads)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        wall = time.time() - t0
        return sum(done), wall

    cores = os.cpu_count() or 1
    c1, w1 = run(1, target_s * 0.3)
    cn, wn = run(cores, target_s * 0.7)
    return {"value": round(cn * wbytes / wn / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"SwiGLU workload cut to N={Ns} rows per projection (K=4096, 4-bit): {cn} oracle calls on "
                      f"{cores} host threads in {wn:.1f} s, and {c1} calls on 1 thread in {w1:.1f} s",
            "value_1_thread": round(c1 * wbytes / w1 / 1e9, 4), "cpu_model": _cpu_model(),
            "us_per_call_full_workload_est_1_thread": round(w1 / c1 * (14336 / Ns) * 1e6, 1)}


def path_ab(steps, warmup):
    """The kernel-family A/B: the SwiGLU projection (4-bit, K=4096, N=14336 per projection) and
    the LN + GELU linear (8-bit, K=2048, N=8192) at T = 1..4 rows, each timed on the int8
    matrix-core kernel (path 0), the vector-ALU kernel (path 2) and the general kernel (path
    1), cold (weights rotated over >= 1 GiB), median over graph replays.  The dispatch
    counters confirm which family ran."""
    import synth
    from decode_linear_amd import qlin_dispatch_count, qlin_gateup_swiglu, qlin_linear, qlin_set_path
    torch = _torch()
    c4 = synth.workload(4)
    g0, u0 = _pack(c4.gate, 4), _pack(c4.up, 4)
    n4 = max(2, -(-ROTATE_BYTES // (g0.nbytes + u0.nbytes)))
    w4 = [(g0, u0)] + [(_clone_q(g0), _clone_q(u0)) for _ in range(n4 - 1)]
    c2 = synth.workload(2)
    q2 = _pack(c2.w_f32, 8)
    n2 = max(2, -(-ROTATE_BYTES // q2.nbytes))
    w2 = [q2] + [_clone_q(q2) for _ in range(n2 - 1)]
    ln2 = (_dev(c2.gamma, c2.x_dtype), _dev(c2.beta, c2.x_dtype), c2.eps)
    gen = torch.Generator(device="cuda").manual_seed(7)
    rows = []
    for T in (1, 2, 3, 4):
        x4 = torch.randn((T, c4.K), device="cuda", generator=gen).to(torch.bfloat16)
        y4 = torch.empty((T, c4.N), dtype=torch.bfloat16, device="cuda")
        x2 = (torch.randn((T, c2.K), device="cuda", generator=gen) + 3.0).to(torch.bfloat16)
        y2 = torch.empty((T, c2.N), dtype=torch.bfloat16, device="cuda")
        for path in (0, 2, 1):
            prev = qlin_set_path(path)
            try:
                before = [qlin_dispatch_count(i) for i in (0, 1, 8, 9)]
                ms = _time_graph(lambda i: qlin_gateup_swiglu(x4, w4[i][0], w4[i][1], out=y4), n4, steps, warmup,
                                 replays=5)
                swiglu = float(np.median(ms)) * 1e3 / steps
                ms = _time_graph(lambda i: qlin_linear(x2, w2[i], ln=ln2, act=1, out=y2), n2, steps, warmup, replays=5)
                lngelu = float(np.median(ms)) * 1e3 / steps
                after = [qlin_dispatch_count(i) for i in (0, 1, 8, 9)]
            finally:
                qlin_set_path(prev)
            calls = after[0] + after[1] - before[0] - before[1]
            fam = ("int8-mfma" if after[2] - before[2] == calls else "valu" if after[3] - before[3] == calls
                   else "general" if after[2] == before[2] and after[3] == before[3] else "mixed")
            rows.append(dict(T=T, path=path, family=fam, swiglu_us=round(swiglu, 3), ln_gelu_us=round(lngelu, 3)))
    print(json.dumps({"path_ab": rows, "swiglu": c4.name, "ln_gelu": c2.name, "steps": steps}))


def copy_probe(nbytes):
    torch = _torch()
    a = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes}))


def measured_traffic():
    """HBM bytes per call of the headline kernel from the committed counter record
    (profiles/traffic.json: FETCH_SIZE and WRITE_SIZE scaled by a plain copy's readings),
    or None once the kernel sources differ from those the counters were taken on."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in rec["source_files"]:
        fp = os.path.join(ROOT, f)
        if not os.path.exists(fp):   # a source the counters were taken on is gone: stale
            return None
        with open(fp, "rb") as fh:
            h.update(fh.read())
    return rec["traffic_bytes"] if h.hexdigest() == rec["source_sha256"] else None


def main():
    a = _args()
    if a.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU: the library has no multi-GPU path; --gpus must be 1",
                          "n_gpus_requested": a.gpus}))
        sys.exit(2)
    from decode_linear_amd import build
    build.ensure_built()
    torch = _torch()
    torch.cuda.init()
    if a.copy_probe:
        copy_probe(a.copy_probe)
        return
    if a.path_ab:
        path_ab(a.steps, a.warmup)
        return
    if a.path:
        from decode_linear_amd import qlin_set_path
        qlin_set_path(a.path)
    main_r = bench_swiglu(a.steps, a.warmup)
    ceil_r = read_ceiling(main_r["weight_bytes"], a.steps, a.warmup)
    extra = {}
    if not a.only_main:
        # each secondary workload is reported on its own: one that fails records its error
        # and does not take the headline line down with it
        runs = [("swiglu-shard8", lambda: bench_swiglu(a.steps, a.warmup, n_override=14336 // 8, replays=5))]
        runs += [(f"linear-config-{c}", lambda c=c: bench_linear(c, a.steps, a.warmup)) for c in (1, 2, 3)]
        runs += [("chain", lambda: bench_chain(max(4, a.steps // 10), max(2, a.warmup // 4))),
                 ("mlp", lambda: bench_mlp(a.steps, a.warmup)), ("attend", lambda: bench_attend(a.steps, a.warmup)),
                 ("sample", lambda: bench_sample(a.steps, a.warmup)), ("kvq", lambda: bench_kvq(a.steps, a.warmup))]
        if a.only:
            keep = set(a.only.split(","))
            runs = [r for r in runs if r[0] in keep]
        for label, run in runs:
            try:
                r = run()
            except Exception as exc:   # reported, not hidden: the line carries the error
                extra[label] = {"error": f"{type(exc).__name__}: {exc}"}
                continue
            extra[r["name"]] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items() if k != "name"}
            if label == "swiglu-shard8":
                extra[r["name"]]["note"] = "one shard of an 8-way split along N (N = 1792 per projection)"
            if "gbs" in r:
                extra[r["name"]]["pct_peak"] = round(100 * r["gbs"] / PEAK_HBM_GBS, 2)
    us = main_r["us"]
    achieved = main_r["weight_bytes"] / (us * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": round(main_r["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "kernel_path": a.path,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": main_r["name"], "rows": main_r["T"], "K": main_r["K"], "N_per_projection": main_r["N"],
                   "weights": "4-bit affine, group 64, fp16 scale/bias", "activations": "bf16",
                   "weight_bytes_per_call": main_r["weight_bytes"], "rotation_copies": main_r["copies"]},
        "us_per_call": round(us, 3),
        "us_per_call_stats": main_r["us_stats"],
        "us_per_call_eager": round(main_r["us_eager"], 3),
        "us_per_call_warm": main_r["us_warm"],
        "pct_peak": round(100 * achieved / PEAK_HBM_GBS, 2),
        "read_ceiling": {"gbs": round(ceil_r["gbs"], 2), "us": round(ceil_r["us"], 3), "bytes": ceil_r["bytes"],
                         "frac_of_peak": round(ceil_r["gbs"] / PEAK_HBM_GBS, 4),
                         "fused_frac_of_ceiling": round(achieved / ceil_r["gbs"], 4),
                         "best_launch": ceil_r["best"], "sweep": ceil_r["sweep"],
                         "note": "plain 16-byte reads of the same byte count; size-dependent"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic()},
    }
    if extra:
        line["workloads"] = extra
    if not a.no_cpu:
        line["cpu_baseline"] = cpu_baseline(a.cpu_seconds)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
