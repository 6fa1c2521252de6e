"""GPU parity of qlin_attend against the oracle ([p1] `_ATTEND` / `attend()`).

kv_out (the cache with this pass's keys and values appended) must equal the oracle's bit
for bit.  The attention output is held to the gates of the linear path: the fp32-output
run within 2e-3 (Gate A), and a 16-bit output equal to RNE of the fp32 output (Gate B).
Shapes span one to 32 positions, empty and full caches, one head to many, head_dim 16 to
512, fp16 and bf16, and the last-row mode."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TORCH_DT, dev_bits, gate_a, gate_b, host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from decode_linear_amd import build
    build.ensure_built()


def _run(case: synth.AttendCase, last=False, out_dtypes=(synth.F32, None)):
    from decode_linear_amd import qlin_attend
    print(f"attend case {case.name} last={last}", flush=True)
    qkv = dev_bits(case.qkv, case.dtype)
    kv = None if case.kv is None else dev_bits(case.kv, case.dtype)
    y64, kv64 = oracle.attend(case.qkv, case.kv, case.dtype, case.H, case.HD, last=last)
    outs = {}
    for od in out_dtypes:
        od = case.dtype if od is None else od
        out, kv_out = qlin_attend(qkv, kv, case.H, case.HD, last=last, out_dtype=TORCH_DT[od])
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(kv_out), kv64), f"{case.name}: kv_out differs from the oracle"
        outs[od] = out
    y32 = outs[synth.F32]
    gate_a(y32, y64, what=case.name)
    if case.dtype in outs:
        gate_b(outs[case.dtype], y32, y64, case.dtype, what=case.name)
    return y32


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F16])
@pytest.mark.parametrize("P,T", [(0, 1), (0, 8), (24, 8), (31, 1), (0, 32), (5, 27), (16, 3)])
def test_attend_positions(dtype, P, T):
    _run(synth.attend_case(10 + P + T, 16, 64, P, T, dtype))


@pytest.mark.parametrize("H,HD", [(1, 16), (3, 48), (8, 128), (2, 512), (40, 32)])
def test_attend_heads(H, HD):
    _run(synth.attend_case(20 + H + HD, H, HD, 9, 4))


@pytest.mark.parametrize("P,T", [(0, 1), (12, 5), (30, 2)])
def test_attend_last(P, T):
    case = synth.attend_case(30 + P, 4, 64, P, T)
    y_all = _run(case)
    y_last = _run(case, last=True)
    assert torch.equal(y_last[0], y_all[-1])


def test_attend_workload_shape_and_determinism():
    from decode_linear_amd import qlin_attend
    case = synth.attend_workload()
    _run(case)
    qkv, kv = dev_bits(case.qkv, case.dtype), dev_bits(case.kv, case.dtype)
    a, ka = qlin_attend(qkv, kv, case.H, case.HD)
    b, kb = qlin_attend(qkv, kv, case.H, case.HD)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(ka.view(torch.int16), kb.view(torch.int16))


def test_attend_large_scores():
    # queries scaled by 32 (exactly): scores reach about a hundred, past fp32's exp range
    # unless the softmax subtracts the maximum first
    case = synth.attend_case(40, 2, 64, 6, 3)
    D = case.H * case.HD
    q = oracle.widen(case.qkv[:, :D], case.dtype)
    case.qkv[:, :D] = oracle.round_to(32.0 * q, case.dtype)
    _run(case)


def test_attend_dispatch_count():
    from decode_linear_amd import qlin_attend, qlin_dispatch_count
    case = synth.attend_case(50, 2, 32, 3, 2)
    before = qlin_dispatch_count(4)
    qlin_attend(dev_bits(case.qkv, case.dtype), dev_bits(case.kv, case.dtype), case.H, case.HD)
    torch.cuda.synchronize()
    assert qlin_dispatch_count(4) == before + 1
