"""The general kernel's merge waits are bounded; a wait that gives up must be observable:
its outputs become NaN and the device counter read by qlin_merge_timeouts rises.  The test
forces every wait to give up at once from the host (spin limit 0: no wait is actually
stuck, every kernel exits normally), then checks that with the default limit the same calls
are correct again and nothing is reported."""
import numpy as np
import pytest
import torch

import synth
from helpers import Packed, dev_bits, run_gateup_case, run_linear_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from decode_linear_amd import build
    build.ensure_built()


@pytest.fixture
def general():
    from decode_linear_amd import qlin_merge_timeouts, qlin_set_merge_spin_limit, qlin_set_path
    prev_path = qlin_set_path(1)
    prev_spin = qlin_set_merge_spin_limit(4194304)
    torch.cuda.synchronize()
    qlin_merge_timeouts(reset=True)
    yield
    qlin_set_merge_spin_limit(prev_spin)
    qlin_set_path(prev_path)
    torch.cuda.synchronize()
    qlin_merge_timeouts(reset=True)


@pytest.mark.parametrize("kind", ["q8-linear", "f16-dense", "q4-gateup"])
def test_forced_give_up_is_reported_as_nan(general, kind):
    from decode_linear_amd import (qlin_dispatch_count, qlin_gateup_swiglu, qlin_linear, qlin_merge_timeouts,
                                   qlin_set_merge_spin_limit)
    if kind == "q4-gateup":
        c = synth.random_gateup(7000, 4, 1024, 40, 4)
        G, U = Packed(c.gate, 4), Packed(c.up, 4)
        x = dev_bits(c.x, c.x_dtype)
        call = lambda: qlin_gateup_swiglu(x, G.q, U.q, out_dtype=torch.float32)
    else:
        bits = 8 if kind == "q8-linear" else 16
        c = synth.random_case(7001 + bits, 4, 1024, 64, bits, x_dtype=synth.BF16 if bits == 8 else synth.F16)
        W = Packed(c.w_f32, 8) if bits == 8 else Packed(bits=16, dense=c.w_dense, dense_dtype=c.w_dtype)
        x = dev_bits(c.x, c.x_dtype)
        call = lambda: qlin_linear(x, W.q, out_dtype=torch.float32)
    before = qlin_dispatch_count(8)
    good = call()
    torch.cuda.synchronize()
    assert torch.isfinite(good).all() and qlin_merge_timeouts() == 0
    qlin_set_merge_spin_limit(0)
    bad = call()
    torch.cuda.synchronize()
    n = qlin_merge_timeouts(reset=True)
    print(f"{kind}: {n} merge waits gave up with the spin limit at 0")
    assert n > 0
    assert torch.isnan(bad).all(), f"{int((~torch.isnan(bad)).sum())} outputs escaped the NaN report"
    qlin_set_merge_spin_limit(4194304)
    again = call()
    torch.cuda.synchronize()
    assert torch.equal(again, good) and qlin_merge_timeouts() == 0
    assert qlin_dispatch_count(8) == before   # the general kernel ran, not the int8 one


def test_default_limit_keeps_parity(general):
    from decode_linear_amd import qlin_merge_timeouts
    run_linear_case(synth.random_case(7010, 5, 2048, 100, 8, x_dtype=synth.BF16, ln=True, act=1))
    run_gateup_case(synth.random_gateup(7011, 3, 512, 24, 4, ln=True))
    torch.cuda.synchronize()
    assert qlin_merge_timeouts() == 0
