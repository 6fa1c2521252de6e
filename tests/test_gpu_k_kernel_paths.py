"""Both kernel families of the 4- and 8-bit linear, against the oracle.

By default the library sends a quantized call to the int8 streaming kernel wherever that
kernel's shape rules admit it, else to the general kernel.  This file checks (1) which
family each kind of call lands on (dispatch counter 8 counts the int8 kernel's launches),
and (2) the general kernel, forced with qlin_set_path(1), on the shapes the int8 kernel
otherwise takes: rows with and without LayerNorm, ragged K and N, long K, epilogues and
gate/up.  The forced path must stay correct: it is what every call falls back to."""
import numpy as np
import pytest
import torch

import synth
from helpers import run_gateup_case, run_linear_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from decode_linear_amd import build
    build.ensure_built()


@pytest.fixture
def general_path():
    from decode_linear_amd import qlin_dispatch_count, qlin_set_path
    prev = qlin_set_path(1)
    before = qlin_dispatch_count(8)
    yield
    assert qlin_set_path(prev) == 1
    assert qlin_dispatch_count(8) == before, "a call ran on the int8 kernel while the general path was forced"


def _s8_launches(fn):
    from decode_linear_amd import qlin_dispatch_count
    before = qlin_dispatch_count(8)
    fn()
    return qlin_dispatch_count(8) - before


@pytest.mark.parametrize("x_dtype,K,N", [(synth.F16, 4096, 14336), (synth.F16, 4096, 7176), (synth.BF16, 512, 14336)])
def test_many_tile_ring(x_dtype, K, N):
    """Workgroups of several tiles on the int8 kernel's ring.  N = 14336 gives 1792 gate/up
    tiles, 7 per workgroup: an odd count, so the ring starts with a zero step whose
    arithmetic is skipped.  N = 7176 gives 897 tiles, 4 per workgroup and 1 in the last
    (which alone takes a zero step).  K = 4096 runs 8 waves, which meet at a barrier per
    step in workgroups of four or more steps; K = 512 runs 4 waves, without the barrier."""
    case = synth.random_gateup(9500 + K + N + x_dtype, 4, K, N, 4, x_dtype=x_dtype)
    assert _s8_launches(lambda: run_gateup_case(case)) == 2   # fp32 and narrow outputs


@pytest.mark.parametrize("bits,ln", [(4, False), (8, True)])
def test_many_tile_ring_ragged_n(bits, ln):
    """Several tiles per workgroup with a partial last tile: N = 8197 makes 513 tiles of 16
    rows (3 per workgroup on a ring of two), the last holding 5 rows; the ring clamps the
    missing rows' loads to the matrix's last row and never stores them."""
    case = synth.random_case(9600 + bits + ln, 4, 256, 8197, bits, x_dtype=synth.BF16, ln=ln, add=True)
    assert _s8_launches(lambda: run_linear_case(case, y_dtypes=(synth.BF16,))) == 2


def test_many_tile_ring_ragged_gateup():
    """The gate/up form of the same: N = 4099 per projection makes 513 tiles of 8 + 8 rows."""
    case = synth.random_gateup(9610, 4, 512, 4099, 4)
    assert _s8_launches(lambda: run_gateup_case(case)) == 2


@pytest.mark.parametrize("kind,expect", [
    ("q4-T4", True), ("q8-T4-ln", True), ("q4-T32-ln", True), ("q8-K16384", True),
    ("gateup-q4", True), ("gateup-q4-ln", False), ("dense-f16", False), ("q4-K192", False)])
def test_family_chosen(kind, expect):
    cases = {
        "q4-T4": lambda: run_linear_case(synth.random_case(9100, 4, 1024, 64, 4, x_dtype=synth.BF16)),
        "q8-T4-ln": lambda: run_linear_case(synth.random_case(9101, 4, 1024, 64, 8, x_dtype=synth.BF16, ln=True)),
        "q4-T32-ln": lambda: run_linear_case(synth.random_case(9102, 32, 512, 48, 4, x_dtype=synth.BF16, ln=True)),
        "q8-K16384": lambda: run_linear_case(synth.random_case(9103, 4, 16384, 32, 8, x_dtype=synth.BF16)),
        "gateup-q4": lambda: run_gateup_case(synth.random_gateup(9104, 4, 1024, 40, 4)),
        "gateup-q4-ln": lambda: run_gateup_case(synth.random_gateup(9105, 4, 1024, 40, 4, ln=True)),
        "dense-f16": lambda: run_linear_case(synth.random_case(9106, 4, 512, 48, 16, x_dtype=synth.F16)),
        "q4-K192": lambda: run_linear_case(synth.random_case(9107, 3, 192, 40, 4, x_dtype=synth.BF16)),
    }
    n = _s8_launches(cases[kind])
    assert (n > 0) == expect, (kind, n)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("T", [1, 4, 5, 9, 17, 32])
@pytest.mark.parametrize("ln", [False, True])
def test_general_rows(general_path, bits, T, ln):
    case = synth.random_case(9200 + 37 * T + bits + ln, T, 512, 72, bits, x_dtype=synth.BF16, ln=ln,
                             x_mean=3.0 if ln else 0.0)
    run_linear_case(case, y_dtypes=(synth.BF16,))


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("K,N", [(64, 17), (192, 40), (4160, 33), (16384, 48)])
def test_general_k_and_n(general_path, bits, K, N):
    case = synth.random_case(9300 + K + N + bits, 3, K, N, bits, x_dtype=synth.F16, ln=True, act=1)
    run_linear_case(case, y_dtypes=(synth.F16,))


@pytest.mark.parametrize("act,res,add", [(1, True, True), (0, True, False)])
def test_general_epilogues(general_path, act, res, add):
    case = synth.random_case(9400 + act + 2 * res, 4, 1024, 64, 8, x_dtype=synth.BF16, act=act, res=res, add=add)
    run_linear_case(case, y_dtypes=(synth.BF16,))


@pytest.mark.parametrize("T", [1, 4, 16])
def test_general_gateup(general_path, T):
    run_gateup_case(synth.random_gateup(9500 + T, T, 1024, 72, 4))
    run_gateup_case(synth.random_gateup(9510 + T, T, 512, 24, 8))


def test_paths_agree_within_tolerance():
    """The same call on both families: each meets the oracle's gate (checked in the helper);
    their outputs differ only by rounding, never by a structural error."""
    from decode_linear_amd import qlin_set_path
    case = synth.random_case(9600, 4, 4096, 256, 4, x_dtype=synth.BF16, ln=True)
    a, _ = run_linear_case(case)
    prev = qlin_set_path(1)
    try:
        b, _ = run_linear_case(case)
    finally:
        qlin_set_path(prev)
    assert np.isfinite(a) and np.isfinite(b)


@pytest.mark.parametrize("bits,T,K,N,ln", [
    (4, 4, 14336, 256, False),    # windows of 16 groups, 14 waves (the MLP's down projection, cut in N)
    (8, 4, 8192, 64, False),      # windows of 8 groups, 16 waves
    (4, 2, 8192, 40, True),       # with LayerNorm (windows of 8 groups)
    (8, 6, 4096, 100, False),     # two 16-row blocks, windows of 4 groups
    (4, 1, 2048, 17, True),       # windows of 2 groups stay on 8 waves
])
def test_one_tile_workgroups_of_up_to_16_waves(bits, T, K, N, ln):
    case = synth.random_case(9700 + bits + T + K // 64 + N, T, K, N, bits, x_dtype=synth.BF16, ln=ln)
    assert _s8_launches(lambda: run_linear_case(case, y_dtypes=(synth.BF16,))) == 2


def test_gateup_shard_shape_on_16_waves():
    """One 8-way shard of the SwiGLU projection (N = 1792 per projection): 224 tiles, one per
    workgroup, windows of 4 groups over 16 waves."""
    assert _s8_launches(lambda: run_gateup_case(synth.random_gateup(9800, 4, 4096, 1792, 4))) == 2


# ---- the vector-ALU kernel (qlin_set_path(2)): T <= 4 -----------------------------------------

@pytest.fixture
def valu_path():
    from decode_linear_amd import qlin_dispatch_count, qlin_set_path
    prev = qlin_set_path(2)
    before = qlin_dispatch_count(9)
    yield lambda: qlin_dispatch_count(9) - before
    assert qlin_set_path(prev) == 2


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("T", [1, 2, 3, 4])
@pytest.mark.parametrize("ln", [False, True])
def test_valu_rows(valu_path, bits, T, ln):
    case = synth.random_case(9900 + 10 * T + bits + ln, T, 1024, 72, bits, x_dtype=synth.BF16, ln=ln,
                             x_mean=3.0 if ln else 0.0)
    run_linear_case(case, y_dtypes=(synth.BF16,))
    assert valu_path() == 2


@pytest.mark.parametrize("bits,T,K,N,ln", [(4, 4, 64, 17, False), (8, 3, 192, 40, True), (4, 2, 320, 33, False),
                                           (8, 4, 2048, 100, True), (4, 4, 4096, 48, False), (8, 1, 4096, 20, True),
                                           (4, 2, 4096, 24, True), (8, 4, 4032, 16, False)])
def test_valu_k_and_n(valu_path, bits, T, K, N, ln):
    case = synth.random_case(9950 + K + N + bits, T, K, N, bits, x_dtype=synth.F16 if K % 128 else synth.BF16,
                             ln=ln, act=1)
    run_linear_case(case, y_dtypes=(case.x_dtype,))
    assert valu_path() == 2


@pytest.mark.parametrize("act,res,add", [(1, True, True), (0, True, False)])
def test_valu_epilogues(valu_path, act, res, add):
    case = synth.random_case(9970 + act + 2 * res, 4, 1024, 64, 8, x_dtype=synth.BF16, act=act, res=res, add=add)
    run_linear_case(case, y_dtypes=(synth.BF16,))
    assert valu_path() == 2


@pytest.mark.parametrize("T", [1, 2, 4])
def test_valu_gateup(valu_path, T):
    run_gateup_case(synth.random_gateup(9980 + T, T, 1024, 72, 4))
    run_gateup_case(synth.random_gateup(9990 + T, T, 512, 24, 8))
    assert valu_path() == 4


def test_valu_falls_back_outside_its_shapes(valu_path):
    # K past 4096, and LayerNorm with gate/up, go to the other kernels
    run_linear_case(synth.random_case(9995, 2, 8192, 32, 4, x_dtype=synth.BF16))
    run_gateup_case(synth.random_gateup(9996, 4, 512, 24, 4, ln=True))
    assert valu_path() == 0


def test_valu_full_size_workloads(valu_path):
    """The LN + GELU workload (T=4, K=2048, N=8192, 8-bit) and the SwiGLU projection (T=4,
    K=4096, N=14336 per projection, 4-bit) on the vector-ALU kernel."""
    run_linear_case(synth.workload(2))
    run_gateup_case(synth.workload(4))
    assert valu_path() == 4


def test_valu_deterministic(valu_path):
    from decode_linear_amd import qlin_linear
    from helpers import Packed, dev_bits
    case = synth.random_case(9997, 4, 2048, 256, 4, x_dtype=synth.BF16, ln=True)
    W = Packed(case.w_f32, 4)
    x = dev_bits(case.x, case.x_dtype)
    ln = (dev_bits(case.gamma, case.x_dtype), dev_bits(case.beta, case.x_dtype), case.eps)
    a = qlin_linear(x, W.q, ln=ln, out_dtype=torch.float32)
    b = qlin_linear(x, W.q, ln=ln, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("T,K,N,ln", [(1, 1024, 1024, False), (2, 512, 72, True), (4, 4096, 40, False),
                                      (3, 2048, 33, True), (4, 64, 17, False)])
def test_valu_dense_fp16(valu_path, T, K, N, ln):
    case = synth.random_case(9800 + T + K // 64 + N, T, K, N, 16, x_dtype=synth.F16, ln=ln, act=int(ln))
    run_linear_case(case, y_dtypes=(synth.F16,))
    assert valu_path() == 2


def test_valu_dense_bf16_stays_off(valu_path):
    run_linear_case(synth.random_case(9810, 2, 512, 40, 16, x_dtype=synth.BF16))
    assert valu_path() == 0
