"""GPU parity of qlin_linear against the oracle (Gates A and B of tests/helpers.py).

Sizes span several 16-column tiles and ragged tails in N, every activation-tile count
(T, with and without LayerNorm), the 4-bit half step (K = 64 mod 128), the long-K
chunked path, all dtypes and the epilogue combinations."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import Packed, dev_bits, host_bits, run_linear_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from decode_linear_amd import build
    build.ensure_built()


@pytest.mark.parametrize("bits", [8, 4, 16])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 24, 31, 32])
@pytest.mark.parametrize("ln", [False, True])
def test_rows_and_layernorm(bits, T, ln):
    case = synth.random_case(1000 + 37 * T + bits + ln, T, 512, 72, bits, x_dtype=synth.BF16, ln=ln,
                             x_mean=3.0 if ln else 0.0)
    run_linear_case(case, y_dtypes=(synth.BF16,))


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("K", [64, 128, 192, 320, 960, 2112, 4160])
def test_k_tails(bits, K):
    case = synth.random_case(2000 + K + bits, 3, K, 40, bits, x_dtype=synth.BF16, ln=True, act=1)
    run_linear_case(case, y_dtypes=(synth.BF16,))


@pytest.mark.parametrize("bits,K,T,ln", [(4, 16384, 4, False), (4, 8192, 8, True), (8, 8192, 4, True),
                                         (8, 6144, 32, True), (16, 4096, 4, True), (16, 8192, 1, False),
                                         (4, 4096, 32, True), (8, 2048, 32, False)])
def test_long_k_chunked(bits, K, T, ln):
    case = synth.random_case(3000 + K + T + bits, T, K, 48, bits, x_dtype=synth.BF16, ln=ln)
    run_linear_case(case, y_dtypes=(synth.BF16,))


@pytest.mark.parametrize("N", [1, 5, 15, 16, 17, 33, 100, 257])
def test_ragged_n(N):
    for bits in (8, 4, 16):
        case = synth.random_case(4000 + N + bits, 4, 256, N, bits, x_dtype=synth.BF16, ln=True, add=True)
        run_linear_case(case, y_dtypes=(synth.BF16,))


@pytest.mark.parametrize("x_dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("bits", [16, 8, 4])
@pytest.mark.parametrize("ln", [False, True])
def test_dtypes(x_dtype, bits, ln):
    case = synth.random_case(5000 + x_dtype * 10 + bits + ln, 6, 384, 96, bits, x_dtype=x_dtype, ln=ln)
    run_linear_case(case, y_dtypes=(synth.F16, synth.BF16))


@pytest.mark.parametrize("act,res,add", [(1, False, False), (0, True, False), (0, False, True), (1, True, True)])
@pytest.mark.parametrize("bits", [8, 4, 16])
def test_epilogues(act, res, add, bits):
    case = synth.random_case(6000 + 8 * act + 4 * res + 2 * add + bits, 5, 256, 80, bits, x_dtype=synth.BF16,
                             ln=True, act=act, res=res, add=add)
    run_linear_case(case, y_dtypes=(synth.BF16,))


def test_extreme_activation_scales():
    """Rows far outside the fp16 range (and tiny ones) keep full accuracy via per-row scaling."""
    for scale in (1e-6, 1e-3, 3e4, 1e8):
        case = synth.random_case(7000, 4, 512, 64, 8, x_dtype=synth.BF16, ln=False)
        x = oracle.widen(case.x, synth.BF16) * scale
        case.x = synth.to_bits(x, synth.BF16)
        run_linear_case(case, y_dtypes=(synth.BF16,))
        case = synth.random_case(7001, 4, 512, 64, 4, x_dtype=synth.BF16, ln=True)
        case.gamma = synth.to_bits(oracle.widen(case.gamma, synth.BF16) * scale, synth.BF16)
        case.beta = synth.to_bits(oracle.widen(case.beta, synth.BF16) * scale, synth.BF16)
        run_linear_case(case, y_dtypes=(synth.BF16,))


def test_constant_row_layernorm():
    """A constant row has zero variance: LN(x) = beta, exercised through the fold."""
    case = synth.random_case(7100, 3, 256, 40, 8, x_dtype=synth.BF16, ln=True)
    x = oracle.widen(case.x, synth.BF16)
    x[1, :] = 2.5
    case.x = synth.to_bits(x, synth.BF16)
    run_linear_case(case, y_dtypes=(synth.BF16,))


def test_exact_small_integer_case_is_bitwise():
    """Small integers, dyadic scales and small codes: every intermediate is exact, so the
    fp32 output equals the oracle exactly."""
    from decode_linear_amd import QWeight, qlin_linear
    rng = np.random.default_rng(17)
    T, K, N, bits = 3, 128, 8, 4
    q = rng.integers(0, 16, (N, K)).astype(np.uint32)
    words = np.zeros((N, K // 8), np.uint32)
    for j in range(8):
        words |= q[:, j::8] << np.uint32(4 * j)
    s = rng.choice([0.5, 0.25, 1.0], (N, K // 64)).astype(np.float16).view(np.uint16)
    b = rng.choice([-2.0, 0.0, 1.5], (N, K // 64)).astype(np.float16).view(np.uint16)
    xv = rng.integers(-4, 5, (T, K)).astype(np.float16)
    y64 = oracle.linear(xv.view(np.uint16), synth.F16, bits, words, scales=s, biases=b)
    Wq = QWeight(bits, N, K, torch.from_numpy(words.view(np.int32)).cuda(), dev_bits(s, synth.F16),
                 dev_bits(b, synth.F16))
    y = qlin_linear(dev_bits(xv.view(np.uint16), synth.F16), Wq, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y64)


def test_deterministic_and_dispatch_counted():
    from decode_linear_amd import qlin_dispatch_count, qlin_linear
    case = synth.random_case(7200, 7, 1024, 300, 4, x_dtype=synth.BF16, ln=True, act=1)
    W = Packed(case.w_f32, 4)
    x = dev_bits(case.x, synth.BF16)
    ln = (dev_bits(case.gamma, synth.BF16), dev_bits(case.beta, synth.BF16), case.eps)
    before = qlin_dispatch_count(0)
    a = qlin_linear(x, W.q, ln=ln, act=1)
    b = qlin_linear(x, W.q, ln=ln, act=1)
    torch.cuda.synchronize()
    assert qlin_dispatch_count(0) == before + 2
    assert np.array_equal(host_bits(a), host_bits(b))


def test_empty_calls_leave_output_untouched():
    from decode_linear_amd import QWeight, qlin_linear
    case = synth.random_case(7300, 2, 128, 16, 8)
    W = Packed(case.w_f32, 8)
    x = dev_bits(case.x, synth.BF16)
    out = torch.full((2, 16), 7.0, dtype=torch.bfloat16, device="cuda")
    qlin_linear(x[:0], W.q, out=out[:0])
    empty = QWeight(8, 0, 128, W.q.data[:0], W.q.scales[:0], W.q.biases[:0])
    qlin_linear(x, empty, out=out[:, :0])
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("T,K", [(1, 1024), (4, 1024), (16, 1024), (4, 8192), (4, 14336)])
def test_wide_range_activations(bits, T, K):
    # activations over many binades: every product of a 32-k MFMA block must keep its
    # precision next to much larger ones (codes entering as subnormals did not)
    run_linear_case(synth.wide_case(4000 + T + K + bits, T, K, 96, bits), y_dtypes=(synth.BF16,))


@pytest.mark.parametrize("bits", [4, 8, 16])
def test_wide_range_activations_fp16(bits):
    run_linear_case(synth.wide_case(4100 + bits, 4, 2048, 80, bits, x_dtype=synth.F16), y_dtypes=(synth.F16,))
