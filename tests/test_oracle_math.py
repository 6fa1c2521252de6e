"""Pins for the oracle's arithmetic: LayerNorm, the contraction, GELU, SwiGLU and
the epilogue order.

Independent anchors used here:
  * the LayerNorm folding identity the pages state for the fused kernel
    ([p1] maya-mac mlx_kernels.py, `_linear_kernel` docstring), evaluated in the
    test with the single-pass shifted statistics, for several shifts x0;
  * textbook special cases (plain GEMV against numpy's matmul, a constant row,
    a balanced +-c row with eps = 0);
  * exact rational arithmetic (fractions) and 60-digit decimals on tiny inputs;
  * standard normal table values (tests/golden/gelu_phi.txt) and scipy's erf;
  * hand-derived epilogue-order and SwiGLU cases (tests/golden/*.txt).
"""
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import erf, expit

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                rows.append([float(p) for p in line.split()])
    return rows


def _qcase(T, K, N, bits, seed, x_mean=3.0):
    c = synth.random_case(seed, T, K, N, bits, x_dtype=synth.BF16, ln=True, x_mean=x_mean)
    words, s, b, _ = oracle.pack_affine(c.w_f32, bits)
    return c, words, s, b


# ---- LayerNorm ------------------------------------------------------------------

@pytest.mark.parametrize("bits", [8, 4])
def test_ln_fold_identity(bits):
    """LN(x).w = rstd * (sum (x-x0) g w - (mean-x0) sum g w) + sum b w, for any shift x0."""
    T, K, N = 3, 256, 24
    c, words, s, b = _qcase(T, K, N, bits, seed=11)
    y = oracle.linear(c.x, c.x_dtype, bits, words, scales=s, biases=b, gamma=c.gamma, beta=c.beta, eps=c.eps)
    x = oracle.widen(c.x, c.x_dtype)
    g = oracle.widen(c.gamma, c.x_dtype)
    be = oracle.widen(c.beta, c.x_dtype)
    W = oracle.dequant_f64(words, s, b, N, K, bits)
    Gw = W @ g
    Bw = W @ be
    eps = float(np.float32(c.eps))
    for t in range(T):
        for x0 in (0.0, x[t, 0], x[t].mean()):
            xv = x[t] - x0
            m = xv.sum() / K                                   # mean - x0
            var = (xv * xv).sum() / K - m * m                  # single-pass, shifted, biased
            rstd = 1.0 / np.sqrt(max(var, 0.0) + eps)
            folded = rstd * (W @ (xv * g) - m * Gw) + Bw
            assert np.allclose(y[t], folded, rtol=1e-12, atol=1e-12 * np.abs(folded).max())


def test_layernorm_constant_row_reduces_to_beta():
    K = 128
    x = np.full((2, K), 5.25)
    x[1] = -3.0
    g = np.linspace(0.5, 1.5, K)
    be = np.linspace(-1.0, 1.0, K)
    out = oracle.layernorm(x, g, be, 1e-5)
    assert np.array_equal(out, np.stack([be, be]))


def test_layernorm_balanced_row_eps0():
    K = 64
    x = np.where(np.arange(K) % 2 == 0, 0.75, -0.75)[None, :]
    g = np.full(K, 2.0)
    be = np.full(K, 0.125)
    out = oracle.layernorm(x, g, be, 0.0)
    # mean 0, biased variance c^2, rstd = 1/c exactly
    assert np.array_equal(out[0], np.where(np.arange(K) % 2 == 0, 2.125, -1.875))


def test_layernorm_is_biased_and_eps_inside_sqrt_decimal():
    getcontext().prec = 60
    rng = np.random.default_rng(9)
    K = 64
    x = np.round(rng.standard_normal((1, K)) * 64) / 64
    g = np.round(rng.standard_normal(K) * 16) / 16
    be = np.round(rng.standard_normal(K) * 16) / 16
    eps = 0.25
    out = oracle.layernorm(x, g, be, eps)[0]
    xs = [Decimal(float(v)) for v in x[0]]
    mu = sum(xs) / K
    var = sum((v - mu) ** 2 for v in xs) / K
    rstd = 1 / (var + Decimal(eps)).sqrt()
    ref = [float((xs[k] - mu) * rstd * Decimal(float(g[k])) + Decimal(float(be[k]))) for k in range(K)]
    assert np.allclose(out, ref, rtol=1e-14, atol=1e-14)


# ---- contraction ----------------------------------------------------------------

@pytest.mark.parametrize("bits", [16, 8, 4])
def test_plain_linear_is_textbook_gemv(bits):
    T, K, N = 5, 192, 40
    c = synth.random_case(21, T, K, N, bits, x_dtype=synth.F16)
    if bits == 16:
        y = oracle.linear(c.x, c.x_dtype, 16, c.w_dense, w_dtype=c.w_dtype)
        W = oracle.widen(c.w_dense, c.w_dtype)
    else:
        words, s, b, _ = oracle.pack_affine(c.w_f32, bits)
        y = oracle.linear(c.x, c.x_dtype, bits, words, scales=s, biases=b)
        W = oracle.dequant_f64(words, s, b, N, K, bits)
    ref = np.matmul(oracle.widen(c.x, c.x_dtype), W.T)
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())


def test_tiny_exact_cases_match_rational_arithmetic():
    """Small integer x, dyadic scale/bias and small codes: every product and partial
    sum is exact in fp64, so the oracle must equal exact rational arithmetic."""
    rng = np.random.default_rng(13)
    for T, K, N, bits in [(1, 64, 3, 8), (3, 128, 8, 4), (2, 64, 5, 4), (3, 128, 2, 8)]:
        per = 32 // bits
        q = rng.integers(0, 2 ** bits, (N, K)).astype(np.uint32)
        words = np.zeros((N, K // per), np.uint32)
        for j in range(per):
            words |= q[:, j::per] << np.uint32(bits * j)
        s_vals = rng.choice([0.5, 0.25, 0.125, 1.5, 0.75], (N, K // 64))
        b_vals = rng.choice([-2.0, -0.5, 0.0, 1.25, 3.0], (N, K // 64))
        s16 = s_vals.astype(np.float16).view(np.uint16)
        b16 = b_vals.astype(np.float16).view(np.uint16)
        xv = rng.integers(-8, 9, (T, K)).astype(np.float64)
        x16 = xv.astype(np.float16).view(np.uint16)
        y = oracle.linear(x16, oracle.F16, bits, words, scales=s16, biases=b16)
        for t in range(T):
            for n in range(N):
                acc = Fraction(0)
                for k in range(K):
                    w = Fraction(int(q[n, k])) * Fraction(s_vals[n, k // 64]) + Fraction(b_vals[n, k // 64])
                    acc += Fraction(int(xv[t, k])) * w
                assert y[t, n] == float(acc) and Fraction(y[t, n]) == acc


# ---- GELU / SwiGLU / epilogue -----------------------------------------------------

@pytest.mark.parametrize("v,phi", _read("gelu_phi.txt"))
def test_gelu_table(v, phi):
    assert oracle.gelu(v) == pytest.approx(v * phi, rel=1e-15, abs=1e-17)


def test_gelu_properties():
    vs = np.concatenate([np.linspace(-8, 8, 401), [1e-30, -1e-30, 30.0, -30.0]])
    for v in vs:
        gv, gm = oracle.gelu(v), oracle.gelu(-v)
        assert gv - gm == pytest.approx(v, rel=1e-14, abs=1e-300)          # GELU(v) - GELU(-v) = v
        assert gv == pytest.approx(0.5 * v * (1.0 + erf(v / np.sqrt(2.0))), rel=1e-13, abs=1e-15)
    assert oracle.gelu(0.0) == 0.0
    # deep negative tail keeps relative accuracy: GELU(-10) = -10 * Phi(-10)
    assert oracle.gelu(-10.0) == pytest.approx(-10.0 * 7.6198530241605260e-24, rel=1e-12)


def test_silu_properties():
    for g in np.linspace(-20, 20, 161):
        assert oracle.silu(g) - oracle.silu(-g) == pytest.approx(g, rel=1e-13, abs=1e-14)  # sigma(g)+sigma(-g)=1
        assert oracle.silu(g) == pytest.approx(g * expit(g), rel=1e-14, abs=1e-300)
    assert oracle.silu(0.0) == 0.0


def _onehot_dense(K, N, entries):
    """fp16 x = e_0 and a dense fp16 W with W[n, 0] = entries[n]."""
    x = np.zeros((1, K), np.float16)
    x[0, 0] = 1.0
    W = np.zeros((N, K), np.float16)
    W[:, 0] = entries
    return x.view(np.uint16), W.view(np.uint16)


@pytest.mark.parametrize("z,r,a,expected", _read("epilogue_order.txt"))
def test_epilogue_order_act_then_res_then_add(z, r, a, expected):
    x, W = _onehot_dense(64, 1, [z])
    res = np.array([[r]], np.float16).view(np.uint16)
    add = np.array([a], np.float16).view(np.uint16)
    y = oracle.linear(x, oracle.F16, 16, W, w_dtype=oracle.F16, act=1, res=res, add=add)
    assert y[0, 0] == pytest.approx(expected, rel=1e-15)


@pytest.mark.parametrize("g,u,expected", _read("swiglu_values.txt"))
def test_gateup_hand_values(g, u, expected):
    x, Wg = _onehot_dense(64, 1, [g])
    _, Wu = _onehot_dense(64, 1, [u])
    y = oracle.gateup(x, oracle.F16, 16, (Wg, None, None), (Wu, None, None), w_dtype=oracle.F16)
    assert y[0, 0] == pytest.approx(expected, rel=1e-15, abs=1e-300)


def test_gateup_is_silu_of_gate_times_up():
    T, K, N = 4, 128, 16
    c = synth.random_gateup(31, T, K, N, 8)
    gw, gs, gb, _ = oracle.pack_affine(c.gate, 8)
    uw, us, ub, _ = oracle.pack_affine(c.up, 8)
    y = oracle.gateup(c.x, c.x_dtype, 8, (gw, gs, gb), (uw, us, ub))
    x = oracle.widen(c.x, c.x_dtype)
    zg = x @ oracle.dequant_f64(gw, gs, gb, N, K, 8).T
    zu = x @ oracle.dequant_f64(uw, us, ub, N, K, 8).T
    assert np.allclose(y, zg * expit(zg) * zu, rtol=1e-12, atol=1e-14)
