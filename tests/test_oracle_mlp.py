"""Pins of the oracle's MLP ([p3] mlx-bun 0.0.10 -> 0.0.12, model/fused-mlp-kernel.ts, the
whole MLP of its header comment: down = (silu(x Wg^T) * (x Wu^T)) Wd^T, the hidden
activation rounded to the activation dtype), each against a fact that does not re-type the
composition:
  * an identity down projection returns the hidden activation exactly, and with a residual
    exactly the hidden activation plus the residual (sums of two bf16 values are exact in
    fp64);
  * a permutation down projection permutes the hidden columns (a transposed operand or a
    wrong axis fails);
  * the hidden activation is within half a unit in the last place of the unrounded
    gate/up product (round to nearest), and is not the unrounded value;
  * a quantized down projection equals numpy's product of the hidden activation with the
    dequantized down matrix (dequantization is pinned on its own)."""
import numpy as np
import pytest

import oracle
import synth

BF16, F16 = synth.BF16, synth.F16


def _dense_case(T=3, K=128, I=64, x_dtype=BF16, seed=11):
    c = synth.random_mlp(seed, T, K, I, I, 16, x_dtype, res=True)
    return c


def test_identity_down_returns_hidden_exactly():
    c = _dense_case()
    eye = synth.to_bits(np.eye(c.I), c.x_dtype)
    h, y = oracle.mlp(c.x, c.x_dtype, 16, (c.gate, None, None), (c.up, None, None), (eye, None, None),
                      w_dtype=c.x_dtype)
    assert np.array_equal(y, oracle.widen(h, c.x_dtype))
    h2, y2 = oracle.mlp(c.x, c.x_dtype, 16, (c.gate, None, None), (c.up, None, None), (eye, None, None),
                        w_dtype=c.x_dtype, res=c.res)
    assert np.array_equal(h2, h)
    assert np.array_equal(y2, oracle.widen(h, c.x_dtype) + oracle.widen(c.res, c.x_dtype))


def test_permutation_down_permutes_hidden_columns():
    c = _dense_case(seed=12)
    perm = np.random.default_rng(5).permutation(c.I)
    P = np.zeros((c.I, c.I))
    P[np.arange(c.I), perm] = 1.0          # output j takes hidden column perm[j]
    h, y = oracle.mlp(c.x, c.x_dtype, 16, (c.gate, None, None), (c.up, None, None),
                      (synth.to_bits(P, c.x_dtype), None, None), w_dtype=c.x_dtype)
    assert np.array_equal(y, oracle.widen(h, c.x_dtype)[:, perm])


@pytest.mark.parametrize("x_dtype", [BF16, F16])
def test_hidden_is_the_rounded_gateup_product(x_dtype):
    c = _dense_case(x_dtype=x_dtype, seed=13)
    eye = synth.to_bits(np.eye(c.I), x_dtype)
    h, _ = oracle.mlp(c.x, x_dtype, 16, (c.gate, None, None), (c.up, None, None), (eye, None, None),
                      w_dtype=x_dtype)
    h64 = oracle.gateup(c.x, x_dtype, 16, (c.gate, None, None), (c.up, None, None), w_dtype=x_dtype)
    hv = oracle.widen(h, x_dtype)
    mant, emin = (7, -126) if x_dtype == BF16 else (10, -14)   # subnormals share the ulp of the least normal
    ulp = 2.0 ** (np.maximum(np.floor(np.log2(np.abs(h64))), emin) - mant)
    assert (np.abs(hv - h64) <= ulp / 2 + 1e-300).all()
    assert not np.array_equal(hv, h64)     # the rounding happened


def test_quantized_down_is_numpy_product():
    c = synth.random_mlp(14, 2, 256, 192, 40, 8, BF16, res=True)
    g = oracle.pack_affine(c.gate, 8)[:3]
    u = oracle.pack_affine(c.up, 8)[:3]
    d = oracle.pack_affine(c.down, 8)[:3]
    h, y = oracle.mlp(c.x, BF16, 8, g, u, d, res=c.res)
    Wd = oracle.dequant_f64(*d, c.Hout, c.I, 8)
    ref = oracle.widen(h, BF16) @ Wd.T + oracle.widen(c.res, BF16)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
