"""Pins for the oracle's quantized-KV decode attention ([p3] mlx-bun 0.0.10 -> 0.0.12,
model/fused-decode-kernel.ts: one query position attending over an affine-quantized K/V
cache, query heads sharing KV heads).  The caches are built here from known integer codes
with a packer written in this file (element d of a row at word d / (32 / bits), low bits
first), and checked against:
  * closed forms: one cached row returns its dequantized value row; a zero query returns
    the mean of the value rows; two rows give the logistic weight (scipy's expit) of their
    score difference (which also fixes that no 1/sqrt(D) scale is applied);
  * invariants: cached rows can be permuted (keys with values) without changing the output,
    and query head h reads KV head h / (H / KV) (equal to a one-KV-head call on its slice);
  * a score gap of hundreds selects one value row exactly (needs the max subtraction)."""
import numpy as np
import pytest
from scipy.special import expit

import oracle

BF16, F16 = oracle.BF16, oracle.F16


def _pack(codes, bits):
    KV, N, D = codes.shape
    per = 32 // bits
    w = np.zeros((KV, N, D // per), np.uint64)
    for j in range(per):
        w |= codes[:, :, j::per].astype(np.uint64) << np.uint64(j * bits)
    return w.astype(np.uint32)


def _cache(rng, KV, N, D, GS, bits, sb=BF16, scale=0.05):
    codes = rng.integers(0, 2 ** bits, (KV, N, D))
    s = oracle.round_to(scale * (0.5 + rng.uniform(size=(KV, N, D // GS))), sb)
    b = oracle.round_to(-scale * 2 ** (bits - 1) * rng.uniform(size=(KV, N, D // GS)), sb)
    deq = codes * np.repeat(oracle.widen(s, sb), GS, axis=2) + np.repeat(oracle.widen(b, sb), GS, axis=2)
    return (_pack(codes, bits), s, b), deq


def _q(rng, H, D, dtype=BF16, scale=1.0):
    bits = oracle.round_to(scale * rng.standard_normal((H, D)), dtype)
    return bits, oracle.widen(bits, dtype)


@pytest.mark.parametrize("bits,GS", [(4, 32), (4, 64), (8, 64), (8, 128)])
def test_one_row_returns_its_value(bits, GS):
    rng = np.random.default_rng(bits + GS)
    k, _ = _cache(rng, 1, 1, 256, GS, bits)
    v, vdeq = _cache(rng, 1, 1, 256, GS, bits)
    qb, _ = _q(rng, 2, 256)
    out = oracle.kvq_decode(qb, BF16, k, v, BF16, 1, GS, bits)
    assert np.array_equal(out, np.repeat(vdeq[0], 2, axis=0))


def test_zero_query_is_the_mean_of_values():
    rng = np.random.default_rng(3)
    k, _ = _cache(rng, 1, 37, 128, 64, 4)
    v, vdeq = _cache(rng, 1, 37, 128, 64, 4)
    out = oracle.kvq_decode(np.zeros((1, 128), np.uint16), BF16, k, v, BF16, 1, 64, 4)
    assert np.allclose(out[0], vdeq[0].mean(axis=0), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("dtype", [BF16, F16])
def test_two_rows_logistic_weight(dtype):
    rng = np.random.default_rng(4)
    k, kdeq = _cache(rng, 1, 2, 64, 32, 8, sb=dtype)
    v, vdeq = _cache(rng, 1, 2, 64, 32, 8, sb=dtype)
    qb, qv = _q(rng, 1, 64, dtype, 0.3)
    s = kdeq[0] @ qv[0]
    w0 = expit(s[0] - s[1])
    out = oracle.kvq_decode(qb, dtype, k, v, dtype, 1, 32, 8)
    assert np.allclose(out[0], w0 * vdeq[0, 0] + (1 - w0) * vdeq[0, 1], rtol=1e-12, atol=1e-12)


def test_row_permutation_invariance():
    rng = np.random.default_rng(5)
    k, _ = _cache(rng, 2, 50, 256, 64, 4)
    v, _ = _cache(rng, 2, 50, 256, 64, 4)
    qb, _ = _q(rng, 4, 256, scale=0.2)
    perm = rng.permutation(50)
    kp = tuple(a[:, perm] for a in k)
    vp = tuple(a[:, perm] for a in v)
    a = oracle.kvq_decode(qb, BF16, k, v, BF16, 2, 64, 4)
    b = oracle.kvq_decode(qb, BF16, kp, vp, BF16, 2, 64, 4)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_query_heads_share_kv_heads():
    rng = np.random.default_rng(6)
    H, KV = 6, 2
    k, _ = _cache(rng, KV, 20, 128, 32, 8)
    v, _ = _cache(rng, KV, 20, 128, 32, 8)
    qb, _ = _q(rng, H, 128, scale=0.2)
    full = oracle.kvq_decode(qb, BF16, k, v, BF16, KV, 32, 8)
    for h in range(H):
        c = h // (H // KV)
        one = oracle.kvq_decode(qb[h:h + 1], BF16, tuple(a[c:c + 1] for a in k), tuple(a[c:c + 1] for a in v),
                                BF16, 1, 32, 8)
        assert np.array_equal(full[h], one[0])


def test_large_score_gap_selects_one_row():
    rng = np.random.default_rng(7)
    D = 64
    codes = np.zeros((1, 3, D), np.int64)
    codes[0, 1] = 15                                   # the middle key is large along every d
    s = oracle.round_to(np.ones((1, 3, D // 32)), BF16)
    b = oracle.round_to(np.zeros((1, 3, D // 32)), BF16)
    k = (_pack(codes, 4), s, b)
    v, vdeq = _cache(rng, 1, 3, D, 32, 4)
    qb = oracle.round_to(np.ones((1, D)), BF16)       # scores 0, 960, 0
    out = oracle.kvq_decode(qb, BF16, k, v, BF16, 1, 32, 4)
    assert np.array_equal(out[0], vdeq[0, 1])
