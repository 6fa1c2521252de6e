"""Pins for the oracle's `attend` ([p1] maya-mac mlx_kernels.py, `_ATTEND` / `attend()`):
append this pass's keys and values to the band's cache, then causal softmax attention of
the new positions over at most 32 positions.

Independent anchors used here:
  * the cache layout, rebuilt with numpy reshapes, transposes and a concatenation (not the
    oracle's index arithmetic);
  * closed forms: one visible key gives its value; a zero query gives the plain mean of
    the visible values; two keys give the logistic weight (scipy's expit) of their score
    difference, which fixes the 1/sqrt(head_dim) scale;
  * invariants: later positions are invisible (causal), cached positions can be permuted
    (keys with their values) without changing the output, heads do not mix, and a score
    gap of hundreds (a top score of 905) selects one value exactly, which needs the max
    subtraction to keep exp finite.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle

BF16, F16 = oracle.BF16, oracle.F16


def _rand(rng, shape, dtype=BF16, scale=1.0):
    return oracle.round_to(scale * rng.standard_normal(shape), dtype)


def _case(seed, H, HD, P, T, dtype=BF16):
    rng = np.random.default_rng(seed)
    qkv = _rand(rng, (T, 3 * H * HD), dtype)
    kv = _rand(rng, (2, H, P, HD), dtype) if P > 0 else None
    return qkv, kv


@pytest.mark.parametrize("H,HD,P,T", [(1, 8, 0, 1), (2, 8, 3, 2), (3, 16, 5, 4), (2, 64, 28, 4), (1, 8, 0, 32)])
def test_cache_layout(H, HD, P, T):
    qkv, kv = _case(11 + P, H, HD, P, T)
    _, kv_out = oracle.attend(qkv, kv, BF16, H, HD)
    D = H * HD
    new_k = qkv[:, D:2 * D].reshape(T, H, HD).transpose(1, 0, 2)
    new_v = qkv[:, 2 * D:].reshape(T, H, HD).transpose(1, 0, 2)
    new = np.stack([new_k, new_v])                       # (2, H, T, HD)
    want = new if kv is None else np.concatenate([kv, new], axis=2)
    assert kv_out.shape == (2, H, P + T, HD)
    assert np.array_equal(kv_out, want)


def test_single_visible_key_returns_its_value():
    H, HD = 2, 8
    qkv, _ = _case(3, H, HD, 0, 1, F16)
    out, _ = oracle.attend(qkv, None, F16, H, HD)
    v = oracle.widen(qkv[0, 2 * H * HD:], F16)
    assert np.array_equal(out[0], v)


def test_zero_query_is_the_mean_of_visible_values():
    H, HD, P, T = 2, 8, 4, 3
    qkv, kv = _case(5, H, HD, P, T)
    qkv[:, :H * HD] = 0                                  # +0.0 bits
    out, kv_out = oracle.attend(qkv, kv, BF16, H, HD)
    vals = oracle.widen(kv_out[1], BF16)                 # (H, P + T, HD)
    for t in range(T):
        want = vals[:, :P + t + 1, :].mean(axis=1).reshape(-1)
        np.testing.assert_allclose(out[t], want, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("a,b,HD", [(1.5, 2.0, 4), (-3.0, 0.75, 16), (2.0, 2.0, 9)])
def test_two_keys_logistic_weight(a, b, HD):
    # one cached key k0 = (b, 0, ...), the new key k1 = 0, query (a, 0, ...):
    # s0 = a b / sqrt(HD), s1 = 0, so p0 = expit(s0) and out = p0 v0 + (1 - p0) v1
    H, P, T = 1, 1, 1
    rng = np.random.default_rng(7)
    qkv = np.zeros((T, 3 * HD), np.uint16)
    kv = np.zeros((2, H, P, HD), np.uint16)
    qkv[0, 0] = oracle.f64_to_bf16(a)
    kv[0, 0, 0, 0] = oracle.f64_to_bf16(b)
    v0 = _rand(rng, HD)
    v1 = _rand(rng, HD)
    kv[1, 0, 0, :] = v0
    qkv[0, 2 * HD:] = v1
    out, _ = oracle.attend(qkv, kv, BF16, H, HD)
    p0 = expit(a * b / np.sqrt(HD))
    want = p0 * oracle.widen(v0, BF16) + (1 - p0) * oracle.widen(v1, BF16)
    np.testing.assert_allclose(out[0], want, rtol=1e-13, atol=1e-15)


def test_causal_later_positions_are_invisible():
    H, HD, P, T = 2, 16, 3, 5
    qkv, kv = _case(9, H, HD, P, T)
    out, _ = oracle.attend(qkv, kv, BF16, H, HD)
    D = H * HD
    rng = np.random.default_rng(10)
    for t in range(T - 1):
        changed = qkv.copy()
        changed[t + 1:, D:] = _rand(rng, (T - t - 1, 2 * D))   # keys and values after t
        o2, _ = oracle.attend(changed, kv, BF16, H, HD)
        assert np.array_equal(o2[:t + 1], out[:t + 1])
        assert not np.array_equal(o2[t + 1:], out[t + 1:])
    # a visible cached value does change every row
    kv2 = kv.copy()
    kv2[1, :, 0, :] = _rand(rng, (H, HD))
    o3, _ = oracle.attend(qkv, kv2, BF16, H, HD)
    assert np.all(np.any(o3 != out, axis=1))


def test_cached_positions_permute_with_their_values():
    H, HD, P, T = 3, 8, 7, 2
    qkv, kv = _case(13, H, HD, P, T)
    out, _ = oracle.attend(qkv, kv, BF16, H, HD)
    perm = np.random.default_rng(14).permutation(P)
    o2, _ = oracle.attend(qkv, kv[:, :, perm, :], BF16, H, HD)
    np.testing.assert_allclose(o2, out, rtol=1e-13, atol=1e-15)
    # moving the keys alone does change the output
    kv3 = kv.copy()
    kv3[0] = kv[0][:, perm, :]
    o3, _ = oracle.attend(qkv, kv3, BF16, H, HD)
    assert not np.allclose(o3, out, rtol=1e-6)


def test_heads_do_not_mix():
    H, HD, P, T = 3, 8, 2, 2
    qkv, kv = _case(15, H, HD, P, T)
    out, _ = oracle.attend(qkv, kv, BF16, H, HD)
    changed = qkv.copy()
    D = H * HD
    for part in range(3):                                 # q, k and v columns of head 1
        changed[:, part * D + HD:part * D + 2 * HD] = _rand(np.random.default_rng(16 + part), (T, HD))
    o2, _ = oracle.attend(changed, kv, BF16, H, HD)
    assert np.array_equal(o2[:, :HD], out[:, :HD])
    assert np.array_equal(o2[:, 2 * HD:], out[:, 2 * HD:])
    assert not np.array_equal(o2[:, HD:2 * HD], out[:, HD:2 * HD])


def test_huge_score_gap_selects_one_value():
    # a score above 709: exp without the max subtraction would overflow even in fp64
    H, HD, P, T = 1, 8, 3, 1
    rng = np.random.default_rng(17)
    qkv = np.zeros((T, 3 * HD), np.uint16)
    kv = np.zeros((2, H, P, HD), np.uint16)
    qkv[0, 0] = oracle.f64_to_bf16(64.0)
    for j, kj in enumerate([10.0, 40.0, -20.0]):
        kv[0, 0, j, 0] = oracle.f64_to_bf16(kj)          # s_j = 64 kj / sqrt(8)
    kv[1] = _rand(rng, (H, P, HD))
    qkv[0, 2 * HD:] = _rand(rng, HD)
    out, _ = oracle.attend(qkv, kv, BF16, H, HD)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out[0], oracle.widen(kv[1, 0, 1], BF16), rtol=1e-15, atol=0)


def test_last_is_the_last_row():
    H, HD, P, T = 2, 16, 6, 4
    qkv, kv = _case(19, H, HD, P, T)
    out, kv_out = oracle.attend(qkv, kv, BF16, H, HD)
    out1, kv_out1 = oracle.attend(qkv, kv, BF16, H, HD, last=True)
    assert out1.shape == (1, H * HD)
    assert np.array_equal(out1[0], out[-1])
    assert np.array_equal(kv_out1, kv_out)


def test_rejects_more_than_32_positions():
    qkv, kv = _case(21, 1, 8, 30, 3)
    with pytest.raises(ValueError):
        oracle.attend(qkv, kv, BF16, 1, 8)
