"""Pins for the oracle's `sample` ([p1] maya-mac mlx_kernels.py, `_SAMPLE` / `sample()`):
exact top-k by order-preserving keys with ties kept, Gumbel-max over the kept codes, and
the chosen code's embedding appended.  Independent anchors:
  * no noise: the code is numpy's first argmax of the logits (for any top_k);
  * top_k = 1 keeps only the largest logit(s), whatever the noise says;
  * the kept count equals numpy's count of logits >= the k-th largest (ties included);
  * -0.0 orders below +0.0 (the keys' total order), so a +0.0 k-th value does not keep -0.0;
  * with noise drawn as Gumbel(0, 1) the codes follow softmax(logits * inv_temp) over the
    kept set (the Gumbel-max theorem), checked on many draws within 5 standard errors;
  * the output rows are the prefix rows, then the table row of the code (bit copies);
  * all-NaN kept scores give code -1 and a zero row."""
import numpy as np
import pytest

import oracle

F32, F16, BF16 = oracle.F32, oracle.F16, oracle.BF16


def _gumbel(rng, n):
    return (-np.log(-np.log(rng.uniform(1e-12, 1.0, n)))).astype(np.float32)


@pytest.mark.parametrize("top_k", [1, 3, 17, 100])
def test_no_noise_picks_first_argmax(top_k):
    rng = np.random.default_rng(top_k)
    x = rng.integers(-5, 6, 100).astype(np.float32)        # many ties
    code, _, _ = oracle.sample(x, F32, np.zeros(100, np.float32), 1.0, top_k)
    assert code == int(np.argmax(x))


def test_top1_ignores_noise_on_other_codes():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(64).astype(np.float32)
    g = np.zeros(64, np.float32)
    g[np.argsort(x)[:-1]] = 1e6                               # huge noise everywhere but the max
    code, _, kept = oracle.sample(x, F32, g, 1.0, 1)
    assert code == int(np.argmax(x)) and kept == 1


@pytest.mark.parametrize("top_k", [1, 2, 5, 10, 37])
def test_kept_count_includes_ties(top_k):
    rng = np.random.default_rng(top_k + 10)
    x = rng.integers(0, 8, 50).astype(np.float32)
    kth = np.sort(x)[::-1][top_k - 1]
    _, _, kept = oracle.sample(x, F32, np.zeros(50, np.float32), 1.0, top_k)
    assert kept == int((x >= kth).sum())


def test_negative_zero_orders_below_positive_zero():
    x = np.array([-1.0, 0.0, -0.0, -2.0], np.float32)        # +0.0 is the largest, then -0.0
    g = np.array([0, 0, 5, 0], np.float32)                    # noise favours -0.0
    code, _, kept = oracle.sample(x, F32, g, 1.0, 1)
    assert (code, kept) == (1, 1)
    code, _, kept = oracle.sample(x, F32, g, 1.0, 2)
    assert (code, kept) == (2, 2)


@pytest.mark.parametrize("top_k,inv_temp", [(4, 1.0), (6, 0.5), (3, 2.0)])
def test_gumbel_max_follows_softmax_of_kept(top_k, inv_temp):
    rng = np.random.default_rng(7)
    x = np.array([1.0, 0.5, 0.0, -0.3, 2.0, -1.0], np.float32)
    keep = x >= np.sort(x)[::-1][top_k - 1]
    p = np.where(keep, np.exp(x.astype(np.float64) * inv_temp), 0.0)
    p /= p.sum()
    draws = 4000
    counts = np.zeros(6)
    for _ in range(draws):
        code, _, _ = oracle.sample(x, F32, _gumbel(rng, 6), inv_temp, top_k)
        counts[code] += 1
    se = np.sqrt(p * (1 - p) / draws) + 1e-9
    assert (np.abs(counts / draws - p) <= 5 * se + 1e-12).all(), (counts / draws, p)


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_embedding_row_appended(dtype):
    rng = np.random.default_rng(3)
    n, D = 40, 24
    logits = oracle.round_to(rng.standard_normal(n), dtype)
    table = rng.integers(0, 2 ** 16, (n, D), dtype=np.uint64).astype(np.uint16)
    prefix = rng.integers(0, 2 ** 16, (3, D), dtype=np.uint64).astype(np.uint16)
    code, out, _ = oracle.sample(logits, dtype, _gumbel(rng, n), 1.0, 8, table=table, prefix=prefix)
    assert np.array_equal(out[:3], prefix) and np.array_equal(out[3], table[code])
    vals = oracle.widen(logits, dtype)
    assert vals[code] >= np.sort(vals)[::-1][7]


def test_all_nan_scores_give_no_code():
    x = np.array([np.nan, 1.0, np.nan], np.float32)
    g = np.array([0.0, np.nan, 0.0], np.float32)
    code, out, _ = oracle.sample(x, F32, g, 1.0, 3, table=np.ones((3, 4), np.float32))
    assert code == -1 and np.array_equal(out, np.zeros((1, 4), np.float32))
