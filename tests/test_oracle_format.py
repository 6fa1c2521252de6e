"""Pins for the oracle's number formats and the affine quantization format.

Each check ties the oracle to something other than itself: IEEE definitions via
numpy/torch conversions (library routines), hand-derived codes of known words
(tests/golden/codes_layout.txt), exact dyadic arithmetic, and quantizer
properties (round trip on exactly representable grids, the error bound, range,
ties to even, the bad-group contract)."""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- binary16 / bfloat16 ------------------------------------------------------

def test_f16_decode_exhaustive_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.widen(bits, oracle.F16)
    ref = bits.view(np.float16).astype(np.float64)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_bf16_decode_exhaustive_is_top_half_of_binary32():
    bits = np.arange(65536, dtype=np.uint32)
    ours = oracle.widen(bits.astype(np.uint16), oracle.BF16)
    ref = (bits << 16).view(np.float32).astype(np.float64)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_f16_known_values():
    assert oracle.f16_to_f64(0x3C00) == 1.0
    assert oracle.f16_to_f64(0xC000) == -2.0
    assert oracle.f16_to_f64(0x7BFF) == 65504.0
    assert oracle.f16_to_f64(0x0400) == 2.0 ** -14
    assert oracle.f16_to_f64(0x0001) == 2.0 ** -24
    assert oracle.f16_to_f64(0x7C00) == float("inf")


def test_f16_rne_matches_numpy_on_random_and_ties():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
                        # exact halfway points between neighbouring binary16 values near 1 and in the subnormal range
                        (2 * np.arange(1, 2000) + 1) * 2.0 ** -11 + 1.0,
                        (2 * np.arange(0, 500) + 1) * 2.0 ** -25,
                        [65504.0, 65519.99, 65520.0, -65520.0, 1e9, 2.0 ** -26, -(2.0 ** -25)]])
    ours = oracle.round_to(v, oracle.F16)
    ref = v.astype(np.float16).view(np.uint16)
    assert (ours == ref).all()


def test_bf16_rne_matches_torch_on_binary32_values_and_ties():
    rng = np.random.default_rng(8)
    f = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32)
    # halfway cases: binary32 values whose low 16 bits are exactly 0x8000
    hb = (rng.integers(0x00800000, 0x7F000000, 2000, dtype=np.int64).astype(np.uint32) & 0xFFFF0000) | 0x8000
    f = np.concatenate([f, hb.view(np.float32)])
    ours = oracle.round_to(f.astype(np.float64), oracle.BF16)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()


# ---- code layout ----------------------------------------------------------------

def _golden_codes():
    rows = []
    with open(os.path.join(GOLDEN, "codes_layout.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            rows.append((int(parts[0]), int(parts[1], 16), [int(p) for p in parts[2:]]))
    return rows


@pytest.mark.parametrize("bits,word,expected", _golden_codes())
def test_codes_of_known_words(bits, word, expected):
    per = 32 // bits
    K = 64
    words = np.zeros((1, K // per), np.uint32)
    words[0, 3] = word                                     # the word holding k = 3*per .. 3*per + per - 1
    q = oracle.codes(words, 1, K, bits)
    assert list(q[0, 3 * per:4 * per]) == expected
    assert q[0, :3 * per].sum() == 0 and q[0, 4 * per:].sum() == 0


def test_dequant_exact_for_dyadic_scale_and_bias():
    # s = 0.375 (0x3600), b = -1.25 (0xBD00); every q*s + b is a short dyadic number.
    N, K = 2, 128
    rng = np.random.default_rng(1)
    for bits in (4, 8):
        q = rng.integers(0, 2 ** bits, (N, K)).astype(np.uint32)
        per = 32 // bits
        words = np.zeros((N, K // per), np.uint32)
        for j in range(per):
            words |= q[:, j::per] << np.uint32(bits * j)
        scales = np.full((N, K // 64), 0x3600, np.uint16)
        biases = np.full((N, K // 64), 0xBD00, np.uint16)
        W = oracle.dequant_f64(words, scales, biases, N, K, bits)
        assert np.array_equal(W, q * 0.375 - 1.25)
        assert np.array_equal(oracle.codes(words, N, K, bits), q)


def test_dequant_f32_is_single_rounding_of_exact_value():
    rng = np.random.default_rng(2)
    N, K = 8, 256
    for bits in (4, 8):
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        words, s, b, _ = oracle.pack_affine(w, bits)
        exact = oracle.dequant_f64(words, s, b, N, K, bits)       # exact in fp64
        f32 = oracle.dequant_f32(words, s, b, N, K, bits)
        assert np.array_equal(f32, exact.astype(np.float32))      # one round-to-nearest of the exact value


# ---- the quantizer ----------------------------------------------------------------

def _pack_grid(bits, s_val, b_val, N=3, K=192, seed=3):
    """w = b + s*q exactly, each group containing q = 0 and q = 2^bits - 1."""
    rng = np.random.default_rng(seed)
    qmax = 2 ** bits - 1
    q = rng.integers(0, qmax + 1, (N, K))
    q[:, ::64] = 0
    q[:, 1::64] = qmax
    w = (b_val + s_val * q).astype(np.float32)
    assert np.array_equal(w.astype(np.float64), b_val + s_val * q)
    return q, w


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("s_val,b_val", [(2.0 ** -8, -0.5), (0.375, -3.0), (2.0 ** -20, 2.0 ** -10)])
def test_pack_round_trips_exact_grids(bits, s_val, b_val):
    q, w = _pack_grid(bits, s_val, b_val)
    words, s, b, flag = oracle.pack_affine(w, bits)
    assert flag == 0
    assert np.array_equal(oracle.codes(words, *w.shape, bits), q)
    assert np.all(oracle.widen(s, oracle.F16) == s_val)
    assert np.all(oracle.widen(b, oracle.F16) == b_val)


@pytest.mark.parametrize("bits", [4, 8])
def test_pack_error_bound_and_range(bits):
    rng = np.random.default_rng(4)
    N, K = 64, 512
    w = (rng.standard_normal((N, K)) * 0.02 + rng.standard_normal((N, 1)) * 0.01).astype(np.float32)
    words, s16, b16, flag = oracle.pack_affine(w, bits)
    assert flag == 0
    q = oracle.codes(words, N, K, bits)
    assert q.max() <= 2 ** bits - 1
    s = oracle.widen(s16, oracle.F16)
    b = oracle.widen(b16, oracle.F16)
    deq = oracle.dequant_f64(words, s16, b16, N, K, bits)
    wg = w.astype(np.float64).reshape(N, K // 64, 64)
    lo, hi = wg.min(-1), wg.max(-1)
    s32 = (hi - lo) / (2 ** bits - 1)
    bound = s / 2 + np.abs(b - lo) + (2 ** bits - 1) * np.abs(s - s32) + 4 * np.spacing(np.abs(wg).max(-1))
    err = np.abs(deq.reshape(N, K // 64, 64) - wg).max(-1)
    assert np.all(err <= bound)
    # the scale is the binary16 rounding of the range / (2^bits - 1)
    assert np.all(np.abs(s - s32) <= np.abs(s32) * 2.0 ** -11 + 2.0 ** -25)


def test_pack_rounds_half_codes_to_even():
    # group with lo = 0 and hi = 15 -> s = 1, b = 0 exactly; halfway values go to the even code
    w = np.zeros((1, 64), np.float32)
    w[0, 1] = 15.0
    w[0, 2:8] = [2.5, 3.5, 0.5, 1.5, 14.5, 6.5]
    words, s, b, flag = oracle.pack_affine(w, 4)
    q = oracle.codes(words, 1, 64, 4)[0]
    assert oracle.f16_to_f64(s[0, 0]) == 1.0 and oracle.f16_to_f64(b[0, 0]) == 0.0
    assert list(q[:8]) == [0, 15, 2, 4, 0, 2, 14, 6]


def test_pack_constant_group():
    w = np.full((2, 128), 0.3, np.float32)
    w[1, 64:] = -7.0
    words, s, b, flag = oracle.pack_affine(w, 8)
    assert flag == 0
    assert np.all(s == 0)
    assert np.all(oracle.codes(words, 2, 128, 8) == 0)
    assert b[0, 0] == np.float16(0.3).view(np.uint16) and b[1, 1] == np.float16(-7.0).view(np.uint16)


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf, 1e6])
def test_pack_bad_group_contract(bad):
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((2, 128)) * 0.1).astype(np.float32)
    good_words, good_s, good_b, _ = oracle.pack_affine(w, 4)
    w[1, 70] = bad                                       # row 1, group 1 (1e6 overflows the binary16 bias/scale)
    words, s, b, flag = oracle.pack_affine(w, 4)
    assert flag == 1
    assert s[1, 1] == 0 and b[1, 1] == 0x7E00
    assert np.all(oracle.codes(words, 2, 128, 4)[1, 64:] == 0)
    # every other group is untouched
    assert np.array_equal(s[0], good_s[0]) and s[1, 0] == good_s[1, 0] and b[1, 0] == good_b[1, 0]
    assert np.array_equal(words[0], good_words[0])
