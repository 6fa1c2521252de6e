"""GPU: the quantizer and dequantizer entry points against the oracle, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import dev_bits, dev_words, host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from decode_linear_amd import build
    build.ensure_built()


def _weights(kind, N, K, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        w = rng.standard_normal((N, K)) * 0.02
    elif kind == "offset":
        w = rng.standard_normal((N, K)) * 0.5 + rng.standard_normal((N, 1)) * 3.0
    elif kind == "wide":
        w = rng.standard_normal((N, K)) * 10.0 ** rng.integers(-6, 3, (N, 1))
    elif kind == "ties":
        # groups with lo = 0, hi = 2^bits - 1 exactly and half-integer values in between
        w = rng.integers(0, 31, (N, K)) * 0.5
        w[:, ::64] = 0.0
        w[:, 1::64] = 15.0
    elif kind == "constant":
        w = np.repeat(rng.standard_normal((N, K // 64)), 64, axis=1)
    else:
        raise ValueError(kind)
    return w.astype(np.float32)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("kind", ["normal", "offset", "wide", "ties", "constant"])
@pytest.mark.parametrize("N,K", [(1, 64), (37, 192), (300, 1024)])
def test_pack_matches_oracle_bitwise(bits, kind, N, K):
    from decode_linear_amd import qlin_pack_affine
    w = _weights(kind, N, K, seed=N + K + bits)
    words, s, b, flag = oracle.pack_affine(w, bits)
    dflag = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = qlin_pack_affine(torch.from_numpy(w).cuda(), bits, flag=dflag)
    torch.cuda.synchronize()
    assert np.array_equal(got.data.cpu().numpy().view(np.uint32), words)
    assert np.array_equal(host_bits(got.scales), s)
    assert np.array_equal(host_bits(got.biases), b)
    assert int(dflag.item()) == flag == 0


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf, 1e6])
def test_pack_bad_groups_match_oracle(bad):
    from decode_linear_amd import qlin_pack_affine
    w = _weights("normal", 9, 256, seed=3)
    w[4, 130] = bad
    words, s, b, flag = oracle.pack_affine(w, 4)
    assert flag == 1
    dflag = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = qlin_pack_affine(torch.from_numpy(w).cuda(), 4, flag=dflag)
    torch.cuda.synchronize()
    assert int(dflag.item()) == 1
    assert np.array_equal(got.data.cpu().numpy().view(np.uint32), words)
    assert np.array_equal(host_bits(got.scales), s)
    assert np.array_equal(host_bits(got.biases), b)


def test_pack_full_size_workload_weights():
    """The 4-bit gate projection of the SwiGLU workload (14336 x 4096), bit for bit."""
    from decode_linear_amd import qlin_pack_affine
    case = synth.workload(4)
    words, s, b, _ = oracle.pack_affine(case.gate, 4)
    got = qlin_pack_affine(torch.from_numpy(case.gate).cuda(), 4)
    torch.cuda.synchronize()
    assert np.array_equal(got.data.cpu().numpy().view(np.uint32), words)
    assert np.array_equal(host_bits(got.scales), s)
    assert np.array_equal(host_bits(got.biases), b)


@pytest.mark.parametrize("bits", [4, 8])
def test_unpack_is_fma_of_code_scale_bias(bits):
    from decode_linear_amd import QWeight, qlin_unpack_affine
    w = _weights("offset", 33, 320, seed=bits)
    words, s, b, _ = oracle.pack_affine(w, bits)
    ref = oracle.dequant_f32(words, s, b, 33, 320, bits)
    q = QWeight(bits, 33, 320, dev_words(words), dev_bits(s, synth.F16), dev_bits(b, synth.F16))
    got = qlin_unpack_affine(q)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_unpack_dense_widens(dtype):
    from decode_linear_amd import QWeight, qlin_unpack_affine
    d = synth.draw(200, 0, "w", (17, 128), 0.0, 1.0, dtype)
    got = qlin_unpack_affine(QWeight(16, 17, 128, dev_bits(d, dtype)))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().astype(np.float64), oracle.widen(d, dtype))
