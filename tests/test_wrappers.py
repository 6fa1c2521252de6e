"""CPU checks of the Python binding's own argument checks: shapes, contiguity, dtypes and
devices are refused with ValueError before the library is called (the C ABI sees only
pointers and sizes, so the binding is where a tensor's shape can be checked)."""
import pytest
import torch

from decode_linear_amd import build as qbuild


@pytest.fixture(scope="module")
def q():
    qbuild.ensure_built()
    from decode_linear_amd import qlin
    return qlin


def _w(q, N=32, K=256, bits=4):
    return q.QWeight(bits, N, K, torch.zeros((N, K * bits // 32), dtype=torch.int32),
                     torch.zeros((N, K // 64), dtype=torch.float16), torch.zeros((N, K // 64), dtype=torch.float16))


def _counts(q):
    return [q.qlin_dispatch_count(i) for i in range(9)]


def test_linear_checks(q):
    before = _counts(q)
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    w = _w(q)
    with pytest.raises(ValueError, match="x must have shape"):
        q.qlin_linear(torch.zeros(256, dtype=torch.bfloat16), w)
    with pytest.raises(ValueError, match="x has dtype"):
        q.qlin_linear(x.float(), w)
    with pytest.raises(ValueError, match="contiguous"):
        q.qlin_linear(torch.zeros((256, 4), dtype=torch.bfloat16).t(), w)
    with pytest.raises(ValueError, match="does not match"):
        q.qlin_linear(torch.zeros((4, 512), dtype=torch.bfloat16), w)
    with pytest.raises(ValueError, match="w.scales must have shape"):
        q.qlin_linear(x, q.QWeight(4, 32, 256, w.data, w.scales[:, :2].contiguous(), w.biases))
    with pytest.raises(ValueError, match="w.data has dtype"):
        q.qlin_linear(x, q.QWeight(4, 32, 256, w.data.float(), w.scales, w.biases))
    with pytest.raises(ValueError, match="gamma"):
        q.qlin_linear(x, w, ln=(torch.zeros(128, dtype=torch.bfloat16), torch.zeros(256, dtype=torch.bfloat16), 1e-5))
    with pytest.raises(ValueError, match="beta has dtype"):
        q.qlin_linear(x, w, ln=(torch.zeros(256, dtype=torch.bfloat16), torch.zeros(256, dtype=torch.float16), 1e-5))
    with pytest.raises(ValueError, match="residual must have shape"):
        q.qlin_linear(x, w, residual=torch.zeros((4, 31), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="add has dtype"):
        q.qlin_linear(x, w, add=torch.zeros(32, dtype=torch.float32))
    with pytest.raises(ValueError, match="out must have shape"):
        q.qlin_linear(x, w, out=torch.zeros((4, 16), dtype=torch.float32))
    with pytest.raises(ValueError, match="must be on a GPU"):
        q.qlin_linear(x, w)
    assert _counts(q) == before


def test_gateup_and_mlp_checks(q):
    before = _counts(q)
    x = torch.zeros((4, 256), dtype=torch.float16)
    g, u = _w(q), _w(q)
    with pytest.raises(ValueError, match="same bits and N"):
        q.qlin_gateup_swiglu(x, g, _w(q, N=16))
    with pytest.raises(ValueError, match="up must be a QWeight"):
        q.qlin_gateup_swiglu(x, g, None)
    with pytest.raises(ValueError, match="out has dtype"):
        q.qlin_gateup_swiglu(x, g, u, out=torch.zeros((4, 32), dtype=torch.int32))
    with pytest.raises(ValueError, match="must be on a GPU"):
        q.qlin_gateup_swiglu(x, g, u)
    d = _w(q, N=256, K=64)        # down's K must be the hidden width, 32
    with pytest.raises(ValueError, match="down.K = 64 does not match"):
        q.qlin_mlp(x, g, u, d)
    d = _w(q, N=256, K=64)
    g2, u2 = _w(q, N=64), _w(q, N=64)
    with pytest.raises(ValueError, match="h must have shape"):
        q.qlin_mlp(x, g2, u2, d, h=torch.zeros((4, 32), dtype=torch.float16))
    with pytest.raises(ValueError, match="h has dtype"):
        q.qlin_mlp(x, g2, u2, d, h=torch.zeros((4, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="residual must have shape"):
        q.qlin_mlp(x, g2, u2, d, residual=torch.zeros((4, 64), dtype=torch.float16))
    with pytest.raises(ValueError, match="must be on a GPU"):
        q.qlin_mlp(x, g2, u2, d)
    assert _counts(q) == before


def test_pack_unpack_checks(q):
    before = _counts(q)
    with pytest.raises(ValueError, match="w has dtype"):
        q.qlin_pack_affine(torch.zeros((8, 128), dtype=torch.float16), 4)
    with pytest.raises(ValueError, match="bits must be 4 or 8"):
        q.qlin_pack_affine(torch.zeros((8, 128)), 16)
    with pytest.raises(ValueError, match="multiple of 64"):
        q.qlin_pack_affine(torch.zeros((8, 96)), 4)
    with pytest.raises(ValueError, match="must be on a GPU"):
        q.qlin_pack_affine(torch.zeros((8, 128)), 4)
    with pytest.raises(ValueError, match="w.bits must be"):
        q.qlin_unpack_affine(q.QWeight(2, 8, 128, torch.zeros((8, 8), dtype=torch.int32)))
    with pytest.raises(ValueError, match="out must have shape"):
        q.qlin_unpack_affine(_w(q), out=torch.zeros((32, 128)))
    assert _counts(q) == before


def test_chain_checks(q):
    B = torch.zeros((3, 4, 256), dtype=torch.bfloat16)
    w = _w(q, N=256)
    ok = dict(x=B[0], T=4, w=w, ln=None, y=B[1])
    with pytest.raises(ValueError, match="x_dtype"):
        q.QlinChain([ok], torch.float32, torch.bfloat16)
    with pytest.raises(ValueError, match="passes\\[1\\].y must have shape"):
        q.QlinChain([ok, dict(ok, y=torch.zeros((4, 128), dtype=torch.bfloat16))], torch.bfloat16, torch.bfloat16)
    with pytest.raises(ValueError, match="fewer than T"):
        q.QlinChain([dict(ok, T=5)], torch.bfloat16, torch.bfloat16)
    with pytest.raises(ValueError, match="passes\\[0\\].x must be on a GPU"):
        q.QlinChain([ok], torch.bfloat16, torch.bfloat16)
