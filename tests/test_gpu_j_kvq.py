"""GPU parity of qlin_kvq_decode (one query position per head over a quantized K/V cache)
against the oracle: the fp32 output under Gate A, the 16-bit output equal to RNE of the fp32
output (Gate B), across bits, group sizes, head dims, row counts (one block, several blocks,
ragged last blocks, the 512-row blocks past 2^21 rows, the merge's 256-block and 4096-block
boundaries) and query/KV head sharing."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TORCH_DT, gate_a, gate_b

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from decode_linear_amd import build
    build.ensure_built()


def _dev16(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).view(TORCH_DT[dt]).cuda()


def _run(c, out16=True):
    from decode_linear_amd import qlin_kvq_decode
    q = _dev16(c.q, c.q_dtype)
    k = (torch.from_numpy(c.k[0].view(np.int32)).cuda(), _dev16(c.k[1], c.sb_dtype), _dev16(c.k[2], c.sb_dtype))
    v = (torch.from_numpy(c.v[0].view(np.int32)).cuda(), _dev16(c.v[1], c.sb_dtype), _dev16(c.v[2], c.sb_dtype))
    y64 = oracle.kvq_decode(c.q, c.q_dtype, c.k, c.v, c.sb_dtype, c.KV, c.GS, c.bits)
    y32 = qlin_kvq_decode(q, k, v, c.KV, c.GS, c.bits, out_dtype=torch.float32)
    torch.cuda.synchronize()
    gate_a(y32, y64, what=c.name)
    if out16:
        y16 = qlin_kvq_decode(q, k, v, c.KV, c.GS, c.bits, out_dtype=TORCH_DT[c.q_dtype])
        torch.cuda.synchronize()
        gate_b(y16, y32, y64, c.q_dtype, what=c.name)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("GS,D", [(g, d) for g in (32, 64, 128) for d in (64, 128, 256, 512) if g <= d])
def test_kvq_formats(bits, GS, D):
    _run(synth.kvq_case(600 + bits + GS + D, 2, 1, 77, D, GS, bits))


@pytest.mark.parametrize("N", [1, 2, 5, 127, 128, 129, 255, 256, 257, 2048, 2049, 5000])
def test_kvq_rows(N):
    _run(synth.kvq_case(700 + N, 4, 2, N, 128, 64, 4), out16=N < 3000)


@pytest.mark.parametrize("H,KV", [(1, 1), (8, 8), (16, 8), (12, 3), (32, 1)])
def test_kvq_heads(H, KV):
    _run(synth.kvq_case(800 + H + KV, H, KV, 300, 256, 64, 8, sb_dtype=synth.F16))


@pytest.mark.parametrize("q_dtype,sb_dtype", [(synth.F16, synth.BF16), (synth.BF16, synth.F16),
                                               (synth.F16, synth.F16), (synth.BF16, synth.BF16)])
@pytest.mark.parametrize("bits", [4, 8])
def test_kvq_query_and_scale_dtypes(q_dtype, sb_dtype, bits):
    # the query's and the scales' dtypes each pick an instantiation of the block kernel
    _run(synth.kvq_case(930 + 4 * q_dtype + sb_dtype + bits, 4, 2, 700, 128, 64, bits, q_dtype=q_dtype,
                        sb_dtype=sb_dtype))


def test_kvq_fp16_and_large_scores():
    _run(synth.kvq_case(900, 4, 4, 200, 256, 32, 4, q_dtype=synth.F16, sb_dtype=synth.F16))
    # queries 40x larger: scores spread over tens, the softmax nearly one-hot
    _run(synth.kvq_case(901, 4, 2, 600, 128, 64, 8, q_sd=40.0 / np.sqrt(128)))


def test_kvq_workload_and_determinism():
    from decode_linear_amd import qlin_dispatch_count, qlin_kvq_decode
    c = synth.kvq_workload()
    _run(c, out16=False)
    q = _dev16(c.q, c.q_dtype)
    k = (torch.from_numpy(c.k[0].view(np.int32)).cuda(), _dev16(c.k[1], c.sb_dtype), _dev16(c.k[2], c.sb_dtype))
    v = (torch.from_numpy(c.v[0].view(np.int32)).cuda(), _dev16(c.v[1], c.sb_dtype), _dev16(c.v[2], c.sb_dtype))
    before = qlin_dispatch_count(7)
    a = qlin_kvq_decode(q, k, v, c.KV, c.GS, c.bits)
    b = qlin_kvq_decode(q, k, v, c.KV, c.GS, c.bits)
    torch.cuda.synchronize()
    assert qlin_dispatch_count(7) == before + 2
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_kvq_rejects_small_workspace():
    from decode_linear_amd import QlinError, qlin_kvq_decode
    c = synth.kvq_case(950, 2, 1, 300, 128, 64, 4)
    q = _dev16(c.q, c.q_dtype)
    k = (torch.from_numpy(c.k[0].view(np.int32)).cuda(), _dev16(c.k[1], c.sb_dtype), _dev16(c.k[2], c.sb_dtype))
    with pytest.raises(QlinError):
        qlin_kvq_decode(q, k, k, c.KV, c.GS, c.bits, workspace=torch.empty(16, device="cuda"))


def test_kvq_large_blocks_past_a_million_rows():
    # past 256 * 8192 rows the blocks grow to 512 rows
    _run(synth.kvq_case(990, 1, 1, 256 * 8192 + 5, 64, 64, 4), out16=False)


@pytest.mark.parametrize("N", [256 * 256, 256 * 256 + 1])
def test_kvq_merge_statistics_at_256_blocks(N):
    # up to 256 blocks every merge thread holds one block's statistics; past that it loops
    _run(synth.kvq_case(992 + N % 2, 2, 1, N, 64, 64, 4), out16=False)


def test_kvq_merge_past_4096_blocks():
    # past 4096 blocks (of 512 rows) the merge takes the block weights in two LDS chunks
    _run(synth.kvq_case(994, 1, 1, 4096 * 512 + 700, 64, 64, 4), out16=False)


def test_kvq_unaligned_query_matches_aligned():
    """A query that is only 2-byte aligned takes the element-wise load path: same result, bit
    for bit, as the 16-byte aligned query."""
    from decode_linear_amd import qlin_kvq_decode
    c = synth.kvq_case(950, 8, 4, 300, 128, 64, 4)
    q = _dev16(c.q, c.q_dtype)
    big = torch.empty(q.numel() + 1, dtype=q.dtype, device="cuda")
    qu = big[1:].view(q.shape)
    qu.copy_(q)
    assert qu.data_ptr() % 16 != 0
    k = (torch.from_numpy(c.k[0].view(np.int32)).cuda(), _dev16(c.k[1], c.sb_dtype), _dev16(c.k[2], c.sb_dtype))
    v = (torch.from_numpy(c.v[0].view(np.int32)).cuda(), _dev16(c.v[1], c.sb_dtype), _dev16(c.v[2], c.sb_dtype))
    a = qlin_kvq_decode(q, k, v, c.KV, c.GS, c.bits, out_dtype=torch.float32)
    b = qlin_kvq_decode(qu, k, v, c.KV, c.GS, c.bits, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
