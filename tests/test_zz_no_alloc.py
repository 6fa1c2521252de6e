"""GPU check of qlin_kvq_decode_noalloc, the allocation-free quantized-KV decode: through the
C ABI, its output equals qlin_kvq_decode's (same kernels, caller workspace) bit for bit, on
two calls in a row, the second smaller than the first (the static scratch still holds the
first call's partials), and both stay within the oracle's tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TORCH_DT, gate_a

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from decode_linear_amd import build
    build.ensure_built()


def _dev16(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).view(TORCH_DT[dt]).cuda()


def _inputs(c):
    q = _dev16(c.q, c.q_dtype)
    k = (torch.from_numpy(c.k[0].view(np.int32)).cuda(), _dev16(c.k[1], c.sb_dtype), _dev16(c.k[2], c.sb_dtype))
    v = (torch.from_numpy(c.v[0].view(np.int32)).cuda(), _dev16(c.v[1], c.sb_dtype), _dev16(c.v[2], c.sb_dtype))
    return q, k, v


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_matches_workspace_entry_point(out_dtype):
    from decode_linear_amd import qlin_dispatch_count, qlin_kvq_decode, qlin_kvq_decode_noalloc
    big = synth.kvq_workload()                               # 16 heads, 8192 rows: 32 blocks per head
    small = synth.kvq_case(1201, 4, 2, 300, 128, 64, 8)      # 2 blocks per head, another head dim
    for c in (big, small):
        print(f"noalloc case {c.name} out {out_dtype}", flush=True)
        q, k, v = _inputs(c)
        H, D = q.shape
        ref = qlin_kvq_decode(q, k, v, c.KV, c.GS, c.bits, out_dtype=out_dtype)
        out = torch.full((H, D), float("nan"), dtype=out_dtype, device="cuda")
        before = qlin_dispatch_count(7)
        qlin_kvq_decode_noalloc(q, k, v, c.KV, c.GS, c.bits, out)
        torch.cuda.synchronize()
        assert qlin_dispatch_count(7) == before + 1
        assert torch.equal(out.view(torch.int16 if out_dtype != torch.float32 else torch.int32),
                           ref.view(torch.int16 if out_dtype != torch.float32 else torch.int32)), c.name
        if out_dtype == torch.float32:
            y64 = oracle.kvq_decode(c.q, c.q_dtype, c.k, c.v, c.sb_dtype, c.KV, c.GS, c.bits)
            gate_a(out, y64, what=c.name)


def test_noalloc_rejects_oversize_before_launch():
    from decode_linear_amd import QlinError, qlin_dispatch_count, qlin_kvq_decode_noalloc
    # 64 heads over 65536 rows of 128: 256 blocks of 256 rows per head, 8.5 MB of partials
    H, KV, N, D = 64, 8, 65536, 128
    q = torch.zeros((H, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((KV, N, D * 4 // 32), dtype=torch.int32, device="cuda")
    sb = torch.zeros((KV, N, D // 64), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((H, D), dtype=torch.bfloat16, device="cuda")
    before = qlin_dispatch_count(7)
    with pytest.raises(QlinError) as e:
        qlin_kvq_decode_noalloc(q, (kc, sb, sb), (kc, sb, sb), KV, 64, 4, out)
    assert e.value.status == -8
    assert qlin_dispatch_count(7) == before
