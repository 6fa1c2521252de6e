"""GPU parity of qlin_sample against the oracle's sample: the code bit-exact (an integer the
fp32 scores decide, computed in fp32 on both sides) and the output rows bit-exact, over
logit dtypes, code counts (ragged ones included), k from 1 to n, ties at the k-th value,
signed zeros, infinities and NaNs, in-place append and no append."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TORCH_DT

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from decode_linear_amd import build
    build.ensure_built()


def _dev(a, dtype):
    if dtype == synth.F32:
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).view(TORCH_DT[dtype]).cuda()


def _host(t, dtype):
    if dtype == synth.F32:
        return t.cpu().numpy()
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _run(case, level, inv_temp, top_k, embed=True, in_place=False):
    from decode_linear_amd import qlin_sample
    lg = _dev(case.logits, case.logit_dtype)
    g = torch.from_numpy(case.gumbel).cuda()
    tb = _dev(case.table, case.emb_dtype)
    n_prev = case.prefix.shape[0]
    ref_code, ref_out, _ = oracle.sample(case.logits, case.logit_dtype, case.gumbel[level], inv_temp, top_k,
                                         table=case.table[level] if embed else None,
                                         prefix=case.prefix if n_prev > 0 else None)
    if in_place:
        buf = torch.zeros((n_prev + 1, case.D), dtype=TORCH_DT[case.emb_dtype], device="cuda")
        buf[:n_prev] = _dev(case.prefix, case.emb_dtype)
        code, out = qlin_sample(lg, g, level, tb, buf[:n_prev], inv_temp, top_k, out=buf)
    else:
        pre = _dev(case.prefix, case.emb_dtype) if n_prev > 0 else None
        code, out = qlin_sample(lg, g, level, tb, pre, inv_temp, top_k, embed=embed)
    torch.cuda.synchronize()
    assert int(code.item()) == ref_code, f"{case.name} level {level} k {top_k}: code {int(code.item())} != {ref_code}"
    if out is not None or ref_out.size:
        assert np.array_equal(_host(out, case.emb_dtype), ref_out.view(_host(out, case.emb_dtype).dtype))


@pytest.mark.parametrize("n", [1, 7, 1000, 2048, 2049, 4096, 4097, 8192])
@pytest.mark.parametrize("kfrac", [0.0, 0.05, 1.0])
def test_sample_sizes(n, kfrac):
    case = synth.sample_case(10 + n, n, 64, 3)
    _run(case, 1, 1.0 / 0.8, max(1, int(kfrac * n)))


@pytest.mark.parametrize("dt", [synth.F32, synth.F16, synth.BF16])
@pytest.mark.parametrize("edt", [synth.F32, synth.F16, synth.BF16])
def test_sample_dtypes(dt, edt):
    case = synth.sample_case(20 + dt * 3 + edt, 2048, 32, 5, logit_dtype=dt, emb_dtype=edt)
    _run(case, 0, 1.0, 64)


def _logit_bits(x, dt):
    """fp32 values (all exact in the 16-bit dtypes used here) as the dtype's logits."""
    x = np.asarray(x, np.float32)
    if dt == synth.F32:
        return x
    if dt == synth.F16:
        return x.astype(np.float16).view(np.uint16)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


# the 16-bit dtypes run the select on their high digits only and fill the rest from the sign
@pytest.mark.parametrize("dt", [synth.F32, synth.F16, synth.BF16])
@pytest.mark.parametrize("k", [1, 2, 9, 50, 300])
def test_sample_ties_at_kth(k, dt):
    case = synth.sample_case(30 + k, 2048, 16, 2, logit_dtype=dt)
    case.logits = _logit_bits(np.random.default_rng(k).integers(-6, 7, 2048), dt)   # heavy ties, both signs
    _run(case, 1, 1.0, k)
    case.gumbel[:] = 0.0                                   # equal scores: the smaller index
    _run(case, 1, 1.0, k)


@pytest.mark.parametrize("dt", [synth.F32, synth.F16, synth.BF16])
def test_sample_special_values(dt):
    case = synth.sample_case(40, 512, 16, 1, logit_dtype=dt)
    x = np.random.default_rng(40).normal(0.0, 2.0, 512).astype(np.float32)   # rounded or cut to the dtype
    x[:8] = [0.0, -0.0, np.inf, -np.inf, np.nan, 3.0, 3.0, -0.0]
    case.logits = _logit_bits(x, dt)
    for k in (1, 2, 3, 6, 9, 512):
        _run(case, 0, 1.0, k)
    g = case.gumbel.copy()
    g[0, :] = np.nan                                       # every score NaN: code -1, zero row
    case.gumbel = g
    _run(case, 0, 1.0, 10)


def test_sample_in_place_and_no_embed():
    case = synth.sample_case(50, 2048, 1024, 16)
    _run(case, 1, 1.25, 50, in_place=True)
    _run(case, 1, 1.25, 50, embed=False)


def test_sample_workload_and_determinism():
    from decode_linear_amd import qlin_dispatch_count, qlin_sample
    case = synth.sample_workload()
    for level in range(case.levels):
        _run(case, level, 1.0 / 0.9, 64)
    lg, g = _dev(case.logits, case.logit_dtype), torch.from_numpy(case.gumbel).cuda()
    tb, pre = _dev(case.table, case.emb_dtype), _dev(case.prefix, case.emb_dtype)
    before = qlin_dispatch_count(6)
    a = qlin_sample(lg, g, 2, tb, pre, 1.1, 64)
    b = qlin_sample(lg, g, 2, tb, pre, 1.1, 64)
    torch.cuda.synchronize()
    assert qlin_dispatch_count(6) == before + 2
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))
