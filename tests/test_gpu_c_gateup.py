"""GPU parity of qlin_gateup_swiglu against the oracle."""
import pytest

import synth
from helpers import run_gateup_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from decode_linear_amd import build
    build.ensure_built()


@pytest.mark.parametrize("bits", [4, 8, 16])
@pytest.mark.parametrize("T", [1, 2, 4, 8, 16, 32])
def test_gateup_rows(bits, T):
    run_gateup_case(synth.random_gateup(100 + T + bits, T, 512, 72, bits))


@pytest.mark.parametrize("N", [1, 7, 8, 9, 100])
@pytest.mark.parametrize("K", [64, 192, 4160])
def test_gateup_ragged(N, K):
    run_gateup_case(synth.random_gateup(200 + N + K, 4, K, N, 4))


@pytest.mark.parametrize("T", [1, 4, 12])
def test_gateup_with_layernorm(T):
    run_gateup_case(synth.random_gateup(300 + T, T, 1024, 40, 4, ln=True))


def test_gateup_fp16():
    run_gateup_case(synth.random_gateup(400, 4, 1024, 64, 4, x_dtype=synth.F16))
    run_gateup_case(synth.random_gateup(401, 3, 512, 24, 16, x_dtype=synth.F16))
