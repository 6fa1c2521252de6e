"""Shared helpers for the parity tests: move seeded numpy inputs to the GPU, run the
library through its C ABI, run the oracle on the same bits, and apply the gates.

Tolerance (the reading of "max relative error 2e-3, fp32 accumulate, bf16/fp16 output"):
  tau   = 1e-2 * rms(y64) over the output tensor (a floor for outputs near zero)
  err_i = |y_i - y64_i| / max(|y64_i|, tau)
  Gate A: the library's fp32-output run has max err <= 2e-3.
  Gate B: a 16-bit output has max err <= 2e-3 + u (u = 2^-8 bf16, 2^-11 fp16) and equals the
          round-to-nearest-even of the fp32-output run bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

TOL = 2e-3
TAU_FRAC = 1e-2
U_OUT = {synth.F16: 2.0 ** -11, synth.BF16: 2.0 ** -8, synth.F32: 0.0}
TORCH_DT = {synth.F32: torch.float32, synth.F16: torch.float16, synth.BF16: torch.bfloat16}


def dev_bits(a: np.ndarray, dtype: int, device="cuda") -> torch.Tensor:
    """uint16 bit patterns (or fp32 values) -> a device tensor of that dtype."""
    if dtype == synth.F32:
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16))
    return t.view(TORCH_DT[dtype]).to(device)


def dev_words(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint32).view(np.int32)).to(device)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """A 16-bit device tensor -> uint16 bit patterns."""
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def host_values(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(y: np.ndarray, y64: np.ndarray):
    tau = TAU_FRAC * float(np.sqrt(np.mean(y64 ** 2))) if y64.size else 0.0
    den = np.maximum(np.abs(y64), tau if tau > 0 else 1e-30)
    return np.abs(y - y64) / den


def gate_a(y32: torch.Tensor, y64: np.ndarray, tol: float = TOL, what: str = ""):
    err = errors(host_values(y32), y64)
    mx = float(err.max()) if err.size else 0.0
    assert np.all(np.isfinite(host_values(y32))), f"{what}: non-finite output"
    assert mx <= tol, f"{what}: Gate A max err {mx:.3e} > {tol:.1e} (p99.9 {np.quantile(err, 0.999):.2e})"
    return mx


def gate_b(y16: torch.Tensor, y32: torch.Tensor, y64: np.ndarray, y_dtype: int, what: str = ""):
    err = errors(host_values(y16), y64)
    mx = float(err.max()) if err.size else 0.0
    assert mx <= TOL + U_OUT[y_dtype], f"{what}: Gate B max err {mx:.3e}"
    rne = host_bits(y32.cpu().to(TORCH_DT[y_dtype]))
    same = host_bits(y16) == rne
    assert same.all(), f"{what}: 16-bit output differs from RNE(fp32 output) at {int((~same).sum())} elements"
    return mx


class Packed:
    """A weight packed by the oracle (the expected format) and its device copy."""

    def __init__(self, w_f32=None, bits=8, dense=None, dense_dtype=synth.F16, device="cuda"):
        from decode_linear_amd import QWeight
        self.bits = bits
        if bits == 16:
            self.words, self.s, self.b = dense, None, None
            self.N, self.K = dense.shape
            self.dtype = dense_dtype
            self.q = QWeight(16, self.N, self.K, dev_bits(dense, dense_dtype, device))
        else:
            self.words, self.s, self.b, self.flag = oracle.pack_affine(w_f32, bits)
            self.N, self.K = w_f32.shape
            self.dtype = synth.F16
            self.q = QWeight(bits, self.N, self.K, dev_words(self.words, device), dev_bits(self.s, synth.F16, device),
                             dev_bits(self.b, synth.F16, device))

    def oracle_args(self):
        if self.bits == 16:
            return dict(wdata=self.words, w_dtype=self.dtype)
        return dict(wdata=self.words, scales=self.s, biases=self.b)

    def oracle_tuple(self):
        return (self.words, self.s, self.b)


def run_linear_case(case: synth.LinearCase, y_dtypes=(None,), device="cuda"):
    """Run a LinearCase through the library (fp32 output plus the listed 16-bit outputs)
    and the oracle; apply Gates A and B.  Returns (max err A, {dtype: max err B})."""
    from decode_linear_amd import qlin_linear
    W = Packed(case.w_f32, case.bits) if case.bits != 16 else Packed(bits=16, dense=case.w_dense,
                                                                      dense_dtype=case.w_dtype)
    x = dev_bits(case.x, case.x_dtype, device)
    ln = None
    if case.gamma is not None:
        ln = (dev_bits(case.gamma, case.x_dtype, device), dev_bits(case.beta, case.x_dtype, device), case.eps)
    res = None if case.res is None else dev_bits(case.res, case.x_dtype, device)
    add = None if case.add is None else dev_bits(case.add, case.x_dtype, device)
    y64 = oracle.linear(case.x, case.x_dtype, case.bits, gamma=case.gamma, beta=case.beta,
                        eps=float(np.float32(case.eps)), act=case.act, res=case.res, add=case.add, **W.oracle_args())
    y32 = qlin_linear(x, W.q, ln=ln, act=case.act, residual=res, add=add, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ea = gate_a(y32, y64, what=case.name)
    eb = {}
    for yd in y_dtypes:
        yd = case.y_dtype if yd is None else yd
        if yd == synth.F32:
            continue
        y16 = qlin_linear(x, W.q, ln=ln, act=case.act, residual=res, add=add, out_dtype=TORCH_DT[yd])
        torch.cuda.synchronize()
        eb[yd] = gate_b(y16, y32, y64, yd, what=case.name)
    return ea, eb


def run_gateup_case(case: synth.GateUpCase, y_dtype=None, device="cuda"):
    from decode_linear_amd import qlin_gateup_swiglu
    if case.bits == 16:
        G = Packed(bits=16, dense=case.gate, dense_dtype=case.x_dtype)
        U = Packed(bits=16, dense=case.up, dense_dtype=case.x_dtype)
        go, uo = (case.gate, None, None), (case.up, None, None)
        wdt = case.x_dtype
    else:
        G, U = Packed(case.gate, case.bits), Packed(case.up, case.bits)
        go, uo = G.oracle_tuple(), U.oracle_tuple()
        wdt = synth.F16
    x = dev_bits(case.x, case.x_dtype, device)
    ln = None
    if case.gamma is not None:
        ln = (dev_bits(case.gamma, case.x_dtype, device), dev_bits(case.beta, case.x_dtype, device), case.eps)
    y64 = oracle.gateup(case.x, case.x_dtype, case.bits, go, uo, w_dtype=wdt, gamma=case.gamma, beta=case.beta,
                        eps=float(np.float32(case.eps)))
    y32 = qlin_gateup_swiglu(x, G.q, U.q, ln=ln, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ea = gate_a(y32, y64, what=case.name)
    yd = case.y_dtype if y_dtype is None else y_dtype
    y16 = qlin_gateup_swiglu(x, G.q, U.q, ln=ln, out_dtype=TORCH_DT[yd])
    torch.cuda.synchronize()
    eb = gate_b(y16, y32, y64, yd, what=case.name)
    return ea, eb
