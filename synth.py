"""Seeded synthetic inputs for the decode-time fused quantized linear.

This module only draws random numbers and rounds them to storage formats.  It
holds none of the method's arithmetic (no quantizer, no LayerNorm, no product),
so both the oracle and the HIP path can consume its arrays without sharing code.

RNG: numpy's PCG64 Generator, one stream per tensor, seeded with
    seed(c, p, id) = 1_000_000 * c + 1_000 * p + id
for workload c (1..5), pass p (0 except in the 124-pass chain) and tensor id
    1 x, 2 W / gate W, 3 up W, 4 gamma, 5 beta, 6 residual, 7 add.
Values are drawn in float64 and rounded to the storage dtype; 16-bit tensors are
returned as uint16 bit patterns, weights to be quantized as float32.

The pages benchmark a trained depth decoder and an MLP geometry whose weights are
not available; these draws stand in for them with the shapes below.

Workloads (N(mu, sd): second parameter is the standard deviation, except
N(0, 1/K) whose 1/K is the variance):
  1  T=1, K=1024, N=1024 plain linear; x fp16 N(0,1); W dense fp16 N(0,1/K); fp16 out
  2  T=4, K=2048, N=8192, LN + exact GELU; x bf16 N(3,1); gamma N(1,0.1); beta N(0,0.1);
     W fp32 N(0,0.02) -> 8-bit affine, group 64; bf16 out
  3  T=32, K=1024, N=4096, LN + residual; x, res bf16 N(0,1); W 8-bit from N(0,0.02); bf16 out
  4  gate+up SwiGLU, M=4, K=4096, N=14336 each; x bf16 N(0,1); gate/up 4-bit from N(0,0.02)
  5  124 dependent LN + linear passes, K=N=1024, T_p = 1 + (p mod 8); buffers B_0..B_124
     (8, 1024) bf16 N(0,1); per pass gamma, beta as in 2, W_p 8-bit from N(0,0.02)
  6  attend over the depth decoder's band: D = 1024 as 16 heads of 64, P = 24 cached and
     T = 8 new positions (the 32-position cap); qkv (T, 3D) and the cache (2, 16, 24, 64)
     bf16 N(0,1), so that scores q.k / sqrt(64) are about N(0,1)
  7  the MLP around workload 4: gate/up as in 4 (K=4096, I=14336, 4-bit) and a down
     projection (Hout=4096, K=I) 4-bit from N(0, 0.02), residual bf16 N(0,1)
  8  one sampling step of the depth decoder: 2048 codes, logits bf16 N(0, 2), Gumbel(0, 1)
     noise for 32 levels (fp32), code embeddings bf16 N(0, 1) of width 1024 for 4 levels,
     a prefix of 16 rows
  9  one decode step of attention over a quantized K/V cache: 16 query heads sharing 8 KV
     heads, head_dim 256, 8192 cached rows, 4-bit codes in groups of 64 (uniform random
     code words), scales bf16 0.05 U(0.5, 1.5), biases bf16 -0.4 U(0, 1); q bf16 N(0, 1/D)
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F32, F16, BF16 = 0, 1, 2
NP_CODES = {F32: np.float32}

TENSOR_IDS = {"x": 1, "w": 2, "up": 3, "gamma": 4, "beta": 5, "res": 6, "add": 7, "qkv": 8, "kv": 9, "down": 10,
              "logits": 11, "gumbel": 12, "table": 13, "prefix": 14, "kcodes": 15, "ks": 16, "kb": 17,
              "vcodes": 18, "vs": 19, "vb": 20}
CHAIN_PASSES = 124
CHAIN_K = CHAIN_N = 1024
CHAIN_TMAX = 8


def seed(c: int, p: int, name: str) -> int:
    return 1_000_000 * c + 1_000 * p + TENSOR_IDS[name]


def normal(s: int, shape, mean: float = 0.0, sd: float = 1.0) -> np.ndarray:
    """float64 draws from N(mean, sd^2) on a PCG64 stream seeded with s."""
    rng = np.random.Generator(np.random.PCG64(s))
    return mean + sd * rng.standard_normal(size=shape, dtype=np.float64)


def to_bits(a64: np.ndarray, dtype: int) -> np.ndarray:
    """Round float64 values to a storage dtype.  fp16 -> uint16 bits (numpy's IEEE
    conversion), bf16 -> uint16 bits (float64 -> float32 -> bfloat16, each step to
    nearest even), fp32 -> float32 values."""
    if dtype == F32:
        return np.asarray(a64, np.float32)
    if dtype == F16:
        return np.asarray(a64, np.float64).astype(np.float16).view(np.uint16)
    f = np.asarray(a64, np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    nan = (f & 0x7FFFFFFF) > 0x7F800000
    r = ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((f[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def draw(c: int, p: int, name: str, shape, mean: float, sd: float, dtype: int) -> np.ndarray:
    return to_bits(normal(seed(c, p, name), shape, mean, sd), dtype)


@dataclass
class LinearCase:
    """One fused-linear call's inputs.  w_f32 is set for quantized weights (to be packed),
    w_dense (uint16 bits) for dense ones."""
    name: str
    T: int
    K: int
    N: int
    x_dtype: int
    bits: int
    y_dtype: int
    x: np.ndarray
    w_f32: Optional[np.ndarray] = None
    w_dense: Optional[np.ndarray] = None
    w_dtype: int = F16
    gamma: Optional[np.ndarray] = None
    beta: Optional[np.ndarray] = None
    eps: float = 1e-5
    act: int = 0
    res: Optional[np.ndarray] = None
    add: Optional[np.ndarray] = None


@dataclass
class GateUpCase:
    name: str
    T: int
    K: int
    N: int
    x_dtype: int
    bits: int
    y_dtype: int
    x: np.ndarray
    gate: np.ndarray          # float32 (N, K) to be quantized, or uint16 dense bits when bits == 16
    up: np.ndarray
    gamma: Optional[np.ndarray] = None
    beta: Optional[np.ndarray] = None
    eps: float = 1e-5


def workload(c: int, scale_n: Optional[int] = None):
    """The synthetic inputs of workload c (1..4).  scale_n, if given, replaces N (smaller
    parity cases drawn from the same distributions)."""
    if c == 1:
        T, K, N = 1, 1024, scale_n or 1024
        return LinearCase("plain-fp16-T1-K1024-N1024", T, K, N, F16, 16, F16,
                          x=draw(1, 0, "x", (T, K), 0.0, 1.0, F16),
                          w_dense=draw(1, 0, "w", (N, K), 0.0, 1.0 / np.sqrt(K), F16), w_dtype=F16)
    if c == 2:
        T, K, N = 4, 2048, scale_n or 8192
        return LinearCase("ln-gelu-q8-T4-K2048-N8192", T, K, N, BF16, 8, BF16,
                          x=draw(2, 0, "x", (T, K), 3.0, 1.0, BF16),
                          w_f32=draw(2, 0, "w", (N, K), 0.0, 0.02, F32),
                          gamma=draw(2, 0, "gamma", (K,), 1.0, 0.1, BF16),
                          beta=draw(2, 0, "beta", (K,), 0.0, 0.1, BF16), eps=1e-5, act=1)
    if c == 3:
        T, K, N = 32, 1024, scale_n or 4096
        return LinearCase("ln-residual-q8-T32-K1024-N4096", T, K, N, BF16, 8, BF16,
                          x=draw(3, 0, "x", (T, K), 0.0, 1.0, BF16),
                          w_f32=draw(3, 0, "w", (N, K), 0.0, 0.02, F32),
                          gamma=draw(3, 0, "gamma", (K,), 1.0, 0.1, BF16),
                          beta=draw(3, 0, "beta", (K,), 0.0, 0.1, BF16), eps=1e-5,
                          res=draw(3, 0, "res", (T, N), 0.0, 1.0, BF16))
    if c == 4:
        T, K, N = 4, 4096, scale_n or 14336
        return GateUpCase("swiglu-q4-M4-K4096-N14336", T, K, N, BF16, 4, BF16,
                          x=draw(4, 0, "x", (T, K), 0.0, 1.0, BF16),
                          gate=draw(4, 0, "w", (N, K), 0.0, 0.02, F32),
                          up=draw(4, 0, "up", (N, K), 0.0, 0.02, F32))
    raise ValueError(f"no single-call workload {c}")


def chain_T(p: int) -> int:
    """Rows of pass p of the 124-pass chain: 1 + (p mod 8)."""
    return 1 + (p % CHAIN_TMAX)


def chain_buffers() -> np.ndarray:
    """B_0..B_124, each (8, 1024) bf16 bits, drawn N(0, 1)."""
    return np.stack([draw(5, p, "x", (CHAIN_TMAX, CHAIN_K), 0.0, 1.0, BF16) for p in range(CHAIN_PASSES + 1)])


def chain_pass(p: int):
    """Per-pass (w_f32 (N, K), gamma, beta) of the chain."""
    return (draw(5, p, "w", (CHAIN_N, CHAIN_K), 0.0, 0.02, F32),
            draw(5, p, "gamma", (CHAIN_K,), 1.0, 0.1, BF16),
            draw(5, p, "beta", (CHAIN_K,), 0.0, 0.1, BF16))


def random_case(s: int, T: int, K: int, N: int, bits: int, x_dtype: int = BF16, ln: bool = False,
                act: int = 0, res: bool = False, add: bool = False, y_dtype: Optional[int] = None,
                x_mean: float = 0.0, w_sd: float = 0.02) -> LinearCase:
    """A parity case of arbitrary shape, drawn like the workloads (stream ids offset by s)."""
    c = 100 + s
    y_dtype = x_dtype if y_dtype is None else y_dtype
    kw = {}
    if bits == 16:
        kw["w_dense"] = draw(c, 0, "w", (N, K), 0.0, 1.0 / np.sqrt(K), x_dtype)
        kw["w_dtype"] = x_dtype
    else:
        kw["w_f32"] = draw(c, 0, "w", (N, K), 0.0, w_sd, F32)
    if ln:
        kw["gamma"] = draw(c, 0, "gamma", (K,), 1.0, 0.1, x_dtype)
        kw["beta"] = draw(c, 0, "beta", (K,), 0.0, 0.1, x_dtype)
    if res:
        kw["res"] = draw(c, 0, "res", (T, N), 0.0, 1.0, x_dtype)
    if add:
        kw["add"] = draw(c, 0, "add", (N,), 0.0, 1.0, x_dtype)
    return LinearCase(f"rand{s}-T{T}-K{K}-N{N}-b{bits}", T, K, N, x_dtype, bits, y_dtype,
                      x=draw(c, 0, "x", (T, K), x_mean, 1.0, x_dtype), act=act, **kw)


def random_gateup(s: int, T: int, K: int, N: int, bits: int, x_dtype: int = BF16, ln: bool = False,
                  y_dtype: Optional[int] = None) -> GateUpCase:
    c = 100 + s
    y_dtype = x_dtype if y_dtype is None else y_dtype
    kw = {}
    if ln:
        kw["gamma"] = draw(c, 0, "gamma", (K,), 1.0, 0.1, x_dtype)
        kw["beta"] = draw(c, 0, "beta", (K,), 0.0, 0.1, x_dtype)
    if bits == 16:
        g = draw(c, 0, "w", (N, K), 0.0, 1.0 / np.sqrt(K), x_dtype)
        u = draw(c, 0, "up", (N, K), 0.0, 1.0 / np.sqrt(K), x_dtype)
    else:
        g = draw(c, 0, "w", (N, K), 0.0, 0.02, F32)
        u = draw(c, 0, "up", (N, K), 0.0, 0.02, F32)
    return GateUpCase(f"gu{s}-T{T}-K{K}-N{N}-b{bits}", T, K, N, x_dtype, bits, y_dtype,
                      x=draw(c, 0, "x", (T, K), 0.0, 1.0, x_dtype), gate=g, up=u, **kw)


@dataclass
class AttendCase:
    name: str
    H: int
    HD: int
    P: int
    T: int
    dtype: int
    qkv: np.ndarray                  # (T, 3 H HD) bit patterns
    kv: Optional[np.ndarray]         # (2, H, P, HD) bit patterns, None when P == 0


ATTEND_H, ATTEND_HD, ATTEND_P, ATTEND_T = 16, 64, 24, 8


def attend_case(s: int, H: int, HD: int, P: int, T: int, dtype: int = BF16, c: Optional[int] = None) -> AttendCase:
    """qkv and the cache drawn N(0, 1) in dtype (workload 6 with its own shapes; parity cases
    use stream ids offset by s)."""
    c = 100 + s if c is None else c
    kv = draw(c, 0, "kv", (2, H, P, HD), 0.0, 1.0, dtype) if P > 0 else None
    return AttendCase(f"att{s}-H{H}-HD{HD}-P{P}-T{T}", H, HD, P, T, dtype,
                      qkv=draw(c, 0, "qkv", (T, 3 * H * HD), 0.0, 1.0, dtype), kv=kv)


def attend_workload() -> AttendCase:
    case = attend_case(0, ATTEND_H, ATTEND_HD, ATTEND_P, ATTEND_T, BF16, c=6)
    case.name = f"attend-H{ATTEND_H}-HD{ATTEND_HD}-P{ATTEND_P}-T{ATTEND_T}"
    return case


@dataclass
class MlpCase:
    name: str
    T: int
    K: int
    I: int
    Hout: int
    x_dtype: int
    bits: int
    x: np.ndarray
    gate: np.ndarray          # float32 (I, K) to be quantized, or uint16 dense bits when bits == 16
    up: np.ndarray
    down: np.ndarray          # (Hout, I), same kinds
    gamma: Optional[np.ndarray] = None
    beta: Optional[np.ndarray] = None
    eps: float = 1e-5
    res: Optional[np.ndarray] = None


def random_mlp(s: int, T: int, K: int, I: int, Hout: int, bits: int, x_dtype: int = BF16, ln: bool = False,
               res: bool = False, c: Optional[int] = None) -> MlpCase:
    """Gate/up (I, K) and down (Hout, I) drawn like workload 4 (stream ids offset by s)."""
    c = 100 + s if c is None else c
    kw = {}
    if ln:
        kw["gamma"] = draw(c, 0, "gamma", (K,), 1.0, 0.1, x_dtype)
        kw["beta"] = draw(c, 0, "beta", (K,), 0.0, 0.1, x_dtype)
    if res:
        kw["res"] = draw(c, 0, "res", (T, Hout), 0.0, 1.0, x_dtype)
    if bits == 16:
        g = draw(c, 0, "w", (I, K), 0.0, 1.0 / np.sqrt(K), x_dtype)
        u = draw(c, 0, "up", (I, K), 0.0, 1.0 / np.sqrt(K), x_dtype)
        d = draw(c, 0, "down", (Hout, I), 0.0, 1.0 / np.sqrt(I), x_dtype)
    else:
        g = draw(c, 0, "w", (I, K), 0.0, 0.02, F32)
        u = draw(c, 0, "up", (I, K), 0.0, 0.02, F32)
        d = draw(c, 0, "down", (Hout, I), 0.0, 0.02, F32)
    return MlpCase(f"mlp{s}-T{T}-K{K}-I{I}-H{Hout}-b{bits}", T, K, I, Hout, x_dtype, bits,
                   x=draw(c, 0, "x", (T, K), 0.0, 1.0, x_dtype), gate=g, up=u, down=d, **kw)


def mlp_workload() -> MlpCase:
    case = random_mlp(0, 4, 4096, 14336, 4096, 4, BF16, res=True, c=7)
    case.name = "mlp-q4-M4-K4096-I14336-H4096"
    return case


def wide_case(s: int, T: int, K: int, N: int, bits: int, x_dtype: int = BF16) -> LinearCase:
    """A parity case whose activations spread over many binades (z1 * exp(1.5 z2), z1 and
    z2 standard normal, a heavy-tailed draw like the hidden activations of an MLP), with
    the weights of random_case."""
    c = 100 + s
    x64 = normal(seed(c, 0, "x"), (T, K)) * np.exp(1.5 * normal(seed(c, 0, "add"), (T, K)))
    base = random_case(s, T, K, N, bits, x_dtype)
    base.name = f"wide{s}-T{T}-K{K}-N{N}-b{bits}"
    base.x = to_bits(x64, x_dtype)
    return base


def gumbel(s: int, shape) -> np.ndarray:
    """float32 Gumbel(0, 1) draws, -log(-log(U)) with U uniform on (0, 1), on a PCG64 stream
    seeded with s (the noise a sampling step takes as input)."""
    rng = np.random.Generator(np.random.PCG64(s))
    u = rng.uniform(np.nextafter(0.0, 1.0), 1.0, size=shape)
    return (-np.log(-np.log(u))).astype(np.float32)


@dataclass
class SampleCase:
    name: str
    n: int
    D: int
    levels: int
    logits: np.ndarray        # (n,) fp32 values or 16-bit bit patterns
    logit_dtype: int
    gumbel: np.ndarray        # (32, n) float32
    table: np.ndarray         # (levels, n, D) bit patterns of emb_dtype
    prefix: np.ndarray        # (n_prev, D)
    emb_dtype: int


def sample_case(s: int, n: int, D: int, n_prev: int, levels: int = 2, logit_dtype: int = BF16,
                emb_dtype: int = BF16, logit_sd: float = 2.0, c: Optional[int] = None) -> SampleCase:
    c = 100 + s if c is None else c
    return SampleCase(f"sample{s}-n{n}-D{D}-p{n_prev}", n, D, levels,
                      logits=draw(c, 0, "logits", (n,), 0.0, logit_sd, logit_dtype), logit_dtype=logit_dtype,
                      gumbel=gumbel(seed(c, 0, "gumbel"), (32, n)),
                      table=draw(c, 0, "table", (levels, n, D), 0.0, 1.0, emb_dtype),
                      prefix=draw(c, 0, "prefix", (n_prev, D), 0.0, 1.0, emb_dtype), emb_dtype=emb_dtype)


def sample_workload() -> SampleCase:
    case = sample_case(0, 2048, 1024, 16, levels=4, c=8)
    case.name = "sample-n2048-D1024-p16"
    return case


@dataclass
class KvqCase:
    name: str
    H: int
    KV: int
    N: int
    D: int
    GS: int
    bits: int
    q_dtype: int
    sb_dtype: int
    q: np.ndarray             # (H, D) bit patterns
    k: tuple                  # (codes (KV, N, D*bits/32) uint32, scales, biases bit patterns)
    v: tuple


def kvq_case(s: int, H: int, KV: int, N: int, D: int, GS: int, bits: int, q_dtype: int = BF16,
             sb_dtype: int = BF16, q_sd: Optional[float] = None, c: Optional[int] = None) -> KvqCase:
    """Codes are uniform random 32-bit words (every word is a valid packing of codes)."""
    c = 100 + s if c is None else c
    words = D * bits // 32

    def cache(tag):
        rng = np.random.Generator(np.random.PCG64(seed(c, 0, tag + "codes")))
        codes = rng.integers(0, 2 ** 32, (KV, N, words), dtype=np.uint64).astype(np.uint32)
        u = np.random.Generator(np.random.PCG64(seed(c, 0, tag + "s"))).uniform(0.5, 1.5, (KV, N, D // GS))
        b = np.random.Generator(np.random.PCG64(seed(c, 0, tag + "b"))).uniform(0.0, 1.0, (KV, N, D // GS))
        lo = 0.05 * (2 ** bits - 1) / 2
        return codes, to_bits(0.05 * u * (15.0 / (2 ** bits - 1)), sb_dtype), to_bits(-lo * b * (15.0 / (2 ** bits - 1)), sb_dtype)

    sd = 1.0 / np.sqrt(D) if q_sd is None else q_sd
    return KvqCase(f"kvq{s}-H{H}-KV{KV}-N{N}-D{D}-g{GS}-b{bits}", H, KV, N, D, GS, bits, q_dtype, sb_dtype,
                   q=draw(c, 0, "x", (H, D), 0.0, sd, q_dtype), k=cache("k"), v=cache("v"))


def kvq_workload() -> KvqCase:
    case = kvq_case(0, 16, 8, 8192, 256, 64, 4, c=9)
    case.name = "kvq-decode-H16-KV8-D256-N8192-q4g64"
    return case
