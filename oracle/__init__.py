"""The oracle: a plain fp64 CPU reference for the decode-time fused quantized linear.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``decode_linear_amd``) never touches it, and it shares no code with that path.

The arithmetic lives in ``oracle/oracle.cpp`` (plain C++17, double precision);
this module only marshals numpy arrays through ctypes.  Page citations for each
function are in that file's comments:
  [p1] maya-mac src/maya_mac/mlx_kernels.py ("Custom Metal kernels for the depth decoder")
  [p2] @mlx-bun/inference 0.0.0-stage -> 1.0.0, kernels/trellis/mixed-gate-up.ts
  [p3] mlx-bun 0.0.10 -> 0.0.12, model/fused-decode-kernel.ts (and fused-mlp-kernel.ts)

dtype codes: 0 = fp32, 1 = fp16, 2 = bf16.  16-bit arrays are passed as their
uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
BUILD_PATH = os.path.join(_HERE, "liboracle.so")
# ORACLE_LIB_PATH names another build of oracle.cpp to load (the sanitizer test uses one).
LIB_PATH = os.environ.get("ORACLE_LIB_PATH") or BUILD_PATH
SRC_PATH = os.path.join(_HERE, "oracle.cpp")

F32, F16, BF16 = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.cpp into liboracle.so with g++ (-O2, no fast-math, no FP contraction)."""
    if not force and os.path.exists(BUILD_PATH):
        return BUILD_PATH
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           SRC_PATH, "-o", BUILD_PATH + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(BUILD_PATH + ".tmp", BUILD_PATH)
    return BUILD_PATH


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def load():
    global _lib
    if _lib is not None:
        return _lib
    if LIB_PATH == BUILD_PATH and not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.orc_f16_to_f64.argtypes = [ctypes.c_uint16]; lib.orc_f16_to_f64.restype = d
    lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]; lib.orc_bf16_to_f64.restype = d
    lib.orc_f64_to_f16.argtypes = [d]; lib.orc_f64_to_f16.restype = ctypes.c_uint16
    lib.orc_f64_to_bf16.argtypes = [d]; lib.orc_f64_to_bf16.restype = ctypes.c_uint16
    lib.orc_round.argtypes = [vp, i64, i32, vp]; lib.orc_round.restype = None
    lib.orc_codes.argtypes = [vp, i64, i64, i32, vp]; lib.orc_codes.restype = None
    lib.orc_dequant_f64.argtypes = [vp, vp, vp, i64, i64, i32, vp]; lib.orc_dequant_f64.restype = None
    lib.orc_dequant_f32.argtypes = [vp, vp, vp, i64, i64, i32, vp]; lib.orc_dequant_f32.restype = None
    lib.orc_pack_affine.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp]; lib.orc_pack_affine.restype = i64
    lib.orc_layernorm.argtypes = [vp, i64, i64, vp, vp, d, vp]; lib.orc_layernorm.restype = None
    lib.orc_gelu.argtypes = [d]; lib.orc_gelu.restype = d
    lib.orc_silu.argtypes = [d]; lib.orc_silu.restype = d
    lib.orc_linear.argtypes = [vp, i32, i64, i64, i64, i32, vp, i32, vp, vp, i32, vp, vp, d, i32, vp, vp, vp]
    lib.orc_linear.restype = i32
    lib.orc_gateup.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, d, vp]
    lib.orc_gateup.restype = i32
    lib.orc_attend.argtypes = [vp, vp, i32, i64, i64, i64, i64, i32, vp, vp]
    lib.orc_attend.restype = i32
    lib.orc_sample.argtypes = [vp, i32, i64, vp, ctypes.c_float, i64, vp, vp, i64, i64, i64, vp, vp, vp]
    lib.orc_sample.restype = i32
    lib.orc_kvq_decode.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, i32, i64, i64, i64, i64, i64, i32, vp]
    lib.orc_kvq_decode.restype = i32
    _lib = lib
    return lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- format helpers -------------------------------------------------------

def f16_to_f64(h: int) -> float:
    return load().orc_f16_to_f64(int(h))


def bf16_to_f64(h: int) -> float:
    return load().orc_bf16_to_f64(int(h))


def f64_to_f16(v: float) -> int:
    return load().orc_f64_to_f16(float(v))


def f64_to_bf16(v: float) -> int:
    return load().orc_f64_to_bf16(float(v))


def round_to(a, dtype: int) -> np.ndarray:
    """Round fp64 values to fp16 (1) or bf16 (2) bit patterns, ties to even."""
    a = _c(a, np.float64)
    out = np.empty(a.shape, np.uint16)
    load().orc_round(_p(a), a.size, dtype, _p(out))
    return out


def widen(bits, dtype: int) -> np.ndarray:
    """fp16/bf16 bit patterns (or fp32 values for dtype 0) -> fp64 values."""
    if dtype == F32:
        return np.asarray(bits, np.float32).astype(np.float64)
    lib = load()
    f = lib.orc_f16_to_f64 if dtype == F16 else lib.orc_bf16_to_f64
    flat = np.asarray(bits, np.uint16).ravel()
    return np.array([f(int(h)) for h in flat], np.float64).reshape(np.shape(bits))


# ---- quantization format --------------------------------------------------

def codes(words, N: int, K: int, bits: int) -> np.ndarray:
    words = _c(words, np.uint32)
    q = np.empty((N, K), np.uint8)
    load().orc_codes(_p(words), N, K, bits, _p(q))
    return q


def dequant_f64(words, scales, biases, N: int, K: int, bits: int) -> np.ndarray:
    words, scales, biases = _c(words, np.uint32), _c(scales, np.uint16), _c(biases, np.uint16)
    W = np.empty((N, K), np.float64)
    load().orc_dequant_f64(_p(words), _p(scales), _p(biases), N, K, bits, _p(W))
    return W


def dequant_f32(words, scales, biases, N: int, K: int, bits: int) -> np.ndarray:
    words, scales, biases = _c(words, np.uint32), _c(scales, np.uint16), _c(biases, np.uint16)
    W = np.empty((N, K), np.float32)
    load().orc_dequant_f32(_p(words), _p(scales), _p(biases), N, K, bits, _p(W))
    return W


def pack_affine(w, bits: int):
    """fp32 (N, K) -> (words (N, K*bits/32) uint32, scales (N, K/64) fp16 bits, biases, flag)."""
    w = _c(w, np.float32)
    N, K = w.shape
    words = np.zeros((N, K * bits // 32), np.uint32)
    scales = np.zeros((N, K // 64), np.uint16)
    biases = np.zeros((N, K // 64), np.uint16)
    flag = np.zeros(1, np.int32)
    load().orc_pack_affine(_p(w), N, K, bits, _p(words), _p(scales), _p(biases), _p(flag))
    return words, scales, biases, int(flag[0])


# ---- the path ---------------------------------------------------------------

def layernorm(x, gamma, beta, eps: float) -> np.ndarray:
    x, gamma, beta = _c(x, np.float64), _c(gamma, np.float64), _c(beta, np.float64)
    T, K = x.shape
    out = np.empty((T, K), np.float64)
    load().orc_layernorm(_p(x), T, K, _p(gamma), _p(beta), float(eps), _p(out))
    return out


def gelu(v: float) -> float:
    return load().orc_gelu(float(v))


def silu(g: float) -> float:
    return load().orc_silu(float(g))


def linear(x, x_dtype: int, bits: int, wdata, w_dtype: int = F16, scales=None, biases=None,
           gamma=None, beta=None, eps: float = 1e-5, act: int = 0, res=None, add=None) -> np.ndarray:
    """y (T, N) fp64 = [add +] [res +] act(LN?(x) @ W.T).  gamma/beta None means no LN."""
    x = _c(x, np.uint16)
    T, K = x.shape
    if bits == 16:
        wdata = _c(wdata, np.uint16)
        N = wdata.shape[0]
    else:
        wdata = _c(wdata, np.uint32)
        N = wdata.shape[0]
        scales, biases = _c(scales, np.uint16), _c(biases, np.uint16)
    has_ln = gamma is not None
    if has_ln:
        gamma, beta = _c(gamma, np.uint16), _c(beta, np.uint16)
    if res is not None:
        res = _c(res, np.uint16)
    if add is not None:
        add = _c(add, np.uint16)
    y = np.empty((T, N), np.float64)
    rc = load().orc_linear(_p(x), x_dtype, T, K, N, bits, _p(wdata), w_dtype, _p(scales), _p(biases),
                           int(has_ln), _p(gamma), _p(beta), float(eps), int(act), _p(res), _p(add), _p(y))
    if rc != 0:
        raise ValueError("oracle.linear: unsupported arguments")
    return y


def gateup(x, x_dtype: int, bits: int, gate, up, w_dtype: int = F16,
           gamma=None, beta=None, eps: float = 1e-5) -> np.ndarray:
    """y (T, N) fp64 = silu(LN?(x) @ Wg.T) * (LN?(x) @ Wu.T).

    gate / up: (data, scales, biases) tuples (scales/biases None for dense)."""
    x = _c(x, np.uint16)
    T, K = x.shape
    gd, gs, gb = gate
    ud, us, ub = up
    if bits == 16:
        gd, ud = _c(gd, np.uint16), _c(ud, np.uint16)
    else:
        gd, ud = _c(gd, np.uint32), _c(ud, np.uint32)
        gs, gb, us, ub = (_c(a, np.uint16) for a in (gs, gb, us, ub))
    N = gd.shape[0]
    has_ln = gamma is not None
    if has_ln:
        gamma, beta = _c(gamma, np.uint16), _c(beta, np.uint16)
    y = np.empty((T, N), np.float64)
    rc = load().orc_gateup(_p(x), x_dtype, T, K, N, bits, _p(gd), _p(gs), _p(gb), _p(ud), _p(us), _p(ub),
                           w_dtype, int(has_ln), _p(gamma), _p(beta), float(eps), _p(y))
    if rc != 0:
        raise ValueError("oracle.gateup: unsupported arguments")
    return y


def mlp(x, x_dtype: int, bits: int, gate, up, down, down_bits: int = None, w_dtype: int = F16,
        gamma=None, beta=None, eps: float = 1e-5, res=None):
    """[p3] mlx-bun 0.0.10 -> 0.0.12, model/fused-mlp-kernel.ts (the whole MLP of its header
    comment): h = silu(LN?(x) @ Wg.T) * (LN?(x) @ Wu.T), rounded once (RNE) to the activation
    dtype as the page rounds the hidden activation to bf16; then y = [res +] h @ Wd.T.
    gate / up / down: (data, scales, biases) tuples.  Returns (h bit patterns, y fp64)."""
    h64 = gateup(x, x_dtype, bits, gate, up, w_dtype, gamma, beta, eps)
    h = round_to(h64, x_dtype)
    dd, ds, db = down
    y = linear(h, x_dtype, bits if down_bits is None else down_bits, dd, w_dtype, ds, db, res=res)
    return h, y


def attend(qkv, kv, dtype: int, heads: int, head_dim: int, last: bool = False):
    """[p1] `attend`: qkv (T, 3D) and kv (2, H, P, HD) or None as fp16/bf16 bit patterns ->
    (out (T, D) fp64, or (1, D) with last; kv_out (2, H, P + T, HD) bit patterns)."""
    qkv = _c(qkv, np.uint16)
    T = qkv.shape[0]
    D = heads * head_dim
    if qkv.shape[1] != 3 * D:
        raise ValueError("oracle.attend: qkv must be (T, 3 * heads * head_dim)")
    P = 0 if kv is None else kv.shape[2]
    if kv is not None:
        kv = _c(kv, np.uint16)
    out = np.empty((1 if last else T, D), np.float64)
    kv_out = np.empty((2, heads, P + T, head_dim), np.uint16)
    rc = load().orc_attend(_p(qkv), _p(kv), dtype, P, T, heads, head_dim, int(last), _p(out), _p(kv_out))
    if rc != 0:
        raise ValueError("oracle.attend: unsupported arguments")
    return out, kv_out


def sample(logits, dtype: int, gumbel, inv_temp: float, top_k: int, table=None, prefix=None):
    """[p1] `sample`: logits (n,) as fp32 values (dtype 0) or fp16/bf16 bit patterns; gumbel
    (n,) float32 noise of this level; table (n, D) / prefix (n_prev, D) arrays of one dtype
    (their bytes are copied).  Returns (code, out (n_prev [+ 1], D), kept count)."""
    if dtype == F32:
        logits = _c(logits, np.float32)
    else:
        logits = _c(logits, np.uint16)
    gumbel = _c(gumbel, np.float32)
    n = logits.shape[0]
    ref = table if table is not None else prefix
    D = 0 if ref is None else ref.shape[1]
    edt = np.uint16 if ref is None else ref.dtype
    es = np.dtype(edt).itemsize
    n_prev = 0 if prefix is None else prefix.shape[0]
    if table is not None:
        table = np.ascontiguousarray(table)
    if prefix is not None:
        prefix = np.ascontiguousarray(prefix)
    out = np.zeros((n_prev + (1 if table is not None else 0), D), edt)
    code = np.zeros(1, np.int32)
    kept = np.zeros(1, np.int64)
    lib = load()
    rc = lib.orc_sample(_p(logits), dtype, n, _p(gumbel), ctypes.c_float(inv_temp), top_k, _p(table), _p(prefix),
                        n_prev, D, es, _p(out), _p(code), _p(kept))
    if rc != 0:
        raise ValueError("oracle.sample: unsupported arguments")
    return int(code[0]), out, int(kept[0])


def kvq_decode(q, q_dtype: int, k, v, sb_dtype: int, kv_heads: int, group: int, bits: int) -> np.ndarray:
    """[p3] fused-decode-kernel.ts: attention of one query position per head over a quantized
    K/V cache.  q (H, D) bit patterns; k, v: (codes (KV, N, D*bits/32) uint32, scales,
    biases (KV, N, D/group) bit patterns of sb_dtype).  Returns out (H, D) fp64."""
    q = _c(q, np.uint16)
    H, D = q.shape
    kc, ks, kb = (_c(k[0], np.uint32), _c(k[1], np.uint16), _c(k[2], np.uint16))
    vc, vs, vb = (_c(v[0], np.uint32), _c(v[1], np.uint16), _c(v[2], np.uint16))
    N = kc.shape[1]
    out = np.empty((H, D), np.float64)
    rc = load().orc_kvq_decode(_p(q), q_dtype, _p(kc), _p(ks), _p(kb), _p(vc), _p(vs), _p(vb), sb_dtype, H,
                               kv_heads, N, D, group, bits, _p(out))
    if rc != 0:
        raise ValueError("oracle.kvq_decode: unsupported arguments")
    return out
