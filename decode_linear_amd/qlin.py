"""Python binding of libqlin (include/qlin.h): argument marshalling only.

Every computation runs in the library's HIP kernels; PyTorch supplies device
memory and the current HIP stream.  The names follow the C ABI:
qlin_linear, qlin_gateup_swiglu, qlin_pack_affine, qlin_unpack_affine,
qlin_mlp, qlin_sample, qlin_kvq_decode, qlin_kvq_decode_noalloc, qlin_attend, qlin_check, qlin_attend_check, qlin_stream_read, qlin_stream_read_config, qlin_status_string,
qlin_dispatch_count, qlin_set_path, qlin_merge_timeouts, qlin_set_merge_spin_limit,
and the chain calls
(QlinChain wraps qlin_chain_create / launch / destroy).

There is no fallback: if libqlin.so is missing or a call fails, this raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

# QLIN_LIB_PATH names another build of the same library (the sanitizer test loads one).
LIB_PATH = os.environ.get("QLIN_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlin.so")

QLIN_F32, QLIN_F16, QLIN_BF16 = 0, 1, 2
QLIN_ACT_NONE, QLIN_ACT_GELU = 0, 1
STATUS = {0: "QLIN_OK", -1: "QLIN_ERR_NULL", -2: "QLIN_ERR_SHAPE", -3: "QLIN_ERR_DTYPE", -4: "QLIN_ERR_BITS",
          -5: "QLIN_ERR_ALIGN", -6: "QLIN_ERR_HIP", -7: "QLIN_ERR_ARG", -8: "QLIN_ERR_SCRATCH"}
QLIN_KVQ_SCRATCH_BYTES = 8 << 20

_TORCH_TO_QLIN = {torch.float32: QLIN_F32, torch.float16: QLIN_F16, torch.bfloat16: QLIN_BF16}
_QLIN_TO_TORCH = {v: k for k, v in _TORCH_TO_QLIN.items()}


class QlinError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({qlin_status_string(status)})")


class _Weight(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group_size", ctypes.c_int32), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64), ("dtype", ctypes.c_int32), ("data", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p)]


class _Ln(ctypes.Structure):
    _fields_ = [("gamma", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("eps", ctypes.c_float)]


class _Pass(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("T", ctypes.c_int32), ("w", _Weight), ("ln_gamma", ctypes.c_void_p),
                ("ln_beta", ctypes.c_void_p), ("ln_eps", ctypes.c_float), ("act", ctypes.c_int32),
                ("residual", ctypes.c_void_p), ("add", ctypes.c_void_p), ("y", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libqlin.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libqlin.so not found at {LIB_PATH}; build it with decode_linear_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    W, Ln = ctypes.POINTER(_Weight), ctypes.POINTER(_Ln)
    L.qlin_linear.argtypes = [vp, i32, i32, W, Ln, i32, vp, vp, vp, i32, vp]
    L.qlin_gateup_swiglu.argtypes = [vp, i32, i32, W, W, Ln, vp, i32, vp]
    L.qlin_pack_affine.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, i32, vp, vp]
    L.qlin_unpack_affine.argtypes = [W, vp, vp]
    L.qlin_check.argtypes = [vp, i32, i32, W, W, Ln, i32, vp, vp, vp, i32]
    L.qlin_attend.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp, i32, vp, vp]
    L.qlin_attend_check.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp, i32, vp]
    L.qlin_chain_create.argtypes = [ctypes.POINTER(_Pass), i32, i32, i32, vp, ctypes.POINTER(vp)]
    L.qlin_chain_launch.argtypes = [vp, vp]
    L.qlin_chain_passes.argtypes = [vp]
    L.qlin_chain_destroy.argtypes = [vp]
    L.qlin_chain_destroy.restype = None
    L.qlin_stream_read.argtypes = [vp, i64, vp, vp]
    L.qlin_stream_read_config.argtypes = [vp, i64, vp, i32, i32, i32, vp]
    L.qlin_mlp.argtypes = [vp, i32, i32, W, W, W, Ln, vp, vp, vp, i32, vp]
    L.qlin_sample.argtypes = [vp, i32, i32, vp, ctypes.c_float, i32, vp, vp, i32, i32, i32, vp, vp, vp]
    L.qlin_kvq_decode_workspace.argtypes = [i32, i32, i32]
    L.qlin_kvq_decode_workspace.restype = i64
    L.qlin_kvq_decode.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp, i64, vp,
                                  i32, vp]
    L.qlin_kvq_decode_noalloc.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp,
                                          i32, vp]
    L.qlin_set_path.argtypes = [i32]
    L.qlin_set_path.restype = i32
    L.qlin_merge_timeouts.argtypes = [i32]
    L.qlin_merge_timeouts.restype = i64
    L.qlin_set_merge_spin_limit.argtypes = [i32]
    L.qlin_set_merge_spin_limit.restype = i32
    L.qlin_dispatch_count.argtypes = [i32]
    L.qlin_dispatch_count.restype = i64
    L.qlin_status_string.argtypes = [i32]
    L.qlin_status_string.restype = ctypes.c_char_p
    for name in ("qlin_linear", "qlin_gateup_swiglu", "qlin_pack_affine", "qlin_unpack_affine", "qlin_check",
                 "qlin_attend", "qlin_attend_check", "qlin_chain_create", "qlin_chain_launch", "qlin_chain_passes",
                 "qlin_stream_read", "qlin_stream_read_config", "qlin_mlp", "qlin_sample", "qlin_kvq_decode",
                 "qlin_kvq_decode_noalloc"):
        getattr(L, name).restype = i32
    _lib = L
    return L


def qlin_status_string(status: int) -> str:
    return lib().qlin_status_string(int(status)).decode()


def qlin_dispatch_count(which: int) -> int:
    return int(lib().qlin_dispatch_count(int(which)))


def qlin_merge_timeouts(reset: bool = False) -> int:
    """Merge waits of the general kernel that gave up on the current device (see qlin.h)."""
    return int(lib().qlin_merge_timeouts(1 if reset else 0))


def qlin_set_merge_spin_limit(limit: int) -> int:
    return int(lib().qlin_set_merge_spin_limit(int(limit)))


def qlin_set_path(path: int) -> int:
    """0: automatic kernel choice (the default); 1: always the general kernel.  Returns the
    previous setting."""
    prev = int(lib().qlin_set_path(int(path)))
    if prev < 0:
        raise ValueError(f"qlin_set_path: unknown path {path}")
    return prev


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _TORCH_TO_QLIN:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _TORCH_TO_QLIN[t.dtype]


@dataclass
class QWeight:
    """A weight in the library's format.  bits 16: data (N, K) fp16/bf16; bits 8/4: data
    (N, K*bits/32) int32 words (bit pattern of uint32), scales/biases (N, K/64) fp16."""
    bits: int
    N: int
    K: int
    data: torch.Tensor
    scales: Optional[torch.Tensor] = None
    biases: Optional[torch.Tensor] = None

    def c(self) -> _Weight:
        if self.bits == 16:
            dt = _dtype(self.data)
        else:
            dt = QLIN_F16 if self.scales is None else _dtype(self.scales)
        return _Weight(self.bits, 64, self.N, self.K, dt, self.data.data_ptr() if self.data.numel() else None,
                       None if self.scales is None else self.scales.data_ptr(),
                       None if self.biases is None else self.biases.data_ptr())

    @property
    def nbytes(self) -> int:
        n = self.data.numel() * self.data.element_size()
        for t in (self.scales, self.biases):
            if t is not None:
                n += t.numel() * t.element_size()
        return n


def _ln(ln) -> Optional[_Ln]:
    if ln is None:
        return None
    gamma, beta, eps = ln
    return _Ln(gamma.data_ptr(), beta.data_ptr(), float(eps))


def _check(status: int, where: str):
    if status != 0:
        raise QlinError(status, where)


_ACT_DTYPES = (torch.float16, torch.bfloat16)
_OUT_DTYPES = (torch.float32, torch.float16, torch.bfloat16)


class _Args:
    """Checks of one call's tensors, raised as ValueError before anything is launched (the C
    ABI sees only pointers and sizes, so a tensor's shape can only be checked here).  Shapes,
    contiguity and dtypes first, for every argument; then that all of them sit on one GPU.
    The passing path is a few attribute reads per tensor; messages are built on failure."""

    __slots__ = ("where", "devs", "names")

    def __init__(self, where: str):
        self.where = where
        self.devs = []
        self.names = []

    def fail(self, msg: str):
        raise ValueError(f"{self.where}: {msg}")

    def need(self, name: str, t, shape, dtypes=None, optional=False):
        """t: a contiguous tensor of `shape` (None entries: any size) and one of `dtypes`."""
        if t is None:
            if optional:
                return
            self.fail(f"{name} is required")
        if not isinstance(t, torch.Tensor):
            self.fail(f"{name} must be a torch.Tensor")
        sh = t.shape
        if None in shape:
            ok = len(sh) == len(shape) and all(e is None or a == e for a, e in zip(sh, shape))
        else:
            ok = sh == shape
        if not ok:
            want = "(" + ", ".join("*" if e is None else str(e) for e in shape) + ")"
            self.fail(f"{name} must have shape {want}, got {tuple(sh)}")
        if not t.is_contiguous():
            self.fail(f"{name} must be contiguous")
        if dtypes is not None and t.dtype not in dtypes:
            self.fail(f"{name} has dtype {t.dtype}, expected one of {list(dtypes)}")
        self.devs.append(t.get_device())   # -1 on the CPU
        self.names.append(name)

    def weight(self, name: str, w, K: Optional[int] = None):
        if not isinstance(w, QWeight):
            self.fail(f"{name} must be a QWeight")
        bits = w.bits
        if bits not in (4, 8, 16):
            self.fail(f"{name}.bits must be 4, 8 or 16, got {bits}")
        if K is not None and w.K != K:
            self.fail(f"{name}.K = {w.K} does not match the activation row length {K}")
        if w.K <= 0 or w.K % 64 or w.N < 0:
            self.fail(f"{name} must have K a positive multiple of 64 and N >= 0")
        if bits == 16:
            self.need(f"{name}.data", w.data, (w.N, w.K), _ACT_DTYPES)
        else:
            self.need(f"{name}.data", w.data, (w.N, w.K * bits // 32), _I32)
            self.need(f"{name}.scales", w.scales, (w.N, w.K // 64), _F16)
            self.need(f"{name}.biases", w.biases, (w.N, w.K // 64), _F16)

    def ln(self, ln, K: int, dtype):
        if ln is None:
            return
        if not isinstance(ln, (tuple, list)) or len(ln) != 3:
            self.fail("ln must be (gamma, beta, eps)")
        self.need("gamma", ln[0], (K,), (dtype,))
        self.need("beta", ln[1], (K,), (dtype,))

    def on_one_gpu(self):
        devs = self.devs
        if not devs:
            return
        d0 = devs[0]
        if d0 >= 0 and devs.count(d0) == len(devs):
            return
        for name, d in zip(self.names, devs):
            if d < 0:
                self.fail(f"{name} must be on a GPU, got cpu")
        for name, d in zip(self.names, devs):
            if d != d0:
                self.fail(f"{name} is on cuda:{d}, the other arguments on cuda:{d0}")


_I32 = (torch.int32,)
_F16 = (torch.float16,)


def qlin_linear(x: torch.Tensor, w: QWeight, ln=None, act: int = QLIN_ACT_NONE,
                residual: Optional[torch.Tensor] = None, add: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None, stream=None) -> torch.Tensor:
    """y (T, N) = [add +] [residual +] act(LN?(x) @ W.T).  ln = (gamma, beta, eps) or None."""
    c = _Args("qlin_linear")
    c.need("x", x, (None, None), _ACT_DTYPES)
    T = x.shape[0]
    c.weight("w", w, x.shape[1])
    c.ln(ln, w.K, x.dtype)
    c.need("residual", residual, (T, w.N), (x.dtype,), optional=True)
    c.need("add", add, (w.N,), (x.dtype,), optional=True)
    c.need("out", out, (T, w.N), _OUT_DTYPES, optional=True)
    c.on_one_gpu()
    if out is None:
        out = torch.empty((T, w.N), dtype=out_dtype or x.dtype, device=x.device)
    lnc = _ln(ln)
    wc = w.c()
    st = lib().qlin_linear(_ptr(x), _dtype(x), T, ctypes.byref(wc), None if lnc is None else ctypes.byref(lnc),
                           int(act), _ptr(residual), _ptr(add), _ptr(out), _dtype(out), _stream(stream))
    _check(st, "qlin_linear")
    return out


def qlin_gateup_swiglu(x: torch.Tensor, gate: QWeight, up: QWeight, ln=None, out: Optional[torch.Tensor] = None,
                       out_dtype: Optional[torch.dtype] = None, stream=None) -> torch.Tensor:
    """y (T, N) = silu(LN?(x) @ Wg.T) * (LN?(x) @ Wu.T)."""
    c = _Args("qlin_gateup_swiglu")
    c.need("x", x, (None, None), _ACT_DTYPES)
    T = x.shape[0]
    c.weight("gate", gate, x.shape[1])
    c.weight("up", up, x.shape[1])
    if (gate.bits, gate.N) != (up.bits, up.N):
        c.fail("gate and up must have the same bits and N")
    c.ln(ln, gate.K, x.dtype)
    c.need("out", out, (T, gate.N), _OUT_DTYPES, optional=True)
    c.on_one_gpu()
    if out is None:
        out = torch.empty((T, gate.N), dtype=out_dtype or x.dtype, device=x.device)
    lnc = _ln(ln)
    gc, uc = gate.c(), up.c()
    st = lib().qlin_gateup_swiglu(_ptr(x), _dtype(x), T, ctypes.byref(gc), ctypes.byref(uc),
                                  None if lnc is None else ctypes.byref(lnc), _ptr(out), _dtype(out), _stream(stream))
    _check(st, "qlin_gateup_swiglu")
    return out


def qlin_mlp(x: torch.Tensor, gate: QWeight, up: QWeight, down: QWeight, ln=None,
             residual: Optional[torch.Tensor] = None, h: Optional[torch.Tensor] = None,
             out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None, stream=None):
    """(y, h): h (T, I) = silu(LN?(x) @ Wg.T) * (LN?(x) @ Wu.T) in x's dtype, then
    y (T, Hout) = [residual +] h @ Wd.T (two dispatches; h is the caller's workspace)."""
    c = _Args("qlin_mlp")
    c.need("x", x, (None, None), _ACT_DTYPES)
    T = x.shape[0]
    c.weight("gate", gate, x.shape[1])
    c.weight("up", up, x.shape[1])
    if (gate.bits, gate.N) != (up.bits, up.N):
        c.fail("gate and up must have the same bits and N")
    c.weight("down", down, gate.N)
    c.ln(ln, gate.K, x.dtype)
    c.need("residual", residual, (T, down.N), (x.dtype,), optional=True)
    c.need("h", h, (T, gate.N), (x.dtype,), optional=True)
    c.need("out", out, (T, down.N), _OUT_DTYPES, optional=True)
    c.on_one_gpu()
    if h is None:
        h = torch.empty((T, gate.N), dtype=x.dtype, device=x.device)
    if out is None:
        out = torch.empty((T, down.N), dtype=out_dtype or x.dtype, device=x.device)
    lnc = _ln(ln)
    gc, uc, dc = gate.c(), up.c(), down.c()
    st = lib().qlin_mlp(_ptr(x), _dtype(x), T, ctypes.byref(gc), ctypes.byref(uc), ctypes.byref(dc),
                        None if lnc is None else ctypes.byref(lnc), _ptr(residual), _ptr(h), _ptr(out), _dtype(out),
                        _stream(stream))
    _check(st, "qlin_mlp")
    return out, h


def qlin_attend(qkv: torch.Tensor, kv: Optional[torch.Tensor], heads: int, head_dim: int, last: bool = False,
                out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                kv_out: Optional[torch.Tensor] = None, stream=None):
    """(out, kv_out) of one attention pass: kv_out (2, H, P + T, HD) = the cache with this
    pass's keys and values appended; out (T, D), or (1, D) with last, = causal softmax
    attention of the new positions.  qkv (T, 3D); kv (2, H, P, HD) or None."""
    T = qkv.shape[0]
    D = heads * head_dim
    P = 0 if kv is None else kv.shape[2]
    # shapes are checked here because the C ABI sees only pointers and sizes
    if qkv.dim() != 2 or qkv.shape[1] != 3 * D or not qkv.is_contiguous():
        raise ValueError("qlin_attend: qkv must be a contiguous (T, 3 * heads * head_dim) tensor")
    if kv is not None and (tuple(kv.shape) != (2, heads, P, head_dim) or not kv.is_contiguous()
                           or kv.dtype != qkv.dtype):
        raise ValueError("qlin_attend: kv must be a contiguous (2, heads, P, head_dim) tensor of qkv's dtype")
    rows = 1 if last else T
    if out is None:
        out = torch.empty((rows, D), dtype=out_dtype or qkv.dtype, device=qkv.device)
    elif tuple(out.shape) != (rows, D) or not out.is_contiguous():
        raise ValueError("qlin_attend: out must be a contiguous (T or 1, heads * head_dim) tensor")
    if kv_out is None:
        kv_out = torch.empty((2, heads, P + T, head_dim), dtype=qkv.dtype, device=qkv.device)
    elif tuple(kv_out.shape) != (2, heads, P + T, head_dim) or not kv_out.is_contiguous() or kv_out.dtype != qkv.dtype:
        raise ValueError("qlin_attend: kv_out must be a contiguous (2, heads, P + T, head_dim) tensor of qkv's dtype")
    st = lib().qlin_attend(_ptr(qkv), _ptr(kv), _dtype(qkv), P, T, heads, head_dim, int(bool(last)), _ptr(out),
                           _dtype(out), _ptr(kv_out), _stream(stream))
    _check(st, "qlin_attend")
    return out, kv_out


def qlin_pack_affine(w: torch.Tensor, bits: int, flag: Optional[torch.Tensor] = None, stream=None) -> QWeight:
    """Quantize an fp32 (N, K) device tensor to the affine group-64 format."""
    c = _Args("qlin_pack_affine")
    c.need("w", w, (None, None), (torch.float32,))
    if bits not in (4, 8):
        c.fail(f"bits must be 4 or 8, got {bits}")
    N, K = w.shape
    dev = w.device
    if K <= 0 or K % 64:
        c.fail(f"K must be a positive multiple of 64, got {K}")
    c.need("flag", flag, (None,), (torch.int32,), optional=True)
    c.on_one_gpu()
    codes = torch.empty((N, K * bits // 32), dtype=torch.int32, device=dev)
    scales = torch.empty((N, K // 64), dtype=torch.float16, device=dev)
    biases = torch.empty((N, K // 64), dtype=torch.float16, device=dev)
    st = lib().qlin_pack_affine(_ptr(w), N, K, bits, 64, _ptr(codes), _ptr(scales), _ptr(biases), QLIN_F16,
                                _ptr(flag), _stream(stream))
    _check(st, "qlin_pack_affine")
    return QWeight(bits, N, K, codes, scales, biases)


def qlin_unpack_affine(w: QWeight, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """fp32 (N, K) = fmaf(q, s, b) (or the widened dense element)."""
    c = _Args("qlin_unpack_affine")
    c.weight("w", w)
    c.need("out", out, (w.N, w.K), (torch.float32,), optional=True)
    c.on_one_gpu()
    if out is None:
        out = torch.empty((w.N, w.K), dtype=torch.float32, device=w.data.device)
    wc = w.c()
    st = lib().qlin_unpack_affine(ctypes.byref(wc), _ptr(out), _stream(stream))
    _check(st, "qlin_unpack_affine")
    return out


def qlin_check(x_ptr, x_dtype: int, T: int, w: _Weight, up: Optional[_Weight] = None, ln: Optional[_Ln] = None,
               act: int = 0, residual=None, add=None, y_ptr=None, y_dtype: int = QLIN_BF16) -> int:
    """Validation only (no GPU needed).  Takes raw ctypes structs / addresses."""
    return int(lib().qlin_check(x_ptr, x_dtype, T, ctypes.byref(w), None if up is None else ctypes.byref(up),
                                None if ln is None else ctypes.byref(ln), act, residual, add, y_ptr, y_dtype))


class QlinChain:
    """A hipGraph of dependent qlin_linear passes (qlin_chain_create / launch / destroy).

    passes: dicts with keys x, T, w (QWeight), ln (tuple or None), act, residual, add, y."""

    def __init__(self, passes: Sequence[dict], x_dtype: torch.dtype, y_dtype: torch.dtype, capture_stream=None):
        c = _Args("QlinChain")
        if x_dtype not in _ACT_DTYPES or y_dtype not in _OUT_DTYPES:
            c.fail("x_dtype must be float16 or bfloat16, y_dtype one of those or float32")
        for i, ps in enumerate(passes):
            w, T, x = ps["w"], int(ps["T"]), ps["x"]
            c.need(f"passes[{i}].x", x, (None, None), (x_dtype,))
            c.weight(f"passes[{i}].w", w, x.shape[1])
            c.ln(ps.get("ln"), w.K, x_dtype)
            c.need(f"passes[{i}].residual", ps.get("residual"), (None, w.N), (x_dtype,), optional=True)
            c.need(f"passes[{i}].add", ps.get("add"), (w.N,), (x_dtype,), optional=True)
            c.need(f"passes[{i}].y", ps["y"], (None, w.N), (y_dtype,))
            for name in ("x", "y", "residual"):
                if ps.get(name) is not None and ps[name].shape[0] < T:
                    c.fail(f"passes[{i}].{name} has fewer than T = {T} rows")
        c.on_one_gpu()
        self._keep = list(passes)
        arr = (_Pass * len(passes))()
        for i, ps in enumerate(passes):
            ln = ps.get("ln")
            arr[i] = _Pass(ps["x"].data_ptr(), ps["T"], ps["w"].c(), None if ln is None else ln[0].data_ptr(),
                           None if ln is None else ln[1].data_ptr(), 0.0 if ln is None else float(ln[2]),
                           int(ps.get("act", 0)), None if ps.get("residual") is None else ps["residual"].data_ptr(),
                           None if ps.get("add") is None else ps["add"].data_ptr(), ps["y"].data_ptr())
        self._stream = capture_stream or torch.cuda.Stream()
        handle = ctypes.c_void_p()
        st = lib().qlin_chain_create(arr, len(passes), _TORCH_TO_QLIN[x_dtype], _TORCH_TO_QLIN[y_dtype],
                                     _stream(self._stream), ctypes.byref(handle))
        _check(st, "qlin_chain_create")
        self._h = handle

    @property
    def passes(self) -> int:
        return int(lib().qlin_chain_passes(self._h))

    def launch(self, stream=None):
        _check(lib().qlin_chain_launch(self._h, _stream(stream)), "qlin_chain_launch")

    def close(self):
        if getattr(self, "_h", None):
            lib().qlin_chain_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


STREAM_READ_BLOCKS = 1024


def qlin_stream_read(buf: torch.Tensor, partial: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One plain 16-byte streaming read of buf (the device's read ceiling); returns the
    (STREAM_READ_BLOCKS,) int32 tensor of per-block XOR folds (entries past the launch's
    blocks are left as they were)."""
    if partial is None:
        partial = torch.zeros(STREAM_READ_BLOCKS, dtype=torch.int32, device=buf.device)
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    st = lib().qlin_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(partial), _stream(stream))
    if st != 0:
        raise QlinError(st, "qlin_stream_read")
    return partial


def qlin_stream_read_config(buf: torch.Tensor, blocks: int, unroll: int, nontemporal: bool,
                            partial: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """qlin_stream_read with its launch chosen: blocks of 512 threads, unroll loads in flight
    per thread, non-temporal or ordinary loads."""
    if partial is None:
        partial = torch.zeros(STREAM_READ_BLOCKS, dtype=torch.int32, device=buf.device)
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    st = lib().qlin_stream_read_config(_ptr(buf), buf.numel() * buf.element_size(), _ptr(partial), int(blocks),
                                       int(unroll), 1 if nontemporal else 0, _stream(stream))
    if st != 0:
        raise QlinError(st, "qlin_stream_read_config")
    return partial


def qlin_sample(logits: torch.Tensor, gumbel: torch.Tensor, level: int, table: Optional[torch.Tensor],
                prefix: Optional[torch.Tensor], inv_temp: float, top_k: int, embed: bool = True,
                out: Optional[torch.Tensor] = None, code: Optional[torch.Tensor] = None, stream=None):
    """One sampling step ([p1] `sample`): logits (n,) or (1, n); gumbel (levels, n) fp32 (row
    `level` is used); table (levels, n, D) (slice `level`) or None; prefix (n_prev, D) or
    None.  Returns (code (1,) int32, out = prefix + [table[level, code]] (n_prev + 1, D), or
    the prefix when embed is False)."""
    lg = logits.reshape(-1)
    n = lg.numel()
    g = gumbel[level]
    tb = table[level] if (embed and table is not None) else None
    ref = tb if tb is not None else prefix
    D = 0 if ref is None else ref.shape[-1]
    n_prev = 0 if prefix is None else prefix.shape[0]
    edt = ref.dtype if ref is not None else torch.float16
    if code is None:
        code = torch.empty(1, dtype=torch.int32, device=lg.device)
    if out is None and (tb is not None or n_prev > 0):
        out = torch.empty((n_prev + (1 if tb is not None else 0), D), dtype=edt, device=lg.device)
    for t in (lg, g, tb, prefix, out):
        if t is not None and not t.is_contiguous():
            raise ValueError("qlin_sample: tensors must be contiguous")
    st = lib().qlin_sample(_ptr(lg), _dtype(lg), n, _ptr(g), ctypes.c_float(inv_temp), int(top_k), _ptr(tb),
                           _ptr(prefix), n_prev, D, _TORCH_TO_QLIN[edt], _ptr(out), _ptr(code), _stream(stream))
    _check(st, "qlin_sample")
    return code, out


def qlin_kvq_decode(q: torch.Tensor, k, v, kv_heads: int, group: int, bits: int, out: Optional[torch.Tensor] = None,
                    out_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Attention of one query position per head over a quantized K/V cache: q (H, D); k, v =
    (codes (KV, N, D*bits/32) int32, scales, biases (KV, N, D/group) fp16 or bf16).  Returns
    out (H, D)."""
    H, D = q.shape
    kc, ks, kb = k
    vc, vs, vb = v
    N = kc.shape[1]
    need = int(lib().qlin_kvq_decode_workspace(H, N, D))
    if workspace is None:
        workspace = torch.empty(max(need, 4) // 4, dtype=torch.float32, device=q.device)
    if out is None:
        out = torch.empty((H, D), dtype=out_dtype or q.dtype, device=q.device)
    for t in (q, kc, ks, kb, vc, vs, vb, out):
        if not t.is_contiguous():
            raise ValueError("qlin_kvq_decode: tensors must be contiguous")
    st = lib().qlin_kvq_decode(_ptr(q), _dtype(q), H, kv_heads, N, D, group, bits, _ptr(kc), _ptr(ks), _ptr(kb),
                               _ptr(vc), _ptr(vs), _ptr(vb), _dtype(ks), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _ptr(out), _dtype(out),
                               _stream(stream))
    _check(st, "qlin_kvq_decode")
    return out


def qlin_kvq_decode_noalloc(q: torch.Tensor, k, v, kv_heads: int, group: int, bits: int, out: torch.Tensor,
                            stream=None):
    """qlin_kvq_decode with the library's static device scratch instead of a workspace: the
    call allocates nothing (out is the caller's).  Calls that overlap on one GPU race."""
    H, D = q.shape
    kc, ks, kb = k
    vc, vs, vb = v
    N = kc.shape[1]
    for t in (q, kc, ks, kb, vc, vs, vb, out):
        if not t.is_contiguous():
            raise ValueError("qlin_kvq_decode_noalloc: tensors must be contiguous")
    st = lib().qlin_kvq_decode_noalloc(_ptr(q), _dtype(q), H, kv_heads, N, D, group, bits, _ptr(kc), _ptr(ks),
                                       _ptr(kb), _ptr(vc), _ptr(vs), _ptr(vb), _dtype(ks), _ptr(out), _dtype(out),
                                       _stream(stream))
    _check(st, "qlin_kvq_decode_noalloc")
    return out
