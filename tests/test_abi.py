"""CPU checks of the C-ABI library: it loads, exports every entry point that
include/qlin.h declares, and rejects bad arguments on the host before any HIP call
(status codes only; nothing is launched, so no GPU is needed)."""
import ctypes
import os
import re

import pytest

from decode_linear_amd import build as qbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def q():
    qbuild.ensure_built()
    from decode_linear_amd import qlin
    return qlin


def _declared():
    src = open(os.path.join(ROOT, "include", "qlin.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qlin_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared()
    for must in ("qlin_linear", "qlin_gateup_swiglu", "qlin_pack_affine", "qlin_unpack_affine", "qlin_check",
                 "qlin_chain_create", "qlin_chain_launch", "qlin_chain_destroy", "qlin_status_string",
                 "qlin_dispatch_count", "qlin_attend", "qlin_attend_check", "qlin_stream_read", "qlin_mlp", "qlin_sample", "qlin_kvq_decode",
                 "qlin_stream_read_config", "qlin_set_path", "qlin_kvq_decode_noalloc"):
        assert must in names


def test_library_exports_every_declared_symbol(q):
    lib = q.lib()
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings(q):
    for s in range(-8, 1):
        assert q.qlin_status_string(s) and q.qlin_status_string(s) != "unknown status"
    assert q.qlin_status_string(0) == "ok"


# fake, suitably aligned device addresses: validation never dereferences them
X, W, S, B, Y, G, BE, R = (0x10000 * i for i in range(1, 9))


def _w(q, bits=8, N=256, K=1024, dtype=None, data=W, scales=S, biases=B, group=64):
    if dtype is None:
        dtype = q.QLIN_F16
    return q._Weight(bits, group, N, K, dtype, data, scales, biases)


def _chk(q, T=4, w=None, up=None, ln=None, act=0, res=None, add=None, x=X, y=Y, x_dtype=None, y_dtype=None):
    x_dtype = q.QLIN_BF16 if x_dtype is None else x_dtype
    y_dtype = q.QLIN_BF16 if y_dtype is None else y_dtype
    return q.qlin_check(x, x_dtype, T, w if w is not None else _w(q), up, ln, act, res, add, y, y_dtype)


def test_valid_calls_pass(q):
    assert _chk(q) == 0
    assert _chk(q, T=32, ln=q._Ln(G, BE, 1e-5), act=1, res=R, add=R + 0x100000) == 0
    assert _chk(q, w=_w(q, bits=4)) == 0
    assert _chk(q, w=_w(q, bits=16, dtype=q.QLIN_BF16)) == 0
    assert _chk(q, w=_w(q), up=_w(q)) == 0
    assert _chk(q, y_dtype=q.QLIN_F32) == 0


def test_empty_problems_are_no_ops(q):
    assert _chk(q, T=0, x=None, y=None) == 0
    assert _chk(q, w=_w(q, N=0, data=None, scales=None, biases=None), x=X) == 0


@pytest.mark.parametrize("T", [-1, 33, 1000])
def test_bad_T(q, T):
    assert _chk(q, T=T) == -2


@pytest.mark.parametrize("K", [0, 32, 100, 1 << 21])
def test_bad_K(q, K):
    assert _chk(q, w=_w(q, K=K)) == -2


def test_bad_N(q):
    assert _chk(q, w=_w(q, N=-5)) == -2


@pytest.mark.parametrize("bits", [0, 2, 3, 5, 12, 32])
def test_bad_bits(q, bits):
    assert _chk(q, w=_w(q, bits=bits)) == -4


def test_bad_group(q):
    assert _chk(q, w=_w(q, group=32)) == -4
    assert _chk(q, w=_w(q, group=128)) == -4


def test_dtypes(q):
    assert _chk(q, x_dtype=q.QLIN_F32) == -3                    # activations must be 16-bit
    assert _chk(q, x_dtype=7) == -3
    assert _chk(q, y_dtype=5) == -3
    assert _chk(q, w=_w(q, bits=16, dtype=q.QLIN_F16)) == -3   # dense W must match x (bf16 here)
    assert _chk(q, w=_w(q, bits=8, dtype=q.QLIN_BF16)) == -3   # scales/biases are fp16


def test_null_pointers(q):
    assert _chk(q, x=None) == -1
    assert _chk(q, y=None) == -1
    assert _chk(q, w=_w(q, data=None)) == -1
    assert _chk(q, w=_w(q, scales=None)) == -1
    assert _chk(q, ln=q._Ln(None, BE, 1e-5)) == -1
    assert q.lib().qlin_check(X, q.QLIN_BF16, 4, None, None, None, 0, None, None, Y, q.QLIN_BF16) == -1


def test_alignment(q):
    assert _chk(q, x=X + 2) == -5
    assert _chk(q, w=_w(q, data=W + 4)) == -5
    assert _chk(q, w=_w(q, scales=S + 1)) == -5
    assert _chk(q, ln=q._Ln(G + 8, BE, 1e-5)) == -5
    assert _chk(q, y=Y + 1) == -5
    assert _chk(q, y=Y + 2, y_dtype=q.QLIN_F32) == -5


def test_bad_act_eps_and_gateup_extras(q):
    assert _chk(q, act=2) == -7
    assert _chk(q, ln=q._Ln(G, BE, -1.0)) == -7
    assert _chk(q, ln=q._Ln(G, BE, float("nan"))) == -7
    assert _chk(q, w=_w(q), up=_w(q), act=1) == -7
    assert _chk(q, w=_w(q), up=_w(q), res=R) == -7


def test_gateup_shape_mismatch(q):
    assert _chk(q, w=_w(q), up=_w(q, N=128)) == -2
    assert _chk(q, w=_w(q), up=_w(q, bits=4)) == -4


def test_output_overlapping_input_rejected(q):
    assert _chk(q, y=X + 16) == -7
    assert _chk(q, res=Y, y=Y) == -7


def test_invalid_linear_call_returns_before_any_hip_call(q):
    # an invalid call goes through the real entry point without needing a device
    w = _w(q, K=100)
    st = q.lib().qlin_linear(X, q.QLIN_BF16, 4, ctypes.byref(w), None, 0, None, None, Y, q.QLIN_BF16, None)
    assert st == -2
    st = q.lib().qlin_pack_affine(None, 4, 64, 3, 64, None, None, None, q.QLIN_F16, None, None)
    assert st == -4
    st = q.lib().qlin_pack_affine(None, 4, 64, 8, 64, None, None, None, q.QLIN_F16, None, None)
    assert st == -1


def test_chain_argument_errors(q):
    h = ctypes.c_void_p()
    assert q.lib().qlin_chain_create(None, 1, 2, 2, None, ctypes.byref(h)) == -1
    arr = (q._Pass * 1)()
    assert q.lib().qlin_chain_create(arr, 0, 2, 2, ctypes.c_void_p(1), ctypes.byref(h)) == -7
    assert q.lib().qlin_chain_passes(None) == 0
    q.lib().qlin_chain_destroy(None)


def test_dispatch_counter_range(q):
    assert q.qlin_dispatch_count(10) == -1
    assert q.qlin_dispatch_count(-1) == -1
    assert q.qlin_dispatch_count(8) >= 0 and q.qlin_dispatch_count(9) >= 0
    assert q.qlin_dispatch_count(0) >= 0
    assert q.qlin_dispatch_count(7) >= 0


# attend: qkv, kv, out, kv_out at fake, 16-byte aligned addresses far apart
QKV, KV, AO, KVO = (0x1000000 * i for i in range(1, 5))


def _att(q, qkv=QKV, kv=KV, dtype=None, P=24, T=8, H=16, HD=64, last=0, out=AO, out_dtype=None, kv_out=KVO):
    dtype = q.QLIN_BF16 if dtype is None else dtype
    out_dtype = q.QLIN_BF16 if out_dtype is None else out_dtype
    return q.lib().qlin_attend_check(qkv, kv, dtype, P, T, H, HD, last, out, out_dtype, kv_out)


def test_attend_valid_calls(q):
    assert _att(q) == 0
    assert _att(q, P=0, kv=None, T=32) == 0
    assert _att(q, P=31, T=1, last=1, out_dtype=q.QLIN_F32) == 0
    assert _att(q, dtype=q.QLIN_F16, out_dtype=q.QLIN_F16, H=1, HD=512) == 0


@pytest.mark.parametrize("P,T", [(0, 0), (-1, 4), (30, 3), (0, 33), (32, 1)])
def test_attend_bad_positions(q, P, T):
    assert _att(q, P=P, T=T) == -2


@pytest.mark.parametrize("H,HD", [(0, 64), (16, 8), (16, 24), (16, 0), (1, 528), (70000, 16)])
def test_attend_bad_heads(q, H, HD):
    assert _att(q, H=H, HD=HD) == -2


def test_attend_dtypes_nulls_alignment_overlap(q):
    assert _att(q, dtype=q.QLIN_F32) == -3
    assert _att(q, out_dtype=7) == -3
    assert _att(q, last=2) == -7
    assert _att(q, qkv=None) == -1
    assert _att(q, kv=None) == -1              # P > 0 needs the cache
    assert _att(q, out=None) == -1
    assert _att(q, kv_out=None) == -1
    assert _att(q, qkv=QKV + 8) == -5
    assert _att(q, kv_out=KVO + 8) == -5
    assert _att(q, out=AO + 1) == -5
    assert _att(q, out=AO + 2, out_dtype=q.QLIN_F32) == -5
    assert _att(q, kv_out=QKV + 16) == -7
    assert _att(q, kv_out=KV + 64) == -7
    assert _att(q, out=KVO) == -7
    assert _att(q, out=QKV + 32) == -7


def test_invalid_attend_call_returns_before_any_hip_call(q):
    st = q.lib().qlin_attend(QKV, KV, q.QLIN_BF16, 30, 3, 16, 64, 0, AO, q.QLIN_BF16, KVO, None)
    assert st == -2


def test_stream_read_validation(q):
    f = q.lib().qlin_stream_read
    assert f(None, 1024, AO, None) == -1
    assert f(QKV, 1024, None, None) == -1
    assert f(QKV, 0, AO, None) == -2
    assert f(QKV, 1000, AO, None) == -2       # not a multiple of 16
    assert f(QKV + 8, 1024, AO, None) == -5
    assert f(QKV, 1024, AO + 2, None) == -5


def test_stream_read_config_validation(q):
    f = q.lib().qlin_stream_read_config
    assert f(None, 1024, AO, 4, 4, 1, None) == -1
    assert f(QKV, 1000, AO, 4, 4, 1, None) == -2
    assert f(QKV, 1024, AO, 0, 4, 1, None) == -7       # blocks below 1
    assert f(QKV, 1024, AO, 1025, 4, 1, None) == -7    # blocks past QLIN_STREAM_READ_BLOCKS
    assert f(QKV, 1024, AO, 4, 3, 1, None) == -7       # unroll not 1, 2, 4, 8 or 16
    assert f(QKV, 1024, AO, 4, 4, 2, None) == -7       # nontemporal not 0 or 1
    assert f(QKV + 8, 1024, AO, 4, 4, 1, None) == -5


def test_set_path_validation(q):
    f = q.lib().qlin_set_path
    assert f(3) == -1 and f(5) == -1 and f(-1) == -1
    prev = f(2)
    assert prev in (0, 1, 2)
    assert f(1) == 2
    assert f(prev) == 1


def test_mlp_validation(q):
    f = q.lib().qlin_mlp
    g = _w(q, bits=4, N=256, K=1024)
    u = _w(q, bits=4, N=256, K=1024, data=W + 0x100000, scales=S + 0x100000, biases=B + 0x100000)
    d = _w(q, bits=8, N=128, K=256, data=W + 0x200000, scales=S + 0x200000, biases=B + 0x200000)
    H = 0x3000000   # (only invalid calls here: a valid one would launch on fake addresses)
    bad_k = _w(q, bits=8, N=128, K=512, data=W + 0x200000, scales=S + 0x200000, biases=B + 0x200000)
    assert f(X, q.QLIN_BF16, 4, ctypes.byref(g), ctypes.byref(u), ctypes.byref(bad_k), None, None, H, Y,
             q.QLIN_BF16, None) == -2
    assert f(X, q.QLIN_BF16, 4, ctypes.byref(g), ctypes.byref(u), None, None, None, H, Y, q.QLIN_BF16, None) == -1
    assert f(X, q.QLIN_BF16, 4, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), None, None, None, Y,
             q.QLIN_BF16, None) == -1
    assert f(X, q.QLIN_BF16, 4, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), None, None, H + 8, Y,
             q.QLIN_BF16, None) == -5
    # h overlapping x, or y
    assert f(X, q.QLIN_BF16, 4, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), None, None, X + 64, Y,
             q.QLIN_BF16, None) == -7
    assert f(X, q.QLIN_BF16, 4, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), None, None, H, H + 64,
             q.QLIN_BF16, None) == -7


def test_sample_validation(q):
    f = q.lib().qlin_sample
    L, G, TB, P, O, C = (0x5000000 + 0x100000 * i for i in range(6))
    ok = dict(logits=L, dt=q.QLIN_BF16, n=2048, g=G, it=1.0, k=50, table=TB, prefix=P, n_prev=4, D=1024,
              edt=q.QLIN_BF16, out=O, code=C)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["logits"], a["dt"], a["n"], a["g"], ctypes.c_float(a["it"]), a["k"], a["table"], a["prefix"],
                 a["n_prev"], a["D"], a["edt"], a["out"], a["code"], None)
    # only invalid calls here: a valid one would launch on fake addresses
    assert call(logits=None) == -1 and call(g=None) == -1 and call(code=None) == -1
    assert call(n=0) == -2 and call(n=8193) == -2 and call(k=0) == -2 and call(k=2049) == -2
    assert call(D=4) == -2            # 8 bytes per row: not a multiple of 16
    assert call(n_prev=-1) == -2
    assert call(dt=7) == -3 and call(edt=9) == -3
    assert call(it=0.0) == -7 and call(it=float("inf")) == -7 and call(it=float("nan")) == -7
    assert call(logits=L + 1) == -5 and call(out=O + 8) == -5 and call(table=TB + 8) == -5
    assert call(prefix=None) == -1 and call(out=None) == -1
    assert call(out=P + 16) == -7     # overlaps the prefix without being it
    assert call(out=TB + 64) == -7    # overlaps the table
    assert call(code=L + 8) == -7     # code inside the logits


def test_kvq_validation(q):
    f, ws = q.lib().qlin_kvq_decode, q.lib().qlin_kvq_decode_workspace
    # blocks of 256 rows up to 256 * 8192 rows, of 512 past that
    assert ws(16, 8192, 256) == 16 * 32 * 258 * 4 and ws(2, 100, 128) == 2 * 1 * 130 * 4 and ws(0, 1, 64) == 0
    assert ws(1, 256 * 8192, 64) == 1 * 8192 * 66 * 4 and ws(1, 256 * 8192 + 1, 64) == 1 * 4097 * 66 * 4
    Q, KC, KS, KB, VC, VS, VB, WS, O = (0x9000000 + 0x1000000 * i for i in range(9))
    ok = dict(q=Q, qdt=q.QLIN_BF16, H=16, KV=8, N=8192, D=256, GS=64, bits=4, kc=KC, ks=KS, kb=KB, vc=VC, vs=VS,
              vb=VB, sbdt=q.QLIN_BF16, ws=WS, wsb=ws(16, 8192, 256), out=O, odt=q.QLIN_BF16)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["qdt"], a["H"], a["KV"], a["N"], a["D"], a["GS"], a["bits"], a["kc"], a["ks"], a["kb"],
                 a["vc"], a["vs"], a["vb"], a["sbdt"], a["ws"], a["wsb"], a["out"], a["odt"], None)
    # only invalid calls here: a valid one would launch on fake addresses
    assert call(q=None) == -1 and call(vb=None) == -1 and call(ws=None) == -1 and call(out=None) == -1
    assert call(qdt=q.QLIN_F32) == -3 and call(sbdt=q.QLIN_F32) == -3 and call(odt=5) == -3
    assert call(bits=2) == -4
    assert call(H=12) == -2 and call(KV=0) == -2 and call(N=0) == -2 and call(D=96) == -2 and call(GS=16) == -2
    assert call(D=64, GS=128) == -2
    assert call(q=Q + 1) == -5 and call(kc=KC + 4) == -5 and call(vc=VC + 8) == -5 and call(ws=WS + 2) == -5
    assert call(out=O + 1) == -5
    assert call(wsb=ws(16, 8192, 256) - 4) == -7
    assert call(out=WS + 64) == -7 and call(out=KC + 64) == -7


def test_kvq_noalloc_validation(q):
    """The allocation-free decode checks its arguments as qlin_kvq_decode does and refuses a
    call whose partials would not fit the static scratch, all before any HIP call."""
    f, ws = q.lib().qlin_kvq_decode_noalloc, q.lib().qlin_kvq_decode_workspace
    assert q.QLIN_KVQ_SCRATCH_BYTES == 8 << 20
    Q, KC, KS, KB, VC, VS, VB, O = (0x9000000 + 0x1000000 * i for i in range(8))
    ok = dict(q=Q, qdt=q.QLIN_BF16, H=16, KV=8, N=8192, D=256, GS=64, bits=4, kc=KC, ks=KS, kb=KB, vc=VC, vs=VS,
              vb=VB, sbdt=q.QLIN_BF16, out=O, odt=q.QLIN_BF16)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["qdt"], a["H"], a["KV"], a["N"], a["D"], a["GS"], a["bits"], a["kc"], a["ks"], a["kb"],
                 a["vc"], a["vs"], a["vb"], a["sbdt"], a["out"], a["odt"], None)
    assert call(q=None) == -1 and call(vb=None) == -1 and call(out=None) == -1
    assert call(qdt=q.QLIN_F32) == -3 and call(bits=2) == -4 and call(H=12) == -2 and call(D=96) == -2
    assert call(q=Q + 1) == -5 and call(out=O + 1) == -5
    assert call(out=KC + 64) == -7
    # 64 heads x 256 blocks of 256 rows x (128 + 2) floats = 8.5 MB of partials: too much
    assert ws(64, 65536, 128) > q.QLIN_KVQ_SCRATCH_BYTES
    assert call(H=64, KV=8, N=65536, D=128) == -8
    # 32 heads of 256: 254 blocks of 256 rows still fit, one more row does not
    assert ws(32, 254 * 256, 256) <= q.QLIN_KVQ_SCRATCH_BYTES < ws(32, 254 * 256 + 1, 256)
    assert call(H=32, KV=8, N=254 * 256 + 1, D=256) == -8


def test_merge_report_entry_points_validate(q):
    lib = q.lib()
    assert lib.qlin_set_merge_spin_limit(-1) == -1
    prev = lib.qlin_set_merge_spin_limit(1000)
    assert prev >= 0
    assert lib.qlin_set_merge_spin_limit(prev) == 1000
    assert lib.qlin_merge_timeouts(2) == -1 and lib.qlin_merge_timeouts(-1) == -1
