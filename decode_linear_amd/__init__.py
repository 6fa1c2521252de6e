"""decode_linear_amd: the MI355X-native decode-time fused quantized linear (libqlin).

The library itself is C-ABI (include/qlin.h, built to decode_linear_amd/libqlin.so by
decode_linear_amd.build); decode_linear_amd.qlin is its thin Python binding."""
from .qlin import (QLIN_ACT_GELU, QLIN_ACT_NONE, QLIN_BF16, QLIN_F16, QLIN_F32, QlinChain, QlinError, QWeight,
                   qlin_attend, qlin_check, qlin_dispatch_count, qlin_gateup_swiglu, qlin_linear, qlin_kvq_decode,
                   qlin_kvq_decode_noalloc, qlin_mlp, qlin_pack_affine,
                   qlin_merge_timeouts, qlin_sample, qlin_set_merge_spin_limit, qlin_set_path,
                   qlin_status_string, qlin_stream_read, qlin_stream_read_config,
                   qlin_unpack_affine)

__all__ = ["QLIN_ACT_GELU", "QLIN_ACT_NONE", "QLIN_BF16", "QLIN_F16", "QLIN_F32", "QlinChain", "QlinError", "QWeight",
           "qlin_attend", "qlin_check", "qlin_dispatch_count", "qlin_gateup_swiglu", "qlin_linear", "qlin_kvq_decode",
           "qlin_kvq_decode_noalloc", "qlin_merge_timeouts", "qlin_mlp", "qlin_pack_affine", "qlin_sample",
           "qlin_set_merge_spin_limit",
           "qlin_set_path", "qlin_status_string", "qlin_stream_read", "qlin_stream_read_config", "qlin_unpack_affine"]
