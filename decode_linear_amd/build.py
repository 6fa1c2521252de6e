"""Build libqlin.so in-tree with hipcc for gfx950.

Every translation unit is compiled to an object in parallel, then linked into
decode_linear_amd/libqlin.so.  Flags:
  --offload-arch=gfx950 -O3       CDNA4 code only
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                  no packed FP32 instructions (v_pk_{add,mul,fma}_f32)
  -fhip-fp32-correctly-rounded-divide-sqrt
                                  IEEE division (the quantizer must be bit exact)
  -mllvm -amdgpu-kernarg-preload-count=16
                                  leading kernel arguments arrive in SGPRs at wave launch
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libqlin.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["qlin_host.cpp", "qlin_pack.hip", "qlin_attend.hip", "qlin_stream.hip", "qlin_sample.hip", "qlin_kvq.hip", "qlin_fused_q4.hip", "qlin_fused_q8.hip",
           "qlin_fused_f16.hip", "qlin_fused_bf16.hip", "qlin_s8_q4_ln0_bf16.hip", "qlin_s8_q4_ln0_f16.hip",
           "qlin_s8_q4_ln1_bf16.hip", "qlin_s8_q4_ln1_f16.hip", "qlin_s8_q8_ln0_bf16.hip", "qlin_s8_q8_ln0_f16.hip",
           "qlin_s8_q8_ln1_bf16.hip", "qlin_s8_q8_ln1_f16.hip", "qlin_valu_q4.hip", "qlin_valu_q8.hip",
           "qlin_valu_f16.hip"]

CFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-mllvm", "-amdgpu-kernarg-preload-count=16",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    """Compile one source; the compiler's per-kernel register, scratch and LDS report goes to
    _build/<source>.resources.txt (a test checks that no kernel spills registers)."""
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-Rpass-analysis=kernel-resource-usage", "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    with open(os.path.join(BUILD_DIR, src + ".resources.txt"), "w") as fh:
        fh.write(r.stderr)
    return obj


def build(jobs: int = 0) -> str:
    """Compile and link libqlin.so (always rebuilds).  Returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def ensure_built() -> str:
    """Build only if no library is present (tests, smoke and bench use this)."""
    if not os.path.exists(LIB_PATH):
        build()
    return LIB_PATH


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else 0))
