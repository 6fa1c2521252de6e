"""The library's host code and the oracle under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  Both are rebuilt with the sanitizers (the host code of libqlin with clang's
ASan + UBSan, its kernels unchanged; oracle.cpp likewise), then the CPU tests that drive them
(the ABI's argument checks, the binding's checks, every oracle pin) run in a child process
that preloads the sanitizer runtime and loads those builds.  Any report fails the run
(UBSan halts on the first error; leak checking is off: the Python interpreter itself is not
built for it)."""
import os
import subprocess
import sys

import pytest

from decode_linear_amd import build as qbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
HIPCC = qbuild.HIPCC
CPU_TESTS = ["tests/test_abi.py", "tests/test_wrappers.py", "tests/test_oracle_format.py", "tests/test_oracle_math.py",
             "tests/test_oracle_mlp.py", "tests/test_oracle_attend.py", "tests/test_oracle_kvq.py",
             "tests/test_oracle_sample.py"]
# the host pass only: each sanitizer flag is scoped to the host compilation
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
CLANG_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _runtime():
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed:\n{r.stderr[-3000:]}"


@pytest.mark.timeout(600)
def test_host_code_and_oracle_under_asan_ubsan(tmp_path):
    rt = _runtime()
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("clang's ASan runtime or hipcc not found")
    qbuild.ensure_built()
    objs = [os.path.join(qbuild.BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in qbuild.SOURCES
            if s != "qlin_host.cpp"]
    if not all(os.path.exists(o) for o in objs):
        qbuild.build()
    host = str(tmp_path / "host_san.o")
    flags = [f for f in qbuild.CFLAGS if f != "-O3"]
    _run([HIPCC, *flags, "-O1", "-g", *HOST_SAN, "-x", "hip", "-c",
          os.path.join(qbuild.CSRC, "qlin_host.cpp"), "-o", host])
    lib = str(tmp_path / "libqlin_san.so")
    link = [CLANG, "-shared", "-fPIC", *CLANG_SAN, "-shared-libasan", host, *objs]
    _run(link + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib])
    orc = str(tmp_path / "liboracle_san.so")
    _run([CLANG, "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", *CLANG_SAN,
          "-shared-libasan", os.path.join(ROOT, "oracle", "oracle.cpp"), "-o", orc])
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", QLIN_LIB_PATH=lib, ORACLE_LIB_PATH=orc)
    r = subprocess.run([sys.executable, "-m", "pytest", *CPU_TESTS, "-q", "-s", "-p", "no:cacheprovider",
                        "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=500)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "passed" in out, out[-6000:]
    for marker in ("runtime error", "ERROR: AddressSanitizer", "SUMMARY: UndefinedBehaviorSanitizer"):
        assert marker not in out, out[-6000:]
