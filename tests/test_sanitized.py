"""The CPU checks again under AddressSanitizer and UndefinedBehaviorSanitizer:
the oracle (oracle/kvq_oracle.c) and the C ABI's host code (argument
validation, layout and byte arithmetic in kvq_api.hip) built instrumented, with
clang's sanitizer runtime preloaded into a child pytest that runs the oracle's
pins and the host-side ABI tests.  Any finding aborts the child.  A planted
out-of-bounds read in a scratch C file, built and loaded the same way, shows
that the instrumentation and the runtime are live in this setup."""
import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
RUNTIMES = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))

pytestmark = pytest.mark.skipif(not (os.path.exists(CLANG) and RUNTIMES),
                                reason="clang sanitizer runtime not installed")

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g"]


def _env(**extra):
    env = dict(os.environ)
    env.update(LD_PRELOAD=RUNTIMES[-1], ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", **extra)
    return env


def test_planted_out_of_bounds_read_is_caught(tmp_path):
    src = tmp_path / "oob.c"
    src.write_text(textwrap.dedent("""
        #include <stdlib.h>
        int oob(int n) { int* a = malloc(4 * sizeof(int)); int v = a[n]; free(a); return v; }
    """))
    lib = tmp_path / "liboob.so"
    subprocess.run([CLANG, "-shared", "-fPIC", *SAN, "-o", str(lib), str(src)], check=True)
    code = f"import ctypes; ctypes.CDLL({str(lib)!r}).oob(4)"
    r = subprocess.run([sys.executable, "-c", code], env=_env(), capture_output=True, text=True)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr and "heap-buffer-overflow" in r.stderr


def test_cpu_checks_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import build as oracle_build
    from visual_autoregressive_kv_amd import build as kvq_build

    oracle_lib = oracle_build.build(out=str(tmp_path / "liboracle_san.so"), sanitize=True,
                                    cc=CLANG)
    kvq_lib = kvq_build.build(sanitize=True, out=str(tmp_path / "libkvq_san.so"))
    tests = ["tests/test_oracle_quant.py", "tests/test_oracle_pack_attend_bytes.py",
             "tests/test_oracle_half.py", "tests/test_abi.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p",
                        "no:cacheprovider", *tests], cwd=ROOT, capture_output=True, text=True,
                       env=_env(KVQR_ORACLE_LIB=oracle_lib, KVQ_LIB=kvq_lib), timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "Sanitizer" not in r.stderr, tail
