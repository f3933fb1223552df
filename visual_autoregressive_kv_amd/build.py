"""Compile libkvq.so (HIP, gfx950) in-tree.

    python -m visual_autoregressive_kv_amd.build [-v]

Every translation unit is compiled for gfx950 only, with floating-point
contraction off (the quantizer's binary32 steps must each round once, as the
statistics and codes are compared bit for bit) and with packed-fp32
instruction selection disabled.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvq.so")
SOURCES = ["kvq_api.hip", "quant_pack.hip", "pack.hip", "attend.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Host-side sanitizer build (libkvq_san.so): AddressSanitizer and
# UndefinedBehaviorSanitizer on the C ABI's host code (kvq_api.hip: argument
# validation, layout arithmetic, descriptors), linked with the ordinary objects
# of the kernel sources.  Loaded with clang's ASan runtime preloaded, by CPU
# tests that never launch a kernel.
SAN_LIB = os.path.join(PKG, "libkvq_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", "_san.o" if sanitize else ".o"))
    cmd = [HIPCC, *CFLAGS, *(SAN_FLAGS if sanitize else []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False, out: str = "") -> str:
    out = out or (SAN_LIB if sanitize else LIB)
    os.makedirs(BUILD, exist_ok=True)

    def one(src):
        if sanitize and src != "kvq_api.hip":
            obj = os.path.join(BUILD, src.replace(".hip", ".o"))
            return obj if os.path.exists(obj) else _compile(src, verbose)
        return _compile(src, verbose, sanitize)

    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, SOURCES))
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
