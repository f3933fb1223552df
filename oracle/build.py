"""Compile the CPU oracle (plain C) into oracle/liboracle.so with gcc.

Test infrastructure only: the oracle is the checker, never the product path.
Floating-point contraction is switched off so every binary32 operation of the
quantizer rounds once, as the C source spells it out.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SOURCES = [os.path.join(HERE, "kvq_oracle.c")]


SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False, cc: str = "gcc") -> str:
    """sanitize: AddressSanitizer + UndefinedBehaviorSanitizer instrumentation
    (any finding aborts); load the result with the sanitizer runtime of the
    compiler `cc` preloaded."""
    cmd = [
        cc, "-std=c11", "-O1" if sanitize else "-O2", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
        "-Wall", "-Wextra", "-Werror", *(SAN_FLAGS if sanitize else []),
        "-o", out + ".tmp", *SOURCES, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
