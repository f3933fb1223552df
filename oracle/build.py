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


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-std=c11", "-O2", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
        "-Wall", "-Wextra", "-Werror",
        "-o", LIB + ".tmp", *SOURCES, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
