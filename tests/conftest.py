import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def oracle():
    """The CPU oracle binding (builds liboracle.so if absent)."""
    from oracle import binding as ob
    from oracle import build as obuild

    if not os.path.exists(ob.LIB_PATH):
        obuild.build()
    ob.lib()
    return ob


@pytest.fixture(scope="session")
def tmp_build_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("cbuild")


def compile_c_helper(src: str, out_dir) -> str:
    out = os.path.join(str(out_dir), os.path.basename(src).replace(".c", ".so"))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", out, src,
                    "-lm"], check=True)
    return out


def pytest_terminal_summary(terminalreporter):
    """Worst attention errors of the GPU parity tests, per case family: per call,
    per (sequence, head) (both asserted <= 2e-3) and per channel (reported)."""
    gc = sys.modules.get("gpu_common")
    if gc is None or not gc.ERR_LOG:
        return
    fam = {}
    for what, e, ebh, ech in gc.ERR_LOG:
        key = what.split(" block")[0].split(",")[0]
        w = fam.setdefault(key, [0, 0.0, 0.0, None])
        w[0] += 1
        w[1], w[2] = max(w[1], e), max(w[2], ebh)
        if ech is not None:
            w[3] = ech if w[3] is None else max(w[3], ech)
    tr = terminalreporter
    tr.write_line(f"attention error vs the binary64 oracle ({len(gc.ERR_LOG)} checks; bound 2e-3 "
                  "per call and per (b,h); per channel reported only):")
    for key, (n, e, ebh, ech) in sorted(fam.items()):
        ch = "n/a" if ech is None else f"{ech:.2e}"
        tr.write_line(f"  {key:<48} n={n:<3} per call {e:.2e}  per (b,h) {ebh:.2e}  per channel {ch}")
