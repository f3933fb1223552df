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
