"""Register-allocation guard for the decode-step attention kernels (CPU: the
gfx950 assembly is compiled here, nothing runs).  The 4- and 8-wave kernels of
the VAR shapes run at 4 waves per SIMD, which caps them at 128 VGPRs; at that
cap a small change elsewhere in a kernel can move a spill into the key-tile
loop, where its reload adds memory latency to every tile (one such move cost
16% on the 100-token block).  Checked, for the head_dim-64 2-, 4- and 8-wave
kernels at every code width, fused and attention-only: the scratch accesses
inside loops (none, or no more than the few some have always had), and the
waves per SIMD their register counts allow."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "visual_autoregressive_kv_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    import sys
    sys.path.insert(0, ROOT)
    from visual_autoregressive_kv_amd import build as kb
    out = str(tmp_path_factory.mktemp("isa") / "attend.s")
    flags = [f for f in kb.CFLAGS if not f.startswith("-W")]
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, "attend.hip"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out).read()


def kernel_body(asm_text, name_re):
    for m in re.finditer(r"^(_Z\S+):\s*;", asm_text, re.M):
        if re.search(name_re, m.group(1)):
            end = asm_text.index(".Lfunc_end", m.start())
            info = asm_text[end: asm_text.index("; Occupancy:", end) + 40]
            return m.group(1), asm_text[m.start():end], info
    raise AssertionError(f"no kernel matches {name_re}")


def loop_scratch_ops(body):
    n, in_loop = 0, False
    for line in body.split("\n"):
        t = line.strip()
        if t.startswith(".LBB"):
            in_loop = "Loop Header" in t or "in Loop" in t
            continue
        if in_loop and t.startswith("scratch_"):
            n += 1
    return n


# attend_kernel<D, BITS, NW, FUSE, SPLIT, BW> -> scratch instructions allowed
# inside loops: none, except the attention-only 2- and 4-wave INT4 kernels and
# the 2- and 4-wave INT2 kernels, which carry the reloads they were built with
# and may not get more.  And the waves per SIMD each keeps: 4 for 4- and 8-wave INT4
# workgroups, 3 for 2-wave ones; one fewer for the 3- and 8-bit codes, which
# hold two words per item in flight (at the INT4 caps they spilled in the loop).
CASES = {}
for bits in (2, 3, 4, 8):
    two_words = bits in (3, 8)
    for nw, occ in ((2, 3), (4, 4), (8, 4)):
        for fuse in (0, 1):
            loops = 2 if (bits in (2, 4) and nw in (2, 4) and fuse == 0) else 0
            if bits == 2:  # INT2 at the INT4 caps: reloads in the 2- and 4-wave loops
                loops = {2: 14 if fuse == 0 else 10, 4: 2, 8: 0}[nw]
            CASES[(bits, nw, fuse)] = (loops, occ - (1 if two_words and nw != 8 else 0))


@pytest.mark.parametrize("bits,nw,fuse", sorted(CASES))
def test_no_spill_in_the_tile_loop(asm, bits, nw, fuse):
    name, body, info = kernel_body(asm, rf"attend_kernelILi64ELi{bits}ELi{nw}ELi{fuse}ELi0ELb0E")
    loops, min_occ = CASES[(bits, nw, fuse)]
    assert loop_scratch_ops(body) <= loops, name
    occ = int(re.search(r"Occupancy: (\d+)", info).group(1))
    assert occ >= min_occ, (name, occ)
