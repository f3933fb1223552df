"""KVQ_DEBUG=1 (synchronize and check after every launch) and the bench's roctx
ranges: both leave the results unchanged.  Each runs in a child process, one
at a time."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.gpu

CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import varq_inputs as vi
import visual_autoregressive_kv_amd as K
from gpu_common import to_dev
wl = vi.Workload("dbg", 1, 2, 3, 64, 3, (1, 7, 40, 256), "bf16", seed=5)
L = K.make_layout(wl.batch, wl.heads, wl.head_dim, wl.bits, wl.blocks)
kc, vc = K.alloc_cache(L), K.alloc_cache(L)
outs = []
for j in range(len(wl.blocks)):
    q = to_dev(vi.q_block(wl, 0, j))
    o = torch.empty(tuple(q.shape), dtype=torch.float32, device="cuda")
    K.kvq_quantize_attend(L, j, to_dev(vi.kv_block(wl, 0, "k", j)),
                          to_dev(vi.kv_block(wl, 0, "v", j)), q, kc, vc, o)
    outs.append(o.cpu().numpy())
np.save({out!r}, np.concatenate([x.ravel() for x in outs]))
"""


def run_child(tmp_path, name, debug):
    out = str(tmp_path / f"{name}.npy")
    env = dict(os.environ)
    env.pop("KVQ_DEBUG", None)
    if debug:
        env["KVQ_DEBUG"] = "1"
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), out=out)
    print(f"[debug-mode] child {name} (KVQ_DEBUG={'1' if debug else 'unset'})", flush=True)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "kvq:" not in r.stderr, r.stderr[-2000:]
    return np.load(out)


def test_debug_mode_changes_no_result(tmp_path):
    plain = run_child(tmp_path, "plain", False)
    debug = run_child(tmp_path, "debug", True)
    assert np.isfinite(plain).all()
    assert np.array_equal(plain.view(np.uint32), debug.view(np.uint32))


def test_bench_with_roctx_ranges():
    print("[debug-mode] bench.py --roctx, one layer, one step", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--roctx", "--steps", "1",
                        "--warmup", "1", "--layers", "1", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    line = [l for l in r.stdout.splitlines() if l.startswith("{")][-1]
    rec = json.loads(line)
    assert rec["value"] > 0 and rec["steps"] == 1
