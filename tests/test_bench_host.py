"""Host-side logic of bench.py (CPU only): the one-GPU guard, the algorithmic
byte and flop model behind `roofline.achieved`, and the rule that `traffic` is
read only from a counter summary taken on the current kernel source."""
import os
import subprocess
import sys

import pytest

import bench
import varq_inputs as vi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 1" in r.stderr


def test_byte_model_against_the_cache_accounting(oracle):
    """Attention reads the packed K and V prefix once: twice the code bytes that
    kvqr_bytes reports for blocks 0..k, plus statistics, Q and O."""
    wl = vi.WORKLOADS["var_d20_b128_int4"]
    L = oracle.layout_of(wl)
    B, H, D = wl.batch, wl.heads, wl.head_dim
    for k in range(len(wl.blocks)):
        code_b, _ = oracle.nbytes(L, k + 1)
        n = wl.blocks[k]
        expect = 2 * code_b + B * H * (2 * (k + 1) * D * 4 + n * D * (2 + 4))
        assert bench.attend_bytes(wl, k) == expect
        # quantize: bf16 K and V in once; their rows and statistics out once
        row = (wl.bits * D + 7) // 8
        assert bench.quant_bytes(wl, k) == 2 * B * H * (n * D * 2 + n * row + D * 4)
        assert bench.attend_flops(wl, k) == 4 * B * H * n * (wl.offset(k) + n) * D


def test_byte_model_of_block_aligned_words(oracle):
    """--pack-mode 2: the attention reads the prefix's words (kvqr_bytes of the
    block-aligned layout) and the quantizer writes the block's words."""
    wl = vi.WORKLOADS["var_d20_b128_int3_rope"]
    L = oracle.layout_of(wl)
    L.pack_mode = 2
    B, H, D = wl.batch, wl.heads, wl.head_dim
    try:
        bench.PACK_MODE = 2
        for k in range(len(wl.blocks)):
            code_b, _ = oracle.nbytes(L, k + 1)
            prev_b, _ = oracle.nbytes(L, k)
            n = wl.blocks[k]
            assert bench.attend_bytes(wl, k) == 2 * code_b + B * H * (2 * (k + 1) * D * 4 +
                                                                      n * D * (2 + 4))
            assert bench.quant_bytes(wl, k) == 2 * (B * H * (n * D * 2 + D * 4) + code_b - prev_b)
    finally:
        bench.PACK_MODE = 0


def test_per_layer_totals_quoted_in_the_docs():
    """VAR-d20 B128 INT4: 570.2 MB quantize+pack, 1020.7 MB attention and 187.7
    GFLOP per layer over the 10 blocks."""
    wl = vi.WORKLOADS["var_d20_b128_int4"]
    q = sum(bench.quant_bytes(wl, k) for k in range(10))
    a = sum(bench.attend_bytes(wl, k) for k in range(10))
    f = sum(bench.attend_flops(wl, k) for k in range(10))
    assert round(q / 1e6, 1) == 570.2
    assert round(a / 1e6, 1) == 1020.7
    assert round(f / 1e9, 1) == 187.7


def test_traffic_only_for_the_profiled_source(monkeypatch):
    path = os.path.join(ROOT, "profiles", "fused_var_d20_b128_int4_hbm_traffic.md")
    committed, sha = None, None
    for line in open(path):
        if line.startswith("- hbm_bytes_per_launch:"):
            committed = float(line.split("`")[1])
        if line.startswith("- kernel_source_sha256_16:"):
            sha = line.split("`")[1]
    assert committed is not None and sha is not None
    current = bench.source_sha(bench.KERNEL_SOURCES["fused"])
    got = bench.measured_traffic("fused", "var_d20_b128_int4")
    assert got == (committed if sha == current else None)
    assert bench.measured_traffic("fused", "no_such_workload") is None
    monkeypatch.setattr(bench, "source_sha", lambda rel: "0" * 16)
    assert bench.measured_traffic("fused", "var_d20_b128_int4") is None
