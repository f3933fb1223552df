"""GPU parity of kvq_attend_packed against the binary64 CPU oracle:
max|gpu - oracle| / max|oracle| <= 2e-3 per call, on caches both sides built
(the GPU cache is first checked bit-exact against the oracle's)."""
import numpy as np
import pytest
import torch

import varq_inputs as vi
import visual_autoregressive_kv_amd as K
from gpu_common import (DEV, assert_cache_equal, check_attn, fill_both, layouts,
                        oracle_attend_batch, to_dev)

pytestmark = pytest.mark.gpu


def gpu_attend(Lg, block, q_np, kg, vg, scale=0.0):
    out = torch.full(tuple(q_np.shape), float("nan"), dtype=torch.float32, device=DEV)
    K.kvq_attend_packed(Lg, block, to_dev(q_np), kg, vg, out, scale=scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_tiny_last_scale(oracle):
    """The small reference case: last scale's 256 queries over all 680 tokens."""
    wl = vi.WORKLOADS["var256_tiny_int4"]
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl)
    assert_cache_equal(kg, ko)
    assert_cache_equal(vg, vo)
    q = vi.q_block(wl, 0, 9)
    ref = oracle.attend(Lo, 9, q, ko, vo).astype(np.float64)
    got = gpu_attend(Lg, 9, q, kg, vg)
    check_attn(got, ref, "tiny last scale")


@pytest.mark.parametrize("name", ["var256_tiny_int4", "var_d20_b128_int4",
                                  "var_d20_b128_int3_rope", "var_d24_b128_int4",
                                  "var_d24_b128_int3", "var_w1920_b768_int3"])
def test_every_scale(oracle, name):
    wl = vi.WORKLOADS[name]
    if wl.batch > 2:
        wl = wl.with_(batch=2)
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl, layer=3)
    for block in range(len(wl.blocks)):
        q = vi.q_block(wl, 3, block)
        ref = oracle.attend(Lo, block, q, ko, vo).astype(np.float64)
        got = gpu_attend(Lg, block, q, kg, vg)
        check_attn(got, ref, f"{name} block {block}")


def test_full_batch_whole_outputs(oracle):
    """VAR-d20 at batch 128, the bench's launch configuration: the whole outputs of
    blocks 10 and 7 against the binary64 oracle (its sequences on host threads)."""
    wl = vi.WORKLOADS["var_d20_b128_int4"]
    Lg, Lo = layouts(oracle, wl)
    kg, vg = K.alloc_cache(Lg), K.alloc_cache(Lg)
    ko, vo = oracle.alloc_cache(Lo), oracle.alloc_cache(Lo)
    for j in range(10):
        kb, vb = vi.kv_block(wl, 0, "k", j), vi.kv_block(wl, 0, "v", j)
        assert oracle.quantize_block(Lo, j, kb, vb, ko, vo) == 0
        K.kvq_quantize_block(Lg, j, to_dev(kb), to_dev(vb), kg, vg)
    torch.cuda.synchronize()
    assert_cache_equal(kg, ko)
    assert_cache_equal(vg, vo)
    for block in (9, 6):
        q = vi.q_block(wl, 0, block)
        got = gpu_attend(Lg, block, q, kg, vg)
        ref = oracle_attend_batch(oracle, Lo, block, q, ko, vo)
        check_attn(got, ref, f"d20 batch 128 block {block}")


def test_video_frame_whole_output(oracle):
    """Next-frame video shape: 40 heads x 128, frames of 1560 tokens (3 frames);
    the third frame's whole output against the binary64 oracle."""
    wl = vi.WORKLOADS["video_16x1560_h40d128_int3"].with_(blocks=(1560, 1560, 1560))
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl)
    q = vi.q_block(wl, 0, 2)
    got = gpu_attend(Lg, 2, q, kg, vg)
    check_attn(got, oracle_attend_batch(oracle, Lo, 2, q, ko, vo), "video frame 3")


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_ragged_edges(oracle, bits, head_dim):
    """Query counts off the 32-row tile (1, 7, 33, 257 -> two workgroups per head),
    prefixes off the 32-key tile, odd batch and heads."""
    wl = vi.Workload("edge", 1, 3, 3, head_dim, bits, (1, 7, 33, 257, 2), "bf16",
                     rope=True, seed=11)
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl)
    for block in range(len(wl.blocks)):
        q = vi.q_block(wl, 0, block)
        ref = oracle.attend(Lo, block, q, ko, vo).astype(np.float64)
        got = gpu_attend(Lg, block, q, kg, vg)
        check_attn(got, ref, f"ragged D={head_dim} INT{bits} block {block}")


def test_explicit_scale_and_determinism(oracle):
    wl = vi.WORKLOADS["var_d20_b128_int3_rope"].with_(batch=2)
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl, upto=8)
    q = vi.q_block(wl, 0, 7)
    ref = oracle.attend(Lo, 7, q, ko, vo, scale=0.05).astype(np.float64)
    a = gpu_attend(Lg, 7, q, kg, vg, scale=0.05)
    b = gpu_attend(Lg, 7, q, kg, vg, scale=0.05)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    check_attn(a, ref, "explicit scale")


def test_reads_only_the_prefix(oracle):
    """Garbage in blocks after k (cache bytes and stats) does not change block k's
    output: the attention reads the packed prefix of blocks 0..k only."""
    wl = vi.WORKLOADS["var_d20_b128_int4"].with_(batch=2)
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl, upto=7)
    q = vi.q_block(wl, 0, 6)
    a = gpu_attend(Lg, 6, q, kg, vg)
    T = wl.offset(7)
    for c in (kg, vg):
        c["codes"][:, :, T:] = 0xFF
        c["zero"][:, :, 7:] = float("nan")
        c["scale"][:, :, 7:] = float("inf")
    b = gpu_attend(Lg, 6, q, kg, vg)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("blocks", [(2,) * 16, (1,) * 40 + (3,), (5, 1, 30, 31, 64),
                                    (1,) * 63 + (70,)])
def test_many_short_blocks(oracle, head_dim, blocks):
    """Short blocks whose statistics do or do not fit the per-wave LDS staging of
    the short-block kernel (16 vs 41 blocks), 30/31/64-query blocks, and the
    64-block maximum (64 KB of staged statistics at head_dim 128)."""
    wl = vi.Workload("short", 1, 2, 5, head_dim, 4 if head_dim == 64 else 3, blocks, "bf16",
                     rope=False, seed=5)
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl)
    for block in sorted({0, 1, len(blocks) // 2, len(blocks) - 2, len(blocks) - 1}):
        q = vi.q_block(wl, 0, block)
        ref = oracle.attend(Lo, block, q, ko, vo).astype(np.float64)
        got = gpu_attend(Lg, block, q, kg, vg)
        check_attn(got, ref, f"short blocks D={head_dim} block {block}")
