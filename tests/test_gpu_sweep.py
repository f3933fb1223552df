"""Seeded sweep over random decode layouts, through every dispatch path of the
library (one-wave, 2/4/8-wave and fused kernels, two-launch fallbacks,
head_dim 64 and 128, INT2, INT3, INT4 and INT8, bf16 and fp32 input, up to 40 blocks, key
ranges).  Per case, block by block:
  * kvq_quantize_attend's output is bit-identical to kvq_quantize_block then
    kvq_attend_packed, and both caches are bit-exact against the oracle's;
  * two of the blocks' outputs are within the attention tolerance of the
    binary64 oracle, and so is kvq_attend_packed_split on the last block.
A second sweep runs INT3 layouts in block-aligned words (pack_mode 2), whose
kernels address each chunk per tile from its key's block.
Sizes keep the oracle to a few seconds per case."""
import numpy as np
import pytest
import torch

import varq_inputs as vi
import visual_autoregressive_kv_amd as K
from gpu_common import DEV, assert_cache_equal, check_attn, layouts, to_dev

pytestmark = pytest.mark.gpu

N_CASES = 48
N_WORD_CASES = 24


def random_workload(i: int) -> vi.Workload:
    rng = np.random.default_rng(1000 + i)
    head_dim = int(rng.choice([64, 128]))
    bits = int(rng.choice([2, 3, 4, 8]))
    src = "f32" if rng.random() < 0.25 else "bf16"
    n_blocks = int(rng.integers(1, 41))
    kind = rng.random()
    if kind < 0.4:    # many short blocks
        blocks = rng.integers(1, 20, n_blocks)
    elif kind < 0.8:  # VAR-like growth
        blocks = np.minimum(1 + (np.arange(n_blocks) * rng.integers(2, 12)) ** 1.3, 300).astype(int)
    else:             # a few long blocks
        blocks = rng.integers(100, 400, max(1, n_blocks // 8))
    total = int(np.sum(blocks))
    while total > 1500:  # bound the oracle's work
        blocks = blocks[:-1]
        total = int(np.sum(blocks))
    batch = int(rng.integers(1, 4))
    heads = int(rng.integers(1, 4))
    return vi.Workload(f"sweep{i}", 1, batch, heads, head_dim, bits,
                       tuple(int(b) for b in blocks), src, rope=bool(rng.random() < 0.3),
                       seed=7000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_layout(oracle, i):
    run_case(oracle, random_workload(i), i, 0)


@pytest.mark.parametrize("i", range(N_WORD_CASES))
def test_random_layout_block_words(oracle, i):
    run_case(oracle, random_workload(N_CASES + i).with_(bits=3), N_CASES + i, 2)


def run_case(oracle, wl, i, pack_mode):
    Lg, Lo = layouts(oracle, wl, pack_mode)
    kf, vf = K.alloc_cache(Lg), K.alloc_cache(Lg)
    ks, vs = K.alloc_cache(Lg), K.alloc_cache(Lg)
    ko, vo = oracle.alloc_cache(Lo), oracle.alloc_cache(Lo)
    nb = len(wl.blocks)
    checked = {nb - 1, int(np.random.default_rng(i).integers(nb))}
    print(f"[sweep] case {i}: B={wl.batch} H={wl.heads} D={wl.head_dim} INT{wl.bits} "
          f"{wl.src} pack_mode {pack_mode} blocks={wl.blocks}", flush=True)
    for j in range(nb):
        kb, vb = vi.kv_block(wl, 0, "k", j), vi.kv_block(wl, 0, "v", j)
        q = vi.q_block(wl, 0, j)
        assert oracle.quantize_block(Lo, j, kb, vb, ko, vo) == 0
        kd, vd, qd = to_dev(kb), to_dev(vb), to_dev(q)
        of = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=DEV)
        os_ = torch.full_like(of, float("nan"))
        K.kvq_quantize_attend(Lg, j, kd, vd, qd, kf, vf, of)
        K.kvq_quantize_block(Lg, j, kd, vd, ks, vs)
        K.kvq_attend_packed(Lg, j, qd, ks, vs, os_)
        torch.cuda.synchronize()
        assert torch.equal(of.view(torch.int32), os_.view(torch.int32)), (i, j)
        if j in checked:
            ref = oracle.attend(Lo, j, q, ko, vo).astype(np.float64)
            check_attn(of.cpu().numpy(), ref, f"sweep {i} block {j}")
            if j == nb - 1:
                ws = torch.empty(K.kvq_attend_split_workspace(Lg, j, 64), dtype=torch.uint8,
                                 device=DEV)
                osp = torch.full_like(of, float("nan"))
                K.kvq_attend_packed_split(Lg, j, qd, ks, vs, osp, ws, max_splits=64)
                torch.cuda.synchronize()
                check_attn(osp.cpu().numpy(), ref, f"sweep {i} block {j} key ranges")
    assert_cache_equal(kf, ko, f"case {i} fused K")
    assert_cache_equal(vf, vo, f"case {i} fused V")
    assert_cache_equal(ks, ko, f"case {i} two-call K")
    assert_cache_equal(vs, vo, f"case {i} two-call V")
