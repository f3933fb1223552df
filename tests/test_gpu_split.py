"""GPU parity of kvq_attend_packed_split (the key prefix of every query tile cut
into ranges attended by separate workgroups, partials merged by log-sum-exp):
against the binary64 oracle within the attention tolerance, close to
kvq_attend_packed, and bit-identical to it when one range is used.

A range rounds its softmax weights to binary16 (toward zero) against its own
running maximum, not the whole prefix's, so its weights round differently from
kvq_attend_packed's by up to 2^-10 relative each; SPLIT_VS_PLAIN bounds the
resulting difference at a tenth of the attention tolerance."""
import numpy as np
import pytest
import torch

import varq_inputs as vi
import visual_autoregressive_kv_amd as K
from gpu_common import (ATTN_TOL, DEV, assert_cache_equal, attn_err, check_attn, fill_both,
                        layouts, oracle_attend_batch, to_dev)

pytestmark = pytest.mark.gpu

SPLIT_VS_PLAIN = ATTN_TOL / 10


def split_and_plain(Lg, block, q_np, kg, vg, max_splits, scale=0.0):
    q = to_dev(q_np)
    ws = torch.empty(K.kvq_attend_split_workspace(Lg, block, max_splits), dtype=torch.uint8,
                     device=DEV)
    ws.fill_(0xFF)  # the call must not depend on the workspace's contents
    got = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=DEV)
    K.kvq_attend_packed_split(Lg, block, q, kg, vg, got, ws, max_splits=max_splits, scale=scale)
    plain = torch.full_like(got, float("nan"))
    K.kvq_attend_packed(Lg, block, q, kg, vg, plain, scale=scale)
    torch.cuda.synchronize()
    return got.cpu().numpy(), plain.cpu().numpy()


def test_video_frames_split(oracle):
    """Next-frame video shape, 3 frames of 1560 tokens: the last frame's 1560
    queries over 4680 keys (147 key tiles) in 4 ranges: 280 query tiles, about
    four workgroups per CU."""
    wl = vi.WORKLOADS["video_16x1560_h40d128_int3"].with_(blocks=(1560, 1560, 1560))
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl)
    q = vi.q_block(wl, 0, 2)
    got, plain = split_and_plain(Lg, 2, q, kg, vg, 8)
    assert np.isfinite(got).all()
    assert attn_err(got, plain.astype(np.float64)) <= SPLIT_VS_PLAIN
    check_attn(got, oracle_attend_batch(oracle, Lo, 2, q, ko, vo), "video frame 3, key ranges")


def test_video_sixteen_frames(oracle):
    """The video shape in full, as the decode benchmark runs it: 16 frames of
    1560 tokens, the packed cache bit-exact against the oracle, then frame 8
    (12480 keys) and frame 16 (24960 keys, 780 key tiles) through
    kvq_attend_packed_split with max_splits 8 (4 ranges per query tile): whole
    outputs against the binary64 oracle, and close to kvq_attend_packed."""
    wl = vi.WORKLOADS["video_16x1560_h40d128_int3"]
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl)
    assert_cache_equal(kg, ko, "video K")
    assert_cache_equal(vg, vo, "video V")
    for block in (7, 15):
        q = vi.q_block(wl, 0, block)
        got, plain = split_and_plain(Lg, block, q, kg, vg, 8)
        assert np.isfinite(got).all()
        assert attn_err(got, plain.astype(np.float64)) <= SPLIT_VS_PLAIN, block
        check_attn(got, oracle_attend_batch(oracle, Lo, block, q, ko, vo),
                   f"video frame {block + 1}, key ranges")


@pytest.mark.parametrize("bits,head_dim", [(4, 64), (3, 64), (4, 128), (3, 128)])
def test_ranges_across_short_blocks(oracle, bits, head_dim):
    """The VAR schedule's ten blocks then a block of 1000 queries: key ranges
    start inside and across the short blocks (statistics change inside a
    range), a partial last tile, several query tiles per head."""
    wl = vi.Workload("split_mix", 1, 2, 3, head_dim, bits, vi.VAR_BLOCKS + (1000,), "bf16",
                     seed=31)
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl)
    last = len(wl.blocks) - 1
    q = vi.q_block(wl, 0, last)
    ref = oracle.attend(Lo, last, q, ko, vo).astype(np.float64)
    for max_splits in (2, 3, 64):
        got, plain = split_and_plain(Lg, last, q, kg, vg, max_splits, scale=0.09)
        assert attn_err(got, plain.astype(np.float64)) <= SPLIT_VS_PLAIN, max_splits
        got_def, _ = split_and_plain(Lg, last, q, kg, vg, max_splits)
        check_attn(got_def, ref, f"key ranges INT{bits} D={head_dim} max_splits {max_splits}")


def test_one_range_is_kvq_attend_packed(oracle):
    wl = vi.WORKLOADS["video_16x1560_h40d128_int3"].with_(blocks=(1560, 1560))
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl)
    q = vi.q_block(wl, 0, 1)
    got, plain = split_and_plain(Lg, 1, q, kg, vg, 1)
    assert np.array_equal(got.view(np.uint32), plain.view(np.uint32))


def test_short_blocks_fall_back(oracle):
    """Blocks of at most 128 queries and short prefixes take one range:
    bit-identical to kvq_attend_packed."""
    wl = vi.WORKLOADS["var_d20_b128_int4"].with_(batch=2)
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl)
    for block in (0, 4, 7, 9):
        q = vi.q_block(wl, 0, block)
        got, plain = split_and_plain(Lg, block, q, kg, vg, 16)
        assert np.array_equal(got.view(np.uint32), plain.view(np.uint32)), block


def test_workspace_errors(oracle):
    wl = vi.WORKLOADS["video_16x1560_h40d128_int3"].with_(blocks=(1560, 1560))
    Lg, _ = layouts(oracle, wl)
    need = K.kvq_attend_split_workspace(Lg, 1, 8)
    assert need == 8 * 1560 * 40 * (128 + 2) * 4
    kg, vg = K.alloc_cache(Lg), K.alloc_cache(Lg)
    q = torch.zeros((1, 1560, 40, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    small = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(K.KvqError):
        K.kvq_attend_packed_split(Lg, 1, q, kg, vg, out, small, max_splits=8)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    for bad in (0, 65):
        with pytest.raises(K.KvqError):
            K.kvq_attend_packed_split(Lg, 1, q, kg, vg, out, ws, max_splits=bad)
