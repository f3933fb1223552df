"""kvq_attend_packed_split_noalloc, the key-range attention whose partials live
in the library's static device scratch array, against kvq_attend_packed_split
with a caller workspace: bit-identical outputs on two calls in a row on one
GPU, the second on a smaller input (the array keeps the first call's
contents), plus the size limit and oracle parity on the small case."""
import numpy as np
import pytest
import torch

import varq_inputs as vi
import visual_autoregressive_kv_amd as K
from gpu_common import DEV, check_attn, fill_both, to_dev

pytestmark = pytest.mark.gpu


def both(Lg, block, q_np, kg, vg, max_splits):
    q = to_dev(q_np)
    ws = torch.empty(K.kvq_attend_split_workspace(Lg, block, max_splits), dtype=torch.uint8,
                     device=DEV)
    a = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=DEV)
    b = torch.full_like(a, float("nan"))
    K.kvq_attend_packed_split(Lg, block, q, kg, vg, a, ws, max_splits=max_splits)
    K.kvq_attend_packed_split_noalloc(Lg, block, q, kg, vg, b, max_splits=max_splits)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


def test_noalloc_matches_workspace_call_twice(oracle):
    # first call: a video frame of 1560 queries over 3120 keys, 40 heads x 128,
    # INT3, 4 key ranges (124 MiB of partials, most of the array)
    big = vi.WORKLOADS["video_16x1560_h40d128_int3"].with_(blocks=(1560, 1560))
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, big)
    q = vi.q_block(big, 0, 1)
    a, b = both(Lg, 1, q, kg, vg, 4)
    assert np.isfinite(a).all()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # second call: a smaller layout (B=2, 3 heads x 64, INT4, 1000 queries over
    # 1680 keys, 3 ranges); the array still holds the first call's partials
    small = vi.Workload("noalloc_small", 1, 2, 3, 64, 4, vi.VAR_BLOCKS + (1000,), "bf16", seed=37)
    Lg2, Lo2, kg2, vg2, ko2, vo2 = fill_both(oracle, small)
    last = len(small.blocks) - 1
    q2 = vi.q_block(small, 0, last)
    a2, b2 = both(Lg2, last, q2, kg2, vg2, 3)
    assert np.array_equal(a2.view(np.uint32), b2.view(np.uint32))
    ref = oracle.attend(Lo2, last, q2, ko2, vo2).astype(np.float64)
    check_attn(b2, ref, "no-alloc key ranges, second call")


def test_noalloc_rejects_more_than_the_array():
    wl = vi.WORKLOADS["video_16x1560_h40d128_int3"].with_(blocks=(1560, 1560))
    Lg = K.make_layout(wl.batch, wl.heads, wl.head_dim, wl.bits, wl.blocks)
    assert K.kvq_attend_split_workspace(Lg, 1, 8) > K.STATIC_SCRATCH_BYTES
    q = torch.zeros((1, 1560, 40, 128), dtype=torch.bfloat16, device=DEV)
    kg, vg = K.alloc_cache(Lg), K.alloc_cache(Lg)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    with pytest.raises(K.KvqError) as e:
        K.kvq_attend_packed_split_noalloc(Lg, 1, q, kg, vg, out, max_splits=8)
    assert e.value.code == -1  # KVQ_E_INVAL, before any launch
