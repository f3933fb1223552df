"""The GPU quantizer's binary16 statistics at every binary32 value of the
binary16 range, bit for bit against the oracle's kvqr_quantize_block.

Every x with |x| <= 65504 (the largest binary16 value) enters two-token groups:
  * {x, x}: the zero point is x rounded down to binary16 (with a zero extreme
    taken as +0), the step is the remainder fp32(x - z) / L rounded up;
  * {0, x} for x >= 0: zero point 0, step fp32(x / L) rounded up.
So the GPU's directed roundings RD16 and RU16 are reached at every input
pattern of the range on the zero side and at one quotient per pattern on the
step side; the oracle's own are pinned against all 2^32 patterns on the CPU
(test_oracle_half.py).  Codes of the groups are compared too.
"""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

import visual_autoregressive_kv_amd as K
from gpu_common import DEV, cache_to_host

pytestmark = pytest.mark.gpu

CHUNK = 1 << 27    # groups per call: 2^21 heads x 64 channels
TOP = 0x477FE000   # bit pattern of 65504.0
SLICES = 16        # oracle threads, one slice of heads each


def _oracle_cache(oracle, src):
    """kvqr_quantize_block over src [1][2][H][64] in SLICES head slices, in parallel."""
    H = src.shape[2]
    h = H // SLICES
    Ls = oracle.make_layout(1, h, 64, 4, (2,))

    def one(i):
        part = np.ascontiguousarray(src[:, :, i * h:(i + 1) * h, :])
        kc, vc = oracle.alloc_cache(Ls), oracle.alloc_cache(Ls)
        assert oracle.quantize_block(Ls, 0, part, part, kc, vc) == oracle.OK
        return kc

    with cf.ThreadPoolExecutor(SLICES) as ex:
        parts = list(ex.map(one, range(SLICES)))
    return {key: np.concatenate([p[key] for p in parts], axis=1) for key in parts[0]}


@pytest.mark.parametrize("mode", ["x_x_positive", "x_x_negative", "zero_x"])
def test_stats_at_every_binary16_range_value(oracle, mode):
    H = CHUNK // 64
    Lg = K.make_layout(1, H, 64, 4, (2,))
    kc, vc = K.alloc_cache(Lg), K.alloc_cache(Lg)
    src = torch.empty((1, 2, H, 64), dtype=torch.float32, device=DEV)
    for start in range(0, TOP + 1, CHUNK):
        n = min(CHUNK, TOP + 1 - start)
        print(f"[stats] {mode} patterns {start:#x} + {n}", flush=True)
        pat = torch.arange(start, start + CHUNK, dtype=torch.int32, device=DEV)
        pat[n:] = 0
        x = pat.view(torch.float32).view(H, 64)
        if mode == "x_x_negative":
            x = -x
        src[0, 0] = 0.0 if mode == "zero_x" else x
        src[0, 1] = x
        K.kvq_quantize_block(Lg, 0, src, src, kc, vc)
        torch.cuda.synchronize()
        got = cache_to_host(kc)
        ref = _oracle_cache(oracle, src.cpu().numpy())
        for key in ("zero", "scale", "codes"):
            if not np.array_equal(got[key], ref[key]):
                idx = tuple(np.argwhere(got[key] != ref[key])[0])
                h, d = idx[1], idx[-1] if key != "codes" else 0
                raise AssertionError(f"{mode} {key} at {idx}: gpu {got[key][idx]} oracle "
                                     f"{ref[key][idx]} (x = {src[0, 1, h, d].item()!r})")
