"""Inputs at the edge of the binary16 range through the whole decode path.

Binary32 input may reach +-65504, and a group such as {0, 65504} or
{-65504, 65504} is in range (status 0), yet its top grid level z + L*s lies
above 65504 once the step is rounded up (INT4: 15 * 4368 = 65520, 65536 for
the symmetric group; INT3: 7 * 9360 = 65520).  The attention forms v_hat in
binary16 for its PV product; it must not overflow there.  Checked against the
oracle, whose dequantized values are binary32 (VAR-Q abstract: massive-value
outlier channels, the regime these groups stand for taken to the limit of the
binary16 statistics)."""
import numpy as np
import pytest
import torch

import varq_inputs as vi
import visual_autoregressive_kv_amd as K
from gpu_common import DEV, assert_cache_equal, check_attn, to_dev

pytestmark = pytest.mark.gpu

EDGE = np.float32(65504.0)


def edge_block(rng, B, n, H, D, tensor):
    """N(0, 1) values with edge groups in heads 0 and 2 (V: the binary16 v_hat of
    the PV product) or head 1 (K: the hi/lo split of k_hat)."""
    x = rng.standard_normal((B, n, H, D)).astype(np.float32)
    heads = (0, 2) if tensor == "v" else (1,)
    for h in heads:
        x[:, :, h, 0] = np.where(np.arange(n) % 2 == 1, EDGE, 0.0)         # {0, 65504}
        x[:, :, h, 1] = np.where(np.arange(n) % 2 == 1, EDGE, -EDGE)       # {-65504, 65504}
        x[:, :, h, 2] = EDGE                                               # constant 65504
        x[:, :, h, 3] = np.where(np.arange(n) % 3 == 0, -EDGE, 0.0)        # {-65504, 0}
        x[:, :, h, 9] = np.where(np.arange(n) % 2 == 0, np.float32(65000.0), EDGE)
        x[:, 0, h, 11] = EDGE                                              # one extreme token
    if n == 1:  # a one-token block: {65504} and {-65504} groups
        for h in heads:
            x[:, 0, h, 1] = -EDGE
    return x


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("blocks,bf16_from", [((1, 4, 9, 16, 25), None), ((5, 40, 33), None),
                                              ((700, 300), None), ((170, 180), 1)],
                         ids=["short", "workgroup", "key_ranges", "bf16_after_edges"])
def test_binary16_edge_groups(oracle, bits, blocks, bf16_from):
    """bf16_from: the first block given as bf16 (N(0, 1) values, no edge groups;
    bf16 input cannot reach a top level above 65504, since its largest value
    below 65504 is 65280): the fused call then takes its workgroup kernels
    (here the 8-wave one), with v_hat halved for the cached edge groups."""
    B, H, D = 2, 3, 64
    rng = np.random.default_rng(1000 + 10 * bits + len(blocks))
    Lg = K.make_layout(B, H, D, bits, blocks)
    Lo = oracle.make_layout(B, H, D, bits, blocks)
    kg, vg = K.alloc_cache(Lg), K.alloc_cache(Lg)
    kf, vf = K.alloc_cache(Lg), K.alloc_cache(Lg)
    ko, vo = oracle.alloc_cache(Lo), oracle.alloc_cache(Lo)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    for j, n in enumerate(blocks):
        if bf16_from is not None and j >= bf16_from:
            kb = vi.f32_to_bf16_bits(rng.standard_normal((B, n, H, D)).astype(np.float32))
            vb = vi.f32_to_bf16_bits(rng.standard_normal((B, n, H, D)).astype(np.float32))
        else:
            kb, vb = edge_block(rng, B, n, H, D, "k"), edge_block(rng, B, n, H, D, "v")
        qf = rng.standard_normal((B, n, H, D)).astype(np.float32)
        # head 1 holds the K edge groups: its queries are scaled by 2^-10 (exact)
        # so that its scores stay in the range the accuracy bound covers
        # (sum_d |scale q_d k_d| of order 10, as on VAR-shaped data)
        qf[:, :, 1, :] *= np.float32(2.0 ** -10)
        q = (qf.view(np.uint32) >> 16).astype(np.uint16)  # bf16 by truncation
        assert oracle.quantize_block(Lo, j, kb, vb, ko, vo) == 0
        K.kvq_quantize_block(Lg, j, to_dev(kb), to_dev(vb), kg, vg, status=status)
        of = torch.full((B, n, H, D), float("nan"), dtype=torch.float32, device=DEV)
        K.kvq_quantize_attend(Lg, j, to_dev(kb), to_dev(vb), to_dev(q), kf, vf, of, status=status)
        out = torch.full_like(of, float("nan"))
        K.kvq_attend_packed(Lg, j, to_dev(q), kg, vg, out)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "in-range edge values flagged"
        ref = oracle.attend(Lo, j, q, ko, vo).astype(np.float64)
        got = out.cpu().numpy()
        check_attn(got, ref, f"edge INT{bits} {blocks} block {j}")
        fused = of.cpu().numpy()
        assert np.array_equal(fused.view(np.uint32), got.view(np.uint32)), j
        if n > 128:
            ws_bytes = K.kvq_attend_split_workspace(Lg, j, 4)
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
            osp = torch.full_like(of, float("nan"))
            K.kvq_attend_packed_split(Lg, j, to_dev(q), kg, vg, osp, ws, max_splits=4)
            torch.cuda.synchronize()
            check_attn(osp.cpu().numpy(), ref, f"edge INT{bits} {blocks} block {j} key ranges")
    assert_cache_equal(kg, ko, "K")
    assert_cache_equal(vg, vo, "V")
    assert_cache_equal(kf, ko, "fused K")
    assert_cache_equal(vf, vo, "fused V")

