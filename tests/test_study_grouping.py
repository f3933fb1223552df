"""Grouping-accuracy study (CPU): VAR-Q's (block, channel) groups against
per-channel-over-sequence and per-token groups on synthetic caches.

Pins the qualitative claim of the VAR-Q abstract (outliers organised along the
channel and block axes; grouping along both of them) on inputs that carry that
structure: the (block, channel) grouping has the lowest dequantization error
and attention error, with and without RoPE on K, and its advantage over
sequence-long channel groups comes from the block axis (it shrinks when the
outlier magnitudes stop shifting between blocks).  The study's grouping code is
in `study_grouping.py`; the full 16-head table comes from running that file.
"""
import numpy as np
import pytest

import study_grouping as sg
import varq_inputs as vi
from oracle import binding as ob

HEADS = 4  # a quarter of the 16-head table's work; same distributions


@pytest.fixture(scope="module")
def results():
    out = {}
    for rope in (False, True):
        for persistent in (False, True):
            wl = sg.study_workload(rope, heads=HEADS, persistent=persistent)
            for bits in (3, 4):
                out[rope, persistent, bits] = sg.grouping_errors(wl, bits)
    return out


@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("bits", [3, 4])
def test_block_channel_is_most_accurate(results, rope, bits):
    r = results[rope, False, bits]
    for metric in ("k_mse", "v_mse", "attn"):
        bc, cs, tok = (r[g][metric] for g in sg.GROUPINGS)
        assert bc < cs < tok, (metric, r)
    # V carries no RoPE: the block axis alone is worth a large factor there
    assert r["channel_seq"]["v_mse"] > 3.0 * r["block_channel"]["v_mse"], r
    # per-token groups mix the massive channels into every group's range
    assert r["token"]["v_mse"] > 30.0 * r["block_channel"]["v_mse"], r


@pytest.mark.parametrize("bits", [3, 4])
def test_block_axis_is_the_source_of_the_gain(results, bits):
    """With the same magnitude in every block the (block, channel) advantage
    over sequence-long channel groups drops to what smaller groups give."""
    shifting = results[False, False, bits]
    fixed = results[False, True, bits]
    gain = lambda r: r["channel_seq"]["v_mse"] / r["block_channel"]["v_mse"]
    assert gain(fixed) < 2.0, fixed
    assert gain(shifting) > 2.0 * gain(fixed), (shifting, fixed)


def test_rope_scatters_k_within_blocks(results):
    """RoPE on K rotates each massive channel into its pair partner at a
    position-dependent angle, widening (block, channel) ranges of K but not
    of V (no RoPE on V)."""
    for bits in (3, 4):
        plain = results[False, False, bits]["block_channel"]
        roped = results[True, False, bits]["block_channel"]
        assert roped["k_mse"] > 5.0 * plain["k_mse"]
        assert roped["v_mse"] == plain["v_mse"]


def test_study_grouping_is_the_cache_grouping():
    """The study's block_channel path equals the oracle's cache path
    (kvqr_quantize_block then kvqr_dequantize), bit for bit."""
    wl = sg.study_workload(False, heads=2)
    k, v, _ = sg.study_cache(wl)
    L = ob.make_layout(1, wl.heads, wl.head_dim, 4, wl.blocks)
    kc, vc = ob.alloc_cache(L), ob.alloc_cache(L)
    for b in range(len(wl.blocks)):
        assert ob.quantize_block(L, b, vi.kv_block(wl, 0, "k", b, [0]),
                                 vi.kv_block(wl, 0, "v", b, [0]), kc, vc) == ob.OK
    kd = ob.dequantize(L, len(wl.blocks), kc)[0].transpose(1, 0, 2)  # [T, H, D]
    vd = ob.dequantize(L, len(wl.blocks), vc)[0].transpose(1, 0, 2)
    np.testing.assert_array_equal(sg.quantize_grouped(k, 4, "block_channel", wl.blocks), kd)
    np.testing.assert_array_equal(sg.quantize_grouped(v, 4, "block_channel", wl.blocks), vd)


def test_attention_helper_against_closed_forms():
    """softmax_attention: equal keys give the mean of V; one dominant key
    returns its value row."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 2, 8))
    v = rng.standard_normal((7, 2, 8))
    k = np.zeros((7, 2, 8))
    np.testing.assert_allclose(sg.softmax_attention(q, k, v),
                               np.broadcast_to(v.mean(0), (3, 2, 8)), rtol=0, atol=1e-12)
    q1 = np.ones((1, 1, 4))
    k1 = np.zeros((5, 1, 4))
    k1[2] = 200.0
    v1 = np.arange(20, dtype=np.float64).reshape(5, 1, 4)
    np.testing.assert_allclose(sg.softmax_attention(q1, k1, v1)[0, 0], v1[2, 0], atol=1e-12)
