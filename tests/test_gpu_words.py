"""GPU parity of the block-aligned word layout (pack_mode 2): each (sequence,
head, block) stream of codes in 32-bit words, ten 3-bit codes per word, every
block from a fresh word.  The caches that kvq_quantize_block and
kvq_quantize_attend write are bit-exact against the oracle's in the same
layout; kvq_bytes is the allocation the calls address; attention over the word
layout is bit-identical to attention over dense rows holding the same codes
(the same dequantized values in the same order), and within the attention
tolerance of the binary64 oracle.  At 2, 4 and 8 bits the layout is byte for
byte the dense rows (head_dim 64 and 128 fill whole words per block)."""
import numpy as np
import pytest
import torch

import varq_inputs as vi
import visual_autoregressive_kv_amd as K
from gpu_common import (DEV, assert_cache_equal, check_attn, fill_both, layouts,
                        oracle_attend_batch, to_dev)

pytestmark = pytest.mark.gpu


def attend(Lg, block, q_np, kg, vg):
    out = torch.full(tuple(q_np.shape), float("nan"), dtype=torch.float32, device=DEV)
    K.kvq_attend_packed(Lg, block, to_dev(q_np), kg, vg, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def same_bits(a, b):
    return np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_bytes_match_the_allocation_and_the_oracle(oracle, bits, head_dim):
    blocks = vi.VAR_BLOCKS
    Lg = K.make_layout(3, 5, head_dim, bits, blocks, pack_mode=2)
    Lo = oracle.make_layout(3, 5, head_dim, bits, blocks, pack_mode=2)
    for n in range(len(blocks) + 1):
        assert K.kvq_bytes(Lg, n) == oracle.nbytes(Lo, n)
    c = K.alloc_cache(Lg)
    assert c["codes"].numel() == K.kvq_bytes(Lg, len(blocks))[0]
    if 32 % bits == 0:  # whole words per block: the dense rows' bytes
        L0 = K.make_layout(3, 5, head_dim, bits, blocks)
        assert K.kvq_bytes(Lg, len(blocks)) == K.kvq_bytes(L0, len(blocks))


def test_var_d20_int3_size_is_the_tables(oracle):
    """VAR-d20 at 2 x 128 sequences, 20 layers, K and V: 3.81 GiB, 77.04%."""
    Lg = K.make_layout(256, 20, 64, 3, vi.VAR_BLOCKS, pack_mode=2)
    cb, sb = K.kvq_bytes(Lg, 10)
    assert cb == 256 * 20 * 4 * 4356
    gib = 2 * 20 * (cb + sb) / float(1 << 30)
    bf16 = 2 * 20 * 256 * 680 * 1280 * 2 / float(1 << 30)
    assert round(gib, 2) == 3.81 and round(100 * (1 - gib / bf16), 2) == 77.04


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_quantize_every_block_bit_exact(oracle, bits):
    """VAR schedule at batch 3, every block (one-pass tiles of 1..256 rows)."""
    wl = vi.WORKLOADS["var_d20_b128_int3_rope"].with_(batch=3, bits=bits)
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl, layer=2, pack_mode=2)
    assert kg["codes"].shape == ko["codes"].shape
    assert_cache_equal(kg, ko, f"int{bits} K")
    assert_cache_equal(vg, vo, f"int{bits} V")
    if bits != 3:  # the same bytes as dense rows
        _, _, k0, _, _, _ = fill_both(oracle, wl, layer=2, pack_mode=0)
        assert np.array_equal(kg["codes"].cpu().numpy().ravel(), k0["codes"].cpu().numpy().ravel())


@pytest.mark.parametrize("head_dim", [64, 128])
def test_quantize_streamed_passes(oracle, head_dim):
    """Blocks too large for registers over many tiles: passes of 5 rows per
    thread, each starting on a word; ragged last pass, odd block sizes."""
    wl = vi.Workload("wstream", 1, 13, 40, head_dim, 3, (3, 333, 161), "bf16", seed=61)
    _, _, kg, vg, ko, vo = fill_both(oracle, wl, pack_mode=2)
    assert_cache_equal(kg, ko, "K")
    assert_cache_equal(vg, vo, "V")


def test_quantize_token_slices(oracle):
    """Few large tiles (batch 1, 40 heads x 128): slices of 80 rows, each on a
    word boundary, extremes parked in the block's words."""
    wl = vi.WORKLOADS["video_16x1560_h40d128_int3"].with_(blocks=(1560, 1561, 7))
    _, _, kg, vg, ko, vo = fill_both(oracle, wl, pack_mode=2)
    assert_cache_equal(kg, ko, "K")
    assert_cache_equal(vg, vo, "V")


def test_quantize_fp32_source(oracle):
    wl = vi.WORKLOADS["var256_tiny_int4"].with_(bits=3)
    _, _, kg, vg, ko, vo = fill_both(oracle, wl, pack_mode=2)
    assert_cache_equal(kg, ko, "K")
    assert_cache_equal(vg, vo, "V")


def test_quantize_writes_only_its_block(oracle):
    """A block's words are written and no other byte: neighbours keep a fill."""
    wl = vi.Workload("only", 1, 2, 3, 64, 3, (5, 17, 9), "bf16", seed=67)
    Lg, Lo = layouts(oracle, wl, 2)
    kg, vg = K.alloc_cache(Lg), K.alloc_cache(Lg)
    for c in (kg, vg):
        c["codes"].fill_(0xA5)
    kb, vb = vi.kv_block(wl, 0, "k", 1), vi.kv_block(wl, 0, "v", 1)
    K.kvq_quantize_block(Lg, 1, to_dev(kb), to_dev(vb), kg, vg)
    torch.cuda.synchronize()
    w0 = oracle.block_word_offset(Lo, 1)
    w1 = oracle.block_word_offset(Lo, 2)
    codes = kg["codes"].cpu().numpy()
    assert (codes[:, :, : 4 * w0] == 0xA5).all() and (codes[:, :, 4 * w1:] == 0xA5).all()
    assert not (codes[:, :, 4 * w0: 4 * w1] == 0xA5).all()


@pytest.mark.parametrize("wl", [
    vi.WORKLOADS["var_d20_b128_int3_rope"].with_(batch=2),
    vi.Workload("edge", 1, 1, 3, 64, 3, (1, 7, 32, 33, 2, 256, 3), "bf16", rope=True, seed=71),
    vi.Workload("edge128", 1, 2, 3, 128, 3, (5, 31, 40, 300), "bf16", seed=73),
    vi.Workload("many_blocks", 1, 2, 3, 64, 3, (1,) * 20 + (5, 40, 3), "bf16", seed=79),
], ids=["d20", "edge", "edge_d128", "many_blocks"])
def test_attention_equals_dense_rows_and_oracle(oracle, wl):
    """Every block: the one-wave, 1/2/4/8-wave kernels over the word layout
    give the dense-row kernels' bits, and the oracle's values."""
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl, pack_mode=2)
    assert_cache_equal(kg, ko, "K")
    assert_cache_equal(vg, vo, "V")
    L0, _, k0, v0, _, _ = fill_both(oracle, wl, pack_mode=0)
    for block in range(len(wl.blocks)):
        q = vi.q_block(wl, 0, block)
        got = attend(Lg, block, q, kg, vg)
        dense = attend(L0, block, q, k0, v0)
        assert same_bits(got, dense), block
        ref = oracle.attend(Lo, block, q, ko, vo).astype(np.float64)
        check_attn(got, ref, f"words {wl.name} block {block}")


def test_split_ranges_equal_dense_rows(oracle):
    """Key ranges (the split kernel) over the word layout: frames of 1560 tokens
    at head_dim 128, 3 frames; the same bits as the dense rows' split call, and
    the whole output against the binary64 oracle."""
    wl = vi.WORKLOADS["video_16x1560_h40d128_int3"].with_(blocks=(1560, 1560, 1560))
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl, pack_mode=2)
    L0, _, k0, v0, _, _ = fill_both(oracle, wl, pack_mode=0)
    q_np = vi.q_block(wl, 0, 2)
    q = to_dev(q_np)
    outs = []
    for L, kc, vc in ((Lg, kg, vg), (L0, k0, v0)):
        ws = torch.empty(K.kvq_attend_split_workspace(L, 2, 8), dtype=torch.uint8, device=DEV)
        o = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=DEV)
        K.kvq_attend_packed_split(L, 2, q, kc, vc, o, ws, max_splits=8)
        torch.cuda.synchronize()
        outs.append(o.cpu().numpy())
    assert same_bits(outs[0], outs[1])
    check_attn(outs[0], oracle_attend_batch(oracle, Lo, 2, q_np, ko, vo), "words video split")


@pytest.mark.parametrize("wl", [
    vi.WORKLOADS["var_d20_b128_int3_rope"].with_(batch=2),
    vi.Workload("edge", 1, 1, 3, 64, 3, (1, 7, 32, 33, 2, 256, 3), "bf16", rope=True, seed=83),
    vi.Workload("f32", 1, 2, 3, 64, 3, (1, 4, 9, 16, 25), "f32", seed=89),
    vi.Workload("d128", 1, 2, 3, 128, 3, (5, 31, 40, 97, 256), "bf16", seed=97),
], ids=["d20", "edge", "f32_short", "d128"])
def test_fused_equals_two_calls_and_oracle(oracle, wl):
    """kvq_quantize_attend over the word layout (the one-wave and workgroup
    fused kernels at head_dim 64 and 128; two launches where none covers the
    shape): the cache is the oracle's and the outputs are those of the two
    calls, bit for bit."""
    Lg, Lo = layouts(oracle, wl, 2)
    kf, vf = K.alloc_cache(Lg), K.alloc_cache(Lg)
    ks, vs = K.alloc_cache(Lg), K.alloc_cache(Lg)
    ko, vo = oracle.alloc_cache(Lo), oracle.alloc_cache(Lo)
    for j in range(len(wl.blocks)):
        kb, vb = vi.kv_block(wl, 0, "k", j), vi.kv_block(wl, 0, "v", j)
        q = vi.q_block(wl, 0, j)
        assert oracle.quantize_block(Lo, j, kb, vb, ko, vo) == 0
        of = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
        os_ = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
        K.kvq_quantize_attend(Lg, j, to_dev(kb), to_dev(vb), to_dev(q), kf, vf, of)
        K.kvq_quantize_block(Lg, j, to_dev(kb), to_dev(vb), ks, vs)
        K.kvq_attend_packed(Lg, j, to_dev(q), ks, vs, os_)
        torch.cuda.synchronize()
        got, two = of.cpu().numpy(), os_.cpu().numpy()
        assert same_bits(got, two), j
        ref = oracle.attend(Lo, j, q, ko, vo).astype(np.float64)
        check_attn(got, ref, f"words fused {wl.name} block {j}")
    assert_cache_equal(kf, ko, "fused K")
    assert_cache_equal(vf, vo, "fused V")


def test_dequantize_matches_oracle(oracle):
    wl = vi.Workload("deq", 1, 2, 3, 64, 3, (1, 4, 9, 16, 25, 36), "bf16", seed=101)
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl, pack_mode=2)
    for n in (1, 3, 6):
        T = sum(wl.blocks[:n])
        out = torch.full((2, 3, T, 64), float("nan"), dtype=torch.float32, device=DEV)
        K.kvq_dequantize(Lg, n, vg, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), oracle.dequantize(Lo, n, vo)), n


def test_full_batch_decode(oracle):
    """VAR-d20 INT3 at batch 128 (the decode configuration), every block through
    kvq_quantize_attend in the word layout: caches bit-exact against the oracle,
    the whole outputs of blocks 4, 7 and 10 against the binary64 oracle (its
    sequences on host threads)."""
    wl = vi.WORKLOADS["var_d20_b128_int3_rope"]
    Lg, Lo = layouts(oracle, wl, 2)
    kg, vg = K.alloc_cache(Lg), K.alloc_cache(Lg)
    ko, vo = oracle.alloc_cache(Lo), oracle.alloc_cache(Lo)
    for j in range(len(wl.blocks)):
        kb, vb = vi.kv_block(wl, 0, "k", j), vi.kv_block(wl, 0, "v", j)
        assert oracle.quantize_block(Lo, j, kb, vb, ko, vo) == 0
        q_np = vi.q_block(wl, 0, j)
        out = torch.full(q_np.shape, float("nan"), dtype=torch.float32, device=DEV)
        K.kvq_quantize_attend(Lg, j, to_dev(kb), to_dev(vb), to_dev(q_np), kg, vg, out)
        torch.cuda.synchronize()
        if j in (3, 6, 9):
            ref = oracle_attend_batch(oracle, Lo, j, q_np, ko, vo)
            check_attn(out.cpu().numpy(), ref, f"words d20 batch 128 block {j}")
    assert_cache_equal(kg, ko, "K")
    assert_cache_equal(vg, vo, "V")


def test_dense_only_calls_reject_stream_mode():
    """pack_mode 1 (one stream per (sequence, head)) is not block-writable."""
    Lg = K.make_layout(1, 2, 64, 3, (4, 9), pack_mode=1)
    c = K.alloc_cache(K.make_layout(1, 2, 64, 3, (4, 9)))
    kb = torch.zeros((1, 4, 2, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(K.KvqError):
        K.kvq_quantize_block(Lg, 0, kb, kb, c, c)
