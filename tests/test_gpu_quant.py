"""GPU parity of kvq_quantize_block / kvq_pack / kvq_unpack / kvq_dequantize
against the CPU oracle: statistics, codes and packed bytes bit for bit."""
import numpy as np
import pytest
import torch

import varq_inputs as vi
import visual_autoregressive_kv_amd as K
from gpu_common import DEV, assert_cache_equal, cache_to_host, fill_both, layouts, to_dev

pytestmark = pytest.mark.gpu


def test_tiny_fp32_int4_all_blocks(oracle):
    wl = vi.WORKLOADS["var256_tiny_int4"]
    _, _, kg, vg, ko, vo = fill_both(oracle, wl)
    assert_cache_equal(kg, ko, "K")
    assert_cache_equal(vg, vo, "V")


@pytest.mark.parametrize("name", ["var_d20_b128_int4", "var_d20_b128_int3_rope",
                                  "var_d24_b128_int3"])
def test_var_shapes_reduced_batch_all_blocks(oracle, name):
    wl = vi.WORKLOADS[name].with_(batch=3)
    _, _, kg, vg, ko, vo = fill_both(oracle, wl, layer=5)
    assert_cache_equal(kg, ko, name + " K")
    assert_cache_equal(vg, vo, name + " V")


@pytest.mark.parametrize("name,block", [("var_d20_b128_int4", 9), ("var_d20_b128_int4", 3),
                                        ("var_d20_b128_int3_rope", 8)])
def test_full_batch_block(oracle, name, block):
    """Full VAR-d20 batch (128) in the bench's launch configuration, one block."""
    wl = vi.WORKLOADS[name]
    Lg, Lo = layouts(oracle, wl)
    kg, vg = K.alloc_cache(Lg), K.alloc_cache(Lg)
    ko, vo = oracle.alloc_cache(Lo), oracle.alloc_cache(Lo)
    kb = vi.kv_block(wl, 11, "k", block)
    vb = vi.kv_block(wl, 11, "v", block)
    assert oracle.quantize_block(Lo, block, kb, vb, ko, vo) == 0
    K.kvq_quantize_block(Lg, block, to_dev(kb), to_dev(vb), kg, vg)
    torch.cuda.synchronize()
    assert_cache_equal(kg, ko, "K")
    assert_cache_equal(vg, vo, "V")


def test_video_frames_two_pass_path(oracle):
    """D=128, 1560-token frames at batch 1 (80 tiles): the token-sliced path."""
    wl = vi.WORKLOADS["video_16x1560_h40d128_int3"].with_(blocks=(1560, 1560, 1560))
    _, _, kg, vg, ko, vo = fill_both(oracle, wl)
    assert_cache_equal(kg, ko, "K")
    assert_cache_equal(vg, vo, "V")


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_large_blocks_many_tiles(oracle, bits):
    """Blocks too large for registers with at least 1024 (tensor, b, h) tiles:
    one workgroup per tile streams it twice."""
    wl = vi.Workload("many", 1, 13, 40, 128, bits, (3, 200), "bf16", seed=11)
    _, _, kg, vg, ko, vo = fill_both(oracle, wl)
    assert_cache_equal(kg, ko, "K")
    assert_cache_equal(vg, vo, "V")


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("src", ["bf16", "f32"])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_ragged_edge_shapes(oracle, bits, src, head_dim):
    """Odd batch/heads, single-token blocks, block sizes off every tile multiple,
    a block just past the register-resident limit (two-pass path)."""
    big = 257 if head_dim == 64 else 129
    wl = vi.Workload("edge", 1, 5, 3, head_dim, bits, (1, 7, 33, big, 3, 2),
                     src, rope=(bits == 3), seed=7)
    _, _, kg, vg, ko, vo = fill_both(oracle, wl)
    assert_cache_equal(kg, ko, "K")
    assert_cache_equal(vg, vo, "V")


def test_writes_stay_inside_the_block(oracle):
    """Canary bytes: only rows [off_k, off_k + n_k) and stats slot k change
    (the 300-token block takes the token-sliced path, which parks its slice
    extremes in the block's own rows)."""
    wl = vi.Workload("canary", 1, 3, 5, 64, 3, (1, 4, 9, 16, 25, 36, 300), "bf16", seed=3)
    Lg, Lo = layouts(oracle, wl)
    for block in range(len(wl.blocks)):
        kg, vg = K.alloc_cache(Lg), K.alloc_cache(Lg)
        for c in (kg, vg):
            c["codes"].fill_(0xA5)
            c["zero"].view(torch.int16).fill_(0x5A5A)
            c["scale"].view(torch.int16).fill_(0x3C3C)
        before = [cache_to_host(kg), cache_to_host(vg)]
        K.kvq_quantize_block(Lg, block, to_dev(vi.kv_block(wl, 0, "k", block)),
                             to_dev(vi.kv_block(wl, 0, "v", block)), kg, vg)
        torch.cuda.synchronize()
        off, n = wl.offset(block), wl.blocks[block]
        for c, b4 in zip((kg, vg), before):
            a = cache_to_host(c)
            mask = np.ones(a["codes"].shape, bool)
            mask[:, :, off:off + n, :] = False
            assert np.array_equal(a["codes"][mask], b4["codes"][mask])
            smask = np.ones(a["zero"].shape, bool)
            smask[:, :, block, :] = False
            assert np.array_equal(a["zero"][smask], b4["zero"][smask])
            assert np.array_equal(a["scale"][smask], b4["scale"][smask])


def test_deterministic(oracle):
    wl = vi.WORKLOADS["var_d20_b128_int3_rope"].with_(batch=4)
    Lg, _ = layouts(oracle, wl)
    outs = []
    kb, vb = to_dev(vi.kv_block(wl, 0, "k", 9)), to_dev(vi.kv_block(wl, 0, "v", 9))
    for _ in range(2):
        kg, vg = K.alloc_cache(Lg), K.alloc_cache(Lg)
        K.kvq_quantize_block(Lg, 9, kb, vb, kg, vg)
        torch.cuda.synchronize()
        outs.append((cache_to_host(kg), cache_to_host(vg)))
    for key in ("codes", "zero", "scale"):
        assert np.array_equal(outs[0][0][key], outs[1][0][key])
        assert np.array_equal(outs[0][1][key], outs[1][1][key])


@pytest.mark.parametrize("src", ["bf16", "f32"])
@pytest.mark.parametrize("n,row", [(16, 2), (300, 290)])
def test_status_flags(oracle, src, n, row):
    """Screened quantization: NaN/Inf and out-of-binary16-range inputs set their
    flags; one register pass (16 tokens) and the token-sliced path (300)."""
    wl = vi.Workload("status", 1, 2, 3, 64, 4, (16, n), src, seed=5)
    Lg, _ = layouts(oracle, wl)
    kb = vi.kv_block(wl, 0, "k", 1)
    vb = vi.kv_block(wl, 0, "v", 1)

    def run(k, v):
        kg, vg = K.alloc_cache(Lg), K.alloc_cache(Lg)
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        K.kvq_quantize_block(Lg, 1, to_dev(k), to_dev(v), kg, vg, status=st)
        torch.cuda.synchronize()
        return int(st.item()), kg, vg

    st, kg, vg = run(kb, vb)
    assert st == 0
    Lo = oracle.layout_of(wl)
    ko, vo = oracle.alloc_cache(Lo), oracle.alloc_cache(Lo)
    oracle.quantize_block(Lo, 1, kb, vb, ko, vo)
    assert np.array_equal(cache_to_host(kg)["codes"][:, :, 16:], ko["codes"][:, :, 16:])

    def put(arr, val):
        a = arr.copy()
        if src == "f32":
            a[1, row, 2, 17] = np.float32(val)
        else:
            a[1, row, 2, 17] = vi.f32_to_bf16_bits(np.array([val], np.float32))[0]
        return a

    for val, flag in [(np.nan, K.S_NONFINITE), (np.inf, K.S_NONFINITE),
                      (-np.inf, K.S_NONFINITE), (70000.0, K.S_RANGE), (-1e6, K.S_RANGE)]:
        st, _, _ = run(put(kb, val), vb)
        assert st & flag, (val, st)
        st, _, _ = run(kb, put(vb, val))
        assert st & flag, (val, st)


# ---------------------------------------------------------------------------
# standalone pack / unpack / dequantize
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("row_len,extra", [(64, 0), (128, 0), (64, 5), (13, 0), (13, 3)])
def test_pack_matches_oracle(oracle, bits, row_len, extra):
    rng = np.random.default_rng(bits * 100 + row_len + extra)
    n_rows = 1003
    codes = rng.integers(0, 256, (n_rows, row_len), dtype=np.uint8)  # high bits ignored
    R = (bits * row_len + 7) // 8
    stride = R + extra
    ref = oracle.pack(bits, codes, dst_row_stride=stride)
    dst = torch.full((n_rows, stride), 0xEE, dtype=torch.uint8, device=DEV)
    K.kvq_pack(bits, torch.from_numpy(codes).to(DEV), dst)
    got = dst.cpu().numpy()
    assert np.array_equal(got[:, :R], ref[:, :R])
    assert (got[:, R:] == 0xEE).all()  # bytes between rows untouched
    back = torch.zeros((n_rows, row_len), dtype=torch.uint8, device=DEV)
    K.kvq_unpack(bits, dst, row_len, back)
    assert np.array_equal(back.cpu().numpy(), codes & ((1 << bits) - 1))


def test_pack_matches_fused_quantizer(oracle):
    """kvq_pack of the oracle's codes gives the bytes the fused kernel stores."""
    wl = vi.WORKLOADS["var_d20_b128_int3_rope"].with_(batch=2)
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl, upto=10)
    codes = oracle.unpack(3, ko["codes"].reshape(-1, 24), 64)
    dst = torch.zeros((codes.shape[0], 24), dtype=torch.uint8, device=DEV)
    K.kvq_pack(3, torch.from_numpy(codes).to(DEV), dst)
    assert np.array_equal(dst.cpu().numpy(), cache_to_host(kg)["codes"].reshape(-1, 24))


@pytest.mark.parametrize("name", ["var256_tiny_int4", "var_d20_b128_int3_rope"])
def test_dequantize_matches_oracle(oracle, name):
    wl = vi.WORKLOADS[name]
    if wl.batch > 2:
        wl = wl.with_(batch=2)
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl)
    for n_filled in (1, 7, 10):
        T = wl.offset(n_filled)
        out = torch.zeros((wl.batch, wl.heads, T, wl.head_dim), dtype=torch.float32, device=DEV)
        K.kvq_dequantize(Lg, n_filled, vg, out)
        ref = oracle.dequantize(Lo, n_filled, vo)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("n_rows,row_len", [(1, 1), (5, 64), (37, 128), (680, 64)])
def test_word_aligned_pack_matches_oracle(oracle, bits, n_rows, row_len):
    """pack_mode 1 (one stream of 32-bit words, floor(32/bits) codes each):
    bit-exact against the oracle, and unpack inverts it."""
    rng = np.random.default_rng(100 * bits + n_rows)
    codes = rng.integers(0, 1 << bits, size=(n_rows, row_len), dtype=np.uint8)
    ref = oracle.pack(bits, codes, pack_mode=1)
    dst = torch.full((ref.size + 16,), 0xA5, dtype=torch.uint8, device=DEV)
    K.kvq_pack(bits, torch.from_numpy(codes).to(DEV), dst, pack_mode=1)
    back = torch.zeros((n_rows, row_len), dtype=torch.uint8, device=DEV)
    K.kvq_unpack(bits, dst, row_len, back, pack_mode=1)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    assert np.array_equal(got[:ref.size], ref)
    assert (got[ref.size:] == 0xA5).all()  # nothing written past the last word
    assert np.array_equal(back.cpu().numpy(), codes)
