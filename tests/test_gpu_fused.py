"""GPU parity of kvq_quantize_attend (one decode step of one layer): the cache it
writes is bit-exact against the oracle, its outputs are bit-identical to
kvq_quantize_block followed by kvq_attend_packed, and within the attention
tolerance of the binary64 oracle."""
import numpy as np
import pytest
import torch

import varq_inputs as vi
import visual_autoregressive_kv_amd as K
from gpu_common import DEV, assert_cache_equal, check_attn, layouts, oracle_attend_batch, to_dev

pytestmark = pytest.mark.gpu


def decode_both_ways(oracle, wl, layer=0, scale=0.0):
    """Block-by-block decode through the fused call and through the two calls."""
    Lg, Lo = layouts(oracle, wl)
    kf, vf = K.alloc_cache(Lg), K.alloc_cache(Lg)
    ks, vs = K.alloc_cache(Lg), K.alloc_cache(Lg)
    ko, vo = oracle.alloc_cache(Lo), oracle.alloc_cache(Lo)
    steps = []
    for j in range(len(wl.blocks)):
        kb, vb = vi.kv_block(wl, layer, "k", j), vi.kv_block(wl, layer, "v", j)
        q = vi.q_block(wl, layer, j)
        assert oracle.quantize_block(Lo, j, kb, vb, ko, vo) == 0
        of = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
        os_ = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
        K.kvq_quantize_attend(Lg, j, to_dev(kb), to_dev(vb), to_dev(q), kf, vf, of, scale=scale)
        K.kvq_quantize_block(Lg, j, to_dev(kb), to_dev(vb), ks, vs)
        K.kvq_attend_packed(Lg, j, to_dev(q), ks, vs, os_, scale=scale)
        torch.cuda.synchronize()
        ref = oracle.attend(Lo, j, q, ko, vo, scale=scale).astype(np.float64)
        steps.append((j, of.cpu().numpy(), os_.cpu().numpy(), ref))
    return kf, vf, ks, vs, ko, vo, steps


@pytest.mark.parametrize("wl", [
    vi.WORKLOADS["var256_tiny_int4"],
    vi.WORKLOADS["var_d20_b128_int4"].with_(batch=2),
    vi.WORKLOADS["var_d20_b128_int3_rope"].with_(batch=2),
    vi.WORKLOADS["var_d24_b128_int4"].with_(batch=2, layers=1),
    vi.Workload("edge", 1, 1, 3, 64, 3, (1, 7, 32, 33, 2), "bf16", rope=True, seed=13),
    vi.Workload("edge128", 1, 2, 3, 128, 4, (5, 31, 40), "bf16", seed=17),
    # 23 blocks: the one-wave fused kernel while the statistics fit its LDS (8
    # blocks), then two launches for short blocks, the workgroup kernel for 40
    vi.Workload("many_blocks", 1, 2, 3, 64, 3, (1,) * 20 + (5, 40, 3), "bf16", seed=29),
    # the INT2 and INT8 widths (the results table's Infinity rows) through every
    # fused kernel shape, and INT8 from fp32 on short blocks
    vi.Workload("int2", 1, 2, 3, 64, 2, vi.VAR_BLOCKS, "bf16", seed=41),
    vi.Workload("int8_rope", 1, 2, 3, 64, 8, (1, 7, 32, 33, 100, 256), "bf16", rope=True, seed=43),
    vi.Workload("int8_f32", 1, 2, 3, 64, 8, (1, 4, 9, 16, 25), "f32", seed=47),
    # head_dim 128 through the workgroup fused kernels (2, 4 and 8 waves; a
    # 2-wave workgroup takes 4 lanes per 8-channel chunk, the others 8 lanes
    # and two waves per row), every width, ragged blocks up to 256 tokens
    vi.Workload("d128_int4", 1, 2, 3, 128, 4, (1, 33, 64, 65, 100, 128, 129, 256), "bf16",
                seed=101),
    vi.Workload("d128_int3_rope", 1, 2, 3, 128, 3, vi.VAR_BLOCKS, "bf16", rope=True, seed=103),
    vi.Workload("d128_int2", 1, 2, 3, 128, 2, (7, 40, 97, 200), "bf16", seed=107),
    vi.Workload("d128_int8", 1, 2, 3, 128, 8, (7, 40, 97, 200), "bf16", seed=109),
    # the 8-wave fused kernel after long cached prefixes (129-256 tokens from
    # key tile 5 on) at every width, with ragged block and prefix ends, and
    # with 16 and 17 blocks of statistics in LDS
    vi.Workload("ovl_int3", 1, 2, 3, 64, 3, (160, 129, 255, 256), "bf16", seed=111),
    vi.Workload("ovl_int8_rope", 1, 2, 3, 64, 8, (1, 170, 193, 131), "bf16", rope=True,
                seed=113),
    vi.Workload("ovl_int2", 1, 2, 3, 64, 2, (161, 250), "bf16", seed=115),
    vi.Workload("ovl_16_blocks", 1, 2, 3, 64, 4, (10,) * 14 + (20, 140), "bf16", seed=117),
    vi.Workload("ovl_17_blocks", 1, 2, 3, 64, 4, (10,) * 16 + (140,), "bf16", seed=119),
], ids=["tiny_f32", "d20_int4", "d20_int3_rope", "d24_int4", "edge_int3", "edge_d128",
        "many_blocks", "int2", "int8_rope", "int8_f32", "d128_int4", "d128_int3_rope",
        "d128_int2", "d128_int8", "ovl_int3", "ovl_int8_rope", "ovl_int2", "ovl_16_blocks",
        "ovl_17_blocks"])
def test_fused_matches_two_calls_and_oracle(oracle, wl):
    kf, vf, ks, vs, ko, vo, steps = decode_both_ways(oracle, wl)
    assert_cache_equal(kf, ko, "fused K")
    assert_cache_equal(vf, vo, "fused V")
    assert_cache_equal(ks, ko, "two-call K")
    for j, of, os_, ref in steps:
        assert np.isfinite(of).all(), j
        assert np.array_equal(of.view(np.uint32), os_.view(np.uint32)), j
        check_attn(of, ref, f"fused {wl.name} block {j}")


def test_fused_explicit_scale(oracle):
    wl = vi.Workload("scale", 1, 2, 4, 64, 4, (1, 4, 9, 16, 25), "bf16", seed=23)
    *_, steps = decode_both_ways(oracle, wl, scale=0.07)
    for j, of, os_, ref in steps:
        assert np.array_equal(of.view(np.uint32), os_.view(np.uint32)), j
        check_attn(of, ref, f"fused explicit scale block {j}")


def test_fused_full_batch_every_block(oracle):
    """VAR-d20 at batch 128, the bench's configuration, every block (all three
    fused kernel shapes: one-wave, 2/4-wave and 8-wave): cache bit-exact against
    the two-call path and the oracle, outputs bit-identical to the two-call
    path, and every block's whole output against the binary64 oracle (its
    sequences on host threads)."""
    wl = vi.WORKLOADS["var_d20_b128_int4"]
    Lg, Lo = layouts(oracle, wl)
    kf, vf = K.alloc_cache(Lg), K.alloc_cache(Lg)
    ks, vs = K.alloc_cache(Lg), K.alloc_cache(Lg)
    ko, vo = oracle.alloc_cache(Lo), oracle.alloc_cache(Lo)
    for j in range(len(wl.blocks)):
        kb_np, vb_np = vi.kv_block(wl, 0, "k", j), vi.kv_block(wl, 0, "v", j)
        assert oracle.quantize_block(Lo, j, kb_np, vb_np, ko, vo) == 0
        kb, vb = to_dev(kb_np), to_dev(vb_np)
        q_np = vi.q_block(wl, 0, j)
        q = to_dev(q_np)
        of = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=DEV)
        os_ = torch.full_like(of, float("nan"))
        K.kvq_quantize_attend(Lg, j, kb, vb, q, kf, vf, of)
        K.kvq_quantize_block(Lg, j, kb, vb, ks, vs)
        K.kvq_attend_packed(Lg, j, q, ks, vs, os_)
        torch.cuda.synchronize()
        assert torch.equal(of.view(torch.int32), os_.view(torch.int32)), j
        ref = oracle_attend_batch(oracle, Lo, j, q_np, ko, vo)
        check_attn(of.cpu().numpy(), ref, f"fused d20 batch 128 block {j}")
    for a, b in ((kf, ks), (vf, vs)):
        for key in ("codes", "zero", "scale"):
            assert torch.equal(a[key], b[key]), key
    assert_cache_equal(kf, ko, "fused K")
    assert_cache_equal(vf, vo, "fused V")


@pytest.mark.parametrize("src,second,head_dim,first", [
    ("bf16", 16, 64, 16), ("f32", 16, 64, 16), ("bf16", 64, 64, 16), ("bf16", 200, 64, 16),
    ("bf16", 64, 128, 16), ("bf16", 200, 128, 16),
    # a 200-token block after 192 cached keys
    ("bf16", 200, 64, 192)])
def test_fused_status_flags(oracle, src, second, head_dim, first):
    """Input screening through the fused call: the one-wave path (16 tokens) and
    the workgroup path (64 and 200 tokens, head_dim 64 and 128, after a short
    and a long cached prefix)."""
    wl = vi.Workload("status", 1, 2, 3, head_dim, 4, (first, second), src, seed=5)
    Lg, _ = layouts(oracle, wl)
    k0, v0 = vi.kv_block(wl, 0, "k", 0), vi.kv_block(wl, 0, "v", 0)
    kb, vb = vi.kv_block(wl, 0, "k", 1), vi.kv_block(wl, 0, "v", 1)
    q = to_dev(vi.q_block(wl, 0, 1))

    def run(k, v):
        kg, vg = K.alloc_cache(Lg), K.alloc_cache(Lg)
        K.kvq_quantize_block(Lg, 0, to_dev(k0), to_dev(v0), kg, vg)
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        out = torch.empty(tuple(q.shape), dtype=torch.float32, device=DEV)
        K.kvq_quantize_attend(Lg, 1, to_dev(k), to_dev(v), q, kg, vg, out, status=st)
        torch.cuda.synchronize()
        return int(st.item())

    assert run(kb, vb) == 0

    def put(arr, val):
        a = arr.copy()
        if src == "f32":
            a[1, 3, 2, 17] = np.float32(val)
        else:
            a[1, 3, 2, 17] = vi.f32_to_bf16_bits(np.array([val], np.float32))[0]
        return a

    for val, flag in [(np.nan, K.S_NONFINITE), (np.inf, K.S_NONFINITE), (70000.0, K.S_RANGE),
                      (-1e6, K.S_RANGE)]:
        assert run(put(kb, val), vb) & flag, val
        assert run(kb, put(vb, val)) & flag, val


def test_fused_batch_768(oracle):
    """The batch-768 shape (30 heads x 64, INT3; 23040 (sequence, head) pairs
    per launch, the largest grids of the decode path), all ten blocks through
    the fused call on device-drawn inputs.  The inputs of three sequences are
    copied back for the oracle: their caches are bit-exact and their whole
    outputs of every block are within the attention tolerance."""
    wl = vi.WORKLOADS["var_w1920_b768_int3"]
    Lg, _ = layouts(oracle, wl)
    seqs = [0, 383, 767]
    Lo = oracle.layout_of(wl, batch=len(seqs))
    kf, vf = K.alloc_cache(Lg), K.alloc_cache(Lg)
    ko, vo = oracle.alloc_cache(Lo), oracle.alloc_cache(Lo)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(wl.seed)
    sel = torch.tensor(seqs, dtype=torch.int64, device=DEV)

    def host_bf16(t):
        return np.ascontiguousarray(t.index_select(0, sel).view(torch.int16).cpu().numpy()
                                    .view(np.uint16))

    for j in range(len(wl.blocks)):
        kb = vi.torch_block(wl, 0, "k", j, DEV, gen)
        vb = vi.torch_block(wl, 0, "v", j, DEV, gen)
        qb = vi.torch_block(wl, 0, "q", j, DEV, gen)
        out = torch.full(tuple(qb.shape), float("nan"), dtype=torch.float32, device=DEV)
        K.kvq_quantize_attend(Lg, j, kb, vb, qb, kf, vf, out)
        torch.cuda.synchronize()
        assert oracle.quantize_block(Lo, j, host_bf16(kb), host_bf16(vb), ko, vo) == 0
        ref = oracle_attend_batch(oracle, Lo, j, host_bf16(qb), ko, vo)
        check_attn(out.index_select(0, sel).cpu().numpy(), ref,
                   f"fused batch 768 block {j} (sequences {seqs})")
        del kb, vb, qb, out
    for dev_cache, ref in ((kf, ko), (vf, vo)):
        got = {key: t.index_select(0, sel) for key, t in dev_cache.items()}
        for key in ("codes", "zero", "scale"):
            g = got[key].cpu().numpy() if key == "codes" else \
                got[key].view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(g, ref[key]), key
