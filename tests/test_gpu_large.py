"""GPU parity of the chunk-per-thread calls (kvq_pack, kvq_unpack,
kvq_dequantize) on inputs of more than 2^30 eight-code chunks, which they
process as several launches: sampled rows (those around the first launch
boundary among them) against the oracle, and the whole buffer round-tripped
through kvq_unpack.  Inputs of this size (8-35 GB) occur for whole caches on a
288 GB device; a single launch of them would exceed the 32-bit work-item count
of one dispatch."""
import numpy as np
import pytest
import torch

import visual_autoregressive_kv_amd as K
from gpu_common import DEV

pytestmark = pytest.mark.gpu

PIECE_CHUNKS = 1 << 30  # eight-code chunks per launch: 2^22 workgroups of 256 threads


def _rand_u8(shape, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randint(0, 256, shape, dtype=torch.uint8, device=DEV, generator=g)


@pytest.mark.parametrize("extra", [0, 1], ids=["dense_rows", "strided_rows"])
def test_pack_unpack_across_launch_pieces(oracle, extra):
    bits, row_len = 3, 40  # 5 chunks per row: the first launch boundary falls inside row 214748364
    n_rows = PIECE_CHUNKS // 5 + 4099
    R = (bits * row_len + 7) // 8
    codes = _rand_u8((n_rows, row_len), 7 + extra)
    dst = torch.full((n_rows, R + extra), 0xEE, dtype=torch.uint8, device=DEV)
    K.kvq_pack(bits, codes, dst)
    torch.cuda.synchronize()
    edge = PIECE_CHUNKS // 5
    rng = np.random.default_rng(11 + extra)
    rows = sorted(set(range(edge - 3, edge + 4)) | {0, n_rows - 1} |
                  set(int(r) for r in rng.integers(0, n_rows, 256)))
    idx = torch.tensor(rows, dtype=torch.int64, device=DEV)
    got = dst.index_select(0, idx).cpu().numpy()
    ref = oracle.pack(bits, codes.index_select(0, idx).cpu().numpy(), dst_row_stride=R)
    assert np.array_equal(got[:, :R], ref)
    if extra:
        assert bool((dst[:, R:] == 0xEE).all())  # bytes between rows untouched
    back = torch.empty_like(codes)
    K.kvq_unpack(bits, dst, row_len, back)
    codes &= (1 << bits) - 1
    assert torch.equal(back, codes)


def test_dequantize_across_launch_pieces(oracle):
    B, H, D, bits, blocks = 1 << 15, 64, 64, 4, (40, 25)
    T = sum(blocks)
    Lg = K.make_layout(B, H, D, bits, blocks)
    assert B * H * T * (D // 8) > PIECE_CHUNKS
    cache = K.alloc_cache(Lg)
    cache["codes"].copy_(_rand_u8(tuple(cache["codes"].shape), 3))
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    zero = (torch.rand(tuple(cache["zero"].shape), generator=g, device=DEV) * 8 - 4).half()
    step = (torch.rand(tuple(cache["scale"].shape), generator=g, device=DEV) * 0.5).half()
    cache["zero"].copy_(zero.view(cache["zero"].dtype))
    cache["scale"].copy_(step.view(cache["scale"].dtype))
    del zero, step
    out = torch.empty((B, H, T, D), dtype=torch.float32, device=DEV)
    K.kvq_dequantize(Lg, len(blocks), cache, out)
    torch.cuda.synchronize()
    # (b, h) pairs whose rows hold the first launch boundary, plus a sample
    edge_bh = (PIECE_CHUNKS // (D // 8)) // T
    rng = np.random.default_rng(9)
    bhs = sorted({edge_bh - 1, edge_bh, edge_bh + 1, 0, B * H - 1} |
                 set(int(x) for x in rng.integers(0, B * H, 60)))
    sel = torch.tensor(bhs, dtype=torch.int64, device=DEV)
    Ls = oracle.make_layout(len(bhs), 1, D, bits, blocks)
    sub = {}
    for key, t in cache.items():
        part = t.view(B * H, *t.shape[2:]).index_select(0, sel).unsqueeze(1)
        if key != "codes":
            part = part.view(torch.int16)
        sub[key] = np.ascontiguousarray(part.cpu().numpy().view(np.uint8 if key == "codes"
                                                                else np.uint16))
    ref = oracle.dequantize(Ls, len(blocks), sub)
    got = out.view(B * H, T, D).index_select(0, sel).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref[:, 0].view(np.uint32))
