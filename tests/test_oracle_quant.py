"""Pins of the oracle quantizer (one (block, channel) group) and dequantizer.

Nothing here re-derives the oracle's formula: groups with closed-form answers,
a brute-force nearest-grid-point search in float64, the half-step bound, the
grid-coverage invariants and numpy's own binary16 tables decide.
"""
import numpy as np
import pytest

import varq_inputs as vi


def f16(bits: int) -> float:
    return float(np.array([bits], np.uint16).view(np.float16)[0])


def next_up16(bits: int) -> float:
    v = np.array([bits], np.uint16).view(np.float16)[0]
    return float(np.nextafter(v, np.float16(np.inf)))


def next_down16(bits: int) -> float:
    v = np.array([bits], np.uint16).view(np.float16)[0]
    return float(np.nextafter(v, np.float16(-np.inf)))


@pytest.mark.parametrize("bits", [4, 3])
def test_identity_grid(oracle, bits):
    L = (1 << bits) - 1
    x = np.arange(L + 1, dtype=np.float32)
    st, z, s, codes = oracle.quantize_group(x, bits)
    assert st == 0
    assert f16(z) == 0.0 and z == 0x0000
    assert f16(s) == 1.0
    assert np.array_equal(codes, np.arange(L + 1))


def test_identity_grid_shuffled_and_shifted(oracle):
    x = np.array([3, 15, 0, 7, 7, 1, 14], np.float32) + 100.0
    st, z, s, codes = oracle.quantize_group(x, 4)
    assert st == 0 and f16(z) == 100.0 and f16(s) == 1.0
    assert np.array_equal(codes, [3, 15, 0, 7, 7, 1, 14])


def test_constant_group_is_lossless(oracle):
    for v in [0.0, 1.5, -3.25, 60.0, -2.0 ** -20]:
        x = np.full(9, v, np.float32)
        st, z, s, codes = oracle.quantize_group(x, 4)
        assert st == 0
        assert f16(s) == 0.0 and s == 0x0000
        assert np.all(codes == 0)
        if np.float16(v) == v:
            assert f16(z) == v


def test_single_token_block(oracle):
    # a binary16-representable value (every bf16 value in the fp16 normal range
    # is one) is stored exactly: z = x, s = 0
    st, z, s, codes = oracle.quantize_group(np.array([0.6875], np.float32), 3)
    assert st == 0 and codes[0] == 0 and f16(z) == 0.6875 and s == 0
    # 0.7 is not: z is the largest binary16 below it, the grid's top level
    # z + 7 s reaches it, and the code picks that top level
    x = np.float32(0.7)
    st, z, s, codes = oracle.quantize_group(np.array([x], np.float32), 3)
    assert st == 0
    assert f16(z) <= x < next_up16(z)
    assert f16(s) > 0 and codes[0] == 7
    assert abs(float(x) - (f16(z) + 7 * f16(s))) <= f16(s) / 2


@pytest.mark.parametrize("bits", [4, 3])
def test_two_point_group(oracle, bits):
    L = (1 << bits) - 1
    st, z, s, codes = oracle.quantize_group(np.array([-1.0, 1.0, -1.0], np.float32), bits)
    assert st == 0
    assert f16(z) == -1.0
    q = np.float32(2.0) / np.float32(L)
    assert next_down16(s) < q <= f16(s)  # smallest binary16 >= fp32(2/L)
    assert list(codes) == [0, L, 0]


def test_signed_zero_is_canonical(oracle):
    st, z, s, codes = oracle.quantize_group(np.array([-0.0, -0.0], np.float32), 4)
    assert st == 0 and z == 0x0000 and s == 0x0000
    st, z, s, codes = oracle.quantize_group(np.array([-0.0, 0.0, 2.0], np.float32), 4)
    assert z == 0x0000


def test_status_codes(oracle):
    S_NONFINITE, S_RANGE = oracle.S_NONFINITE, oracle.S_RANGE
    assert oracle.quantize_group(np.array([1, np.nan], np.float32), 4)[0] == S_NONFINITE
    assert oracle.quantize_group(np.array([1, np.inf], np.float32), 4)[0] == S_NONFINITE
    assert oracle.quantize_group(np.array([1, -np.inf], np.float32), 4)[0] == S_NONFINITE
    assert oracle.quantize_group(np.array([1, 70000.0], np.float32), 4)[0] == S_RANGE
    assert oracle.quantize_group(np.array([-70000.0, 1], np.float32), 3)[0] == S_RANGE
    assert oracle.quantize_group(np.array([-65504.0, 65504.0], np.float32), 4)[0] == 0


def _groups(rng, n_groups=3000):
    """Tiny random groups: gaussian, outlier-shifted, wide, tiny-magnitude, ties."""
    out = []
    for i in range(n_groups):
        n = int(rng.integers(1, 24))
        kind = i % 6
        if kind == 0:
            x = rng.standard_normal(n)
        elif kind == 1:
            x = rng.standard_normal(n) + rng.uniform(-60, 60)
        elif kind == 2:
            x = rng.uniform(-3000, 3000, n)
        elif kind == 3:
            x = rng.standard_normal(n) * 1e-5
        elif kind == 4:
            x = rng.integers(-8, 8, n) * 0.5  # exact grid values, many ties
        else:
            x = vi.bf16_bits_to_f32(vi.f32_to_bf16_bits(
                (rng.standard_normal(n) * 4 + 20).astype(np.float32)))
        out.append(np.asarray(x, np.float32))
    return out


@pytest.mark.parametrize("bits", [4, 3, 2, 8])
def test_grid_invariants_and_brute_force_argmin(oracle, bits):
    rng = np.random.default_rng(1234 + bits)
    L = (1 << bits) - 1
    for x in _groups(rng):
        st, zb, sb, codes = oracle.quantize_group(x, bits)
        assert st == 0
        z, s = f16(zb), f16(sb)
        mn, mx = float(x.min()), float(x.max())
        # zero: largest binary16 <= min
        assert z <= mn < next_up16(zb) or (mn == 0 and z == 0)
        # grid covers the group: z + L*s >= max; the step is the smallest binary16
        # at or above the binary32 quotient
        assert z + L * s >= mx
        q = np.float32(np.float32(mx if mx != 0 else 0.0) - np.float32(z)) / np.float32(L)
        if s > 0:
            assert next_down16(sb) < q <= s
        else:
            assert q == 0
        grid = z + s * np.arange(L + 1, dtype=np.float64)
        for xi, c in zip(x.astype(np.float64), codes.astype(int)):
            assert 0 <= c <= L
            d = np.abs(xi - grid)
            best = d.min()
            # nearest grid point; ties and last-ulp products may pick the neighbour
            tol = 2.0 ** -21 * max(abs(xi), abs(z) + L * s) + 1e-300
            assert d[c] <= best + tol, (x, xi, c, d)
            # half-step bound on the dequantized value
            xh = np.float32(np.float64(c) * s + z)  # fmaf(code, s, z): one rounding
            assert abs(xi - float(xh)) <= s / 2 + tol * 2


def test_dequantize_is_one_fma(oracle):
    """x_hat = RN32(code * s + z): checked against exact float64 arithmetic."""
    wl = vi.WORKLOADS["var256_tiny_int4"].with_(heads=2)
    L = oracle.layout_of(wl)
    kc, vc = oracle.alloc_cache(L), oracle.alloc_cache(L)
    for k in range(len(wl.blocks)):
        assert oracle.quantize_block(L, k, vi.kv_block(wl, 0, "k", k),
                                     vi.kv_block(wl, 0, "v", k), kc, vc) == 0
    deq = oracle.dequantize(L, len(wl.blocks), kc)
    codes = oracle.unpack(4, kc["codes"].reshape(-1, 32), 64).reshape(1, 2, 680, 64)
    blk = np.concatenate([np.full(n, i) for i, n in enumerate(wl.blocks)])
    z = kc["zero"].view(np.float16).astype(np.float64)[:, :, blk, :]
    s = kc["scale"].view(np.float16).astype(np.float64)[:, :, blk, :]
    ref = (codes.astype(np.float64) * s + z).astype(np.float32)
    assert np.array_equal(deq, ref)


def test_quantize_block_matches_groupwise(oracle):
    """The block call is the group quantizer applied to every (b, h, d) column and
    packed row by row; checked with the group call and the pack call directly."""
    wl = vi.WORKLOADS["var_d20_b128_int3_rope"].with_(batch=2, heads=3)
    L = oracle.layout_of(wl)
    kc, vc = oracle.alloc_cache(L), oracle.alloc_cache(L)
    k = 7
    for j in range(k + 1):
        kb = vi.kv_block(wl, 2, "k", j)
        vb = vi.kv_block(wl, 2, "v", j)
        assert oracle.quantize_block(L, j, kb, vb, kc, vc) == 0
    kb = vi.bf16_bits_to_f32(vi.kv_block(wl, 2, "k", k))
    off, n = wl.offset(k), wl.blocks[k]
    for b in range(2):
        for h in range(3):
            tile = np.zeros((n, 64), np.uint8)
            for d in range(64):
                st, z, s, codes = oracle.quantize_group(kb[b, :, h, d], 3)
                assert kc["zero"][b, h, k, d] == z and kc["scale"][b, h, k, d] == s
                tile[:, d] = codes
            assert np.array_equal(kc["codes"][b, h, off:off + n], oracle.pack(3, tile))


def test_edge_groups_top_level_exceeds_binary16(oracle):
    """In-range binary32 groups whose top grid level z + L*s exceeds the binary16
    maximum (the premise of tests/test_gpu_range.py): the statistics are
    binary16, the grid top is not."""
    for bits, vals, top in [(4, [0.0, 65504.0], 65520.0), (4, [-65504.0, 65504.0], 65536.0),
                            (3, [0.0, 65504.0], 65520.0)]:
        st, zb, sb, _ = oracle.quantize_group(np.array(vals, np.float32), bits)
        assert st == 0
        z, s = float(oracle.h2f(np.array([zb]))[0]), float(oracle.h2f(np.array([sb]))[0])
        assert z + ((1 << bits) - 1) * s == top, (bits, vals, z, s)
