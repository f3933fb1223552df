"""Pins of the oracle's packing, attention and byte accounting.

pack/unpack  hand-worked bytes (tests/golden/pack_examples.txt), exhaustive
             round trips (every INT4 byte, every 8-code INT3 word), the
             bit-position formula evaluated by numpy integer arithmetic;
attend       an independent float64 scipy/numpy softmax attention on the
             dequantized cache, closed forms (one key, identical keys), block
             causality and key-permutation invariance;
bytes        the KV-memory column of the pages' table
             (tests/golden/kv_table.txt).
"""
import os

import numpy as np
import pytest
from scipy.special import softmax

import varq_inputs as vi

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_pack_examples():
    rows = []
    for line in open(os.path.join(GOLDEN, "pack_examples.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        b, codes, hexes = [p.strip() for p in line.split("|")]
        rows.append((int(b), [int(c) for c in codes.split()],
                     bytes(int(h, 16) for h in hexes.split())))
    return rows


@pytest.mark.parametrize("bits,codes,expect", read_pack_examples())
def test_pack_worked_examples(oracle, bits, codes, expect):
    got = oracle.pack(bits, np.array([codes], np.uint8))[0]
    assert bytes(got) == expect
    assert list(oracle.unpack(bits, got[None], len(codes))[0]) == codes


def test_int4_every_byte_round_trips(oracle):
    b = np.arange(256, dtype=np.uint8)[:, None]
    codes = oracle.unpack(4, b, 2)
    assert np.array_equal(codes[:, 0], b[:, 0] & 15) and np.array_equal(codes[:, 1], b[:, 0] >> 4)
    assert np.array_equal(oracle.pack(4, codes), b)


def test_int3_every_word_round_trips(oracle):
    """All 8^8 eight-code words: pack, compare with the integer formula, unpack."""
    w = np.arange(1 << 24, dtype=np.uint32)
    codes = np.stack([(w >> (3 * i)) & 7 for i in range(8)], axis=1).astype(np.uint8)
    packed = oracle.pack(3, codes)
    expect = np.stack([w & 255, (w >> 8) & 255, (w >> 16) & 255], axis=1).astype(np.uint8)
    assert np.array_equal(packed, expect)
    assert np.array_equal(oracle.unpack(3, packed, 8), codes)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
def test_generic_widths_round_trip_and_bit_positions(oracle, bits):
    rng = np.random.default_rng(bits)
    for row_len in [1, 7, 8, 13, 64, 128]:
        codes = rng.integers(0, 1 << bits, (17, row_len), dtype=np.uint8)
        packed = oracle.pack(bits, codes)
        assert packed.shape[1] == (bits * row_len + 7) // 8
        # bit j of the row stream is bit j%8 of byte j//8; code d sits at [bits*d, ...)
        stream = np.unpackbits(packed, axis=1, bitorder="little")
        for d in range(row_len):
            val = np.zeros(17, np.int64)
            for j in range(bits):
                val |= stream[:, bits * d + j].astype(np.int64) << j
            assert np.array_equal(val, codes[:, d])
        # padding bits of the last byte are zero
        assert not stream[:, bits * row_len:].any()
        assert np.array_equal(oracle.unpack(bits, packed, row_len), codes)


def test_pack_row_stride_and_masking(oracle):
    codes = np.array([[17, 2, 255, 4]], np.uint8)  # high bits beyond the width are ignored
    got = oracle.pack(4, codes, dst_row_stride=5)
    assert bytes(got[0][:2]) == bytes([0x21, 0x4F])
    assert not got[0][2:].any()  # bytes past the row are left alone


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _filled(oracle, wl, layer=0, upto=None):
    L = oracle.layout_of(wl)
    kc, vc = oracle.alloc_cache(L), oracle.alloc_cache(L)
    upto = len(wl.blocks) if upto is None else upto
    for j in range(upto):
        st = oracle.quantize_block(L, j, vi.kv_block(wl, layer, "k", j),
                                   vi.kv_block(wl, layer, "v", j), kc, vc)
        assert st == 0
    return L, kc, vc


def _numpy_attention(q_bits, kh, vh, scale):
    q = vi.bf16_bits_to_f32(q_bits).astype(np.float64)  # [B][n][H][D]
    out = np.zeros(q.shape)
    for b in range(q.shape[0]):
        for h in range(q.shape[2]):
            s = scale * q[b, :, h, :] @ kh[b, h].astype(np.float64).T
            out[b, :, h, :] = softmax(s, axis=1) @ vh[b, h].astype(np.float64)
    return out


@pytest.mark.parametrize("block", [0, 3, 9])
def test_attend_matches_library_softmax(oracle, block):
    wl = vi.WORKLOADS["var256_tiny_int4"].with_(heads=4)
    L, kc, vc = _filled(oracle, wl, upto=block + 1)
    q = vi.q_block(wl, 0, block)
    got = oracle.attend(L, block, q, kc, vc)
    T = wl.offset(block) + wl.blocks[block]
    kh = oracle.dequantize(L, block + 1, kc)
    vh = oracle.dequantize(L, block + 1, vc)
    ref = _numpy_attention(q, kh[:, :, :T], vh[:, :, :T], 1 / 8.0)
    assert np.allclose(got, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())
    # single rows in binary64
    for (b, i, h) in [(0, 0, 0), (0, wl.blocks[block] - 1, 3)]:
        row = oracle.attend_row(L, block, q, kc, vc, b, i, h)
        assert np.allclose(row, ref[b, i, h], rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_attend_single_key_is_that_value(oracle):
    wl = vi.WORKLOADS["var256_tiny_int4"].with_(heads=3)
    L, kc, vc = _filled(oracle, wl, upto=1)
    q = vi.q_block(wl, 0, 0)
    got = oracle.attend(L, 0, q, kc, vc)
    vh = oracle.dequantize(L, 1, vc)
    assert np.array_equal(got[0, 0], vh[0, :, 0, :])


def test_attend_identical_keys_average_values(oracle):
    wl = vi.WORKLOADS["var256_tiny_int4"].with_(heads=2)
    L, kc, vc = _filled(oracle, wl, upto=4)
    # overwrite K: every row the same packed bytes and every block the same stats
    kc["codes"][:] = kc["codes"][:, :, :1, :]
    kc["zero"][:] = kc["zero"][:, :, :1, :]
    kc["scale"][:] = kc["scale"][:, :, :1, :]
    q = vi.q_block(wl, 0, 3)
    got = oracle.attend(L, 3, q, kc, vc).astype(np.float64)
    T = wl.offset(3) + wl.blocks[3]
    vh = oracle.dequantize(L, 4, vc).astype(np.float64)[:, :, :T]
    mean = vh.mean(axis=2)  # [B][H][D]
    for i in range(wl.blocks[3]):
        assert np.allclose(got[:, i], mean, rtol=1e-6, atol=1e-6)


def test_attend_is_block_causal(oracle):
    wl = vi.WORKLOADS["var256_tiny_int4"].with_(heads=2)
    L, kc, vc = _filled(oracle, wl)
    q = vi.q_block(wl, 0, 5)
    a = oracle.attend(L, 5, q, kc, vc)
    T = wl.offset(6)
    kc2 = {k: v.copy() for k, v in kc.items()}
    vc2 = {k: v.copy() for k, v in vc.items()}
    kc2["codes"][:, :, T:] ^= 0x5A
    vc2["codes"][:, :, T:] ^= 0xA5
    kc2["zero"][:, :, 6:] = 0x3C00
    vc2["scale"][:, :, 6:] = 0x4000
    b = oracle.attend(L, 5, q, kc2, vc2)
    assert np.array_equal(a, b)
    # ... while a change inside the prefix (block 5 itself) does change it
    vc2["codes"][:, :, T - 1] ^= 0xFF
    c = oracle.attend(L, 5, q, kc2, vc2)
    assert not np.array_equal(a, c)


def test_attend_is_invariant_to_key_order(oracle):
    """Permuting the prefix's tokens (rows + their block stats) leaves O unchanged."""
    blocks = (3, 3, 3)  # equal-size blocks so permuted tokens stay in a block slot
    wl = vi.Workload("perm", 1, 1, 2, 64, 4, blocks, "bf16", seed=99)
    L, kc, vc = _filled(oracle, wl)
    q = vi.q_block(wl, 0, 2)
    a = oracle.attend(L, 2, q, kc, vc).astype(np.float64)
    perm = [2, 0, 1]  # move whole blocks
    kc2 = {k: v.copy() for k, v in kc.items()}
    vc2 = {k: v.copy() for k, v in vc.items()}
    for c2, c in ((kc2, kc), (vc2, vc)):
        for dst, src in enumerate(perm):
            c2["codes"][:, :, 3 * dst:3 * dst + 3] = c["codes"][:, :, 3 * src:3 * src + 3]
            c2["zero"][:, :, dst] = c["zero"][:, :, src]
            c2["scale"][:, :, dst] = c["scale"][:, :, src]
    b = oracle.attend(L, 2, q, kc2, vc2).astype(np.float64)
    assert np.allclose(a, b, rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------------------
# byte accounting vs the pages' table
# ---------------------------------------------------------------------------

def read_kv_table():
    rows = []
    for line in open(os.path.join(GOLDEN, "kv_table.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        m, layers, width, batch, method, prec, kv, saving = line.split()
        rows.append((m, int(layers), int(width), int(batch), method, prec, float(kv),
                     None if saving == "-" else float(saving)))
    return rows


GIB = float(1 << 30)


def _bf16_gib(layers, width, seqs, tokens):
    return 2 * layers * seqs * tokens * width * 2 / GIB  # K and V, 2 bytes each


def test_bytes_reproduce_the_pages_int4_and_bf16_rows(oracle):
    rows = read_kv_table()
    seen = 0
    for m, layers, width, batch, method, prec, kv, saving in rows:
        seqs = 2 * batch  # conditional + unconditional sequence per image (CFG)
        bf16 = _bf16_gib(layers, width, seqs, 680)
        if prec == "BF16":
            assert round(bf16, 2) == kv, (m, bf16)
            seen += 1
        elif prec == "INT4":
            L = oracle.make_layout(seqs, width // 64, 64, 4, vi.VAR_BLOCKS)
            cb, sb = oracle.nbytes(L, 10)
            gib = 2 * layers * (cb + sb) / GIB
            assert round(gib, 2) == kv, (m, gib)
            assert round(100 * (1 - gib / bf16), 2) == saving
            seen += 1
    assert seen == 6


def test_bytes_dense_int3_and_the_tables_int3_rows(oracle):
    """Dense 3-bit rows give 78.31% on the VAR schedule; the table's INT3 rows
    (77.06%, 3.81 / 5.48 / 8.57) are reproduced by the word-aligned layout
    (pack_mode 1, 10 codes per 32-bit word), one stream per (sequence, head)
    that the decode path cannot write a block at a time."""
    seen = 0
    for m, layers, width, batch, method, prec, kv, saving in read_kv_table():
        if prec != "INT3":
            continue
        seqs = 2 * batch
        bf16 = _bf16_gib(layers, width, seqs, 680)
        L = oracle.make_layout(seqs, width // 64, 64, 3, vi.VAR_BLOCKS)
        cb, sb = oracle.nbytes(L, 10)
        dense = 2 * layers * (cb + sb) / GIB
        assert round(100 * (1 - dense / bf16), 2) == 78.31
        assert cb == seqs * (width // 64) * 680 * 24
        Lw = oracle.make_layout(seqs, width // 64, 64, 3, vi.VAR_BLOCKS, pack_mode=1)
        cw, sw = oracle.nbytes(Lw, 10)
        assert sw == sb
        assert cw == seqs * (width // 64) * 4 * ((680 * 64 + 9) // 10)
        gib = 2 * layers * (cw + sw) / GIB
        assert round(gib, 2) == kv, (m, gib)
        assert round(100 * (1 - gib / bf16), 2) == saving
        seen += 1
    assert seen == 3


def read_word_examples():
    out = []
    for line in open(os.path.join(GOLDEN, "pack_words_examples.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        bits, codes, packed = [x.strip() for x in line.split("|")]
        out.append((int(bits), [int(c) for c in codes.split()], bytes.fromhex(packed)))
    return out


@pytest.mark.parametrize("bits,codes,expect", read_word_examples())
def test_word_aligned_pack_worked_examples(oracle, bits, codes, expect):
    c = np.array([codes], np.uint8)
    got = oracle.pack(bits, c, pack_mode=1)
    assert got.tobytes() == expect
    assert np.array_equal(oracle.unpack(bits, got, len(codes), pack_mode=1, n_rows=1), c)


@pytest.mark.parametrize("bits", range(1, 9))
def test_word_aligned_round_trip_and_size(oracle, bits):
    rng = np.random.default_rng(bits)
    for n_rows, row_len in [(1, 1), (3, 7), (5, 64), (17, 128)]:
        codes = rng.integers(0, 1 << bits, size=(n_rows, row_len), dtype=np.uint8)
        packed = oracle.pack(bits, codes, pack_mode=1)
        cpw = 32 // bits
        assert oracle.codes_per_word(bits) == cpw
        assert packed.size == 4 * -(-n_rows * row_len // cpw)
        assert np.array_equal(oracle.unpack(bits, packed, row_len, pack_mode=1, n_rows=n_rows), codes)
        # spare top bits of every word are zero
        words = packed.view("<u4")
        if 32 % bits:
            assert not (words >> (bits * cpw)).any()


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
def test_word_aligned_equals_dense_stream_when_words_fill(oracle, bits):
    """When bits divides 32 the word layout is the dense LSB-first stream."""
    rng = np.random.default_rng(10 + bits)
    codes = rng.integers(0, 1 << bits, size=(4, 96), dtype=np.uint8)
    words = oracle.pack(bits, codes, pack_mode=1)
    dense = oracle.pack(bits, codes.reshape(1, -1))
    assert words.tobytes() == dense.tobytes()


def test_word_aligned_layout_rejected_on_the_decode_path(oracle):
    """One stream per (b, h) cannot take a block at a time: pack_mode 1 is for
    size accounting only; pack_mode 3 does not exist."""
    wl = vi.Workload("w", 1, 1, 2, 64, 3, (4, 9), "bf16", seed=3)
    L = oracle.make_layout(1, 2, 64, 3, (4, 9), pack_mode=1)
    c = oracle.alloc_cache(oracle.make_layout(1, 2, 64, 3, (4, 9)))
    assert oracle.quantize_block(L, 0, vi.kv_block(wl, 0, "k", 0), vi.kv_block(wl, 0, "v", 0),
                                 c, c) == oracle.E_INVAL
    L.pack_mode = 3
    with pytest.raises(Exception):
        oracle.nbytes(L, 1)


def read_block_words_example():
    blocks, packed = {}, None
    for line in open(os.path.join(GOLDEN, "block_words_example.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, val = [x.strip() for x in line.split("|")]
        if key == "packed":
            packed = bytes.fromhex(val)
        else:
            blocks[int(key)] = np.array([[float(v) for v in r.split()] for r in val.split(";")],
                                        np.float32)
    return blocks, packed


def test_block_words_worked_example(oracle):
    """Hand-worked bytes of the block-aligned word layout (two INT3 blocks)."""
    rows, expect = read_block_words_example()
    sizes = tuple(rows[k].shape[0] for k in sorted(rows))
    L = oracle.make_layout(1, 1, 8, 3, sizes, pack_mode=2)
    assert oracle.block_word_offset(L, 1) == 2 and oracle.block_word_offset(L, 2) == 5
    kc, vc = oracle.alloc_cache(L), oracle.alloc_cache(L)
    assert kc["codes"].shape == (1, 1, 20)
    for k in sorted(rows):
        x = rows[k].reshape(1, -1, 1, 8)  # [b][t][h][d]
        assert oracle.quantize_block(L, k, x, 7.0 - x, kc, vc) == oracle.OK
        assert (oracle.h2f(kc["zero"][0, 0, k]) == 0).all()
        assert (oracle.h2f(kc["scale"][0, 0, k]) == 1).all()
    assert kc["codes"].tobytes() == expect
    # V = 7 - K: every code complemented, padding bits still zero
    vwords = vc["codes"].view("<u4").ravel()
    kwords = kc["codes"].view("<u4").ravel()
    live = [(1 << 30) - 1, (1 << 18) - 1, (1 << 30) - 1, (1 << 30) - 1, (1 << 12) - 1]
    assert [int(v) for v in vwords] == [int(k) ^ m for k, m in zip(kwords, live)]
    assert oracle.nbytes(L, 1)[0] == 8 and oracle.nbytes(L, 2)[0] == 20


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
def test_block_words_decode_equal_to_dense_rows(oracle, bits):
    """The layout changes where codes sit, not what they are: dequantized
    caches and attention outputs are identical to dense rows, on ragged blocks
    whose streams end mid-word."""
    blocks = (1, 3, 7, 12)
    wl = vi.Workload("w", 1, 2, 3, 24, bits, blocks, "bf16", seed=40 + bits)
    L0 = oracle.make_layout(2, 3, 24, bits, blocks)
    L2 = oracle.make_layout(2, 3, 24, bits, blocks, pack_mode=2)
    c0 = [oracle.alloc_cache(L0), oracle.alloc_cache(L0)]
    c2 = [oracle.alloc_cache(L2), oracle.alloc_cache(L2)]
    for k in range(len(blocks)):
        ks, vs = vi.kv_block(wl, 0, "k", k), vi.kv_block(wl, 0, "v", k)
        assert oracle.quantize_block(L0, k, ks, vs, *c0) == oracle.OK
        assert oracle.quantize_block(L2, k, ks, vs, *c2) == oracle.OK
        n = k + 1
        for a, b in zip(c0, c2):
            assert np.array_equal(a["zero"], b["zero"]) and np.array_equal(a["scale"], b["scale"])
            assert np.array_equal(oracle.dequantize(L0, n, a), oracle.dequantize(L2, n, b))
        q = vi.q_block(wl, 0, k)
        assert np.array_equal(oracle.attend(L0, k, q, *c0), oracle.attend(L2, k, q, *c2))
        # each block's stream: ceil(n_k D / cpw) words, from a fresh word
        cpw = 32 // bits
        W = [-(-blocks[j] * 24 // cpw) for j in range(len(blocks))]
        assert oracle.block_word_offset(L2, k) == sum(W[:k])
        assert oracle.nbytes(L2, n)[0] == 2 * 3 * 4 * sum(W[:n])


def test_block_words_reproduce_the_tables_int3_rows(oracle):
    """Per-block words at VAR-dN: 4356 words per (sequence, head), four more than
    one stream of all 680 tokens, so 3.81 / 5.49 / 8.58 GiB and a 77.04% saving
    beside the table's 3.81 / 5.48 / 8.57 and 77.06%."""
    seen = 0
    for m, layers, width, batch, method, prec, kv, saving in read_kv_table():
        if prec != "INT3":
            continue
        seqs = 2 * batch
        bf16 = _bf16_gib(layers, width, seqs, 680)
        L = oracle.make_layout(seqs, width // 64, 64, 3, vi.VAR_BLOCKS, pack_mode=2)
        cb, sb = oracle.nbytes(L, 10)
        assert cb == seqs * (width // 64) * 4 * 4356
        gib = 2 * layers * (cb + sb) / GIB
        assert abs(gib - kv) <= 0.011, (m, gib)
        assert round(100 * (1 - gib / bf16), 2) == 77.04
        assert abs(100 * (1 - gib / bf16) - saving) < 0.03
        seen += 1
    assert seen == 3


def test_bytes_formula_pieces(oracle):
    L = oracle.make_layout(3, 5, 128, 3, (4, 9, 1560))
    cb, sb = oracle.nbytes(L, 2)
    assert cb == 3 * 5 * 13 * 48  # ceil(3*128/8) = 48 bytes per row
    assert sb == 3 * 5 * 2 * 128 * 4
    assert oracle.nbytes(L, 0) == (0, 0)
