"""ctypes binding of the CPU oracle (oracle/liboracle.so) on numpy arrays.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg.  Argument marshalling only; every step of the
arithmetic is in kvq_oracle.c.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# KVQR_ORACLE_LIB names another build of the same source (the sanitizer build)
LIB_PATH = os.environ.get("KVQR_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

MAX_BLOCKS = 64
OK, E_INVAL = 0, -1
S_NONFINITE, S_RANGE = 1, 2
F32, BF16 = 0, 1


class Layout(C.Structure):
    _fields_ = [
        ("batch", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32),
        ("bits", C.c_int32), ("n_blocks", C.c_int32), ("pack_mode", C.c_int32),
        ("block_tokens", C.c_int32 * MAX_BLOCKS),
    ]


class Cache(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("zero", C.c_void_p), ("scale", C.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b  # noqa: F401
            _b.build()
        L = C.CDLL(LIB_PATH)
        L.kvqr_h2f.restype = C.c_float
        L.kvqr_h2f.argtypes = [C.c_uint16]
        L.kvqr_rd16.restype = C.c_uint16
        L.kvqr_rd16.argtypes = [C.c_float]
        L.kvqr_ru16.restype = C.c_uint16
        L.kvqr_ru16.argtypes = [C.c_float]
        for f in (L.kvqr_rd16_n, L.kvqr_ru16_n):
            f.restype = None
            f.argtypes = [C.c_void_p, C.c_int64, C.c_void_p]
        L.kvqr_row_bytes.restype = C.c_int32
        L.kvqr_row_bytes.argtypes = [C.c_int32, C.c_int32]
        L.kvqr_codes_per_word.restype = C.c_int32
        L.kvqr_codes_per_word.argtypes = [C.c_int32]
        L.kvqr_stream_words.restype = C.c_int64
        L.kvqr_stream_words.argtypes = [C.c_int32, C.c_int64]
        L.kvqr_block_word_offset.restype = C.c_int64
        L.kvqr_block_word_offset.argtypes = [C.POINTER(Layout), C.c_int32]
        L.kvqr_quantize_group.restype = C.c_int
        L.kvqr_quantize_group.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_int32,
                                          C.c_void_p, C.c_void_p, C.c_void_p]
        L.kvqr_quantize_block.restype = C.c_int
        L.kvqr_quantize_block.argtypes = [C.POINTER(Layout), C.c_int32, C.c_int32, C.c_void_p,
                                          C.c_void_p, Cache, Cache]
        L.kvqr_pack.restype = C.c_int
        L.kvqr_pack.argtypes = [C.c_int32, C.c_int32, C.c_void_p, C.c_int64, C.c_int32,
                                C.c_void_p, C.c_int64]
        L.kvqr_unpack.restype = C.c_int
        L.kvqr_unpack.argtypes = [C.c_int32, C.c_int32, C.c_void_p, C.c_int64, C.c_int64,
                                  C.c_int32, C.c_void_p]
        L.kvqr_dequantize.restype = C.c_int
        L.kvqr_dequantize.argtypes = [C.POINTER(Layout), C.c_int32, Cache, C.c_void_p]
        L.kvqr_attend.restype = C.c_int
        L.kvqr_attend.argtypes = [C.POINTER(Layout), C.c_int32, C.c_void_p, Cache, Cache,
                                  C.c_double, C.c_void_p, C.c_int32, C.c_int32]
        L.kvqr_attend_row.restype = C.c_int
        L.kvqr_attend_row.argtypes = [C.POINTER(Layout), C.c_int32, C.c_void_p, Cache, Cache,
                                      C.c_double, C.c_int32, C.c_int32, C.c_int32, C.c_void_p]
        L.kvqr_bytes.restype = C.c_int
        L.kvqr_bytes.argtypes = [C.POINTER(Layout), C.c_int32, C.POINTER(C.c_uint64),
                                 C.POINTER(C.c_uint64)]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


def make_layout(batch: int, heads: int, head_dim: int, bits: int,
                blocks: Sequence[int], pack_mode: int = 0) -> Layout:
    L = Layout()
    L.batch, L.heads, L.head_dim, L.bits = batch, heads, head_dim, bits
    L.n_blocks, L.pack_mode = len(blocks), pack_mode
    for i, n in enumerate(blocks):
        L.block_tokens[i] = n
    return L


def layout_of(wl, batch=None) -> Layout:
    return make_layout(wl.batch if batch is None else batch, wl.heads, wl.head_dim, wl.bits,
                       wl.blocks)


def row_bytes(bits: int, head_dim: int) -> int:
    return int(lib().kvqr_row_bytes(bits, head_dim))


def h2f(h: np.ndarray) -> np.ndarray:
    f = np.vectorize(lambda v: lib().kvqr_h2f(int(v)), otypes=[np.float32])
    return f(np.asarray(h, dtype=np.uint16))


def rd16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().kvqr_rd16_n(_p(x), x.size, _p(out))
    return out


def ru16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().kvqr_ru16_n(_p(x), x.size, _p(out))
    return out


def quantize_group(x: np.ndarray, bits: int):
    """-> (status, zero_bits, scale_bits, codes[n])"""
    x = np.ascontiguousarray(x, dtype=np.float32)
    z = np.zeros(1, np.uint16)
    s = np.zeros(1, np.uint16)
    codes = np.zeros(max(1, x.size), np.uint8)
    st = lib().kvqr_quantize_group(_p(x), x.size, 1, bits, _p(z), _p(s), _p(codes))
    return int(st), int(z[0]), int(s[0]), codes[: x.size]


def block_word_offset(L: Layout, block: int) -> int:
    return int(lib().kvqr_block_word_offset(C.byref(L), block))


def alloc_cache(L: Layout) -> Dict[str, np.ndarray]:
    T = int(sum(L.block_tokens[i] for i in range(L.n_blocks)))
    if L.pack_mode == 2:  # [B][H] word streams, one per block, 4 bytes a word
        codes = np.zeros((L.batch, L.heads, 4 * block_word_offset(L, L.n_blocks)), np.uint8)
    else:
        codes = np.zeros((L.batch, L.heads, T, row_bytes(L.bits, L.head_dim)), np.uint8)
    return {
        "codes": codes,
        "zero": np.zeros((L.batch, L.heads, L.n_blocks, L.head_dim), np.uint16),
        "scale": np.zeros((L.batch, L.heads, L.n_blocks, L.head_dim), np.uint16),
    }


def _cache(c: Dict[str, np.ndarray]) -> Cache:
    return Cache(_p(c["codes"]).value, _p(c["zero"]).value, _p(c["scale"]).value)


def quantize_block(L: Layout, block: int, k_src: np.ndarray, v_src: np.ndarray,
                   k_cache, v_cache) -> int:
    dt = F32 if k_src.dtype == np.float32 else BF16
    assert k_src.dtype == v_src.dtype and k_src.dtype in (np.float32, np.uint16)
    k_src = np.ascontiguousarray(k_src)
    v_src = np.ascontiguousarray(v_src)
    return int(lib().kvqr_quantize_block(C.byref(L), block, dt, _p(k_src), _p(v_src),
                                         _cache(k_cache), _cache(v_cache)))


def pack(bits: int, codes: np.ndarray, dst_row_stride: int = 0, pack_mode: int = 0):
    """pack_mode 0: rows [n_rows, stride]; pack_mode 1: one word-aligned stream (bytes)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    n_rows, row_len = codes.shape
    if pack_mode == 1:
        dst = np.zeros(4 * stream_words(bits, n_rows * row_len), np.uint8)
        st = lib().kvqr_pack(bits, 1, _p(codes), n_rows, row_len, _p(dst), 0)
    else:
        R = row_bytes(bits, row_len)
        stride = dst_row_stride or R
        dst = np.zeros((n_rows, stride), np.uint8)
        st = lib().kvqr_pack(bits, pack_mode, _p(codes), n_rows, row_len, _p(dst), stride)
    if st != OK:
        raise ValueError(f"kvqr_pack: {st}")
    return dst


def unpack(bits: int, packed: np.ndarray, row_len: int, pack_mode: int = 0, n_rows: int = None):
    """pack_mode 0: packed [n_rows, stride]; pack_mode 1: a stream of n_rows * row_len codes."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    if pack_mode == 1:
        codes = np.zeros((n_rows, row_len), np.uint8)
        st = lib().kvqr_unpack(bits, 1, _p(packed), 0, n_rows, row_len, _p(codes))
    else:
        n_rows, stride = packed.shape
        codes = np.zeros((n_rows, row_len), np.uint8)
        st = lib().kvqr_unpack(bits, pack_mode, _p(packed), stride, n_rows, row_len, _p(codes))
    if st != OK:
        raise ValueError(f"kvqr_unpack: {st}")
    return codes


def codes_per_word(bits: int) -> int:
    return int(lib().kvqr_codes_per_word(bits))


def stream_words(bits: int, n_codes: int) -> int:
    return int(lib().kvqr_stream_words(bits, n_codes))


def dequantize(L: Layout, n_filled: int, cache) -> np.ndarray:
    T = int(sum(L.block_tokens[i] for i in range(n_filled)))
    out = np.zeros((L.batch, L.heads, T, L.head_dim), np.float32)
    st = lib().kvqr_dequantize(C.byref(L), n_filled, _cache(cache), _p(out))
    if st != OK:
        raise ValueError(f"kvqr_dequantize: {st}")
    return out


def attend(L: Layout, block: int, q: np.ndarray, k_cache, v_cache, scale: float = 0.0,
           b0: int = 0, b1: int = -1, out: np.ndarray = None) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint16)
    if b1 < 0:
        b1 = L.batch
    if out is None:
        out = np.zeros(q.shape, np.float32)
    st = lib().kvqr_attend(C.byref(L), block, _p(q), _cache(k_cache), _cache(v_cache),
                           float(scale), _p(out), b0, b1)
    if st != OK:
        raise ValueError(f"kvqr_attend: {st}")
    return out


def attend_row(L: Layout, block: int, q: np.ndarray, k_cache, v_cache, b: int, i: int, h: int,
               scale: float = 0.0) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint16)
    o = np.zeros(L.head_dim, np.float64)
    st = lib().kvqr_attend_row(C.byref(L), block, _p(q), _cache(k_cache), _cache(v_cache),
                               float(scale), b, i, h, _p(o))
    if st != OK:
        raise ValueError(f"kvqr_attend_row: {st}")
    return o


def nbytes(L: Layout, n_filled: int):
    cb, sb = C.c_uint64(), C.c_uint64()
    st = lib().kvqr_bytes(C.byref(L), n_filled, C.byref(cb), C.byref(sb))
    if st != OK:
        raise ValueError(f"kvqr_bytes: {st}")
    return int(cb.value), int(sb.value)
