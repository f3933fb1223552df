"""Pins of the oracle's binary16 helpers against numpy's binary16 decoder.

kvqr_h2f   -- all 65536 patterns equal numpy float16 -> float64.
kvqr_rd16 / kvqr_ru16 -- exhaustive over all 2^32 binary32 patterns against
the defining property of directed rounding, checked by a C walker
(tests/csrc/half_walk.c) whose expectations come only from numpy's table.
"""
import ctypes as C
import os

import numpy as np
import pytest

from conftest import compile_c_helper

HERE = os.path.dirname(os.path.abspath(__file__))


def half_tables():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    val = bits.view(np.float16).astype(np.float64)
    finite = np.unique(val[np.isfinite(val)])  # ascending, one zero
    ladder = np.concatenate([[-np.inf], finite, [np.inf]])
    up = np.full(65536, np.nan)
    down = np.full(65536, np.nan)
    ok = ~np.isnan(val)
    iu = np.searchsorted(ladder, val[ok], side="right")
    idn = np.searchsorted(ladder, val[ok], side="left") - 1
    up[ok] = np.where(iu < ladder.size, ladder[np.minimum(iu, ladder.size - 1)], np.inf)
    down[ok] = np.where(idn >= 0, ladder[np.maximum(idn, 0)], -np.inf)
    # +inf has no larger value; -inf no smaller one
    up[val == np.inf] = np.inf
    down[val == -np.inf] = -np.inf
    return val, up, down


def test_h2f_all_patterns(oracle):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.lib().kvqr_h2f(int(b)) for b in bits], dtype=np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero is kept
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_rd_ru_special_values(oracle):
    f = np.array([0.0, -0.0, 65504.0, 65505.0, 70000.0, -70000.0, np.inf, -np.inf,
                  2.0 ** -24, 2.0 ** -25, -(2.0 ** -25), 1.0 + 2.0 ** -11],
                 dtype=np.float32)
    rd = oracle.rd16(f)
    ru = oracle.ru16(f)
    assert rd[0] == 0x0000 and ru[0] == 0x0000
    assert rd[1] == 0x8000 and ru[1] == 0x8000
    assert rd[2] == 0x7BFF and ru[2] == 0x7BFF
    assert rd[3] == 0x7BFF and ru[3] == 0x7C00  # above the largest finite: up -> +inf
    assert rd[4] == 0x7BFF and ru[4] == 0x7C00
    assert rd[5] == 0xFC00 and ru[5] == 0xFBFF
    assert rd[6] == 0x7C00 and ru[6] == 0x7C00
    assert rd[7] == 0xFC00 and ru[7] == 0xFC00
    assert rd[8] == 0x0001 and ru[8] == 0x0001  # smallest subnormal exactly
    assert rd[9] == 0x0000 and ru[9] == 0x0001
    assert rd[10] == 0x8001 and ru[10] == 0x8000
    assert rd[11] == 0x3C00 and ru[11] == 0x3C01
    nan = oracle.rd16(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0


@pytest.mark.slow
def test_rd_ru_exhaustive_all_fp32_patterns(oracle, tmp_build_dir):
    so = compile_c_helper(os.path.join(HERE, "csrc", "half_walk.c"), tmp_build_dir)
    w = C.CDLL(so)
    w.walk.restype = C.c_int64
    w.walk.argtypes = [C.c_void_p] * 5 + [C.c_uint64, C.c_uint64, C.c_int, C.POINTER(C.c_uint32)]
    val, up, down = half_tables()
    lib = oracle.lib()
    rd = C.cast(lib.kvqr_rd16_n, C.c_void_p)
    ru = C.cast(lib.kvqr_ru16_n, C.c_void_p)
    first = C.c_uint32(0)
    nthreads = max(1, min(16, os.cpu_count() or 1))
    fails = w.walk(val.ctypes.data, up.ctypes.data, down.ctypes.data, rd, ru, 0, 1 << 32,
                   nthreads, C.byref(first))
    assert fails == 0, f"{fails} patterns fail, first 0x{first.value:08x}"


def test_rd_ru_walker_catches_a_planted_mistake(tmp_build_dir):
    """The walker itself must reject a wrong rounding (round-to-nearest)."""
    so = compile_c_helper(os.path.join(HERE, "csrc", "half_walk.c"), tmp_build_dir)
    w = C.CDLL(so)
    w.walk.restype = C.c_int64
    w.walk.argtypes = [C.c_void_p] * 5 + [C.c_uint64, C.c_uint64, C.c_int, C.POINTER(C.c_uint32)]
    val, up, down = half_tables()

    FN = C.CFUNCTYPE(None, C.POINTER(C.c_float), C.c_int64, C.POINTER(C.c_uint16))

    def nearest(x, n, out):
        xs = np.ctypeslib.as_array(x, (n,))
        o = np.ctypeslib.as_array(out, (n,))
        o[:] = xs.astype(np.float16).view(np.uint16)

    cb = FN(nearest)
    first = C.c_uint32(0)
    # 1.0 .. 1.0 + a few ulps: nearest rounding breaks RD or RU there
    lo = np.array([1.0], np.float32).view(np.uint32)[0]
    fails = w.walk(val.ctypes.data, up.ctypes.data, down.ctypes.data,
                   C.cast(cb, C.c_void_p), C.cast(cb, C.c_void_p), int(lo), int(lo) + 4096, 1,
                   C.byref(first))
    assert fails > 0
