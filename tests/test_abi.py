"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/kvq.h declares, rejects bad arguments before touching a
device, and its byte accounting agrees with the oracle's (an independent
implementation pinned to the pages' table)."""
import ctypes as C

import pytest

import varq_inputs as vi
import visual_autoregressive_kv_amd as K
from visual_autoregressive_kv_amd import kvq as kb


def test_library_exports_every_declared_symbol():
    lib = K.lib()
    names = K.header_symbols()
    assert set(names) >= {"kvq_quantize_block", "kvq_pack", "kvq_attend_packed", "kvq_bytes"}
    for n in names:
        assert hasattr(lib, n), n
    assert "gfx950" in K.kvq_version()


@pytest.mark.parametrize("wl", list(vi.WORKLOADS.values()), ids=list(vi.WORKLOADS))
def test_bytes_match_oracle(oracle, wl):
    Lg = K.make_layout(wl.batch, wl.heads, wl.head_dim, wl.bits, wl.blocks)
    Lo = oracle.layout_of(wl)
    for n_filled in range(len(wl.blocks) + 1):
        assert K.kvq_bytes(Lg, n_filled) == oracle.nbytes(Lo, n_filled)


def test_bytes_rejects_bad_input():
    L = K.make_layout(2, 3, 64, 4, (1, 4))
    with pytest.raises(K.KvqError):
        K.kvq_bytes(L, 3)
    with pytest.raises(K.KvqError):
        K.kvq_bytes(K.make_layout(2, 3, 60, 4, (1, 4)), 1)  # head_dim % 8
    with pytest.raises(K.KvqError):
        K.kvq_bytes(K.make_layout(2, 3, 64, 9, (1, 4)), 1)  # bits
    with pytest.raises(K.KvqError):
        K.kvq_bytes(K.make_layout(0, 3, 64, 4, (1, 4)), 1)
    with pytest.raises(K.KvqError):
        K.kvq_bytes(K.make_layout(1, 3, 64, 4, (1, 0)), 1)
    assert K.lib().kvq_bytes(C.byref(L), 1, None, None) == kb.E_INVAL


FAKE = 0x10000  # an aligned address that is never dereferenced: every call below
                # must return before any launch


def _cache(p=FAKE):
    return kb.Cache(p, p, p)


def test_quantize_argument_errors_return_before_launch():
    lib = K.lib()
    L = K.make_layout(2, 3, 64, 4, (1, 4, 9))
    E = kb.E_INVAL
    q = lib.kvq_quantize_block
    assert q(C.byref(L), 3, kb.BF16, FAKE, FAKE, _cache(), _cache(), None, None) == E
    assert q(C.byref(L), -1, kb.BF16, FAKE, FAKE, _cache(), _cache(), None, None) == E
    assert q(C.byref(L), 0, 7, FAKE, FAKE, _cache(), _cache(), None, None) == E
    assert q(C.byref(L), 0, kb.BF16, None, FAKE, _cache(), _cache(), None, None) == E
    assert q(C.byref(L), 0, kb.BF16, FAKE + 8, FAKE, _cache(), _cache(), None, None) == E
    assert q(C.byref(L), 0, kb.BF16, FAKE, FAKE, kb.Cache(FAKE, None, FAKE), _cache(),
             None, None) == E
    assert q(C.byref(L), 0, kb.BF16, FAKE, FAKE, _cache(), _cache(FAKE + 4), None, None) == E
    assert q(C.byref(L), 0, kb.BF16, FAKE, FAKE, _cache(), _cache(), FAKE + 2, None) == E
    assert q(None, 0, kb.BF16, FAKE, FAKE, _cache(), _cache(), None, None) == E
    # valid but not built for the GPU: 5-bit codes, head_dim 32
    L5 = K.make_layout(2, 3, 64, 5, (1, 4, 9))
    assert q(C.byref(L5), 0, kb.BF16, FAKE, FAKE, _cache(), _cache(), None, None) == \
        kb.E_UNSUPPORTED
    L32 = K.make_layout(2, 3, 32, 4, (1, 4, 9))
    assert q(C.byref(L32), 0, kb.BF16, FAKE, FAKE, _cache(), _cache(), None, None) == \
        kb.E_UNSUPPORTED
    # 2^25 (sequence, head) pairs: valid for the byte accounting, too many for one decode call
    Lbig = K.make_layout(1 << 15, 1 << 10, 64, 4, (1, 4, 9))
    assert K.kvq_bytes(Lbig, 3)[0] == (1 << 25) * 14 * 32
    assert q(C.byref(Lbig), 0, kb.BF16, FAKE, FAKE, _cache(), _cache(), None, None) == \
        kb.E_UNSUPPORTED
    assert lib.kvq_attend_packed(C.byref(Lbig), 0, FAKE, _cache(), _cache(), 0.0, FAKE, None) == \
        kb.E_UNSUPPORTED
    assert lib.kvq_quantize_attend(C.byref(Lbig), 0, kb.BF16, FAKE, FAKE, FAKE, _cache(),
                                   _cache(), 0.0, FAKE, None, None) == kb.E_UNSUPPORTED


def test_attend_and_pack_argument_errors_return_before_launch():
    lib = K.lib()
    L = K.make_layout(2, 3, 64, 3, (1, 4, 9))
    E = kb.E_INVAL
    a = lib.kvq_attend_packed
    assert a(C.byref(L), 3, FAKE, _cache(), _cache(), 0.0, FAKE, None) == E
    assert a(C.byref(L), 0, None, _cache(), _cache(), 0.0, FAKE, None) == E
    assert a(C.byref(L), 0, FAKE, _cache(), _cache(), 0.0, FAKE + 4, None) == E
    assert a(C.byref(L), 0, FAKE, _cache(), _cache(), float("nan"), FAKE, None) == E
    assert a(C.byref(L), 0, FAKE, _cache(), _cache(), float("inf"), FAKE, None) == E
    p = lib.kvq_pack
    assert p(0, 0, FAKE, 4, 64, FAKE, 32, None) == E      # bits
    assert p(9, 0, FAKE, 4, 64, FAKE, 72, None) == E
    assert p(4, 1, FAKE, 4, 64, FAKE, 32, None) == E      # pack_mode
    assert p(4, 0, FAKE, 4, 64, FAKE, 31, None) == E      # stride < row bytes
    assert p(3, 0, FAKE, 4, 64, FAKE, 23, None) == E
    assert p(4, 0, FAKE, -1, 64, FAKE, 32, None) == E
    assert p(4, 0, None, 4, 64, FAKE, 32, None) == E
    assert p(4, 0, FAKE, 0, 64, None, 32, None) == kb.OK  # nothing to do
    u = lib.kvq_unpack
    assert u(4, 0, FAKE, 31, 4, 64, FAKE, None) == E
    assert lib.kvq_stream_copy(FAKE, FAKE, 15, None) == E
    assert lib.kvq_stream_copy(FAKE, FAKE, 0, None) == kb.OK


def test_attend_split_argument_errors_return_before_launch():
    lib = K.lib()
    L = K.make_layout(1, 40, 128, 3, (1560, 1560))
    E = kb.E_INVAL
    need = C.c_uint64()
    assert lib.kvq_attend_split_workspace(C.byref(L), 1, 8, C.byref(need)) == kb.OK
    assert need.value == 8 * 1560 * 40 * (128 + 2) * 4
    assert lib.kvq_attend_split_workspace(C.byref(L), 2, 8, C.byref(need)) == E  # block
    assert lib.kvq_attend_split_workspace(C.byref(L), 1, 0, C.byref(need)) == E
    assert lib.kvq_attend_split_workspace(C.byref(L), 1, 65, C.byref(need)) == E
    assert lib.kvq_attend_split_workspace(C.byref(L), 1, 8, None) == E
    n = need.value
    f = lib.kvq_attend_packed_split

    def call(block=1, ms=8, ws=FAKE, nb=n, layout=L):
        return f(C.byref(layout), block, FAKE, _cache(), _cache(), 0.0, FAKE, ms, ws, nb, None)

    assert call(block=2) == E
    assert call(ms=0) == E
    assert call(ms=65) == E
    assert call(ws=None) == E
    assert call(ws=FAKE + 8) == E       # workspace alignment
    assert call(nb=n - 1) == E          # workspace too small
    assert call(layout=K.make_layout(1, 40, 128, 5, (1560, 1560))) == kb.E_UNSUPPORTED


def test_layout_limits():
    lib = K.lib()
    L = K.make_layout(2, 3, 64, 4, (1,) * 64)
    cb, sb = K.kvq_bytes(L, 64)
    assert cb == 2 * 3 * 64 * 32 and sb == 2 * 3 * 64 * 64 * 4
    L.n_blocks = 65
    assert lib.kvq_bytes(C.byref(L), 1, C.byref(C.c_uint64()), C.byref(C.c_uint64())) == \
        kb.E_INVAL


def test_quantize_attend_argument_errors_return_before_launch():
    lib = K.lib()
    L = K.make_layout(2, 3, 64, 4, (1, 4, 9))
    E = kb.E_INVAL
    f = lib.kvq_quantize_attend
    ok = (kb.BF16, FAKE, FAKE, FAKE, _cache(), _cache(), 0.0, FAKE, None, None)
    assert f(C.byref(L), 3, *ok) == E                        # block
    assert f(C.byref(L), 0, 7, *ok[1:]) == E                 # dtype
    assert f(C.byref(L), 0, kb.BF16, None, *ok[2:]) == E     # k_src
    assert f(C.byref(L), 0, kb.BF16, FAKE, FAKE, None, *ok[4:]) == E          # q
    assert f(C.byref(L), 0, kb.BF16, FAKE, FAKE, FAKE + 2, *ok[4:]) == E      # q alignment
    assert f(C.byref(L), 0, kb.BF16, FAKE, FAKE, FAKE, _cache(FAKE + 4), _cache(), 0.0, FAKE,
             None, None) == E
    assert f(C.byref(L), 0, kb.BF16, FAKE, FAKE, FAKE, _cache(), _cache(), float("nan"), FAKE,
             None, None) == E
    assert f(C.byref(L), 0, kb.BF16, FAKE, FAKE, FAKE, _cache(), _cache(), 0.0, None, None,
             None) == E
    assert f(C.byref(L), 0, kb.BF16, FAKE, FAKE, FAKE, _cache(), _cache(), 0.0, FAKE, FAKE + 2,
             None) == E
    L5 = K.make_layout(2, 3, 64, 5, (1, 4, 9))
    assert f(C.byref(L5), 0, *ok) == kb.E_UNSUPPORTED


def test_word_aligned_mode_bytes_and_errors(oracle):
    """pack_mode 1: byte accounting agrees with the oracle, the stream packer
    rejects a row stride, and the decode calls report it unsupported."""
    lib = K.lib()
    for bits in (2, 3, 5, 8):
        Lg = K.make_layout(3, 5, 64, bits, vi.VAR_BLOCKS, pack_mode=1)
        Lo = oracle.make_layout(3, 5, 64, bits, vi.VAR_BLOCKS, pack_mode=1)
        for n_filled in (0, 1, 7, 10):
            assert K.kvq_bytes(Lg, n_filled) == oracle.nbytes(Lo, n_filled)
    E = kb.E_INVAL
    assert lib.kvq_pack(3, 1, FAKE, 4, 64, FAKE, 32, None) == E   # stream: stride must be 0
    assert lib.kvq_unpack(3, 1, FAKE, 24, 4, 64, FAKE, None) == E
    assert lib.kvq_pack(3, 2, FAKE, 4, 64, FAKE, 0, None) == E    # no pack_mode 2
    assert lib.kvq_pack(3, 1, FAKE, 0, 64, None, 0, None) == kb.OK  # nothing to do
    L = K.make_layout(2, 3, 64, 3, (1, 4, 9), pack_mode=1)
    U = kb.E_UNSUPPORTED
    assert lib.kvq_quantize_block(C.byref(L), 0, kb.BF16, FAKE, FAKE, _cache(), _cache(), None,
                                  None) == U
    assert lib.kvq_attend_packed(C.byref(L), 0, FAKE, _cache(), _cache(), 0.0, FAKE, None) == U
    assert lib.kvq_quantize_attend(C.byref(L), 0, kb.BF16, FAKE, FAKE, FAKE, _cache(), _cache(),
                                   0.0, FAKE, None, None) == U
    L.pack_mode = 3
    with pytest.raises(K.KvqError):
        K.kvq_bytes(L, 1)


def test_block_words_bytes_and_errors(oracle):
    """pack_mode 2 (block-aligned words): byte accounting agrees with the oracle
    at every width, the decode calls accept it where the kernels are built and
    reject what they are not built for (no GPU call is made: every rejected
    case fails in host validation)."""
    lib = K.lib()
    for bits in (1, 2, 3, 5, 7, 8):
        for d in (64, 128, 24):
            Lg = K.make_layout(3, 5, d, bits, vi.VAR_BLOCKS, pack_mode=2)
            Lo = oracle.make_layout(3, 5, d, bits, vi.VAR_BLOCKS, pack_mode=2)
            for n_filled in (0, 1, 7, 10):
                assert K.kvq_bytes(Lg, n_filled) == oracle.nbytes(Lo, n_filled)
    U = kb.E_UNSUPPORTED
    L = K.make_layout(2, 3, 64, 5, (1, 4, 9), pack_mode=2)  # 5-bit codes: not built
    assert lib.kvq_quantize_block(C.byref(L), 0, kb.BF16, FAKE, FAKE, _cache(), _cache(), None,
                                  None) == U
    assert lib.kvq_attend_packed(C.byref(L), 0, FAKE, _cache(), _cache(), 0.0, FAKE, None) == U
    L = K.make_layout(2, 3, 64, 3, (1, 4, 9), pack_mode=2)
    assert lib.kvq_attend_packed(C.byref(L), 0, FAKE, _cache(), _cache(), float("nan"), FAKE,
                                 None) == kb.E_INVAL
