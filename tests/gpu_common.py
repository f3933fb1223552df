"""Shared helpers of the GPU parity tests: feed the same seeded inputs to the
HIP library and to the CPU oracle and bring results back for comparison."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import varq_inputs as vi
import visual_autoregressive_kv_amd as K

DEV = "cuda"
ATTN_TOL = 2e-3  # max|gpu - oracle| / max|oracle|, per call and per (sequence, head)

# (case, per-call error, per-(b,h) error, per-channel error or None) of every
# attention check in this session; conftest.py prints the worst at the end
ERR_LOG = []


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy input (float32, or uint16 bf16 bit patterns) -> device tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def cache_to_host(c):
    return {"codes": c["codes"].cpu().numpy(),
            "zero": c["zero"].view(torch.int16).cpu().numpy().view(np.uint16),
            "scale": c["scale"].view(torch.int16).cpu().numpy().view(np.uint16)}


def layouts(oracle, wl, pack_mode=0):
    """The workload's layout for the library and for the oracle (pack_mode 0:
    dense rows; 2: block-aligned words)."""
    Lo = oracle.layout_of(wl)
    Lo.pack_mode = pack_mode
    return (K.make_layout(wl.batch, wl.heads, wl.head_dim, wl.bits, wl.blocks, pack_mode), Lo)


def fill_both(oracle, wl, layer=0, upto=None, status=None, pack_mode=0):
    """Quantize blocks 0..upto-1 on the GPU and in the oracle."""
    Lg, Lo = layouts(oracle, wl, pack_mode)
    kg, vg = K.alloc_cache(Lg), K.alloc_cache(Lg)
    ko, vo = oracle.alloc_cache(Lo), oracle.alloc_cache(Lo)
    upto = len(wl.blocks) if upto is None else upto
    for j in range(upto):
        kb = vi.kv_block(wl, layer, "k", j)
        vb = vi.kv_block(wl, layer, "v", j)
        assert oracle.quantize_block(Lo, j, kb, vb, ko, vo) == 0
        K.kvq_quantize_block(Lg, j, to_dev(kb), to_dev(vb), kg, vg, status=status)
    torch.cuda.synchronize()
    return Lg, Lo, kg, vg, ko, vo


def oracle_threads() -> int:
    """Host threads for the oracle: this process's cores, capped by OMP_NUM_THREADS
    when the host sets it (the GPU machine's CPU share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    return max(1, min(n, cap) if cap > 0 else n)


def oracle_attend_batch(oracle, Lo, block, q, k_cache, v_cache, scale=0.0):
    """The oracle's whole attention output [B][n][H][D], its (sequence, head) pairs
    split over host threads.  Each pair is handed to the oracle as a sequence of
    its own (batch B*H, one head): the caches' [B][H][...] arrays already have
    that layout, and the queries are transposed to [B*H][n][1][D].  The oracle
    attends every (sequence, head) on its own, so the values are those of one
    call on the original layout; each thread's call writes only its own rows
    (the oracle is single-threaded and releases the interpreter lock)."""
    B, H = Lo.batch, Lo.heads
    blocks = [Lo.block_tokens[i] for i in range(Lo.n_blocks)]
    L1 = oracle.make_layout(B * H, 1, Lo.head_dim, Lo.bits, blocks, Lo.pack_mode)

    def pairs(c):  # [B][H][...] -> [B*H][1][...], same memory
        return {k: np.ascontiguousarray(v).reshape((B * H, 1) + v.shape[2:]) for k, v in c.items()}

    q = np.ascontiguousarray(q, dtype=np.uint16)
    n, D = q.shape[1], q.shape[3]
    q1 = np.ascontiguousarray(q.transpose(0, 2, 1, 3)).reshape(B * H, n, 1, D)
    out1 = np.zeros(q1.shape, np.float32)
    k1, v1 = pairs(k_cache), pairs(v_cache)
    t = min(oracle_threads(), B * H)
    cuts = [B * H * i // t for i in range(t + 1)]
    with ThreadPoolExecutor(t) as ex:
        list(ex.map(lambda i: oracle.attend(L1, block, q1, k1, v1, scale=scale,
                                            b0=cuts[i], b1=cuts[i + 1], out=out1), range(t)))
    return out1.reshape(B, H, n, D).transpose(0, 2, 1, 3).astype(np.float64)


def assert_cache_equal(g, o, what=""):
    gh = cache_to_host(g)
    for key in ("zero", "scale", "codes"):
        a, b = gh[key], o[key]
        if not np.array_equal(a, b):
            idx = np.argwhere(a != b)
            raise AssertionError(f"{what} {key}: {len(idx)} mismatches, first at "
                                 f"{tuple(idx[0])}: gpu {a[tuple(idx[0])]} oracle "
                                 f"{b[tuple(idx[0])]}")


def attn_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max|got - ref| / max|ref| over one call's output [B][n][H][D]."""
    return float(np.abs(got.astype(np.float64) - ref).max() / np.abs(ref).max())


def attn_err_bh(got: np.ndarray, ref: np.ndarray) -> float:
    """The same error normalized within each (sequence, head): the largest over
    (b, h) of max_{i,d}|got - ref| / max_{i,d}|ref| (output [B][n][H][D])."""
    d = np.abs(got.astype(np.float64) - ref).max(axis=(1, 3))
    m = np.abs(ref).max(axis=(1, 3))
    return float((d / np.maximum(m, np.finfo(np.float64).tiny)).max())


def attn_err_channel(got: np.ndarray, ref: np.ndarray) -> float:
    """Normalized within each (sequence, head, channel): max over (b, h, d) of
    max_i|got - ref| / max_i|ref|.  It sees the ordinary channels, whose values
    are one to two orders of magnitude below the massive-value channels that
    set the per-(b, h) scale.  Reported, not asserted: the pages fix no bound for it."""
    d = np.abs(got.astype(np.float64) - ref).max(axis=1)
    m = np.abs(ref).max(axis=1)
    return float((d / np.maximum(m, np.finfo(np.float64).tiny)).max())


def check_attn(got: np.ndarray, ref: np.ndarray, what: str = "", tol: float = ATTN_TOL):
    """Assert the 2e-3 bound per call and per (sequence, head); print the per-call,
    per-(b, h) and per-channel errors.  Returns (per call, per (b, h), per channel)."""
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    e, ebh, ech = attn_err(got, ref), attn_err_bh(got, ref), attn_err_channel(got, ref)
    print(f"[attn] {what}: err per call {e:.2e}, per (b,h) {ebh:.2e}, per channel {ech:.2e}",
          flush=True)
    ERR_LOG.append((what, e, ebh, ech))
    assert e <= tol, (what, e)
    assert ebh <= tol, (what, "per (b,h)", ebh)
    return e, ebh, ech
