"""Shared helpers of the GPU parity tests: feed the same seeded inputs to the
HIP library and to the CPU oracle and bring results back for comparison."""
import numpy as np
import torch

import varq_inputs as vi
import visual_autoregressive_kv_amd as K

DEV = "cuda"
ATTN_TOL = 2e-3  # max|gpu - oracle| / max|oracle| per call


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy input (float32, or uint16 bf16 bit patterns) -> device tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def cache_to_host(c):
    return {"codes": c["codes"].cpu().numpy(),
            "zero": c["zero"].view(torch.int16).cpu().numpy().view(np.uint16),
            "scale": c["scale"].view(torch.int16).cpu().numpy().view(np.uint16)}


def layouts(oracle, wl):
    return (K.make_layout(wl.batch, wl.heads, wl.head_dim, wl.bits, wl.blocks),
            oracle.layout_of(wl))


def fill_both(oracle, wl, layer=0, upto=None, status=None):
    """Quantize blocks 0..upto-1 on the GPU and in the oracle."""
    Lg, Lo = layouts(oracle, wl)
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
    return float(np.abs(got.astype(np.float64) - ref).max() / np.abs(ref).max())
