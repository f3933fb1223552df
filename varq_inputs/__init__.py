"""Seeded synthetic inputs shaped like VAR KV caches.

This module only draws inputs: it holds none of the quantizer, packing or
attention arithmetic, so both the CPU oracle (tests) and the GPU library
(tests, benchmark) can be fed from it without sharing any of the method.

Recipe (the pages give shapes and qualitative structure, no data):
  * schedule: VAR 256px next-scale blocks of s*s tokens for
    s = 1,2,3,4,5,6,8,10,13,16 (680 tokens); next-frame video blocks of
    1560 tokens;
  * per (layer, K or V): a per-channel projection bias mu[h, d] ~ N(0, 2)
    (variance 2) and 4 outlier channels per head with a fixed sign each
    ("projection bias" and "massive-value channels" in the VAR-Q abstract);
  * per (layer, K or V, block, head, outlier channel): a magnitude
    m ~ U[20, 60], shared by the batch -- persistent inside a (block, channel)
    cell and shifting across cells (VAR-Q abstract, second finding);
  * x[b, t, h, d] = N(0, 1) + mu[h, d] + sign * m  (outlier term on the 4
    channels only); queries are N(0, 1);
  * optional RoPE on K and Q (interleaved pairs (2i, 2i+1), angle
    pos * 10000^(-2i/D), pos = global token index): "RoPE-induced scattering";
  * stored as binary32 or rounded to bfloat16 (round to nearest even).

Every array comes from numpy's default bit generator keyed by
(seed, layer, tensor, block, stream, sequence), so any sequence of any block
can be regenerated alone.  `torch_block` draws the same distributions on a
torch device for the benchmark (different random stream, same recipe).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence, Tuple

import numpy as np

VAR_SCALES = (1, 2, 3, 4, 5, 6, 8, 10, 13, 16)
VAR_BLOCKS = tuple(s * s for s in VAR_SCALES)  # 680 tokens
VIDEO_BLOCKS = (1560,) * 16

SEED_BASE = 0x5641525100
TENSOR_ID = {"k": 0, "v": 1, "q": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    heads: int
    head_dim: int
    bits: int
    blocks: Tuple[int, ...]
    src: str = "bf16"  # "bf16" | "f32"
    rope: bool = False
    seed: int = SEED_BASE
    n_outliers: int = 4
    outlier_lo: float = 20.0
    outlier_hi: float = 60.0
    bias_var: float = 2.0

    @property
    def total_tokens(self) -> int:
        return int(sum(self.blocks))

    def offset(self, block: int) -> int:
        return int(sum(self.blocks[:block]))

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    # 1 layer, batch 1, 16x64, fp32, INT4, last scale's 256 queries over 680
    "var256_tiny_int4": Workload("var256_tiny_int4", 1, 1, 16, 64, 4, VAR_BLOCKS, "f32",
                                 seed=SEED_BASE + 1),
    # VAR-d20 shape: 20 layers, 20x64, batch 128, bf16, INT4
    "var_d20_b128_int4": Workload("var_d20_b128_int4", 20, 128, 20, 64, 4, VAR_BLOCKS,
                                  seed=SEED_BASE + 2),
    # same with dense INT3 and RoPE on K/Q
    "var_d20_b128_int3_rope": Workload("var_d20_b128_int3_rope", 20, 128, 20, 64, 3, VAR_BLOCKS,
                                       rope=True, seed=SEED_BASE + 3),
    # VAR-d24 shape, INT4 and INT3
    "var_d24_b128_int4": Workload("var_d24_b128_int4", 24, 128, 24, 64, 4, VAR_BLOCKS,
                                  seed=SEED_BASE + 4),
    "var_d24_b128_int3": Workload("var_d24_b128_int3", 24, 128, 24, 64, 3, VAR_BLOCKS,
                                  seed=SEED_BASE + 4),
    # width 1920 (VAR-d30), batch 768 = 6 x 128
    "var_w1920_b768_int3": Workload("var_w1920_b768_int3", 30, 768, 30, 64, 3, VAR_BLOCKS,
                                    seed=SEED_BASE + 5),
    # next-frame video: 16 frame blocks of 1560 tokens, 40x128, batch 1
    "video_16x1560_h40d128_int3": Workload("video_16x1560_h40d128_int3", 30, 1, 40, 128, 3,
                                           VIDEO_BLOCKS, seed=SEED_BASE + 6),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) & 0xFFFFFFFFFFFF for k in key])


def channel_structure(wl: Workload, layer: int, tensor: str):
    """Per (layer, K/V): bias mu[H, D], outlier channels idx[H, n_out], signs[H, n_out]."""
    tid = TENSOR_ID[tensor]
    g = _rng(wl.seed, layer, tid, 1 << 20, 0)
    mu = (np.sqrt(wl.bias_var) * g.standard_normal((wl.heads, wl.head_dim))).astype(np.float64)
    idx = np.stack([g.choice(wl.head_dim, wl.n_outliers, replace=False) for _ in range(wl.heads)])
    sign = np.where(g.random((wl.heads, wl.n_outliers)) < 0.5, -1.0, 1.0)
    return mu, idx, sign


def outlier_magnitudes(wl: Workload, layer: int, tensor: str, block: int) -> np.ndarray:
    """m[H, n_out] ~ U[lo, hi] for one block (shared across the batch)."""
    g = _rng(wl.seed, layer, TENSOR_ID[tensor], block, 1)
    return g.uniform(wl.outlier_lo, wl.outlier_hi, (wl.heads, wl.n_outliers))


def rope_rotate(x: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """Interleaved-pair rotary embedding along the last axis; x[..., t, h, d]."""
    D = x.shape[-1]
    i = np.arange(D // 2, dtype=np.float64)
    inv_freq = 10000.0 ** (-2.0 * i / D)
    ang = positions[:, None].astype(np.float64) * inv_freq[None, :]  # [t, D/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x0 = x[..., 0::2].astype(np.float64)
    x1 = x[..., 1::2].astype(np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 to bfloat16, nearest-even; returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _finish(wl: Workload, x: np.ndarray) -> np.ndarray:
    if wl.src == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    return f32_to_bf16_bits(x.astype(np.float32))


def kv_block(wl: Workload, layer: int, tensor: str, block: int,
             seqs: Optional[Sequence[int]] = None) -> np.ndarray:
    """K or V of one block: [len(seqs)][n_k][H][D] as float32 or bf16 bits."""
    assert tensor in ("k", "v")
    seqs = range(wl.batch) if seqs is None else seqs
    n = wl.blocks[block]
    H, D = wl.heads, wl.head_dim
    mu, idx, sign = channel_structure(wl, layer, tensor)
    mag = outlier_magnitudes(wl, layer, tensor, block)
    shift = mu.copy()
    for h in range(H):
        shift[h, idx[h]] += sign[h] * mag[h]
    out = np.empty((len(seqs), n, H, D), dtype=np.float32)
    pos = np.arange(wl.offset(block), wl.offset(block) + n)
    for j, b in enumerate(seqs):
        g = _rng(wl.seed, layer, TENSOR_ID[tensor], block, 2, b)
        x = g.standard_normal((n, H, D), dtype=np.float32).astype(np.float64) + shift[None]
        if wl.rope and tensor == "k":
            x = rope_rotate(x, pos)
        out[j] = x.astype(np.float32)
    return _finish(wl, out)


def q_block(wl: Workload, layer: int, block: int,
            seqs: Optional[Sequence[int]] = None) -> np.ndarray:
    """Queries of one block: [len(seqs)][n_k][H][D] bf16 bits (always bf16)."""
    seqs = range(wl.batch) if seqs is None else seqs
    n = wl.blocks[block]
    H, D = wl.heads, wl.head_dim
    out = np.empty((len(seqs), n, H, D), dtype=np.float32)
    pos = np.arange(wl.offset(block), wl.offset(block) + n)
    for j, b in enumerate(seqs):
        g = _rng(wl.seed, layer, TENSOR_ID["q"], block, 3, b)
        x = g.standard_normal((n, H, D), dtype=np.float32).astype(np.float64)
        if wl.rope:
            x = rope_rotate(x, pos)
        out[j] = x.astype(np.float32)
    return f32_to_bf16_bits(out)


# --------------------------------------------------------------------------
# torch-side drawing of the same recipe (benchmark inputs made on the device)
# --------------------------------------------------------------------------

def torch_block(wl: Workload, layer: int, tensor: str, block: int, device, generator=None):
    """Same distributions as kv_block / q_block, drawn with torch on `device`.

    Returns a bf16 (or fp32) tensor [B][n_k][H][D].  The random stream differs
    from the numpy one; only the recipe is shared.
    """
    import torch

    n = wl.blocks[block]
    B, H, D = wl.batch, wl.heads, wl.head_dim
    x = torch.randn((B, n, H, D), device=device, dtype=torch.float32, generator=generator)
    if tensor in ("k", "v"):
        mu, idx, sign = channel_structure(wl, layer, tensor)
        mag = outlier_magnitudes(wl, layer, tensor, block)
        shift = mu.copy()
        for h in range(H):
            shift[h, idx[h]] += sign[h] * mag[h]
        x += torch.from_numpy(shift.astype(np.float32)).to(device)[None, None]
    if wl.rope and tensor in ("k", "q"):
        pos = torch.arange(wl.offset(block), wl.offset(block) + n, device=device,
                           dtype=torch.float64)
        i = torch.arange(D // 2, device=device, dtype=torch.float64)
        ang = pos[:, None] * (10000.0 ** (-2.0 * i / D))[None, :]
        c = torch.cos(ang)[None, :, None, :].float()
        s = torch.sin(ang)[None, :, None, :].float()
        x0, x1 = x[..., 0::2].clone(), x[..., 1::2].clone()
        x[..., 0::2] = x0 * c - x1 * s
        x[..., 1::2] = x0 * s + x1 * c
    if tensor == "q" or wl.src == "bf16":
        return x.to(torch.bfloat16)
    return x


def checksum(*arrays: np.ndarray) -> str:
    """blake2b-64 of the input bytes, logged next to results."""
    import hashlib

    h = hashlib.blake2b(digest_size=8)
    for a in arrays:
        h.update(np.ascontiguousarray(a).view(np.uint8).tobytes())
    return h.hexdigest()
