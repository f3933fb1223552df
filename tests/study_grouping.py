"""Grouping-accuracy study on synthetic VAR caches (CPU, oracle arithmetic).

The VAR-Q abstract states that the outliers of visual-autoregressive KV caches
sit on two axes, the feature channel and the decoding block, and that VAR-Q
therefore gives every (block, channel) cell its own zero point and scale.
This module measures what that buys on the synthetic caches of
`varq_inputs`, which carry exactly that structure (per-channel bias, a few
massive channels whose magnitude is fixed inside a block and redrawn per
block, optional RoPE on K), against two other group shapes that use the same
quantizer per group:

  * ``block_channel`` -- one group per (block, channel): the VAR-Q grouping;
  * ``channel_seq``   -- one group per channel over the whole sequence
                         (block boundaries ignored);
  * ``token``         -- one group per token over head_dim.

Each group goes through the oracle's single-group quantizer
(`kvqr_quantize_group`: asymmetric min/max, zero and scale stored as
binary16) and is dequantized as code * scale + zero.  Errors reported:

  * relative dequantization MSE of K and of V: mean((x_hat - x)^2) / mean(x^2);
  * relative attention error of the last block's queries over the whole
    cache (the last block sees every key under block-causal masking):
    ||O(K_hat, V_hat) - O(K, V)||_F / ||O(K, V)||_F, softmax attention in
    float64 with scale 1/sqrt(D).

TEST INFRASTRUCTURE ONLY (it calls the oracle).  `python tests/study_grouping.py`
prints the full table at the 16-head shape.
"""
from __future__ import annotations

import os
import sys
from typing import Dict, Sequence

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import varq_inputs as vi  # noqa: E402
from oracle import binding as ob  # noqa: E402

GROUPINGS = ("block_channel", "channel_seq", "token")


def _dequant_group(x: np.ndarray, bits: int) -> np.ndarray:
    st, z, s, codes = ob.quantize_group(x, bits)
    if st != ob.OK:
        raise ValueError(f"kvqr_quantize_group status {st}")
    zf = float(ob.h2f(np.array([z], np.uint16))[0])
    sf = float(ob.h2f(np.array([s], np.uint16))[0])
    # code * scale + zero is exact in float64 (a <=8-bit code times a binary16
    # scale, plus a binary16 zero); one rounding to binary32 matches fmaf.
    return (codes.astype(np.float64) * sf + zf).astype(np.float32)


def quantize_grouped(x: np.ndarray, bits: int, grouping: str,
                     blocks: Sequence[int]) -> np.ndarray:
    """Quantize-dequantize x[T, H, D] with one (zero, scale) per group."""
    T, H, D = x.shape
    out = np.empty_like(x, dtype=np.float32)
    if grouping == "block_channel":
        off = 0
        for n in blocks:
            for h in range(H):
                for d in range(D):
                    out[off:off + n, h, d] = _dequant_group(x[off:off + n, h, d], bits)
            off += n
    elif grouping == "channel_seq":
        for h in range(H):
            for d in range(D):
                out[:, h, d] = _dequant_group(x[:, h, d], bits)
    elif grouping == "token":
        for t in range(T):
            for h in range(H):
                out[t, h, :] = _dequant_group(x[t, h, :], bits)
    else:
        raise ValueError(grouping)
    return out


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """q[n, H, D] attends to every row of k, v [T, H, D]; float64."""
    D = q.shape[-1]
    s = np.einsum("ihd,thd->hit", q.astype(np.float64), k.astype(np.float64)) / np.sqrt(D)
    s -= s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return np.einsum("hit,thd->ihd", p, v.astype(np.float64))


def study_cache(wl: vi.Workload, layer: int = 0, seq: int = 0):
    """K, V [T, H, D] (float32) of one sequence over all blocks, and the last block's Q."""
    nb = len(wl.blocks)
    k = np.concatenate([vi.kv_block(wl, layer, "k", b, [seq])[0] for b in range(nb)])
    v = np.concatenate([vi.kv_block(wl, layer, "v", b, [seq])[0] for b in range(nb)])
    q = vi.bf16_bits_to_f32(vi.q_block(wl, layer, nb - 1, [seq])[0])
    if k.dtype == np.uint16:
        k, v = vi.bf16_bits_to_f32(k), vi.bf16_bits_to_f32(v)
    return k, v, q


def _rel_mse(xh: np.ndarray, x: np.ndarray) -> float:
    x = x.astype(np.float64)
    return float(np.mean((xh.astype(np.float64) - x) ** 2) / np.mean(x ** 2))


def grouping_errors(wl: vi.Workload, bits: int,
                    groupings: Sequence[str] = GROUPINGS) -> Dict[str, Dict[str, float]]:
    k, v, q = study_cache(wl)
    ref = softmax_attention(q, k, v)
    res = {}
    for g in groupings:
        kh = quantize_grouped(k, bits, g, wl.blocks)
        vh = quantize_grouped(v, bits, g, wl.blocks)
        o = softmax_attention(q, kh, vh)
        res[g] = {
            "k_mse": _rel_mse(kh, k),
            "v_mse": _rel_mse(vh, v),
            "attn": float(np.linalg.norm(o - ref) / np.linalg.norm(ref)),
        }
    return res


def study_workload(rope: bool, heads: int = 16, persistent: bool = False) -> vi.Workload:
    """The 680-token VAR schedule, binary32 source, one sequence.

    ``persistent`` fixes every outlier magnitude to 40 in every block, which
    removes the block axis of the outlier structure (control case).
    """
    wl = vi.WORKLOADS["var256_tiny_int4"].with_(rope=rope, heads=heads)
    if persistent:
        wl = wl.with_(outlier_lo=40.0, outlier_hi=40.0)
    return wl


def main() -> None:
    print("| RoPE on K | outlier magnitude | bits | grouping | K rel. MSE | V rel. MSE | attention rel. error |")
    print("|---|---|---|---|---|---|---|")
    for rope in (False, True):
        for persistent in (False, True):
            wl = study_workload(rope, persistent=persistent)
            for bits in (2, 3, 4):
                r = grouping_errors(wl, bits)
                for g in GROUPINGS:
                    e = r[g]
                    print(f"| {'yes' if rope else 'no'} | {'fixed 40' if persistent else 'per block U[20,60]'} "
                          f"| {bits} | {g} | {e['k_mse']:.2e} | {e['v_mse']:.2e} | {e['attn']:.2e} |")


if __name__ == "__main__":
    main()
