"""Operand-precision study of the packed-cache attention (CPU, oracle caches).

The attention's contractions run on matrix cores whose operands are 8- or
16-bit floating point, so the design has to choose a format for each operand:
the dequantized keys k_hat and values v_hat, the queries q and the softmax
weights P.  This study emulates each candidate by rounding the operands the
way the kernel would and then doing the arithmetic exactly (float64), and
measures the attention output against the binary64 attention over the same
dequantized cache (the oracle's definition).  Accumulation rounding (fp32 in
the kernel) is not modelled; only the operand formats are.

Formats, written from their definitions:
  * bf16: 8 significant bits; round to nearest even, or truncation;
  * binary16: 11 significant bits (numpy float16), nearest even, or toward zero;
  * e4m3 (OCP FP8 E4M3FN): 4 significant bits, exponent bias 7, smallest normal
    2^-6, subnormal step 2^-9, largest finite 448 (saturated here);
  * fixed point of B bits per (query, block): step = max|v| / (2^(B-1) - 1).

Candidates for the QK^T product (P and v_hat as in the kernel):
  * ``kernel``        k_hat = fp32 fma(code, s, z) split into a truncated bf16
                      high part and a nearest-even bf16 remainder; two bf16
                      MFMAs against the bf16 query (what attend.hip runs);
  * ``bf16``          k_hat rounded once to bf16;
  * ``f16``           k_hat rounded once to binary16;
  * ``f16_cs_bias``   binary16 (code * s) with the zero point folded into a
                      per-(query, block) bias q . z;
  * ``fix16``/``fix24`` the scale folded into the query (q (.) s per block in
                      B-bit fixed point) against the raw integer codes, plus
                      the bias q . z: the integer-MFMA form;
  * ``e4m3_kq``       k_hat and q in e4m3.
Candidates for the PV product (QK^T as in the kernel):
  * ``kernel``        P rounded toward zero and v_hat to nearest, binary16;
  * ``bf16_pv``       P truncated and v_hat rounded to bf16;
  * ``e4m3_pv``       P and v_hat in e4m3;
  * ``e4m3_all``      k_hat, q, P and v_hat in e4m3.

Data: the synthetic caches of `varq_inputs` (per-channel bias, massive
channels redrawn per block, optional RoPE on K), quantized by the oracle:
  * ``var_d20_int3_rope``: VAR-d20 shape, one sequence, 20 heads x 64, INT3
    with RoPE, the last block's 256 queries over all 680 keys;
  * ``video_int3``, ``video_int3_rope``, ``video_int4_rope``: the next-frame
    video shape, 4 of its heads x 128, the last of 3 frames of 1560 tokens
    (every 8th query) over the 4680 keys of the three frames.
Error: max |O - O_ref| / max |O_ref| over the call (the tests' metric).

TEST INFRASTRUCTURE ONLY (it calls the oracle).  `python tests/study_operand_precision.py`
prints the table.
"""
from __future__ import annotations

import os
import sys
from typing import Dict

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import varq_inputs as vi  # noqa: E402
from oracle import binding as ob  # noqa: E402

QK_VARIANTS = ("kernel", "bf16", "f16", "f16_cs_bias", "fix16", "fix24", "e4m3_kq")
PV_VARIANTS = ("kernel", "bf16_pv", "e4m3_pv", "e4m3_all")

# ---------------------------------------------------------------------------
# formats
# ---------------------------------------------------------------------------


def bf16_rne(x: np.ndarray) -> np.ndarray:
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def bf16_trunc(x: np.ndarray) -> np.ndarray:
    u = np.asarray(x, np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def f16_rne(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def f16_rtz(x: np.ndarray) -> np.ndarray:
    """binary16 toward zero, for x >= 0."""
    x = np.asarray(x, np.float64)
    h = x.astype(np.float16)
    over = h.astype(np.float64) > x
    h = np.where(over, np.nextafter(h, np.float16(0)), h)
    return h.astype(np.float64)


def e4m3(x: np.ndarray) -> np.ndarray:
    """OCP E4M3FN, nearest even, saturating at +-448."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)  # subnormals share the step of 2^-6 .. 2^-5
    ulp = np.exp2(e - 3.0)
    r = np.minimum(np.round(a / ulp) * ulp, 448.0)
    return np.sign(x) * r


def fixed(v: np.ndarray, bits: int) -> np.ndarray:
    """B-bit fixed point with one step per row (last axis reduced)."""
    m = np.abs(v).max(axis=-1, keepdims=True)
    step = np.where(m > 0, m / (2.0 ** (bits - 1) - 1.0), 1.0)
    return np.round(v / step) * step


# ---------------------------------------------------------------------------
# caches and the exact reference
# ---------------------------------------------------------------------------


def build_case(wl: vi.Workload, last: int, qstride: int):
    """Quantize blocks 0..last with the oracle; return per head the codes,
    per-key zero/step (expanded from the (block, channel) groups), the block of
    every key, q (bf16 values) of block `last` (every qstride-th query)."""
    L = ob.layout_of(wl)
    kc, vc = ob.alloc_cache(L), ob.alloc_cache(L)
    for j in range(last + 1):
        st = ob.quantize_block(L, j, vi.kv_block(wl, 0, "k", j), vi.kv_block(wl, 0, "v", j), kc, vc)
        assert st == ob.OK
    T = wl.offset(last) + wl.blocks[last]
    blk = np.repeat(np.arange(last + 1), wl.blocks[: last + 1])
    H, D = wl.heads, wl.head_dim
    out = {}
    for name, c in (("k", kc), ("v", vc)):
        codes = ob.unpack(wl.bits, c["codes"][0].reshape(H * c["codes"].shape[2], -1), D)
        codes = codes.reshape(H, -1, D)[:, :T].astype(np.float64)
        z = ob.h2f(c["zero"][0]).astype(np.float64)[:, blk, :]    # [H][T][D]
        s = ob.h2f(c["scale"][0]).astype(np.float64)[:, blk, :]
        out[name] = (codes, z, s)
    q = vi.bf16_bits_to_f32(vi.q_block(wl, 0, last)[0]).astype(np.float64)  # [n][H][D]
    q = np.transpose(q, (1, 0, 2))[:, ::qstride]                             # [H][nq][D]
    return out, blk, q


def softmax_weights(S: np.ndarray, scale: float) -> np.ndarray:
    m = S.max(axis=-1, keepdims=True)
    return np.exp2((S - m) * scale * np.log2(np.e))


def attention_errors(case, blk, q) -> Dict[str, Dict[str, float]]:
    (kcode, kz, ks), (vcode, vz, vs) = case["k"], case["v"]
    H, nq, D = q.shape
    scale = 1.0 / np.sqrt(D)
    k64 = kcode * ks + kz                       # exact dequantized values
    v64 = vcode * vs + vz
    k32 = k64.astype(np.float32)                # fp32 fma: one rounding of the exact value
    v32 = v64.astype(np.float32)
    nb = int(blk.max()) + 1
    ref = np.empty((H, nq, D))
    for h in range(H):
        P = softmax_weights(q[h] @ k64[h].T, scale)
        ref[h] = (P @ v64[h]) / P.sum(axis=-1, keepdims=True)
    refmax = np.abs(ref).max()

    def qk(h, variant):
        if variant == "kernel":
            hi = bf16_trunc(k32[h])
            lo = bf16_rne((k32[h].astype(np.float64) - hi).astype(np.float32))
            return q[h] @ (hi + lo).T
        if variant == "bf16":
            return q[h] @ bf16_rne(k32[h]).T
        if variant == "f16":
            return q[h] @ f16_rne(k32[h]).T
        if variant == "e4m3_kq":
            return e4m3(q[h]) @ e4m3(k32[h]).T
        # forms with the zero point as a per-(query, block) bias q . z
        S = np.empty((nq, k64.shape[1]))
        for b in range(nb):
            sel = blk == b
            z_b, s_b, c_b = kz[h][sel][0], ks[h][sel][0], kcode[h][sel]
            bias = q[h] @ z_b
            if variant == "f16_cs_bias":
                S[:, sel] = q[h] @ f16_rne(c_b * s_b).T + bias[:, None]
            else:  # fix16 / fix24: q (.) s_b in fixed point against the integer codes
                qs = fixed(q[h] * s_b, 16 if variant == "fix16" else 24)
                S[:, sel] = qs @ c_b.T + bias[:, None]
        return S

    errs = {"qk": {}, "pv": {}}
    kernel_S = [qk(h, "kernel") for h in range(H)]
    for variant in QK_VARIANTS:
        out = np.empty_like(ref)
        for h in range(H):
            S = kernel_S[h] if variant == "kernel" else qk(h, variant)
            P = f16_rtz(softmax_weights(S, scale))
            out[h] = (P @ f16_rne(v32[h])) / P.sum(axis=-1, keepdims=True)
        errs["qk"][variant] = float(np.abs(out - ref).max() / refmax)
    for variant in PV_VARIANTS:
        out = np.empty_like(ref)
        for h in range(H):
            if variant == "e4m3_all":
                S = qk(h, "e4m3_kq")
            else:
                S = kernel_S[h]
            p = softmax_weights(S, scale)
            if variant == "kernel":
                P, V = f16_rtz(p), f16_rne(v32[h])
            elif variant == "bf16_pv":
                P, V = bf16_trunc(p.astype(np.float32)), bf16_rne(v32[h])
            else:
                P, V = e4m3(p), e4m3(v32[h])
            out[h] = (P @ V) / P.sum(axis=-1, keepdims=True)
        errs["pv"][variant] = float(np.abs(out - ref).max() / refmax)
    return errs


def datasets():
    var = vi.WORKLOADS["var_d20_b128_int3_rope"].with_(batch=1)
    video = vi.WORKLOADS["video_16x1560_h40d128_int3"].with_(heads=4, blocks=(1560, 1560, 1560))
    return {
        "var_d20_int3_rope": (var, len(var.blocks) - 1, 1),
        "video_int3": (video, 2, 8),
        "video_int3_rope": (video.with_(rope=True), 2, 8),
        "video_int4_rope": (video.with_(rope=True, bits=4), 2, 8),
    }


def run_study() -> Dict[str, Dict[str, Dict[str, float]]]:
    res = {}
    for name, (wl, last, stride) in datasets().items():
        case, blk, q = build_case(wl, last, stride)
        res[name] = attention_errors(case, blk, q)
    return res


if __name__ == "__main__":
    res = run_study()
    names = list(res)
    print("| product | operand format | " + " | ".join(names) + " |")
    print("|---|---|" + "---|" * len(names))
    for part, variants in (("qk", QK_VARIANTS), ("pv", PV_VARIANTS)):
        for v in variants:
            print(f"| {'QK^T' if part == 'qk' else 'PV'} | {v} | "
                  + " | ".join(f"{res[n][part][v]:.2e}" for n in names) + " |")
