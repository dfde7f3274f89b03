"""8-bit floating point (OCP E4M3) quantisation of q, k, v for FP8 attention
(oracle).

"DiT, Flow Matching e 3D Attention", section "Engenharia de inferência e
paralelismo de contexto: Ulysses, Ring Attention e FP8", pairs FlashAttention-3
with 8-bit floating point quantisation and names the E4M3 and E5M2 formats. The
attention itself is unchanged: it runs on the dequantised values, so its
oracle is oracle.attention on decode(code) * scale.

E4M3 (the OCP 8-bit format): 1 sign bit, 4 exponent bits with bias 7, 3
mantissa bits; exponent field 0 holds subnormals m * 2^-9; no infinities; the
largest finite value is 448 (exponent 15, mantissa 6); exponent 15 with
mantissa 7 is NaN. Encoding rounds to the nearest representable value, ties to
an even mantissa.

Readings taken here (the page gives none of these details):
  * one scale per (tensor, head): amax_h = max |x[:, h, :]| over all tokens,
    x is multiplied by 448 / amax_h (float32) so amax_h maps to 448, and the
    dequantisation scale is amax_h / 448 (float32); an all-zero head keeps
    scale 1 and codes 0;
  * the float32 product x * (448 / amax_h) is what is rounded to E4M3 (the
    integer code is decided in float32, the precision the GPU path uses).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Code bytes -> float64 values (NaN codes give nan)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    v = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return s * v


def e4m3_encode(x) -> np.ndarray:
    """float32 values with |x| <= 448 -> code bytes, round to nearest, ties to
    even: the value is scaled by its spacing (2^(e-3) for normal magnitudes in
    [2^e, 2^(e+1)), 2^-9 below 2^-6) and rounded half-to-even to an integer."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > E4M3_MAX) or np.any(~np.isfinite(x)):
        raise ValueError("e4m3_encode expects finite |x| <= 448")
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    spacing = np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(e - 3))
    q = np.rint(a / spacing)                     # half-to-even
    v = q * spacing                              # the rounded magnitude (may reach the next binade)
    out = np.zeros(x.shape, dtype=np.int64)
    sub = v < 2.0 ** -6
    out = np.where(sub, np.rint(v / 2.0 ** -9), 0)
    en = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    mant = np.rint((v / np.exp2(en) - 1.0) * 8.0)
    normal = ((en + 7).astype(np.int64) << 3) | mant.astype(np.int64)
    out = np.where(sub, out, normal).astype(np.int64)
    out = np.where(np.signbit(x), out | 0x80, out)   # negative values keep the sign, also when they round to 0
    return out.astype(np.uint8)


def quantize_per_head(x: np.ndarray):
    """x [tokens, heads, hd] (float32 values) -> (codes [tokens, heads, hd] uint8,
    amax [heads] float32, scale [heads] float32)."""
    x = np.asarray(x, dtype=np.float32)
    heads = x.shape[1]
    amax = np.abs(x).max(axis=(0, 2)).astype(np.float32) if x.size else np.zeros(heads, np.float32)
    codes = np.zeros(x.shape, dtype=np.uint8)
    scale = np.ones(heads, dtype=np.float32)
    for h in range(heads):
        if amax[h] == 0:
            continue
        inv = np.float32(E4M3_MAX) / amax[h]                    # float32 division
        y = (x[:, h, :] * inv).astype(np.float32)               # float32 product
        y = np.clip(y, -E4M3_MAX, E4M3_MAX)
        codes[:, h, :] = e4m3_encode(y)
        scale[h] = amax[h] / np.float32(E4M3_MAX)
    return codes, amax, scale


def dequantize(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """codes [tokens, heads, hd], scale [heads] -> float64 values."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[None, :, None]
