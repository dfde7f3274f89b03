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
  * k and v: one scale per (tensor, head): amax_h = max |x[:, h, :]| over all
    tokens, x is multiplied by 448 / amax_h (float32) so amax_h maps to 448,
    and the dequantisation scale is amax_h / 448 (float32); an all-zero head
    keeps scale 1 and codes 0. Below amax_h = 2^-100 the float32 quotient
    448 / amax_h can overflow, so there the product is formed as
    (x 2^64) (448 / (amax_h 2^64)): exact power-of-two scalings, the same
    float32 value wherever the plain form is finite;
  * q: one scale per head too, chosen together with k's so that the score
    scale -- the product of the two dequantisation scales and log2(e)/sqrt(d),
    which turns code dot products into base-2 exponents of the softmax -- is a
    power of two 2^n: n is the smallest integer with
    2^n >= amax_q amax_k log2(e) / (448^2 sqrt(d)) (so the largest |q| maps
    into (224, 448] rather than onto 448), decided in float64; q is multiplied
    by g = amax_k log2(e) / (448 sqrt(d)) 2^-n (float64, rounded once to
    float32) and the dequantisation scale is sq = 2^n sqrt(d) / (sk log2(e)),
    sk = k's scale. When amax_q or amax_k is 0 every score is 0 whatever q
    holds: q's codes are then 0, n = 0, sq = 1; likewise when n would lie
    below -127 (every score below 2^-127 times the largest product of codes,
    under 1e-31: uniform weights to float32 precision whatever q holds). Above
    127, n is kept at 127;
  * the float32 product x * multiplier is what is rounded to E4M3 (the
    integer code is decided in float32, the precision the GPU path uses).
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
N_MIN, N_MAX = -127, 127      # range of the score-scale exponent n (below: q's codes 0)


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
        if amax[h] < np.float32(2.0 ** -100):                   # pre-scaled: no overflow
            inv = np.float32(E4M3_MAX) / (amax[h] * np.float32(2.0 ** 64))
            y = ((x[:, h, :] * np.float32(2.0 ** 64)).astype(np.float32) * inv).astype(np.float32)
        else:
            inv = np.float32(E4M3_MAX) / amax[h]                # float32 division
            y = (x[:, h, :] * inv).astype(np.float32)           # float32 product
        y = np.clip(y, -E4M3_MAX, E4M3_MAX)
        codes[:, h, :] = e4m3_encode(y)
        scale[h] = amax[h] / np.float32(E4M3_MAX)
    return codes, amax, scale


def dequantize(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """codes [tokens, heads, hd], scale [heads] -> float64 values."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[None, :, None]


def _exponent(amax_q: float, amax_k: float, head_dim: int) -> int:
    """The smallest integer n with 2^n >= amax_q amax_k log2(e) / (448^2
    sqrt(head_dim)), decided in float64."""
    t = np.float64(amax_q) * np.float64(amax_k) * (np.log2(np.e) / (E4M3_MAX * E4M3_MAX * np.sqrt(np.float64(head_dim))))
    f, e = math.frexp(float(t))          # t = f 2^e, f in [0.5, 1)
    return e - 1 if f == 0.5 else e


def q_codes_zero(amax_q: float, amax_k: float, head_dim: int) -> bool:
    """q's codes are all 0: a zero amax, or every score below 2^-127 (n < N_MIN)."""
    return amax_q == 0 or amax_k == 0 or _exponent(amax_q, amax_k, head_dim) < N_MIN


def score_exponent(amax_q: float, amax_k: float, head_dim: int) -> int:
    """The score-scale exponent n (module docstring): 0 when q's codes are all
    0, at most N_MAX."""
    if q_codes_zero(amax_q, amax_k, head_dim):
        return 0
    return int(min(_exponent(amax_q, amax_k, head_dim), N_MAX))


def q_multiplier(amax_q: float, amax_k: float, head_dim: int) -> np.float32:
    """q's float32 multiplier g = amax_k log2(e) / (448 sqrt(head_dim)) 2^-n
    (float64, rounded once to float32); 0 when q's codes are all 0."""
    if q_codes_zero(amax_q, amax_k, head_dim):
        return np.float32(0.0)
    n = score_exponent(amax_q, amax_k, head_dim)
    return np.float32(np.float64(amax_k) * (np.log2(np.e) / (E4M3_MAX * np.sqrt(np.float64(head_dim)))) * 2.0 ** -float(n))


def quantize_q(q: np.ndarray, amax_k: np.ndarray):
    """q [tokens, heads, d] (float32 values) and k's per-head amax ->
    (codes uint8, amax_q [heads] float32, scale [heads] float64, n [heads] int64)
    with scale_q * (amax_k / 448) * log2(e) / sqrt(d) = 2^n."""
    q = np.asarray(q, dtype=np.float32)
    heads, d = q.shape[1], q.shape[2]
    amax = np.abs(q).max(axis=(0, 2)).astype(np.float32) if q.size else np.zeros(heads, np.float32)
    amax_k = np.asarray(amax_k, dtype=np.float32)
    codes = np.zeros(q.shape, dtype=np.uint8)
    scale = np.ones(heads, dtype=np.float64)
    n = np.zeros(heads, dtype=np.int64)
    for h in range(heads):
        if q_codes_zero(float(amax[h]), float(amax_k[h]), d):
            continue
        n[h] = score_exponent(float(amax[h]), float(amax_k[h]), d)
        g = q_multiplier(float(amax[h]), float(amax_k[h]), d)
        y = (q[:, h, :] * g).astype(np.float32)                 # float32 product
        y = np.clip(y, -E4M3_MAX, E4M3_MAX)
        codes[:, h, :] = e4m3_encode(y)
        sk = np.float64(amax_k[h] / np.float32(E4M3_MAX))       # k's float32 scale
        scale[h] = 2.0 ** float(n[h]) * np.sqrt(np.float64(d)) / (sk * np.log2(np.e))
    return codes, amax, scale, n


def quantize_qkv(q: np.ndarray, k: np.ndarray, v: np.ndarray):
    """The three tensors of one FP8 attention: k and v by quantize_per_head, q by
    quantize_q against k's amax. Returns (codes (q, k, v), amax [3, heads]
    float32, scale [3, heads] float64, n [heads])."""
    ck, ak, sk = quantize_per_head(k)
    cv, av, sv = quantize_per_head(v)
    cq, aq, sq, n = quantize_q(q, ak)
    return (cq, ck, cv), np.stack([aq, ak, av]), np.stack([sq, sk.astype(np.float64), sv.astype(np.float64)]), n
