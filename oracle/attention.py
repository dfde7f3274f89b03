"""Scaled dot-product attention over patch tokens (oracle).

Follows "Por que é absurdamente difícil gerar um filme inteiro usando IA",
section "Matemática por trás" (Attention(Q, K, V) = softmax(Q K^T / sqrt(d)) V),
and "DiT, Flow Matching e 3D Attention", section "3D-RoPE e atenção
espaço-temporal", which fixes the scale as 1 / sqrt(d_head) on rotated q, k.
Full-sequence video models attend bidirectionally over every frame
("Flowception", technical summary, section 1), so there is no mask inside a
sequence; packed sequences (cu_seqlens) never attend to each other.

The softmax is the plain definition: subtract the row maximum, exponentiate,
divide by the row sum, over the FULL key set of the row's sequence. Rows are
processed in blocks only to bound memory; each block sees every key.
"""
from __future__ import annotations

import math

import numpy as np


def softmax_rows(s: np.ndarray) -> np.ndarray:
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=-1, keepdims=True)


def _seq_of(cu: np.ndarray, tok: np.ndarray) -> np.ndarray:
    return np.searchsorted(cu, tok, side="right") - 1


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens,
              rows=None, row_block: int = 1024) -> np.ndarray:
    """O[tok, h] = softmax(q[tok, h] . K_s[:, h]^T / sqrt(hd)) V_s[:, h].

    q, k, v: [tokens, heads, hd]. cu_seqlens: [num_seqs + 1] offsets.
    rows: optional sorted token indices; if given, only those rows are computed
    and the result is [len(rows), heads, hd]. float64 throughout."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    tokens, heads, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    rows = np.arange(tokens, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    out = np.empty((len(rows), heads, hd), dtype=np.float64)
    seq = _seq_of(cu, rows)
    for s in np.unique(seq):
        sel = np.nonzero(seq == s)[0]
        lo, hi = int(cu[s]), int(cu[s + 1])
        for h in range(heads):
            K = np.asarray(k[lo:hi, h, :], dtype=np.float64)
            V = np.asarray(v[lo:hi, h, :], dtype=np.float64)
            for b0 in range(0, len(sel), row_block):
                idx = sel[b0:b0 + row_block]
                Q = np.asarray(q[rows[idx], h, :], dtype=np.float64)
                P = softmax_rows((Q @ K.T) * scale)
                out[idx, h, :] = P @ V
    return out


def attention_bruteforce(q, k, v, cu_seqlens):
    """Pure-Python loops over (token, head, key, dim); for tiny inputs only."""
    cu = [int(c) for c in cu_seqlens]
    tokens, heads, hd = len(q), len(q[0]), len(q[0][0])
    scale = 1.0 / math.sqrt(hd)
    out = [[[0.0] * hd for _ in range(heads)] for _ in range(tokens)]
    for s in range(len(cu) - 1):
        for i in range(cu[s], cu[s + 1]):
            for h in range(heads):
                scores = []
                for j in range(cu[s], cu[s + 1]):
                    acc = 0.0
                    for e in range(hd):
                        acc += float(q[i][h][e]) * float(k[j][h][e])
                    scores.append(acc * scale)
                m = max(scores)
                w = [math.exp(x - m) for x in scores]
                tot = sum(w)
                for e in range(hd):
                    acc = 0.0
                    for jj, j in enumerate(range(cu[s], cu[s + 1])):
                        acc += w[jj] * float(v[j][h][e])
                    out[i][h][e] = acc / tot
    return out
