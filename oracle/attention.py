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


def _offsets(cu, tokens, num_seqs):
    if cu is None:
        per = tokens // num_seqs
        return np.arange(0, tokens + 1, per, dtype=np.int64)
    return np.asarray(cu, dtype=np.int64)


def attention_lse(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q, cu_k, num_seqs: int = 1,
                  rows=None, row_block: int = 1024):
    """Attention of each sequence's queries against that sequence's own key block,
    with the row log-sum-exp.

    Ring attention ("DiT, Flow Matching e 3D Attention", section "Engenharia de
    inferência e paralelismo de contexto: Ulysses, Ring Attention e FP8") passes
    key / value blocks between GPUs, so each GPU attends its queries to one block
    at a time; the log-sum-exp is what lets the block results be combined
    (merge below).

    Sequence s owns queries q[cu_q[s]:cu_q[s+1]] and keys / values
    k, v[cu_k[s]:cu_k[s+1]] (the query and key sets may differ in size, as when
    the keys of a sequence are split into blocks). For query row i of sequence s
    and head h, with scores s_j = q_i . k_j / sqrt(hd):
        lse[i, h] = ln sum_j exp(s_j)
        o[i, h]   = sum_j exp(s_j - lse) v_j
    which is the softmax of the page formula written through its normaliser. A
    sequence with no keys has an empty sum: lse = -inf and o = 0. cu_q / cu_k
    None means dense: num_seqs equal sequences. Returns (o, lse) in float64;
    with `rows` (sorted query indices) only those rows, shapes [len(rows), ...].
    The log-sum-exp is evaluated as max + ln sum exp(s - max) (the same number,
    without overflow)."""
    tq, heads, hd = q.shape
    cq = _offsets(cu_q, tq, num_seqs)
    ck = _offsets(cu_k, len(k), num_seqs)
    scale = 1.0 / math.sqrt(hd)
    rows = np.arange(tq, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    o = np.zeros((len(rows), heads, hd), dtype=np.float64)
    lse = np.full((len(rows), heads), -np.inf, dtype=np.float64)
    seq = _seq_of(cq, rows)
    for s in np.unique(seq):
        sel = np.nonzero(seq == s)[0]
        lo, hi = int(ck[s]), int(ck[s + 1])
        if hi == lo:
            continue
        for h in range(heads):
            K = np.asarray(k[lo:hi, h, :], dtype=np.float64)
            V = np.asarray(v[lo:hi, h, :], dtype=np.float64)
            for b0 in range(0, len(sel), row_block):
                idx = sel[b0:b0 + row_block]
                Q = np.asarray(q[rows[idx], h, :], dtype=np.float64)
                S = (Q @ K.T) * scale
                mx = S.max(axis=1, keepdims=True)
                L = mx + np.log(np.exp(S - mx).sum(axis=1, keepdims=True))
                o[idx, h, :] = np.exp(S - L) @ V
                lse[idx, h] = L[:, 0]
    return o, lse


def merge(o_a: np.ndarray, lse_a: np.ndarray, o_b: np.ndarray, lse_b: np.ndarray):
    """Combine two partial attentions of the same query rows over disjoint key
    sets A and B (two ring steps, same section as attention_lse) into the
    attention over A u B:
        lse = ln(exp(lse_a) + exp(lse_b))
        o   = exp(lse_a - lse) o_a + exp(lse_b - lse) o_b
    (each partial o is normalised by its own sum; the weights re-normalise them
    to the joint sum). Rows where both sets are empty stay o = 0, lse = -inf.
    o_*: [rows, heads, hd]; lse_*: [rows, heads]. float64."""
    lse_a = np.asarray(lse_a, np.float64)
    lse_b = np.asarray(lse_b, np.float64)
    lse = np.logaddexp(lse_a, lse_b)
    live = np.isfinite(lse)
    ref = np.where(live, lse, 0.0)   # any finite value where both sets are empty
    wa = np.where(live, np.exp(lse_a - ref), 0.0)
    wb = np.where(live, np.exp(lse_b - ref), 0.0)
    o = wa[..., None] * np.asarray(o_a, np.float64) + wb[..., None] * np.asarray(o_b, np.float64)
    return o, lse
