"""Helpers for the GPU parity tests: move synthetic inputs to the device in the
workload's dtype, bring results back as float64, and the tolerances."""
import numpy as np
import pytest
import torch

import synth

# max-abs error bars against the unrounded float64 oracle, unit-variance inputs
TOL = {"f32": 1e-4, "bf16": 2e-2}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def tdtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def dev(a, w=None, dtype=None):
    """numpy float32 (bf16-exact for bf16 workloads) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    dt = dtype if dtype is not None else (tdtype(w) if w is not None else torch.float32)
    return t.to(dt).cuda()


def host64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def maxabs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    if a.size == 0:
        return 0.0
    assert np.all(np.isfinite(a)), "non-finite values in GPU output"
    return float(np.max(np.abs(a - b)))


def sample_rows(w, per_seq=48, edge=8, seed=99):
    """Token rows to check at full size: the first/last `edge` rows of every
    sequence plus `per_seq` seeded random rows of each."""
    r = np.random.default_rng(seed)
    cu = w.cu_seqlens.astype(np.int64)
    rows = []
    for s in range(w.num_seqs):
        lo, hi = int(cu[s]), int(cu[s + 1])
        n = hi - lo
        rows += list(range(lo, lo + min(edge, n)))
        rows += list(range(max(lo, hi - edge), hi))
        rows += list(lo + r.choice(n, size=min(per_seq, n), replace=False))
    return np.unique(np.asarray(rows, dtype=np.int64))


def note(msg):
    print(msg, flush=True)


# ---- the persistent attention launch's tail split, replicated from its
# definition (dit_attn_common.hpp): which work items a launch cuts into pieces
def xcd_slice(total, x):
    per, rem = divmod(total, 8)
    ln = per + (1 if x < rem else 0)
    start = x * (per + 1) if x < rem else rem * (per + 1) + (x - rem) * per
    return start, ln


def split_plan(ln, C, max_s=16):
    """(T, s): the last T items of an XCD range of ln items are cut into s pieces."""
    if C > 32 or C <= 0 or ln < 2 * C:
        return 0, 1
    if ln % C == 0:
        return C, 2
    t = ln % C
    best, bn, bd = 1, 1, 1
    for c in range(2, max_s + 1):
        if t * c > 2 * C:
            break
        num = -(-(t * c) // C)
        if num * bd < bn * c:
            best, bn, bd = c, num, c
    return (t, best) if best > 1 else (0, 1)


def split_items(total, cus):
    """{item index: pieces} of a persistent launch of `total` work items on a
    device with `cus` compute units (one block per unit)."""
    out = {}
    if cus % 8:
        return out
    C = cus // 8
    for x in range(8):
        start, ln = xcd_slice(total, x)
        T, s = split_plan(ln, C)
        for i in range(start + ln - T, start + ln):
            out[i] = s
    return out


def item_rows(w, item, bq=256):
    """Work item -> (head, token rows) for the attention work numbering: head-major
    over the query tiles of every sequence, longest sequence first (index order
    among equals, or plain index order past 32 sequences)."""
    lens = [int(w.cu_seqlens[s + 1] - w.cu_seqlens[s]) for s in range(w.num_seqs)]
    tiles = [-(-n // bq) for n in lens]
    per_head = sum(tiles)
    head, r = divmod(item, per_head)
    order = list(range(w.num_seqs)) if w.num_seqs > 32 else sorted(range(w.num_seqs), key=lambda s: (-lens[s], s))
    for s in order:
        if r < tiles[s]:
            lo = int(w.cu_seqlens[s]) + r * bq
            return head, np.arange(lo, min(lo + bq, int(w.cu_seqlens[s + 1])), dtype=np.int64)
        r -= tiles[s]
    raise ValueError(item)


def attn_items_total(w, bq=256):
    return w.heads * sum(-(-int(w.cu_seqlens[s + 1] - w.cu_seqlens[s]) // bq) for s in range(w.num_seqs))
