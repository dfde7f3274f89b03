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
