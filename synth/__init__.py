"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module only draws random numbers and stores them; it holds none of the
method's arithmetic (no LayerNorm, rotation, softmax, residual or Euler math).
Both sides of every parity check receive exactly the arrays produced here:
the GPU path as device tensors, the oracle as float64 copies of the same values.

Workloads follow the shapes of the pages' image and video latents:
  * C1 tiny fp32 block (2x8x8 latent, patch 1x2x2 -> 2x4x4 = 32 tokens),
  * C2 image latent 128x128, patch 2x2 -> 64x64 = 4096 tokens, batch 2,
  * C3 480P video latent T=21, H=60, W=104, patch 1x2x2 -> 21x30x52 tokens,
  * C4 720P video latent T=31, H=44, W=80, patch 1x2x2 -> 31x22x40 tokens,
  * C5 four packed variable-length clips of 5/9/13/21 frames on a 30x52 grid.
Token counts and cu_seqlens are written out literally as the workload
definitions state them; the oracle derives them independently from the grid.

Seeding: every tensor draws from numpy.random.default_rng([seed, tensor_id]),
seed = 1000 + config number, so any tensor can be regenerated alone.
bf16 workloads draw in float32 and round once to bf16 (round to nearest even);
the rounded values are the inputs of both sides.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

# Fixed tensor ids: part of the seeding recipe, never reorder.
TENSOR_IDS = {
    "x": 0, "gamma": 1, "beta": 2, "alpha": 3, "q": 4, "k": 5, "v": 6,
    "z": 7, "u": 8, "tflow": 9, "x0": 10, "x1": 11, "lam": 12,
}

LATENT_CHANNELS = 64  # C * p_t * p_h * p_w = 16 * 1 * 2 * 2 values per token


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                      # "f32" or "bf16": storage of activations
    grid_hw: Tuple[int, int]        # patched H', W' (shared by every sequence)
    frames: Tuple[int, ...]         # patched T' of each packed sequence
    seqlens: Tuple[int, ...]        # tokens of each sequence (literal)
    heads: int
    head_dim: int
    rope_split: Tuple[int, int, int]  # (d_t, d_h, d_w)
    rope_base: float
    tokens_per_row: int             # tokens sharing one adaLN / dt parameter row
    seed: int
    alpha_dist: str = "normal"      # "normal" N(0, 0.1) or "uniform" U(0, 1)
    per_frame_time: bool = False    # dt_rows from per-frame flow times t_f
    dt: float = 1.0 / 30.0
    eps: float = 1e-6

    @property
    def d_model(self) -> int:
        return self.heads * self.head_dim

    @property
    def tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def rows(self) -> int:
        return self.tokens // self.tokens_per_row

    @property
    def num_seqs(self) -> int:
        return len(self.seqlens)

    @property
    def max_seqlen(self) -> int:
        return int(max(self.seqlens))

    @property
    def dense(self) -> bool:
        return len(set(self.seqlens)) == 1 and len(set(self.frames)) == 1

    @property
    def cu_seqlens(self) -> np.ndarray:
        cu = np.zeros(len(self.seqlens) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(np.asarray(self.seqlens, dtype=np.int64))
        return cu

    def attn_flops(self) -> int:
        """Matmul flops of attention: two products of 2*N*N*hd per sequence and head."""
        return int(sum(4 * n * n * self.heads * self.head_dim for n in self.seqlens))


C1 = Workload("c1_tiny_f32", "f32", (4, 4), (2,), (32,), 2, 64, (16, 24, 24), 10000.0,
              32, 1001, alpha_dist="uniform")
C2 = Workload("c2_image_4096_bf16", "bf16", (64, 64), (1, 1), (4096, 4096), 24, 128,
              (0, 64, 64), 10000.0, 4096, 1002)
C3 = Workload("c3_video480p_32760_bf16", "bf16", (30, 52), (21,), (32760,), 40, 128,
              (44, 42, 42), 10000.0, 32760, 1003)
C4 = Workload("c4_video720p_27280_bf16", "bf16", (22, 40), (31,), (27280,), 24, 128,
              (44, 42, 42), 10000.0, 27280, 1004)
C5 = Workload("c5_varlen_frames_bf16", "bf16", (30, 52), (5, 9, 13, 21),
              (7800, 14040, 20280, 32760), 24, 128, (44, 42, 42), 10000.0, 1560, 1005,
              per_frame_time=True)

WORKLOADS: Dict[str, Workload] = {w.name: w for w in (C1, C2, C3, C4, C5)}
ORDERED = (C1, C2, C3, C4, C5)


def custom(name: str, dtype: str, grid_hw: Tuple[int, int], frames: Sequence[int],
           heads: int, head_dim: int, rope_split: Tuple[int, int, int],
           tokens_per_row: Optional[int] = None, seed: int = 7,
           alpha_dist: str = "normal", per_frame_time: bool = False,
           rope_base: float = 10000.0) -> Workload:
    """A small workload for edge-case tests (ragged tails, tiny N, varlen)."""
    hw = grid_hw[0] * grid_hw[1]
    seqlens = tuple(int(f) * hw for f in frames)
    tpr = tokens_per_row if tokens_per_row is not None else seqlens[0]
    return Workload(name, dtype, tuple(grid_hw), tuple(int(f) for f in frames), seqlens,
                    heads, head_dim, tuple(rope_split), rope_base, tpr, seed,
                    alpha_dist=alpha_dist, per_frame_time=per_frame_time)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32.

    Storage rounding of synthetic inputs only (finite inputs assumed)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))
    out = ((bits + bias) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return out.view(np.float32)


def _rng(w: Workload, name: str) -> np.random.Generator:
    return np.random.default_rng([w.seed, TENSOR_IDS[name]])


def _normal(w: Workload, name: str, shape, std: float = 1.0) -> np.ndarray:
    a = _rng(w, name).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _store(w: Workload, a: np.ndarray) -> np.ndarray:
    return bf16_round(a) if w.dtype == "bf16" else np.ascontiguousarray(a, np.float32)


def flow_times(w: Workload) -> np.ndarray:
    """Per-row flow time t ~ U(0, 1) (one per frame when per_frame_time)."""
    return _rng(w, "tflow").random(size=w.rows, dtype=np.float64).astype(np.float32)


def dt_rows(w: Workload) -> np.ndarray:
    """Per-row Euler step size.

    Per-frame schedules take dt_f = min(1/30, 1 - t_f) so no frame passes t = 1;
    otherwise every row steps by the workload's dt."""
    if w.per_frame_time:
        t = flow_times(w).astype(np.float64)
        return np.minimum(w.dt, 1.0 - t).astype(np.float32)
    return np.full(w.rows, w.dt, dtype=np.float32)


def make(w: Workload, names: Iterable[str]) -> Dict[str, np.ndarray]:
    """Generate the requested tensors for workload ``w`` (float32 arrays).

    Activations: x [tokens, D], q/k/v [tokens, heads, hd], z/u [tokens, 64].
    Parameters (always float32): gamma/beta/alpha [rows, D], dt [rows].
    """
    out: Dict[str, np.ndarray] = {}
    T, D, H, hd = w.tokens, w.d_model, w.heads, w.head_dim
    for n in names:
        if n == "x":
            out[n] = _store(w, _normal(w, n, (T, D)))
        elif n in ("q", "k", "v"):
            out[n] = _store(w, _normal(w, n, (T, H, hd)))
        elif n in ("z", "u", "x0", "x1"):
            out[n] = _store(w, _normal(w, n, (T, LATENT_CHANNELS)))
        elif n in ("gamma", "beta"):
            out[n] = _normal(w, n, (w.rows, D), std=0.1)
        elif n == "alpha":
            if w.alpha_dist == "uniform":
                out[n] = _rng(w, n).random(size=(w.rows, D), dtype=np.float32)
            else:
                out[n] = _normal(w, n, (w.rows, D), std=0.1)
        elif n == "dt":
            out[n] = dt_rows(w)
        elif n == "tflow":
            out[n] = flow_times(w)
        elif n == "cu_seqlens":
            out[n] = w.cu_seqlens
        else:
            raise KeyError(f"unknown synthetic tensor {n!r}")
    return out


def uniform_keys(w: Workload, seed_tensor: str = "k") -> np.ndarray:
    """One key vector repeated for every token (identical-keys invariant)."""
    row = _store(w, _normal(w, seed_tensor, (1, w.heads, w.head_dim)))
    return np.ascontiguousarray(np.broadcast_to(row, (w.tokens, w.heads, w.head_dim)))


def dyadic(w: Workload, name: str, shape, lo: float = -4.0, hi: float = 4.0,
           step: float = 1.0 / 16.0) -> np.ndarray:
    """Values on the grid step*Z inside [lo, hi]: exact in bf16 and fp32, and their
    differences too (used for exact Euler landing checks)."""
    n_lo, n_hi = int(round(lo / step)), int(round(hi / step))
    ints = _rng(w, name).integers(n_lo, n_hi + 1, size=shape)
    return (ints.astype(np.float64) * step).astype(np.float32)
