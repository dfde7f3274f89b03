"""Patch-grid indexing (oracle).

Follows "DiT, Flow Matching e 3D Attention", section "A ruptura da U-Net: por
que o Diffusion Transformer escala melhor?": a latent volume C x T x H x W is cut
into p_t x p_h x p_w patches, giving N = (T/p_t)(H/p_h)(W/p_w) tokens.

The page gives only the count; the token order is a reading: time-major,
row-major, w' fastest, so token n of a sequence sits at
t' = n // (H'W'), h' = (n // W') % H', w' = n % W'. Packed sequences restart
their coordinates at 0 (each clip is its own grid).
"""
from __future__ import annotations

import numpy as np


def num_tokens(T: int, H: int, W: int, p_t: int, p_h: int, p_w: int) -> int:
    """N = (T / p_t) * (H / p_h) * (W / p_w); each side must divide exactly."""
    for side, p in ((T, p_t), (H, p_h), (W, p_w)):
        if side % p != 0:
            raise ValueError(f"latent side {side} is not a multiple of patch {p}")
    return (T // p_t) * (H // p_h) * (W // p_w)


def coords(n: np.ndarray, grid_h: int, grid_w: int) -> np.ndarray:
    """Closed form: local token index -> (t', h', w') as int64 [len(n), 3]."""
    n = np.asarray(n, dtype=np.int64)
    hw = grid_h * grid_w
    return np.stack([n // hw, (n // grid_w) % grid_h, n % grid_w], axis=-1)


def coords_bruteforce(frames: int, grid_h: int, grid_w: int) -> np.ndarray:
    """Enumerate the grid in token order with three nested loops."""
    out = []
    for t in range(frames):
        for h in range(grid_h):
            for w in range(grid_w):
                out.append((t, h, w))
    return np.asarray(out, dtype=np.int64).reshape(-1, 3)


def token_of(c: np.ndarray, grid_h: int, grid_w: int) -> np.ndarray:
    """Inverse map (t', h', w') -> local token index."""
    c = np.asarray(c, dtype=np.int64)
    return (c[..., 0] * grid_h + c[..., 1]) * grid_w + c[..., 2]


def positions(cu_seqlens: np.ndarray, grid_h: int, grid_w: int) -> np.ndarray:
    """Position ids [tokens, 3] of a packed batch; coordinates restart per sequence."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    parts = []
    for s in range(len(cu) - 1):
        n = np.arange(cu[s + 1] - cu[s], dtype=np.int64)
        parts.append(coords(n, grid_h, grid_w))
    if not parts:
        return np.zeros((0, 3), dtype=np.int64)
    return np.concatenate(parts, axis=0)

