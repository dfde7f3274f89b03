"""3D rotary position embedding (oracle).

Follows "DiT, Flow Matching e 3D Attention", section "3D-RoPE e atenção
espaço-temporal": the head dimension splits as d_head = d_t + d_h + d_w, one
slice per axis (frame index t, row y, column x); each slice carries rotations
of coordinate pairs driven by its own coordinate (as 1D text RoPE does with the
token index), and the combined orthogonal rotation R_3D(t, y, x) multiplies q
and k before the attention dot product. V is not rotated.

Readings where the page is silent: slices are laid out [t | h | w] in the
order the page lists them; within a slice of width d_a the pairs are adjacent
coordinates (o_a + 2j, o_a + 2j + 1); the pair frequency is
theta_{a,j} = base^(-2j / d_a) with each axis using its own width d_a; the
pair (x0, x1) turns by +phi, phi = pos_a * theta_{a,j}:
    x0' = x0 cos(phi) - x1 sin(phi),   x1' = x0 sin(phi) + x1 cos(phi).
"""
from __future__ import annotations

import numpy as np


def pair_table(split, base: float):
    """For every pair of a head vector: (axis, first dim, frequency theta)."""
    table = []
    off = 0
    for axis, d_a in enumerate(split):
        if d_a % 2:
            raise ValueError("each RoPE axis width must be even")
        for j in range(d_a // 2):
            table.append((axis, off + 2 * j, float(base) ** (-2.0 * j / d_a)))
        off += d_a
    return table


def rotation_angles(pos: np.ndarray, split, base: float) -> np.ndarray:
    """phi[token, pair] = pos[token, axis(pair)] * theta(pair), float64."""
    pos = np.asarray(pos, dtype=np.float64)
    table = pair_table(split, base)
    axis = np.array([a for a, _, _ in table], dtype=np.int64)
    theta = np.array([t for _, _, t in table], dtype=np.float64)
    return pos[:, axis] * theta[None, :]


def apply_rope(x: np.ndarray, pos: np.ndarray, split, base: float) -> np.ndarray:
    """R_3D(pos) applied to every head of x [tokens, heads, head_dim] (float64 out)."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    if sum(split) != hd:
        raise ValueError("d_t + d_h + d_w must equal head_dim")
    phi = rotation_angles(pos, split, base)          # [tokens, hd/2]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out
