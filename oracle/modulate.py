"""adaLN-Zero modulation (oracle).

Follows "DiT, Flow Matching e 3D Attention", section "A ruptura da U-Net": the
block feeds SelfAttention with gamma_1 * LayerNorm(x_l) + beta_1 (and the MLP
with gamma_2 * LayerNorm(x'_l) + beta_2), the six modulation parameters coming
from a shallow conditioning network.

Readings where the page is silent: LayerNorm normalises each token row over
d_model with the biased (population) variance and eps inside the square root;
it carries no affine of its own; the modulation is literally gamma * LN + beta
(not (1 + gamma)); gamma and beta are per-channel rows, one row per sample or
per frame, selected by token // tokens_per_row.
"""
from __future__ import annotations

import numpy as np


def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) over the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    mu = x.sum(axis=-1, keepdims=True) / d
    xc = x - mu
    var = (xc * xc).sum(axis=-1, keepdims=True) / d
    return xc / np.sqrt(var + eps)


def adaln_modulate(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray,
                   tokens_per_row: int, eps: float) -> np.ndarray:
    """y[tok] = gamma[row] * LayerNorm(x[tok]) + beta[row], row = tok // tokens_per_row."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    b = np.asarray(beta, dtype=np.float64)
    rows = np.arange(x.shape[0]) // int(tokens_per_row)
    return g[rows] * layer_norm(x, eps) + b[rows]
