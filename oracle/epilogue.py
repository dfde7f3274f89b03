"""Gated residual and rectified-flow Euler update (oracle).

Gated residual: "DiT, Flow Matching e 3D Attention", section "A ruptura da
U-Net": x'_l = x_l + alpha_1 * SelfAttention(...), with alpha initialised at
zero so every block starts as the identity. The attention branch enters with
its heads merged (column h * head_dim + i) and no output projection (a reading:
the projection needs trained weights). alpha is a per-channel row selected by
token // tokens_per_row.

Euler update: same page, section "Flow Matching e Rectified Flow": the path
x_t = (1 - t) x_0 + t x_1 runs from noise (t = 0) to data (t = 1) with constant
velocity x_1 - x_0, and a plain ODE sampler such as Euler follows it with few,
large steps: z <- z + dt * u, dt > 0 moving toward the data. dt is per row
(per sample, or per frame for per-frame local times as in "Flowception",
technical summary, section 2).
"""
from __future__ import annotations

import numpy as np


def gated_residual(x: np.ndarray, branch: np.ndarray, alpha: np.ndarray,
                   tokens_per_row: int) -> np.ndarray:
    """x_out[tok, c] = x[tok, c] + alpha[row, c] * branch[tok, c] (branch heads merged)."""
    x = np.asarray(x, dtype=np.float64)
    b = np.asarray(branch, dtype=np.float64).reshape(x.shape)
    a = np.asarray(alpha, dtype=np.float64)
    rows = np.arange(x.shape[0]) // int(tokens_per_row)
    return x + a[rows] * b


def euler_step(z: np.ndarray, u: np.ndarray, dt_rows: np.ndarray,
               tokens_per_row: int) -> np.ndarray:
    """z_out[tok] = z[tok] + dt_rows[row] * u[tok]."""
    z = np.asarray(z, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    dt = np.asarray(dt_rows, dtype=np.float64)
    rows = np.arange(z.shape[0]) // int(tokens_per_row)
    return z + dt[rows][:, None] * u


def interpolant(x0: np.ndarray, x1: np.ndarray, t) -> np.ndarray:
    """x_t = (1 - t) x_0 + t x_1 (t broadcast per row)."""
    x0 = np.asarray(x0, dtype=np.float64)
    x1 = np.asarray(x1, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    if t.ndim == 1:
        t = t[:, None]
    return (1.0 - t) * x0 + t * x1


def velocity(x0: np.ndarray, x1: np.ndarray) -> np.ndarray:
    """d/dt x_t = x_1 - x_0 for the linear path."""
    return np.asarray(x1, dtype=np.float64) - np.asarray(x0, dtype=np.float64)


def _rows(n: int, tokens_per_row: int) -> np.ndarray:
    return np.arange(n) // int(tokens_per_row)


def interpolant_rows(x0: np.ndarray, x1: np.ndarray, t_rows: np.ndarray,
                     tokens_per_row: int) -> np.ndarray:
    """Training input of the straight path ("DiT, Flow Matching e 3D Attention",
    section "Flow Matching e Rectified Flow"): x_t = (1 - t) x_0 + t x_1 with one
    flow time per row (sample or frame), row = token // tokens_per_row."""
    x0 = np.asarray(x0, dtype=np.float64)
    t = np.asarray(t_rows, dtype=np.float64)[_rows(x0.shape[0], tokens_per_row)]
    return interpolant(x0, x1, t)


def cfm_loss(u: np.ndarray, x0: np.ndarray, x1: np.ndarray, tokens_per_row: int):
    """Conditional flow-matching regression target (same section): the squared
    distance between the predicted velocity u and the path's velocity x_1 - x_0.

    Returns (per_token, per_row): per_token[tok] = sum over the token's channels
    of (u - (x_1 - x_0))^2; per_row[r] = sum of per_token over the row's tokens,
    i.e. the squared norm of the whole sample (or frame). The expectation over
    samples in the page's loss is the mean of per_row over the rows (a reading:
    the norm is taken over the sample's whole latent, not averaged per element)."""
    e = np.asarray(u, dtype=np.float64) - velocity(x0, x1)
    per_tok = (e * e).sum(axis=1)
    rows = _rows(e.shape[0], tokens_per_row)
    per_row = np.zeros(int(rows[-1]) + 1 if len(rows) else 0, dtype=np.float64)
    np.add.at(per_row, rows, per_tok)
    return per_tok, per_row


def midpoint_half(z: np.ndarray, u: np.ndarray, dt_rows: np.ndarray,
                  tokens_per_row: int) -> np.ndarray:
    """First stage of the explicit midpoint rule, the second ODE sampler the same
    section names beside Euler: z_mid = z + (dt / 2) u(z, t). The step then
    finishes with z + dt u(z_mid, t + dt / 2) (euler_step with the midpoint
    velocity)."""
    z = np.asarray(z, dtype=np.float64)
    dt = np.asarray(dt_rows, dtype=np.float64)[_rows(z.shape[0], tokens_per_row)]
    return z + 0.5 * dt[:, None] * np.asarray(u, dtype=np.float64)
