"""Flowception frame insertion and per-frame time schedule (oracle).

"Flowception: Temporally Expansive Flow Matching for Video Generation"
(technical summary, section 2, "Metodologia: Flowception"): sampling interleaves
denoising of the existing frames with stochastic insertion of new frames
between them. Every frame carries a local time t_i; a frame inserted during
sampling starts as unit Gaussian noise with its local time reset to 0, so later
frames have less time left to denoise; a global time runs from 0 to 1. Active
frames may receive insertions to their right, passive ones block them.

Readings taken here (the summary gives no formulas for these steps):
  * insertion counts are given per existing frame -- the number of new frames
    placed immediately after it (the random draw from the predicted rates is
    an input; passive frames carry 0);
  * new frames are taken from the given noise in order of their position in
    the packed batch;
  * a frame's step is dt_f = min(dt_max, 1 - t_f): frames advance together
    from their own local times and none passes t = 1.

Layout: a packed batch of sequences of frames; each frame is tokens_per_frame
consecutive token rows of the latent [tokens, channels]; cu_seqlens holds the
token offsets of the sequences. Plain Python loops over frames: test
infrastructure, written for clarity, not speed.
"""
from __future__ import annotations

import numpy as np


def insert_frames(z: np.ndarray, t_frames: np.ndarray, cu_seqlens, counts, noise: np.ndarray,
                  tokens_per_frame: int):
    """Insert counts[f] noise frames right after every existing frame f.

    Returns (z_out, t_out, cu_out, src): the new latent, per-frame local times
    (inserted frames at 0), the new token offsets of the sequences, and per
    output frame its source: the existing frame index, or -1 - n for the n-th
    noise frame."""
    tpf = int(tokens_per_frame)
    z = np.asarray(z)
    counts = [int(c) for c in counts]
    cu = [int(c) for c in cu_seqlens]
    frames_of_seq = [(cu[s] // tpf, cu[s + 1] // tpf) for s in range(len(cu) - 1)]
    blocks, t_out, src, cu_out = [], [], [], [0]
    n_noise = 0
    for (f0, f1) in frames_of_seq:
        for f in range(f0, f1):
            blocks.append(z[f * tpf:(f + 1) * tpf])
            t_out.append(float(t_frames[f]))
            src.append(f)
            for _ in range(counts[f]):
                blocks.append(noise[n_noise * tpf:(n_noise + 1) * tpf])
                t_out.append(0.0)
                src.append(-1 - n_noise)
                n_noise += 1
        cu_out.append(len(src) * tpf)
    z_out = np.concatenate(blocks, axis=0) if blocks else z[:0]
    return (z_out, np.asarray(t_out, dtype=np.float64), np.asarray(cu_out, dtype=np.int64),
            np.asarray(src, dtype=np.int64))


def frame_schedule(t_frames: np.ndarray, dt_max: float):
    """Per-frame step and advanced local times: dt_f = min(dt_max, 1 - t_f),
    t_f' = t_f + dt_f."""
    t = np.asarray(t_frames, dtype=np.float64)
    dt = np.minimum(float(dt_max), 1.0 - t)
    return dt, t + dt
