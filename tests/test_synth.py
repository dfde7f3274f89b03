"""Seeded input generation (CPU only)."""
import numpy as np
import torch

import synth


def test_bf16_round_matches_torch():
    r = np.random.default_rng(0)
    a = np.concatenate([r.standard_normal(100000).astype(np.float32) * s for s in (1e-3, 1, 1e3)])
    ours = synth.bf16_round(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)


def test_seeding_reproducible_and_independent():
    w = synth.custom("t", "bf16", (3, 5), (2,), 2, 64, (0, 32, 32))
    a = synth.make(w, ["q", "k"])
    b = synth.make(w, ["k"])
    assert np.array_equal(a["k"], b["k"])
    assert not np.array_equal(a["q"], a["k"])
    assert np.array_equal(synth.bf16_round(a["q"]), a["q"])


def test_workload_literals():
    assert synth.C3.tokens == 32760 and synth.C4.tokens == 27280 and synth.C2.tokens == 8192
    assert list(synth.C5.cu_seqlens) == [0, 7800, 21840, 42120, 74880]
    assert synth.C5.rows == 48 and synth.C2.rows == 2
    assert synth.C2.attn_flops() == 412316860416
    assert synth.C3.attn_flops() == 21979496448000


def test_per_frame_dt():
    dt = synth.dt_rows(synth.C5)
    t = synth.flow_times(synth.C5)
    assert dt.shape == (48,)
    assert np.all(dt >= 0) and np.all(dt <= np.float32(1 / 30))
    assert np.all(t.astype(np.float64) + dt.astype(np.float64) <= 1.0 + 1e-6)
