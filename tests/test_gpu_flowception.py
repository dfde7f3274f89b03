"""GPU parity of Flowception frame insertion and the per-frame schedule against
the oracle, through the C-ABI binding. Insertion is data movement: the latent,
local times, offsets and source map must match the oracle exactly. The
schedule's float32 arithmetic matches within 2e-7 and clipped steps land on
exactly 1.

Insertion counts are the random draws of the method (from the predicted
rates, which need a trained model): here seeded Poisson draws with the
passive frames set to 0, as the method prescribes for them.
"""
import numpy as np
import pytest
import torch

import diffusion_transformer_video_amd as dit
import synth
from gpu_util import need_gpu, note
from oracle import flowception as o_flow

pytestmark = pytest.mark.gpu


def _case(frames_per_seq, tpf, ch, dtype, seed, rate=0.7, passive_every=3):
    r = np.random.default_rng(seed)
    F = int(sum(frames_per_seq))
    z = r.standard_normal((F * tpf, ch)).astype(np.float32)
    t = r.random(F).astype(np.float32)
    counts = r.poisson(rate, size=F).astype(np.int32)
    counts[::passive_every] = 0                      # passive frames block insertions
    noise = r.standard_normal((int(counts.sum()) * tpf, ch)).astype(np.float32)
    if dtype == "bf16":
        z, noise = synth.bf16_round(z), synth.bf16_round(noise)
    cu = (np.concatenate([[0], np.cumsum(frames_per_seq)]) * tpf).astype(np.int32)
    return z, t, cu, counts, noise


def _run(z, t, cu, counts, noise, tpf, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    F, Fo = len(t), len(t) + int(counts.sum())
    zd = torch.from_numpy(z).to(tdt).cuda()
    nd = torch.from_numpy(noise).to(tdt).cuda() if Fo > F else None
    z_out = torch.empty(Fo * tpf, z.shape[1], dtype=tdt, device="cuda")
    t_out = torch.empty(Fo, dtype=torch.float32, device="cuda")
    cu_out = torch.empty(len(cu), dtype=torch.int32, device="cuda")
    src = torch.empty(Fo, dtype=torch.int32, device="cuda")
    dit.flow_insert_frames(z_out, t_out, cu_out, src, zd, torch.from_numpy(t).cuda(),
                           torch.from_numpy(cu).cuda(), torch.from_numpy(counts).cuda(), nd, tpf)
    torch.cuda.synchronize()
    return z_out.float().cpu().numpy(), t_out.cpu().numpy(), cu_out.cpu().numpy(), src.cpu().numpy()


def _check(z, t, cu, counts, noise, tpf, dtype):
    got = _run(z, t, cu, counts, noise, tpf, dtype)
    ref = o_flow.insert_frames(z, t, cu, counts, noise, tpf)
    assert np.array_equal(got[0], ref[0].astype(np.float32)), "latent"
    assert np.array_equal(got[1], ref[1].astype(np.float32)), "local times"
    assert np.array_equal(got[2], ref[2]), "offsets"
    assert np.array_equal(got[3], ref[3]), "source map"
    return got


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_packed_frames_workload(dtype):
    """The packed-frames workload's batch: sequences of 5, 9, 13, 21 frames of
    30 x 52 tokens, 64 latent channels."""
    need_gpu()
    w = synth.C5
    tpf = w.grid_hw[0] * w.grid_hw[1]
    z, t, cu, counts, noise = _case(list(w.frames), tpf, synth.LATENT_CHANNELS, dtype, seed=3)
    got = _check(z, t, cu, counts, noise, tpf, dtype)
    note(f"insert {dtype}: {len(t)} -> {len(got[1])} frames, offsets {got[2].tolist()}")


def test_no_insertions_is_identity():
    need_gpu()
    z, t, cu, counts, noise = _case([3, 4], 16, 64, "bf16", seed=4)
    counts[:] = 0
    got = _check(z, t, cu, counts, noise[:0], 16, "bf16")
    assert np.array_equal(got[0], z)


def test_edges_empty_and_single_frame_sequences():
    """An empty sequence at the start, in the middle and at the end, a
    one-frame sequence, insertions after the last frame of a sequence, a
    frame with many insertions."""
    need_gpu()
    tpf, ch = 7, 16
    fps = [0, 1, 4, 0, 2, 0]
    r = np.random.default_rng(9)
    F = sum(fps)
    z = synth.bf16_round(r.standard_normal((F * tpf, ch)).astype(np.float32))
    t = r.random(F).astype(np.float32)
    counts = np.array([2, 0, 1, 0, 5, 0, 3], dtype=np.int32)   # last frames of sequences insert too
    noise = synth.bf16_round(r.standard_normal((int(counts.sum()) * tpf, ch)).astype(np.float32))
    cu = (np.concatenate([[0], np.cumsum(fps)]) * tpf).astype(np.int32)
    _check(z, t, cu, counts, noise, tpf, "bf16")


def test_many_frames_multiple_scan_chunks():
    """More frames than one pass of the scan block (1024)."""
    need_gpu()
    z, t, cu, counts, noise = _case([700, 1, 1500, 333], 2, 8, "f32", seed=5, rate=1.5)
    _check(z, t, cu, counts, noise, 2, "f32")


def test_counts_inconsistent_with_frames_out_stays_in_bounds():
    """Counts summing to more than frames_out - frames (device data the host
    cannot check): the call stays inside its outputs; frames that fit are
    placed as the oracle places them."""
    need_gpu()
    z, t, cu, counts, noise = _case([4, 5], 8, 16, "bf16", seed=6, rate=2.0)
    short = int(counts.sum()) - 3
    tdt = torch.bfloat16
    F, Fo = len(t), len(t) + short
    z_out = torch.empty(Fo * 8, 16, dtype=tdt, device="cuda")
    t_out = torch.empty(Fo, dtype=torch.float32, device="cuda")
    cu_out = torch.empty(len(cu), dtype=torch.int32, device="cuda")
    src = torch.empty(Fo, dtype=torch.int32, device="cuda")
    dit.flow_insert_frames(z_out, t_out, cu_out, src, torch.from_numpy(z).to(tdt).cuda(),
                           torch.from_numpy(t).cuda(), torch.from_numpy(cu).cuda(),
                           torch.from_numpy(counts).cuda(), torch.from_numpy(noise[:short * 8]).to(tdt).cuda(), 8)
    torch.cuda.synchronize()
    ref = o_flow.insert_frames(z, t, cu, counts, noise, 8)
    assert np.array_equal(src.cpu().numpy(), ref[3][:Fo])


def test_schedule():
    need_gpu()
    r = np.random.default_rng(10)
    t = r.random(1000).astype(np.float32)
    t[:4] = [0.0, 1.0, 1.0 - 1.0 / 64, 0.99]
    td = torch.from_numpy(t).cuda()
    dt = torch.empty_like(td)
    dit.flow_frame_schedule(dt, td, 1.0 / 30)
    torch.cuda.synchronize()
    rdt, rt = o_flow.frame_schedule(t, 1.0 / 30)
    assert np.max(np.abs(dt.cpu().numpy() - rdt)) <= 2e-7
    assert np.max(np.abs(td.cpu().numpy() - rt)) <= 2e-7
    got = td.cpu().numpy()
    assert got[1] == 1.0 and got[2] == 1.0 and got[3] == 1.0   # clipped steps land on exactly 1
    # repeated steps bring every frame to exactly 1 and no further
    for _ in range(40):
        dit.flow_frame_schedule(dt, td, 1.0 / 30)
    torch.cuda.synchronize()
    assert bool((td == 1.0).all()) and bool((dt == 0.0).all())
