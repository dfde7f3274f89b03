"""GPU parity of the bandwidth-bound kernels (modulate, RoPE, gated residual,
Euler) against the float64 oracle, through the C-ABI binding."""
import numpy as np
import pytest
import torch

import diffusion_transformer_video_amd as dit
import synth
from gpu_util import TOL, dev, host64, maxabs, need_gpu, note, sample_rows
from oracle import epilogue as o_epi
from oracle import grid as o_grid
from oracle import modulate as o_mod
from oracle import rope as o_rope

pytestmark = pytest.mark.gpu

SMALL = [
    synth.C1,
    synth.custom("ragged_bf16", "bf16", (3, 5), (3, 1, 2), 3, 64, (16, 24, 24), tokens_per_row=15),
    synth.custom("hd128_bf16", "bf16", (4, 6), (2,), 2, 128, (44, 42, 42)),
    synth.custom("one_token_f32", "f32", (1, 1), (1,), 1, 64, (0, 32, 32)),
]
FULL = [synth.C2, synth.C3, synth.C4, synth.C5]


CHUNK = 8192   # token rows per oracle chunk at full size (bounds host memory)


def _chunks(rows):
    for i in range(0, len(rows), CHUNK):
        yield rows[i:i + CHUNK]


def _modulate_case(w, rows=None):
    """Every element (rows=None), compared chunk by chunk, or the given rows."""
    need_gpu()
    inp = synth.make(w, ["x", "gamma", "beta"])
    x = dev(inp["x"], w)
    y = torch.empty_like(x)
    dit.dit_adaln_modulate(y, x, dev(inp["gamma"]), dev(inp["beta"]), w.tokens_per_row, w.eps)
    torch.cuda.synchronize()
    rows = np.arange(w.tokens, dtype=np.int64) if rows is None else rows
    err = 0.0
    for c in _chunks(rows):
        ref = o_mod.adaln_modulate(inp["x"][c], inp["gamma"][c // w.tokens_per_row],
                                   inp["beta"][c // w.tokens_per_row], 1, w.eps)
        err = max(err, maxabs(host64(y[torch.from_numpy(c).cuda()]), ref))
    note(f"modulate {w.name}: {len(rows)} rows, max-abs {err:.3e}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_modulate_small(w):
    _modulate_case(w)


# wide bf16 rows (2048+ values): parameter rows staged once per block of 8 tokens;
# these also cover a block whose tokens straddle two parameter rows (rows of 15
# tokens), a partial last block (90 tokens), a row width that leaves lanes idle
# (2056 = 257 chunks of 8) and the widest supported row (8192)
WIDE = [
    synth.custom("wide2048_rows15", "bf16", (3, 5), (3, 1, 2), 16, 128, (44, 42, 42), tokens_per_row=15),
    synth.custom("wide2056_ragged", "bf16", (2, 7), (3,), 257, 8, (4, 2, 2), tokens_per_row=7),
    synth.custom("wide8192", "bf16", (4, 5), (2,), 64, 128, (44, 42, 42), tokens_per_row=20),
]


@pytest.mark.parametrize("w", WIDE, ids=lambda w: w.name)
def test_modulate_wide(w):
    _modulate_case(w)


# 16K+ wide bf16 rows: each row split over two waves, 8 rows per block; a ragged
# last block (16,389 rows), a width whose halves differ (257 chunks: 129 + 128),
# blocks straddling parameter rows (9 and 20 tokens per row), the widest row
WIDE_MANY = [
    synth.custom("pairs2056_ragged", "bf16", (27, 607), (1,), 257, 8, (4, 2, 2), tokens_per_row=9),
    synth.custom("pairs8192_rows20", "bf16", (41, 400), (1,), 64, 128, (44, 42, 42), tokens_per_row=20),
]


@pytest.mark.parametrize("w", WIDE_MANY, ids=lambda w: w.name)
def test_modulate_wide_many_rows(w):
    _modulate_case(w, sample_rows(w, per_seq=2048, edge=64))


@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
def test_modulate_full(w):
    _modulate_case(w)


def _rope_case(w, rows=None):
    need_gpu()
    inp = synth.make(w, ["q", "k"])
    q, k = dev(inp["q"], w), dev(inp["k"], w)
    pos = torch.full((w.tokens, 3), -1, dtype=torch.int32, device="cuda")
    cu = None if w.dense else torch.from_numpy(w.cu_seqlens).cuda()
    dit.dit_rope3d(q, k, (w.frames[0], *w.grid_hw), w.rope_split, w.rope_base,
                   cu_seqlens=cu, num_seqs=w.num_seqs, pos_out=pos)
    torch.cuda.synchronize()
    ref_pos = o_grid.positions(w.cu_seqlens, *w.grid_hw)
    assert np.array_equal(pos.cpu().numpy().astype(np.int64), ref_pos), "position ids differ"
    rows = np.arange(w.tokens, dtype=np.int64) if rows is None else rows
    eq = ek = 0.0
    for c in _chunks(rows):
        rt = torch.from_numpy(c).cuda()
        eq = max(eq, maxabs(host64(q[rt]), o_rope.apply_rope(inp["q"][c], ref_pos[c], w.rope_split, w.rope_base)))
        ek = max(ek, maxabs(host64(k[rt]), o_rope.apply_rope(inp["k"][c], ref_pos[c], w.rope_split, w.rope_base)))
    note(f"rope {w.name}: {len(rows)} rows, max-abs q {eq:.3e} k {ek:.3e}")
    assert eq <= TOL[w.dtype] and ek <= TOL[w.dtype]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_rope_small(w):
    _rope_case(w)


@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
def test_rope_full(w):
    _rope_case(w)


def test_rope_origin_is_identity_and_v_untouched():
    need_gpu()
    w = synth.custom("origin", "bf16", (1, 1), (1,), 4, 128, (44, 42, 42))
    inp = synth.make(w, ["q", "k"])
    q, k = dev(inp["q"], w), dev(inp["k"], w)
    dit.dit_rope3d(q, k, (1, 1, 1), w.rope_split)
    torch.cuda.synchronize()
    assert torch.equal(q.cpu(), dev(inp["q"], w).cpu()) and torch.equal(k.cpu(), dev(inp["k"], w).cpu())


def test_rope_relative_position_on_gpu():
    """Same q0 / k0 at every token: after rotation the score between tokens a, b
    depends only on their 3D offset (checked within bf16 rounding)."""
    need_gpu()
    w = synth.custom("relpos", "f32", (4, 5), (3,), 1, 64, (16, 24, 24))
    r = np.random.default_rng(5)
    q0 = r.standard_normal(64).astype(np.float32)
    k0 = r.standard_normal(64).astype(np.float32)
    q = dev(np.broadcast_to(q0, (w.tokens, 1, 64)).copy(), w)
    k = dev(np.broadcast_to(k0, (w.tokens, 1, 64)).copy(), w)
    dit.dit_rope3d(q, k, (3, 4, 5), w.rope_split)
    torch.cuda.synchronize()
    s = host64(q)[:, 0, :] @ host64(k)[:, 0, :].T
    pos = o_grid.positions(w.cu_seqlens, 4, 5)
    off = {}
    for a in range(w.tokens):
        for b in range(w.tokens):
            key = tuple(pos[b] - pos[a])
            if key in off:
                assert abs(s[a, b] - off[key]) < 1e-4
            else:
                off[key] = s[a, b]


def _epilogue_case(w, fused):
    need_gpu()
    inp = synth.make(w, ["x", "alpha", "z", "u", "dt"])
    br_np = synth.make(w, ["v"])["v"].reshape(w.tokens, w.d_model)  # stands in for the attention output
    x, br = dev(inp["x"], w), dev(br_np, w)
    z, u = dev(inp["z"], w), dev(inp["u"], w)
    dt = dev(inp["dt"])
    x_out = torch.empty_like(x)
    z_out = torch.empty_like(z)
    if fused:
        dit.dit_gated_residual(x_out, x, br, dev(inp["alpha"]), w.tokens_per_row,
                               euler=(z_out, z, u, dt, w.tokens_per_row))
    else:
        dit.dit_gated_residual(x_out, x, br, dev(inp["alpha"]), w.tokens_per_row)
        dit.rf_euler_step(z_out, z, u, dt, w.tokens_per_row)
    torch.cuda.synchronize()
    rx = o_epi.gated_residual(inp["x"], br_np, inp["alpha"], w.tokens_per_row)
    rz = o_epi.euler_step(inp["z"], inp["u"], inp["dt"], w.tokens_per_row)
    ex, ez = maxabs(host64(x_out), rx), maxabs(host64(z_out), rz)
    note(f"epilogue {w.name} fused={fused}: residual {ex:.3e} euler {ez:.3e}")
    assert ex <= TOL[w.dtype] and ez <= TOL[w.dtype]


@pytest.mark.parametrize("w", SMALL + FULL, ids=lambda w: w.name)
def test_epilogue_fused(w):
    _epilogue_case(w, True)


@pytest.mark.parametrize("w", [synth.C1, synth.C5, SMALL[1]], ids=lambda w: w.name)
def test_epilogue_separate(w):
    _epilogue_case(w, False)


def test_alpha_zero_is_identity_and_dt_zero_is_identity():
    need_gpu()
    w = synth.C2
    inp = synth.make(w, ["x", "z", "u"])
    x = dev(inp["x"], w)
    br = torch.randn_like(x)
    x_out = torch.empty_like(x)
    z = dev(inp["z"], w)
    z_out = torch.empty_like(z)
    dit.dit_gated_residual(x_out, x, br, torch.zeros(w.rows, w.d_model, device="cuda"), w.tokens_per_row,
                           euler=(z_out, z, dev(inp["u"], w), torch.zeros(w.rows, device="cuda"),
                                  w.tokens_per_row))
    torch.cuda.synchronize()
    assert torch.equal(x_out, x) and torch.equal(z_out, z)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_euler_exact_landing(dtype):
    """One Euler step of size 1 from x0 with u = x1 - x0 lands exactly on x1 when
    the values sit on a dyadic grid (so u is exact in the storage type)."""
    need_gpu()
    w = synth.custom("dyadic", dtype, (30, 52), (5, 9), 1, 64, (0, 32, 32), tokens_per_row=1560)
    x0 = synth.dyadic(w, "x0", (w.tokens, 64))
    x1 = synth.dyadic(w, "x1", (w.tokens, 64))
    u = (x1.astype(np.float64) - x0).astype(np.float32)
    z = dev(x0, w)
    dit.rf_euler_step(z, z, dev(u, w), torch.ones(w.rows, device="cuda"), w.tokens_per_row)
    torch.cuda.synchronize()
    assert np.array_equal(host64(z), x1.astype(np.float64))


def test_euler_per_frame_lands_on_data():
    """Frames at local time t_f step by 1 - t_f along u = x1 - x0 and reach x1."""
    need_gpu()
    w = synth.custom("perframe", "f32", (30, 52), (5,), 1, 64, (0, 32, 32), tokens_per_row=1560,
                     per_frame_time=True)
    x0 = synth.make(w, ["x0"])["x0"]
    x1 = synth.make(w, ["x1"])["x1"]
    t = synth.flow_times(w).astype(np.float64)
    xt = o_epi.interpolant(x0, x1, np.repeat(t, 1560)).astype(np.float32)
    u = (x1.astype(np.float64) - x0).astype(np.float32)
    z = dev(xt, w)
    dit.rf_euler_step(z, z, dev(u, w), dev((1.0 - t).astype(np.float32)), 1560)
    torch.cuda.synchronize()
    assert maxabs(host64(z), x1) <= 1e-4


# ---- every kernel writes exactly its outputs (guard bands of canary values
# around them keep their values) and is deterministic (a second run on the same
# inputs gives the same bits): modulate, RoPE, the fused epilogue
def _guarded(shape, dtype, fill=7.0, pad=4096):
    """A tensor of `shape` inside a flat buffer with `pad` canary elements on each side."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * pad,), fill, dtype=dtype, device="cuda")
    return buf, buf[pad:pad + n].view(shape), pad


def _canaries_ok(buf, pad, fill=7.0):
    return bool(torch.all(buf[:pad] == fill)) and bool(torch.all(buf[-pad:] == fill))


GUARD = [synth.C1, SMALL[1], synth.custom("guard_wide", "bf16", (5, 9), (3, 2), 24, 128, (44, 42, 42),
                                          tokens_per_row=45)]


@pytest.mark.parametrize("w", GUARD, ids=lambda w: w.name)
def test_modulate_guard_and_determinism(w):
    need_gpu()
    inp = synth.make(w, ["x", "gamma", "beta"])
    x = dev(inp["x"], w)
    outs = []
    for _ in range(2):
        buf, y, pad = _guarded(x.shape, x.dtype)
        dit.dit_adaln_modulate(y, x, dev(inp["gamma"]), dev(inp["beta"]), w.tokens_per_row, w.eps)
        torch.cuda.synchronize()
        assert _canaries_ok(buf, pad)
        outs.append(y.clone())
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("w", GUARD, ids=lambda w: w.name)
def test_rope_guard_and_determinism(w):
    need_gpu()
    inp = synth.make(w, ["q", "k"])
    cu = None if w.dense else torch.from_numpy(w.cu_seqlens).cuda()
    outs = []
    for _ in range(2):
        bq, q, pad = _guarded(inp["q"].shape, torch.bfloat16 if w.dtype == "bf16" else torch.float32)
        bk, k, _ = _guarded(inp["k"].shape, q.dtype)
        q.copy_(dev(inp["q"], w))
        k.copy_(dev(inp["k"], w))
        bp, pos, _ = _guarded((w.tokens, 3), torch.int32, fill=-7)
        dit.dit_rope3d(q, k, (w.frames[0], *w.grid_hw), w.rope_split, w.rope_base, cu_seqlens=cu,
                       num_seqs=w.num_seqs, pos_out=pos)
        torch.cuda.synchronize()
        assert _canaries_ok(bq, pad) and _canaries_ok(bk, pad) and _canaries_ok(bp, pad, -7)
        outs.append((q.clone(), k.clone(), pos.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("w", GUARD, ids=lambda w: w.name)
def test_epilogue_guard_and_determinism(w):
    need_gpu()
    inp = synth.make(w, ["x", "alpha", "z", "u", "dt"])
    br = dev(synth.make(w, ["v"])["v"].reshape(w.tokens, w.d_model), w)
    x, z, u = dev(inp["x"], w), dev(inp["z"], w), dev(inp["u"], w)
    outs = []
    for _ in range(2):
        bx, x_out, pad = _guarded(x.shape, x.dtype)
        bz, z_out, _ = _guarded(z.shape, z.dtype)
        dit.dit_gated_residual(x_out, x, br, dev(inp["alpha"]), w.tokens_per_row,
                               euler=(z_out, z, u, dev(inp["dt"]), w.tokens_per_row))
        torch.cuda.synchronize()
        assert _canaries_ok(bx, pad) and _canaries_ok(bz, pad)
        outs.append((x_out.clone(), z_out.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
