"""Pins for the oracle: checks against what the pages and the mathematics fix.

Each pin takes an ``impl`` namespace holding the functions under test, so the
same checks run on the real oracle (tests/test_oracle_pins.py) and on copies
with a planted mistake (tests/test_oracle_mutations.py), which must fail at
least one pin. Nothing here retypes an oracle formula: the references are
closed forms, invariants, torch CPU float64 library routines, brute-force
loops written differently, and the pages' worked numbers.
"""
from __future__ import annotations

import cmath
import json
import math
import os
import types

import numpy as np
import torch

import oracle
from oracle import attention as o_attn
from oracle import epilogue as o_epi
from oracle import flowception as o_flow
from oracle import fp8 as o_fp8
from oracle import grid as o_grid
from oracle import modulate as o_mod
from oracle import rope as o_rope

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def real_impl():
    return types.SimpleNamespace(
        num_tokens=o_grid.num_tokens, coords=o_grid.coords, token_of=o_grid.token_of,
        positions=o_grid.positions, coords_bruteforce=o_grid.coords_bruteforce,
        layer_norm=o_mod.layer_norm, adaln_modulate=o_mod.adaln_modulate,
        apply_rope=o_rope.apply_rope,
        attention=o_attn.attention, attention_bruteforce=o_attn.attention_bruteforce,
        attention_lse=o_attn.attention_lse, merge=o_attn.merge,
        gated_residual=o_epi.gated_residual, euler_step=o_epi.euler_step,
        interpolant=o_epi.interpolant, velocity=o_epi.velocity,
        interpolant_rows=o_epi.interpolant_rows, cfm_loss=o_epi.cfm_loss, midpoint_half=o_epi.midpoint_half,
        insert_frames=o_flow.insert_frames, frame_schedule=o_flow.frame_schedule,
        e4m3_encode=o_fp8.e4m3_encode, e4m3_decode=o_fp8.e4m3_decode, quantize_per_head=o_fp8.quantize_per_head,
        dequantize=o_fp8.dequantize, quantize_qkv=o_fp8.quantize_qkv,
    )


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- grid
def pin_grid_bruteforce(impl):
    for (T, H, W) in [(2, 4, 4), (1, 64, 64), (21, 30, 52), (5, 3, 7), (1, 1, 1)]:
        bf = impl.coords_bruteforce(T, H, W)
        cf = impl.coords(np.arange(T * H * W), H, W)
        assert np.array_equal(bf, cf), (T, H, W)
        assert np.array_equal(impl.token_of(cf, H, W), np.arange(T * H * W))


def pin_grid_worked_counts(impl):
    g = json.load(open(os.path.join(GOLDEN, "worked_counts.json")))
    vae = g["vae_latent_720p_5s"]
    lat = [vae["frames"] // vae["factor_t"], vae["height"] // vae["factor_h"],
           vae["width"] // vae["factor_w"]]
    assert lat == vae["latent"]
    assert impl.num_tokens(vae["frames"], vae["height"], vae["width"], vae["factor_t"],
                           vae["factor_h"], vae["factor_w"]) == 30 * 90 * 160
    tk = g["tokens_30x90x160_patch2x2"]
    assert impl.num_tokens(*tk["latent"], *tk["patch"]) == tk["tokens"]
    assert tk["tokens"] // tk["gpus"] == tk["tokens_per_gpu"]
    assert tk["heads"] // tk["gpus"] == tk["heads_per_gpu"]
    px = g["pixel_values_720p_5s"]
    assert 120 * 3 * 720 * 1280 == px["product"] > px["lower_bound"]


def pin_grid_workload_counts(impl):
    import synth
    # latent (T, H, W) and patch per workload, from the workload definitions
    lat = {"c1_tiny_f32": ((2, 8, 8), (1, 2, 2)),
           "c2_image_4096_bf16": ((1, 128, 128), (1, 2, 2)),
           "c3_video480p_32760_bf16": ((21, 60, 104), (1, 2, 2)),
           "c4_video720p_27280_bf16": ((31, 44, 80), (1, 2, 2))}
    for name, (L, P) in lat.items():
        w = synth.WORKLOADS[name]
        assert impl.num_tokens(*L, *P) == w.seqlens[0], name
    w5 = synth.WORKLOADS["c5_varlen_frames_bf16"]
    for f, n in zip(w5.frames, w5.seqlens):
        assert impl.num_tokens(f, 60, 104, 1, 2, 2) == n


def pin_grid_varlen_restart(impl):
    cu = np.array([0, 12, 12 + 20, 12 + 20 + 4])
    pos = impl.positions(cu, 2, 2)
    assert np.array_equal(pos[0], [0, 0, 0]) and np.array_equal(pos[12], [0, 0, 0])
    assert np.array_equal(pos[32], [0, 0, 0])
    assert np.array_equal(pos[11], [2, 1, 1]) and np.array_equal(pos[31], [4, 1, 1])


# ---------------------------------------------------------------- modulate
def pin_modulate_gamma0(impl):
    r = _rng(1)
    x = r.standard_normal((9, 48))
    g = np.zeros((3, 48))
    b = r.standard_normal((3, 48))
    y = impl.adaln_modulate(x, g, b, 3, 1e-6)
    assert np.array_equal(y, b[np.arange(9) // 3])


def pin_modulate_moments(impl):
    r = _rng(2)
    x = r.standard_normal((7, 64)) * 0.01 + 3.0  # small variance: eps matters
    eps = 1e-6
    y = impl.adaln_modulate(x, np.ones((1, 64)), np.zeros((1, 64)), 7, eps)
    var_pop = x.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0.0, atol=1e-12)
    assert np.allclose(y.var(axis=1), var_pop / (var_pop + eps), rtol=1e-12, atol=0)


def pin_modulate_constant_row(impl):
    x = np.full((4, 32), 0.75)
    r = _rng(3)
    g = r.standard_normal((1, 32))
    b = r.standard_normal((1, 32))
    y = impl.adaln_modulate(x, g, b, 4, 1e-6)
    assert np.array_equal(y, np.broadcast_to(b, (4, 32)))


def pin_modulate_library(impl):
    r = _rng(4)
    x = r.standard_normal((12, 96))
    g = r.standard_normal((3, 96))
    b = r.standard_normal((3, 96))
    y = impl.adaln_modulate(x, g, b, 4, 1e-6)
    ln = torch.nn.functional.layer_norm(torch.from_numpy(x), (96,), eps=1e-6).numpy()
    ref = ln * np.repeat(g, 4, axis=0) + np.repeat(b, 4, axis=0)
    assert np.allclose(y, ref, rtol=0, atol=1e-12)


def pin_modulate_bruteforce(impl):
    r = _rng(5)
    x = r.standard_normal((3, 10))
    g = r.standard_normal((3, 10))
    b = r.standard_normal((3, 10))
    y = impl.adaln_modulate(x, g, b, 1, 1e-5)
    for i in range(3):
        row = [float(v) for v in x[i]]
        m = math.fsum(row) / len(row)
        var = math.fsum((v - m) ** 2 for v in row) / len(row)
        for c in range(10):
            ref = g[i, c] * (row[c] - m) / math.sqrt(var + 1e-5) + b[i, c]
            assert abs(y[i, c] - ref) < 1e-12


# ---------------------------------------------------------------- rope
SPLIT = (16, 24, 24)


def pin_rope_origin_identity(impl):
    r = _rng(6)
    x = r.standard_normal((3, 2, 64))
    y = impl.apply_rope(x, np.zeros((3, 3)), SPLIT, 10000.0)
    assert np.array_equal(y, x)


def pin_rope_pair_norms(impl):
    r = _rng(7)
    x = r.standard_normal((20, 3, 64))
    pos = r.integers(0, 50, size=(20, 3))
    y = impl.apply_rope(x, pos, SPLIT, 10000.0)
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.allclose(nx, ny, rtol=1e-12, atol=1e-12)


def _rope1d_textbook(vec, pos, d, base):
    """Text RoPE on one d-wide vector: pair j as a complex number turned by
    pos / base^(2j/d)."""
    out = []
    for j in range(d // 2):
        zc = complex(vec[2 * j], vec[2 * j + 1]) * cmath.exp(1j * pos / (base ** (2 * j / d)))
        out += [zc.real, zc.imag]
    return out


def pin_rope_axis_special_cases(impl):
    r = _rng(8)
    base = 10000.0
    offs = (0, SPLIT[0], SPLIT[0] + SPLIT[1])
    for axis in range(3):
        for p in (1, 5, 37):
            pos = np.zeros((1, 3))
            pos[0, axis] = p
            x = r.standard_normal((1, 1, 64))
            y = impl.apply_rope(x, pos, SPLIT, base)
            lo, hi = offs[axis], offs[axis] + SPLIT[axis]
            ref = _rope1d_textbook(x[0, 0, lo:hi], p, SPLIT[axis], base)
            assert np.allclose(y[0, 0, lo:hi], ref, rtol=0, atol=1e-12)
            rest = np.r_[0:lo, hi:64]
            assert np.array_equal(y[0, 0, rest], x[0, 0, rest])


def pin_rope_relative(impl):
    r = _rng(9)
    base = 10000.0
    q = r.standard_normal((1, 1, 64))
    k = r.standard_normal((1, 1, 64))
    for _ in range(5):
        p = r.integers(0, 30, size=3).astype(float)
        pp = r.integers(0, 30, size=3).astype(float)
        sh = r.integers(-10, 40, size=3).astype(float)
        a = (impl.apply_rope(q, p[None], SPLIT, base) * impl.apply_rope(k, pp[None], SPLIT, base)).sum()
        b = (impl.apply_rope(q, (p + sh)[None], SPLIT, base) *
             impl.apply_rope(k, (pp + sh)[None], SPLIT, base)).sum()
        assert abs(a - b) < 1e-10


def pin_rope_composition(impl):
    r = _rng(10)
    x = r.standard_normal((4, 2, 64))
    p1 = r.integers(0, 20, size=(4, 3))
    p2 = r.integers(0, 20, size=(4, 3))
    y = impl.apply_rope(impl.apply_rope(x, p1, SPLIT, 500.0), p2, SPLIT, 500.0)
    z = impl.apply_rope(x, p1 + p2, SPLIT, 500.0)
    assert np.allclose(y, z, rtol=0, atol=1e-11)


# ---------------------------------------------------------------- attention
def _qkv(seed, n, h=2, d=16, scale=1.0):
    r = _rng(seed)
    return [r.standard_normal((n, h, d)) * scale for _ in range(3)]


def pin_attn_ones(impl):
    q, k, _ = _qkv(11, 37)
    v = np.ones_like(q)
    o = impl.attention(q, k, v, [0, 37])
    assert np.allclose(o, 1.0, rtol=0, atol=1e-12)


def pin_attn_identical_keys(impl):
    q, k, v = _qkv(12, 29)
    k[:] = k[0:1]
    o = impl.attention(q, k, v, [0, 29])
    assert np.allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=1e-12)


def pin_attn_zero_query(impl):
    _, k, v = _qkv(13, 23)
    q = np.zeros_like(k)
    o = impl.attention(q, k, v, [0, 23])
    assert np.allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=1e-12)


def pin_attn_single_token(impl):
    q, k, v = _qkv(14, 1)
    o = impl.attention(q, k, v, [0, 1])
    assert np.allclose(o, v, atol=1e-14)


def pin_attn_dominant_key(impl):
    q, k, v = _qkv(15, 19)
    j = 7
    q[:] = 40.0 * k[j][None] / np.linalg.norm(k[j], axis=-1, keepdims=True)[None]
    o = impl.attention(q, k, v, [0, 19])
    # scores for key j exceed the rest by a wide margin -> output is V_j
    assert np.allclose(o, np.broadcast_to(v[j], o.shape), atol=1e-3)


def pin_attn_permutation(impl):
    q, k, v = _qkv(16, 31)
    perm = _rng(17).permutation(31)
    o = impl.attention(q, k, v, [0, 31])
    o_p = impl.attention(q[perm], k[perm], v[perm], [0, 31])
    assert np.allclose(o_p, o[perm], atol=1e-12)
    o_kv = impl.attention(q, k[perm], v[perm], [0, 31])
    assert np.allclose(o_kv, o, atol=1e-12)


def pin_attn_varlen_blocks(impl):
    q, k, v = _qkv(18, 40)
    cu = [0, 9, 9 + 17, 40]
    o = impl.attention(q, k, v, cu)
    for s in range(3):
        lo, hi = cu[s], cu[s + 1]
        oi = impl.attention(q[lo:hi], k[lo:hi], v[lo:hi], [0, hi - lo])
        assert np.allclose(o[lo:hi], oi, atol=1e-13)


def pin_attn_library(impl):
    q, k, v = _qkv(19, 45, h=3, d=32, scale=1.5)
    o = impl.attention(q, k, v, [0, 45])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))  # [h, n, d]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v)).numpy()
    assert np.allclose(o, ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def pin_attn_bruteforce(impl):
    q, k, v = _qkv(20, 11, h=2, d=8)
    cu = [0, 4, 11]
    o = impl.attention(q, k, v, cu)
    ref = np.array(impl.attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), cu))
    assert np.allclose(o, ref, atol=1e-12)


def pin_attn_row_subset(impl):
    q, k, v = _qkv(21, 50)
    cu = [0, 20, 50]
    rows = np.array([0, 3, 19, 20, 33, 49])
    full = impl.attention(q, k, v, cu)
    sub = impl.attention(q, k, v, cu, rows=rows)
    assert np.allclose(sub, full[rows], atol=1e-14)


# ---------------------------------------------------------------- epilogue
# ------------------------------------------------- attention LSE and merge
def pin_lse_zero_query(impl):
    """q = 0: every score is 0, so lse = ln(number of keys) and o = mean(V)."""
    _, k, v = _qkv(31, 23)
    q = np.zeros((5, 2, 16))
    o, lse = impl.attention_lse(q, k, v, [0, 5], [0, 23])
    assert np.allclose(lse, math.log(23), rtol=0, atol=1e-12)
    assert np.allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=1e-12)


def pin_lse_single_key(impl):
    """One key: lse is that key's score q.k / sqrt(d) and o is its value."""
    q, k, v = _qkv(32, 6)
    o, lse = impl.attention_lse(q, k[:1], v[:1], [0, 6], [0, 1])
    ref = np.einsum("nhd,hd->nh", q, k[0]) / 4.0   # sqrt(16)
    assert np.allclose(lse, ref, rtol=0, atol=1e-12)
    assert np.allclose(o, np.broadcast_to(v[0], o.shape), atol=1e-12)


def pin_lse_identical_keys(impl):
    """N identical keys: lse = score + ln N."""
    q, k, v = _qkv(33, 11)
    k[:] = k[0:1]
    _, lse = impl.attention_lse(q, k, v, [0, 11], [0, 11])
    ref = np.einsum("nhd,hd->nh", q, k[0]) / 4.0 + math.log(11)
    assert np.allclose(lse, ref, rtol=0, atol=1e-12)


def pin_lse_library(impl):
    """lse and o against torch's CPU float64 logsumexp / softmax on the scores,
    with query and key sets of different sizes and a large score offset."""
    r = _rng(34)
    q = r.standard_normal((7, 3, 16)) * 6.0
    k = r.standard_normal((19, 3, 16)) * 6.0
    v = r.standard_normal((19, 3, 16))
    o, lse = impl.attention_lse(q, k, v, [0, 7], [0, 19])
    S = torch.einsum("qhd,khd->hqk", torch.from_numpy(q), torch.from_numpy(k)) / 4.0
    ref_lse = torch.logsumexp(S, dim=-1).T.numpy()
    ref_o = torch.einsum("hqk,khd->qhd", torch.softmax(S, dim=-1), torch.from_numpy(v)).numpy()
    assert np.allclose(lse, ref_lse, rtol=0, atol=1e-10)
    assert np.allclose(o, ref_o, rtol=0, atol=1e-12)


def pin_lse_empty_keys(impl):
    """A sequence whose key set is empty: lse = -inf, o = 0; others unaffected."""
    q, k, v = _qkv(35, 9)
    o, lse = impl.attention_lse(q, k, v, [0, 4, 9], [0, 0, 9])
    assert np.all(np.isneginf(lse[:4])) and np.all(o[:4] == 0.0)
    o2, lse2 = impl.attention_lse(q[4:], k, v, [0, 5], [0, 9])
    assert np.allclose(o[4:], o2, atol=1e-14) and np.allclose(lse[4:], lse2, atol=1e-14)


def pin_lse_matches_softmax_attention(impl):
    """With each sequence's queries and keys the same token set, o is the
    attention of the block (and lse is finite)."""
    q, k, v = _qkv(36, 30)
    cu = [0, 12, 30]
    o, lse = impl.attention_lse(q, k, v, cu, cu)
    assert np.allclose(o, impl.attention(q, k, v, cu), atol=1e-12)
    assert np.all(np.isfinite(lse))


def pin_merge_split_equals_full(impl):
    """Attention over a key set equals the merge of the attentions over any
    split of it into two disjoint parts (the ring / context-parallel identity),
    for several sequences with different split points."""
    r = _rng(37)
    q = r.standard_normal((10, 2, 16)) * 2.0
    k = r.standard_normal((15, 2, 16)) * 2.0
    v = r.standard_normal((15, 2, 16))
    cq, ck = [0, 4, 10], [0, 7, 15]
    o, lse = impl.attention_lse(q, k, v, cq, ck)
    i1, i2 = np.r_[0:2, 7:13], np.r_[2:7, 13:15]
    o1, l1 = impl.attention_lse(q, k[i1], v[i1], cq, [0, 2, 8])
    o2, l2 = impl.attention_lse(q, k[i2], v[i2], cq, [0, 5, 7])
    om, lm = impl.merge(o1, l1, o2, l2)
    assert np.allclose(om, o, rtol=0, atol=1e-12) and np.allclose(lm, lse, rtol=0, atol=1e-12)
    om, lm = impl.merge(o2, l2, o1, l1)   # order does not matter
    assert np.allclose(om, o, rtol=0, atol=1e-12) and np.allclose(lm, lse, rtol=0, atol=1e-12)


def pin_merge_empty_identity(impl):
    """Merging with an empty partial (lse = -inf) leaves a partial unchanged;
    two empty partials stay empty (o = 0, lse = -inf)."""
    r = _rng(38)
    o = r.standard_normal((6, 2, 16))
    lse = r.standard_normal((6, 2)) * 3.0
    zo, zl = np.zeros_like(o), np.full_like(lse, -np.inf)
    om, lm = impl.merge(o, lse, zo, zl)
    assert np.allclose(om, o, atol=1e-15) and np.array_equal(lm, lse)
    om, lm = impl.merge(zo, zl, zo, zl)
    assert np.all(om == 0.0) and np.all(np.isneginf(lm))


def pin_merge_weights_bruteforce(impl):
    """Merge against a per-element loop that re-weights each partial by its share
    of the joint exponential sum, computed as exp(l_a) / (exp(l_a) + exp(l_b))
    on moderate values (no overflow)."""
    r = _rng(39)
    oa, ob = r.standard_normal((3, 2, 4)), r.standard_normal((3, 2, 4))
    la, lb = r.standard_normal((3, 2)), r.standard_normal((3, 2))
    om, lm = impl.merge(oa, la, ob, lb)
    for i in range(3):
        for h in range(2):
            ea, eb = math.exp(la[i, h]), math.exp(lb[i, h])
            assert abs(lm[i, h] - math.log(ea + eb)) < 1e-13
            for d in range(4):
                ref = (ea * oa[i, h, d] + eb * ob[i, h, d]) / (ea + eb)
                assert abs(om[i, h, d] - ref) < 1e-13


def pin_residual_alpha0(impl):
    r = _rng(22)
    x = r.standard_normal((6, 32))
    br = r.standard_normal((6, 2, 16))
    y = impl.gated_residual(x, br, np.zeros((2, 32)), 3)
    assert np.array_equal(y, x)


def pin_residual_bruteforce(impl):
    r = _rng(23)
    x = r.standard_normal((4, 6))
    br = r.standard_normal((4, 2, 3))
    a = r.standard_normal((2, 6))
    y = impl.gated_residual(x, br, a, 2)
    for t in range(4):
        for h in range(2):
            for i in range(3):
                c = h * 3 + i
                assert abs(y[t, c] - (x[t, c] + a[t // 2, c] * br[t, h, i])) < 1e-15


def pin_euler_dt0(impl):
    r = _rng(24)
    z = r.standard_normal((5, 64))
    u = r.standard_normal((5, 64))
    assert np.array_equal(impl.euler_step(z, u, np.zeros(5), 1), z)


def pin_euler_exact_landing(impl):
    r = _rng(25)
    step = 1.0 / 16.0
    x0 = r.integers(-64, 65, size=(8, 64)) * step
    x1 = r.integers(-64, 65, size=(8, 64)) * step
    # the page's straight path: x_t at t = 0 is the noise, its velocity is x1 - x0
    assert np.array_equal(impl.interpolant(x0, x1, np.zeros(8)), x0)
    assert np.array_equal(impl.interpolant(x0, x1, np.ones(8)), x1)
    u = impl.velocity(x0, x1)
    assert np.array_equal(impl.euler_step(x0, u, np.ones(8), 1), x1)


def pin_euler_per_frame(impl):
    r = _rng(26)
    x0 = r.standard_normal((12, 64))
    x1 = r.standard_normal((12, 64))
    t = r.random(4)  # 4 frames of 3 tokens
    xt = impl.interpolant(x0, x1, np.repeat(t, 3))
    y = impl.euler_step(xt, impl.velocity(x0, x1), 1.0 - t, 3)
    assert np.allclose(y, x1, rtol=0, atol=1e-12)
    # a direction check: a small step moves toward x1 along the path
    xs = impl.euler_step(xt, impl.velocity(x0, x1), np.full(4, 0.01), 3)
    assert np.allclose(xs, impl.interpolant(x0, x1, np.repeat(t + 0.01, 3)), atol=1e-12)


def pin_euler_30_steps(impl):
    r = _rng(27)
    x0 = r.standard_normal((3, 64))
    x1 = r.standard_normal((3, 64))
    u = impl.velocity(x0, x1)
    z = x0.copy()
    for _ in range(30):
        z = impl.euler_step(z, u, np.full(3, 1.0 / 30.0), 1)
    assert np.allclose(z, x1, rtol=0, atol=1e-12)


# ------------------------------------------------ CFM loss, midpoint sampler
def pin_interpolant_rows_endpoints(impl):
    """t = 0 gives the noise, t = 1 the data, t = 1/2 the average, per row."""
    r = _rng(50)
    x0, x1 = r.standard_normal((12, 8)), r.standard_normal((12, 8))
    xt = impl.interpolant_rows(x0, x1, np.array([0.0, 1.0, 0.5]), 4)
    assert np.array_equal(xt[:4], x0[:4]) and np.array_equal(xt[4:8], x1[4:8])
    assert np.allclose(xt[8:], (x0[8:] + x1[8:]) / 2, atol=1e-15)


def pin_cfm_exact_velocity_zero(impl):
    """The path's own velocity has zero loss, exactly."""
    r = _rng(51)
    x0, x1 = r.standard_normal((10, 16)), r.standard_normal((10, 16))
    per_tok, per_row = impl.cfm_loss(x1 - x0, x0, x1, 5)
    assert np.all(per_tok == 0.0) and np.all(per_row == 0.0)


def pin_cfm_bruteforce(impl):
    """Per-token and per-row sums against loops over (token, channel)."""
    r = _rng(52)
    u, x0, x1 = (r.standard_normal((9, 5)) for _ in range(3))
    per_tok, per_row = impl.cfm_loss(u, x0, x1, 3)
    for tok in range(9):
        acc = 0.0
        for c in range(5):
            d = u[tok, c] - x1[tok, c] + x0[tok, c]
            acc += d * d
        assert abs(per_tok[tok] - acc) < 1e-12
    for row in range(3):
        assert abs(per_row[row] - sum(per_tok[3 * row + i] for i in range(3))) < 1e-12
    assert per_row.shape == (3,)


def pin_cfm_translation_and_scale(impl):
    """Shifting noise and data together leaves the loss unchanged; doubling the
    velocity error quadruples it."""
    r = _rng(53)
    x0, x1, e = (r.standard_normal((6, 4)) for _ in range(3))
    _, a = impl.cfm_loss(x1 - x0 + e, x0, x1, 3)
    _, b = impl.cfm_loss(x1 - x0 + e, x0 + 7.0, x1 + 7.0, 3)
    _, c = impl.cfm_loss(x1 - x0 + 2 * e, x0, x1, 3)
    assert np.allclose(a, b, rtol=1e-12) and np.allclose(c, 4 * a, rtol=1e-12)


def _midpoint_solve(impl, z0, lam, n):
    """Integrate dz/dt = lam(t) z on [0, 1] with n explicit-midpoint steps."""
    dt = 1.0 / n
    z = z0.copy()
    for i in range(n):
        t = i * dt
        zm = impl.midpoint_half(z, lam(t) * z, np.array([dt]), len(z))
        z = impl.euler_step(z, lam(t + dt / 2) * zm, np.array([dt]), len(z))
    return z


def pin_midpoint_second_order(impl):
    """On dz/dt = lam(t) z (closed form z0 exp(int lam)) the midpoint sampler's
    error falls 4x when the step halves (second order; Euler's falls 2x)."""
    lam = lambda t: math.cos(3.0 * t) - 0.5
    z0 = np.array([[1.0, -2.0], [0.5, 3.0]])
    exact = z0 * math.exp(math.sin(3.0) / 3.0 - 0.5)
    e1 = np.abs(_midpoint_solve(impl, z0, lam, 32) - exact).max()
    e2 = np.abs(_midpoint_solve(impl, z0, lam, 64) - exact).max()
    assert 3.5 < e1 / e2 < 4.5, e1 / e2


def pin_midpoint_straight_path(impl):
    """Constant velocity x1 - x0 (the straight path): one midpoint step of size
    1 from the noise lands on the data; the half stage stops at the middle."""
    r = _rng(54)
    x0, x1 = r.standard_normal((6, 4)), r.standard_normal((6, 4))
    u = x1 - x0
    zm = impl.midpoint_half(x0, u, np.array([1.0, 1.0]), 3)
    assert np.allclose(zm, (x0 + x1) / 2, atol=1e-15)
    assert np.allclose(impl.euler_step(x0, u, np.array([1.0, 1.0]), 3), x1, atol=1e-15)
    assert np.array_equal(impl.midpoint_half(x0, u, np.zeros(2), 3), x0)


# ------------------------------------------------ Flowception insertion
def _packed(seed, frames_per_seq, tpf=3, ch=2):
    r = _rng(seed)
    F = sum(frames_per_seq)
    z = r.standard_normal((F * tpf, ch))
    t = r.random(F)
    cu = np.concatenate([[0], np.cumsum(frames_per_seq)]) * tpf
    return z, t, cu


def pin_insert_none_is_identity(impl):
    z, t, cu = _packed(60, [2, 3, 1])
    zo, to, co, src = impl.insert_frames(z, t, cu, np.zeros(6, int), np.zeros((0, 2)), 3)
    assert np.array_equal(zo, z) and np.array_equal(to, t) and np.array_equal(co, cu)
    assert np.array_equal(src, np.arange(6))


def pin_insert_worked_example(impl):
    """Two sequences of frames A B | C, counts (1, 0 | 2): the result is
    A n0 B | C n1 n2 with the new frames at time 0 and the offsets grown."""
    tpf = 2
    z = np.array([[1.0], [1.5], [2.0], [2.5], [3.0], [3.5]])   # frames A, B, C
    t = np.array([0.25, 0.5, 0.75])
    noise = -np.arange(1.0, 7.0).reshape(6, 1)                 # frames n0, n1, n2
    zo, to, co, src = impl.insert_frames(z, t, [0, 4, 6], [1, 0, 2], noise, tpf)
    assert np.array_equal(zo[:, 0], [1.0, 1.5, -1.0, -2.0, 2.0, 2.5, 3.0, 3.5, -3.0, -4.0, -5.0, -6.0])
    assert np.array_equal(to, [0.25, 0.0, 0.5, 0.75, 0.0, 0.0])
    assert np.array_equal(co, [0, 6, 12])
    assert np.array_equal(src, [0, -1, 1, 2, -2, -3])


def pin_insert_invariants(impl):
    """Random counts: sizes grow by the counts per sequence; deleting the
    inserted frames gives back the input; inserted frames hold the noise in
    order with time 0; no frame crosses into another sequence."""
    r = _rng(61)
    fps = [4, 1, 6, 2]
    z, t, cu = _packed(62, fps, tpf=5, ch=3)
    counts = r.poisson(0.8, size=sum(fps))
    noise = r.standard_normal((counts.sum() * 5, 3))
    zo, to, co, src = impl.insert_frames(z, t, cu, counts, noise, 5)
    assert len(to) == sum(fps) + counts.sum() and zo.shape == (len(to) * 5, 3)
    fo = np.concatenate([[0], np.cumsum(fps)])
    for s in range(4):
        assert co[s + 1] - co[s] == 5 * (fps[s] + counts[fo[s]:fo[s + 1]].sum())
        seg = src[co[s] // 5:co[s + 1] // 5]
        assert set(seg[seg >= 0]) == set(range(fo[s], fo[s + 1]))
    keep = src >= 0
    assert np.array_equal(src[keep], np.arange(sum(fps)))
    assert np.array_equal(zo.reshape(-1, 5, 3)[keep].reshape(-1, 3), z)
    assert np.array_equal(to[keep], t)
    new = ~keep
    assert np.array_equal(-1 - src[new], np.arange(counts.sum()))
    assert np.array_equal(zo.reshape(-1, 5, 3)[new].reshape(-1, 3), noise) and np.all(to[new] == 0.0)


def pin_insert_bruteforce(impl):
    """Against list splicing: insert each frame's new frames by walking the
    existing frames from the last to the first and splicing into a list."""
    r = _rng(63)
    fps = [3, 2]
    z, t, cu = _packed(64, fps, tpf=2, ch=1)
    counts = r.integers(0, 3, size=5)
    noise = r.standard_normal((counts.sum() * 2, 1))
    frames = [("x", f) for f in range(5)]
    starts = np.concatenate([[0], np.cumsum(counts)])
    for f in reversed(range(5)):
        for j in reversed(range(counts[f])):
            frames.insert(f + 1, ("n", starts[f] + j))
    zo, to, _, src = impl.insert_frames(z, t, cu, counts, noise, 2)
    for o, (kind, i) in enumerate(frames):
        blk = z[2 * i:2 * i + 2] if kind == "x" else noise[2 * i:2 * i + 2]
        assert np.array_equal(zo[2 * o:2 * o + 2], blk)
        assert src[o] == (i if kind == "x" else -1 - i)


def pin_schedule(impl):
    """Frames step by dt_max until the last step lands exactly on 1; a frame at
    1 stays; inserted frames (t = 0) take full steps."""
    dt, tn = impl.frame_schedule(np.array([0.0, 0.5, 1.0 - 1.0 / 64, 1.0]), 1.0 / 30)
    assert np.allclose(dt, [1 / 30, 1 / 30, 1 / 64, 0.0], rtol=0, atol=1e-15)
    assert np.allclose(tn, [1 / 30, 0.5 + 1 / 30, 1.0, 1.0], rtol=0, atol=1e-15)
    t = np.array([0.0, 0.3])
    for _ in range(40):
        _, t = impl.frame_schedule(t, 1.0 / 30)
    assert np.all(t == 1.0)


# ------------------------------------------------ FP8 (OCP E4M3)
def pin_e4m3_spec_values(impl):
    """Landmarks of the OCP E4M3 format: 1 = 0x38, -2 = 0xC0, the largest
    finite value 448 = 0x7E, 240 = 0x77, the smallest normal 2^-6 = 0x08, the
    smallest subnormal 2^-9 = 0x01, 0x7F / 0xFF are NaN."""
    pairs = {1.0: 0x38, -2.0: 0xC0, 448.0: 0x7E, 240.0: 0x77, 2.0 ** -6: 0x08, 2.0 ** -9: 0x01, 0.0: 0x00}
    for v, c in pairs.items():
        assert int(impl.e4m3_encode(np.array([v], np.float32))[0]) == c, (v, hex(c))
        assert impl.e4m3_decode(np.array([c], np.uint8))[0] == v
    assert np.all(np.isnan(impl.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))))


def pin_e4m3_roundtrip(impl):
    """Every finite code decodes to a value that encodes back to that code."""
    c = np.array([i for i in range(256) if i not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(impl.e4m3_encode(impl.e4m3_decode(c).astype(np.float32)), c)


def pin_e4m3_nearest_ties_even(impl):
    """Random values and exact midpoints against a search over all finite
    codes: the nearest value, ties to the code with an even mantissa."""
    vals = np.array(sorted({float(v) for v in o_fp8_values()}))
    r = _rng(70)
    xs = list(r.uniform(-448, 448, 300)) + list(r.uniform(-0.05, 0.05, 300))
    xs += [(vals[i] + vals[i + 1]) / 2 for i in range(len(vals) - 1)]   # midpoints
    xs = np.array(xs, dtype=np.float32)
    got = impl.e4m3_encode(xs)
    for x, c in zip(xs, got):
        d = np.abs(vals - float(x))
        best = vals[d == d.min()]
        if len(best) > 1:   # tie: the even mantissa
            best = [b for b in best if int(impl.e4m3_encode(np.array([b], np.float32))[0]) % 2 == 0]
        want = abs(best[0]) if x >= 0 else -abs(best[0])
        if want == 0.0 and np.signbit(x):
            want = -0.0
        assert impl.e4m3_decode(np.array([c], np.uint8))[0] == want, (float(x), hex(int(c)))


def o_fp8_values():
    """All finite E4M3 values, listed from the format's definition (sign,
    exponent with bias 7, 3-bit mantissa; subnormals at exponent 0)."""
    out = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
            out += [v, -v]
    return out


def pin_quantize_per_head(impl):
    """Each head's largest magnitude maps to +-448 (0x7E / 0xFE); every value is
    within half a code spacing (relative 2^-4) of its dequantised value; an
    all-zero head stays zero with scale 1. Also for a head of magnitude 1e-37,
    where the float32 quotient 448 / amax would overflow."""
    r = _rng(71)
    x = r.standard_normal((40, 4, 16)).astype(np.float32) * np.array([1.0, 30.0, 0.0, 1e-37], np.float32)[None, :, None]
    codes, amax, scale = impl.quantize_per_head(x)
    for h in (0, 1, 3):
        i = np.unravel_index(np.argmax(np.abs(x[:, h, :])), x[:, h, :].shape)
        assert codes[i[0], h, i[1]] in (0x7E, 0xFE)
        deq = impl.e4m3_decode(codes[:, h, :]) * float(scale[h])
        assert np.all(np.abs(deq - x[:, h, :]) <= np.maximum(np.abs(x[:, h, :]) * 2.0 ** -4, 2.0 ** -10 * scale[h]) * (1 + 1e-6))
        assert amax[h] == np.abs(x[:, h, :]).max()
    assert np.all(codes[:, 2, :] == 0) and scale[2] == 1.0


def pin_dequantize_per_head(impl):
    """dequantize(codes, scale) gives back the quantised tensor: shape
    [tokens, heads, d] with tokens, heads and d all different; the element of
    largest magnitude of each head comes back as +-amax to float32 precision
    (448 times the scale amax / 448); every element within half a code spacing
    (relative 2^-4, or 2^-10 of the scale below E4M3's normal range) of the
    value it came from; an all-zero head is zero. Also on hand-built codes,
    against values listed from the format's definition: code 0x38 (1.0) gives
    exactly the head's scale, 0x7E (448) gives 448 times it, 0xC0 (-2) minus
    twice it, 0x01 (2^-9) 2^-9 times it."""
    r = _rng(72)
    mags = np.array([1.0, 30.0, 0.0, 0.01], np.float32)
    x = r.standard_normal((40, 4, 16)).astype(np.float32) * mags[None, :, None]
    codes, amax, scale = impl.quantize_per_head(x)
    deq = np.asarray(impl.dequantize(codes, scale))
    assert deq.shape == x.shape
    for h in range(4):
        xh = x[:, h, :].astype(np.float64)
        dh = deq[:, h, :]
        if mags[h] == 0:
            assert np.all(dh == 0)
            continue
        i = np.unravel_index(np.argmax(np.abs(xh)), xh.shape)
        assert abs(abs(dh[i]) - float(amax[h])) <= float(amax[h]) * 2.0 ** -23
        assert np.sign(dh[i]) == np.sign(xh[i])
        assert np.all(np.abs(dh - xh) <= np.maximum(np.abs(xh) * 2.0 ** -4, 2.0 ** -10 * float(scale[h])) * (1 + 1e-6))
    sc = np.array([0.5, 3.0, 1e-3], np.float32)
    vals = {0x38: 1.0, 0x7E: 448.0, 0xC0: -2.0, 0x01: 2.0 ** -9, 0x00: 0.0}
    for c, v in vals.items():
        cc = np.full((5, 3, 2), c, np.uint8)
        got = np.asarray(impl.dequantize(cc, sc))
        want = v * sc.astype(np.float64)[None, :, None] * np.ones((5, 3, 2))
        assert np.array_equal(got, want), hex(c)


def pin_q_score_scale_power_of_two(impl):
    """q's scale makes the score scale a power of two: for heads of very
    different magnitudes (and tokens != heads != dims), sq * sk * log2(e) /
    sqrt(d) equals 2^n with n an integer; it is the smallest such scale that
    keeps q's codes inside E4M3 (the largest |q| / sq lies in (224, 448], so
    2^(n-1) would overflow 448); every q element lies within half a code spacing
    of its dequantised value; code dot products times 2^n are the dequantised
    scores in base-2 units; k and v are quantised per head as on their own.
    When k's head is all zero the scores are zero whatever q holds: q's codes
    are 0 there; an all-zero q head also has codes 0, and so has a head whose
    scores all lie below 2^-127 (q and k of magnitude 1e-20: the exponent would
    be below -127)."""
    r = _rng(73)
    d = 32
    mq = np.array([1.0, 30.0, 1e-3, 2.0, 0.0, 1e-20], np.float32)
    mk = np.array([1.0, 0.05, 500.0, 0.0, 1.0, 1e-20], np.float32)
    x = [r.standard_normal((24, 6, d)).astype(np.float32) for _ in range(3)]
    q, k, v = x[0] * mq[None, :, None], x[1] * mk[None, :, None], x[2]
    (cq, ck, cv), amax, scale, n = impl.quantize_qkv(q, k, v)
    ck2, ak2, sk2 = impl.quantize_per_head(k)
    cv2, _, sv2 = impl.quantize_per_head(v)
    assert np.array_equal(ck, ck2) and np.array_equal(cv, cv2)
    assert np.array_equal(scale[1], sk2.astype(np.float64)) and np.array_equal(scale[2], sv2.astype(np.float64))
    qd = np.asarray(impl.dequantize(cq, scale[0]))
    kd = np.asarray(impl.dequantize(ck, scale[1]))
    for h in range(6):
        if mq[h] == 0 or mk[h] == 0 or mq[h] < 1e-10:
            assert np.all(cq[:, h, :] == 0) and n[h] == 0
            continue
        nh = int(n[h])
        assert nh == n[h]
        c = float(scale[0][h]) * float(scale[1][h]) * math.log2(math.e) / math.sqrt(d)
        assert abs(c / 2.0 ** nh - 1.0) < 1e-13, (h, c, nh)
        top = float(np.abs(q[:, h, :]).max()) / float(scale[0][h])
        assert 224.0 * (1 - 1e-6) < top <= 448.0 * (1 + 1e-6), (h, top)
        qh = q[:, h, :].astype(np.float64)
        err = np.abs(qd[:, h, :] - qh)
        assert np.all(err <= np.maximum(np.abs(qh) * 2.0 ** -4, 2.0 ** -10 * float(scale[0][h])) * (1 + 1e-6))
        codes_dot = impl.e4m3_decode(cq[:, h, :]) @ impl.e4m3_decode(ck[:, h, :]).T
        s2 = qd[:, h, :] @ kd[:, h, :].T * (math.log2(math.e) / math.sqrt(d))
        assert np.allclose(codes_dot * 2.0 ** nh, s2, rtol=1e-12, atol=1e-300)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
