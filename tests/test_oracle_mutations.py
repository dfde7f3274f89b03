"""Plant plausible mistakes in copies of the oracle (CPU only) and check that
the pins catch every one: evidence that the pins constrain each function."""
import math

import numpy as np
import pytest

import oracle_pins as P
from oracle import attention as o_attn
from oracle import rope as o_rope


def _ln_unbiased(x, eps):
    x = np.asarray(x, dtype=np.float64)
    xc = x - x.mean(axis=-1, keepdims=True)
    return xc / np.sqrt(xc.var(axis=-1, ddof=1, keepdims=True) + eps)


def _ln_eps_outside(x, eps):
    x = np.asarray(x, dtype=np.float64)
    xc = x - x.mean(axis=-1, keepdims=True)
    return xc / (np.sqrt((xc * xc).mean(axis=-1, keepdims=True)) + eps)


def _mod_with(ln, one_plus=False, row_mod=False):
    def f(x, gamma, beta, tpr, eps):
        x = np.asarray(x, dtype=np.float64)
        n = x.shape[0]
        rows = (np.arange(n) % len(gamma)) if row_mod else (np.arange(n) // tpr)
        g = np.asarray(gamma)[rows]
        return ((1.0 + g) if one_plus else g) * ln(x, eps) + np.asarray(beta)[rows]
    return f


def _rope_with(sign=1.0, freq_dim=None, axis_perm=(0, 1, 2), half_split=False):
    def f(x, pos, split, base):
        x = np.asarray(x, dtype=np.float64)
        pos = np.asarray(pos, dtype=np.float64)[:, list(axis_perm)]
        hd = x.shape[-1]
        table = []
        off = 0
        for a, d_a in enumerate(split):
            for j in range(d_a // 2):
                dd = freq_dim if freq_dim else d_a
                table.append((a, off + 2 * j, float(base) ** (-2.0 * j / dd)))
            off += d_a
        ax = np.array([t[0] for t in table])
        th = np.array([t[2] for t in table])
        phi = pos[:, ax] * th
        c, s = np.cos(phi)[:, None, :], sign * np.sin(phi)[:, None, :]
        if half_split:
            i0, i1 = np.arange(hd // 2), np.arange(hd // 2, hd)
        else:
            i0, i1 = np.arange(0, hd, 2), np.arange(1, hd, 2)
        out = np.empty_like(x)
        out[..., i0] = x[..., i0] * c - x[..., i1] * s
        out[..., i1] = x[..., i0] * s + x[..., i1] * c
        return out
    return f


def _attn_with(scale_pow=0.5, use_k_as_v=False, ignore_cu=False, transpose_scores=False):
    def f(q, k, v, cu, rows=None, row_block=1024):
        q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
        n, h, d = q.shape
        cu = [0, n] if ignore_cu else list(cu)
        out = np.zeros_like(q)
        for s in range(len(cu) - 1):
            lo, hi = cu[s], cu[s + 1]
            for hh in range(h):
                S = q[lo:hi, hh] @ k[lo:hi, hh].T / d ** scale_pow
                if transpose_scores:
                    S = S.T
                P_ = o_attn.softmax_rows(S)
                out[lo:hi, hh] = P_ @ (k if use_k_as_v else v)[lo:hi, hh]
        return out if rows is None else out[np.asarray(rows)]
    return f


def _lse_with(log2=False, no_scale=False, lse_of_max=False):
    def f(q, k, v, cu_q, cu_k, num_seqs=1, rows=None, row_block=1024):
        o, lse = o_attn.attention_lse(q, k, v, cu_q, cu_k, num_seqs, rows, row_block)
        if log2:
            lse = lse / math.log(2.0)
        if lse_of_max:   # drops the log-sum term: returns the row max only
            cq, ck = list(cu_q), list(cu_k)
            out = np.full_like(lse, -np.inf)
            for s in range(len(cq) - 1):
                if ck[s + 1] > ck[s]:
                    S = np.einsum("qhd,khd->qhk", q[cq[s]:cq[s + 1]], k[ck[s]:ck[s + 1]]) / math.sqrt(q.shape[-1])
                    out[cq[s]:cq[s + 1]] = S.max(axis=-1)
            lse = out
        if no_scale:
            lse = lse * math.sqrt(q.shape[-1])
        return o, lse
    return f


def _merge_with(swap_weights=False, no_renorm=False):
    def f(o_a, lse_a, o_b, lse_b):
        o, lse = o_attn.merge(o_a, lse_a, o_b, lse_b)
        if swap_weights or no_renorm:
            la, lb = np.asarray(lse_a), np.asarray(lse_b)
            live = np.isfinite(lse)
            ref = np.where(live, lse, 0.0)
            wa = np.where(live, np.exp(la - ref), 0.0)
            wb = np.where(live, np.exp(lb - ref), 0.0)
            if swap_weights:
                wa, wb = wb, wa
            if no_renorm:
                wa, wb = np.ones_like(wa), np.ones_like(wb)
            o = wa[..., None] * o_a + wb[..., None] * o_b
        return o, lse
    return f


def _cfm_with(abs_err=False, plus=False, mean=False):
    def f(u, x0, x1, tpr):
        v = np.asarray(x1, np.float64) + np.asarray(x0, np.float64) if plus else \
            np.asarray(x1, np.float64) - np.asarray(x0, np.float64)
        e = np.asarray(u, np.float64) - v
        per_tok = np.abs(e).sum(axis=1) if abs_err else (e * e).sum(axis=1)
        if mean:
            per_tok = per_tok / e.shape[1]
        rows = np.arange(len(e)) // tpr
        per_row = np.zeros(rows[-1] + 1)
        np.add.at(per_row, rows, per_tok)
        return per_tok, per_row
    return f


def _midpoint_full_step(z, u, dt, tpr):
    rows = np.arange(len(z)) // tpr
    return np.asarray(z, np.float64) + np.asarray(dt, np.float64)[rows][:, None] * u


def _insert_before(z, t, cu, counts, noise, tpf):
    """Puts each frame's new frames before it instead of after it."""
    blocks, t_out, src, cu_out = [], [], [], [0]
    n = 0
    for s in range(len(cu) - 1):
        for f in range(cu[s] // tpf, cu[s + 1] // tpf):
            for _ in range(int(counts[f])):
                blocks.append(noise[n * tpf:(n + 1) * tpf]); t_out.append(0.0); src.append(-1 - n); n += 1
            blocks.append(z[f * tpf:(f + 1) * tpf]); t_out.append(float(t[f])); src.append(f)
        cu_out.append(len(src) * tpf)
    return np.concatenate(blocks), np.array(t_out), np.array(cu_out), np.array(src)


def _insert_keep_time(z, t, cu, counts, noise, tpf):
    """Inserted frames inherit the time of the frame before them (no reset)."""
    zo, to, co, src = P.real_impl().insert_frames(z, t, cu, counts, noise, tpf)
    to = to.copy()
    for o in range(1, len(src)):
        if src[o] < 0:
            to[o] = to[o - 1]
    return zo, to, co, src


def _schedule_no_clip(t, dt_max):
    t = np.asarray(t, np.float64)
    dt = np.full_like(t, dt_max)
    return dt, t + dt


def _e4m3_truncate(x):
    """Rounds magnitudes toward zero instead of to nearest."""
    from oracle import fp8
    x = np.asarray(x, np.float64)
    vals = np.array(sorted({abs(float(v)) for v in fp8.e4m3_decode(np.arange(127, dtype=np.uint8)) if not np.isnan(v)}))
    a = np.abs(x)
    idx = np.searchsorted(vals, a, side="right") - 1
    return fp8.e4m3_encode(np.copysign(vals[idx], x).astype(np.float32))


def _e4m3_decode_bias8(codes):
    c = np.asarray(codes, np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e, m = (c >> 3) & 15, c & 7
    return s * np.where(e == 0, m * 2.0 ** -10, (1 + m / 8) * np.exp2(e - 8.0))


def _quantize_per_tensor(x):
    from oracle import fp8
    x = np.asarray(x, np.float32)
    amax = np.float32(np.abs(x).max())
    inv = np.float32(448.0) / amax
    codes = fp8.e4m3_encode(np.clip((x * inv).astype(np.float32), -448, 448))
    h = x.shape[1]
    return codes, np.full(h, amax, np.float32), np.full(h, amax / np.float32(448), np.float32)


def _dequant_by_amax(codes, scale):
    from oracle import fp8
    return fp8.e4m3_decode(codes) * (np.asarray(scale, np.float64) * 448.0)[None, :, None]


def _dequant_over_tokens(codes, scale):
    from oracle import fp8
    return fp8.e4m3_decode(codes) * np.asarray(scale, np.float64)[:, None, None]


def _dequant_over_dims(codes, scale):
    from oracle import fp8
    return fp8.e4m3_decode(codes) * np.asarray(scale, np.float64)[None, None, :]


def _qkv_with(rule):
    """quantize_qkv with q's scale chosen by another rule."""
    def f(q, k, v):
        from oracle import fp8
        ck, ak, sk = fp8.quantize_per_head(k)
        cv, av, sv = fp8.quantize_per_head(v)
        q = np.asarray(q, np.float32)
        d = q.shape[2]
        aq = np.abs(q).max(axis=(0, 2)).astype(np.float32)
        cq = np.zeros(q.shape, np.uint8)
        sq = np.ones(q.shape[1])
        n = np.zeros(q.shape[1], np.int64)
        for h in range(q.shape[1]):
            if aq[h] == 0 or ak[h] == 0:
                continue
            skh = float(ak[h] / np.float32(448))
            if rule == "clamp_low":         # exponents below -127 clamped instead of zero codes
                t = float(aq[h]) * float(ak[h]) * np.log2(np.e) / (448.0 * 448.0 * np.sqrt(d))
                n[h] = max(int(np.ceil(np.log2(t))), -127)
                sq[h] = 2.0 ** n[h] * np.sqrt(d) / (skh * np.log2(np.e))
            elif rule == "ignore_k":          # the k / v rule: amax -> 448
                sq[h] = float(aq[h] / np.float32(448))
                n[h] = int(np.floor(np.log2(sq[h] * skh * np.log2(np.e) / np.sqrt(d))))
            else:
                lg = np.log2(np.e) if rule == "floor" else 1.0     # "natural": no log2(e)
                t = float(aq[h]) * float(ak[h]) * lg / (448.0 * 448.0 * np.sqrt(d))
                n[h] = int(np.floor(np.log2(t))) if rule == "floor" else int(np.ceil(np.log2(t)))
                sq[h] = 2.0 ** n[h] * np.sqrt(d) / (skh * lg)
            y = np.clip((q[:, h, :] * np.float32(1.0 / sq[h])).astype(np.float32), -448, 448)
            cq[:, h, :] = fp8.e4m3_encode(y)
        return (cq, ck, cv), np.stack([aq, ak, av]), np.stack([sq, sk.astype(np.float64), sv.astype(np.float64)]), n
    return f


def _coords_swapped(n, gh, gw):
    n = np.asarray(n, dtype=np.int64)
    return np.stack([n // (gh * gw), n % gw, (n // gw) % gh], axis=-1)


def _interp_reversed(x0, x1, t):
    t = np.asarray(t, dtype=np.float64)
    t = t[:, None] if t.ndim == 1 else t
    return t * np.asarray(x0, np.float64) + (1 - t) * np.asarray(x1, np.float64)


def _euler_minus(z, u, dt, tpr):
    rows = np.arange(len(z)) // tpr
    return np.asarray(z, np.float64) - np.asarray(dt, np.float64)[rows][:, None] * u


def _residual_rowmod(x, br, a, tpr):
    x = np.asarray(x, np.float64)
    rows = np.arange(len(x)) % len(a)
    return x + np.asarray(a)[rows] * np.asarray(br).reshape(x.shape)


def _residual_unmerged(x, br, a, tpr):
    x = np.asarray(x, np.float64)
    b = np.asarray(br).transpose(0, 2, 1).reshape(x.shape)  # wrong head merge
    rows = np.arange(len(x)) // tpr
    return x + np.asarray(a)[rows] * b


MUTANTS = {
    "ln_unbiased_variance": dict(adaln_modulate=_mod_with(_ln_unbiased), layer_norm=_ln_unbiased),
    "ln_eps_outside_sqrt": dict(adaln_modulate=_mod_with(_ln_eps_outside), layer_norm=_ln_eps_outside),
    "modulate_one_plus_gamma": dict(adaln_modulate=_mod_with(P.real_impl().layer_norm, one_plus=True)),
    "modulate_wrong_row": dict(adaln_modulate=_mod_with(P.real_impl().layer_norm, row_mod=True)),
    "rope_negative_angle": dict(apply_rope=_rope_with(sign=-1.0)),
    "rope_freq_over_head_dim": dict(apply_rope=_rope_with(freq_dim=64)),
    "rope_axes_reversed": dict(apply_rope=_rope_with(axis_perm=(2, 1, 0))),
    "rope_half_split_pairs": dict(apply_rope=_rope_with(half_split=True)),
    "attn_scale_over_d": dict(attention=_attn_with(scale_pow=1.0)),
    "attn_no_scale": dict(attention=_attn_with(scale_pow=0.0)),
    "attn_k_as_v": dict(attention=_attn_with(use_k_as_v=True)),
    "attn_across_sequences": dict(attention=_attn_with(ignore_cu=True)),
    "attn_transposed_scores": dict(attention=_attn_with(transpose_scores=True)),
    "lse_base2": dict(attention_lse=_lse_with(log2=True)),
    "lse_unscaled": dict(attention_lse=_lse_with(no_scale=True)),
    "lse_max_only": dict(attention_lse=_lse_with(lse_of_max=True)),
    "merge_swapped_weights": dict(merge=_merge_with(swap_weights=True)),
    "merge_no_renormalise": dict(merge=_merge_with(no_renorm=True)),
    "cfm_abs_error": dict(cfm_loss=_cfm_with(abs_err=True)),
    "cfm_wrong_velocity_sign": dict(cfm_loss=_cfm_with(plus=True)),
    "cfm_mean_not_norm": dict(cfm_loss=_cfm_with(mean=True)),
    "midpoint_full_step": dict(midpoint_half=_midpoint_full_step),
    "insert_before_frame": dict(insert_frames=_insert_before),
    "insert_keeps_time": dict(insert_frames=_insert_keep_time),
    "schedule_overshoots": dict(frame_schedule=_schedule_no_clip),
    "e4m3_truncating": dict(e4m3_encode=_e4m3_truncate),
    "e4m3_bias_8": dict(e4m3_decode=_e4m3_decode_bias8),
    "fp8_scale_per_tensor": dict(quantize_per_head=_quantize_per_tensor),
    "dequant_scale_is_amax": dict(dequantize=_dequant_by_amax),
    "dequant_scale_over_tokens": dict(dequantize=_dequant_over_tokens),
    "dequant_scale_over_dims": dict(dequantize=_dequant_over_dims),
    "q_scale_ignores_k": dict(quantize_qkv=_qkv_with("ignore_k")),
    "q_scale_exponent_floor": dict(quantize_qkv=_qkv_with("floor")),
    "q_scale_natural_log": dict(quantize_qkv=_qkv_with("natural")),
    "q_scale_clamps_tiny_exponent": dict(quantize_qkv=_qkv_with("clamp_low")),
    "grid_h_w_swapped": dict(coords=_coords_swapped),
    "interpolant_reversed": dict(interpolant=_interp_reversed),
    "euler_wrong_sign": dict(euler_step=_euler_minus),
    "residual_wrong_row": dict(gated_residual=_residual_rowmod),
    "residual_wrong_head_merge": dict(gated_residual=_residual_unmerged),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    impl = P.real_impl()
    for k, v in MUTANTS[name].items():
        setattr(impl, k, v)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(impl)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"
