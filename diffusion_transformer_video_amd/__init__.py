"""Python binding of libdit (include/dit.h): the DiT attention-block hot path
on MI355X (gfx950).

Argument marshalling only. Each function takes torch tensors that already live
on the GPU, checks dtype/shape/contiguity, and calls the C entry point of the
same name on torch's current stream; every step runs in the HIP kernels. There
is no fallback: if libdit.so is missing or the device is not gfx950 the call
raises.

Layout: activations are token-major and contiguous -- hidden [tokens, d_model],
q/k/v/o [tokens, heads, head_dim], latent [tokens, channels]; parameter tables
gamma/beta/alpha [rows, d_model] and dt_rows [rows] are float32 with
row = token // tokens_per_row.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build, next to this file; no other copy is ever loaded
LIB_PATH = os.path.join(_PKG, "libdit.so")

DIT_F32, DIT_BF16 = 0, 1
DIT_OK, DIT_E_INVAL, DIT_E_UNSUPPORTED, DIT_E_HIP = 0, 1, 2, 3

EXPORTS = ("dit_last_error", "dit_version", "dit_adaln_modulate", "dit_rope3d",
           "dit_attn3d", "dit_attn3d_noalloc", "dit_attn3d_lse", "dit_attn_merge", "dit_gated_residual", "rf_euler_step",
           "rf_midpoint_half", "rf_interpolant", "rf_cfm_loss", "flow_insert_frames",
           "flow_frame_schedule", "dit_fp8_v_stride", "dit_quant_fp8", "dit_attn3d_fp8")


class DitError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class EulerArgs(ctypes.Structure):
    _fields_ = [("z_out", ctypes.c_void_p), ("z", ctypes.c_void_p), ("u", ctypes.c_void_p),
                ("dt_rows", ctypes.c_void_p), ("tokens", ctypes.c_int64),
                ("channels", ctypes.c_int32), ("tokens_per_row", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdit.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m diffusion_transformer_video_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.dit_last_error.restype = ctypes.c_char_p
        L.dit_last_error.argtypes = []
        L.dit_version.restype = ctypes.c_int
        L.dit_version.argtypes = []
        L.dit_adaln_modulate.restype = ctypes.c_int
        L.dit_adaln_modulate.argtypes = [vp, vp, vp, vp, i64, i32, i64, f32, i32, vp]
        L.dit_rope3d.restype = ctypes.c_int
        L.dit_rope3d.argtypes = [vp, vp, i64, i32, i32, i32, i32, i32, vp, i32,
                                 i32, i32, i32, f32, vp, i32, vp]
        for name in ("dit_attn3d", "dit_attn3d_noalloc"):
            getattr(L, name).restype = ctypes.c_int
            getattr(L, name).argtypes = [vp, vp, vp, vp, i64, i32, i32, vp, i32, i32, i32, vp]
        L.dit_attn3d_lse.restype = ctypes.c_int
        L.dit_attn3d_lse.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, vp, vp, i32, i32, i32, i32, vp]
        L.dit_attn_merge.restype = ctypes.c_int
        L.dit_attn_merge.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, vp]
        L.dit_gated_residual.restype = ctypes.c_int
        L.dit_gated_residual.argtypes = [vp, vp, vp, vp, i64, i32, i64,
                                         ctypes.POINTER(EulerArgs), i32, vp]
        L.rf_euler_step.restype = ctypes.c_int
        L.rf_euler_step.argtypes = [vp, vp, vp, vp, i64, i32, i64, i32, vp]
        for name in ("rf_midpoint_half", "rf_interpolant"):
            getattr(L, name).restype = ctypes.c_int
            getattr(L, name).argtypes = [vp, vp, vp, vp, i64, i32, i64, i32, vp]
        L.dit_fp8_v_stride.restype = ctypes.c_int64
        L.dit_fp8_v_stride.argtypes = [i64, i32]
        L.dit_quant_fp8.restype = ctypes.c_int
        L.dit_quant_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, vp, i32, i32, i64, i32, vp]
        L.dit_attn3d_fp8.restype = ctypes.c_int
        L.dit_attn3d_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, vp, i32, i32, i64, vp]
        L.flow_insert_frames.restype = ctypes.c_int
        L.flow_insert_frames.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i64, i64, i32, i32, i32, vp]
        L.flow_frame_schedule.restype = ctypes.c_int
        L.flow_frame_schedule.argtypes = [vp, vp, i64, f32, vp]
        L.rf_cfm_loss.restype = ctypes.c_int
        L.rf_cfm_loss.argtypes = [vp, vp, vp, vp, vp, i64, i32, i64, i32, vp]
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != DIT_OK:
        raise DitError(rc, lib().dit_last_error().decode(errors="replace"))


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DIT_BF16
    if t.dtype == torch.float32:
        return DIT_F32
    raise TypeError(f"activations must be bfloat16 or float32, got {t.dtype}")


def _dev(*ts) -> None:
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _f32(*ts) -> None:
    torch = _torch()
    for t in ts:
        if t.dtype != torch.float32:
            raise TypeError("parameter tables (gamma, beta, alpha, dt_rows) and lse / accumulators must be float32")


def _offsets(*pairs) -> None:
    """Sequence offsets (cu_seqlens) must be int32 [num_seqs + 1]: the kernels
    read them as int32, so int64 offsets (torch's default integer type) would be
    taken as pairs of int32 values. Checked before anything else, so a wrong
    type raises before any launch."""
    torch = _torch()
    for name, t in pairs:
        if t is None:
            continue
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32, got {t.dtype}")
        if t.dim() != 1 or t.numel() < 2:
            raise ValueError(f"{name} must be a 1-D tensor of num_seqs + 1 >= 2 offsets")


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def dit_adaln_modulate(y, x, gamma, beta, tokens_per_row: int, eps: float = 1e-6, stream=None):
    """y = gamma[row] * LayerNorm(x) + beta[row]; x, y [tokens, d_model]."""
    _dev(y, x, gamma, beta)
    _f32(gamma, beta)
    if x.dim() != 2 or y.shape != x.shape or x.dtype != y.dtype:
        raise ValueError("x and y must be [tokens, d_model] of one dtype")
    tokens, d = x.shape
    _check(lib().dit_adaln_modulate(_ptr(y), _ptr(x), _ptr(gamma), _ptr(beta), tokens, d,
                                    int(tokens_per_row), float(eps), _dtype_code(x), _stream(stream)))
    return y


def dit_rope3d(q, k, grid: Sequence[int], split: Sequence[int], base: float = 10000.0,
               cu_seqlens=None, num_seqs: int = 1, pos_out=None, stream=None):
    """Rotate q and k ([tokens, heads, head_dim]) in place by R_3D(t', h', w').

    grid = (T', H', W'); with cu_seqlens, T' is ignored and positions restart per
    packed sequence. split = (d_t, d_h, d_w). pos_out (optional): int32 with at
    least 3 * tokens elements, receives (t', h', w') per token."""
    torch = _torch()
    _offsets(("cu_seqlens", cu_seqlens))
    if pos_out is not None and (pos_out.dtype != torch.int32 or pos_out.numel() < 3 * q.shape[0]):
        raise TypeError("pos_out must be int32 with at least 3 * tokens elements")
    _dev(q, k, cu_seqlens, pos_out)
    if q.dim() != 3 or (k is not None and (k.shape != q.shape or k.dtype != q.dtype)):
        raise ValueError("q and k must be [tokens, heads, head_dim] of one dtype")
    tokens, heads, hd = q.shape
    if cu_seqlens is not None:
        num_seqs = cu_seqlens.numel() - 1
    _check(lib().dit_rope3d(_ptr(q), _ptr(k), tokens, heads, hd, int(grid[0]), int(grid[1]),
                            int(grid[2]), _ptr(cu_seqlens), int(num_seqs), int(split[0]),
                            int(split[1]), int(split[2]), float(base), _ptr(pos_out),
                            _dtype_code(q), _stream(stream)))
    return q, k


def _attn3d(entry, o, q, k, v, cu_seqlens, num_seqs, max_seqlen, stream):
    _offsets(("cu_seqlens", cu_seqlens))
    _dev(o, q, k, v, cu_seqlens)
    if q.dim() != 3 or any(t.shape != q.shape or t.dtype != q.dtype for t in (k, v, o)):
        raise ValueError("o, q, k, v must be [tokens, heads, head_dim] of one dtype")
    tokens, heads, hd = q.shape
    if cu_seqlens is not None:
        num_seqs = cu_seqlens.numel() - 1
    _check(getattr(lib(), entry)(_ptr(o), _ptr(q), _ptr(k), _ptr(v), tokens, heads, hd,
                                 _ptr(cu_seqlens), int(num_seqs), int(max_seqlen), _dtype_code(q),
                                 _stream(stream)))
    return o


def dit_attn3d(o, q, k, v, cu_seqlens=None, num_seqs: int = 1, max_seqlen: int = 0, stream=None):
    """o = softmax(q k^T / sqrt(head_dim)) v per (sequence, head); all [tokens, heads, hd].
    cu_seqlens: None (dense, num_seqs equal sequences) or device int32 [num_seqs + 1]."""
    return _attn3d("dit_attn3d", o, q, k, v, cu_seqlens, num_seqs, max_seqlen, stream)


def dit_attn3d_noalloc(o, q, k, v, cu_seqlens=None, num_seqs: int = 1, max_seqlen: int = 0, stream=None):
    """dit_attn3d without any allocation at call time (the library's fixed scratch slot;
    calls that overlap on one device race). Arguments as dit_attn3d."""
    return _attn3d("dit_attn3d_noalloc", o, q, k, v, cu_seqlens, num_seqs, max_seqlen, stream)


def dit_attn3d_lse(o, lse, q, k, v, cu_seqlens_q=None, cu_seqlens_k=None, num_seqs: int = 1,
                   max_seqlen_q: int = 0, max_seqlen_k: int = 0, stream=None):
    """One ring step: o, lse of each sequence's queries against its own key block.

    q, o [tokens_q, heads, hd]; k, v [tokens_k, heads, hd]; lse [tokens_q, heads]
    float32 (natural log). cu_seqlens_q / cu_seqlens_k: both None (dense,
    num_seqs equal sequences) or both device int32 [num_seqs + 1]."""
    _offsets(("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k))
    if (cu_seqlens_q is None) != (cu_seqlens_k is None):
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be given together")
    _dev(o, lse, q, k, v, cu_seqlens_q, cu_seqlens_k)
    _f32(lse)
    if q.dim() != 3 or o.shape != q.shape or any(t.dtype != q.dtype for t in (k, v, o)):
        raise ValueError("o, q must be [tokens_q, heads, head_dim] and k, v share their dtype")
    if k.dim() != 3 or v.shape != k.shape or k.shape[1:] != q.shape[1:]:
        raise ValueError("k, v must be [tokens_k, heads, head_dim] with the heads and head_dim of q")
    if lse.shape != q.shape[:2]:
        raise ValueError("lse must be [tokens_q, heads]")
    tq, heads, hd = q.shape
    if cu_seqlens_q is not None:
        num_seqs = cu_seqlens_q.numel() - 1
        if cu_seqlens_k is None or cu_seqlens_k.numel() != num_seqs + 1:
            raise ValueError("cu_seqlens_k must have as many sequences as cu_seqlens_q")
    _check(lib().dit_attn3d_lse(_ptr(o), _ptr(lse), _ptr(q), _ptr(k), _ptr(v), tq, k.shape[0], heads, hd,
                                _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), int(num_seqs), int(max_seqlen_q),
                                int(max_seqlen_k), _dtype_code(q), _stream(stream)))
    return o, lse


def dit_attn_merge(o_acc, lse_acc, o_b, lse_b, stream=None):
    """(o_acc, lse_acc) <- merge with the partial (o_b, lse_b), in place.
    o_acc float32 [tokens, heads, hd]; o_b [tokens, heads, hd] (bf16 or float32);
    lse_acc, lse_b float32 [tokens, heads]."""
    _dev(o_acc, lse_acc, o_b, lse_b)
    _f32(o_acc, lse_acc, lse_b)
    if o_acc.dim() != 3 or o_b.shape != o_acc.shape or lse_acc.shape != o_acc.shape[:2] or lse_b.shape != lse_acc.shape:
        raise ValueError("o_acc, o_b must be [tokens, heads, head_dim] and lse_acc, lse_b [tokens, heads]")
    tokens, heads, hd = o_acc.shape
    _check(lib().dit_attn_merge(_ptr(o_acc), _ptr(lse_acc), _ptr(o_b), _ptr(lse_b), tokens, heads, hd,
                                _dtype_code(o_b), _stream(stream)))
    return o_acc, lse_acc


def dit_gated_residual(x_out, x, branch, alpha, tokens_per_row: int, euler=None, stream=None):
    """x_out = x + alpha[row] * branch (branch heads merged); optional fused Euler
    pass: euler = (z_out, z, u, dt_rows, tokens_per_row)."""
    _dev(x_out, x, branch, alpha)
    _f32(alpha)
    if x.dim() != 2 or x_out.shape != x.shape or branch.numel() != x.numel():
        raise ValueError("x, x_out must be [tokens, d_model] and branch the same size")
    if branch.dtype != x.dtype or x_out.dtype != x.dtype:
        raise ValueError("x, x_out and branch must share one dtype")
    tokens, d = x.shape
    ea = None
    if euler is not None:
        z_out, z, u, dt_rows, tpr = euler
        _dev(z_out, z, u, dt_rows)
        _f32(dt_rows)
        if z.dim() != 2 or z_out.shape != z.shape or u.shape != z.shape or z.dtype != x.dtype:
            raise ValueError("Euler tensors must be [tokens, channels] in the residual's dtype")
        ea = EulerArgs(_ptr(z_out), _ptr(z), _ptr(u), _ptr(dt_rows), z.shape[0], z.shape[1], int(tpr))
    _check(lib().dit_gated_residual(_ptr(x_out), _ptr(x), _ptr(branch), _ptr(alpha), tokens, d,
                                    int(tokens_per_row), ctypes.byref(ea) if ea is not None else None,
                                    _dtype_code(x), _stream(stream)))
    return x_out


def rf_euler_step(z_out, z, u, dt_rows, tokens_per_row: int, stream=None):
    """z_out = z + dt_rows[row] * u; z, u [tokens, channels]."""
    _dev(z_out, z, u, dt_rows)
    _f32(dt_rows)
    if z.dim() != 2 or z_out.shape != z.shape or u.shape != z.shape or u.dtype != z.dtype:
        raise ValueError("z, z_out, u must be [tokens, channels] of one dtype")
    tokens, ch = z.shape
    _check(lib().rf_euler_step(_ptr(z_out), _ptr(z), _ptr(u), _ptr(dt_rows), tokens, ch,
                               int(tokens_per_row), _dtype_code(z), _stream(stream)))
    return z_out


def rf_midpoint_half(z_mid, z, u, dt_rows, tokens_per_row: int, stream=None):
    """z_mid = z + (dt_rows[row] / 2) * u; z, u [tokens, channels]."""
    _dev(z_mid, z, u, dt_rows)
    _f32(dt_rows)
    if z.dim() != 2 or z_mid.shape != z.shape or u.shape != z.shape or u.dtype != z.dtype or z_mid.dtype != z.dtype:
        raise ValueError("z, z_mid, u must be [tokens, channels] of one dtype")
    tokens, ch = z.shape
    _check(lib().rf_midpoint_half(_ptr(z_mid), _ptr(z), _ptr(u), _ptr(dt_rows), tokens, ch,
                                  int(tokens_per_row), _dtype_code(z), _stream(stream)))
    return z_mid


def rf_interpolant(x_t, x0, x1, t_rows, tokens_per_row: int, stream=None):
    """x_t = (1 - t[row]) x0 + t[row] x1; x0, x1 [tokens, channels]."""
    _dev(x_t, x0, x1, t_rows)
    _f32(t_rows)
    if x0.dim() != 2 or x1.shape != x0.shape or x_t.shape != x0.shape or \
            x1.dtype != x0.dtype or x_t.dtype != x0.dtype:
        raise ValueError("x_t, x0, x1 must be [tokens, channels] of one dtype")
    tokens, ch = x0.shape
    _check(lib().rf_interpolant(_ptr(x_t), _ptr(x0), _ptr(x1), _ptr(t_rows), tokens, ch,
                                int(tokens_per_row), _dtype_code(x0), _stream(stream)))
    return x_t


def rf_cfm_loss(loss_tokens, loss_rows, u, x0, x1, tokens_per_row: int, stream=None):
    """loss_tokens[tok] = sum_c (u - (x1 - x0))^2; loss_rows (or None) the per-row sums."""
    _dev(loss_tokens, loss_rows, u, x0, x1)
    _f32(loss_tokens, *(() if loss_rows is None else (loss_rows,)))
    if u.dim() != 2 or x0.shape != u.shape or x1.shape != u.shape or x0.dtype != u.dtype or x1.dtype != u.dtype:
        raise ValueError("u, x0, x1 must be [tokens, channels] of one dtype")
    tokens, ch = u.shape
    if loss_tokens.shape != (tokens,):
        raise ValueError("loss_tokens must be [tokens]")
    if loss_rows is not None and loss_rows.shape != (tokens // int(tokens_per_row),):
        raise ValueError("loss_rows must be [tokens // tokens_per_row]")
    _check(lib().rf_cfm_loss(_ptr(loss_tokens), _ptr(loss_rows), _ptr(u), _ptr(x0), _ptr(x1), tokens, ch,
                             int(tokens_per_row), _dtype_code(u), _stream(stream)))
    return loss_tokens, loss_rows


def flow_insert_frames(z_out, t_out, cu_out, src_out, z, t_frames, cu_seqlens, counts, noise,
                       tokens_per_frame: int, stream=None):
    """Insert counts[f] noise frames right after every existing frame f of the packed
    batch z ([frames * tokens_per_frame, channels]); see include/dit.h."""
    torch = _torch()
    _offsets(("cu_seqlens", cu_seqlens), ("cu_out", cu_out))
    _dev(z_out, t_out, cu_out, src_out, z, t_frames, cu_seqlens, counts, noise)
    _f32(t_out, t_frames)
    for t in (cu_out, src_out, cu_seqlens, counts):
        if t.dtype != torch.int32:
            raise TypeError("offsets, counts and src_out must be int32")
    if z.dim() != 2 or z_out.dim() != 2 or z_out.shape[1] != z.shape[1] or z_out.dtype != z.dtype:
        raise ValueError("z and z_out must be [tokens, channels] of one dtype")
    tpf = int(tokens_per_frame)
    frames, frames_out = t_frames.numel(), t_out.numel()
    if z.shape[0] != frames * tpf or z_out.shape[0] != frames_out * tpf or counts.numel() != frames:
        raise ValueError("z / z_out rows must be frames * tokens_per_frame and counts [frames]")
    if src_out.numel() != frames_out or cu_out.numel() != cu_seqlens.numel():
        raise ValueError("src_out must be [frames_out] and cu_out shaped like cu_seqlens")
    if noise is not None and (noise.dtype != z.dtype or noise.shape != ((frames_out - frames) * tpf, z.shape[1])):
        raise ValueError("noise must be [(frames_out - frames) * tokens_per_frame, channels] in z's dtype")
    _check(lib().flow_insert_frames(_ptr(z_out), _ptr(t_out), _ptr(cu_out), _ptr(src_out), _ptr(z),
                                    _ptr(t_frames), _ptr(cu_seqlens), cu_seqlens.numel() - 1, _ptr(counts),
                                    _ptr(noise), frames, frames_out, tpf, z.shape[1], _dtype_code(z),
                                    _stream(stream)))
    return z_out, t_out, cu_out, src_out


def flow_frame_schedule(dt_out, t_frames, dt_max: float, stream=None):
    """dt_out = min(dt_max, 1 - t_frames); t_frames += dt_out (in place)."""
    _dev(dt_out, t_frames)
    _f32(dt_out, t_frames)
    if dt_out.shape != t_frames.shape or t_frames.dim() != 1:
        raise ValueError("dt_out and t_frames must be [frames]")
    _check(lib().flow_frame_schedule(_ptr(dt_out), _ptr(t_frames), t_frames.numel(), float(dt_max),
                                     _stream(stream)))
    return dt_out, t_frames


def dit_fp8_v_stride(tokens: int, num_seqs: int) -> int:
    """Bytes per row of the transposed 8-bit V (see dit_quant_fp8)."""
    return int(lib().dit_fp8_v_stride(int(tokens), int(num_seqs)))


def dit_quant_fp8(q8, k8, v8t, amax, q, k, v, cu_seqlens=None, num_seqs: int = 1, max_seqlen: int = 0,
                  stream=None):
    """q, k, v (bf16 [tokens, heads, 128]) -> E4M3 codes q8, k8 (uint8, same shape),
    v8t (uint8 [heads, 128, v_stride]) and amax (float32 [3, heads])."""
    torch = _torch()
    _offsets(("cu_seqlens", cu_seqlens))
    _dev(q8, k8, v8t, amax, q, k, v, cu_seqlens)
    _f32(amax)
    if any(t.dtype != torch.uint8 for t in (q8, k8, v8t)):
        raise TypeError("q8, k8 and v8t must be uint8")
    if q.dim() != 3 or any(t.shape != q.shape for t in (k, v, q8, k8)) or q.dtype != torch.bfloat16:
        raise ValueError("q, k, v must be bf16 [tokens, heads, head_dim] and q8, k8 of that shape")
    tokens, heads, hd = q.shape
    if cu_seqlens is not None:
        num_seqs = cu_seqlens.numel() - 1
    if v8t.dim() != 3 or v8t.shape[:2] != (heads, hd) or amax.shape != (3, heads):
        raise ValueError("v8t must be [heads, head_dim, v_stride] and amax [3, heads]")
    _check(lib().dit_quant_fp8(_ptr(q8), _ptr(k8), _ptr(v8t), _ptr(amax), _ptr(q), _ptr(k), _ptr(v), tokens,
                               heads, hd, _ptr(cu_seqlens), int(num_seqs), int(max_seqlen), v8t.shape[2],
                               _dtype_code(q), _stream(stream)))
    return q8, k8, v8t, amax


def dit_attn3d_fp8(o, q8, k8, v8t, amax, cu_seqlens=None, num_seqs: int = 1, max_seqlen: int = 0, stream=None):
    """o (bf16 [tokens, heads, 128]) = attention on the E4M3 codes written by dit_quant_fp8."""
    torch = _torch()
    _offsets(("cu_seqlens", cu_seqlens))
    _dev(o, q8, k8, v8t, amax, cu_seqlens)
    _f32(amax)
    if o.dtype != torch.bfloat16 or o.dim() != 3 or q8.shape != o.shape or k8.shape != o.shape:
        raise ValueError("o must be bf16 [tokens, heads, head_dim] and q8, k8 of that shape")
    tokens, heads, hd = o.shape
    if cu_seqlens is not None:
        num_seqs = cu_seqlens.numel() - 1
    _check(lib().dit_attn3d_fp8(_ptr(o), _ptr(q8), _ptr(k8), _ptr(v8t), _ptr(amax), tokens, heads, hd,
                                _ptr(cu_seqlens), int(num_seqs), int(max_seqlen), v8t.shape[2], _stream(stream)))
    return o
