"""The C-ABI library loads, exports every symbol include/dit.h declares, and
rejects bad arguments before touching the device (CPU only: every call below
fails validation, so nothing is launched)."""
import ctypes
import os
import re

import pytest

import diffusion_transformer_video_amd as dit
from libdit_loader import ensure_built

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dit.h")
FAKE = 0x10000  # aligned, never dereferenced: every call here fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("dit_adaln_modulate", "dit_rope3d", "dit_attn3d", "dit_attn3d_lse", "dit_attn_merge",
              "dit_gated_residual", "rf_euler_step", "rf_midpoint_half", "rf_interpolant", "rf_cfm_loss",
              "dit_last_error", "dit_version"):
        assert n in names
    assert set(names) == set(dit.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ensure_built()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert L.dit_version() == 10000


def _err():
    return dit.lib().dit_last_error().decode()


def test_modulate_validation():
    L = ensure_built()
    assert L.dit_adaln_modulate(None, FAKE, FAKE, FAKE, 8, 64, 8, 1e-6, 1, None) == dit.DIT_E_INVAL
    assert "NULL" in _err()
    assert L.dit_adaln_modulate(FAKE, FAKE, FAKE, FAKE, 0, 64, 1, 1e-6, 1, None) == dit.DIT_E_INVAL
    assert L.dit_adaln_modulate(FAKE, FAKE, FAKE, FAKE, 10, 64, 3, 1e-6, 1, None) == dit.DIT_E_INVAL
    assert "tokens_per_row" in _err()
    assert L.dit_adaln_modulate(FAKE, FAKE, FAKE, FAKE, 8, 64, 8, 0.0, 1, None) == dit.DIT_E_INVAL
    assert L.dit_adaln_modulate(FAKE, FAKE, FAKE, FAKE, 8, 60, 8, 1e-6, 1, None) == dit.DIT_E_UNSUPPORTED
    assert L.dit_adaln_modulate(FAKE, FAKE, FAKE, FAKE, 8, 64, 8, 1e-6, 7, None) == dit.DIT_E_UNSUPPORTED
    assert "dtype" in _err()
    assert L.dit_adaln_modulate(FAKE + 4, FAKE, FAKE, FAKE, 8, 64, 8, 1e-6, 1, None) == dit.DIT_E_UNSUPPORTED
    assert "aligned" in _err()
    # y partially overlapping x
    assert L.dit_adaln_modulate(FAKE + 16, FAKE, FAKE * 4, FAKE * 8, 8, 64, 8, 1e-6, 1, None) == dit.DIT_E_INVAL


def test_rope_validation():
    L = ensure_built()
    args = dict(q=FAKE, k=FAKE * 8, tokens=32, heads=2, hd=64, gt=2, gh=4, gw=4, cu=None, ns=1,
                dt_=16, dh=24, dw=24, base=10000.0, pos=None, dtype=0)

    def call(**kw):
        a = dict(args, **kw)
        return L.dit_rope3d(a["q"], a["k"], a["tokens"], a["heads"], a["hd"], a["gt"], a["gh"], a["gw"],
                            a["cu"], a["ns"], a["dt_"], a["dh"], a["dw"], a["base"], a["pos"], a["dtype"], None)
    assert call(q=None) == dit.DIT_E_INVAL
    assert call(dh=26) == dit.DIT_E_INVAL and "head_dim" in _err()
    assert call(dt_=15, dh=25) == dit.DIT_E_INVAL and "even" in _err()
    assert call(base=1.0) == dit.DIT_E_INVAL
    assert call(tokens=33) == dit.DIT_E_INVAL and "dense" in _err()
    assert call(gt=0) == dit.DIT_E_INVAL
    assert call(hd=96, dt_=32, dh=32, dw=32, tokens=32) == dit.DIT_E_UNSUPPORTED
    assert call(k=FAKE + 64) == dit.DIT_E_INVAL and "overlap" in _err()


def test_attn_validation():
    L = ensure_built()
    o, q, k, v = FAKE * 16, FAKE, FAKE * 4, FAKE * 8
    assert L.dit_attn3d(None, q, k, v, 64, 2, 128, None, 1, 0, 1, None) == dit.DIT_E_INVAL
    assert L.dit_attn3d(o, q, k, v, 65, 2, 128, None, 2, 0, 1, None) == dit.DIT_E_INVAL
    assert "multiples of num_seqs" in _err()
    assert L.dit_attn3d(o, q, k, v, 64, 2, 96, None, 1, 0, 1, None) == dit.DIT_E_UNSUPPORTED
    assert L.dit_attn3d(o, q, k, v, 64, 2, 128, FAKE * 32, 2, 0, 1, None) == dit.DIT_E_INVAL
    assert "max_seqlen" in _err()
    assert L.dit_attn3d(q, q, k, v, 64, 2, 128, None, 1, 0, 1, None) == dit.DIT_E_INVAL
    assert "overlap" in _err()
    assert L.dit_attn3d(o, q, k, v, 0, 2, 128, None, 1, 0, 1, None) == dit.DIT_E_INVAL


def test_attn_noalloc_validation():
    """The allocation-free entry point validates exactly as dit_attn3d, under its own name."""
    L = ensure_built()
    o, q, k, v = FAKE * 16, FAKE, FAKE * 4, FAKE * 8
    assert L.dit_attn3d_noalloc(None, q, k, v, 64, 2, 128, None, 1, 0, 1, None) == dit.DIT_E_INVAL
    assert "dit_attn3d_noalloc" in _err() and "NULL" in _err()
    assert L.dit_attn3d_noalloc(o, q, k, v, 65, 2, 128, None, 2, 0, 1, None) == dit.DIT_E_INVAL
    assert L.dit_attn3d_noalloc(o, q, k, v, 64, 2, 96, None, 1, 0, 1, None) == dit.DIT_E_UNSUPPORTED
    assert L.dit_attn3d_noalloc(o, q, k, v, 64, 2, 128, FAKE * 32, 2, 0, 1, None) == dit.DIT_E_INVAL
    assert L.dit_attn3d_noalloc(q, q, k, v, 64, 2, 128, None, 1, 0, 1, None) == dit.DIT_E_INVAL
    assert "overlap" in _err()
    assert L.dit_attn3d_noalloc(o, q, k, v, 64, 2, 128, None, 1, 0, 7, None) == dit.DIT_E_UNSUPPORTED


def test_attn_lse_validation():
    L = ensure_built()
    o, lse, q, k, v = FAKE * 16, FAKE * 24, FAKE, FAKE * 4, FAKE * 8
    cu_q, cu_k = FAKE * 32, FAKE * 33

    def call(**kw):
        a = dict(o=o, lse=lse, q=q, k=k, v=v, tq=64, tk=48, h=2, hd=128, cq=None, ck=None, ns=1,
                 mq=0, mk=0, dtype=1)
        a.update(kw)
        return L.dit_attn3d_lse(a["o"], a["lse"], a["q"], a["k"], a["v"], a["tq"], a["tk"], a["h"], a["hd"],
                                a["cq"], a["ck"], a["ns"], a["mq"], a["mk"], a["dtype"], None)
    assert call(lse=None) == dit.DIT_E_INVAL and "NULL" in _err()
    assert call(tk=0) == dit.DIT_E_INVAL
    assert call(cq=cu_q) == dit.DIT_E_INVAL and "both" in _err()
    assert call(tk=47, ns=2, tq=64) == dit.DIT_E_INVAL and "multiples" in _err()
    assert call(cq=cu_q, ck=cu_k, ns=2, mq=0, mk=10) == dit.DIT_E_INVAL and "max_seqlen" in _err()
    assert call(cq=cu_q, ck=cu_k, ns=2, mq=32, mk=49) == dit.DIT_E_INVAL and "key" in _err()
    assert call(hd=96) == dit.DIT_E_UNSUPPORTED
    assert call(lse=FAKE * 24 + 2) == dit.DIT_E_UNSUPPORTED and "lse" in _err()
    assert call(lse=q + 64) == dit.DIT_E_INVAL and "lse must not overlap" in _err()
    assert call(o=k + 32) == dit.DIT_E_INVAL and "overlap" in _err()
    assert call(dtype=5) == dit.DIT_E_UNSUPPORTED


def test_attn_merge_validation():
    L = ensure_built()
    oa, la, ob, lb = FAKE, FAKE * 16, FAKE * 32, FAKE * 48
    assert L.dit_attn_merge(None, la, ob, lb, 8, 2, 64, 1, None) == dit.DIT_E_INVAL
    assert L.dit_attn_merge(oa, la, ob, lb, 0, 2, 64, 1, None) == dit.DIT_E_INVAL
    assert L.dit_attn_merge(oa, la, ob, lb, 8, 2, 32, 1, None) == dit.DIT_E_UNSUPPORTED
    assert L.dit_attn_merge(oa + 8, la, ob, lb, 8, 2, 64, 1, None) == dit.DIT_E_UNSUPPORTED
    assert L.dit_attn_merge(oa, oa + 64, ob, lb, 8, 2, 64, 1, None) == dit.DIT_E_INVAL
    assert "overlap" in _err()
    assert L.dit_attn_merge(oa, la, ob, lb, 8, 2, 64, 9, None) == dit.DIT_E_UNSUPPORTED


def test_epilogue_validation():
    L = ensure_built()
    assert L.rf_euler_step(FAKE, FAKE, FAKE * 4, None, 32, 64, 32, 1, None) == dit.DIT_E_INVAL
    assert L.rf_euler_step(FAKE, FAKE, FAKE * 4, FAKE * 8, 32, 60, 32, 1, None) == dit.DIT_E_UNSUPPORTED
    assert L.rf_euler_step(FAKE, FAKE, FAKE, FAKE * 8, 32, 64, 32, 1, None) == dit.DIT_E_INVAL
    assert "overlaps u" in _err()
    assert L.dit_gated_residual(FAKE, FAKE, FAKE * 4, FAKE * 8, 30, 64, 7, None, 1, None) == dit.DIT_E_INVAL
    bad = dit.EulerArgs(FAKE * 16, FAKE * 16, FAKE * 20, None, 32, 64, 32)
    assert L.dit_gated_residual(FAKE, FAKE, FAKE * 4, FAKE * 8, 32, 64, 32, ctypes.byref(bad), 1,
                                None) == dit.DIT_E_INVAL
    assert "euler" in _err()


def test_flow_validation():
    L = ensure_built()
    # midpoint half step: the Euler checks
    assert L.rf_midpoint_half(FAKE, FAKE, FAKE * 4, None, 32, 64, 32, 1, None) == dit.DIT_E_INVAL
    assert L.rf_midpoint_half(FAKE, FAKE, FAKE, FAKE * 8, 32, 64, 32, 1, None) == dit.DIT_E_INVAL
    assert L.rf_midpoint_half(FAKE, FAKE, FAKE * 4, FAKE * 8, 32, 60, 32, 1, None) == dit.DIT_E_UNSUPPORTED
    # interpolant
    assert L.rf_interpolant(FAKE, FAKE * 4, FAKE * 8, None, 32, 64, 32, 1, None) == dit.DIT_E_INVAL
    assert L.rf_interpolant(FAKE, FAKE * 4, FAKE * 8, FAKE * 12, 30, 64, 7, 1, None) == dit.DIT_E_INVAL
    assert L.rf_interpolant(FAKE, FAKE * 4, FAKE * 8, FAKE * 12, 32, 12, 32, 1, None) == dit.DIT_E_UNSUPPORTED
    assert L.rf_interpolant(FAKE + 64, FAKE, FAKE * 8, FAKE * 12, 32, 64, 32, 1, None) == dit.DIT_E_INVAL
    assert "overlaps" in _err()
    # cfm loss
    assert L.rf_cfm_loss(None, None, FAKE, FAKE * 4, FAKE * 8, 32, 64, 32, 1, None) == dit.DIT_E_INVAL
    assert L.rf_cfm_loss(FAKE * 12, None, FAKE, FAKE * 4, FAKE * 8, 32, 64, 5, 1, None) == dit.DIT_E_INVAL
    assert L.rf_cfm_loss(FAKE * 12 + 2, None, FAKE, FAKE * 4, FAKE * 8, 32, 64, 32, 1, None) == dit.DIT_E_UNSUPPORTED
    assert L.rf_cfm_loss(FAKE + 64, None, FAKE, FAKE * 4, FAKE * 8, 32, 64, 32, 1, None) == dit.DIT_E_INVAL
    assert "overlap" in _err()
    assert L.rf_cfm_loss(FAKE * 12, FAKE * 12, FAKE, FAKE * 4, FAKE * 8, 32, 64, 32, 1, None) == dit.DIT_E_INVAL


def test_flowception_validation():
    L = ensure_built()
    zo, to, co, so = FAKE * 64, FAKE * 80, FAKE * 81, FAKE * 82
    z, t, cu, c, nz = FAKE, FAKE * 96, FAKE * 97, FAKE * 98, FAKE * 112

    def call(**kw):
        a = dict(zo=zo, to=to, co=co, so=so, z=z, t=t, cu=cu, ns=2, c=c, nz=nz, f=10, fo=14, tpf=16, ch=64,
                 dtype=1)
        a.update(kw)
        return L.flow_insert_frames(a["zo"], a["to"], a["co"], a["so"], a["z"], a["t"], a["cu"], a["ns"], a["c"],
                                    a["nz"], a["f"], a["fo"], a["tpf"], a["ch"], a["dtype"], None)
    assert call(c=None) == dit.DIT_E_INVAL
    assert call(fo=9) == dit.DIT_E_INVAL and "frames_out" in _err()
    assert call(nz=None) == dit.DIT_E_INVAL and "noise" in _err()
    assert call(ch=12) == dit.DIT_E_UNSUPPORTED
    assert call(tpf=0) == dit.DIT_E_INVAL
    assert call(fo=1 << 30) == dit.DIT_E_UNSUPPORTED and "int32" in _err()
    assert call(zo=z + 64) == dit.DIT_E_INVAL and "overlap" in _err()
    assert call(to=t) == dit.DIT_E_INVAL
    assert call(t=FAKE * 96 + 2) == dit.DIT_E_UNSUPPORTED
    assert L.flow_frame_schedule(None, FAKE, 8, 1.0 / 30, None) == dit.DIT_E_INVAL
    assert L.flow_frame_schedule(FAKE, FAKE * 2, 0, 1.0 / 30, None) == dit.DIT_E_INVAL
    assert L.flow_frame_schedule(FAKE, FAKE * 2, 8, 0.0, None) == dit.DIT_E_INVAL
    assert L.flow_frame_schedule(FAKE, FAKE + 8, 8, 0.1, None) == dit.DIT_E_INVAL and "overlap" in _err()


def test_fp8_validation():
    L = ensure_built()
    assert L.dit_fp8_v_stride(100, 2) == 256 and L.dit_fp8_v_stride(0, 1) == 0
    q8, k8, v8t, am, q, k, v = FAKE * 16, FAKE * 24, FAKE * 32, FAKE * 64, FAKE, FAKE * 4, FAKE * 8
    vs = L.dit_fp8_v_stride(64, 1)

    def quant(**kw):
        a = dict(q8=q8, k8=k8, vt=v8t, am=am, q=q, k=k, v=v, t=64, h=2, hd=128, cu=None, ns=1, mx=0, vs=vs, dt=1)
        a.update(kw)
        return L.dit_quant_fp8(a["q8"], a["k8"], a["vt"], a["am"], a["q"], a["k"], a["v"], a["t"], a["h"], a["hd"],
                               a["cu"], a["ns"], a["mx"], a["vs"], a["dt"], None)
    assert quant(dt=0) == dit.DIT_E_UNSUPPORTED and "bf16" in _err()
    assert quant(q8=None) == dit.DIT_E_INVAL
    assert quant(hd=64) == dit.DIT_E_UNSUPPORTED and "128" in _err()
    assert quant(vs=vs - 64) == dit.DIT_E_INVAL and "v_stride" in _err()
    assert quant(vs=vs + 8) == dit.DIT_E_INVAL
    assert quant(cu=FAKE * 80, ns=2, mx=0) == dit.DIT_E_INVAL and "max_seqlen" in _err()
    assert quant(q8=q + 64) == dit.DIT_E_INVAL and "overlap" in _err()
    assert L.dit_attn3d_fp8(None, q8, k8, v8t, am, 64, 2, 128, None, 1, 0, vs, None) == dit.DIT_E_INVAL
    assert L.dit_attn3d_fp8(q, q8, k8, v8t, am, 64, 2, 64, None, 1, 0, vs, None) == dit.DIT_E_UNSUPPORTED
    assert L.dit_attn3d_fp8(q8, q8, k8, v8t, am, 64, 2, 128, None, 1, 0, vs, None) == dit.DIT_E_INVAL


def test_error_text_is_thread_local_and_cleared_on_new_error():
    L = ensure_built()
    L.rf_euler_step(None, None, None, None, 0, 0, 0, 1, None)
    first = _err()
    L.dit_attn3d(None, None, None, None, 1, 1, 64, None, 1, 0, 1, None)
    assert _err() != first and _err().startswith("dit_attn3d")


def test_binding_raises_without_gpu_tensors():
    import torch
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        dit.rf_euler_step(x, x, x, torch.zeros(1), 4)


def test_binding_rejects_int64_offsets_before_any_launch():
    """Sequence offsets must be int32: an int64 tensor (torch's default integer
    type) would be read as pairs of int32 values. The binding raises TypeError
    before the device check and before any call into the library."""
    import torch
    q = torch.zeros(8, 2, 64)
    cu64 = torch.tensor([0, 3, 8], dtype=torch.int64)
    with pytest.raises(TypeError):
        dit.dit_attn3d(q, q, q, q, cu_seqlens=cu64, max_seqlen=5)
    with pytest.raises(TypeError):
        dit.dit_attn3d_lse(q, torch.zeros(8, 2), q, q, q, cu64, cu64, max_seqlen_q=5, max_seqlen_k=5)
    with pytest.raises(TypeError):
        dit.dit_rope3d(q, q, (1, 1, 8), (0, 32, 32), cu_seqlens=cu64)
    with pytest.raises(TypeError):
        dit.dit_quant_fp8(q, q, q, q, q, q, q, cu_seqlens=cu64, max_seqlen=5)
    with pytest.raises(TypeError):
        dit.dit_attn3d_fp8(q, q, q, q, q, cu_seqlens=cu64, max_seqlen=5)
    # pos_out: int32 with room for (t', h', w') of every token
    with pytest.raises(TypeError):
        dit.dit_rope3d(q, q, (1, 1, 8), (0, 32, 32), pos_out=torch.zeros(24, dtype=torch.int64))
    with pytest.raises(TypeError):
        dit.dit_rope3d(q, q, (1, 1, 8), (0, 32, 32), pos_out=torch.zeros(23, dtype=torch.int32))


def test_binding_loads_the_in_tree_library():
    """The binding loads only the libdit.so built next to it."""
    pkg = os.path.dirname(os.path.abspath(dit.__file__))
    assert dit.LIB_PATH == os.path.join(pkg, "libdit.so")
    assert dit.lib()._name == dit.LIB_PATH
