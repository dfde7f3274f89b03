"""GPU parity of 8-bit (OCP E4M3) attention: the quantisation of q, k, v
(bit-exact against the oracle's codes, per-head amax exact, the transposed V
layout), and the attention on the codes against the float64 attention oracle on
the dequantised values.

Tolerance of the attention (derived from the arithmetic; checked per element):
the only rounding between the dequantised inputs and the float32 accumulators
is the E4M3 rounding of the probabilities before the second product. In the
kernel's units P_k = 2^(s_k log2 e - m + 6) with an integer running max m
(raised to the ceiling of a tile max that exceeds it by more than 2), the
largest weight lies in [2^5, 2^8]; rounding to nearest moves P_k by d_k, at
most half its spacing: 2^-4 P_k for normal values, 2^-10 below 2^-6
(subnormals). Relative to the row total L = sum P >= 2^5 that is
|d_k| / L <= h_k = 2^-4 w_k + 2^-15 (w = the softmax weights). The kernel's row sum adds the same rounded values the product uses
(a product against a constant ones operand), so the output is
sum (P_k + d_k) v_k / (L + D) with D = sum d_k, and its error is
    sum_k d_k (v_k - o) / (L + D)  =  [sum_k (d_k / L)(v_k - o)] / (1 + D / L).
With independent, zero-mean d_k / L in [-h_k, h_k] the numerator has standard
deviation at most sigma = sqrt(sum_k h_k^2 / 3 (|v_k| + |o|)^2), and
D / L has standard deviation at most sigma_D = sqrt(sum_k h_k^2 / 3). Bar per
element: 7 sigma / (1 - 7 sigma_D) (a Gaussian tail of ~1e-12 per element for
either sum) + 2^-8 |o| (the bf16 store) + 1e-4.
"""
import math

import numpy as np
import pytest
import torch

import diffusion_transformer_video_amd as dit
import synth
from gpu_util import need_gpu, note, sample_rows
from oracle import attention as o_attn
from oracle import fp8 as o_fp8

pytestmark = pytest.mark.gpu


def _vt_col(w):
    b, q, h, i = w >> 5, (w >> 3) & 3, (w >> 2) & 1, w & 3
    return 32 * h + 16 * b + 4 * q + i


def _quant_gpu(q, k, v, cu, num_seqs, max_seqlen):
    tokens, heads, hd = q.shape
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()
    qd, kd, vd = d(q), d(k), d(v)
    vs = dit.dit_fp8_v_stride(tokens, num_seqs)
    q8 = torch.empty(q.shape, dtype=torch.uint8, device="cuda")
    k8 = torch.empty_like(q8)
    v8t = torch.full((heads, hd, vs), 0x7F, dtype=torch.uint8, device="cuda")   # NaN codes where not written
    amax = torch.empty(3, heads, dtype=torch.float32, device="cuda")
    cut = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    dit.dit_quant_fp8(q8, k8, v8t, amax, qd, kd, vd, cut, num_seqs, max_seqlen)
    torch.cuda.synchronize()
    return q8, k8, v8t, amax, cut


def _check_quant(q, k, v, cu, q8, k8, v8t, amax):
    """Codes and amax exactly as the oracle's; V transposed with the tile
    permutation, sequences padded with zero codes to whole tiles."""
    heads = q.shape[1]
    codes, ref_amax, _, _ = o_fp8.quantize_qkv(q, k, v)
    assert np.array_equal(q8.cpu().numpy(), codes[0]) and np.array_equal(k8.cpu().numpy(), codes[1])
    assert np.array_equal(amax.cpu().numpy(), ref_amax)
    vt = v8t.cpu().numpy()
    vc = codes[2]
    col = 0
    cu = np.asarray(cu, np.int64)
    perm = np.array([_vt_col(w) for w in range(64)])
    for s in range(len(cu) - 1):
        n = int(cu[s + 1] - cu[s])
        nt = (n + 63) // 64
        for j in range(nt):
            keys = np.arange(64 * j, min(64 * j + 64, n))
            blk = vt[:, :, col + 64 * j:col + 64 * j + 64]                    # [heads, 128, 64]
            want = np.zeros((heads, 128, 64), np.uint8)
            want[:, :, perm[keys - 64 * j]] = vc[cu[s] + keys].transpose(1, 2, 0)
            assert np.array_equal(blk, want), (s, j)
        col += 64 * nt


def _fp8_bound(qd, kd, vd, cu, rows):
    """Oracle output on the dequantised values and the per-element bar (module
    docstring) for the given query rows."""
    o, _ = o_attn.attention_lse(qd, kd, vd, cu, cu, rows=rows)
    tol = np.zeros_like(o)
    cu = np.asarray(cu, np.int64)
    seq = np.searchsorted(cu, rows, side="right") - 1
    scale = 1.0 / math.sqrt(qd.shape[2])
    for s in np.unique(seq):
        sel = np.nonzero(seq == s)[0]
        lo, hi = int(cu[s]), int(cu[s + 1])
        for h in range(qd.shape[1]):
            S = qd[rows[sel], h, :] @ kd[lo:hi, h, :].T * scale
            w = np.exp(S - S.max(axis=1, keepdims=True))
            w /= w.sum(axis=1, keepdims=True)
            hk = 2.0 ** -4 * w + 2.0 ** -15                                   # [rows, keys]
            V = np.abs(vd[lo:hi, h, :])                                       # [keys, 128]
            oo = np.abs(o[sel, h, :])                                         # [rows, 128]
            # sum_k hk^2 (|v_k| + |o|)^2 = sum hk^2 v^2 + 2|o| sum hk^2 |v| + o^2 sum hk^2
            h2 = hk * hk
            var = (h2 @ (V * V) + 2 * oo * (h2 @ V) + oo * oo * h2.sum(axis=1, keepdims=True)) / 3.0
            sig_d = np.sqrt(h2.sum(axis=1, keepdims=True) / 3.0)              # of D / L, per row
            assert np.all(7.0 * sig_d < 0.5)
            tol[sel, h, :] = 7.0 * np.sqrt(var) / (1.0 - 7.0 * sig_d) + 2.0 ** -8 * oo + 1e-4
    return o, tol


def _run_case(q, k, v, cu, num_seqs, max_seqlen, rows=None, dense=False):
    q8, k8, v8t, amax, cut = _quant_gpu(q, k, v, None if dense else cu, num_seqs, max_seqlen)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    dit.dit_attn3d_fp8(o, q8, k8, v8t, amax, None if dense else cut, num_seqs, max_seqlen)
    torch.cuda.synchronize()
    codes, _, scales, _ = o_fp8.quantize_qkv(q, k, v)
    qd, kd, vd = (o_fp8.dequantize(c, sc) for c, sc in zip(codes, scales))
    rows = np.arange(q.shape[0]) if rows is None else rows
    ref, tol = _fp8_bound(qd, kd, vd, cu, rows)
    got = o[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    note(f"fp8 attention {q.shape}: max err {err.max():.3e}, max err / bar {np.max(err / tol):.3f}, "
         f"median bar {np.median(tol):.2e}")
    assert np.all(err <= tol)
    return q8, k8, v8t, amax


def _inputs(w_or_lens, heads=2, seed=1):
    if isinstance(w_or_lens, synth.Workload):
        w = w_or_lens
        inp = synth.make(w, ["q", "k", "v"])
        return (np.asarray(inp[n], np.float32) for n in ("q", "k", "v")), w.cu_seqlens.astype(np.int64)
    lens = w_or_lens
    r = np.random.default_rng(seed)
    T = int(sum(lens))
    x = [synth.bf16_round(r.standard_normal((T, heads, 128)).astype(np.float32)) for _ in range(3)]
    return x, np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def test_quantisation_bit_exact():
    need_gpu()
    (q, k, v), cu = _inputs([1, 63, 64, 65, 300], heads=3, seed=2)
    q[:, 2, :] *= 40.0   # one head with a much larger range
    q = synth.bf16_round(q)
    q8, k8, v8t, amax, _ = _quant_gpu(q, k, v, cu, 5, 300)
    _check_quant(q, k, v, cu, q8, k8, v8t, amax)


def test_quantisation_all_zero_head():
    need_gpu()
    (q, k, v), cu = _inputs([70, 5], heads=2, seed=3)
    k[:, 1, :] = 0.0
    q8, k8, v8t, amax, _ = _quant_gpu(q, k, v, cu, 2, 70)
    _check_quant(q, k, v, cu, q8, k8, v8t, amax)
    assert bool((k8[:, 1, :] == 0).all())


def test_ragged_packed():
    need_gpu()
    (q, k, v), cu = _inputs([1, 63, 64, 65, 300, 129], heads=2, seed=4)
    _run_case(q, k, v, cu, 6, 300)


def test_all_zero_q_and_k_heads():
    """A head whose q (or k) is all zero has all scores 0: each query gets the
    plain mean of its sequence's dequantised V rows, partial tiles included."""
    need_gpu()
    (q, k, v), cu = _inputs([70, 5, 130], heads=3, seed=9)
    q[:, 1, :] = 0.0
    k[:, 2, :] = 0.0
    _run_case(q, k, v, cu, 3, 130)


def test_dense_batch():
    need_gpu()
    (q, k, v), cu = _inputs([200, 200, 200], heads=2, seed=5)
    _run_case(q, k, v, cu, 3, 200, dense=True)


def test_peaked_scores():
    """Large-magnitude q, k (sharply peaked softmax rows: the running max moves
    and the probabilities span E4M3's range)."""
    need_gpu()
    (q, k, v), cu = _inputs([500, 77], heads=2, seed=6)
    q, k = synth.bf16_round(q * 4.0), synth.bf16_round(k * 4.0)
    _run_case(q, k, v, cu, 2, 500)


def test_scores_beyond_the_unshifted_range():
    """Running maxima outside [-100, 120] (base 2): every wave forms its
    probabilities with the shift subtracted before the exponential -- a head
    whose scores are all far above the range (q, k 40x larger), a head whose
    scores are all far below it (every key nearly opposite its query), and a
    head where the last keys' scores leave the range only late in the
    sequence, so waves switch form in the middle of the key loop."""
    need_gpu()
    (q, k, v), cu = _inputs([700, 130], heads=3, seed=11)
    q[:, 0, :] *= 40.0
    k[:, 0, :] *= 40.0
    u = np.ones(128, np.float32)
    q[:, 1, :] = 3.0 * u + 0.3 * q[:, 1, :]
    k[:, 1, :] = -3.0 * u + 0.3 * k[:, 1, :]
    k[600:700, 2, :] *= 60.0
    q, k = synth.bf16_round(q), synth.bf16_round(k)
    _run_case(q, k, v, cu, 2, 700)


@pytest.mark.parametrize("w", [synth.C2, synth.C3, synth.C4, synth.C5], ids=lambda w: w.name)
def test_full_size_sampled_rows(w):
    need_gpu()
    (q, k, v), cu = _inputs(w)
    rows = sample_rows(w, per_seq=32, edge=4)
    q8, k8, v8t, amax = _run_case(q, k, v, cu, w.num_seqs, w.max_seqlen, rows=rows, dense=w.dense)
    codes, ref_amax, _, _ = o_fp8.quantize_qkv(q, k, v)
    assert np.array_equal(amax.cpu().numpy(), ref_amax)
    assert np.array_equal(q8.cpu().numpy(), codes[0])


def test_scores_below_the_exponent_range():
    """q and k of magnitude 1e-20 in one head (every score below 2^-127 of the
    largest code product): q's codes are 0 there, bit-exact with the oracle, and
    each query gets the plain mean of its sequence's dequantised V rows."""
    need_gpu()
    (q, k, v), cu = _inputs([130, 65], heads=2, seed=12)
    q[:, 1, :] *= 1e-20
    k[:, 1, :] *= 1e-20
    q, k = synth.bf16_round(q), synth.bf16_round(k)
    q8, k8, v8t, amax, _ = _quant_gpu(q, k, v, cu, 2, 130)
    _check_quant(q, k, v, cu, q8, k8, v8t, amax)
    assert bool((q8[:, 1, :] == 0).all())
    _run_case(q, k, v, cu, 2, 130)


def test_tiny_k_and_v_heads():
    """A k head and a v head of magnitude 1e-37, where the float32 quotient
    448 / amax would overflow (the multiplier is then formed pre-scaled): codes
    bit-exact with the oracle, attention against it."""
    need_gpu()
    (q, k, v), cu = _inputs([130, 65], heads=3, seed=13)
    k[:, 1, :] *= 1e-37
    v[:, 2, :] *= 1e-37
    k, v = synth.bf16_round(k), synth.bf16_round(v)
    q8, k8, v8t, amax, _ = _quant_gpu(q, k, v, cu, 2, 130)
    _check_quant(q, k, v, cu, q8, k8, v8t, amax)
    _run_case(q, k, v, cu, 2, 130)


def test_ulysses_share_shape():
    """One GPU's share of the 480P video workload under head-sharded context
    parallelism over 8 GPUs (5 heads x 32,760 tokens): 640 blocks, 2.5 per CU."""
    need_gpu()
    r = np.random.default_rng(1103)
    T = 32760
    q, k, v = (synth.bf16_round(r.standard_normal((T, 5, 128)).astype(np.float32)) for _ in range(3))
    cu = np.array([0, T], np.int64)
    w = synth.Workload("c3_share_5heads", "bf16", (30, 52), (21,), (32760,), 5, 128, (44, 42, 42), 10000.0, 32760, 1103)
    _run_case(q, k, v, cu, 1, T, rows=sample_rows(w, per_seq=256, edge=8))


def test_deterministic():
    need_gpu()
    (q, k, v), cu = _inputs([700, 64], heads=2, seed=7)
    outs = []
    for _ in range(2):
        q8, k8, v8t, amax, cut = _quant_gpu(q, k, v, cu, 2, 700)
        o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
        dit.dit_attn3d_fp8(o, q8, k8, v8t, amax, cut, 2, 700)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_quantisation_guard_and_determinism():
    """The quantisation writes exactly its outputs (canaries around the q and k
    codes and the amax table keep their values) and is deterministic."""
    need_gpu()
    (q, k, v), cu = _inputs([300, 65], heads=3, seed=9)
    tokens, heads, hd = q.shape
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()
    qd, kd, vd = d(q), d(k), d(v)
    cut = torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    vs = dit.dit_fp8_v_stride(tokens, 2)
    outs = []
    for _ in range(2):
        pad = 4096
        bq8 = torch.full((tokens * heads * hd + 2 * pad,), 0x5A, dtype=torch.uint8, device="cuda")
        bk8 = torch.full_like(bq8, 0x5A)
        ba = torch.full((3 * heads + 2 * 64,), 7.0, dtype=torch.float32, device="cuda")
        q8 = bq8[pad:pad + tokens * heads * hd].view(tokens, heads, hd)
        k8 = bk8[pad:pad + tokens * heads * hd].view(tokens, heads, hd)
        amax = ba[64:64 + 3 * heads].view(3, heads)
        v8t = torch.zeros((heads, hd, vs), dtype=torch.uint8, device="cuda")
        dit.dit_quant_fp8(q8, k8, v8t, amax, qd, kd, vd, cut, 2, 300)
        torch.cuda.synchronize()
        for b in (bq8, bk8):
            assert bool(torch.all(b[:pad] == 0x5A)) and bool(torch.all(b[-pad:] == 0x5A))
        assert bool(torch.all(ba[:64] == 7.0)) and bool(torch.all(ba[-64:] == 7.0))
        outs.append((q8.clone(), k8.clone(), v8t.clone(), amax.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
