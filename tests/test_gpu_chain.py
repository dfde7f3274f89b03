"""The attention half of a DiT block end to end on the GPU, through the C-ABI
binding, in the order one sampling step runs it: adaLN-Zero modulate of x,
3D-RoPE of q and k in place, attention on the rotated q and k, the gated
residual x' = x + alpha * o with the fused Euler step of the latent. Outputs
are compared with the float64 oracle's composition of the same steps from the
original inputs (no intermediate rounding on the oracle side).

Tolerance: the block's rows already meet 1e-4 (fp32) / 2e-2 (bf16) one at a
time. Chained, the GPU also rounds the rotated q, k and the attention output to
the storage type. For unit-variance q, k with head_dim d, rounding q and k to
bf16 moves a score by about 2^-9 (the relative rounding, times a unit-variance
sum normalised by sqrt(d)), so the softmax weights by ~0.2-0.4% and o by well
under 1e-2; o enters x' scaled by alpha ~ N(0, 0.1), and x' itself is rounded
once (2^-9 |x'| <= 1.6e-2 for |x'| < 8). Every chained output therefore stays
within the same bar as the single steps: 1e-4 fp32, 2e-2 bf16.
"""
import numpy as np
import pytest
import torch

import diffusion_transformer_video_amd as dit
import synth
from gpu_util import TOL, dev, host64, maxabs, need_gpu, note, sample_rows
from oracle import attention as o_attn
from oracle import epilogue as o_epi
from oracle import grid as o_grid
from oracle import modulate as o_mod
from oracle import rope as o_rope

pytestmark = pytest.mark.gpu

CHAIN = [
    synth.C1,
    synth.custom("chain_ragged_bf16", "bf16", (6, 10), (3, 1, 4), 3, 128, (44, 42, 42), tokens_per_row=60),
    synth.C2,
]


def _gpu_step(w, inp, alpha=None):
    x, q, k, v, z, u = (dev(inp[n], w) for n in ("x", "q", "k", "v", "z", "u"))
    g, b = dev(inp["gamma"]), dev(inp["beta"])
    al = dev(inp["alpha"] if alpha is None else alpha)
    dt = dev(inp["dt"])
    cu = None if w.dense else torch.from_numpy(w.cu_seqlens).cuda()
    y, o = torch.empty_like(x), torch.empty_like(q)
    x_out, z_out = torch.empty_like(x), torch.empty_like(z)
    dit.dit_adaln_modulate(y, x, g, b, w.tokens_per_row, w.eps)
    dit.dit_rope3d(q, k, (w.frames[0], *w.grid_hw), w.rope_split, w.rope_base, cu_seqlens=cu, num_seqs=w.num_seqs)
    if cu is None:
        dit.dit_attn3d(o, q, k, v, num_seqs=w.num_seqs)
    else:
        dit.dit_attn3d(o, q, k, v, cu_seqlens=cu, max_seqlen=w.max_seqlen)
    dit.dit_gated_residual(x_out, x, o.view(w.tokens, w.d_model), al, w.tokens_per_row,
                           euler=(z_out, z, u, dt, w.tokens_per_row))
    torch.cuda.synchronize()
    return x, y, o, x_out, z_out


@pytest.mark.parametrize("w", CHAIN, ids=lambda w: w.name)
def test_block_chain_against_oracle_composition(w):
    need_gpu()
    inp = synth.make(w, ["x", "gamma", "beta", "alpha", "q", "k", "v", "z", "u", "dt"])
    _, y, o, x_out, z_out = _gpu_step(w, inp)
    rows = None if w.tokens <= 4096 else sample_rows(w, per_seq=96)
    sel = slice(None) if rows is None else rows
    tpr = w.tokens_per_row
    # oracle composition from the original inputs
    pos = o_grid.positions(w.cu_seqlens, *w.grid_hw)
    rq = o_rope.apply_rope(inp["q"], pos, w.rope_split, w.rope_base)
    rk = o_rope.apply_rope(inp["k"], pos, w.rope_split, w.rope_base)
    ref_o = o_attn.attention(rq, rk, inp["v"], w.cu_seqlens, rows=rows)
    idx = np.arange(w.tokens)[sel]
    ref_y = o_mod.adaln_modulate(inp["x"][sel], inp["gamma"][idx // tpr], inp["beta"][idx // tpr], 1, w.eps)
    ref_x = o_epi.gated_residual(inp["x"][sel], ref_o.reshape(len(idx), w.d_model), inp["alpha"][idx // tpr], 1)
    ref_z = o_epi.euler_step(inp["z"], inp["u"], inp["dt"], tpr)
    pick = (lambda t: host64(t)) if rows is None else (lambda t: host64(t[torch.from_numpy(rows).cuda()]))
    errs = {"y": maxabs(pick(y), ref_y), "o": maxabs(pick(o), ref_o), "x'": maxabs(pick(x_out), ref_x),
            "z'": maxabs(host64(z_out), ref_z)}
    note(f"chain {w.name} ({w.dtype}): " + ", ".join(f"{n} {e:.3e}" for n, e in errs.items()))
    assert all(e <= TOL[w.dtype] for e in errs.values()), errs


@pytest.mark.parametrize("w", CHAIN[:2], ids=lambda w: w.name)
def test_block_identity_at_alpha_zero(w):
    """adaLN-Zero: with every alpha = 0 the whole chain leaves x unchanged, bit
    for bit, whatever the modulate, RoPE and attention steps produced."""
    need_gpu()
    inp = synth.make(w, ["x", "gamma", "beta", "alpha", "q", "k", "v", "z", "u", "dt"])
    x, _, _, x_out, _ = _gpu_step(w, inp, alpha=np.zeros_like(inp["alpha"]))
    assert torch.equal(x_out, x)


def test_step_captured_in_a_graph_replays_bitwise():
    """The whole step (modulate, RoPE in place on fresh copies of q and k,
    attention, residual with the fused Euler update) captured into one graph and
    replayed three times, with eager runs of the same step between the replays:
    every replay's outputs equal the eager outputs bit for bit (no entry point of
    the step keeps state between launches or records a memset; attention under
    capture takes its one-block-per-item form, which is what the eager launch
    takes at this size)."""
    need_gpu()
    w = CHAIN[1]
    inp = synth.make(w, ["x", "gamma", "beta", "alpha", "q", "k", "v", "z", "u", "dt"])
    x, q0, k0, v, z, u = (dev(inp[n], w) for n in ("x", "q", "k", "v", "z", "u"))
    g, b, al, dt = dev(inp["gamma"]), dev(inp["beta"]), dev(inp["alpha"]), dev(inp["dt"])
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    grid = (w.frames[0], *w.grid_hw)

    def step(q, k, y, o, x_out, z_out):
        q.copy_(q0)
        k.copy_(k0)
        dit.dit_adaln_modulate(y, x, g, b, w.tokens_per_row, w.eps)
        dit.dit_rope3d(q, k, grid, w.rope_split, w.rope_base, cu_seqlens=cu, num_seqs=w.num_seqs)
        dit.dit_attn3d(o, q, k, v, cu_seqlens=cu, max_seqlen=w.max_seqlen)
        dit.dit_gated_residual(x_out, x, o.view(w.tokens, w.d_model), al, w.tokens_per_row,
                               euler=(z_out, z, u, dt, w.tokens_per_row))

    def buffers():
        return (torch.empty_like(q0), torch.empty_like(k0), torch.empty_like(x), torch.empty_like(q0),
                torch.empty_like(x), torch.empty_like(z))

    eager = buffers()
    step(*eager)
    torch.cuda.synchronize()
    cap = buffers()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(*cap)
    for r in range(3):
        for t in cap:
            t.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, e in zip(("q", "k", "y", "o", "x'", "z'"), cap, eager):
            assert torch.equal(a, e), (r, name)
        again = buffers()
        step(*again)
        torch.cuda.synchronize()
        for a, e in zip(again, eager):
            assert torch.equal(a, e), r
