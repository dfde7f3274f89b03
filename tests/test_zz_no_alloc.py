"""dit_attn3d_noalloc, the allocation-free form of dit_attn3d, against dit_attn3d
through the C-ABI binding: two calls in a row that take the persistent launch
(so its queue counters live in the library's static scratch slot), the second
with a smaller input; then a packed varlen call at head_dim 64 and a float32
call. Bar: the bf16 bar of the attention tests (2e-2 max-abs) against
dit_attn3d's output and against the float64 oracle on sampled rows, and bit
for bit on every head whose work items dit_attn3d's launch does not cut along
the keys (the allocation-free launch never cuts, and uncut items run the same
code in both)."""
import numpy as np
import pytest
import torch

import diffusion_transformer_video_amd as dit
import synth
from gpu_util import TOL, attn_items_total, dev, host64, item_rows, maxabs, need_gpu, note, sample_rows, split_items
from oracle import attention as o_attn

pytestmark = pytest.mark.gpu


def _workload(name, dtype, seqlens, heads, hd, seed):
    return synth.custom(name, dtype, (1, 1), tuple(seqlens), heads, hd, (0, hd // 2, hd // 2), seed=seed)


def _split_heads(w):
    """Heads with a work item that dit_attn3d's persistent launch of w cuts along the keys."""
    if w.head_dim != 128:
        return set()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return {item_rows(w, i)[0] for i in split_items(attn_items_total(w), cus)}


def _both(w):
    inp = synth.make(w, ["q", "k", "v"])
    q, k, v = (dev(inp[n], w) for n in ("q", "k", "v"))
    o_ref, o_na = torch.empty_like(q), torch.empty_like(q)
    o_na.fill_(float("nan"))   # every element must be written
    kw = dict(num_seqs=w.num_seqs) if w.dense else dict(cu_seqlens=torch.from_numpy(w.cu_seqlens).cuda(),
                                                        max_seqlen=w.max_seqlen)
    dit.dit_attn3d(o_ref, q, k, v, **kw)
    dit.dit_attn3d_noalloc(o_na, q, k, v, **kw)
    torch.cuda.synchronize()
    return inp, o_ref, o_na


def _check(w):
    need_gpu()
    inp, o_ref, o_na = _both(w)
    got = host64(o_na)
    ref = host64(o_ref)
    err_ref = maxabs(got, ref)
    split = _split_heads(w)
    keep = [h for h in range(w.heads) if h not in split]
    same = np.array_equal(got[:, keep], ref[:, keep])
    rows = sample_rows(w, per_seq=32, edge=4)
    err_or = maxabs(got[rows], o_attn.attention(inp["q"], inp["k"], inp["v"], w.cu_seqlens, rows=rows))
    note(f"noalloc {w.name} ({w.dtype}, seqlens {w.seqlens}, heads {w.heads}, hd {w.head_dim}): "
         f"vs dit_attn3d max-abs {err_ref:.3e}, bitwise on {len(keep)}/{w.heads} uncut heads {same}; "
         f"vs oracle on {len(rows)} rows {err_or:.3e}")
    assert err_ref <= TOL[w.dtype]
    assert same
    assert err_or <= TOL[w.dtype]


def test_noalloc_two_calls_second_smaller():
    """16,384 then 8,192 tokens x 40 heads x 128: 2,560 and 1,280 work items,
    both at least 4 per compute unit (the persistent form on a 256-CU device)."""
    _check(_workload("na_16k", "bf16", (16384,), 40, 128, seed=71))
    _check(_workload("na_8k", "bf16", (8192,), 40, 128, seed=72))


def test_noalloc_packed_head_dim_64():
    """Packed (8192, 300) x 32 heads x 64: 2,144 items of 128 queries, the
    persistent form of the two-blocks-per-CU kernel."""
    _check(_workload("na_hd64", "bf16", (8192, 300), 32, 64, seed=73))


def test_noalloc_float32():
    need_gpu()
    w = _workload("na_f32", "f32", (300, 77), 2, 64, seed=74)
    _, o_ref, o_na = _both(w)
    assert torch.equal(o_ref, o_na)


def test_noalloc_graph_replays_bitwise():
    """Captured into a graph (its clear kernel and its persistent launch, with the
    scratch slot's address baked in) and replayed three times, with eager calls of
    both entry points and synchronisations between the replays: every replay
    equals the eager allocation-free result bit for bit, so the slot is cleared
    for each replay and left clean for the eager calls."""
    need_gpu()
    w = _workload("na_graph", "bf16", (8192,), 40, 128, seed=75)
    inp = synth.make(w, ["q", "k", "v"])
    q, k, v = (dev(inp[n], w) for n in ("q", "k", "v"))
    eager = torch.empty_like(q)
    dit.dit_attn3d_noalloc(eager, q, k, v)
    torch.cuda.synchronize()
    cap = torch.empty_like(q)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dit.dit_attn3d_noalloc(cap, q, k, v)
    ref = torch.empty_like(q)
    for r in range(3):
        cap.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(cap, eager), r
        again = torch.empty_like(q)
        dit.dit_attn3d_noalloc(again, q, k, v)
        dit.dit_attn3d(ref, q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(again, eager), r
    note(f"noalloc graph: 3 replays bitwise equal to the eager call ({w.tokens} tokens x {w.heads} heads)")
