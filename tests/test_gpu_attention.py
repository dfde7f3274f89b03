"""GPU parity of dit_attn3d (bf16 MFMA and fp32 paths) against the float64
oracle, through the C-ABI binding: tiny and ragged shapes in full, the
full-size workloads on sampled query rows (all heads, exact full-row softmax)."""
import numpy as np
import pytest
import torch

import diffusion_transformer_video_amd as dit
import synth
from gpu_util import TOL, dev, host64, maxabs, need_gpu, note, sample_rows
from oracle import attention as o_attn

pytestmark = pytest.mark.gpu


def _seq_workload(name, dtype, seqlens, heads, hd, seed=11):
    # a 1 x n grid per sequence: attention does not look at positions
    frames = tuple(seqlens)
    return synth.custom(name, dtype, (1, 1), frames, heads, hd, (0, hd // 2, hd // 2), seed=seed)


def _run(w, inp, rows=None, packed=None):
    q, k, v = (dev(inp[n], w) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    packed = (not w.dense) if packed is None else packed
    if packed:
        cu = torch.from_numpy(w.cu_seqlens).cuda()
        dit.dit_attn3d(o, q, k, v, cu_seqlens=cu, max_seqlen=w.max_seqlen)
    else:
        dit.dit_attn3d(o, q, k, v, num_seqs=w.num_seqs)
    torch.cuda.synchronize()
    if rows is None:
        return host64(o)
    return host64(o[torch.from_numpy(rows).cuda()])


def _check(w, rows=None, packed=None):
    need_gpu()
    inp = synth.make(w, ["q", "k", "v"])
    got = _run(w, inp, rows, packed)
    ref = o_attn.attention(inp["q"], inp["k"], inp["v"], w.cu_seqlens, rows=rows)
    err = maxabs(got, ref)
    note(f"attn {w.name} ({w.dtype}, seqlens {w.seqlens[:4]}{'...' if w.num_seqs > 4 else ''}, "
         f"heads {w.heads}, hd {w.head_dim}, packed {packed}): max-abs {err:.3e}")
    assert err <= TOL[w.dtype]


TINY = [(n, hd) for n in (1, 7, 33, 64, 65, 127, 200, 1000) for hd in (64, 128)]


@pytest.mark.parametrize("n,hd", TINY, ids=[f"n{n}_hd{hd}" for n, hd in TINY])
def test_bf16_single_sequence(n, hd):
    _check(_seq_workload(f"bf16_n{n}", "bf16", (n,), 2, hd))


@pytest.mark.parametrize("hd", [64, 128])
def test_bf16_dense_batch(hd):
    _check(_seq_workload("bf16_b3", "bf16", (300, 300, 300), 3, hd))


@pytest.mark.parametrize("hd", [64, 128])
def test_bf16_packed_varlen(hd):
    _check(_seq_workload("bf16_varlen", "bf16", (1, 65, 134, 133, 64, 257), 3, hd))


def test_bf16_packed_equals_dense_when_lengths_match():
    need_gpu()
    w = _seq_workload("bf16_pd", "bf16", (256, 256), 2, 128)
    inp = synth.make(w, ["q", "k", "v"])
    a = _run(w, inp, packed=False)
    b = _run(w, inp, packed=True)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("n,hd", [(1, 64), (7, 128), (100, 64), (129, 128)])
def test_f32_small(n, hd):
    _check(_seq_workload(f"f32_n{n}", "f32", (n,), 2, hd))


def test_f32_varlen():
    _check(_seq_workload("f32_varlen", "f32", (3, 64, 70), 2, 64))


def test_c1_tiny_block_f32():
    _check(synth.C1)


@pytest.mark.parametrize("w", [synth.C2, synth.C3, synth.C4, synth.C5], ids=lambda w: w.name)
def test_full_size_sampled_rows(w):
    _check(w, rows=sample_rows(w, per_seq=48 if w.tokens > 10000 else 128))


# Launches with at least 4 work items per resident block take the persistent
# path (one block per compute unit, items drawn from per-XCD queues); smaller
# ones run one block per item. Every item is computed by the same code either
# way, so a sequence's output cannot depend on which path ran it.
PERSISTENT = [(128, 16), (64, 32)]   # (head_dim, heads): packed (8192, 300) takes the persistent path


@pytest.mark.parametrize("hd,heads", PERSISTENT, ids=[f"hd{hd}" for hd, _ in PERSISTENT])
def test_persistent_launch_sampled_rows(hd, heads):
    w = _seq_workload(f"pers{hd}", "bf16", (8192, 300), heads, hd)
    _check(w, rows=sample_rows(w, per_seq=64))


@pytest.mark.parametrize("hd,heads", PERSISTENT, ids=[f"hd{hd}" for hd, _ in PERSISTENT])
def test_persistent_equals_per_item_launch(hd, heads):
    """The 300-token sequence of the persistent launch above, bit for bit the
    same as that sequence attended alone (a one-block-per-item launch)."""
    need_gpu()
    big = _seq_workload(f"pers{hd}", "bf16", (8192, 300), heads, hd)
    inp = synth.make(big, ["q", "k", "v"])
    got_big = _run(big, inp)
    small = _seq_workload(f"pers{hd}_tail", "bf16", (300,), heads, hd)
    got_small = _run(small, {n: inp[n][8192:] for n in ("q", "k", "v")})
    assert np.array_equal(got_big[8192:], got_small)


def test_persistent_launch_many_sequences():
    """A packed batch of 40 ragged sequences (more than 32: the item numbering
    walks them in index order) large enough for the persistent launch (2,304
    query tiles over 12 heads), on sampled rows of every sequence."""
    r = np.random.default_rng(17)
    lens = tuple(int(n) for n in r.integers(1, 2400, size=40))
    w = _seq_workload("pers_many", "bf16", lens, 12, 128)
    assert sum(-(-n // 256) for n in lens) * 12 >= 1024
    _check(w, rows=sample_rows(w, per_seq=8, edge=2))


def test_persistent_queue_slots_reused():
    """More persistent launches in a row than there are queue-counter slots (each
    launch's last block clears its slot for the next launch that uses it):
    every launch gives the same output, bit for bit."""
    need_gpu()
    w = _seq_workload("pers_slots", "bf16", (8192, 300), 16, 128)
    inp = synth.make(w, ["q", "k", "v"])
    q, k, v = (dev(inp[n], w) for n in ("q", "k", "v"))
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    ref = torch.empty_like(q)
    dit.dit_attn3d(ref, q, k, v, cu_seqlens=cu, max_seqlen=w.max_seqlen)
    o = torch.empty_like(q)
    for i in range(140):
        o.fill_(0.0)
        dit.dit_attn3d(o, q, k, v, cu_seqlens=cu, max_seqlen=w.max_seqlen)
        assert torch.equal(o, ref), i


def test_ulysses_share_shape():
    """One GPU's share of the 480P video workload under head-sharded context
    parallelism over 8 GPUs: 5 heads x 32,760 tokens."""
    w = synth.Workload("c3_share_5heads", "bf16", (30, 52), (21,), (32760,), 5, 128, (44, 42, 42),
                       10000.0, 32760, 1103)
    _check(w, rows=sample_rows(w, per_seq=64))


def test_ones_values_and_identical_keys():
    need_gpu()
    w = _seq_workload("inv", "bf16", (777,), 2, 128)
    inp = synth.make(w, ["q", "k", "v"])
    inp["v"] = np.ones_like(inp["v"])
    got = _run(w, inp)
    assert maxabs(got, np.ones_like(got)) <= 2e-2
    inp = synth.make(w, ["q", "v"])
    inp["k"] = synth.uniform_keys(w)
    got = _run(w, inp)
    mean_v = inp["v"].astype(np.float64).mean(axis=0)
    assert maxabs(got, np.broadcast_to(mean_v, got.shape)) <= 2e-2


def test_deterministic_bitwise():
    need_gpu()
    w = _seq_workload("det", "bf16", (1000, 555), 4, 128)
    inp = synth.make(w, ["q", "k", "v"])
    a = _run(w, inp)
    b = _run(w, inp)
    assert np.array_equal(a, b)


def test_rows_past_end_untouched():
    """The kernel writes exactly the output tensor: a guard band around o keeps
    its canary values (ragged tail, packed batch)."""
    need_gpu()
    w = _seq_workload("guard", "bf16", (65, 130), 2, 128)
    inp = synth.make(w, ["q", "k", "v"])
    q, k, v = (dev(inp[n], w) for n in ("q", "k", "v"))
    per = w.heads * w.head_dim
    buf = torch.full((w.tokens + 64, per), 7.0, dtype=torch.bfloat16, device="cuda")
    o = buf[32:32 + w.tokens].view(w.tokens, w.heads, w.head_dim)
    dit.dit_attn3d(o, q, k, v, cu_seqlens=torch.from_numpy(w.cu_seqlens).cuda(), max_seqlen=130)
    torch.cuda.synchronize()
    assert torch.all(buf[:32] == 7.0) and torch.all(buf[32 + w.tokens:] == 7.0)
