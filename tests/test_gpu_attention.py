"""GPU parity of dit_attn3d (bf16 MFMA and fp32 paths) against the float64
oracle, through the C-ABI binding: tiny and ragged shapes in full, the
full-size workloads on sampled query rows (all heads, exact full-row softmax)."""
import numpy as np
import pytest
import torch

import diffusion_transformer_video_amd as dit
import synth
from gpu_util import TOL, attn_items_total, dev, host64, item_rows, maxabs, need_gpu, note, sample_rows, split_items
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


def tile_rows(w, n_random=2048, bq=256, seed=7):
    """Rows that reach every work item of every head at full size: the first and
    last rows of every sequence, one seeded row inside every 256-query tile of
    every sequence, and n_random seeded rows over all tokens."""
    r = np.random.default_rng(seed)
    rows = list(sample_rows(w, per_seq=0, edge=4))
    for s in range(w.num_seqs):
        lo, hi = int(w.cu_seqlens[s]), int(w.cu_seqlens[s + 1])
        for t0 in range(lo, hi, bq):
            rows.append(int(r.integers(t0, min(t0 + bq, hi))))
    rows += list(r.choice(w.tokens, size=min(n_random, w.tokens), replace=False))
    return np.unique(np.asarray(rows, dtype=np.int64))


def test_full_size_image_every_row():
    """The image workload (2 x 4,096 tokens, 24 heads): every output row."""
    _check(synth.C2)


@pytest.mark.parametrize("w", [synth.C3, synth.C4, synth.C5], ids=lambda w: w.name)
def test_full_size_tile_rows(w):
    """Video and packed workloads: a row in every 256-query tile of every
    sequence (so every work item of every head is compared), sequence edges,
    and 2,048 seeded rows, all heads, exact full-row softmax."""
    _check(w, rows=tile_rows(w))


@pytest.mark.parametrize("w", [synth.C3, synth.C4, synth.C5], ids=lambda w: w.name)
def test_full_size_one_whole_head(w):
    """Every row of one seeded head at full size."""
    need_gpu()
    h = int(np.random.default_rng(w.seed).integers(w.heads))
    inp = synth.make(w, ["q", "k", "v"])
    got = _run(w, inp)[:, h]
    ref = o_attn.attention(inp["q"][:, h:h + 1], inp["k"][:, h:h + 1], inp["v"][:, h:h + 1], w.cu_seqlens)[:, 0]
    err = maxabs(got, ref)
    note(f"attn {w.name} head {h}, every row: max-abs {err:.3e}")
    assert err <= TOL[w.dtype]


# Launches with at least 4 work items per resident block (or 2, when one block
# per item would leave its last round under 90% full) take the persistent path
# (one block per compute unit, items drawn from per-XCD queues); smaller ones
# run one block per item. An item the persistent launch does not split is
# computed by the same code either way, so its output cannot depend on which
# path ran it.
PERSISTENT = [(128, 16), (64, 32)]   # (head_dim, heads): packed (8192, 300) takes the persistent path


@pytest.mark.parametrize("hd,heads", PERSISTENT, ids=[f"hd{hd}" for hd, _ in PERSISTENT])
def test_persistent_launch_sampled_rows(hd, heads):
    w = _seq_workload(f"pers{hd}", "bf16", (8192, 300), heads, hd)
    _check(w, rows=sample_rows(w, per_seq=64))


@pytest.mark.parametrize("hd,heads", PERSISTENT, ids=[f"hd{hd}" for hd, _ in PERSISTENT])
def test_persistent_equals_per_item_launch(hd, heads):
    """The 300-token sequence of the persistent launch above, bit for bit the
    same as that sequence attended alone (a one-block-per-item launch), on
    every head whose items the persistent launch did not split along the keys
    (split items sum their keys in pieces: checked against the oracle in
    test_split_tail_against_oracle)."""
    need_gpu()
    big = _seq_workload(f"pers{hd}", "bf16", (8192, 300), heads, hd)
    inp = synth.make(big, ["q", "k", "v"])
    got_big = _run(big, inp)
    small = _seq_workload(f"pers{hd}_tail", "bf16", (300,), heads, hd)
    got_small = _run(small, {n: inp[n][8192:] for n in ("q", "k", "v")})
    keep = [h for h in range(heads) if h not in _split_heads(big)]
    assert keep
    assert np.array_equal(got_big[8192:, keep], got_small[:, keep])


def _split_heads(w):
    """Heads with an item that a persistent launch of w splits along the keys."""
    if w.head_dim != 128:
        return set()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return {item_rows(w, i)[0] for i in split_items(attn_items_total(w), cus)}


def _same_launch(got, ref, split_heads):
    """got against ref from another launch of the same call: bit for bit on heads
    no launch form splits, within the bf16 bar on the others (a split item sums
    its keys in pieces, a one-block-per-item launch in one pass)."""
    keep = [h for h in range(got.shape[1]) if h not in split_heads]
    if not torch.equal(got[:, keep], ref[:, keep]):
        return False
    cut = sorted(split_heads)
    return not cut or float((got[:, cut].float() - ref[:, cut].float()).abs().max()) <= TOL["bf16"]


def test_concurrent_streams():
    """Eight streams issuing ten persistent-size launches each without waiting
    for one another: 80 launches in flight against 64 queue-counter slots and
    one split array, so some launches share nothing and run one block per item
    or unsplit. Every output equals the launch run alone."""
    need_gpu()
    w = _seq_workload("pers_streams", "bf16", (8192, 300), 16, 128)
    inp = synth.make(w, ["q", "k", "v"])
    q, k, v = (dev(inp[n], w) for n in ("q", "k", "v"))
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    ref = torch.empty_like(q)
    dit.dit_attn3d(ref, q, k, v, cu_seqlens=cu, max_seqlen=w.max_seqlen)
    streams = [torch.cuda.Stream() for _ in range(8)]
    outs = [[torch.empty_like(q) for _ in range(10)] for _ in streams]
    torch.cuda.synchronize()
    for r in range(10):
        for s, o in zip(streams, outs):
            with torch.cuda.stream(s):
                dit.dit_attn3d(o[r], q, k, v, cu_seqlens=cu, max_seqlen=w.max_seqlen)
    torch.cuda.synchronize()
    split_heads = _split_heads(w)
    for i, o in enumerate(outs):
        for r, x in enumerate(o):
            assert _same_launch(x, ref, split_heads), (i, r)


def test_graph_capture_replays():
    """The call captured into a graph (under capture it runs one block per item,
    which keeps no device state between launches) and replayed three times, with
    eager launches of the same call between the replays: every replay equals the
    eager output, and the eager launches stay bit-identical."""
    need_gpu()
    w = _seq_workload("pers_graph", "bf16", (8192, 300), 16, 128)
    inp = synth.make(w, ["q", "k", "v"])
    q, k, v = (dev(inp[n], w) for n in ("q", "k", "v"))
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    ref = torch.empty_like(q)
    dit.dit_attn3d(ref, q, k, v, cu_seqlens=cu, max_seqlen=w.max_seqlen)
    torch.cuda.synchronize()
    o = torch.empty_like(q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dit.dit_attn3d(o, q, k, v, cu_seqlens=cu, max_seqlen=w.max_seqlen)
    split_heads = _split_heads(w)
    first = None
    for r in range(3):
        o.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same_launch(o, ref, split_heads), r
        if first is None:
            first = o.clone()
        assert torch.equal(o, first), r
        eager = torch.empty_like(q)
        dit.dit_attn3d(eager, q, k, v, cu_seqlens=cu, max_seqlen=w.max_seqlen)
        torch.cuda.synchronize()
        assert torch.equal(eager, ref), r


def test_persistent_launch_many_sequences():
    """A packed batch of 40 ragged sequences (more than 32: the item numbering
    walks them in index order) large enough for the persistent launch (2,304
    query tiles over 12 heads), on sampled rows of every sequence."""
    r = np.random.default_rng(17)
    lens = tuple(int(n) for n in r.integers(1, 2400, size=40))
    w = _seq_workload("pers_many", "bf16", lens, 12, 128)
    assert sum(-(-n // 256) for n in lens) * 12 >= 1024
    _check(w, rows=sample_rows(w, per_seq=8, edge=2))


def test_persistent_launch_with_few_items():
    """The launch form is chosen from the grid bound (longest sequence x heads x
    sequences), not the item count: one 8,192-token sequence and 63 one-token
    sequences on one head give a grid of 2,048 (the persistent form) but only 95
    work items, so most blocks find their XCD's queue empty at once and some
    XCD ranges hold a dozen items. Every row against the oracle."""
    lens = (8192,) + (1,) * 63
    w = _seq_workload("pers_few", "bf16", lens, 1, 128, seed=41)
    assert -(-max(lens) // 256) * w.heads * w.num_seqs >= 4 * 256
    _check(w)


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


def test_full_size_head_dim_64():
    """The other supported head size at the 480P video workload's tokens and
    d_model: 32,760 tokens x 80 heads x 64 (the persistent launch's 4-wave
    blocks, two per CU). A row in every 256-query tile of every head, the
    sequence edges and 2,048 seeded rows, all heads, against the oracle."""
    w = synth.Workload("c3_hd64_80heads", "bf16", (30, 52), (21,), (32760,), 80, 64, (20, 22, 22),
                       10000.0, 32760, 1113)
    _check(w, rows=tile_rows(w))


def test_full_size_peaked_scores():
    """The 480P video workload with q and k four times larger (scores 16 times
    larger: sharply peaked rows whose running max keeps rising, so the lazy
    rescale runs throughout the persistent launch and its split tail), on a row
    in every 256-query tile of every head, the edges and 2,048 seeded rows."""
    need_gpu()
    w = synth.C3
    inp = synth.make(w, ["q", "k", "v"])
    inp["q"] = synth.bf16_round(np.asarray(inp["q"], np.float32) * 4.0)
    inp["k"] = synth.bf16_round(np.asarray(inp["k"], np.float32) * 4.0)
    rows = tile_rows(w)
    got = _run(w, inp, rows)
    ref = o_attn.attention(inp["q"], inp["k"], inp["v"], w.cu_seqlens, rows=rows)
    err = maxabs(got, ref)
    note(f"attn {w.name}, q and k x4: max-abs {err:.3e}")
    assert err <= TOL[w.dtype]


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


# The persistent launch cuts the last work items of each XCD's range along the
# keys (pieces merged by log-sum-exp in the kernel); these shapes put different
# plans on the tail: 480P (the whole last round in halves), 720P (one item per
# XCD in 16 pieces), one GPU's Ulysses share (16 items per XCD in halves),
# ragged packed sequences, and short sequences with more pieces than key tiles
# (empty pieces).
SPLIT_CASES = {
    "video480p": lambda: synth.C3,
    "video720p": lambda: synth.C4,
    "ulysses_share": lambda: synth.Workload("c3_share_5heads", "bf16", (30, 52), (21,), (32760,), 5, 128,
                                            (44, 42, 42), 10000.0, 32760, 1103),
    "ragged": lambda: _seq_workload("split_ragged", "bf16", (1000, 513, 77), 80, 128, seed=23),
    "empty_pieces": lambda: _seq_workload("split_empty", "bf16", (2000, 50), 200, 128, seed=29),
}


@pytest.mark.parametrize("case", sorted(SPLIT_CASES))
def test_split_tail_against_oracle(case):
    """Every row of every split work item (its head) against the oracle, plus one
    unsplit item per XCD range as a control; the launch's plan is computed from
    the device's compute-unit count."""
    need_gpu()
    w = SPLIT_CASES[case]()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    total = attn_items_total(w)
    plan = split_items(total, cus)
    if not plan:
        pytest.skip(f"{total} items on {cus} compute units: no split tail")
    inp = synth.make(w, ["q", "k", "v"])
    q, k, v = (dev(inp[n], w) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    if w.dense:
        dit.dit_attn3d(o, q, k, v, num_seqs=w.num_seqs)
    else:
        dit.dit_attn3d(o, q, k, v, cu_seqlens=torch.from_numpy(w.cu_seqlens).cuda(), max_seqlen=w.max_seqlen)
    torch.cuda.synchronize()
    items = sorted(plan)
    # a control: the first item of every XCD range is never split
    items += [x * (total // 8) for x in range(8)]
    by_head = {}
    for it in items:
        h, rows = item_rows(w, it)
        by_head.setdefault(h, []).append(rows)
    worst = 0.0
    for h, parts in by_head.items():
        rows = np.unique(np.concatenate(parts))
        ref = o_attn.attention(inp["q"][:, h:h + 1], inp["k"][:, h:h + 1], inp["v"][:, h:h + 1], w.cu_seqlens,
                               rows=rows)[:, 0]
        got = host64(o[torch.from_numpy(rows).cuda(), h])
        worst = max(worst, maxabs(got, ref))
    note(f"split tail {case}: {len(plan)} split items ({sorted(set(plan.values()))} pieces), "
         f"{len(by_head)} heads checked, max-abs {worst:.3e}")
    assert worst <= TOL["bf16"]
