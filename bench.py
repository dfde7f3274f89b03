#!/usr/bin/env python3
"""Throughput of the DiT attention-block hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  dit_adaln_modulate (x -> y), dit_rope3d (q, k in place), dit_attn3d (q, k, v -> o),
  dit_gated_residual fused with the rectified-flow Euler update (x + alpha*o, z + dt*u).
Inputs are seeded synthetic tensors shaped like the pages' video latents (default:
the 480P latent T=21, H=60, W=104, patch 1x2x2 -> 32,760 tokens, 40 heads x 128,
3D-RoPE 44/42/42), resident in HBM before timing starts.

Prints ONE JSON line. value = attention FLOPs per step / wall time per step
(whole path), in TFLOP/s. roofline = the attention kernel's own rate, timed with
HIP events (without the system-scope fence) around each of its launches on the
stream it runs on, against the 2.5 PFLOP/s dense bf16 MFMA peak. cpu_baseline = the float64 numpy oracle on a
bounded sample of the same workload, scaled to the whole step.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0
WORKLOAD_KEYS = {"c1": "c1_tiny_f32", "c2": "c2_image_4096_bf16", "c3": "c3_video480p_32760_bf16",
                 "c4": "c4_video720p_27280_bf16", "c5": "c5_varlen_frames_bf16"}
CSRC = os.path.join(ROOT, "diffusion_transformer_video_amd", "csrc")
# what the bf16 attention kernel's machine code is built from
ATTN_SRCS = [os.path.join(CSRC, f) for f in ("k_attn_bf16.hip", "dit_attn_common.hpp", "dit_device.hpp",
                                            "dit_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50,
                   help="timed steps (50 attention launches bracketed by events at the default)")
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--warmup-min-s", type=float, default=0.0,
                   help="optional floor: keep running untimed warmup steps beyond --warmup until "
                        "this much wall time has passed (an idle MI355X needs about 40 ms of load "
                        "to reach its sustained clocks; 5 steps of the 480P workload take ~95 ms, "
                        "5 steps of the image workload only ~2.5 ms). Off by default: exactly "
                        "--warmup steps run")
    p.add_argument("--workload", default="c3", choices=sorted(WORKLOAD_KEYS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time budget of the oracle sample")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="after timing, run a plain device copy of this many MiB (read once, "
                        "written once) so hardware byte counters can be scaled against it")
    return p.parse_args()


class TimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence (0x20000000).

    Recording a default event performs a system-scope release: the L2 is written
    back before the event completes, which holds the next kernel on the stream
    for ~5 us. The attention launches inside the timed steps are bracketed with
    these events instead, so that the brackets do not lengthen the steps they
    measure. They come from the HIP runtime torch has already loaded (the one the
    kernels' library shares), found in this process's memory map."""

    _hip = None

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64.so" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded in this process")
            L = ctypes.CDLL(path)
            vp = ctypes.c_void_p
            L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            L.hipEventRecord.argtypes = [vp, vp]
            L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            L.hipEventDestroy.argtypes = [vp]
            cls._hip = L
        return cls._hip

    def __init__(self):
        import torch
        # recorded on the stream current at creation: the one the kernels run on
        self.stream = ctypes.c_void_p(int(torch.cuda.current_stream().cuda_stream))
        self.ev = ctypes.c_void_p()
        rc = self._runtime().hipEventCreateWithFlags(ctypes.byref(self.ev), 0x20000000)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        rc = self._hip.hipEventRecord(self.ev, self.stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        ms = ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


def attn_kernel_name(w):
    """The bf16 attention kernel the library launches for this workload: the
    persistent form on the whole chip (256 CUs) from 4 query tiles (256 queries)
    per compute unit, or from 2 when one block per tile would leave the last
    round under 90% full (the rule dit_attn3d documents); else one block per
    tile."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = -(-w.max_seqlen // 256) * w.heads * w.num_seqs
    last = grid % cus
    pers = cus == 256 and (grid >= 4 * cus or (grid >= 2 * cus and last != 0 and 10 * last < 9 * cus))
    return "attn_bf16_persistent<128,8,1>" if pers else "attn_bf16_kernel<128,8,1>"


def kernel_sha():
    """Hash of the bf16 attention kernel's sources (comments and blank lines
    dropped) and its per-file compile flags: hardware-counter figures belong to
    one build of the kernel."""
    import re

    from diffusion_transformer_video_amd import build as _build
    h = hashlib.sha256()
    for p in ATTN_SRCS:
        code = re.sub(r"//[^\n]*", "", open(p).read())
        h.update("\n".join(l.rstrip() for l in code.splitlines() if l.strip()).encode())
    h.update(repr(_build.FILE_FLAGS.get("k_attn_bf16.hip", [])).encode())
    return h.hexdigest()[:16]


def traffic_for(workload):
    """HBM bytes per attention launch from committed rocprofv3 counter runs, or
    None if there are none for this workload or the kernel changed since."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("source_sha") != kernel_sha():
        return None
    return e.get("traffic_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(sharding is a design note only); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import diffusion_transformer_video_amd as dit
    import synth

    w = synth.WORKLOADS[WORKLOAD_KEYS[args.workload]]
    torch.cuda.set_device(0)
    dit.lib()
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    esz = 2 if w.dtype == "bf16" else 4

    inp = synth.make(w, ["x", "gamma", "beta", "alpha", "q", "k", "v", "z", "u", "dt"])
    d = lambda a, t=tdt: torch.from_numpy(np.ascontiguousarray(a)).to(t).cuda()
    x, q, k, v, z, u = (d(inp[n]) for n in ("x", "q", "k", "v", "z", "u"))
    g, b, al, dtr = (d(inp[n], torch.float32) for n in ("gamma", "beta", "alpha", "dt"))
    cu = None if w.dense else torch.from_numpy(w.cu_seqlens).cuda()
    y, o = torch.empty_like(x), torch.empty_like(q)
    x_out, z_out = torch.empty_like(x), torch.empty_like(z)
    o2d = o.view(w.tokens, w.d_model)
    grid = (w.frames[0], *w.grid_hw)
    del inp

    def launch(name):
        if name == "modulate":
            dit.dit_adaln_modulate(y, x, g, b, w.tokens_per_row, w.eps)
        elif name == "rope":
            dit.dit_rope3d(q, k, grid, w.rope_split, w.rope_base, cu_seqlens=cu, num_seqs=w.num_seqs)
        elif name == "attn":
            if cu is None:
                dit.dit_attn3d(o, q, k, v, num_seqs=w.num_seqs)
            else:
                dit.dit_attn3d(o, q, k, v, cu_seqlens=cu, max_seqlen=w.max_seqlen)
        else:
            dit.dit_gated_residual(x_out, x, o2d, al, w.tokens_per_row,
                                   euler=(z_out, z, u, dtr, w.tokens_per_row))

    attn_ev = []

    def step(record):
        launch("modulate")
        launch("rope")
        if record:   # the dominant kernel, bracketed on the stream it runs on
            a0, a1 = TimingEvent(), TimingEvent()
            a0.record()
            launch("attn")
            a1.record()
            attn_ev.append((a0, a1))
        else:
            launch("attn")
        launch("residual_euler")

    warm_steps = 0
    t_warm = time.time()
    while warm_steps < args.warmup or time.time() - t_warm < args.warmup_min_s:
        step(False)
        warm_steps += 1
        if warm_steps % 8 == 0:
            torch.cuda.synchronize()   # the wall clock must see the GPU's progress
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: {warm_steps} warmup steps done, timing {args.steps} steps",
          file=sys.stderr, flush=True)

    # timed region: K whole steps; the attention launches inside it carry their own events
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step(True)
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    attn_each = [a.elapsed_time(bb) for a, bb in attn_ev]
    kern_ms = {"attn": float(np.mean(attn_each))}

    # the short bandwidth-bound kernels: batches of back-to-back launches between two
    # events (a single launch is too short for an event pair to time it faithfully),
    # rotating over buffer copies worth >= 1 GiB so that no launch is served from the
    # 256 MB last-level cache
    def rotation(nbytes):
        return max(2, min(16, -(-(1 << 30) // nbytes)))

    def timed_batch(fns):
        """Mean GPU time per launch of fns, launched back to back. A spin kernel
        (torch.cuda._sleep) holds the stream while the host enqueues the timed
        launches, so that they run with no idle gap between them: the host's
        per-call cost (argument checks, ctypes; ~20 us) would otherwise leave the
        GPU idle between kernels that take ~20 us themselves. The spin is sized
        from the host's measured enqueue time and lies before the first event."""
        t = time.perf_counter()
        for f in fns:   # warm, and time the host's enqueue rate
            f()
        host_s = time.perf_counter() - t
        torch.cuda.synchronize()
        cycles = int(min(2e8, max(2e6, 2 * 2 * host_s * 2.5e9)))   # 2 rounds, 2x margin, >= 2.4 GHz
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        spin = getattr(torch.cuda, "_sleep", None)   # absent: launches as the host issues them
        if spin is not None:
            spin(cycles)
        e0.record()
        for _ in range(2):
            for f in fns:
                f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (2 * len(fns))

    R = rotation(2 * w.tokens * w.d_model * esz)
    xs = [x.clone() for _ in range(R)]
    ys = [torch.empty_like(x) for _ in range(R)]
    kern_ms["modulate"] = timed_batch([
        (lambda i=i: dit.dit_adaln_modulate(ys[i], xs[i], g, b, w.tokens_per_row, w.eps)) for i in range(R)])
    del ys
    R = rotation(4 * w.tokens * w.d_model * esz)
    qs = [q.clone() for _ in range(R)]
    ks = [k.clone() for _ in range(R)]
    kern_ms["rope"] = timed_batch([
        (lambda i=i: dit.dit_rope3d(qs[i], ks[i], grid, w.rope_split, w.rope_base, cu_seqlens=cu,
                                    num_seqs=w.num_seqs)) for i in range(R)])
    del qs, ks
    R = rotation(3 * w.tokens * w.d_model * esz)
    xs = xs[:R] + [x.clone() for _ in range(R - len(xs))]
    os_ = [o2d.clone() for _ in range(R)]
    xo = [torch.empty_like(x) for _ in range(R)]
    zs = [z.clone() for _ in range(R)]
    us = [u.clone() for _ in range(R)]
    zo = [torch.empty_like(z) for _ in range(R)]
    kern_ms["residual_euler"] = timed_batch([
        (lambda i=i: dit.dit_gated_residual(xo[i], xs[i], os_[i], al, w.tokens_per_row,
                                            euler=(zo[i], zs[i], us[i], dtr, w.tokens_per_row)))
        for i in range(R)])
    del xs, os_, xo, zs, us, zo

    # ring-attention building blocks (not part of the step): attention with the row
    # log-sum-exp (keys = the queries' own tokens, so its flops equal attn's), and
    # the fold of a bf16 partial into a float32 accumulator
    lse = torch.empty(w.tokens, w.heads, dtype=torch.float32, device="cuda")

    def attn_lse():
        if cu is None:
            dit.dit_attn3d_lse(o, lse, q, k, v, num_seqs=w.num_seqs)
        else:
            dit.dit_attn3d_lse(o, lse, q, k, v, cu, cu, max_seqlen_q=w.max_seqlen, max_seqlen_k=w.max_seqlen)
    attn_lse()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        attn_lse()
    e1.record()
    torch.cuda.synchronize()
    kern_ms["attn_lse"] = e0.elapsed_time(e1) / 3
    merge_bytes = w.tokens * w.d_model * (4 + 4 + esz) + w.tokens * w.heads * (4 + 4 + 4)
    R = rotation(merge_bytes)
    accs = [torch.zeros(w.tokens, w.heads, w.head_dim, dtype=torch.float32, device="cuda") for _ in range(R)]
    laccs = [lse.clone() for _ in range(R)]
    obs = [o.clone() for _ in range(R)]
    lbs = [lse.clone() for _ in range(R)]
    kern_ms["merge"] = timed_batch([(lambda i=i: dit.dit_attn_merge(accs[i], laccs[i], obs[i], lbs[i]))
                                    for i in range(R)])
    del accs, laccs, obs, lbs

    # 8-bit attention (not part of the bf16 step): E4M3 quantisation of q, k, v (per
    # head scales, V transposed) and the attention on the codes, same sequences
    if w.dtype == "bf16" and w.head_dim == 128:
        vs = dit.dit_fp8_v_stride(w.tokens, w.num_seqs)
        q8 = torch.empty(q.shape, dtype=torch.uint8, device="cuda")
        k8 = torch.empty_like(q8)
        v8t = torch.zeros((w.heads, w.head_dim, vs), dtype=torch.uint8, device="cuda")
        amax = torch.empty(3, w.heads, dtype=torch.float32, device="cuda")
        fp8_kw = ({"num_seqs": w.num_seqs, "max_seqlen": w.max_seqlen} if cu is None
                  else {"cu_seqlens": cu, "max_seqlen": w.max_seqlen})

        def quant():
            dit.dit_quant_fp8(q8, k8, v8t, amax, q, k, v, **fp8_kw)

        def attn_fp8():
            dit.dit_attn3d_fp8(o, q8, k8, v8t, amax, **fp8_kw)
        quant()
        attn_fp8()
        torch.cuda.synchronize()
        # as many launches as fill ~50 ms (at least 3), after the same again untimed
        # (a change of kernel re-ramps the clocks)
        t_one = time.time()
        attn_fp8()
        torch.cuda.synchronize()
        reps = max(3, int(0.05 / max(time.time() - t_one, 1e-6)))
        for _ in range(reps):
            attn_fp8()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            attn_fp8()
        e1.record()
        torch.cuda.synchronize()
        kern_ms["attn_fp8"] = e0.elapsed_time(e1) / reps
        # quantisation: reads q, k, v twice (amax, then codes), writes 3 byte-codes
        quant_bytes = 3 * w.tokens * w.d_model * (2 * esz + 1)
        R = rotation(quant_bytes)
        qs_ = [q.clone() for _ in range(R)]
        q8s = [torch.empty_like(q8) for _ in range(R)]

        def quant_i(i):
            dit.dit_quant_fp8(q8s[i], k8, v8t, amax, qs_[i], k, v, **fp8_kw)
        kern_ms["quant_fp8"] = timed_batch([(lambda i=i: quant_i(i)) for i in range(R)])
        del qs_, q8s, q8, k8, v8t

    # one GPU's share of Ulysses context parallelism at the 480P video workload on 8
    # GPUs (all 32,760 tokens, 40 / 8 = 5 heads): the attention each GPU runs
    # between the two all-to-alls (the collectives themselves are not part of
    # this single-GPU build)
    if w.dtype == "bf16" and w.head_dim == 128:
        ush = (32760, 5, 128)
        gen = torch.Generator(device="cuda").manual_seed(1003)
        uq, uk, uv = (torch.randn(ush, device="cuda", generator=gen).to(torch.bfloat16) for _ in range(3))
        uo = torch.empty_like(uq)

        def attn_share():
            dit.dit_attn3d(uo, uq, uk, uv, num_seqs=1)
        attn_share()
        torch.cuda.synchronize()
        for _ in range(3):
            attn_share()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            attn_share()
        e1.record()
        torch.cuda.synchronize()
        kern_ms["attn_ulysses_share"] = e0.elapsed_time(e1) / 5
        ulysses_flops = 4 * 32760 ** 2 * 5 * 128
        del uq, uk, uv, uo
        # the same workload's tokens and d_model as heads of 64 (the other head
        # size the attention kernel supports): 2 x 4096-token sequences here
        hsh = (w.tokens, w.heads * 2, 64)
        hq, hk, hv = (torch.randn(hsh, device="cuda", generator=gen).to(torch.bfloat16) for _ in range(3))
        ho = torch.empty_like(hq)
        hd64_kw = ({"num_seqs": w.num_seqs} if cu is None else {"cu_seqlens": cu, "max_seqlen": w.max_seqlen})

        def attn_hd64():
            dit.dit_attn3d(ho, hq, hk, hv, **hd64_kw)
        attn_hd64()
        torch.cuda.synchronize()
        for _ in range(3):
            attn_hd64()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            attn_hd64()
        e1.record()
        torch.cuda.synchronize()
        kern_ms["attn_hd64"] = e0.elapsed_time(e1) / 5
        del hq, hk, hv, ho

    # flow-matching training side (not part of the sampling step): the straight-path
    # interpolant and the flow-matching loss over the latent
    P_ = synth.LATENT_CHANNELS
    R = rotation(3 * w.tokens * P_ * esz)
    x0s = [z.clone() for _ in range(R)]
    x1s = [u.clone() for _ in range(R)]
    xts = [torch.empty_like(z) for _ in range(R)]
    trows = torch.rand(w.rows, dtype=torch.float32, device="cuda")
    kern_ms["interpolant"] = timed_batch([
        (lambda i=i: dit.rf_interpolant(xts[i], x0s[i], x1s[i], trows, w.tokens_per_row)) for i in range(R)])
    ltok = [torch.empty(w.tokens, dtype=torch.float32, device="cuda") for _ in range(R)]
    lrow = [torch.empty(w.rows, dtype=torch.float32, device="cuda") for _ in range(R)]
    kern_ms["cfm_loss"] = timed_batch([
        (lambda i=i: dit.rf_cfm_loss(ltok[i], lrow[i], xts[i], x0s[i], x1s[i], w.tokens_per_row)) for i in range(R)])
    del x0s, x1s, xts, ltok, lrow

    # Flowception frame insertion (not part of the step): one new noise frame after
    # every other frame of the batch (frames = H' x W' token planes)
    tpf = w.grid_hw[0] * w.grid_hw[1]
    nfr = w.tokens // tpf
    cnt = torch.zeros(nfr, dtype=torch.int32, device="cuda")
    cnt[::2] = 1
    nfo = nfr + int(cnt.sum())
    ins_bytes = 2 * nfo * tpf * P_ * esz
    R = rotation(ins_bytes)
    tfr = torch.rand(nfr, dtype=torch.float32, device="cuda")
    cu_fr = torch.from_numpy(w.cu_seqlens.astype(np.int32)).cuda()   # whole frames per sequence
    zs_ = [z.clone() for _ in range(R)]
    nzs = [torch.randn((nfo - nfr) * tpf, P_, device="cuda").to(tdt) for _ in range(R)]
    zos = [torch.empty(nfo * tpf, P_, dtype=tdt, device="cuda") for _ in range(R)]
    tos = [torch.empty(nfo, dtype=torch.float32, device="cuda") for _ in range(R)]
    cos = [torch.empty_like(cu_fr) for _ in range(R)]
    sos = [torch.empty(nfo, dtype=torch.int32, device="cuda") for _ in range(R)]
    kern_ms["insert_frames"] = timed_batch([
        (lambda i=i: dit.flow_insert_frames(zos[i], tos[i], cos[i], sos[i], zs_[i], tfr, cu_fr, cnt, nzs[i], tpf))
        for i in range(R)])
    del zs_, nzs, zos, tos, cos, sos

    flops = w.attn_flops()
    tok, D, P = w.tokens, w.d_model, synth.LATENT_CHANNELS
    algo_bytes = {
        "modulate": 2 * tok * D * esz,
        "rope": 4 * tok * D * esz,
        "residual_euler": 3 * tok * D * esz + 3 * tok * P * esz,
        "merge": merge_bytes,
        "interpolant": 3 * tok * P * esz,
        "cfm_loss": 3 * tok * P * esz + tok * 4 + w.rows * 4,
        "insert_frames": ins_bytes,
    }
    if "quant_fp8" in kern_ms:
        algo_bytes["quant_fp8"] = quant_bytes
    attn_s = kern_ms["attn"] * 1e-3
    achieved = flops / attn_s / 1e12
    traffic = traffic_for(w.name)
    kernels = {"attn": {"us": round(kern_ms["attn"] * 1e3, 2), "tflops": round(achieved, 2),
                        "us_median": round(float(np.median(attn_each)) * 1e3, 2),
                        "us_min": round(float(np.min(attn_each)) * 1e3, 2),
                        "us_max": round(float(np.max(attn_each)) * 1e3, 2), "launches": len(attn_each)},
               "attn_lse": {"us": round(kern_ms["attn_lse"] * 1e3, 2),
                            "tflops": round(flops / (kern_ms["attn_lse"] * 1e-3) / 1e12, 2)}}
    if "attn_ulysses_share" in kern_ms:
        tu = ulysses_flops / (kern_ms["attn_ulysses_share"] * 1e-3) / 1e12
        kernels["attn_ulysses_share"] = {"us": round(kern_ms["attn_ulysses_share"] * 1e3, 2), "tflops": round(tu, 2),
                                         "shape": "32760 tokens x 5 heads x 128 (480P video, 8-way Ulysses share)"}
    if "attn_hd64" in kern_ms:
        kernels["attn_hd64"] = {"us": round(kern_ms["attn_hd64"] * 1e3, 2),
                                "tflops": round(flops / (kern_ms["attn_hd64"] * 1e-3) / 1e12, 2),
                                "shape": f"{w.tokens} tokens x {w.heads * 2} heads x 64 (the workload's d_model)"}
    if "attn_fp8" in kern_ms:
        tf8 = flops / (kern_ms["attn_fp8"] * 1e-3) / 1e12
        kernels["attn_fp8"] = {"us": round(kern_ms["attn_fp8"] * 1e3, 2), "tflops": round(tf8, 2),
                               "frac_fp8_peak": round(tf8 / PEAK_FP8_TFLOPS, 4)}
    for n, nb in algo_bytes.items():
        gbs = nb / (kern_ms[n] * 1e-3) / 1e9
        kernels[n] = {"us": round(kern_ms[n] * 1e3, 2), "gbs": round(gbs, 1),
                      "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "bytes": nb}

    out = {
        "metric": "3D-attention TFLOP/s (fwd, bf16) at 1 MI355X and % of MFMA peak",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warm_steps,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,0.1) adaLN parameters)",
        "config": {"workload": w.name, "tokens": tok, "batch": w.num_seqs, "seq_len": w.max_seqlen,
                   "seqlens": list(w.seqlens), "heads": w.heads, "head_dim": w.head_dim,
                   "d_model": D, "latent_channels": P, "grid_thw": [w.frames[0], *w.grid_hw],
                   "rope_split": list(w.rope_split), "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": attn_kernel_name(w),
                     "flops_per_launch": flops},
        "kernels": kernels,
    }
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)   # elementwise: reads n*4 bytes, writes n*4 bytes
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = n * 4
        del src, dst
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline(w, budget_s):
    """The float64 oracle on a bounded sample: whole (sequence, head) attention
    problems plus the elementwise steps on the same share of tokens, scaled up
    by the share to one whole step."""
    import numpy as np

    import synth
    from oracle import attention as o_attn
    from oracle import epilogue as o_epi
    from oracle import grid as o_grid
    from oracle import modulate as o_mod
    from oracle import rope as o_rope

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    print(f"[bench] cpu baseline: oracle on up to ~{budget_s:.0f}s of work", file=sys.stderr, flush=True)
    inp = synth.make(w, ["q", "k", "v"])
    cu = w.cu_seqlens
    total_pairs = w.num_seqs * w.heads
    t_attn, pairs_done = 0.0, 0
    # whole (sequence, head) problems until ~80% of the budget is spent; a small
    # workload is gone through again (passes) so that the sample is not too short
    # to time
    while pairs_done == 0 or t_attn < 0.8 * budget_s:
        s, h = divmod(pairs_done % total_pairs, w.heads)
        lo, hi = int(cu[s]), int(cu[s + 1])
        sl = slice(lo, hi)
        t = time.perf_counter()
        o_attn.attention(inp["q"][sl, h:h + 1], inp["k"][sl, h:h + 1], inp["v"][sl, h:h + 1], [0, hi - lo])
        t_attn += time.perf_counter() - t
        pairs_done += 1
    # share of the step's attention flops covered by the sample
    done_flops = sum(4 * (int(cu[(p % total_pairs) // w.heads + 1]) - int(cu[(p % total_pairs) // w.heads])) ** 2
                     * w.head_dim for p in range(pairs_done))
    share = done_flops / w.attn_flops()
    rows = max(1, min(w.tokens, int(round(share * w.tokens))))
    e = synth.make(w, ["x", "gamma", "beta", "alpha", "z", "u", "dt"])
    pos = o_grid.positions(w.cu_seqlens, *w.grid_hw)[:rows]
    t = time.perf_counter()
    o_mod.adaln_modulate(e["x"][:rows], e["gamma"], e["beta"], w.tokens_per_row, w.eps)
    o_rope.apply_rope(inp["q"][:rows], pos, w.rope_split, w.rope_base)
    o_rope.apply_rope(inp["k"][:rows], pos, w.rope_split, w.rope_base)
    o_epi.gated_residual(e["x"][:rows], inp["v"][:rows], e["alpha"], w.tokens_per_row)
    o_epi.euler_step(e["z"][:rows], e["u"][:rows], e["dt"], w.tokens_per_row)
    t_elem = time.perf_counter() - t
    step_s = t_attn / share + t_elem * w.tokens / rows
    passes = f" ({share:.2f} passes over all pairs)" if share > 1 else ""
    return {"value": round(w.attn_flops() / step_s / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": (f"float64 numpy oracle: attention for {pairs_done} (sequence, head) problems of the "
                       f"step's {total_pairs}{passes} plus modulate/RoPE/residual/Euler on {rows} of "
                       f"{w.tokens} tokens; {t_attn + t_elem:.1f} s measured, scaled to one step "
                       f"({step_s:.1f} s)")}


if __name__ == "__main__":
    main()
