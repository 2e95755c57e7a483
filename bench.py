"""Benchmark: block-causal ReLU linear attention forward (one step = one
sva_lin_attn_fwd call: per-block reduction, prefix scan, output pass) on the
720p-shaped workload, B=1, H=16, d=64, bf16, 21 x 45 x 80 latent grid
(75,600 tokens), blocks of 3 frames, numerator-only 3D RoPE split 16/24/24,
K scaled by 0.5.  Inputs are seeded synthetic draws, resident in HBM before
timing; two buffer sets alternate so the 256 MB Infinity Cache cannot hold a
step's working set.

Prints one JSON line.  `value` = tokens/s over all heads (B*N tokens per
step / step time) over K uninstrumented steps after W warm-up steps.  The
`roofline` object rates the dominant kernel by its algorithmic bytes (its
inputs read once + its outputs written once) over its average duration,
timed live on the launch stream over K back-to-back launches of that kernel
alone (sva_lin_attn_fwd_stages), with no event between launches.  The same
line carries the median and minimum step over further runs, each kernel's
time and HBM fraction, a plain device copy's bandwidth (the practical
ceiling), and the other workloads (480p, the minute stream, the tiny fp32
case, the cached denoising step and its commit), all measured in this
process before the headline timing.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense fp4 (MX) matrix peak
KERNEL_SRC = os.path.join(ROOT, "block_causal_linear_phi_amd", "csrc", "sva.hip")
TCONV_SRC = os.path.join(ROOT, "block_causal_linear_phi_amd", "csrc", "tconv.hip")
PROJ_SRC = os.path.join(ROOT, "block_causal_linear_phi_amd", "csrc", "proj.hip")
PROFILES = os.path.join(ROOT, "profiles")
CALIB_KERNEL = "MulFunctor"  # the plain streaming kernel of copy_calibration()


def source_sha256(path: str = KERNEL_SRC) -> str:
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"sva_traffic_{workload}.json")


def upload(w, tensor: str, step: int = 0, n_tokens=None):
    """The workload's seeded [B, H, N, d] tensor `tensor` for `step` (the
    first n_tokens tokens of each sequence, or all), on cuda:0; the (b, h)
    slices are drawn in a thread pool (numpy's generator releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    import torch
    from block_causal_linear_phi_amd import workloads as wl

    n = w.N if n_tokens is None else n_tokens
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    x = torch.empty((w.B, w.H, n, w.d), dtype=tdt, device=torch.device("cuda:0"))

    def one(bh):
        b, h = bh
        _, raw = wl.slice_qkv(w, tensor, b, h, step, n)
        return bh, raw

    with ThreadPoolExecutor(16) as ex:
        for (b, h), raw in ex.map(one, [(b, h) for b in range(w.B) for h in range(w.H)]):
            src = torch.from_numpy(raw.view("int16") if w.dtype == "bf16" else raw)
            x[b, h].copy_(src.view(tdt) if w.dtype == "bf16" else src)
    return x


def _timed(stream, fn, n):
    """ms per call of fn(i) over n back-to-back calls between two events."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def warm_for(fn, calls: int, min_ms: float = 0.0):
    """Runs fn(i) for `calls` calls, then, when min_ms is set, more calls
    until about min_ms of GPU time has run (estimated from the first calls):
    after the host has set up a workload the GPU has been idle, and its
    clocks come back over a few milliseconds of work.  Returns the number of
    calls made."""
    import torch
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(calls):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    n = calls
    if min_ms > 0 and calls > 0:
        per = max(a.elapsed_time(b) / calls, 1e-3)
        extra = int(max(0.0, min_ms - a.elapsed_time(b)) / per) + 1
        for i in range(extra):
            fn(calls + i)
        torch.cuda.synchronize()
        n += extra
    return n


def graph_timed(fn, n: int, replays: int = 5):
    """ms per call of fn(i) for n calls captured in one HIP graph (torch's
    CUDAGraph on its capture stream) and replayed `replays` times: the launch
    cost of the host is out of the figure, which matters for kernels of a
    few microseconds.  The library issues only kernel launches, so the graph
    holds kernel nodes only."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(replays):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / (replays * n)
    del g
    return ms


class ForwardBench:
    """The forward (sva_lin_attn_fwd) of workload w on `sets` input/output
    buffer sets that alternate between steps (uploaded at construction)."""

    def __init__(self, w, sets: int):
        import torch
        from block_causal_linear_phi_amd import sva

        self.w, self.sets, self.sva = w, sets, sva
        dev = torch.device("cuda:0")
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        base = {t: upload(w, t) for t in ("q", "k", "v")}
        self.bufs = [base] + [{t: base[t].clone() for t in base} for _ in range(sets - 1)]
        self.outs = [torch.empty((w.B, w.H, w.N, w.d), dtype=tdt, device=dev) for _ in range(sets)]
        desc = sva.make_desc(w.B, w.H, w.d, (w.T, w.Hs, w.Ws), w.F, t0=w.t0, rope=w.rope, split=w.split,
                             base=w.base, eps=w.eps, dtype=sva.SVA_BF16 if w.dtype == "bf16" else sva.SVA_F32)
        self.ws = torch.zeros(sva.sva_lin_attn_fwd_workspace(desc), dtype=torch.uint8, device=dev)
        # a whole step is one prepared call per buffer set (the binding's
        # checks done here, once)
        self.calls = [sva.prepare_lin_attn_fwd(x["q"], x["k"], x["v"], (w.T, w.Hs, w.Ws), w.F, t0=w.t0,
                                               rope=w.rope, split=w.split, base=w.base, eps=w.eps,
                                               out=self.outs[s_], ws=self.ws)
                      for s_, x in enumerate(self.bufs)]
        torch.cuda.synchronize()

    def step(self, i, stages=7):
        w, s_ = self.w, i % self.sets
        if stages == 7:
            self.calls[s_]()
            return
        x = self.bufs[s_]
        self.sva.sva_lin_attn_fwd(x["q"], x["k"], x["v"], (w.T, w.Hs, w.Ws), w.F, t0=w.t0, rope=w.rope,
                                  split=w.split, base=w.base, eps=w.eps, out=self.outs[s_], ws=self.ws,
                                  stages=stages)

    def run(self, steps: int, warmup: int, repeats: int = 0, stage_calls: int = 0, min_warm_ms: float = 0.0):
        """Returns a dict:
          ms          ms per step over W untimed + K timed uninstrumented steps;
          repeat_ms   per-step ms of `repeats` further runs of K steps each;
          stage_us    per-launch us of each kernel, each timed alone over
                      `stage_calls` back-to-back launches (sva_lin_attn_fwd_stages)
                      on the same buffers, no event between two launches;
          stage_graph_us  the same launches captured in a HIP graph and
                      replayed (no host launch cost).
        The headline passes min_warm_ms = 0: exactly `warmup` untimed steps."""
        import torch
        stream = torch.cuda.current_stream()
        warmup = warm_for(self.step, warmup, min_warm_ms)
        res = {"ms": _timed(stream, lambda i: self.step(warmup + i), steps)}
        res["repeat_ms"] = [_timed(stream, self.step, steps) for _ in range(repeats)]
        res["stage_us"], res["stage_graph_us"] = {}, {}
        if stage_calls:
            sva = self.sva
            for name, st in (("reduce", sva.SVA_STAGE_REDUCE), ("scan", sva.SVA_STAGE_SCAN),
                             ("apply", sva.SVA_STAGE_APPLY)):
                self.step(0)  # a full call leaves the prefix operands each stage reads
                torch.cuda.synchronize()
                res["stage_us"][name] = 1e3 * _timed(stream, lambda i: self.step(i, st), stage_calls)
            for name, st in (("reduce", sva.SVA_STAGE_REDUCE), ("scan", sva.SVA_STAGE_SCAN),
                             ("apply", sva.SVA_STAGE_APPLY)):
                self.step(0)
                torch.cuda.synchronize()
                res["stage_graph_us"][name] = 1e3 * graph_timed(lambda i: self.step(i, st), stage_calls)
        return res

    def free(self):
        del self.calls, self.bufs, self.outs, self.ws


def gpu_leg(w, steps: int, warmup: int, sets: int, repeats: int = 0, stage_calls: int = 0,
            min_warm_ms: float = 0.0):
    """ForwardBench(w, sets).run(...), buffers freed afterwards."""
    fb = ForwardBench(w, sets)
    res = fb.run(steps, warmup, repeats, stage_calls, min_warm_ms)
    fb.free()
    return res


def bwd_leg(w, steps: int, warmup: int, sets: int):
    """The backward (sva_lin_attn_bwd) of the workload: dout is one more
    seeded N(0,1) tensor; the prefix states come from sva_lin_attn_fwd_save
    (the forward's output itself is not an input).  Returns ms
    per backward call over `steps` uninstrumented calls, with the saved
    states and with the states recomputed."""
    import torch
    from block_causal_linear_phi_amd import sva

    base = {t: upload(w, t) for t in ("q", "k", "v", "dout")}
    bufs = [base] + [{t: base[t].clone() for t in base} for _ in range(sets - 1)]
    kw = dict(t0=w.t0, rope=w.rope, split=w.split, base=w.base, eps=w.eps)
    for x in bufs:
        _, x["states"] = sva.sva_lin_attn_fwd_save(x["q"], x["k"], x["v"], (w.T, w.Hs, w.Ws), w.F, **kw)
        x["dq"], x["dk"], x["dv"] = (torch.empty_like(x[t]) for t in ("q", "k", "v"))
    desc = sva.make_desc(w.B, w.H, w.d, (w.T, w.Hs, w.Ws), w.F, eps=w.eps, **{k: kw[k] for k in ("t0", "rope",
                                                                                                    "split", "base")})
    ws = torch.zeros(sva.sva_lin_attn_bwd_workspace(desc), dtype=torch.uint8, device=torch.device("cuda:0"))
    stream = torch.cuda.current_stream()

    def step(i, saved):
        x = bufs[i % sets]
        sva.sva_lin_attn_bwd(x["q"], x["k"], x["v"], x["dout"], (w.T, w.Hs, w.Ws), w.F, dq=x["dq"],
                             dk=x["dk"], dv=x["dv"], states=x["states"] if saved else None, ws=ws,
                             stream=stream, **kw)

    res = []
    for saved in (True, False):
        for i in range(warmup):
            step(i, saved)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(steps):
            step(i, saved)
        b.record(stream)
        torch.cuda.synchronize()
        res.append(a.elapsed_time(b) / steps)
    return res[0], res[1]


def cached_leg(w, steps: int, warmup: int, min_warm_ms: float = 0.0):
    """Streaming generation: a cache committed from the workload's prior
    blocks, then `steps` denoising steps of one block against it
    (sva_block_cache_apply, the cache read only), cycling over the workload's
    per-step q, k, v; then commits of the last step's k, v.  Each is timed
    over back-to-back calls, and again replayed from a HIP graph (no host
    launch cost), as is the workspace-free apply.  Returns ms per call:
    apply_ms, commit_ms, apply_graph_ms, commit_graph_ms, noalloc_graph_ms."""
    import torch
    from block_causal_linear_phi_amd import sva

    dev = torch.device("cuda:0")
    fg = (w.F, w.Hs, w.Ws)
    kw = dict(rope=w.rope, split=w.split, base=w.base)
    S = torch.zeros((w.B, w.H, w.d, w.d), dtype=torch.float32, device=dev)
    z = torch.zeros((w.B, w.H, w.d), dtype=torch.float32, device=dev)
    for pb in range(w.prior_blocks):
        sva.sva_block_cache_commit(S, z, upload(w, "k_prior", pb), upload(w, "v_prior", pb), fg,
                                   t0=pb * w.F, **kw)
    data = [{t: upload(w, t, st) for t in ("q", "k", "v")} for st in range(w.steps)]
    out = torch.empty_like(data[0]["q"])
    desc = sva.make_desc(w.B, w.H, w.d, fg, w.F, t0=w.t0, eps=w.eps,
                         dtype=sva.SVA_BF16 if w.dtype == "bf16" else sva.SVA_F32, **kw)
    ws = torch.zeros(sva.sva_block_cache_workspace(desc), dtype=torch.uint8, device=dev)
    S2, z2 = S.clone(), z.clone()  # a second cache for the commits
    stream = torch.cuda.current_stream()

    def apply(i):
        x = data[i % w.steps]
        sva.sva_block_cache_apply(S, z, x["q"], x["k"], x["v"], fg, t0=w.t0, eps=w.eps, out=out, ws=ws, **kw)

    def noalloc(i):
        x = data[i % w.steps]
        sva.sva_block_cache_apply_noalloc(S, z, x["q"], x["k"], x["v"], fg, t0=w.t0, eps=w.eps, out=out, **kw)

    last = data[w.steps - 1]

    def commit(i):
        sva.sva_block_cache_commit(S2, z2, last["k"], last["v"], fg, t0=w.t0, ws=ws, **kw)

    warm_for(apply, warmup, min_warm_ms)
    res = {"apply_ms": _timed(stream, apply, steps), "commit_ms": _timed(stream, commit, steps)}
    res["apply_graph_ms"] = graph_timed(apply, steps)
    res["commit_graph_ms"] = graph_timed(commit, steps)
    res["noalloc_graph_ms"] = graph_timed(noalloc, steps)
    return res


def stream_leg(w, reps: int, warmup: int):
    """Block-by-block generation of the whole workload on one constant-size
    cache, for each block c in order, two ways:
      fused: one sva_lin_attn_fwd over the block with the cache as both S0
             and S_out (output and commit in one call, k and v read once);
      split: sva_block_cache_apply (the block's output against the blocks
             before it and itself) then sva_block_cache_commit of its k, v.
    Returns ms per full pass over all blocks for each (the two tiny zero
    fills that reset the cache per pass included)."""
    import torch
    from block_causal_linear_phi_amd import sva

    dev = torch.device("cuda:0")
    fg = (w.F, w.Hs, w.Ws)
    kw = dict(rope=w.rope, split=w.split, base=w.base)
    bt = w.block_tokens
    blocks = []
    for t in ("q", "k", "v"):
        full = upload(w, t)
        blocks.append([full[:, :, c * bt:(c + 1) * bt].contiguous() for c in range(w.nb)])
        del full
    S = torch.zeros((w.B, w.H, w.d, w.d), dtype=torch.float32, device=dev)
    z = torch.zeros((w.B, w.H, w.d), dtype=torch.float32, device=dev)
    out = torch.empty_like(blocks[0][0])
    desc = sva.make_desc(w.B, w.H, w.d, fg, w.F, t0=0, eps=w.eps,
                         dtype=sva.SVA_BF16 if w.dtype == "bf16" else sva.SVA_F32, **kw)
    ws = torch.zeros(sva.sva_block_cache_workspace(desc), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    fws = torch.zeros(sva.sva_lin_attn_fwd_workspace(desc), dtype=torch.uint8, device=dev)

    def split_pass():
        S.zero_()
        z.zero_()
        for c in range(w.nb):
            q, k, v = blocks[0][c], blocks[1][c], blocks[2][c]
            sva.sva_block_cache_apply(S, z, q, k, v, fg, t0=c * w.F, eps=w.eps, out=out, ws=ws, stream=stream, **kw)
            sva.sva_block_cache_commit(S, z, k, v, fg, t0=c * w.F, ws=ws, stream=stream, **kw)

    def fused_pass():
        S.zero_()
        z.zero_()
        for c in range(w.nb):
            q, k, v = blocks[0][c], blocks[1][c], blocks[2][c]
            sva.sva_lin_attn_fwd(q, k, v, fg, w.F, t0=c * w.F, eps=w.eps, S0=S, z0=z, S_out=S, z_out=z, out=out,
                                 ws=fws, stream=stream, **kw)

    res = []
    for one_pass in (fused_pass, split_pass):
        for _ in range(warmup):
            one_pass()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            one_pass()
        b.record(stream)
        torch.cuda.synchronize()
        res.append(a.elapsed_time(b) / reps)
    return res[0], res[1]


def tconv_leg(w, steps: int, warmup: int, sets: int, streaming: bool = True):
    """The causal temporal convolution (sva_tconv_fwd) over all blocks of the
    workload's activations, `sets` input/output buffer sets alternating;
    then, if `streaming`, apply of one block against a cache and the commit.
    Returns (ms per one-shot call, ms per block apply, ms per commit); the
    last two are None without `streaming`."""
    import torch
    from block_causal_linear_phi_amd import sva
    from block_causal_linear_phi_amd import workloads as wl

    dev = torch.device("cuda:0")
    x0 = torch.empty((w.B, w.T, w.Hs, w.Ws, w.C), dtype=torch.bfloat16, device=dev)
    for b in range(w.B):
        for t in range(w.T):
            _, raw = wl.tconv_frame(w, b, t)
            x0[b, t].copy_(torch.from_numpy(raw.view("int16")).view(torch.bfloat16))
    taps, bias = (torch.from_numpy(a).to(dev) for a in wl.tconv_params(w))
    xs = [x0] + [x0.clone() for _ in range(sets - 1)]
    ys = [torch.empty_like(x0) for _ in range(sets)]
    stream = torch.cuda.current_stream()

    def timed(fn):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(steps):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    fwd_ms = timed(lambda i: sva.sva_tconv_fwd(xs[i % sets], taps, bias, w.F, y=ys[i % sets], stream=stream))
    if not streaming:
        return fwd_ms, None, None
    blk = x0[:, :w.F].contiguous()
    yb = torch.empty_like(blk)
    cache = x0[:, w.F - 1].clone()
    apply_ms = timed(lambda i: sva.sva_tconv_apply(cache, blk, taps, bias, y=yb, stream=stream))
    commit_ms = timed(lambda i: sva.sva_tconv_commit(cache, blk, stream=stream))
    return fwd_ms, apply_ms, commit_ms


def tconv_cpu_leg(w, min_secs: float = 10.0, max_frames: int = 24):
    """The fp64 temporal-conv oracle on the host: sample 0's first
    min(T, max_frames) frames (whole blocks), all positions and channels,
    repeated until `min_secs` have passed; throughput in tokens per second."""
    import numpy as np
    from block_causal_linear_phi_amd import workloads as wl
    from oracle import tconv_oracle

    frames = min(w.T, max_frames) // w.F * w.F
    x = np.stack([wl.tconv_frame(w, 0, t)[0] for t in range(frames)])[None]
    taps, bias = wl.tconv_params(w)
    reps, t0 = 0, time.perf_counter()
    while True:
        tconv_oracle.tconv_fwd(x, taps, bias, w.F)
        reps += 1
        secs = time.perf_counter() - t0
        if secs >= min_secs:
            break
    tok = reps * frames * w.Hs * w.Ws
    return {"value": tok / secs, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{w.name}: sample 0, first {frames} frames, all {w.Hs * w.Ws} positions and {w.C} "
                      f"channels, {reps} passes, {secs:.1f} s, numpy fp64 (single-threaded elementwise)"}


def proj_leg(w, steps: int, warmup: int, sets: int):
    """The QKV projection with MXFP4 weights (sva_qkv_proj_mxfp4) on the
    workload's tokens, `sets` input/output buffer sets alternating.
    Returns ms per call."""
    import torch
    from block_causal_linear_phi_amd import sva
    from block_causal_linear_phi_amd import workloads as wl

    dev = torch.device("cuda:0")
    x0 = torch.empty((w.B, w.N, w.C), dtype=torch.bfloat16, device=dev)
    for bi in range(w.B):
        for j, s0 in enumerate(range(0, w.N, 4096)):
            n = min(4096, w.N - s0)
            _, raw = wl.draw((n, w.C), wl.seed_for(w.name, "x", bi, j), 1.0, "bf16")
            x0[bi, s0:s0 + n].copy_(torch.from_numpy(raw.view("int16")).view(torch.bfloat16))
    codes, scales = wl.mxfp4_weights(w.n_out, w.C, wl.seed_for(w.name, "w", 0, 0))
    cd = torch.from_numpy(wl.pack_nibbles(codes)).to(dev)
    sd = torch.from_numpy(scales).to(dev)
    wp = sva.sva_mxfp4_pack_weights(cd, sd, w.H, w.d)  # once, as at weight load
    bias = torch.from_numpy(wl.draw((w.n_out,), wl.seed_for(w.name, "bias", 0, 0), 0.1, "f32")[0]).to(dev)
    xs = [x0] + [x0.clone() for _ in range(sets - 1)]
    outs = [[torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev) for _ in range(3)]
            for _ in range(sets)]
    stream = torch.cuda.current_stream()

    def step(i):
        o = outs[i % sets]
        sva.sva_qkv_proj_mxfp4(xs[i % sets], wp, bias, w.H, w.d, q=o[0], k=o[1], v=o[2], stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        step(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def proj_w4a4_leg(w, steps: int, warmup: int, sets: int):
    """The W4A4 QKV projection on the workload's tokens: one step = the MX
    conversion of x (sva_mxfp4_quant_acts) then the 4-bit GEMM
    (sva_qkv_proj_w4a4), `sets` input/output buffer sets alternating.
    Returns ms per step, and ms per call of each kernel alone (back to back,
    no event between launches)."""
    import torch
    from block_causal_linear_phi_amd import sva
    from block_causal_linear_phi_amd import workloads as wl

    dev = torch.device("cuda:0")
    x0 = torch.empty((w.B, w.N, w.C), dtype=torch.bfloat16, device=dev)
    for bi in range(w.B):
        for j, s0 in enumerate(range(0, w.N, 4096)):
            n = min(4096, w.N - s0)
            _, raw = wl.draw((n, w.C), wl.seed_for(w.name, "x", bi, j), 1.0, "bf16")
            x0[bi, s0:s0 + n].copy_(torch.from_numpy(raw.view("int16")).view(torch.bfloat16))
    codes, scales = wl.mxfp4_weights(w.n_out, w.C, wl.seed_for(w.name, "w", 0, 0))
    wp = sva.sva_mxfp4_pack_weights(torch.from_numpy(wl.pack_nibbles(codes)).to(dev),
                                    torch.from_numpy(scales).to(dev), w.H, w.d)  # once, as at weight load
    bias = torch.from_numpy(wl.draw((w.n_out,), wl.seed_for(w.name, "bias", 0, 0), 0.1, "f32")[0]).to(dev)
    xs = [x0] + [x0.clone() for _ in range(sets - 1)]
    xqs = [sva.sva_mxfp4_quant_acts(x) for x in xs]
    outs = [[torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev) for _ in range(3)]
            for _ in range(sets)]
    stream = torch.cuda.current_stream()

    def quant(i):
        sva.sva_mxfp4_quant_acts(xs[i % sets], out=xqs[i % sets], stream=stream)

    def gemm(i):
        o = outs[i % sets]
        sva.sva_qkv_proj_w4a4(xqs[i % sets], wp, bias, w.B, w.N, w.C, w.H, w.d, q=o[0], k=o[1], v=o[2],
                              stream=stream)

    def step(i):
        quant(i)
        gemm(i)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ms = _timed(stream, step, steps)
    return ms, _timed(stream, quant, steps), _timed(stream, gemm, steps)


def fused_leg(w, aw, steps: int, warmup: int, sets: int, rounds: int = 5, w4a4: bool = False):
    """Projection + attention at the workload's token count, two ways, each
    timed over `steps` calls with `sets` input/output sets alternating:
      fused: sva_proj_lin_attn_fwd (k, v reduced inside the projection);
      two calls: sva_qkv_proj_mxfp4 then sva_lin_attn_fwd on the stored
      q, k, v.  With w4a4 both ways take the activations through
      sva_mxfp4_quant_acts first and use the 4-bit-activation calls
      (sva_proj_lin_attn_fwd_w4a4; sva_qkv_proj_w4a4).  Returns (fused ms,
      two-call ms), medians over `rounds` alternating rounds."""
    import torch
    from block_causal_linear_phi_amd import sva
    from block_causal_linear_phi_amd import workloads as wl

    dev = torch.device("cuda:0")
    x0 = torch.empty((w.B, w.N, w.C), dtype=torch.bfloat16, device=dev)
    for bi in range(w.B):
        for j, s0 in enumerate(range(0, w.N, 4096)):
            n = min(4096, w.N - s0)
            _, raw = wl.draw((n, w.C), wl.seed_for(w.name, "x", bi, j), 1.0, "bf16")
            x0[bi, s0:s0 + n].copy_(torch.from_numpy(raw.view("int16")).view(torch.bfloat16))
    codes, scales = wl.mxfp4_weights(w.n_out, w.C, wl.seed_for(w.name, "w", 0, 0))
    wp = sva.sva_mxfp4_pack_weights(torch.from_numpy(wl.pack_nibbles(codes)).to(dev),
                                    torch.from_numpy(scales).to(dev), w.H, w.d)
    bias = torch.from_numpy(wl.draw((w.n_out,), wl.seed_for(w.name, "bias", 0, 0), 0.1, "f32")[0]).to(dev)
    xs = [x0] + [x0.clone() for _ in range(sets - 1)]
    outs = [torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev) for _ in range(sets)]
    qkv = [torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    grid = (aw.T, aw.Hs, aw.Ws)
    kw = dict(t0=aw.t0, rope=aw.rope, split=aw.split, base=aw.base, eps=aw.eps)
    fdesc = sva.make_desc(w.B, w.H, w.d, grid, aw.F, dtype=sva.SVA_BF16, **kw)
    pdesc = sva.SvaProjDesc(w.B, w.N, w.C, w.H, w.d)
    n = ctypes.c_size_t()
    sva._check(sva.lib().sva_proj_lin_attn_fwd_workspace(ctypes.byref(fdesc), ctypes.byref(pdesc), ctypes.byref(n)),
               "sva_proj_lin_attn_fwd_workspace")
    fws = torch.zeros(n.value, dtype=torch.uint8, device=dev)
    aws = torch.zeros(sva.sva_lin_attn_fwd_workspace(fdesc), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    xq = torch.empty(sva.mxfp4_acts_bytes(w.B * w.N, w.C), dtype=torch.uint8, device=dev) if w4a4 else None

    def fused(i):
        if w4a4:
            sva.sva_mxfp4_quant_acts(xs[i % sets], out=xq, stream=stream)
            sva.sva_proj_lin_attn_fwd_w4a4(xq, wp, bias, w.B, w.C, w.H, grid, aw.F, out=outs[i % sets], ws=fws,
                                           stream=stream, **kw)
        else:
            sva.sva_proj_lin_attn_fwd(xs[i % sets], wp, bias, w.H, grid, aw.F, out=outs[i % sets], ws=fws,
                                      stream=stream, **kw)

    def two(i):
        if w4a4:
            sva.sva_mxfp4_quant_acts(xs[i % sets], out=xq, stream=stream)
            sva.sva_qkv_proj_w4a4(xq, wp, bias, w.B, w.N, w.C, w.H, w.d, q=qkv[0], k=qkv[1], v=qkv[2], stream=stream)
        else:
            sva.sva_qkv_proj_mxfp4(xs[i % sets], wp, bias, w.H, w.d, q=qkv[0], k=qkv[1], v=qkv[2], stream=stream)
        sva.sva_lin_attn_fwd(qkv[0], qkv[1], qkv[2], grid, aw.F, out=outs[i % sets], ws=aws, stream=stream, **kw)

    # The two ways alternate over `rounds` rounds of `steps` calls each, and
    # each reports its median round: the MFMA-heavy projection's speed drifts
    # with the clocks over a run, and a fixed order would hand that drift to
    # one of the two.
    for fn in (fused, two):
        for i in range(warmup):
            fn(i)
    torch.cuda.synchronize()
    times = {fused: [], two: []}
    for r in range(rounds):
        for fn in ((fused, two) if r % 2 == 0 else (two, fused)):
            times[fn].append(_timed(stream, fn, steps))
    med = {fn: sorted(t)[len(t) // 2] for fn, t in times.items()}
    return med[fused], med[two]


def proj_cpu_leg(w, min_secs: float = 10.0, tokens: int = 1024):
    """The fp64 projection oracle on the host over the workload's first
    `tokens` tokens, repeated until `min_secs` have passed."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from block_causal_linear_phi_amd import workloads as wl
    from oracle import proj_oracle

    cores = min(len(os.sched_getaffinity(0)), 16)
    x = wl.draw((tokens, w.C), wl.seed_for(w.name, "x", 0, 0), 1.0, "bf16")[0][None]
    codes, scales = wl.mxfp4_weights(w.n_out, w.C, wl.seed_for(w.name, "w", 0, 0))
    with threadpool_limits(limits=cores):
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        reps, t0 = 0, time.perf_counter()
        while True:
            proj_oracle.qkv_project(x, codes, scales, None, w.H, w.d)
            reps += 1
            secs = time.perf_counter() - t0
            if secs >= min_secs:
                break
    return {"value": reps * tokens / secs, "unit": "tokens/s", "cores": int(min(cores, blas)), "kind": "oracle",
            "sample": f"{w.name}: first {tokens} tokens, {reps} passes, {secs:.1f} s, numpy fp64 "
                      f"(decode per pass; BLAS threads {blas} of {cores} host cores)"}


def copy_calibration(mib: int, reps: int = 5):
    """A plain streaming kernel of known size (torch.mul(x, 1.0, out=y) on
    fp32: reads and writes mib MiB each).  Its FETCH_SIZE / WRITE_SIZE
    counters scale the library kernels' counters to bytes, and its bandwidth
    is the practical HBM ceiling on this machine.  Reported on stderr."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        torch.mul(x, 1.0, out=y)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    gbs = 2 * n * 4 / (ms * 1e-3) / 1e9
    print(json.dumps({"copy_calibration": {"kernel": "torch.mul fp32 out-of-place", "read_bytes": n * 4,
                                           "write_bytes": n * 4, "us": ms * 1e3, "GB/s": gbs}}),
          file=sys.stderr, flush=True)
    del x, y


def copy_ceiling(mib: int = 512, reps: int = 10):
    """A plain device copy (torch copy_ of mib MiB, bf16) on this GPU: the
    practical HBM ceiling that the roofline fractions are read against."""
    import torch
    n = mib * (1 << 20) // 2
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    ms = _timed(torch.cuda.current_stream(), lambda i: y.copy_(x), reps)
    gbs = 2 * n * 2 / (ms * 1e-3) / 1e9
    del x, y
    return {"kernel": f"torch copy_ of {mib} MiB (read + write)", "us": ms * 1e3, "GB/s": gbs,
            "frac_of_peak": gbs / HBM_PEAK_GBS}


def other_workloads(steps: int, warmup: int, sets: int):
    """The other configurations, each timed in this process with the
    forward's buffer rotation: 480p and the minute stream (one-shot forward,
    with per-kernel times), the tiny fp32 case, and the cached denoising step
    (us per step and per commit)."""
    from block_causal_linear_phi_amd import workloads as wl

    out = {}
    for name, k_steps in (("480p", steps), ("minute", max(2, steps // 4)), ("tiny", steps)):
        w = wl.WORKLOADS[name]
        res = gpu_leg(w, k_steps, warmup, sets if name != "tiny" else 1, stage_calls=k_steps if name != "tiny" else 0,
                      min_warm_ms=SECONDARY_WARM_MS)
        esz = 2 if w.dtype == "bf16" else 4
        step_bytes = 4 * w.B * w.H * w.N * w.d * esz
        ent = {"us_per_step": res["ms"] * 1e3, "tokens_per_s": w.B * w.N / (res["ms"] * 1e-3),
               "hbm_frac_step": step_bytes / (res["ms"] * 1e-3) / (HBM_PEAK_GBS * 1e9), "steps": k_steps}
        if res["stage_us"]:
            ent["kernels_us"] = {k: round(v, 2) for k, v in res["stage_graph_us"].items()}
            ent["kernels_eager_us"] = {k: round(v, 2) for k, v in res["stage_us"].items()}
        out[name] = ent
    w = wl.WORKLOADS["cached_step"]
    c = cached_leg(w, steps, warmup, SECONDARY_WARM_MS)
    out["cached_step"] = {"us_per_step": c["apply_ms"] * 1e3, "commit_us": c["commit_ms"] * 1e3,
                          "us_per_step_graph": c["apply_graph_ms"] * 1e3,
                          "commit_us_graph": c["commit_graph_ms"] * 1e3,
                          "us_per_step_noalloc_graph": c["noalloc_graph_ms"] * 1e3,
                          "tokens_per_s": w.B * w.block_tokens / (c["apply_ms"] * 1e-3)}
    return out


SECONDARY_WARMUP = 50  # warm-up calls of each leg after the headline
SECONDARY_WARM_MS = 30.0  # and at least this much GPU time of warm-up calls (the other workloads)
SECONDARY_STEPS = 100  # timed steps of each other workload, at least


def extension_rows(steps: int, warmup: int, sets: int):
    """The rows beyond the forward, each timed in this process at the 720p
    size (after the headline): the backward from saved states, the temporal
    convolution, the QKV projection with bf16 and with MXFP4 activations,
    projection + attention fused against two calls (720p and 480p; bf16
    and MXFP4 activations), and
    block-by-block generation.  Fewer steps than the headline: each row is a
    mean over `steps` back-to-back calls after `warmup`."""
    import torch
    from block_causal_linear_phi_amd import workloads as wl

    w720 = wl.WORKLOADS["720p"]
    out = {}
    ms, ms_re = bwd_leg(w720, steps, warmup, sets)
    out["backward_720p"] = {"us_per_step": ms * 1e3, "tokens_per_s": w720.B * w720.N / (ms * 1e-3),
                            "us_per_step_recomputing_states": ms_re * 1e3,
                            "alg_bytes": 7 * w720.B * w720.H * w720.N * w720.d * 2}
    torch.cuda.empty_cache()
    tw = wl.TCONV_WORKLOADS["tconv_720p"]
    t_ms, t_apply, t_commit = tconv_leg(tw, steps, warmup, sets, True)
    tbytes = 2 * tw.B * tw.T * tw.Hs * tw.Ws * tw.C * (2 if tw.dtype == "bf16" else 4)
    out["tconv_720p"] = {"us_per_step": t_ms * 1e3, "hbm_frac_step": tbytes / (t_ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                         "block_apply_us": t_apply * 1e3, "block_commit_us": t_commit * 1e3}
    torch.cuda.empty_cache()
    pw = wl.PROJ_WORKLOADS["proj_720p"]
    flops = 2.0 * pw.B * pw.N * pw.C * pw.n_out
    p_ms = proj_leg(pw, steps, warmup, sets)
    out["proj_w4a16_720p"] = {"us_per_step": p_ms * 1e3, "tflops": flops / (p_ms * 1e-3) / 1e12,
                              "frac_of_bf16_peak": flops / (p_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    torch.cuda.empty_cache()
    s_ms, q_ms, g_ms = proj_w4a4_leg(pw, steps, warmup, sets)
    out["proj_w4a4_720p"] = {"us_per_step": s_ms * 1e3, "quant_acts_us": q_ms * 1e3, "gemm_us": g_ms * 1e3,
                             "gemm_frac_of_fp4_peak": flops / (g_ms * 1e-3) / 1e12 / MFMA_FP4_PEAK_TFLOPS}
    torch.cuda.empty_cache()
    for w4a4 in (False, True):
        for name in ("720p", "480p"):
            f_ms, two_ms = fused_leg(wl.PROJ_WORKLOADS["proj_" + name], wl.WORKLOADS[name], steps, warmup, sets,
                                     w4a4=w4a4)
            out[("fused_w4a4_" if w4a4 else "fused_") + name] = {
                "us_per_step": f_ms * 1e3, "two_calls_us_per_step": two_ms * 1e3,
                "speedup_over_two_calls": two_ms / f_ms}
            torch.cuda.empty_cache()
    st_ms, sp_ms = stream_leg(w720, steps, warmup)
    out["stream_720p"] = {"us_per_block": st_ms * 1e3 / w720.nb, "us_per_block_apply_then_commit": sp_ms * 1e3 / w720.nb}
    torch.cuda.empty_cache()
    return out


def cpu_leg(w, reps: int):
    """The fp64 oracle on the host: all heads of the workload, `reps` times."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from block_causal_linear_phi_amd import workloads as wl
    from oracle import sva_oracle

    cores = min(len(os.sched_getaffinity(0)), 16)  # a one-GPU share of the host
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    data = {bh: tuple(wl.slice_qkv(w, t, *bh)[0][None, None] for t in "qkv") for bh in heads}
    with threadpool_limits(limits=cores):
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        t0 = time.perf_counter()
        for _ in range(reps):
            for bh in heads:
                q, k, v = data[bh]
                sva_oracle.lin_attn_fwd(q, k, v, (w.T, w.Hs, w.Ws), w.F, t0=w.t0, rope=w.rope, split=w.split,
                                        base=w.base, eps=w.eps)
        secs = time.perf_counter() - t0
    tok_s = w.B * w.N * reps / secs
    return {"value": tok_s, "unit": "tokens/s", "cores": int(min(cores, blas_threads)), "kind": "oracle",
            "sample": f"{w.name}: all {len(heads)} heads, {reps} passes, {secs:.1f} s, numpy fp64 "
                      f"(BLAS threads {blas_threads} of {cores} host cores; elementwise steps single-threaded)"}


def _short_kernel(name: str) -> str:
    for k in ("sva_reduce_kernel", "sva_scan_kernel", "sva_apply_kernel", "sva_prep_kernel",
              "sva_bwd_out_kernel", "sva_bwd_kv_kernel", "sva_tconv_kernel", "sva_tconv_commit_kernel",
              "sva_qkv_proj_kernel", "sva_mxfp4_pack_kernel", "sva_mxfp4_quant_kernel", "sva_qkv_proj_w4a4_kernel",
              "sva_kv_proj_reduce_kernel", "sva_kv_proj_reduce_w4a4_kernel", "sva_q_proj_apply_kernel"):
        if k in name:
            short = k.replace("sva_", "").replace("_kernel", "")
            if k == "sva_tconv_kernel" and "sva_tconv_commit_kernel" in name:
                continue
            m = re.search(r"sva_reduce_kernel<([^>]*)>", name)
            if m and m.group(1).replace(" ", "").split(",")[-1] == "true":
                short += " (weighted, backward)"
            return short
    return name.split("(")[0][-60:]


MFMA_COUNTERS = ("SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32")


def summarize_mfma(args):
    """MFMA activity per kernel from one rocprofv3 --pmc pass of
    MFMA_COUNTERS and a --kernel-trace pass of the same command: MFMA
    instructions and flops per launch (MOPS x 512 flops), the achieved rate
    over the kernel's average duration, and its fraction of the dense peak."""
    import csv
    import glob
    from collections import defaultdict

    def csvs(d, suffix):
        return [f for f in glob.glob(os.path.join(d, "**", "*.csv"), recursive=True) if f.endswith(suffix)]

    dur = defaultdict(list)
    for r in csv.DictReader(open(csvs(args.trace_dir, "kernel_trace.csv")[0])):
        if "sva_" in r["Kernel_Name"]:
            dur[_short_kernel(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    cnt = defaultdict(lambda: defaultdict(list))
    for r in csv.DictReader(open(csvs(args.pmc_dir, "counter_collection.csv")[0])):
        if "sva_" in r["Kernel_Name"]:
            cnt[_short_kernel(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    name = ("proj_" if args.proj else "") + args.workload + args.label
    lines = [f"# MFMA activity per kernel, {name} workload", "",
             "Commands (run from the repository root on one MI355X):", ""]
    lines += [f"    {c}" for c in args.commands]
    lines += ["", "Per launch (mean over the profiled launches). flops = SQ_INSTS_VALU_MFMA_MOPS_* x 512;",
              "rate = flops / the kernel's mean duration in the trace pass; peak: 2.5 PFLOP/s bf16,",
              "157.3 TFLOP/s fp32 (dense).", "",
              "| kernel | mean us | MFMA instructions | bf16 GFLOP | fp32 GFLOP | TFLOP/s | % of peak |",
              "|---|---|---|---|---|---|---|"]
    out = {}
    for k in sorted(cnt):
        c = {n: sum(v) / len(v) for n, v in cnt[k].items()}
        us = sum(dur[k]) / len(dur[k]) if dur.get(k) else float("nan")
        fb = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        ff = c.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0) * 512
        rate = (fb + ff) / (us * 1e-6) / 1e12 if us == us and us > 0 else float("nan")
        peak = MFMA_BF16_PEAK_TFLOPS if fb >= ff else 157.3
        out[k] = {"us": us, "mfma_insts": c.get("SQ_INSTS_MFMA"), "bf16_flops": fb, "f32_flops": ff,
                  "tflops": rate, "frac_of_peak": rate / peak}
        lines.append(f"| {k} | {us:.2f} | {c.get('SQ_INSTS_MFMA', 0):.4g} | {fb / 1e9:.2f} | {ff / 1e9:.2f} | "
                     f"{rate:.1f} | {100 * rate / peak:.1f} |")
    src = PROJ_SRC if args.proj else KERNEL_SRC
    lines += ["", f"Kernel source sha256: `{source_sha256(src)}`", ""]
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"sva_mfma_{name}.md"), "w") as f:
        f.write("\n".join(lines))
    print(json.dumps({"summarized_mfma": name, "per_launch": out}))


def summarize_profile(args):
    """Turn rocprofv3 CSV output into the committed summaries: a kernel-time
    table and per-launch HBM traffic (FETCH_SIZE / WRITE_SIZE scaled by what
    the same counters read for the plain streaming kernel of known size)."""
    import csv
    import glob
    from collections import defaultdict

    def one(pattern):
        hits = glob.glob(os.path.join(pattern, "**", "*.csv"), recursive=True)
        return hits

    stats = [f for f in one(args.trace_dir) if f.endswith("kernel_stats.csv")][0]
    rows = list(csv.DictReader(open(stats)))
    # The longest run of consecutive launches of each kernel in the trace:
    # bench.py times each kernel over such a run (its back-to-back stage
    # launches), so the run's mean duration is the figure to compare.
    trace = [f for f in one(args.trace_dir) if f.endswith("kernel_trace.csv")]
    runs = {}
    if trace:
        disp = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), _short_kernel(r["Kernel_Name"]))
                       for r in csv.DictReader(open(trace[0]))), key=lambda t: t[0])
        i = 0
        while i < len(disp):
            j = i
            while j + 1 < len(disp) and disp[j + 1][2] == disp[i][2]:
                j += 1
            n = j - i + 1
            if n > runs.get(disp[i][2], (0, 0.0, 0.0))[0]:
                durs = [(e - b) / 1e3 for b, e, _ in disp[i:j + 1]]
                gaps = [(disp[m + 1][0] - disp[m][1]) / 1e3 for m in range(i, j)]
                runs[disp[i][2]] = (n, sum(durs) / n, (sum(gaps) / len(gaps)) if gaps else 0.0)
            i = j + 1
    counters = defaultdict(list)
    with_traffic = bool(args.fetch_dir and args.write_dir)
    for d, cname in ((args.fetch_dir, "FETCH_SIZE"), (args.write_dir, "WRITE_SIZE")) if with_traffic else ():
        f = [x for x in one(d) if x.endswith("counter_collection.csv")][0]
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == cname:
                counters[(r["Kernel_Name"], cname)].append(float(r["Counter_Value"]))
    calib_bytes = args.calib_mib * (1 << 20)

    def mean_for(substr, cname):
        vals = [v for (k, c), vs in counters.items() if substr in k and c == cname for v in vs]
        return sum(vals) / len(vals) if vals else None

    f_scale = calib_bytes / (mean_for(CALIB_KERNEL, "FETCH_SIZE") * 1024) if with_traffic else None
    w_scale = calib_bytes / (mean_for(CALIB_KERNEL, "WRITE_SIZE") * 1024) if with_traffic else None
    by_short = defaultdict(lambda: defaultdict(list))
    for (kname, cname), vs in counters.items():
        if "sva_" in kname:
            by_short[_short_kernel(kname)][cname] += vs
    traffic = {}

    def add_traffic(key, fs, ws):
        fk, wk = sum(fs) / len(fs), sum(ws) / len(ws)
        traffic[key] = {"fetch_kib": fk, "write_kib": wk, "read_bytes": fk * 1024 * f_scale,
                        "write_bytes": wk * 1024 * w_scale, "bytes": fk * 1024 * f_scale + wk * 1024 * w_scale}

    for k, cs in by_short.items():
        if not cs["FETCH_SIZE"] or not cs["WRITE_SIZE"]:
            continue
        ws = cs["WRITE_SIZE"]
        if len(ws) == len(cs["FETCH_SIZE"]) and max(ws) > 2 * min(ws) > 0:
            # one kernel launched on two sizes (the fused leg's q-only and
            # q, k, v projections): a row for each, split at the geometric mean
            cut = (max(ws) * min(ws)) ** 0.5
            lo = [i for i, w in enumerate(ws) if w < cut]
            hi = [i for i, w in enumerate(ws) if w >= cut]
            add_traffic(k + " (smaller launches)", [cs["FETCH_SIZE"][i] for i in lo], [ws[i] for i in lo])
            add_traffic(k + " (larger launches)", [cs["FETCH_SIZE"][i] for i in hi], [ws[i] for i in hi])
        else:
            add_traffic(k, cs["FETCH_SIZE"], ws)
    name = ("tconv_" if args.tconv else "proj_" if args.proj else "") + args.workload
    src = TCONV_SRC if args.tconv else PROJ_SRC if args.proj else KERNEL_SRC
    doc = {"workload": name, "source_sha256": source_sha256(src),
           "fetch_scale": f_scale,
           "write_scale": w_scale, "calibration": f"{CALIB_KERNEL} kernel reading and writing "
                                                  f"{calib_bytes} bytes", "per_launch": traffic,
           "commands": args.commands}
    os.makedirs(PROFILES, exist_ok=True)
    if with_traffic:
        with open(traffic_file(name + args.label), "w") as f:
            json.dump(doc, f, indent=1)
    what = ("causal temporal convolution" if args.tconv
            else "W4A4 QKV projection (MXFP4 activations and weights)" if args.proj and args.label == "_w4a4"
            else "QKV projection with MXFP4 weights" if args.proj
            else "backward" if args.label == "_bwd"
            else "fused QKV projection (MXFP4 weights) + attention forward, and the two-call path"
            if args.label == "_fused"
            else "fused QKV projection (MXFP4 weights and activations) + attention forward, and the two-call path"
            if args.label == "_fused_w4a4"
            else "denoising step and commit" if args.workload == "cached_step"
            else "forward")
    lines = [f"# Kernel times and HBM traffic, {args.workload} workload, {what}", "",
             "Commands (run from the repository root on one MI355X):", ""]
    lines += [f"    {c}" for c in args.commands]
    lines += ["", "## rocprofv3 --kernel-trace --stats", "",
              "| kernel | calls | average us | min us | max us | % |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {_short_kernel(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    long_runs = {k: v for k, v in runs.items() if v[0] >= 10}
    if long_runs:
        lines += ["", "## Longest run of back-to-back launches of each kernel", "",
                  "The figure bench.py's roofline uses (it times each kernel over such a run).", "",
                  "| kernel | launches | mean us | mean gap to the next launch us |", "|---|---|---|---|"]
        for k, (n, mu, gap) in sorted(long_runs.items(), key=lambda kv: -kv[1][0]):
            lines.append(f"| {k} | {n} | {mu:.2f} | {gap:.2f} |")
    if trace:
        lib = [d for d in disp if d[2] in ("reduce", "scan", "apply")]
        gaps = defaultdict(list)
        for a_, b_ in zip(lib, lib[1:]):
            if b_[0] - a_[1] < 20000:  # within one call sequence (under 20 us apart)
                gaps[(a_[2], b_[2])].append((b_[0] - a_[1]) / 1e3)
        if gaps:
            lines += ["", "## Gaps between consecutive library kernels (under the profiler)", "",
                      "| from | to | count | mean gap us |", "|---|---|---|---|"]
            for (x, y), g in sorted(gaps.items()):
                lines.append(f"| {x} | {y} | {len(g)} | {sum(g) / len(g):.2f} |")
    if with_traffic:
        lines += ["", "## HBM traffic per launch (FETCH_SIZE, WRITE_SIZE)", "",
                  f"Scale factors from the {CALIB_KERNEL} streaming kernel over {calib_bytes} bytes: "
                  f"FETCH_SIZE x {f_scale:.4f}, WRITE_SIZE x {w_scale:.4f}.", "",
                  "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB | write MB | total MB |",
                  "|---|---|---|---|---|---|"]
        for k, t in traffic.items():
            lines.append(f"| {k} | {t['fetch_kib']:.0f} | {t['write_kib']:.0f} | {t['read_bytes'] / 1e6:.1f} | "
                         f"{t['write_bytes'] / 1e6:.1f} | {t['bytes'] / 1e6:.1f} |")
    lines += ["", f"Kernel source sha256: `{doc['source_sha256']}`", ""]
    if args.label in ("_fused", "_fused_w4a4"):  # the fused path runs kernels of both sources
        lines[-1:-1] = [f"Projection source sha256: `{source_sha256(PROJ_SRC)}`"]
    with open(os.path.join(PROFILES, f"sva_kernels_{name}{args.label}.md"), "w") as f:
        f.write("\n".join(lines))
    print(json.dumps({"summarized": name, "traffic": traffic, "back_to_back": runs}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the clocks settle after ~100 steps (about 13 ms of this workload)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="720p")
    ap.add_argument("--sets", type=int, default=2, help="input buffer sets that alternate between steps")
    ap.add_argument("--cpu-reps", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--proj-w4a4", action="store_true",
                    help="time the W4A4 QKV projection (activation conversion + 4-bit GEMM)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (sva_lin_attn_bwd) instead of the forward")
    ap.add_argument("--tconv", action="store_true",
                    help="time the causal temporal convolution of the Mix-FFN on the workload's grid instead")
    ap.add_argument("--fused", action="store_true",
                    help="projection + attention: the fused entry point against the two calls")
    ap.add_argument("--w4a4", action="store_true",
                    help="with --fused: MXFP4 activations (conversion + the W4A4 calls) in both ways")
    ap.add_argument("--proj", action="store_true",
                    help="time the QKV projection with MXFP4 weights on the workload's tokens instead")
    ap.add_argument("--stream", action="store_true",
                    help="block-by-block generation on one cache (apply + commit per block); --steps passes")
    ap.add_argument("--no-streaming", action="store_true",
                    help="with --tconv: time the one-shot call only (profiling runs)")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="also run a plain fp32 streaming kernel over MIB MiB (counter calibration)")
    ap.add_argument("--summarize-mfma", action="store_true",
                    help="write profiles/sva_mfma_<workload>.md from --pmc-dir and --trace-dir")
    ap.add_argument("--pmc-dir")
    ap.add_argument("--summarize-profile", action="store_true",
                    help="write profiles/ summaries from rocprofv3 output directories, then exit")
    ap.add_argument("--trace-dir")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--calib-mib", type=int, default=256)
    ap.add_argument("--commands", nargs="*", default=[])
    ap.add_argument("--label", default="", help="summary name suffix, e.g. _bwd")
    ap.add_argument("--repeats", type=int, default=10,
                    help="further runs of K steps for the median and min step time")
    ap.add_argument("--no-others", action="store_true",
                    help="720p: skip the other workloads and the copy ceiling")
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profile(args)
        return
    if args.summarize_mfma:
        summarize_mfma(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (heads and samples shard "
              "with no communication; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from block_causal_linear_phi_amd import workloads as wl
    if args.copy_calib:
        copy_calibration(args.copy_calib)
    if args.fused:
        pw = wl.PROJ_WORKLOADS["proj_" + args.workload]
        aw = wl.WORKLOADS[args.workload]
        ms, ms_two = fused_leg(pw, aw, args.steps, args.warmup, args.sets, w4a4=args.w4a4)
        flops = 2.0 * pw.B * pw.N * pw.C * pw.n_out
        acts = "MXFP4 weights and activations, conversion included" if args.w4a4 else "MXFP4 weights"
        print(json.dumps({
            "metric": f"tokens/s of the QKV projection ({acts}) and block-causal attention forward, fused",
            "value": pw.B * pw.N / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) activations; uniform E2M1 codes, E8M0 scales 2^-7..2^-3; resident in HBM)",
            "config": {"workload": f"{pw.name} + {aw.name}: x [{pw.B}, {pw.N}, {pw.C}] -> q, k, v of {pw.H} heads x "
                                   f"{pw.d} -> block-causal attention, grid {aw.T}x{aw.Hs}x{aw.Ws}, blocks of {aw.F}",
                       "B": pw.B, "tokens": pw.N, "C": pw.C, "H": pw.H, "d": pw.d},
            "ms_per_step_two_calls": ms_two, "speedup_over_two_calls": ms_two / ms,
            "projection_tflops": flops / (ms * 1e-3) / 1e12,
        }), flush=True)
        return
    if args.proj_w4a4:
        pw = wl.PROJ_WORKLOADS["proj_" + args.workload]
        ms, q_ms, g_ms = proj_w4a4_leg(pw, args.steps, args.warmup, args.sets)
        M = pw.B * pw.N
        flops = 2.0 * M * pw.C * pw.n_out
        x_bytes = M * pw.C * 2
        xq_bytes = M * pw.C // 2 + M * pw.C // 32
        w_bytes = pw.n_out * pw.C * (0.5 + 1 / 32)
        out_bytes = M * pw.n_out * 2
        gemm_io = xq_bytes + w_bytes + out_bytes + pw.n_out * 4
        quant_io = x_bytes + xq_bytes
        gemm_gbs = gemm_io / (g_ms * 1e-3) / 1e9
        line = {
            "metric": "tokens/s of the QKV projection, W4A4 (MXFP4 activations and weights; q, k, v for all heads)",
            "value": M / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp4",
            "data": "synthetic (seeded N(0,1) activations; uniform E2M1 codes, E8M0 scales 2^-7..2^-3; resident in HBM)",
            "config": {"workload": f"{pw.name}: B={pw.B} N={pw.N} tokens, C={pw.C} -> 3 x {pw.H} heads x {pw.d}, "
                                   "MXFP4 activations (converted in the step) and weights, bf16 outputs",
                       "B": pw.B, "tokens": pw.N, "C": pw.C, "H": pw.H, "d": pw.d},
            # the GEMM writes 2 bytes per output for 2 C / 4 bits of operands: bound by its output stream
            "roofline": {"bound": "hbm", "kernel": "qkv_proj_w4a4", "achieved": gemm_gbs, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": gemm_gbs / HBM_PEAK_GBS, "traffic": None, "io_bytes": gemm_io},
            "kernels_us": {"quant_acts": q_ms * 1e3, "qkv_proj_w4a4": g_ms * 1e3},
            "hbm_gbs_step": (quant_io + gemm_io) / (ms * 1e-3) / 1e9,
            "quant_hbm_frac": quant_io / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "gemm_fp4_mfma_frac": flops / (g_ms * 1e-3) / 1e12 / MFMA_FP4_PEAK_TFLOPS,
        }
        try:
            with open(traffic_file(pw.name + "_w4a4")) as f:
                prof = json.load(f)
            if prof.get("source_sha256") == source_sha256(PROJ_SRC) and "qkv_proj_w4a4" in prof.get("per_launch", {}):
                line["roofline"]["traffic"] = prof["per_launch"]["qkv_proj_w4a4"]["bytes"] / 1e9
        except (OSError, ValueError):
            pass
        print(json.dumps(line), flush=True)
        return
    if args.proj:
        pw = wl.PROJ_WORKLOADS["proj_" + args.workload]
        ms = proj_leg(pw, args.steps, args.warmup, args.sets)
        flops = 2.0 * pw.B * pw.N * pw.C * pw.n_out
        tflops = flops / (ms * 1e-3) / 1e12
        io = pw.B * pw.N * (pw.C + pw.n_out) * 2 + pw.n_out * pw.C * (0.5 + 1 / 32) + pw.n_out * 4
        line = {
            "metric": "tokens/s of the QKV projection with MXFP4 weights (q, k, v for all heads)",
            "value": pw.B * pw.N / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) activations; uniform E2M1 codes, E8M0 scales 2^-7..2^-3; resident in HBM)",
            "config": {"workload": f"{pw.name}: B={pw.B} N={pw.N} tokens, C={pw.C} -> 3 x {pw.H} heads x {pw.d}, "
                                   "MXFP4 weights, bf16 activations and outputs",
                       "B": pw.B, "tokens": pw.N, "C": pw.C, "H": pw.H, "d": pw.d},
            # bf16 MFMA after an exact weight decode: priced against the bf16 dense peak
            "roofline": {"bound": "mfma", "kernel": "qkv_proj", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                         "flops": flops, "io_bytes": io},
            "hbm_gbs": io / (ms * 1e-3) / 1e9,
        }
        try:
            with open(traffic_file(pw.name)) as f:
                prof = json.load(f)
            if prof.get("source_sha256") == source_sha256(PROJ_SRC) and "qkv_proj" in prof.get("per_launch", {}):
                line["roofline"]["traffic"] = prof["per_launch"]["qkv_proj"]["bytes"] / 1e9
        except (OSError, ValueError):
            pass
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = proj_cpu_leg(pw)
        print(json.dumps(line), flush=True)
        return
    if args.tconv:
        tw = wl.TCONV_WORKLOADS["tconv_" + args.workload]
        fwd_ms, apply_ms, commit_ms = tconv_leg(tw, args.steps, args.warmup, args.sets, not args.no_streaming)
        act = tw.elems * 2
        gbs = 2 * act / (fwd_ms * 1e-3) / 1e9
        line = {
            "metric": "tokens/s of the causal temporal convolution (all channels); % of HBM peak",
            "value": tw.B * tw.T * tw.Hs * tw.Ws / (fwd_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": fwd_ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) activations, N(0,1/3) taps, N(0,0.01) bias; resident in HBM)",
            "config": {"workload": f"{tw.name}: B={tw.B} grid {tw.T}x{tw.Hs}x{tw.Ws}, C={tw.C} channels, "
                                   f"blocks of {tw.F} frames, bf16, 3-tap depthwise, one-frame cache",
                       "B": tw.B, "tokens": tw.T * tw.Hs * tw.Ws, "C": tw.C, "blocks": tw.nb},
            "hbm_frac_step": gbs / HBM_PEAK_GBS,
            # one kernel per step: x read once, y written once
            "roofline": {"bound": "hbm", "kernel": "tconv", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None, "alg_bytes": 2 * act / 1e9},
        }
        if apply_ms is not None:
            line["block_apply_us"], line["block_commit_us"] = apply_ms * 1e3, commit_ms * 1e3
        try:
            with open(traffic_file(tw.name)) as f:
                prof = json.load(f)
            if prof.get("source_sha256") == source_sha256(TCONV_SRC) and "tconv" in prof.get("per_launch", {}):
                line["roofline"]["traffic"] = prof["per_launch"]["tconv"]["bytes"] / 1e9
        except (OSError, ValueError):
            pass
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = tconv_cpu_leg(tw)
        print(json.dumps(line), flush=True)
        return
    w = wl.WORKLOADS[args.workload]
    data_note = "synthetic (seeded N(0,1) draws" + (f", K x{w.k_scale:g}" if w.k_scale != 1.0 else "") + \
        "; resident in HBM)"
    if args.backward:
        ms, ms_recompute = bwd_leg(w, args.steps, args.warmup, args.sets)
        esz = 2 if w.dtype == "bf16" else 4
        tensor = w.B * w.H * w.N * w.d * esz
        print(json.dumps({
            "metric": "tokens/s (all heads) block-causal linear attn backward (dq, dk, dv); % of HBM peak",
            "value": w.B * w.N / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": data_note,
            "config": {"workload": f"{w.name} backward: B={w.B} H={w.H} d={w.d} grid {w.T}x{w.Hs}x{w.Ws} "
                                   f"({w.N} tokens), blocks of {w.F} frames",
                       "B": w.B, "H": w.H, "d": w.d, "tokens": w.N, "blocks": w.nb},
            # q, k, v, dout read once and dq, dk, dv written once
            "alg_bytes": 7 * tensor,
            "hbm_frac_step": 7 * tensor / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
            "states": "saved by the forward (sva_lin_attn_fwd_save)",
            "ms_per_step_recomputing_states": ms_recompute,
        }), flush=True)
        return
    if args.stream:
        ms, ms_split = stream_leg(w, args.steps, args.warmup)
        esz = 2 if w.dtype == "bf16" else 4
        tensor = w.B * w.H * w.N * w.d * esz
        cache = w.B * w.H * (w.d * w.d + w.d) * 4
        # per block: q, k, v read and out written once, the cache read and
        # written once
        alg = 4 * tensor + 2 * cache * w.nb
        print(json.dumps({
            "metric": "tokens/s (all heads) of block-by-block generation on one cache (output + commit per block)",
            "value": w.B * w.N / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": data_note,
            "config": {"workload": f"{w.name} streamed: B={w.B} H={w.H} d={w.d} grid {w.T}x{w.Hs}x{w.Ws} "
                                   f"({w.N} tokens) as {w.nb} blocks of {w.F} frames, one {cache}-byte cache",
                       "B": w.B, "H": w.H, "d": w.d, "tokens": w.N, "blocks": w.nb},
            "us_per_block": ms * 1e3 / w.nb,
            "calls": "one sva_lin_attn_fwd per block, the cache as S0 and S_out",
            "ms_per_step_apply_then_commit": ms_split, "us_per_block_apply_then_commit": ms_split * 1e3 / w.nb,
            "alg_bytes": alg, "hbm_frac_step": alg / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
        }), flush=True)
        return
    if w.prior_blocks:
        c = cached_leg(w, args.steps, args.warmup)
        apply_ms, commit_ms = c["apply_ms"], c["commit_ms"]
        tok = w.B * w.block_tokens
        print(json.dumps({
            "metric": "tokens/s of one cached denoising step (block apply against the cache)",
            "value": tok / (apply_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": apply_ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": data_note,
            "config": {"workload": f"{w.name}: B={w.B} H={w.H} d={w.d} one block of {w.F}x{w.Hs}x{w.Ws} "
                                   f"({w.block_tokens} tokens) at t0={w.t0} against a cache of "
                                   f"{w.prior_blocks} committed blocks, {w.dtype}",
                       "B": w.B, "H": w.H, "d": w.d, "tokens": w.block_tokens},
            "us_per_step": apply_ms * 1e3, "commit_us": commit_ms * 1e3,
            "us_per_step_graph": c["apply_graph_ms"] * 1e3, "commit_us_graph": c["commit_graph_ms"] * 1e3,
            "us_per_step_noalloc_graph": c["noalloc_graph_ms"] * 1e3,
            "hbm_frac_step": 4 * w.B * w.H * w.block_tokens * w.d * (2 if w.dtype == "bf16" else 4)
            / (apply_ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
        }), flush=True)
        return
    # The W warm-up and K timed steps of the headline workload come first
    # (measured: running the other workloads before them made the timed steps
    # about 3 us slower); its repeats and per-kernel timings, the copy
    # ceiling and the other workloads follow in the same process.
    fb = ForwardBench(w, args.sets)
    res = fb.run(args.steps, args.warmup, repeats=args.repeats, stage_calls=args.steps)
    fb.free()
    others = {}
    ext = {}
    copy = None
    if not args.no_others and w.name == "720p":
        copy = copy_ceiling()
        # The other workloads and the extension rows are steady-state figures
        # whatever K and W the headline takes: a leg's first calls after it
        # sets up its buffers run slower (720p backward over 20 calls: 255 us
        # after 5 warm-up calls, 240.7 us after 50), and over a few calls the
        # host's first launches weigh in (480p: 63.1 us over 20 steps, 57.3
        # over 200), so each leg warms up at least SECONDARY_WARMUP calls and
        # the other workloads time at least SECONDARY_STEPS.
        others = other_workloads(max(args.steps, SECONDARY_STEPS), max(args.warmup, SECONDARY_WARMUP), args.sets)
        ext = extension_rows(min(args.steps, 20), SECONDARY_WARMUP, args.sets)
    ms_per_step = res["ms"]
    esz = 2 if w.dtype == "bf16" else 4
    elems = w.B * w.H * w.N * w.d
    alg_bytes = {"reduce": 2 * elems * esz, "apply": 2 * elems * esz}
    # kernel durations: back-to-back launches replayed from a HIP graph (the
    # same figure rocprofv3's trace gives for a run of back-to-back launches)
    stage_us = res["stage_graph_us"]
    dom = "reduce" if stage_us["reduce"] >= stage_us["apply"] else "apply"
    achieved = alg_bytes[dom] / (stage_us[dom] * 1e-6) / 1e9
    traffic = None
    try:
        with open(traffic_file(w.name)) as f:
            prof = json.load(f)
        if prof.get("source_sha256") == source_sha256() and dom in prof.get("per_launch", {}):
            traffic = prof["per_launch"][dom]["bytes"] / 1e9  # GB per launch, from the counters
    except (OSError, ValueError):
        traffic = None
    step_bytes = 4 * elems * esz
    reps = sorted(res["repeat_ms"]) or [ms_per_step]
    line = {
        "metric": "tokens/s (all heads) block-causal linear attn fwd; % of HBM peak",
        "value": w.B * w.N / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": data_note,
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} d={w.d} grid {w.T}x{w.Hs}x{w.Ws} "
                               f"({w.N} tokens) blocks of {w.F} frames ({w.nb} blocks), {w.dtype}, "
                               f"numerator-only 3D RoPE {w.split[0]}/{w.split[1]}/{w.split[2]}",
                   "B": w.B, "H": w.H, "d": w.d, "tokens": w.N, "blocks": w.nb},
        "hbm_frac_step": step_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
        # the step over `repeats` further runs of K steps each (GPU time)
        "step_us": {"mean": ms_per_step * 1e3, "median": reps[len(reps) // 2] * 1e3, "min": reps[0] * 1e3,
                    "max": reps[-1] * 1e3, "runs": len(res["repeat_ms"])},
        # dominant kernel: algorithmic bytes per launch / its duration, the
        # duration from K back-to-back launches of that kernel alone
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_unit": "GB per launch", "alg_bytes": alg_bytes[dom] / 1e9},
        "kernels_us": {k: round(v, 2) for k, v in stage_us.items()},
        # the same launches issued one Python call at a time (the scan's few
        # microseconds are below the host's cost per call)
        "kernels_eager_us": {k: round(v, 2) for k, v in res["stage_us"].items()},
        "kernels_frac": {k: round(alg_bytes[k] / (stage_us[k] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                         for k in ("reduce", "apply")},
    }
    if copy is not None:
        line["copy_ceiling"] = copy
        line["hbm_frac_of_copy_ceiling"] = step_bytes / (ms_per_step * 1e-3) / 1e9 / copy["GB/s"]
    if others:
        line["other_workloads"] = others
    if ext:
        line["extension_rows"] = {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                                  for k, v in ext.items()}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_leg(w, args.cpu_reps)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
