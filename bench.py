"""Decode-step benchmark: selector scoring + dual top-p + sparse attention at L=128K.

    python bench.py [--steps K] [--warmup W] [--workload c3_128k_b8] [--no-cpu-baseline]

Times K back-to-back decode steps (the three C calls per step, enqueued on one stream)
between device synchronisations, with inputs already resident in HBM, and prints one
JSON line. The sparse-attention call is the dominant kernel: HIP events on its launch
stream around K back-to-back calls give its average duration, and its algorithmic
bytes per launch over that duration is the roofline figure. A second pass with events
between the calls gives a per-call breakdown, and a third replays the step captured as
a HIP graph. The CPU baseline is the fp64 oracle timed on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

import numpy as np
import torch

import block_sparse_long_spot_amd as spot
from block_sparse_long_spot_amd import workloads as W
from block_sparse_long_spot_amd.decode import DecodeBuffers, DecodeStep

METRIC = "decode step µs (select+top-p+sparse attn) at L=128K; achieved HBM GB/s %peak"
HBM_PEAK_GBPS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def selected_tokens(sel_idx, sel_cnt, L, block):
    idx = sel_idx.cpu().numpy()
    cnt = sel_cnt.cpu().numpy()
    tot = 0
    nbl = -(-L // block)
    for b in range(idx.shape[0]):
        for blk in idx[b, : int(cnt[b])]:
            if 0 <= blk < nbl:
                tot += min((int(blk) + 1) * block, L) - int(blk) * block
    return tot


def byte_budget(wl, B, tokens):
    """Algorithmic bytes of one step, split by call."""
    es = 4 if wl.dtype == "f32" else 2
    n_el = B * wl.nb * wl.kpb * wl.H_idx * wl.d_idx
    if wl.sel_k_dtype == "int4":
        selk = n_el // 2 + (n_el // 32) * 2
    else:
        selk = n_el * (4 if wl.sel_k_dtype == "f32" else 2)
    score = selk + B * wl.H_idx * (wl.d_idx * es + 4) + B * wl.nb * 4
    topp = B * wl.nb * 4 + B * wl.K_max * 4 + B * 8
    attn = tokens * wl.Hkv * wl.d * 2 * es + B * wl.Hq * wl.d * 2 * es
    algorithmic = selk + B * wl.H_idx * (wl.d_idx * es + 4) + tokens * wl.Hkv * wl.d * 2 * es \
        + B * wl.Hq * wl.d * 2 * es
    return {"score": score, "topp": topp, "attn": attn, "step": algorithmic}


ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILE = os.path.join(ROOT, "profiles", "attn_mfma_c3_128k_b8.md")
ATTN_SRC = os.path.join(ROOT, "block_sparse_long_spot_amd", "csrc", "attn.hip")


def profiled_traffic():
    """HBM bytes per sparse-attention call from the committed rocprofv3 counter summary,
    or None when the attention source changed since those counters were taken."""
    try:
        fields = dict(re.findall(r"^(\w+): (\S+)$", open(PROFILE).read(), re.M))
        digest = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    if fields.get("source_sha256_16") != digest:
        return None
    return int(fields["traffic_bytes_per_launch"])


def time_back_to_back(fn, steps, warmup, stream, events=True):
    """K calls of `fn` enqueued back to back on `stream`, after `warmup` untimed ones,
    bracketed by device synchronisations. Returns (wall us per call, HIP-event us per
    call) with the two events recorded on `stream` around the K calls; with
    events=False none are recorded (each adds a gap on the stream) and the second value
    is None."""
    torch.cuda.synchronize()  # inputs made on torch's default stream are complete
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        if events:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        if events:
            a.record(stream)
        for _ in range(steps):
            fn()
        if events:
            b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    return wall * 1e6 / steps, (a.elapsed_time(b) * 1e3 / steps if events else None)


def settle(fn, seconds, stream, chunk=500):
    """Untimed calls of `fn` back to back on `stream` for about `seconds`; returns how
    many were made."""
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        with torch.cuda.stream(stream):
            for _ in range(chunk):
                fn()
        torch.cuda.synchronize()
        n += chunk
    return n


def time_steps(inp, wl, bufs, steps, warmup, stream):
    """Per-call breakdown: events between the three calls of every step. Each event adds
    a gap on the stream, so these per-call times are diagnostics, not the step time."""
    step = DecodeStep(inp, wl, bufs, stream=stream)
    torch.cuda.synchronize()  # inputs made on torch's default stream are complete
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    score, topp, attn = step.calls
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(steps):
            ev[i][0].record(stream)
            score()
            ev[i][1].record(stream)
            topp()
            ev[i][2].record(stream)
            attn()
            ev[i][3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {"score": [], "topp": [], "attn": [], "step": []}
    for e in ev:
        per["score"].append(e[0].elapsed_time(e[1]) * 1e3)
        per["topp"].append(e[1].elapsed_time(e[2]) * 1e3)
        per["attn"].append(e[2].elapsed_time(e[3]) * 1e3)
        per["step"].append(e[0].elapsed_time(e[3]) * 1e3)
    gpu_total_us = ev[0][0].elapsed_time(ev[-1][3]) * 1e3
    return wall, gpu_total_us, per


def time_graph(inp, wl, bufs, steps, warmup, stream):
    """The same step captured once as a HIP graph and replayed: identical kernels and
    arguments, without per-launch host work between them."""
    g = torch.cuda.CUDAGraph()
    step = DecodeStep(inp, wl, bufs, stream=stream)
    torch.cuda.synchronize()  # inputs made on torch's default stream are complete
    step()   # warm the code objects before capture
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        step()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e6 / steps, a.elapsed_time(b) * 1e3 / steps


class GraphSteps:
    """K decode steps as HIP graphs, the way a server captures the launch-bound part of a
    token (one graph of up to 200 steps, replayed K // 200 times, plus one graph for the
    rest): the same kernels with the same arguments as the stream-launched steps,
    dispatched without host work between them. Calling it runs the K steps on `stream`.
    `output_matches`: a replay leaves the output the stream-launched steps leave."""

    MAX_STEPS = 200

    def __init__(self, step, steps, stream, out):
        self.stream = stream
        self.k = steps
        g_n = min(steps, self.MAX_STEPS)
        self.full, self.n_full = self._capture(step, g_n), steps // g_n
        rest = steps - self.n_full * g_n
        self.rest = self._capture(step, rest) if rest else None
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            step()
        torch.cuda.synchronize()
        ref = out.clone()
        out.zero_()
        torch.cuda.synchronize()
        self()
        torch.cuda.synchronize()
        self.output_matches = bool(torch.equal(ref, out))

    def _capture(self, step, n):
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=self.stream):
            for _ in range(n):
                step()
        torch.cuda.synchronize()
        return g

    def __call__(self):
        for _ in range(self.n_full):
            self.full.replay()
        if self.rest is not None:
            self.rest.replay()


def time_flushed_call(fn, reps, stream):
    """us of single calls of `fn` on `stream`, each after a 1 GiB write (outside the
    events), so that no call reads data left in the last-level caches by the one before."""
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    times = []
    torch.cuda.synchronize()  # inputs made on torch's default stream are complete
    with torch.cuda.stream(stream):
        for _ in range(reps):
            scratch.fill_(1.0)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e3)
    del scratch
    return times


def time_flushed(inp, wl, bufs, reps, stream):
    """Per-step time with a 1 GiB write between steps (outside the events)."""
    return time_flushed_call(DecodeStep(inp, wl, bufs, stream=stream), reps, stream)


def time_flushed_graph(step, stream, n=20, reps=15):
    """Per-step time after a 1 GiB write, without an event beside every step (each adds a
    gap of about 2 us): one HIP graph of n (write, step) pairs and one of the n writes
    alone, each replayed `reps` times between device synchronisations; the step's time
    is the difference of the two medians divided by n. The write is a fill kernel."""
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    graphs = []
    for with_step in (True, False):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(n):
                scratch.fill_(1.0)
                if with_step:
                    step()
        graphs.append(g)
    torch.cuda.synchronize()
    med = []
    for g in graphs:
        g.replay()  # untimed first replay
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
        med.append(statistics.median(ts))
    del graphs, scratch
    torch.cuda.empty_cache()
    return round((med[0] - med[1]) * 1e6 / n, 3)


def time_step_distribution(fn, n, warmup, stream):
    """Per-step times of n back-to-back steps: one HIP event recorded on `stream` at every
    step boundary (each adds a small gap, so the mean sits a little above the headline's
    wall-clock mean). Returns median, p10, p90 and mean in us."""
    torch.cuda.synchronize()  # inputs made on torch's default stream are complete
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    with torch.cuda.stream(stream):
        ev[0].record(stream)
        for i in range(n):
            fn()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n)])
    return {"median": round(float(np.median(t)), 3), "p10": round(float(np.percentile(t, 10)), 3),
            "p90": round(float(np.percentile(t, 90)), 3), "mean": round(float(t.mean()), 3),
            "n": n}


def burst_stats(fn, steps, stream, reps=None):
    """The headline measurement repeated: `reps` bursts of `steps` back-to-back steps, each
    after one warm-up step and bracketed by device synchronisations; quantiles of the
    per-step wall time over the bursts (no events inside a burst)."""
    reps = reps or min(100, max(10, 2000 // steps))
    return quantiles([time_back_to_back(fn, steps, 1, stream, events=False)[0]
                      for _ in range(reps)])


def quantiles(xs):
    return {"median": round(statistics.median(xs), 3),
            "p10": round(float(np.percentile(xs, 10)), 3),
            "p90": round(float(np.percentile(xs, 90)), 3), "reps": len(xs)}


def prefill_leg(steps, warmup, stream):
    """The 128-query prefill tile at 32K: tile scoring, top-p, causal sparse attention.
    Returns per-call µs and the attention's achieved TFLOP/s (algorithmic flops:
    4 * d per visible (query, head, token) in the selected blocks)."""
    wl = W.WORKLOADS["c5_prefill_32k"]
    inp = W.make_inputs(wl, device="cuda")
    q_pos0, Tq, nb_vis = wl.q_pos0, wl.prefill_Tq, wl.nb
    scores = torch.empty(wl.B, nb_vis, device="cuda")
    idx = torch.empty(wl.B, nb_vis, dtype=torch.int32, device="cuda")
    cnt = torch.empty(wl.B, dtype=torch.int32, device="cuda")
    out = torch.empty(wl.B, wl.Hq, Tq, wl.d, dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(wl.d)

    def run(ev=None):
        if ev:
            ev[0].record(stream)
        spot.spot_prefill_select_score(inp["sel_q"], inp["sel_w"], inp["sel_k"], scores, q_pos0,
                                       stream=stream)
        if ev:
            ev[1].record(stream)
        spot.spot_select_topp(scores, idx, cnt, None, wl.p, wl.K_min, nb_vis, wl.n_sink,
                              wl.n_rec, stream=stream)
        if ev:
            ev[2].record(stream)
        spot.spot_prefill_attn(inp["q"], inp["K"], inp["V"], idx, cnt, out, q_pos0, scale,
                               stream=stream)
        if ev:
            ev[3].record(stream)

    torch.cuda.synchronize()  # inputs made on torch's default stream are complete
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for e in evs:
            run(e)
    torch.cuda.synchronize()
    t = {k: statistics.fmean([e[i].elapsed_time(e[i + 1]) * 1e3 for e in evs])
         for i, k in enumerate(["score", "topp", "attn"])}
    sel = idx[0, : int(cnt[0])].cpu().tolist()
    vis = 0
    for i in range(Tq):
        pos = q_pos0 + i
        for blk in sel:
            vis += max(0, min((blk + 1) * wl.block, pos + 1, wl.L) - blk * wl.block)
    flops = 4.0 * wl.d * vis * wl.Hq
    return {"workload": wl.name, "selected_blocks": len(sel), "visible_blocks": nb_vis,
            "per_call_us_mean": {k: round(v, 3) for k, v in t.items()},
            "attn_flops": flops,
            "attn_TFLOPs": round(flops / (t["attn"] * 1e-6) / 1e12, 2),
            "attn_frac_of_bf16_mfma_peak": round(flops / (t["attn"] * 1e-6) / 2.5e15, 4)}


def prefill_sequence_leg(steps, warmup, stream):
    """A whole 32K prefill of the c5 layer (32 query / 8 KV heads, d 128, selector 4 x
    64, block 64) in 256 tiles of 128 queries: tile scoring, per-tile top-p (sink 1,
    recency 4 blocks at each tile's diagonal, p 0.95) and causal sparse attention, one
    launch each. Reports per-call µs, the attention's algorithmic TFLOP/s and the
    fraction of dense causal attention's flops that the selection keeps."""
    wl = W.WORKLOADS["c5_prefill_32k"]
    B, T, Tq, d, H, di, block = 1, wl.L, wl.prefill_Tq, wl.d, wl.H_idx, wl.d_idx, wl.block
    L, nb = wl.L, wl.nb
    n_tiles = -(-T // Tq)
    g = torch.Generator(device="cuda")
    g.manual_seed(49)
    sel_q = torch.randn(B, T, H, di, generator=g, device="cuda").bfloat16()
    sel_w = torch.randn(B, T, H, generator=g, device="cuda").abs()
    sel_k = torch.randn(B, nb, 1, H, di, generator=g, device="cuda").bfloat16()
    Q = torch.randn(B, wl.Hq, T, d, generator=g, device="cuda").bfloat16()
    K = torch.randn(B, wl.Hkv, L, d, generator=g, device="cuda").bfloat16()
    V = torch.randn(B, wl.Hkv, L, d, generator=g, device="cuda").bfloat16()
    scores = torch.empty(B, n_tiles, nb, device="cuda")
    idx = torch.empty(B, n_tiles, nb, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, n_tiles, dtype=torch.int32, device="cuda")
    out = torch.empty(B, wl.Hq, T, d, dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(d)
    calls = {
        "score": lambda: spot.spot_prefill_select_score(sel_q, sel_w, sel_k, scores, 0, Tq=Tq,
                                                        stream=stream),
        "topp": lambda: spot.spot_prefill_select_topp(scores, idx, cnt, None, wl.p, wl.K_min,
                                                      nb, wl.n_sink, wl.n_rec, 0, T, Tq=Tq,
                                                      stream=stream),
        "attn": lambda: spot.spot_prefill_attn(Q, K, V, idx, cnt, out, 0, scale, Tq=Tq,
                                               stream=stream),
    }

    def whole():
        for f in calls.values():
            f()

    us_total, _ = time_back_to_back(whole, steps, warmup, stream)
    per = {k: round(time_back_to_back(f, steps, warmup, stream)[0], 3) for k, f in calls.items()}
    # the same whole-prompt tile scoring with the selector key cache quantised (§5.3)
    fmts = {}
    raw_k = sel_k.float()
    for fmt in ("int4", "fp4", "int8", "fp8"):
        codes, ks = W.quantize_selector(raw_k, fmt)
        nbytes = codes.numel() * codes.element_size() + (
            ks.numel() * ks.element_size() if ks.numel() > 1 else 0)
        us, _ = time_back_to_back(
            lambda: spot.spot_prefill_select_score(sel_q, sel_w, codes, scores, 0, Tq=Tq,
                                                   stream=stream, sel_k_scale=ks),
            steps, warmup, stream)
        fmts[fmt] = {"us": round(us, 3), "key_bytes": nbytes}
    fmts["bf16"] = {"us": per["score"], "key_bytes": sel_k.numel() * 2}
    whole()
    torch.cuda.synchronize()
    ic, cc = idx.cpu().numpy()[0], cnt.cpu().numpy()[0]
    vis = 0
    for t in range(n_tiles):
        pos = np.arange(t * Tq, min((t + 1) * Tq, T))
        for blk in ic[t, : cc[t]]:
            lo = blk * block
            vis += int(np.clip(np.minimum(pos + 1, lo + block) - lo, 0, None).sum())
    flops = 4.0 * d * vis * wl.Hq
    dense = 4.0 * d * wl.Hq * T * (T + 1) / 2
    return {"T": T, "tiles": n_tiles, "us_total": round(us_total, 3), "per_call_us": per,
            "score_by_key_format": fmts,
            "selected_blocks_mean": round(float(cc.mean()), 2),
            "attn_flops": flops, "dense_causal_flops": dense,
            "flop_fraction_of_dense": round(flops / dense, 5),
            "attn_TFLOPs": round(flops / (per["attn"] * 1e-6) / 1e12, 2)}


def static_topk_leg(inp, wl, steps, warmup, stream):
    """Static top-K (Eq. 6) with K = half the blocks, no reserved blocks: the paper's
    K = 0.5L decode rows (Table 1), on the same 128K batch-8 inputs. Four times the
    attention bytes of the top-p headline."""
    K = wl.nb // 2
    ws = wl.with_(p=0.0, K_min=K, K_max=K, n_sink=0, n_rec=0)
    bufs = DecodeBuffers.of(ws, inp["q"].dtype)
    us, _ = time_back_to_back(DecodeStep(inp, ws, bufs, stream=stream), steps, warmup, stream)
    _, _, per = time_steps(inp, ws, bufs, max(10, steps // 10), warmup, stream)
    tok = selected_tokens(bufs.sel_idx, bufs.sel_cnt, ws.L, ws.block)
    bb = byte_budget(ws, ws.B, tok)
    return {"K_blocks": K, "us_per_step": round(us, 3), "algorithmic_bytes": bb["step"],
            "GBps": round(bb["step"] / (us * 1e-6) / 1e9, 1),
            "frac": round(bb["step"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "per_call_us_mean": {k: round(statistics.fmean(v), 3) for k, v in per.items()}}


def budgets_vary_leg(wl, steps, warmup, stream):
    """The 128K batch-8 layer with the Zipf exponent of each batch row spread over
    [1.3, 2.0], so the p = 0.95 nucleus (and the selected set) differs from row to row
    instead of every row hitting the K_max cap: the case top-p exists for. Reports the
    step, the attention call and the per-row block counts."""
    ws = wl.with_(zipf_spread=(1.3, 2.0))
    inp = W.make_inputs(ws, device="cuda")
    bufs = DecodeBuffers.of(ws, inp["q"].dtype)
    us, _ = time_back_to_back(DecodeStep(inp, ws, bufs, stream=stream), steps, warmup, stream)
    scale = 1.0 / math.sqrt(ws.d)
    attn_us, _ = time_back_to_back(
        lambda: spot.spot_sparse_attn(inp["q"], inp["K"], inp["V"], bufs.sel_idx,
                                      bufs.sel_cnt, bufs.out, bufs.workspace, scale,
                                      block=ws.block, stream=stream), steps, warmup, stream)
    tok = selected_tokens(bufs.sel_idx, bufs.sel_cnt, ws.L, ws.block)
    bb = byte_budget(ws, ws.B, tok)
    res = {"zipf_exponents": [1.3, 2.0], "selected_blocks": bufs.sel_cnt.tolist(),
           "us_per_step": round(us, 3), "algorithmic_bytes": bb["step"],
           "GBps": round(bb["step"] / (us * 1e-6) / 1e9, 1),
           "attn_call_us": round(attn_us, 3),
           "attn_GBps": round(bb["attn"] / (attn_us * 1e-6) / 1e9, 1)}
    del inp, bufs
    torch.cuda.empty_cache()
    return res


def page_geometry_step(steps, warmup, stream):
    """A whole decode step at the paper's own geometry and inference settings (Appendix
    A, Table 3): 16-token blocks, one selector key per token (4 heads x 128), sink 128
    tokens, recency 256, K_min 512 tokens, p = 0.9, no cap; 128K context, batch 1,
    Zipf(1.1) selector masses. Table 1 reports the selector at 1.55 ms per decoded
    token for Qwen3-8B; read as the sum over its 36 layers that is about 43 us per
    layer, on one NVIDIA B200 (context, not a target)."""
    wl = W.WORKLOADS["page_128k_b1"]
    inp = W.make_inputs(wl, device="cuda")
    bufs = DecodeBuffers.of(wl, inp["q"].dtype)
    step = DecodeStep(inp, wl, bufs, stream=stream)
    us, _ = time_back_to_back(step, steps, warmup, stream)
    _, _, per = time_steps(inp, wl, bufs, steps, warmup, stream)
    tok = selected_tokens(bufs.sel_idx, bufs.sel_cnt, wl.L, wl.block)
    bb = byte_budget(wl, wl.B, tok)
    mean = {k: statistics.fmean(v) for k, v in per.items()}
    # the step and the attention call after a 1 GiB write each, and the read-only kernel
    # over the call's K/V bytes the same way (as 16 KiB blocks: the call reads 4 KiB
    # pieces, which a read-only kernel of that size reads within a few per cent as fast)
    fl = quantiles(time_flushed_call(step, 200, stream))
    fa = quantiles(time_flushed_call(step.calls[2], 200, stream))
    rc = read_ceiling(bb["attn"], stream, reps=200, flushed=True)
    rc["attn_frac_of_it"] = round(bb["attn"] / (fa["median"] * 1e-6) / 1e9 / rc["GBps"], 4)
    res = {"workload": wl.name,
           "geometry": "L 131072, block 16, 16 per-token selector keys per block, 4 x 128 "
                       "bf16, batch 1; p 0.9, K_min 32, sink 8, recency 16 blocks, no cap",
           "us_per_step": round(us, 3), "algorithmic_bytes": bb["step"],
           "GBps": round(bb["step"] / (us * 1e-6) / 1e9, 1),
           "frac": round(bb["step"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
           "selected_blocks": int(bufs.sel_cnt[0]),
           "per_call_us_mean": {k: round(v, 3) for k, v in mean.items()},
           "score_bytes": bb["score"],
           "score_GBps": round(bb["score"] / (mean["score"] * 1e-6) / 1e9, 1),
           "flushed_step_us": fl, "flushed_attn_call_us": fa, "read_ceiling_flushed": rc,
           "paper_selector_us_per_layer_B200": round(1550.0 / 36, 1)}
    del inp, bufs, step
    torch.cuda.empty_cache()
    return res


def selector_formats_leg(steps, warmup, stream):
    """Scoring alone at the paper's page geometry (128K context, 16 per-token keys per
    16-token block, 4 heads x 128, batch 1) with the key cache in each precision of
    §5.3 / Table 9: µs per call (events around back-to-back calls) and key bytes per
    second. Table 1 reports the paper's selector slower at INT4 (1.91 ms) and FP4
    (2.51 ms) than at BF16 (1.55 ms) on one B200, from dequantisation overhead."""
    wl = W.WORKLOADS["page_128k_b1"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(48)
    shape_k = (1, wl.nb, wl.kpb, wl.H_idx, wl.d_idx)
    raw = torch.randn(*shape_k, generator=gen, device="cuda")
    sel_q = torch.randn(1, wl.H_idx, wl.d_idx, generator=gen, device="cuda").bfloat16()
    sel_w = torch.randn(1, wl.H_idx, generator=gen, device="cuda").abs()
    scores = torch.empty(1, wl.nb, device="cuda")
    res = {"geometry": "L 131072, block 16, 16 keys per block, 4 x 128, batch 1, bf16 query",
           "quantize": "spot_quantize_selector over the whole bf16 cache (131072 rows of "
                       "512): bytes read + written per second"}
    rows_bf16 = raw.reshape(-1, wl.H_idx * wl.d_idx).bfloat16().contiguous()
    for fmt in ("bf16", "int8", "fp8", "int4", "fp4"):
        codes, scale = W.quantize_selector(raw, fmt)
        nbytes = codes.numel() * codes.element_size() + (
            scale.numel() * scale.element_size() if scale is not None and scale.numel() > 1
            else 0)
        us, _ = time_back_to_back(
            lambda: spot.spot_select_score(sel_q, sel_w, codes, scale, scores, kpb=wl.kpb,
                                           stream=stream), steps, warmup, stream)
        res[fmt] = {"us": round(us, 3), "key_bytes": nbytes,
                    "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
        if fmt != "bf16":
            c2 = codes.view(torch.uint8).reshape(rows_bf16.shape[0], -1)
            s2 = scale.reshape(rows_bf16.shape[0], -1) if scale.numel() > 1 else None
            ts = scale if scale.numel() == 1 else None
            qus, _ = time_back_to_back(
                lambda: spot.spot_quantize_selector(rows_bf16, fmt, c2, scales=s2,
                                                    tensor_scale=ts, stream=stream),
                steps, warmup, stream)
            moved = rows_bf16.numel() * 2 + nbytes
            res[fmt]["quantize_us"] = round(qus, 3)
            res[fmt]["quantize_GBps"] = round(moved / (qus * 1e-6) / 1e9, 1)
        del codes, scale
    del rows_bf16
    del raw
    torch.cuda.empty_cache()
    return res


def calibration_copy():
    """A plain 256 MiB device copy, outside every timed region: its FETCH_SIZE and
    WRITE_SIZE counters scale the counters of the other kernels to bytes."""
    n = 1 << 26
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    return n * 4


PROBE_SRC = os.path.join(ROOT, "read_ceiling.hip")
PROBE_LIB = os.path.join(ROOT, "libspot_probe.so")


def build_read_ceiling(verbose=False):
    """Compile the read-only reference kernel (read_ceiling.hip, beside this file) into
    libspot_probe.so, a library of its own: it is the benchmark's yardstick, not part of
    the decode path."""
    import shutil
    import subprocess
    hipcc = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


def launch_floor(stream, reps=2000):
    """Per-launch time of back-to-back launches that do (almost) nothing: an empty kernel
    of 256 work-groups, and a kernel reading and writing 65536 floats (one memory round
    trip). HIP events around `reps` launches on `stream`; what any one dependent kernel
    of a step costs at least."""
    import ctypes
    lib = ctypes.CDLL(PROBE_LIB)
    lib.spot_probe_empty.restype = ctypes.c_int
    lib.spot_probe_empty.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.spot_probe_touch.restype = ctypes.c_int
    lib.spot_probe_touch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_void_p]
    n = 1 << 16
    a = torch.ones(n, device="cuda")
    b = torch.empty(n, device="cuda")
    torch.cuda.synchronize()
    res = {}
    for name, go in (("empty_us", lambda k: lib.spot_probe_empty(256, k, stream.cuda_stream)),
                     ("read_write_us", lambda k: lib.spot_probe_touch(
                         a.data_ptr(), b.data_ptr(), n, k, stream.cuda_stream))):
        if go(50) != 0:
            raise RuntimeError("launch-floor probe failed")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if go(reps) != 0:
            raise RuntimeError("launch-floor probe failed")
        e1.record(stream)
        e1.synchronize()
        res[name] = round(e0.elapsed_time(e1) * 1e3 / reps, 3)
    return res


def read_ceiling(nbytes, stream, reps=20, flushed=False):
    """What a kernel that only reads sustains on this GPU for the attention's access
    pattern: about `nbytes` as 16 KiB blocks (one 64-token block of one KV head at
    d = 128 in bf16) picked in random order from a buffer twice that size, 16-byte
    non-temporal loads, no compute. Best of 256, 512 and 1024 work-groups, HIP events
    around `reps` back-to-back launches on `stream`; flushed: the median of `reps`
    single launches, each after a 1 GiB write (as a decode step meets the K/V cache
    when other work ran in between)."""
    import ctypes
    lib = ctypes.CDLL(PROBE_LIB)
    lib.spot_probe_read_blocks.restype = ctypes.c_int
    lib.spot_probe_read_blocks.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    blk = 16384
    n = max(512, nbytes // blk // 512 * 512)
    buf = torch.ones(2 * n * blk // 2, dtype=torch.bfloat16, device="cuda")
    g = torch.Generator().manual_seed(7)
    lst = torch.randperm(2 * n, generator=g)[:n].to(torch.int32).cuda()
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    per = {}
    with torch.cuda.stream(stream):
        for wgs in (256, 512, 1024):
            if n % (2 * wgs):
                continue
            def go():
                st = lib.spot_probe_read_blocks(buf.data_ptr(), lst.data_ptr(), n, wgs,
                                                sink.data_ptr(), stream.cuda_stream)
                if st != 0:
                    raise RuntimeError("spot_probe_read_blocks failed")
            for _ in range(3):
                go()
            if flushed:
                us = statistics.median(time_flushed_call(go, reps, stream))
            else:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    go()
                e1.record(stream)
                e1.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / reps
            per[wgs] = {"us": round(us, 3), "GBps": round(n * blk / (us * 1e-6) / 1e9, 1)}
    del buf, lst, sink
    best = max(v["GBps"] for v in per.values())
    return {"GBps": best, "bytes": n * blk, "per_workgroups": per,
            "what": "read-only kernel, the same bytes as 16 KiB blocks in random order, "
                    "16-byte non-temporal loads, no compute (read_ceiling.hip)"
                    + (", one launch after a 1 GiB write, median" if flushed else "")}


def cpu_baseline(wl, inp, b_sample, b_single=None):
    """The fp64 oracle (scoring, dual top-p, dense masked attention over all L keys) on
    batch rows [0, b_sample), all heads, full L: the median of 3 runs with the BLAS
    thread pool at every core this process may run on, plus one run with a single thread
    on rows [0, b_single). Inputs are copied to the host and widened to fp64 before the
    clock starts, so only the oracle's arithmetic is timed; times are scaled to one whole
    step of the batch."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import spot_oracle as O   # test infrastructure, CPU baseline only
    cores = len(os.sched_getaffinity(0))
    b_single = b_single or max(1, b_sample // 4)
    f64 = lambda t: t[:b_sample].to("cpu").to(torch.float64).numpy()
    sel_q, sel_w, q = f64(inp["sel_q"]), f64(inp["sel_w"]), f64(inp["q"])
    if inp["sel_k"].dtype == torch.uint8:
        keys = O.dequant_int4_g32(inp["sel_k"][:b_sample].cpu().numpy(),
                                  inp["sel_k_scale"][:b_sample].cpu().numpy())
    else:
        keys = f64(inp["sel_k"])
    K, V = f64(inp["K"]), f64(inp["V"])
    pf = float(np.float32(wl.p))

    def run(nb_rows):
        t0 = time.perf_counter()
        s = O.select_score(sel_q[:nb_rows], sel_w[:nb_rows], keys[:nb_rows])
        sels, _ = O.select_topp(s, pf, wl.K_min, wl.K_max, wl.n_sink, wl.n_rec)
        O.sparse_attention(q[:nb_rows], K[:nb_rows], V[:nb_rows], sels, wl.block,
                           1 / math.sqrt(wl.d))
        return time.perf_counter() - t0

    with threadpool_limits(limits=cores):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        runs = [run(b_sample) for _ in range(3)]
    with threadpool_limits(limits=1):
        one = run(b_single)
    del K, V
    B = inp["q"].shape[0]
    med = statistics.median(runs)
    return {"value": round(med * 1e6 * B / b_sample, 1), "unit": "us", "cores": int(threads),
            "kind": "oracle",
            "runs_s": [round(r, 3) for r in runs],
            "single_thread": {"value": round(one * 1e6 * B / b_single, 1), "unit": "us",
                              "cores": 1, "sample": f"batch rows 0..{b_single - 1}, one run "
                                                    f"({one:.2f} s), scaled x{B / b_single:g}"},
            "sample": f"batch rows 0..{b_sample - 1} of {B} (all {wl.Hq} heads, L={wl.L}): "
                      f"median of 3 runs ({med:.2f} s) with the BLAS pool at {threads} "
                      f"threads ({cores} cores in the process affinity), scaled "
                      f"x{B / b_sample:g} to one step; fp64 scoring, sort-based top-p and "
                      "dense masked attention over all L keys; inputs copied to the host and "
                      "widened to fp64 before timing"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="c3_128k_b8", choices=sorted(W.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flushed-reps", type=int, default=200)
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of untimed back-to-back steps before any timing")
    ap.add_argument("--extra-b1", action="store_true", default=True)
    ap.add_argument("--no-extra-b1", dest="extra_b1", action="store_false")
    ap.add_argument("--no-prefill", dest="prefill", action="store_false", default=True)
    ap.add_argument("--no-int4", dest="int4", action="store_false", default=True)
    ap.add_argument("--no-static", dest="static", action="store_false", default=True)
    ap.add_argument("--no-page-geometry", dest="page_geometry", action="store_false",
                    default=True)
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the two prefill legs (for profiling) and print them as "
                         "one JSON line instead of the decode headline")
    a = ap.parse_args()
    if a.gpus != 1:
        print("bench.py measures one GPU only: the decode step runs on one device and "
              "there is no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    spot.load()
    if a.prefill_only:
        stream = torch.cuda.Stream()
        calibration_copy()
        out = {"prefill": prefill_leg(max(10, a.steps // 4), 5, stream),
               "prefill_sequence": prefill_sequence_leg(max(5, a.steps // 50), 3, stream)}
        print(json.dumps(out), flush=True)
        return
    wl = W.WORKLOADS[a.workload]
    if wl.prefill_Tq:
        print("choose a decode workload", file=sys.stderr)
        sys.exit(2)
    log(f"bench: workload {wl.name}, generating inputs on the GPU")
    inp = W.make_inputs(wl, device="cuda")
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    dt = inp["q"].dtype
    bufs = DecodeBuffers.of(wl, dt)
    log(f"bench: warmup {a.warmup}, timing {a.steps} steps")
    scale = 1.0 / math.sqrt(wl.d)

    step = DecodeStep(inp, wl, bufs, stream=stream)

    attn_call = step.calls[2]

    # about a second of untimed steps first, so that every timed pass starts from the
    # GPU's steady state under load (in 20-step runs, 0, 0.3, 1 and 3 s of it gave the
    # same step times within noise)
    settled = settle(step, a.settle_s, stream)
    log(f"bench: {settled} untimed steps to settle the clocks")
    # per-call breakdown first: a diagnostic pass of at least 500 steps (~50 ms)
    n_diag = max(a.steps, 500)
    wall, gpu_total_us, per = time_steps(inp, wl, bufs, n_diag, a.warmup, stream)
    us_step_percall = wall * 1e6 / n_diag
    # headline: K whole steps, captured as HIP graphs and replayed, bracketed by device
    # synchronisations; beside it the same K steps launched from the host one by one
    graph_steps = GraphSteps(step, a.steps, stream, bufs.out)
    # after any idle gap (the capture above, a pause) the GPU needs about 10 ms of load to
    # reach its steady clocks: the first 20-step bursts after a 0.5 s pause ran 100, 98,
    # 98 and 97 us per step against 95 after that. So the timed steps follow ~30 ms of
    # untimed replays with nothing but the bracketing synchronisation in between.
    settle(graph_steps, 0.03, stream, chunk=1)
    us_step = time_back_to_back(graph_steps, 1, 1, stream, events=False)[0] / a.steps
    us_stream, _ = time_back_to_back(step, a.steps, a.warmup, stream, events=False)
    _, us_step_events = time_back_to_back(step, a.steps, 1, stream)
    log(f"bench: {us_step:.1f} us/step (graphs), {us_stream:.1f} us/step (stream launches), "
        f"{us_step_events:.1f} us/step events")
    reps = min(100, max(10, 2000 // a.steps))
    step_stats = {"bursts": quantiles([time_back_to_back(graph_steps, 1, 1, stream,
                                                         events=False)[0] / a.steps
                                       for _ in range(reps)]),
                  "stream_launch_bursts": burst_stats(step, a.steps, stream),
                  "per_step_events": time_step_distribution(step, max(200, a.steps), a.warmup,
                                                            stream)}
    graphs_ok = graph_steps.output_matches
    del graph_steps
    log(f"bench: step statistics {step_stats}")
    tokens = selected_tokens(bufs.sel_idx, bufs.sel_cnt, wl.L, wl.block)
    budget = byte_budget(wl, wl.B, tokens)
    # dominant call: K attention calls back to back on the same stream, same selection
    attn_wall, attn_us = time_back_to_back(attn_call, a.steps, a.warmup, stream)
    mean = {k: statistics.fmean(v) for k, v in per.items()}
    med = {k: statistics.median(v) for k, v in per.items()}
    log(f"bench: per-call event means {mean}")
    flushed = time_flushed(inp, wl, bufs, a.flushed_reps, stream) if a.flushed_reps else []
    flushed_attn = (quantiles(time_flushed_call(attn_call, a.flushed_reps, stream))
                    if a.flushed_reps else None)
    flushed_graph = time_flushed_graph(step, stream) if a.flushed_reps else None
    g_wall, g_event = time_graph(inp, wl, bufs, a.steps, a.warmup, stream)
    log(f"bench: graph replay {g_wall:.1f} us/step wall")
    attn_gbps = budget["attn"] / (attn_us * 1e-6) / 1e9
    result = {
        "metric": METRIC,
        "value": round(us_step, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "settle_steps": settled,
        "ms_per_step": round(us_step / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt == torch.bfloat16 else "f32",
        "data": "synthetic (seeded; Zipf(1.1) selector masses, N(0,1) KV cache)",
        "config": {"workload": wl.name, "batch": wl.B, "L": wl.L, "Hq": wl.Hq, "Hkv": wl.Hkv,
                   "head_dim": wl.d, "block": wl.block, "H_idx": wl.H_idx, "d_idx": wl.d_idx,
                   "selector_cache": wl.sel_k_dtype, "p": wl.p, "K_min": wl.K_min,
                   "K_max": wl.K_max, "n_sink": wl.n_sink, "n_rec": wl.n_rec,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "spot_sparse_attn call: attn_mfma (split-K runs) + attn_combine (merge)",
                     "achieved": round(attn_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(attn_gbps / HBM_PEAK_GBPS, 4), "traffic": profiled_traffic(),
                     "bytes_per_launch": budget["attn"], "avg_launch_us": round(attn_us, 3)},
        "step_hbm": {"algorithmic_bytes": budget["step"],
                     "GBps": round(budget["step"] / (us_step * 1e-6) / 1e9, 1),
                     "frac": round(budget["step"] / (us_step * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                     "selected_tokens": tokens},
        "queries_per_s": round(wl.B / (us_step * 1e-6), 1),
        "step_us_stats": step_stats,
        "timing": "value = wall time of K steps, captured once as HIP graphs (graphs."
                  "steps_per_graph steps each, as a server captures a token's launches) and "
                  "replayed on one stream, bracketed by device synchronisations, divided by "
                  "K, after settle_steps untimed steps, ~30 ms of untimed replays right before "
                  "(the GPU's clocks drop in idle gaps) and one untimed replay; "
                  "stream_launch_us_per_step = the same K steps launched from the host one "
                  "call at a time (three library calls each, arguments marshalled once, no "
                  "host synchronisation or events between them); events_us_per_step = a "
                  "stream-launched pass with a HIP event on each side; "
                  "step_us_stats.bursts = the graph measurement repeated, "
                  "stream_launch_bursts the stream-launched one; "
                  "step_us_stats.per_step_events = an event at every "
                  "step boundary (each event adds a gap of about 2 us); "
                  "roofline.avg_launch_us = HIP events on the same stream around K "
                  "back-to-back spot_sparse_attn calls, divided by K; per_call_us = a "
                  "separate pass with events between the calls (each event adds a gap)",
        "events_us_per_step": round(us_step_events, 3),
        "attn_call_wall_us": round(attn_wall, 3),
        "percall_pass_us_per_step": round(us_step_percall, 3),
        "per_call_us": {"mean": {k: round(v, 3) for k, v in mean.items()},
                        "median": {k: round(v, 3) for k, v in med.items()}},
        "gpu_event_us_per_step": round(gpu_total_us / n_diag, 3),
        "percall_pass_steps": n_diag,
        "graph_replay_us_per_step": {"wall": round(g_wall, 3), "events": round(g_event, 3),
                                     "note": "one step per HIP graph; each graph launch "
                                             "adds a gap before its first kernel"},
        "graphs": {"steps_per_graph": min(a.steps, GraphSteps.MAX_STEPS),
                   "output_matches_stream_launch": graphs_ok},
        "stream_launch_us_per_step": round(us_stream, 3),
        "flushed_step_us": quantiles(flushed) if flushed else None,
        "flushed_attn_call_us": flushed_attn,
        "flushed_graph_us_per_step": flushed_graph,
        "pages_context": "paper: 3.9x FlashAttention, 1.8x Twilight end-to-end decode tok/s "
                         "at 128K on one NVIDIA B200 (not comparable to this metric)",
    }
    log("bench: read-only reference kernel over the attention's bytes")
    rc = read_ceiling(budget["attn"], stream)
    rc["attn_frac_of_it"] = round(attn_gbps / rc["GBps"], 4)
    rc["step_frac_of_it"] = round(budget["step"] / (us_step * 1e-6) / 1e9 / rc["GBps"], 4)
    if flushed_attn:
        rcf = read_ceiling(budget["attn"], stream, reps=a.flushed_reps, flushed=True)
        rcf["attn_frac_of_it"] = round(
            budget["attn"] / (flushed_attn["median"] * 1e-6) / 1e9 / rcf["GBps"], 4)
        rc["flushed"] = rcf
    result["read_ceiling"] = rc
    result["launch_floor"] = launch_floor(stream)
    if a.extra_b1 and wl.name == "c3_128k_b8":
        wl1 = W.WORKLOADS["c3_128k_b1"]
        inp1 = {k: (v[:1].contiguous() if isinstance(v, torch.Tensor) else v)
                for k, v in inp.items()}
        bufs1 = DecodeBuffers.of(wl1, dt)
        step1 = DecodeStep(inp1, wl1, bufs1, stream=stream)
        gs1 = GraphSteps(step1, a.steps, stream, bufs1.out)
        settle(gs1, 0.03, stream, chunk=1)  # steady clocks first, as for the headline
        u1 = time_back_to_back(gs1, 1, 1, stream, events=False)[0] / a.steps
        u1s, _ = time_back_to_back(step1, a.steps, a.warmup, stream, events=False)
        w1, g1, p1 = time_steps(inp1, wl1, bufs1, a.steps, a.warmup, stream)
        st1 = {"bursts": quantiles([time_back_to_back(gs1, 1, 1, stream, events=False)[0]
                                    / a.steps for _ in range(reps)]),
               "stream_launch_bursts": burst_stats(step1, a.steps, stream),
               "per_step_events": time_step_distribution(step1, max(200, a.steps), a.warmup,
                                                         stream)}
        fl1 = time_flushed(inp1, wl1, bufs1, max(200, a.flushed_reps), stream)
        fa1 = quantiles(time_flushed_call(step1.calls[2], max(200, a.flushed_reps), stream))
        fg1 = time_flushed_graph(step1, stream)
        tok1 = selected_tokens(bufs1.sel_idx, bufs1.sel_cnt, wl1.L, wl1.block)
        b1 = byte_budget(wl1, 1, tok1)
        fl1q = quantiles(fl1)
        rc1 = read_ceiling(b1["attn"], stream, reps=max(200, a.flushed_reps), flushed=True)
        rc1["attn_frac_of_it"] = round(b1["attn"] / (fa1["median"] * 1e-6) / 1e9 / rc1["GBps"],
                                       4)
        result["batch1"] = {
            "us_per_step": round(u1, 3),
            "stream_launch_us_per_step": round(u1s, 3),
            "graphs_output_match": gs1.output_matches,
            "GBps": round(b1["step"] / (u1 * 1e-6) / 1e9, 1),
            "step_us_stats": st1,
            "flushed_step_us": fl1q,
            "flushed_hbm": {"algorithmic_bytes": b1["step"],
                            "GBps": round(b1["step"] / (fl1q["median"] * 1e-6) / 1e9, 1),
                            "frac": round(b1["step"] / (fl1q["median"] * 1e-6) / 1e9
                                          / HBM_PEAK_GBPS, 4)},
            "flushed_attn_call_us": fa1,
            "flushed_graph_us_per_step": fg1,
            "flushed_graph_hbm": {"GBps": round(b1["step"] / (fg1 * 1e-6) / 1e9, 1),
                                  "frac": round(b1["step"] / (fg1 * 1e-6) / 1e9
                                                / HBM_PEAK_GBPS, 4)},
            "read_ceiling_flushed": rc1,
            "queries_per_s": round(1 / (u1 * 1e-6), 1),
            "per_call_us_mean": {k: round(statistics.fmean(v), 3) for k, v in p1.items()},
            "note": "batch row 0 of the same inputs. us_per_step / GBps: K steps back to "
                    "back as HIP graphs (stream_launch_us_per_step: launched one call at a "
                    "time), so the 68 MB a step reads partly come from the 256 MB "
                    "last-level cache; flushed_step_us / flushed_hbm: a 1 GiB write between "
                    "steps (outside the events), the HBM figure; flushed_attn_call_us: the "
                    "attention call alone, the same way; flushed_graph_us_per_step: the same "
                    "write before every step with no event beside the steps (graphs of 20 "
                    "write + step pairs minus graphs of the 20 writes); read_ceiling_flushed: "
                    "the read-only kernel over the call's K/V bytes, the same way as "
                    "flushed_attn_call_us"}
        del inp1, bufs1, gs1
    if a.static and wl.name == "c3_128k_b8":
        log("bench: static top-K at half the context")
        result["static_topk_half"] = static_topk_leg(inp, wl, a.steps, a.warmup, stream)
    if a.int4 and wl.name == "c3_128k_b8":
        log("bench: INT4 selector cache workload")
        wl4 = W.WORKLOADS["c4_128k_b8_int4"]
        del inp
        torch.cuda.empty_cache()
        inp4 = W.make_inputs(wl4, device="cuda")
        bufs4 = DecodeBuffers.of(wl4, dt)
        step4 = DecodeStep(inp4, wl4, bufs4, stream=stream)
        u4, _ = time_back_to_back(step4, a.steps, a.warmup, stream, events=False)
        w4, _, p4 = time_steps(inp4, wl4, bufs4, a.steps, a.warmup, stream)
        # the headline's timing: K steps as HIP graphs after ~30 ms of untimed replays
        gs4 = GraphSteps(step4, a.steps, stream, bufs4.out)
        settle(gs4, 0.03, stream, chunk=1)
        g4 = time_back_to_back(gs4, 1, 1, stream, events=False)[0] / a.steps
        tok4 = selected_tokens(bufs4.sel_idx, bufs4.sel_cnt, wl4.L, wl4.block)
        b4 = byte_budget(wl4, wl4.B, tok4)
        result["int4_selector"] = {
            "workload": wl4.name, "us_per_step": round(g4, 3),
            "GBps": round(b4["step"] / (g4 * 1e-6) / 1e9, 1),
            "frac": round(b4["step"] / (g4 * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "stream_launch_us_per_step": round(u4, 3),
            "graphs_output_match": gs4.output_matches,
            "selected_blocks_mean": round(tok4 / wl4.block / wl4.B, 1),
            "algorithmic_bytes": b4["step"],
            "per_call_us_mean": {k: round(statistics.fmean(v), 3) for k, v in p4.items()},
            "score_GBps": round(b4["score"] / (statistics.fmean(p4["score"]) * 1e-6) / 1e9, 1)}
        del inp4, bufs4, step4, gs4
        torch.cuda.empty_cache()
        log("bench: budgets that vary across the batch")
        result["budgets_vary"] = budgets_vary_leg(wl, a.steps, a.warmup, stream)
        inp = W.make_inputs(wl, device="cuda") if not a.no_cpu_baseline else None
    if a.prefill:
        log("bench: prefill tile")
        result["prefill"] = prefill_leg(max(10, a.steps // 4), 5, stream)
        log("bench: whole-sequence sparse prefill")
        result["prefill_sequence"] = prefill_sequence_leg(max(5, a.steps // 50), 3, stream)
    if a.page_geometry:
        log("bench: selector at the paper's page geometry")
        result["page_geometry"] = page_geometry_step(max(10, a.steps // 4), 20, stream)
        log("bench: selector cache formats at the paper's page geometry")
        result["selector_formats"] = selector_formats_leg(max(10, a.steps // 4), 20, stream)
    result["calibration_copy_bytes"] = calibration_copy()
    if not a.no_cpu_baseline:
        log("bench: timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(wl, inp, b_sample=wl.B,
                                              b_single=max(1, wl.B // 4))
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
