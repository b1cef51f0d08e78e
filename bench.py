#!/usr/bin/env python3
"""Benchmark of the SFA hot path on one MI355X.

One step = one pass of the prefill hot path over the n=4 workload
(n=4, B=2, L=1024 -> nL=4096, 32 query / 8 KV heads, D=128, bf16):
    hd_expand (vocab 151936, hidden 4096)  ->  within-stream layer  ->  mixing layer.
``value`` is useful attention TFLOP/s of the step (4*D FLOPs per visible
(query, key) pair per query head; the expansion moves bytes, no FLOPs).

Also reported on the same JSON line:
  roofline      the prefill attention kernel against the bf16 MFMA peak,
                timed with HIP events on the stream it runs on;
  kernels       per-kernel times and rooflines (expansion and decode: HBM);
  decode        the decode step (64 sequences x 16384 cached entries, n=4,
                32/8 heads) in both modes: useful GB/s against HBM peak;
  stack         n=8, L=2048 stack (3 within + 1 mixing) vs the n=1 stack;
  cpu_baseline  the CPU oracle timed on a bounded sample of the same
                workload, on the host cores (a reported baseline only).

Inputs are resident in HBM before the timed region starts.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SFA attention useful TFLOP/s (prefill) and GB/s (decode), % of MI355X roofline"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


WINDOW = 1024                 # sliding window measured (positions; 256 tokens at n=4)
DECODE_WINDOW = 4096          # decode sliding window (positions; 1024 tokens at n=4)
DECODE_WARM_CALLS = 350


def pairs(n, L, mode, window=None):
    """Visible (query, key) pairs per (batch, head): n*L*(L+1)/2 within-stream,
    N*(N+1)/2 mixing (N = n*L); with a sliding window W < N, row i sees
    min(i+1, W) keys: W*(W+1)/2 + (N-W)*W."""
    N = n * L
    if mode == "within":
        return n * L * (L + 1) // 2
    if window is not None and window < N:
        return window * (window + 1) // 2 + (N - window) * window
    return N * (N + 1) // 2


def attn_flops(B, n, L, Hq, D, mode, window=None):
    return 4 * D * Hq * B * pairs(n, L, mode, window)


def decode_bytes(S, n, T, Hkv, D):
    """K+V bytes of the whole live cache (T+1 tokens x n streams) per call."""
    return S * (T + 1) * n * Hkv * D * 2 * 2


# the sources that make up each measured kernel (its file, the generated
# assembly it includes, the shared header), hashed in this order
KERNEL_SOURCES = {"prefill_source_sha256": ("prefill.hip", "prefill_asm.h", "common.h"),
                  "decode_source_sha256": ("decode.hip", "common.h")}


def kernel_source_sha256(key):
    """SHA-256 over the bytes of a kernel's source files (KERNEL_SOURCES)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[key]:
        with open(os.path.join(ROOT, "sequence_length_latent_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, src):
    """HBM bytes per launch of `kernel` (read + write, averaged over the
    within-stream and mixing launches) from the rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary in profiles/traffic.json -- only if that summary was
    taken on the current kernel source, else None."""
    try:
        t = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
        key = "prefill_source_sha256" if src == "prefill.hip" else "decode_source_sha256"
        if t.get(key) != kernel_source_sha256(key):
            return None
        per = t[kernel]
        return round(sum(v["read"] + v["write"] for v in per.values()) / len(per))
    except (OSError, KeyError, ValueError):
        return None


def _events(k):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(k)]


def bench_prefill(args, torch, hd, si):
    cfg = si.N4
    dev = torch.device("cuda")
    ids, tab = si.expand_inputs(cfg, device=dev)
    q, k, v = si.prefill_qkv(cfg, device=dev)
    x = torch.empty((cfg.B, cfg.N, cfg.hidden), dtype=torch.bfloat16, device=dev)
    ow = torch.empty_like(q)
    om = torch.empty_like(q)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev: ev[0].record()
        hd.expand(ids, tab, out=x)
        if ev: ev[1].record()
        hd.stream_attn(q, k, v, cfg.n, cfg.scale, out=ow)
        if ev: ev[2].record()
        hd.mix_attn(q, k, v, cfg.n, cfg.scale, out=om)
        if ev: ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # keep the GPU busy for ~0.5 s more so clocks have ramped before timing
    t_end = time.perf_counter() + 0.5
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()
    # whole-step timing: K steps back to back, no events inside
    t0, t1 = _events(2)
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    # per-kernel timing: events around each launch on the same stream
    evs = [_events(4) for _ in range(args.steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    t_exp = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    t_w = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    t_m = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    fw = attn_flops(cfg.B, cfg.n, cfg.L, cfg.Hq, cfg.D, "within")
    fm = attn_flops(cfg.B, cfg.n, cfg.L, cfg.Hq, cfg.D, "mix")
    exp_bytes = cfg.B * cfg.N * cfg.hidden * 2 * 2 + cfg.B * cfg.L * 4
    res = dict(cfg=cfg, ms_step=ms_step, t_exp=t_exp, t_w=t_w, t_m=t_m, fw=fw, fm=fm,
               exp_bytes=exp_bytes)
    if not args.only_step:
        res.update(bench_prefill_extras(args, torch, hd, si, cfg, ids, tab, q, k, v, x, ow, om))
    del ids, tab, q, k, v, x, ow, om
    torch.cuda.empty_cache()
    return res


def bench_prefill_extras(args, torch, hd, si, cfg, ids, tab, q, k, v, x, ow, om):
    """Kernels outside the step, on the step's n4 inputs: the sliding-window
    mixing layer, final-stream rows, cyclic replication and training."""
    dev = q.device
    # the sliding-window mixing layer (not part of the step): same inputs
    for _ in range(3):
        hd.mix_attn_window(q, k, v, cfg.n, cfg.scale, WINDOW, out=om)
    ew = _events(2)
    ew[0].record()
    for _ in range(args.steps):
        hd.mix_attn_window(q, k, v, cfg.n, cfg.scale, WINDOW, out=om)
    ew[1].record()
    torch.cuda.synchronize()
    t_mw = ew[0].elapsed_time(ew[1]) / args.steps
    # final-stream rows of the expanded hidden states (the LM head's input)
    fsr = torch.empty((cfg.B, cfg.L, cfg.hidden), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        hd.final_stream_rows(x, cfg.n, out=fsr)
    ew[0].record()
    for _ in range(args.steps):
        hd.final_stream_rows(x, cfg.n, out=fsr)
    ew[1].record()
    torch.cuda.synchronize()
    t_fs = ew[0].elapsed_time(ew[1]) / args.steps
    fs_bytes = 2 * cfg.B * cfg.L * cfg.hidden * 2
    # Cyclic Replication Initialization 2 -> 4 tables in place (after the step
    # timings: tables 2 and 3 become copies of 0 and 1)
    for _ in range(2):
        hd.cyclic_replicate(tab[:2], cfg.n, out=tab)
    ew[0].record()
    reps = max(1, args.steps // 4)
    for _ in range(reps):
        hd.cyclic_replicate(tab[:2], cfg.n, out=tab)
    ew[1].record()
    torch.cuda.synchronize()
    t_cr = ew[0].elapsed_time(ew[1]) / reps
    cr_bytes = 2 * (cfg.n - 2) * cfg.vocab * cfg.hidden * 2
    # training: forward with log-sum-exp, then the gradients, for both layers
    do = si.randn_bf16(q.shape, 1.0, 0x5FA0F00D, dev)
    bwd = {}
    for name, mode, win in (("within", hd.WITHIN, None), ("mix", hd.MIX, None),
                            ("mix_window", hd.MIX, WINDOW)):
        o_, lse = hd.attn_fwd(q, k, v, cfg.n, cfg.scale, mode, window=win)
        grads = hd.attn_bwd(q, k, v, do, lse, cfg.n, cfg.scale, mode, window=win)
        torch.cuda.synchronize()
        reps = max(2, args.steps // 4)
        ew[0].record()
        for _ in range(reps):
            hd.attn_fwd(q, k, v, cfg.n, cfg.scale, mode, out=o_, lse=lse, window=win)
        ew[1].record()
        torch.cuda.synchronize()
        t_f = ew[0].elapsed_time(ew[1]) / reps
        ew[0].record()
        for _ in range(reps):
            hd.attn_bwd(q, k, v, do, lse, cfg.n, cfg.scale, mode, *grads, window=win)
        ew[1].record()
        torch.cuda.synchronize()
        bwd[name] = (t_f, ew[0].elapsed_time(ew[1]) / reps)
        del o_, lse, grads

    fmw = attn_flops(cfg.B, cfg.n, cfg.L, cfg.Hq, cfg.D, "mix", WINDOW)
    del fsr, do
    return dict(t_mw=t_mw, fmw=fmw, t_fs=t_fs, fs_bytes=fs_bytes, t_cr=t_cr, cr_bytes=cr_bytes,
                bwd=bwd)


def _time_calls(torch, fn, reps, warm=2):
    """Mean ms of fn() over reps back-to-back calls (HIP events on the
    current stream, which is the one the library launches on)."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = _events(2)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def bench_long_prefill(args, torch, hd, si):
    """The long-context workload: n=4, B=1, L=8192 (nL=32768), 64/4 heads,
    D=128; the within-stream and mixing layers, each timed on its own."""
    cfg = si.LONG
    q, k, v = si.prefill_qkv(cfg, device=torch.device("cuda"))
    out = torch.empty_like(q)
    reps = max(2, args.steps // 4)
    res = {"workload": "long: n=4, batch 1, L=8192 tokens (nL=32768), 64 query / 4 KV heads "
                       "(GQA 16:1), head_dim 128, Q ~ N(0,1) log2(e)/sqrt(128), K, V ~ N(0,1); "
                       "scores in log2 units (scale ln 2)"}
    for name, fn in (("within", hd.stream_attn), ("mix", hd.mix_attn)):
        ms = _time_calls(torch, lambda: fn(q, k, v, cfg.n, cfg.scale, out=out), reps, warm=1)
        fl = attn_flops(cfg.B, cfg.n, cfg.L, cfg.Hq, cfg.D, name)
        tf = fl / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms, 4), "useful_gflop": round(fl / 1e9, 2), "achieved": round(tf, 2),
                     "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS, "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    del q, k, v, out
    torch.cuda.empty_cache()
    return res


def bench_scale_modes(args, torch, hd, si):
    """The n4 layers with the softmax scale carried other ways than the step's
    log2-unit scores: Q ~ N(0,1)/sqrt(128) with scale 1 (the scale folded into
    Q only) and unscaled Q ~ N(0,1) with scale 1/sqrt(128) passed to the call.
    Same FLOPs and precision; the kernel's exponent argument takes one more
    operand (a literal log2(e), or the scale from the arguments)."""
    import math
    cfg = si.N4
    dev = torch.device("cuda")
    reps = max(3, args.steps // 2)
    res = {}
    for name, q_std, scale in (("unit_scale", 1 / math.sqrt(cfg.D), 1.0),
                               ("any_scale", 1.0, 1 / math.sqrt(cfg.D))):
        q, k, v = si.prefill_qkv(cfg, device=dev, q_std=q_std)
        out = torch.empty_like(q)
        entry = {"q_std": round(q_std, 6), "softmax_scale": round(scale, 6)}
        for mode, fn in (("within", hd.stream_attn), ("mix", hd.mix_attn)):
            ms = _time_calls(torch, lambda: fn(q, k, v, cfg.n, scale, out=out), reps)
            fl = attn_flops(cfg.B, cfg.n, cfg.L, cfg.Hq, cfg.D, mode)
            tf = fl / (ms * 1e-3) / 1e12
            entry[mode] = {"ms": round(ms, 4), "achieved": round(tf, 2), "unit": "TFLOP/s",
                           "peak": PEAK_BF16_TFLOPS, "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        res[name] = entry
        del q, k, v, out
    torch.cuda.empty_cache()
    return res


def bench_decode(args, torch, hd, si):
    cfg = si.DECODE
    dev = torch.device("cuda")
    qn, kn, vn, kc, vc, tb = si.decode_inputs(cfg, device=dev)
    ws = torch.empty(hd.decode_workspace_size(cfg.S, cfg.n, cfg.Hq, cfg.Hkv, cfg.D, cfg.T),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(qn)
    reps = max(3, args.steps // 2)
    res = {}
    for mode, name in ((0, "within"), (1, "mix")):
        # ~0.3 s of calls first (the clock settles under load); a fixed count
        # keeps the dispatch sequence the same from run to run
        for _ in range(DECODE_WARM_CALLS):
            hd.decode_step(qn, kn, vn, kc, vc, tb, cfg.n, cfg.T, mode, cfg.scale, ws, out)
        torch.cuda.synchronize()
        e0, e1 = _events(2)
        e0.record()
        for _ in range(reps):
            hd.decode_step(qn, kn, vn, kc, vc, tb, cfg.n, cfg.T, mode, cfg.scale, ws, out)
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / reps
    # sliding-window mixing decode: the last DECODE_WINDOW + n - 1 entries of each sequence
    for _ in range(3):
        hd.decode_step(qn, kn, vn, kc, vc, tb, cfg.n, cfg.T, 1, cfg.scale, ws, out,
                       window=DECODE_WINDOW)
    e0, e1 = _events(2)
    e0.record()
    for _ in range(reps):
        hd.decode_step(qn, kn, vn, kc, vc, tb, cfg.n, cfg.T, 1, cfg.scale, ws, out,
                       window=DECODE_WINDOW)
    e1.record()
    torch.cuda.synchronize()
    res["mix_window"] = e0.elapsed_time(e1) / reps
    res["bytes_window"] = cfg.S * (DECODE_WINDOW + cfg.n - 1) * cfg.Hkv * cfg.D * 2 * 2
    res["bytes"] = decode_bytes(cfg.S, cfg.n, cfg.T, cfg.Hkv, cfg.D)
    res["cfg"] = cfg
    del qn, kn, vn, kc, vc, tb, ws, out
    torch.cuda.empty_cache()
    # long context: one layer over 32 sequences x 32768 tokens x 4 streams
    lc = si.DECODE_LONG
    qn, kn, vn, kc, vc, tb = si.decode_inputs(lc, device=dev)
    ws = torch.empty(hd.decode_workspace_size(lc.S, lc.n, lc.Hq, lc.Hkv, lc.D, lc.T),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(qn)
    lreps = max(2, args.steps // 4)
    for mode, name in ((0, "long_within"), (1, "long_mix")):
        for _ in range(2):
            hd.decode_step(qn, kn, vn, kc, vc, tb, lc.n, lc.T, mode, lc.scale, ws, out)
        e0.record()
        for _ in range(lreps):
            hd.decode_step(qn, kn, vn, kc, vc, tb, lc.n, lc.T, mode, lc.scale, ws, out)
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / lreps
    res["bytes_long"] = decode_bytes(lc.S, lc.n, lc.T, lc.Hkv, lc.D)
    del qn, kn, vn, kc, vc, tb, ws, out
    torch.cuda.empty_cache()
    return res


def bench_decode_stack(args, torch, hd, si):
    """One decode step of every attention layer of the pages' 80B and 617B
    schedules (paged caches, 32 sequences x 2048 tokens x 4 streams)."""
    from sequence_length_latent_amd import schedule as sch
    S, n, Hq, Hkv, D, P, T, W = 32, 4, 32, 8, 128, 64, 2048, DECODE_WINDOW
    dev = torch.device("cuda")
    mp = -(-((T + 1) * n) // P)
    res = {}
    for name in ("80B", "617B"):
        kinds = sch.layer_kinds(name)
        st = sch.PagedDecodeStack(kinds, S, n, Hq, Hkv, D, P, mp, W, device=dev)
        for pool in st.k_pools + st.v_pools:
            pool.normal_()
        qs = [torch.randn((S, n, Hq, D), device=dev).to(torch.bfloat16) for _ in kinds]
        ks = [torch.randn((S, n, Hkv, D), device=dev).to(torch.bfloat16) for _ in kinds]
        vs = [torch.randn((S, n, Hkv, D), device=dev).to(torch.bfloat16) for _ in kinds]
        outs = [torch.empty_like(q) for q in qs]
        tb = torch.full((S,), T, dtype=torch.int32, device=dev)
        ws = st.workspace(T)
        st.step(qs, ks, vs, tb, T, D ** -0.5, outs, ws)
        torch.cuda.synchronize()
        reps = 3
        e0, e1 = _events(2)
        e0.record()
        for _ in range(reps):
            st.step(qs, ks, vs, tb, T, D ** -0.5, outs, ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        # the same step recorded as one HIP graph and replayed
        graph = st.capture(qs, ks, vs, tb, T, D ** -0.5, outs, ws)
        graph.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ms_graph = e0.elapsed_time(e1) / reps
        del graph
        entry = Hkv * D * 2 * 2
        nbytes = sum(S * ((W + n - 1) if k == sch.SLIDING else (T + 1) * n) * entry for k in kinds)
        res[name] = {"layers": len(kinds), "counts": sch.SCHEDULES[name], "ms_per_step": round(ms, 3),
                     "bytes_per_step": nbytes, "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "unit": "GB/s", "peak": PEAK_HBM_GBS,
                     "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "tokens_per_s": round(S / (ms * 1e-3), 1),
                     "ms_per_step_graph": round(ms_graph, 3)}
        del st, qs, ks, vs, outs, ws
        torch.cuda.empty_cache()
    res["workload"] = (f"{S} sequences x {T} tokens x {n} streams cached, {Hq}/{Hkv} heads, head_dim {D}, "
                       f"pages of {P} entries, sliding window {W} positions; one decode step of every "
                       "attention layer (append + attention + combine per layer); tokens_per_s counts one "
                       "token per sequence per step, attention only; ms_per_step_graph: the same step "
                       "replayed as one captured HIP graph")
    return res


def bench_stack(args, torch, hd, si):
    """n=8, L=2048 stack of 3 within + 1 mixing layers vs the n=1 stack
    (4 causal layers at L=2048, same heads)."""
    cfg = si.N8STACK
    dev = torch.device("cuda")
    layers = [si.prefill_qkv(cfg, layer=i, device=dev) for i in range(4)]
    base = [si.prefill_qkv(cfg, layer=i, device=dev, B=1, L=cfg.L // 1) for i in range(4)]
    base = [(q[:, :cfg.L].contiguous(), k[:, :cfg.L].contiguous(), v[:, :cfg.L].contiguous())
            for q, k, v in base]
    out = torch.empty_like(layers[0][0])
    out1 = torch.empty_like(base[0][0])
    reps = max(2, args.steps // 4)

    def run_hd():
        for i, (q, k, v) in enumerate(layers):
            fn = hd.mix_attn if cfg.layers[i] == "mix" else hd.stream_attn
            fn(q, k, v, cfg.n, cfg.scale, out=out)

    def run_base():
        for q, k, v in base:
            hd.mix_attn(q, k, v, 1, cfg.scale, out=out1)

    # the n = 1 layer has as many work items as compute units: the key-split
    # launch takes each item's key tiles in two halves on different workgroups
    ws1 = hd.split_workspace(base[0][0], base[0][1], 1, hd.MIX)

    def run_base_split():
        for q, k, v in base:
            hd.attn_split(q, k, v, 1, cfg.scale, hd.MIX, ws1, out=out1)

    def timeit(fn):
        t_end = time.perf_counter() + 0.2
        while time.perf_counter() < t_end:
            fn()
            torch.cuda.synchronize()
        e0, e1 = _events(2)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    t_hd = timeit(run_hd)
    t_base = timeit(run_base)
    t_base_split = timeit(run_base_split)
    q, k, v = layers[0]
    t_w = timeit(lambda: hd.stream_attn(q, k, v, cfg.n, cfg.scale, out=out))
    t_m = timeit(lambda: hd.mix_attn(q, k, v, cfg.n, cfg.scale, out=out))
    fl_hd = 3 * attn_flops(1, cfg.n, cfg.L, cfg.Hq, cfg.D, "within") + \
        attn_flops(1, cfg.n, cfg.L, cfg.Hq, cfg.D, "mix")
    fl_base = 4 * attn_flops(1, 1, cfg.L, cfg.Hq, cfg.D, "mix")
    del layers, base, out, out1, ws1
    torch.cuda.empty_cache()
    return {
        "workload": "n=8 B=1 L=2048 (nL=16384) Hq=32 Hkv=8 D=128; 3 within + 1 mixing layer "
                    "vs n=1 stack of 4 causal layers at L=2048",
        "ms_stack": round(t_hd, 4), "ms_stack_n1": round(t_base, 4),
        "time_ratio_vs_n1": round(t_hd / t_base, 3), "flop_ratio_vs_n1": round(fl_hd / fl_base, 3),
        "ms_stack_n1_key_split": round(t_base_split, 4),
        "time_ratio_vs_n1_key_split": round(t_hd / t_base_split, 3),
        "ms_within": round(t_w, 4), "ms_mix": round(t_m, 4),
        "mix_over_within_time": round(t_m / t_w, 3),
        "mix_over_within_flops": round(attn_flops(1, cfg.n, cfg.L, cfg.Hq, cfg.D, "mix") /
                                       attn_flops(1, cfg.n, cfg.L, cfg.Hq, cfg.D, "within"), 3),
        "stack_tflops": round(fl_hd / (t_hd * 1e-3) / 1e12, 2),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        return os.cpu_count()


def _oracle_prefill_sample(si, oracle, cfg, layer_modes, budget_s, block=64, heads=None):
    """Oracle on the last query rows of batch 0 (the most expensive ones),
    every head (or the given ones), every layer in layer_modes [(layer,
    mode)], growing the sample until budget_s seconds have been spent.
    Returns (useful FLOPs, wall s, CPU s, rows)."""
    import numpy as np
    bits = {}
    for layer, _ in layer_modes:
        if layer not in bits:
            q, k, v = si.prefill_qkv(cfg, layer=layer, B=1)
            bits[layer] = (si.bits(q), si.bits(k), si.bits(v))
            del q, k, v
    N = cfg.N
    flops = 0
    rows_done = 0
    c0, t0 = time.process_time(), time.perf_counter()
    while time.perf_counter() - t0 < budget_s and rows_done < N:
        hi = N - rows_done
        rows = np.arange(hi - block, hi)
        for layer, mode in layer_modes:
            qb, kb, vb = bits[layer]
            oracle.prefill_ref(qb, kb, vb, cfg.n, mode, cfg.scale, rows=rows, heads=heads)
            keys = (rows // cfg.n + 1) if mode == oracle.WITHIN else (rows + 1)
            flops += 4 * cfg.D * (cfg.Hq if heads is None else len(heads)) * int(keys.sum())
        rows_done += block
    return flops, time.perf_counter() - t0, time.process_time() - c0, rows_done


def cpu_baseline(si, budget_s):
    """The float64 oracle as it stands, timed on the host cores.  The reported
    value is a bounded sample of the n4 workload (the last query rows of
    batch 0, all 32 heads, both layers, grown until ``budget_s`` seconds of
    work).  ``per_config`` times every workload the same way: the tiny one in
    full (with all BLAS threads and with one), the others on bounded samples
    whose useful rate gives an estimate of the full workload's oracle time."""
    import oracle
    from threadpoolctl import threadpool_limits
    W, M = oracle.WITHIN, oracle.MIX
    threads = _blas_threads()
    per = {}

    # tiny: the whole workload (both layers), all threads and a single thread
    cfg = si.TINY
    q, k, v = si.prefill_qkv(cfg)
    qb, kb, vb = si.bits(q), si.bits(k), si.bits(v)
    fl = sum(4 * cfg.D * cfg.Hq * cfg.B * oracle.count_pairs(cfg.N, cfg.n, m) for m in (W, M))
    for key, lim in (("all_threads", None), ("single_thread", 1)):
        with threadpool_limits(lim):
            t0 = time.perf_counter()
            for m in (W, M):
                oracle.prefill_ref(qb, kb, vb, cfg.n, m, cfg.scale)
            dt = time.perf_counter() - t0
        per.setdefault("tiny", {"sample": "whole workload, both layers", "useful_gflop": round(fl / 1e9, 6)})
        per["tiny"][key] = {"s": round(dt, 4), "gflop_per_s": round(fl / dt / 1e9, 3),
                            "threads": threads if lim is None else 1}

    # n4 (the reported value)
    cfg = si.N4
    flops, dt, cpu_s, rows = _oracle_prefill_sample(si, oracle, cfg, [(0, W), (0, M)], budget_s)
    full = sum(4 * cfg.D * cfg.Hq * cfg.B * oracle.count_pairs(cfg.N, cfg.n, m) for m in (W, M))
    rate = flops / dt
    per["n4"] = {"sample": f"batch 0, all heads, last {rows} of {cfg.N} query rows, both layers",
                 "s": round(dt, 2), "gflop_per_s": round(rate / 1e9, 3),
                 "est_full_workload_s": round(full / rate, 1)}
    value = rate / 1e12
    main = {"dt": dt, "cpu_s": cpu_s, "rows": rows, "flops": flops}

    # n8 stack and long context: bounded samples
    side = max(2.0, budget_s / 4)
    for name, cfg, lm, hs in (("n8stack", si.N8STACK, [(0, W), (3, M)], None),
                              ("long", si.LONG, [(0, W), (0, M)], list(range(0, 64, 8)))):
        flops, dt, _, rows = _oracle_prefill_sample(si, oracle, cfg, lm, side, block=32, heads=hs)
        if name == "n8stack":
            full = (3 * 4 * cfg.D * cfg.Hq * cfg.B * cfg.n * cfg.L * (cfg.L + 1) // 2 +
                    4 * cfg.D * cfg.Hq * cfg.B * cfg.N * (cfg.N + 1) // 2)
        else:
            full = (4 * cfg.D * cfg.Hq * cfg.B * (cfg.n * cfg.L * (cfg.L + 1) // 2 + cfg.N * (cfg.N + 1) // 2))
        rate = flops / dt
        per[name] = {"sample": f"batch 0, {'all heads' if hs is None else f'heads {hs}'}, last {rows} "
                               f"of {cfg.N} query rows, layers {[l for l, _ in lm]}",
                     "s": round(dt, 2), "gflop_per_s": round(rate / 1e9, 3),
                     "est_full_workload_s": round(full / rate, 1)}

    # decode: a few sequences of the decode workload's shape, both modes
    dc = si.DECODE
    S = 2
    qn, kn, vn, kc, vc, tb = si.decode_inputs(dc, S=S)
    t0 = time.perf_counter()
    k2, v2 = oracle.decode_append_ref(si.bits(kc), si.bits(vc), si.bits(kn), si.bits(vn), tb.numpy(), dc.n)
    nbytes = 0
    for m in (W, M):
        oracle.decode_ref(si.bits(qn), k2, v2, tb.numpy(), dc.n, m, dc.scale)
        nbytes += S * (dc.T + 1) * dc.n * dc.Hkv * dc.D * 2 * 2
    dt = time.perf_counter() - t0
    full_bytes = 2 * dc.S * (dc.T + 1) * dc.n * dc.Hkv * dc.D * 2 * 2
    per["decode"] = {"sample": f"{S} sequences of 4096 tokens x 4 streams, append + both modes",
                     "s": round(dt, 2), "gb_per_s": round(nbytes / dt / 1e9, 3),
                     "est_full_workload_s": round(full_bytes / (nbytes / dt), 1)}
    del qn, kn, vn, kc, vc, k2, v2

    return {
        "value": round(value, 6), "unit": "TFLOP/s", "cores": threads,
        "kind": "oracle",
        "sample": f"n4 workload, batch 0, all 32 heads, last {main['rows']} query rows of the "
                  f"4096 (within-stream and mixing layers), float64 NumPy oracle, "
                  f"{main['dt']:.1f} s wall, {main['flops'] / 1e9:.2f} useful GFLOP",
        "cores_note": "cores = threads of the BLAS pool the oracle's products ran on; "
                      "effective_cores = process CPU seconds / wall seconds of the n4 sample",
        "effective_cores": round(main["cpu_s"] / main["dt"], 2),
        "cpu_model": _cpu_model(),
        "os_cpu_count": os.cpu_count(),
        "per_config": per,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of CPU oracle work for cpu_baseline (0 to skip)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--only-step", action="store_true",
                    help="time the step, the long-context layers and the scale modes only "
                         "(for counter profiles)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run one plain device copy (negation) of MIB MiB, the "
                         "reference kernel for scaling HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs the SFA hot path on a single "
              "MI355X (no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import sequence_length_latent_amd as hd
    import sfa_inputs as si
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    hd.load()

    if args.copy_calibration > 0:
        nel = args.copy_calibration * (1 << 20) // 2
        src = torch.ones(nel, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: {nel * 2} bytes read, {nel * 2} bytes written",
              file=sys.stderr, flush=True)
        del src, dst

    pf = bench_prefill(args, torch, hd, si)
    print(f"[bench] prefill done: step {pf['ms_step']:.4f} ms", file=sys.stderr, flush=True)
    longp = bench_long_prefill(args, torch, hd, si)
    print(f"[bench] long prefill done: within {longp['within']['ms']:.3f} ms mix {longp['mix']['ms']:.3f} ms",
          file=sys.stderr, flush=True)
    modes = bench_scale_modes(args, torch, hd, si)
    print("[bench] scale modes done", file=sys.stderr, flush=True)
    if args.only_step:
        args.no_decode = args.no_stack = True
        args.cpu_budget = 0
    dec = None if args.no_decode else bench_decode(args, torch, hd, si)
    if dec:
        print(f"[bench] decode done: within {dec['within']:.4f} ms mix {dec['mix']:.4f} ms",
              file=sys.stderr, flush=True)
    dstack = None if args.no_decode else bench_decode_stack(args, torch, hd, si)
    if dstack:
        print("[bench] decode stack done", file=sys.stderr, flush=True)
    stack = None if args.no_stack else bench_stack(args, torch, hd, si)
    if stack:
        print("[bench] stack done", file=sys.stderr, flush=True)
    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(si, args.cpu_budget)
        print("[bench] cpu baseline done", file=sys.stderr, flush=True)

    cfg = pf["cfg"]
    flops = pf["fw"] + pf["fm"]
    value = flops / (pf["ms_step"] * 1e-3) / 1e12
    attn_ms = pf["t_w"] + pf["t_m"]
    ach = flops / (attn_ms * 1e-3) / 1e12
    kernels = {
        "hd_expand": {"ms": round(pf["t_exp"], 4), "bound": "hbm",
                      "achieved": round(pf["exp_bytes"] / (pf["t_exp"] * 1e-3) / 1e9, 1),
                      "unit": "GB/s", "peak": PEAK_HBM_GBS},
        "sfa_stream_attn": {"ms": round(pf["t_w"], 4), "bound": "mfma",
                            "achieved": round(pf["fw"] / (pf["t_w"] * 1e-3) / 1e12, 2),
                            "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS},
        "sfa_mix_attn": {"ms": round(pf["t_m"], 4), "bound": "mfma",
                         "achieved": round(pf["fm"] / (pf["t_m"] * 1e-3) / 1e12, 2),
                         "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS},
    }
    if "t_mw" in pf:
        kernels.update({
            "sfa_mix_attn_window": {"ms": round(pf["t_mw"], 4), "bound": "mfma",
                                    "achieved": round(pf["fmw"] / (pf["t_mw"] * 1e-3) / 1e12, 2),
                                    "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS,
                                    "window": WINDOW, "useful_gflop": round(pf["fmw"] / 1e9, 3),
                                    "note": "sliding-window mixing layer, same n4 inputs; "
                                            "not part of the step"},
            "hd_final_stream_rows": {"ms": round(pf["t_fs"], 4), "bound": "hbm",
                                     "achieved": round(pf["fs_bytes"] / (pf["t_fs"] * 1e-3) / 1e9, 1),
                                     "unit": "GB/s", "peak": PEAK_HBM_GBS,
                                     "note": "[2, 4096, 4096] -> [2, 1024, 4096]; not part of the step"},
            **{f"sfa_attn_bwd_{name}": {
                "ms": round(pf["bwd"][name][1], 4), "bound": "mfma",
                "achieved": round(2.5 * pf[fk] / (pf["bwd"][name][1] * 1e-3) / 1e12, 2),
                "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS,
                "fwd_with_lse_ms": round(pf["bwd"][name][0], 4),
                "note": "gradients dq, dk, dv of the n4 layer" + (f" (sliding window {WINDOW})"
                                                                    if name == "mix_window" else "")
                        + "; useful work counted as 2.5x the forward's (five products per visible "
                          "pair); not part of the step"}
               for name, fk in (("within", "fw"), ("mix", "fm"), ("mix_window", "fmw"))},
            "hd_cyclic_replicate": {"ms": round(pf["t_cr"], 4), "bound": "hbm",
                                    "achieved": round(pf["cr_bytes"] / (pf["t_cr"] * 1e-3) / 1e9, 1),
                                    "unit": "GB/s", "peak": PEAK_HBM_GBS,
                                    "note": "2 -> 4 tables of 151936 x 4096 in place (2.49 GB read + "
                                            "written); not part of the step"},
        })
    for kk in kernels.values():
        kk["frac"] = round(kk["achieved"] / kk["peak"], 4)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pf["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "n4: n=4 streams, batch 2, L=1024 tokens (nL=4096), 32 query / 8 KV "
                        "heads, head_dim 128; step = hd_expand (vocab 151936, hidden 4096) + "
                        "within-stream layer + mixing layer",
            "n": cfg.n, "batch": cfg.B, "L": cfg.L, "nL": cfg.N, "Hq": cfg.Hq, "Hkv": cfg.Hkv,
            "head_dim": cfg.D, "useful_gflop_per_step": round(flops / 1e9, 3),
        },
        "roofline": {
            "kernel": "sfa_prefill_kernel<128, 2> (log2-unit scores; both layers, 2 launches per step)",
            "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("sfa_prefill_kernel_n4", "prefill.hip"),
            "traffic_unit": "bytes per launch (HBM read + write)",
            "algorithmic_flop_per_launch": round(flops / 2),
        },
        "kernels": kernels,
    }
    line["prefill_long"] = longp
    line["scale_modes"] = modes
    if dec:
        line["decode"] = {
            "workload": "64 sequences x 4096 tokens x 4 streams cached (16388 live entries after "
                        "the append), 32/8 heads, head_dim 128; one decode step = append + "
                        "attention + split combine",
            "bytes_per_call": dec["bytes"],
        }
        for name in ("within", "mix"):
            gbs = dec["bytes"] / (dec[name] * 1e-3) / 1e9
            line["decode"][name] = {"ms": round(dec[name], 4), "achieved": round(gbs, 1),
                                    "unit": "GB/s", "peak": PEAK_HBM_GBS,
                                    "frac": round(gbs / PEAK_HBM_GBS, 4)}
        gbs = dec["bytes_window"] / (dec["mix_window"] * 1e-3) / 1e9
        line["decode"]["mix_window"] = {
            "ms": round(dec["mix_window"], 4), "achieved": round(gbs, 1), "unit": "GB/s",
            "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4), "window": DECODE_WINDOW,
            "bytes_per_call": dec["bytes_window"],
            "note": "sliding-window mixing decode: K+V of the last window + n - 1 entries per "
                    "sequence; not part of the step"}
        line["decode"]["long_context"] = {
            "workload": "one layer over 32 sequences x 32768 tokens x 4 streams cached (131076 live "
                        "entries after the append, 17.2 GB of K+V), 32/8 heads, head_dim 128",
            "bytes_per_call": dec["bytes_long"]}
        for name, key in (("within", "long_within"), ("mix", "long_mix")):
            gbs = dec["bytes_long"] / (dec[key] * 1e-3) / 1e9
            line["decode"]["long_context"][name] = {"ms": round(dec[key], 4), "achieved": round(gbs, 1),
                                                    "unit": "GB/s", "peak": PEAK_HBM_GBS,
                                                    "frac": round(gbs / PEAK_HBM_GBS, 4)}
        line["decode"]["traffic"] = measured_traffic("decode_attend_kernel", "decode.hip")
    if stack:
        line["stack"] = stack
    if dstack:
        line["decode_stack"] = dstack
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
