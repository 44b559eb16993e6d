"""Benchmark of the SSE hot path on one MI355X.

One step = one sse_forward over the main workload (bf16, B=4, H=16, T=8192,
c=d=128, N=16, k=2, router std 1.5): routing + counts, grouping, chunked
GLA over all partition segments with the combine into o.  ``value`` is that
forward's throughput in tokens/s (B*T tokens per step, all heads), with the
inputs already resident in HBM, timed over --steps calls after 0.3 s of
untimed forwards and --warmup warm-up calls (the first forwards on an idle
GPU run slower); "step_ms" gives median, min and max of further forwards
timed one by one.  The decode step (256 sequences x H=16, c=d=128, N=16,
k=2, 64 consecutive steps), the varlen forward, the masking schedule, the
backward and the row-sparse variant are timed in the same run; --fig6 adds
the operator-timing sweep of the page's Fig. 6 (forward of both schedules,
forward + backward of the varlen schedule).

roofline: the dominant kernel is the chunked GLA pass with the longest
time (the routed pass); its duration comes from HIP events recorded around it
on the library's stream (sse_trace_*) in a second run of the same number of
steps, after the timed steps (which run without events).  Its
algorithmic bytes per launch are what the pass itself must move: the routed
pass reads every token's q, key logits, log decay and v rows once and writes
the routed partitions' final states (its e-gated reads go to workspace
slots, an implementation cost, not counted); the shared pass reads the same
rows, writes o and the shared final states.  "traffic" is the HBM bytes the
committed FETCH_SIZE/WRITE_SIZE counter runs measured for it (null if the
kernel source changed since).  forward_roofline gives the whole forward's
fraction (all launches, algorithmic bytes of the layer).

cpu_baseline: the fp64 oracle (untuned) on the whole main workload (all 64
(sequence, head) units), threads over units on the host cores; plus the
single-thread rate on the small bf16 workload (per-core figure).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSE fwd tokens/s (T=8K,c=d=128,N=16,k=2) + decode tok/s; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MFMA_F32_PEAK_TFLOPS = 157.3    # MI355X dense fp32 MFMA
NAMES = ("q", "key_logits", "v", "log_alpha", "router_logits")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(a).to("cuda")


def forward_bytes(T, S, H, c, d, N, in_bytes=2):
    """Algorithmic HBM bytes of one forward: token inputs read once (q, key
    logits, log_alpha, v, router logits), o written once (fp32), final
    states written once (fp32)."""
    inputs = T * H * in_bytes * (3 * c + d + N)
    return inputs + T * H * 4 * d + S * H * (N + 1) * c * d * 4


def pass_bytes(T, S, H, c, d, parts, writes_o, in_bytes=2):
    """Algorithmic bytes of one chunked-GLA pass over `parts` partitions of
    every (sequence, head): each token's q, key logits, log_alpha and v read
    once, the pass's final states written once, and o written once if the
    pass writes it (the shared pass does; the routed pass does not)."""
    return (T * H * in_bytes * (3 * c + d) + (T * H * 4 * d if writes_o else 0)
            + S * H * parts * c * d * 4)


def chunk_flops(records, c, d, C=64):
    """Algorithmic flops of the chunked form: 2 (C c/2 + C d/2 + 2 c d) per record."""
    return records * 2 * (C * c / 2 + C * d / 2 + 2 * c * d)


def run_forward(args, w, si, sse, torch, inp=None, schedule=None, step_stats=None, prewarm_s=0.0):
    """Time sse_forward (or sse_forward_ex with the given schedule) on w.
    With prewarm_s > 0, forwards run untimed for that long before the
    warm-up steps: on a GPU that has been idle the first forwards run about
    10 % slower (3 warm-up forwards: 0.87 ms per timed step on the main
    workload; 30: 0.78), so the timed window would otherwise measure the
    clock ramp rather than the steady state.
    With a dict `step_stats`, also time `args.steps` more calls one by one
    (an event pair around each, after the timed window) and put their
    median, min and max in it."""
    if inp is None:
        inp = si.forward_inputs(w)
    cu = inp["cu_seqlens"]
    T = int(cu[-1])
    S = len(cu) - 1
    max_len = int((cu[1:] - cu[:-1]).max())
    d_in = {n: to_dev(inp[n]) for n in NAMES + ("cu_seqlens",)}
    del inp
    o = torch.empty((T, w.H, w.d), dtype=torch.float32, device="cuda")
    fs = torch.empty((S, w.H, w.N + 1, w.c, w.d), dtype=torch.float32, device="cuda")
    ws = torch.empty(sse.sse_forward_workspace_bytes(T, S, max_len, w.H, w.c, w.d, w.N, w.topk),
                     dtype=torch.uint8, device="cuda")

    def step():
        if schedule is None:
            sse.sse_forward(*(d_in[n] for n in NAMES), w.N, w.topk, d_in["cu_seqlens"], max_len,
                            o=o, final_states=fs, workspace=ws)
        else:
            sse.sse_forward_ex(*(d_in[n] for n in NAMES), w.N, w.topk, d_in["cu_seqlens"],
                               max_len, schedule=schedule, o=o, final_states=fs, workspace=ws)

    if prewarm_s > 0:
        t_end = time.perf_counter() + prewarm_s
        while time.perf_counter() < t_end:
            for _ in range(4):
                step()
            torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed steps run without stage events (each event in the stream
    # costs time of its own); a second, traced run gives the stage split
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    sse.sse_trace_enable(True)
    for _ in range(args.steps):
        step()
    stages, calls = sse.sse_trace_read()
    sse.sse_trace_enable(False)
    if step_stats is not None:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for a, b in ev:
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        per = sorted(a.elapsed_time(b) for a, b in ev)
        step_stats.update({"median": per[len(per) // 2], "min": per[0], "max": per[-1],
                           "calls": len(per)})
    return T, S, total_ms, {k: v / max(calls, 1) for k, v in stages.items()}, calls


def fwd_bwd_ms(w, si, sse, torch, inp, steps=10, warmup=2):
    """ms of one sse_forward followed by one sse_backward of <d_o, o> (all
    input gradients, no initial states) on the inputs `inp`."""
    cu = inp["cu_seqlens"]
    T, S = int(cu[-1]), len(cu) - 1
    max_len = int((cu[1:] - cu[:-1]).max())
    d_in = {n: to_dev(inp[n]) for n in NAMES + ("cu_seqlens",)}
    o = torch.empty((T, w.H, w.d), dtype=torch.float32, device="cuda")
    fs = torch.empty((S, w.H, w.N + 1, w.c, w.d), dtype=torch.float32, device="cuda")
    wsf = torch.empty(sse.sse_forward_workspace_bytes(T, S, max_len, w.H, w.c, w.d, w.N, w.topk),
                      dtype=torch.uint8, device="cuda")
    do = torch.randn((T, w.H, w.d), dtype=torch.float32, device="cuda")
    out = {nm: torch.empty(shp, dtype=torch.float32, device="cuda") for nm, shp in (
        ("dq", (T, w.H, w.c)), ("dkey_logits", (T, w.H, w.c)), ("dlog_alpha", (T, w.H, w.c)),
        ("dv", (T, w.H, w.d)), ("drouter_logits", (T, w.H, w.N)))}
    wsb = torch.empty(sse.sse_backward_workspace_bytes(T, S, max_len, w.H, w.c, w.d, w.N, w.topk),
                      dtype=torch.uint8, device="cuda")

    def step():
        sse.sse_forward(*(d_in[n] for n in NAMES), w.N, w.topk, d_in["cu_seqlens"], max_len,
                        o=o, final_states=fs, workspace=wsf)
        sse.sse_backward(*(d_in[n] for n in NAMES), w.N, w.topk, d_in["cu_seqlens"], do,
                         max_len, workspace=wsb, out=out)

    return timed(torch, step, steps, warmup)


def fig6_sweep(args, si, sse, torch):
    """Forward time of the varlen path in the operator-timing setting of
    "Scaling Linear Attention with Sparse State Expansion: 中文研读笔记"
    (§2.6, Fig. 6): 8 heads, head dim 128, one routed partition per token,
    two sequences of L/2 tokens, N = 4, 8, 16; bf16 inputs here.  That figure
    times forward plus backward on another GPU and gives no values in the
    text.  Both schedules' forwards are timed, and the varlen schedule's
    forward plus backward (the masked schedule has no backward here), to see
    how the time moves with N at fixed k."""
    from types import SimpleNamespace
    ns = SimpleNamespace(warmup=2, steps=10)
    rows = []
    for L in (256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 65536):
        # one draw per L; the router logits of N partitions are the first N
        # columns of the N = 16 draw (still N(0, 1) and free of ties)
        base = si.forward_inputs(si.Workload(f"fig6_L{L}", "bf16", H=8, c=128, d=128, N=16,
                                             topk=1, B=2, T=L // 2))
        for N in (4, 8, 16):
            w = si.Workload(f"fig6_N{N}_L{L}", "bf16", H=8, c=128, d=128, N=N, topk=1, B=2,
                            T=L // 2)
            inp = dict(base)
            inp["router_logits"] = np.ascontiguousarray(base["router_logits"][..., :N])
            for sched in ("varlen", "masked"):
                T, S, total_ms, stages, _ = run_forward(ns, w, si, sse, torch, inp=inp,
                                                        schedule=sched)
                ms = total_ms / ns.steps
                row = {"L": L, "N": N, "schedule": sched, "ms": ms,
                       "tokens_per_s": T / (ms * 1e-3), "stage_ms": stages}
                if sched == "varlen":
                    row["fwd_bwd_ms"] = fwd_bwd_ms(w, si, sse, torch, inp)
                rows.append(row)
                log(f"fig6 L={L} N={N} {sched}: {ms:.3f} ms" +
                    (f", forward + backward {row['fwd_bwd_ms']:.3f} ms" if sched == "varlen" else ""))
    spread, spread_fb, faster = {}, {}, {}
    for L in sorted({r["L"] for r in rows}):
        t = [r["ms"] for r in rows if r["L"] == L and r["schedule"] == "varlen"]
        spread[str(L)] = max(t) / min(t)
        t = [r["fwd_bwd_ms"] for r in rows if r["L"] == L and r["schedule"] == "varlen"]
        spread_fb[str(L)] = max(t) / min(t)
        for N in (4, 8, 16):
            tv = [r["ms"] for r in rows if r["L"] == L and r["N"] == N and r["schedule"] == "varlen"][0]
            tm = [r["ms"] for r in rows if r["L"] == L and r["N"] == N and r["schedule"] == "masked"][0]
            faster[f"L{L}_N{N}"] = "masked" if tm < tv else "varlen"
    return {"setting": "H=8, c=d=128, k=1, cu_seqlens=[0, L/2, L], N in {4, 8, 16}, bf16 "
                       "inputs, router logits N(0,1), forward of both schedules, forward + backward "
                       "of the varlen schedule",
            "rows": rows, "varlen_max_over_min_across_N": spread,
            "varlen_fwd_bwd_max_over_min_across_N": spread_fb, "faster_schedule": faster}


def timed(torch, fn, steps, warmup):
    """Mean ms of fn over `steps` calls after `warmup` calls (HIP events on
    the current stream)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def run_backward(args, w, si, sse, torch):
    """sse_backward on the main workload: all five input gradients and the
    initial-state gradient."""
    inp = si.forward_inputs(w)
    cu = inp["cu_seqlens"]
    T, S = int(cu[-1]), len(cu) - 1
    max_len = int((cu[1:] - cu[:-1]).max())
    d_in = {n: to_dev(inp[n]) for n in NAMES + ("cu_seqlens",)}
    del inp
    do = torch.randn((T, w.H, w.d), dtype=torch.float32, device="cuda")
    out = {nm: torch.empty(shp, dtype=torch.float32, device="cuda") for nm, shp in (
        ("dq", (T, w.H, w.c)), ("dkey_logits", (T, w.H, w.c)), ("dlog_alpha", (T, w.H, w.c)),
        ("dv", (T, w.H, w.d)), ("drouter_logits", (T, w.H, w.N)),
        ("dinitial_states", (S, w.H, w.N + 1, w.c, w.d)))}
    ws = torch.empty(sse.sse_backward_workspace_bytes(T, S, max_len, w.H, w.c, w.d, w.N, w.topk),
                     dtype=torch.uint8, device="cuda")

    def step():
        sse.sse_backward(*(d_in[n] for n in NAMES), w.N, w.topk, d_in["cu_seqlens"], do,
                         max_len, want_dinitial=True, workspace=ws, out=out)

    ms = timed(torch, step, args.bwd_steps, 1)
    HT = T * w.H
    records = HT * (w.topk + 1)
    # inputs read once (bf16), do read once, the five input gradients written
    # once, the initial-state gradients written once (fp32)
    nbytes = (HT * 2 * (3 * w.c + w.d + w.N) + HT * 4 * w.d + HT * 4 * (3 * w.c + w.d + w.N)
              + S * w.H * (w.N + 1) * w.c * w.d * 4)
    # five c x d products and three causal C x c / C x d pairs per record (C = 64).
    # With bf16 inputs all of them run on bf16 MFMA (Qt S_in, Kh G~, g S_in^T,
    # V G~^T, the A and GV tiles and the products over a chunk's records in
    # the chunk pass, Qt^T g in the reverse sweep) and are priced at its peak
    C = 64
    flops = records * 2 * (1.5 * C * w.c + 1.5 * C * w.d + 5 * w.c * w.d)
    hbm_ms = nbytes / (HBM_PEAK_GBS * 1e9) * 1e3
    mfma_ms = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3
    roof_ms = max(hbm_ms, mfma_ms)
    bound = ("hbm: inputs and do read once, the gradients written once, at 8 TB/s" if hbm_ms >= mfma_ms
             else "mfma: every product at the bf16 peak (2.5 PFLOP/s)")
    return {"workload": w.notes + ", gradients of all five inputs and the initial states",
            "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "algorithmic_bytes": nbytes,
            "algorithmic_flops": flops, "roofline_ms": roof_ms, "frac": roof_ms / ms,
            "hbm_ms": hbm_ms, "mfma_ms": mfma_ms, "bound": bound}


def run_rowsparse(args, si, sse, torch):
    """Row-sparse top-k key variant on the main shape (B=4, H=16, T=8192,
    c=d=128), k = 32 of 128 rows, identity transition on unselected rows."""
    w = si.Workload("rowsparse_main", "bf16", H=16, c=128, d=128, N=1, topk=1, B=4, T=8192)
    inp = si.forward_inputs(w)
    cu = inp["cu_seqlens"]
    T, S = int(cu[-1]), len(cu) - 1
    d_in = {n: to_dev(inp[n]) for n in ("q", "key_logits", "v", "log_alpha", "cu_seqlens")}
    del inp
    o = torch.empty((T, w.H, w.d), dtype=torch.float32, device="cuda")
    fs = torch.empty((S, w.H, w.c, w.d), dtype=torch.float32, device="cuda")
    ws = torch.empty(sse.sse_rowsparse_workspace_bytes(T, S, w.T, w.H, w.c, w.d),
                     dtype=torch.uint8, device="cuda")

    def step():
        sse.sse_rowsparse_forward(d_in["q"], d_in["key_logits"], d_in["v"], d_in["log_alpha"], 32,
                                  d_in["cu_seqlens"], w.T, o=o, final_states=fs, workspace=ws)

    ms = timed(torch, step, args.steps, args.warmup)
    HT = T * w.H
    nbytes = HT * 2 * (3 * w.c + w.d) + HT * 4 * w.d + S * w.H * w.c * w.d * 4
    flops = chunk_flops(HT, w.c, w.d)
    roof_ms = max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e3
    return {"workload": "bf16, B=4 H=16 T=8192 c=d=128, row top-k 32 of 128, identity on "
                        "unselected rows", "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
            "algorithmic_bytes": nbytes, "algorithmic_flops": flops, "roofline_ms": roof_ms,
            "frac": roof_ms / ms}


def run_decode(args, si, sse, torch):
    w = si.WORKLOADS["decode_bf16"]
    states0 = torch.empty((w.B, w.H, w.N + 1, w.c, w.d), dtype=torch.float32, device="cuda")
    for b in range(w.B):
        states0[b].copy_(torch.from_numpy(si.decode_states(w, b)))
    toks = si.decode_inputs(w)
    d_in = {n: to_dev(toks[n]) for n in NAMES}
    del toks
    st = states0.clone()
    o = torch.empty((w.B, w.H, w.d), dtype=torch.float32, device="cuda")
    steps = w.decode_steps

    def run():
        for t in range(steps):
            sse.sse_decode_step(*(d_in[n][t] for n in NAMES), w.N, w.topk, st, o=o)

    run()  # warm-up pass
    best = None
    stream = torch.cuda.current_stream()
    for _ in range(args.decode_reps):
        st.copy_(states0)  # restore pristine states outside the timed region
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    per_step_ms = best / steps
    # per step: k+1 states of c*d fp32 read and written per (b, h); inputs; o
    state_bytes = w.B * w.H * (w.topk + 1) * w.c * w.d * 4 * 2
    in_bytes = w.B * w.H * 2 * (3 * w.c + w.d + w.N) + w.B * w.H * 4 * w.d
    gbs = (state_bytes + in_bytes) / (per_step_ms * 1e-3) / 1e9
    return {
        "workload": "decode_bf16: 256 seqs x H=16, c=d=128, N=16, k=2, 64 steps, states N(0,0.1)",
        "tokens_per_s": w.B * steps / (best * 1e-3),
        "ms_per_step": per_step_ms,
        "bytes_per_step": state_bytes + in_bytes,
        "achieved_GBs": gbs,
        "hbm_frac": gbs / HBM_PEAK_GBS,
        "reps": args.decode_reps,
    }


def cpu_baseline(args, w, si):
    """The untuned fp64 oracle on the whole main workload (every one of its
    64 distinct (sequence, head) units), threads over units, plus its
    single-thread rate on the small workload."""
    import oracle
    affinity = len(os.sched_getaffinity(0))
    threads = min(affinity, 16)
    inp = si.forward_inputs(w)
    cu = inp["cu_seqlens"]
    T = int(cu[-1])
    lib = oracle.load()
    t0 = time.perf_counter()
    oracle.forward(*(inp[n] for n in NAMES), cu, w.N, w.topk, threads=threads, lib=lib)
    el = time.perf_counter() - t0
    ws = si.WORKLOADS["small_bf16"]
    inp_s = si.forward_inputs(ws)
    t1 = time.perf_counter()
    oracle.forward(*(inp_s[n] for n in NAMES), inp_s["cu_seqlens"], ws.N, ws.topk, threads=1,
                   lib=lib)
    el1 = time.perf_counter() - t1
    T1 = int(inp_s["cu_seqlens"][-1])
    return {
        "value": T / el,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"the whole main workload: {T} tokens x {w.H} heads, all "
                  f"{(len(cu) - 1) * w.H} (sequence, head) units, {el:.1f} s wall on {threads} "
                  f"threads ({threads * el:.0f} thread-seconds)",
        "host_cpus": os.cpu_count(),
        "affinity_cpus": affinity,
        "single_thread_small_bf16": {"tokens_per_s": T1 / el1, "seconds": el1,
                                     "workload": ws.notes},
    }


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chunk_ws_main_bf16_traffic.json")
# the dominant kernel's source and the headers it includes
KERNEL_SRC = [os.path.join(ROOT, "sparse_state_linear_amd", "csrc", f)
              for f in ("chunk_ws.hip", "chunk_common.h", "sse_device.h", "sse_launch.h")]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(stage):
    """HBM bytes per launch of the dominant kernel from the committed
    FETCH_SIZE/WRITE_SIZE counter runs (scaled by the copy-kernel
    calibration), or None when the kernel source changed since then."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(stage)
    return None if k is None else k["hbm_bytes_per_launch"]


def measured_peaks(torch):
    """Achievable rates on this GPU for scale: a 1 GiB device copy, an
    in-place read-modify-write of 1 GiB (the decode's access type) and a
    bf16 GEMM of 8192^3 (library MFMA code), each the best of 5."""
    n = (1 << 30) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    a = torch.randn((8192, 8192), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((8192, 8192), dtype=torch.bfloat16, device="cuda")

    def best_ms(f, reps=5):
        f()
        torch.cuda.synchronize()
        out = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            out = ms if out is None else min(out, ms)
        return out

    copy = 2 * n * 4 / (best_ms(lambda: y.copy_(x)) * 1e-3) / 1e9
    rmw = 2 * n * 4 / (best_ms(lambda: x.mul_(1.0)) * 1e-3) / 1e9
    gemm = 2 * 8192 ** 3 / (best_ms(lambda: torch.matmul(a, b)) * 1e-3) / 1e12
    del x, y, a, b
    return {"copy_GBs": copy, "inplace_rmw_GBs": rmw, "bf16_gemm_TFLOPs": gemm}


def calib_copy(torch, mib=1024, reps=3):
    """A plain device copy of known size, run under the same counters as the
    benchmark to calibrate FETCH_SIZE / WRITE_SIZE."""
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n * 4, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-reps", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode timing")
    ap.add_argument("--no-varlen", action="store_true", help="skip the varlen forward timing")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak calibration")
    ap.add_argument("--bwd-steps", type=int, default=5, help="timed backward calls")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the backward, masked-schedule and row-sparse timings")
    ap.add_argument("--fig6", action="store_true",
                    help="also time the forward over L and N in the operator-timing setting (Fig. 6)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--only", choices=("varlen", "decode", "masked", "backward", "rowsparse"),
                    help="run only this leg (for kernel traces) and print its record")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_state_linear_amd as sse
    import sse_inputs as si

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calib_copy:
        calib_copy(torch)
        return
    w = si.WORKLOADS["main_bf16"]
    if args.only:
        if args.only == "varlen":
            wv = si.WORKLOADS["varlen_bf16"]
            Tv, _, v_total_ms, v_stages, _ = run_forward(args, wv, si, sse, torch)
            rec = {"ms_per_step": v_total_ms / args.steps, "tokens": Tv, "stage_ms": v_stages}
        elif args.only == "decode":
            rec = run_decode(args, si, sse, torch)
        elif args.only == "masked":
            _, _, m_total_ms, m_stages, _ = run_forward(args, w, si, sse, torch, schedule="masked")
            rec = {"ms_per_step": m_total_ms / args.steps, "stage_ms": m_stages}
        elif args.only == "backward":
            rec = run_backward(args, w, si, sse, torch)
        else:
            rec = run_rowsparse(args, si, sse, torch)
        print(json.dumps({"only": args.only, **rec}), flush=True)
        return
    log("forward", w.notes)
    step_stats = {}
    T, S, total_ms, stages, calls = run_forward(args, w, si, sse, torch, step_stats=step_stats,
                                                prewarm_s=0.3)
    ms = total_ms / args.steps
    tokens_per_s = T / (ms * 1e-3)
    # dominant kernel: the routed pass (k of the k+1 partition reads)
    kern = {"routed": ("chunk_ws_kernel<128,128,routed>", w.N, T * w.H * w.topk, False),
            "shared": ("chunk_ws_kernel<128,128,shared>", 1, T * w.H, True)}
    dom = max(kern, key=lambda k: stages[k])
    kname, parts, records, writes_o = kern[dom]
    kb = pass_bytes(T, S, w.H, w.c, w.d, parts, writes_o)
    kf = chunk_flops(records, w.c, w.d)
    k_ms = stages[dom]
    achieved = kb / (k_ms * 1e-3) / 1e9
    fb = forward_bytes(T, S, w.H, w.c, w.d, w.N)
    ff = chunk_flops(T * w.H * (w.topk + 1), w.c, w.d)
    roof_ms = max(fb / (HBM_PEAK_GBS * 1e9), ff / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e3
    log(f"forward {ms:.3f} ms/step; stages {stages}")

    varlen = None
    if not args.no_varlen:
        wv = si.WORKLOADS["varlen_bf16"]
        log("forward", wv.notes)
        Tv, Sv, v_total_ms, v_stages, _ = run_forward(args, wv, si, sse, torch)
        v_ms = v_total_ms / args.steps
        vb = forward_bytes(Tv, Sv, wv.H, wv.c, wv.d, wv.N)
        vf = chunk_flops(Tv * wv.H * (wv.topk + 1), wv.c, wv.d)
        v_roof = max(vb / (HBM_PEAK_GBS * 1e9), vf / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e3
        varlen = {
            "workload": "varlen_bf16: 8 packed sequences, lengths U[1024,16384] (seed 0), "
                        "H=16, c=d=128, N=32, k=4 + shared partition, bf16 inputs",
            "tokens": Tv,
            "ms_per_step": v_ms,
            "tokens_per_s": Tv / (v_ms * 1e-3),
            "algorithmic_bytes": vb,
            "algorithmic_flops": vf,
            "roofline_ms": v_roof,
            "frac": v_roof / v_ms,
            "stage_ms": v_stages,
        }
        log(f"varlen forward {v_ms:.3f} ms/step ({Tv} tokens); stages {v_stages}")

    decode = None
    if not args.no_decode:
        log("decode", si.WORKLOADS["decode_bf16"].notes)
        decode = run_decode(args, si, sse, torch)
        log(f"decode {decode['ms_per_step'] * 1e3:.1f} us/step, {decode['achieved_GBs']:.0f} GB/s")

    peaks = None
    if not args.no_peaks:
        peaks = measured_peaks(torch)
        # the forward's roofline time against the measured rates instead of
        # the spec peaks
        roof_meas_ms = max(fb / (peaks["copy_GBs"] * 1e9),
                           ff / (peaks["bf16_gemm_TFLOPs"] * 1e12)) * 1e3
        peaks["forward_frac"] = roof_meas_ms / ms
        if decode is not None:
            peaks["decode_frac"] = decode["achieved_GBs"] / peaks["inplace_rmw_GBs"]
        log(f"measured peaks {peaks}")

    extra = None
    if not args.no_extra:
        log("masked schedule forward", w.notes)
        Tm, _, m_total_ms, m_stages, _ = run_forward(args, w, si, sse, torch, schedule="masked")
        m_ms = m_total_ms / args.steps
        log(f"masked forward {m_ms:.3f} ms/step; stages {m_stages}")
        log("backward", w.notes)
        bwd = run_backward(args, w, si, sse, torch)
        log(f"backward {bwd['ms_per_step']:.3f} ms/step")
        log("row-sparse forward")
        rs = run_rowsparse(args, si, sse, torch)
        log(f"row-sparse forward {rs['ms_per_step']:.3f} ms/step")
        extra = {
            "masked_forward": {"workload": w.notes + ", masked schedule",
                               "ms_per_step": m_ms, "tokens_per_s": Tm / (m_ms * 1e-3),
                               "roofline_ms": roof_ms, "frac": roof_ms / m_ms,
                               "stage_ms": m_stages},
            "backward": bwd,
            "rowsparse_forward": rs,
        }

    fig6 = fig6_sweep(args, si, sse, torch) if args.fig6 else None

    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(args, w, si)

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "main_bf16: SSE forward, B=4 H=16 T=8192 c=d=128 N=16 k=2 + shared "
                        "partition, bf16 inputs, fp32 state, router logits N(0,1.5)",
            "tokens_per_step": T,
            "head_tokens_per_step": T * w.H,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kname,
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(dom),
            "kernel_ms": k_ms,
            "algorithmic_bytes_per_launch": kb,
            "algorithmic_flops_per_launch": kf,
            "mfma_frac": kf / (k_ms * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
        },
        "forward_roofline": {
            "algorithmic_bytes": fb,
            "algorithmic_flops": ff,
            "roofline_ms": roof_ms,
            "frac": roof_ms / ms,
            "stage_ms": stages,
            "traced_calls": calls,
        },
        "step_ms": step_stats,
        "varlen_forward": varlen,
        "measured_peaks": peaks,
        "decode": decode,
        "masked_forward": None if extra is None else extra["masked_forward"],
        "backward": None if extra is None else extra["backward"],
        "rowsparse_forward": None if extra is None else extra["rowsparse_forward"],
        "fig6_sweep": fig6,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
