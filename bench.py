#!/usr/bin/env python3
"""Benchmark of the HAD inference-attention hot path on one MI355X.

One step = the whole path over one batch of seeded synthetic input already
resident in HBM: had_forward, i.e. the pack of Q and K (sign bits and sigma
partials) in one launch, then the attention launch, which also finalizes both
sigmas (--separate-calls times had_pack(Q), had_pack(K), had_attention
instead).  Everything runs on torch's current stream.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

Default workload: the T5-base-shaped long-document encoder attention
(B=8, H=12, n=1024, d=64, N=256, bf16 V), on which the metric is quoted.

Roofline of the dominant kernel (had_attention), algorithmic work only:
    int ops = visible_pairs * (2W + 2) + kept * 2   (XOR+popcount per word,
              histogram + compaction per pair, weight per kept entry)
    flops   = 2 * kept * d                           (weighted sum of V)
    lane-op equivalents = int ops + flops / 4        (a packed fp32 FMA lane
              does 4 flops per lane-op issue)
    peak    = 256 CU * 4 SIMD * 16 lanes * 2.4 GHz = 39.32 T lane-ops/s
The kernel puts the logits and the V product on the matrix cores, so it can
run faster than this vector-unit bound (frac > 1).
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

METRIC = "query rows/sec of HAD attention at n={n},N={topn}; % of HBM/VALU roofline"  # headline: n=1024, N=256
VALU_PEAK = 256 * 4 * 16 * 2.4e9  # int32 lane-ops/s
HBM_PEAK = 8.0e12  # B/s


def work_model(w):
    """Algorithmic work of one had_attention launch on workload w."""
    W = (w.dim + 31) // 32
    bh = w.batch * w.heads
    n, N = w.seq, w.topn
    if w.causal:
        vis = n * (n + 1) // 2
        kept = sum(min(N, i + 1) for i in range(n))
    else:
        vis = n * n
        kept = n * min(N, n)
    vis *= bh
    kept *= bh
    int_ops = vis * (2 * W + 2) + kept * 2
    flops = 2 * kept * w.dim
    lane_ops = int_ops + flops / 4.0
    vbytes = 2 if w.v_dtype == "bf16" else 4
    hbm = bh * n * (2 * W * 4 + w.dim * vbytes + w.dim * 4)
    return {"visible_pairs": vis, "kept": kept, "int_ops": int_ops, "flops": flops,
            "lane_ops": lane_ops, "hbm_bytes": hbm}


def traffic_for(workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    from sparse_attention_had_amd.profiling import source_hash

    path = os.path.join(ROOT, "profiles", f"traffic_had_attention_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, inp, budget_s):
    """The plain oracle on a bounded sample of the same workload, one thread."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    import oracle

    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    rows = 0
    heads = 0
    t0 = time.perf_counter()
    try:
        for bh in range(w.batch * w.heads):
            b, h = divmod(bh, w.heads)
            oracle.sigma(inp["q"][b, h])
            oracle.forward(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], w.topn, w.scale,
                           causal=w.causal)
            rows += w.seq
            heads += 1
            if time.perf_counter() - t0 > budget_s:
                break
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "query rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{heads} of {w.batch * w.heads} (batch, head) slices, all {w.seq} rows each "
                      f"(sign, pack, sigma of the slice, logits, stable-sort top-N, softmax, AV), "
                      f"{dt:.1f} s wall, numpy float64, 1 thread"}


def decode_model(w, fp32_rows=False):
    """Algorithmic HBM bytes of one had_decode call on decode workload w: the
    cached key words once, the kept V rows of every new row, the new rows'
    query words (float32 rows for had_decode_forward) and outputs."""
    W = (w.dim + 31) // 32
    bh = w.batch * w.heads
    vbytes = 2 if w.v_dtype == "bf16" else 4
    kept = 0
    for i in range(w.n_q):
        vis = min(w.n_k, w.q_pos0 + i + 1) if w.causal else w.n_k
        kept += min(w.topn, vis)
    qbytes = w.dim * 4 if fp32_rows else W * 4
    per_slice = w.n_k * W * 4 + kept * w.dim * vbytes + w.n_q * (qbytes + w.dim * 4)
    return {"kept": bh * kept, "hbm_bytes": bh * per_slice}


def decode_cpu_baseline(w, inp, budget_s):
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    import oracle

    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    rows = heads = 0
    t0 = time.perf_counter()
    try:
        for bh in range(w.batch * w.heads):
            b, h = divmod(bh, w.heads)
            oracle.decode(inp["q_new"][b, h], inp["k"][b, h], inp["v"][b, h], w.topn, w.scale,
                          q_pos0=w.q_pos0, causal=w.causal)
            rows += w.n_q
            heads += 1
            if time.perf_counter() - t0 > budget_s:
                break
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "query rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{heads} of {w.batch * w.heads} (batch, head) slices, {w.n_q} new rows "
                      f"each against {w.n_k} cached keys (sign, pack, logits, stable-sort "
                      f"top-N, softmax, AV), {dt:.1f} s wall, numpy float64, 1 thread"}


def settle(step, seconds):
    """Untimed steps until `seconds` of wall time have passed (at most 20000):
    the GPU ramps its clocks up over the first tens of milliseconds of load,
    and the timed steps should see the steady state.  Returns the count."""
    import torch

    if seconds <= 0:
        return 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < 20000:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break
    return n


def bench_decode(args, w):
    """One step = had_decode_forward: the new rows' float32 queries against the
    packed cache (packed once, outside the timed region); their sign words are
    built inside the first of its three launches.  --separate-calls times
    had_pack of the new rows + had_decode instead."""
    import torch
    import sparse_attention_had_amd as had
    from had_workloads import decode_inputs

    inp = decode_inputs(w)
    dev = torch.device("cuda:0")
    qn = torch.from_numpy(inp["q_new"]).to(dev)
    kc = torch.from_numpy(inp["k"]).to(dev)
    v = torch.from_numpy(inp["v"])
    v = (v.to(torch.bfloat16) if w.v_dtype == "bf16" else v).to(dev)
    kb, _ = had.pack(kc, with_sigma=False)
    del kc
    W = had.words_per_row(w.dim)
    qb = torch.empty((w.batch, w.heads, w.n_q, W), dtype=torch.int32, device=dev)
    out = torch.empty((w.batch, w.heads, w.n_q, w.dim), dtype=torch.float32, device=dev)
    ws = torch.empty(had.decode_workspace_bytes(w.batch, w.heads, w.n_q, w.n_k, w.n_k, w.dim),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def decode_call():
        if args.separate_calls:
            had.decode(qb, kb, v, w.topn, w.scale, q_pos0=w.q_pos0, causal=w.causal, out=out,
                       workspace=ws)
        else:
            had.decode_forward(qn, kb, v, w.topn, w.scale, q_pos0=w.q_pos0, causal=w.causal,
                               out=out, workspace=ws)

    def step():
        if args.separate_calls:
            had.pack(qn, out=qb, with_sigma=False)
        decode_call()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    settled = settle(step, args.settle_s)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    if args.separate_calls:
        had.pack(qn, out=qb, with_sigma=False)
    for _ in range(args.steps):
        decode_call()
    d1.record(stream)
    torch.cuda.synchronize()
    dec_s = d0.elapsed_time(d1) / args.steps / 1e3
    model = decode_model(w, fp32_rows=not args.separate_calls)
    achieved = model["hbm_bytes"] / dec_s
    rec = {
        "metric": f"query rows/sec of HAD decode against a {w.n_k}-key cache; % of HBM roofline",
        "value": w.rows / (ms_step / 1e3),
        "unit": "query rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settled,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.v_dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "n_k": w.n_k,
                   "n_q": w.n_q, "dim": w.dim, "topn": w.topn, "causal": w.causal,
                   "v_dtype": w.v_dtype, "scale": w.scale,
                   "step": ("had_pack(new rows' Q) + had_decode (4 launches)" if args.separate_calls
                            else "had_decode_forward (3 launches; the new rows' sign words are built "
                                 "inside the first)")},
        "decode_us": dec_s * 1e6,
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK, "traffic": None,
                     "kernel": "had_decode%s (dec_hist, dec_gather, dec_reduce)"
                               % ("" if args.separate_calls else "_forward"),
                     "work_per_launch": {k2: float(v2) for k2, v2 in model.items()}},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = decode_cpu_baseline(w, inp, args.cpu_budget)
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-s", type=float, default=0.2,
                    help="untimed steps for this many seconds after the warmup steps, so "
                         "that the timed steps run at steady-state clocks (0: none)")
    ap.add_argument("--attention-only", action="store_true",
                    help="time only had_attention launches (for profiling runs)")
    ap.add_argument("--separate-calls", action="store_true",
                    help="step = had_pack(Q), had_pack(K), had_attention (5 launches) "
                         "instead of had_forward (2 launches); for a decode workload, "
                         "had_pack(new rows) + had_decode instead of had_decode_forward")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="for HBM counter runs: 3 attention launches, then one plain "
                         "64 MiB device copy that calibrates FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only; --gpus must be 1 (the path would shard by "
              "(batch, head) slice with no communication, one process per GPU).", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_had_amd as had
    from had_workloads import DECODE_WORKLOADS, HEADLINE, WORKLOADS, workload_inputs

    name = args.workload or HEADLINE
    if name in DECODE_WORKLOADS:
        return bench_decode(args, DECODE_WORKLOADS[name])
    w = WORKLOADS[name]
    inp = workload_inputs(w)
    dev = torch.device("cuda:0")
    q = torch.from_numpy(inp["q"]).to(dev)
    k = torch.from_numpy(inp["k"]).to(dev)
    v = torch.from_numpy(inp["v"])
    v = (v.to(torch.bfloat16) if w.v_dtype == "bf16" else v).to(dev)
    W = had.words_per_row(w.dim)
    qb = torch.empty((w.batch, w.heads, w.seq, W), dtype=torch.int32, device=dev)
    kb = torch.empty_like(qb)
    sq = torch.empty(1, dtype=torch.float32, device=dev)
    sk = torch.empty(1, dtype=torch.float32, device=dev)
    out = torch.empty((w.batch, w.heads, w.seq, w.dim), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ws_q = torch.zeros(had.pack_workspace_bytes(q.shape), dtype=torch.uint8, device=dev)
    ws_k = torch.zeros_like(ws_q)
    ws_f = torch.zeros(2 * ws_q.numel(), dtype=torch.uint8, device=dev)

    if args.traffic_probe:
        from sparse_attention_had_amd.profiling import COPY_BYTES

        had.pack(q, out=qb, sigma=sq, workspace=ws_q)
        had.pack(k, out=kb, sigma=sk, workspace=ws_k)
        for _ in range(3):
            had.attention(qb, kb, v, w.topn, w.scale, w.causal, out=out)
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": name, "copy_bytes": COPY_BYTES}), flush=True)
        return

    def step():
        if args.attention_only:
            had.attention(qb, kb, v, w.topn, w.scale, w.causal, out=out)
        elif args.separate_calls:
            had.pack(q, out=qb, sigma=sq, workspace=ws_q)
            had.pack(k, out=kb, sigma=sk, workspace=ws_k)
            had.attention(qb, kb, v, w.topn, w.scale, w.causal, out=out)
        else:
            had.forward(q, k, v, w.topn, w.scale, w.causal, out=out, qbits=qb, kbits=kb,
                        sigma_q=sq, sigma_k=sk, workspace=ws_f)

    had.pack(q, out=qb, sigma=sq, workspace=ws_q)
    had.pack(k, out=kb, sigma=sk, workspace=ws_k)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    settled = settle(step, args.settle_s)

    # timed region 1: whole steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps

    # timed region 2: back-to-back had_attention launches on the same stream,
    # bracketed by HIP events, for the dominant kernel's average duration
    a_start = torch.cuda.Event(enable_timing=True)
    a_end = torch.cuda.Event(enable_timing=True)
    a_start.record(stream)
    for _ in range(args.steps):
        had.attention(qb, kb, v, w.topn, w.scale, w.causal, out=out)
    a_end.record(stream)
    torch.cuda.synchronize()
    attn_avg_s = a_start.elapsed_time(a_end) / args.steps / 1e3

    rows = w.rows
    model = work_model(w)
    achieved = model["lane_ops"] / attn_avg_s
    traffic = traffic_for(name)
    rec = {
        "metric": METRIC.format(n=w.seq, topn=w.topn),
        "value": rows / (ms_step / 1e3),
        "unit": "query rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settled,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": name, "batch": w.batch, "heads": w.heads, "seq": w.seq, "dim": w.dim,
            "topn": w.topn, "causal": w.causal, "v_dtype": w.v_dtype, "scale": w.scale,
            "step": ("attention only" if args.attention_only else
                     "had_pack(Q), had_pack(K), had_attention" if args.separate_calls else
                     "had_forward: pack(Q)+pack(K) in one launch, attention with sigma finalize"),
            "arithmetic": "int8 matrix-core logits (exact), int32 selection, fp32 softmax weights "
                          "as bf16 hi+lo, bf16 matrix-core V product with fp32 accumulation",
        },
        "attention_us": attn_avg_s * 1e6,
        "attention_rows_per_s": rows / attn_avg_s,
        "roofline": {
            "bound": "alu",
            "achieved": achieved / 1e12,
            "peak": VALU_PEAK / 1e12,
            "unit": "Tops/s",
            "frac": achieved / VALU_PEAK,
            "traffic": traffic,
            "kernel": "had_attn_kernel",
            "work_per_launch": {k2: float(v2) for k2, v2 in model.items()},
            "hbm_frac": (model["hbm_bytes"] / attn_avg_s) / HBM_PEAK,
        },
        "wall_s_timed_region": wall,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
