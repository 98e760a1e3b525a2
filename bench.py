#!/usr/bin/env python3
"""Benchmark of the GSA decode / prefill hot path on one MI355X.

Default workload: the batched GQA decode step (batch 32, 32 query heads over 8
kv-heads, head_dim 128, bf16 cache, 32768-token context, chunk 16, top-16
chunks, 64-token tail). One step = one gsa_decode call over the whole batch,
i.e. every stage of the path: gist scoring + attention over all gists, exact
top-k, unfold gather + attention over the chosen chunks and the tail, merge.

Cold-cache protocol without flushes: the benchmark keeps several copies
("layers") of the KV cache and step i reads layer i mod L, so a step's data was
last touched L-1 steps (>= 0.9 GB of other traffic) earlier and is no longer in
the 256 MB Infinity Cache -- as in a real model, where each layer has its own
cache. Inputs are resident in HBM before timing starts.

Prints one JSON line (see the fields below). `--config` picks another
workload (parity configs listed in gsa_inputs.CONFIGS).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GSA decode query-heads/s + achieved HBM GB/s (32K ctx, C=16, k=16, bf16)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_algorithmic_bytes(cfg, sel) -> int:
    """Bytes the method must touch once per step: every gist row (K+V), the raw
    rows of the selected chunks not already in the tail, the tail rows, q, the
    fp32 output, lse and the selected indices."""
    eb = 2 if cfg.dtype == "bf16" else 4
    row = 2 * cfg.head_dim * eb                      # K + V
    units = cfg.batch * cfg.n_kv_heads
    tail0 = cfg.n_raw - cfg.tail
    sel = np.asarray(sel).reshape(units, -1) if cfg.topk else np.zeros((units, 0), np.int64)
    raw_sel = 0
    C = cfg.chunk
    for u in range(units):
        for m in sel[u]:
            raw_sel += max(0, min(C, tail0 - int(m) * C))
    rows = units * cfg.M + raw_sel + units * cfg.tail
    q = cfg.batch * cfg.n_q_heads * cfg.head_dim * eb
    out = cfg.batch * cfg.n_q_heads * cfg.head_dim * 4
    lse = cfg.batch * cfg.n_q_heads * 4
    idx = units * cfg.topk * 4
    return rows * row + q + out + lse + idx


def cpu_baseline_decode(inp, cfg, budget_s: float):
    """Time the fp64 oracle (as it stands) on whole decode steps, single thread."""
    import oracle
    from threadpoolctl import threadpool_limits
    g = cfg.n_q_heads // cfg.n_kv_heads
    q = inp.q.float().cpu().numpy()
    units = [(b, j) for b in range(cfg.batch) for j in range(cfg.n_kv_heads)]
    t_total, n_qh, reps = 0.0, 0, 0
    with threadpool_limits(1):
        while t_total < budget_s and reps < 1000:
            for b, j in units:
                K = inp.k_cache[b, j].float().cpu().numpy()   # host copy, not timed
                V = inp.v_cache[b, j].float().cpu().numpy()
                t0 = time.perf_counter()
                oracle.decode_unit(q[b, j * g:(j + 1) * g], K, V, n_raw=cfg.n_raw, n_gist=cfg.M,
                                   chunk=cfg.chunk, topk=cfg.topk, tail=cfg.tail)
                t_total += time.perf_counter() - t0
                n_qh += g
                if t_total >= budget_s:
                    break
            reps += 1
    return {"value": n_qh / t_total, "unit": "query-heads/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_qh // g} (batch, kv-head) units of the same workload "
                      f"({n_qh} query heads), fp64 numpy, 1 thread, {t_total:.1f} s"}


def run_decode_bench(args):
    import torch
    import decode_gsa_amd as gsa
    import gsa_inputs as gi

    cfg = gi.CONFIGS[args.config]
    dev = torch.device("cuda", 0)
    log(f"[bench] generating {cfg.name} inputs ...")
    inp = gi.make_decode(cfg, 1000 + 2, device=dev)
    stream = torch.cuda.current_stream(dev)
    # cache copies for the cold-cache rotation
    step_bytes_cache = cfg.batch * cfg.n_kv_heads * cfg.R * cfg.head_dim * (2 if cfg.dtype == "bf16" else 4) * 2
    layers = args.layers or max(1, min(8, math.ceil(1.0e9 / max(1.0, 0.3e9)) + 1))
    free = torch.cuda.mem_get_info(dev)[0]
    layers = max(1, min(layers, int(0.8 * free // step_bytes_cache)))
    ks = [inp.k_cache] + [inp.k_cache.clone() for _ in range(layers - 1)]
    vs = [inp.v_cache] + [inp.v_cache.clone() for _ in range(layers - 1)]
    B, Hq, D = inp.q.shape
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    sel = torch.empty(B, cfg.n_kv_heads, max(cfg.topk, 1), dtype=torch.int32, device=dev)
    p = gsa.decode_params(B, Hq, cfg.n_kv_heads, D, cfg.n_raw, cfg.M, cfg.chunk, cfg.topk,
                          cfg.tail, 0.0, gsa.GSA_BF16 if cfg.dtype == "bf16" else gsa.GSA_F32)
    ws = gsa.new_workspace(gsa.decode_workspace_size(p), dev)

    def step(i):
        l = i % layers
        gsa.gsa_decode(inp.q, ks[l], vs[l], chunk=cfg.chunk, topk=cfg.topk, tail=cfg.tail,
                       n_gist=cfg.M, out=out, lse=lse, sel_idx=sel, workspace=ws, stream=stream)

    # parity spot check of this exact launch configuration (selection must be the planted set)
    step(0)
    torch.cuda.synchronize()
    if cfg.topk > 0 and inp.planted is not None:
        assert torch.equal(sel.long(), inp.planted), "selection differs from the planted top-k"
    alg_bytes = decode_algorithmic_bytes(cfg, sel.cpu().numpy() if cfg.topk else [])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(args.warmup + i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = np.array([a.elapsed_time(b) for a, b in evs])
    ms_per_step = 1e3 * wall / args.steps
    qheads = B * Hq
    value = qheads / (ms_per_step / 1e3)
    call_ms = float(np.mean(ev_ms))
    achieved = alg_bytes / (call_ms / 1e3) / 1e9

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "query-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian q/K/V, planted top-k margin >= 0.5)",
        "config": {"workload": f"{cfg.name}: GQA decode step, B={cfg.batch}, Hq={cfg.n_q_heads}, "
                               f"Hkv={cfg.n_kv_heads}, D={cfg.head_dim}, N={cfg.n_raw}, "
                               f"C={cfg.chunk}, k={cfg.topk}, T={cfg.tail}, {cfg.dtype} cache",
                   "global_batch": cfg.batch, "seq_len": cfg.n_raw, "parallelism": "none (1 GPU)",
                   "cache_layers_rotated": layers},
        "tokens_per_s": cfg.batch / (ms_per_step / 1e3),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "scope": "whole gsa_decode call (all its kernels) per step, HIP events on "
                              "the launch stream",
                     "algorithmic_bytes_per_call": alg_bytes,
                     "call_ms_mean": call_ms, "call_ms_p10": float(np.percentile(ev_ms, 10)),
                     "call_ms_p90": float(np.percentile(ev_ms, 90))},
    }
    if not args.no_cpu:
        log("[bench] timing the CPU oracle ...")
        res["cpu_baseline"] = cpu_baseline_decode(inp, cfg, args.cpu_seconds)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="gqa_32k")
    ap.add_argument("--layers", type=int, default=0, help="cache copies rotated per step")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(decode units are independent; sharding is described in DESIGN.md).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import gsa_inputs as gi
    cfg = gi.CONFIGS[args.config]
    if isinstance(cfg, gi.DecodeConfig):
        res = run_decode_bench(args)
    else:
        raise SystemExit(f"--config {args.config}: not a single-level decode workload yet")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
