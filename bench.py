#!/usr/bin/env python3
"""Benchmark of the GSA hot path on one MI355X.

Default workload (gqa_32k): the batched GQA decode step -- batch 32, 32 query
heads over 8 kv-heads, head_dim 128, bf16 interleaved cache, 32768-token
context, chunk 16, top-16 chunks, 64-token tail. One step = one gsa_decode
call over the whole batch, i.e. every stage of the path: gist scoring +
attention over all gists and the tail, exact top-k, unfold of the chosen
chunks and the merge, in one launch of unit_kernel: one workgroup per
(batch, kv-head) unit for its 256 units (configurations with fewer units use
several workgroups per unit and a second launch, unit_unfold_kernel, that
selects, unfolds and merges).

`--config prefill_64k` times the causal block-sparse prefill instead (4096
query positions at the end of a 65536-token sequence, 32/8 heads, k=16, W=64).
`--config gist_64k` times the cache-building step of a 65536-token prompt:
gsa_cache_append of its raw and gist rows into an empty cache, then
gsa_gist_prefill of its 4096 gist tokens.
`--config varlen_32k` times gsa_decode_varlen on the same batch shape with
sequence lengths uniform in [4K, 32K] (one workgroup per unit: a step lasts
as long as its longest sequence).
`--scaling` sweeps the context from 32K to 16M tokens (one sequence, Hq 32 /
Hkv 8, C 16, k 16, T 64) over single-level, two-level and L-level decode
(fanout 16, levels added until the top holds at most 256 gists) and prints
one JSON line per (context, variant): wall time per step, the device time of
a call (event hook: first kernel's start to last kernel's end) and the
algorithmic bytes per step.

Cold-cache protocol without flushes: the benchmark keeps several copies
("layers") of the KV cache and step i reads layer i mod L, so a step's data was
last touched L-1 steps (>= 0.9 GB of other traffic) earlier and is no longer in
the 256 MB Infinity Cache -- as in a real model, where each layer has its own
cache. Inputs are resident in HBM before timing starts.

Timing: `value` and `ms_per_step` come from the wall clock around K
uninstrumented steps (device synchronizations on both sides). Per-kernel
times come from K more steps in which the library attaches HIP events to its
kernel launches (gsa_profile_events: the runtime stamps them with each
kernel's start and end), so the roofline of the dominant kernel is measured
live in bench.py (mean, median, p10, p90 per launch). Instrumented launches
do not overlap their neighbours and cost a few microseconds each, which is
why they are kept out of the throughput figure. The decode line also carries
the machine's practical streaming rate (plain 1 GiB device copies).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DECODE_METRIC = "GSA decode query-heads/s + achieved HBM GB/s (32K ctx, C=16, k=16, bf16)"
PREFILL_METRIC = "GSA block-sparse prefill query-positions/s + MFMA utilisation (64K ctx, 4096 queries)"
VARLEN_METRIC = "GSA variable-length decode query-heads/s + achieved HBM GB/s (4K-32K ctx, C=16, k=16, bf16)"
PAGED_METRIC = "GSA paged decode query-heads/s + achieved HBM GB/s (4K-32K ctx, 16-chunk pages, C=16, k=16, bf16)"
GIST_METRIC = "GSA cache build (append + gist-token attention) prompt tokens/s (64K prompt, C=16)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
GIST_SET_NAMES = {"selected": "selected chunks' gists + raw + tail (SG+SR)",
                  "none": "selected raw + tail (SR-only)"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------ HIP events ---

class HipEvents:
    """Raw hipEvent_t handles (the library's timing hook records them)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(h.value)

    def ms(self, a: int, b: int) -> float:
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(self.ev[a]),
                                        ctypes.c_void_p(self.ev[b])) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(h))


def timed_steps(gsa, step, args, n_marks):
    """Warm up, then time exactly args.steps steps (wall clock between two
    device synchronizations, no instrumentation). Then the same number of
    steps again with the library recording n_marks events per step (one
    before the first launch, one after each): a launch that records events
    starts only after the previous one has finished and costs a few
    microseconds more, so the instrumented steps give each kernel's own
    duration but not the throughput. Returns (wall ms per step of the first
    region, [steps, n_marks-1] ms per launch of the second)."""
    import torch
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = HipEvents(args.steps * n_marks)
    try:
        for i in range(args.steps):
            gsa.gsa_profile_events(ev.ev[i * n_marks:(i + 1) * n_marks])
            step(args.warmup + args.steps + i)
        torch.cuda.synchronize()
        gsa.gsa_profile_events([])
        per = np.array([[ev.ms(i * n_marks + j, i * n_marks + j + 1) for j in range(n_marks - 1)]
                        for i in range(args.steps)])
    finally:
        gsa.gsa_profile_events([])
        ev.close()
    return 1e3 * wall / args.steps, per


def pcts(x) -> dict:
    """Median, p10 and p90 of per-launch times (ms)."""
    x = np.asarray(x, dtype=np.float64)
    return {"ms_p50": float(np.percentile(x, 50)), "ms_p10": float(np.percentile(x, 10)),
            "ms_p90": float(np.percentile(x, 90))}


def source_sha(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "decode_gsa_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(key: str, sha: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, if it was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not t or t.get("source_sha") != sha:
        return None
    return t.get("bytes_per_launch")


# ---------------------------------------------------------------- decode ---

def decode_bytes(cfg, sel, gist_set="all"):
    """Algorithmic bytes per call: (gist pass, unfold pass). Gist pass: every
    gist row and every tail row (K + V), q. Unfold pass: the raw rows of the
    selected chunks not in the tail (K + V), the fp32 output, lse and the
    selected ids. With gist_set "selected" / "none" the gist pass reads the
    gists' K rows only (scores), and "selected" adds the chosen gists' V
    rows to the unfold pass."""
    eb = 2 if cfg.dtype == "bf16" else 4
    row = 2 * cfg.head_dim * eb
    units = cfg.batch * cfg.n_kv_heads
    tail0 = cfg.n_raw - cfg.tail
    raw_sel = 0
    if cfg.topk:
        sel = np.asarray(sel).reshape(units, -1)
        for u in range(units):
            for m in sel[u]:
                raw_sel += max(0, min(cfg.chunk, tail0 - int(m) * cfg.chunk))
    q = cfg.batch * cfg.n_q_heads * cfg.head_dim * eb
    out = cfg.batch * cfg.n_q_heads * (cfg.head_dim + 1) * 4 + units * cfg.topk * 4
    if gist_set == "all":
        gist = units * (cfg.M + cfg.tail) * row + q
        unfold = raw_sel * row + out
    else:
        gist = units * cfg.M * (row // 2) + units * cfg.tail * row + q
        unfold = raw_sel * row + (units * cfg.topk * (row // 2) if gist_set == "selected" else 0) + out
    return gist, unfold


def host_cpu():
    """(cores this process may run on, CPU model name)."""
    cores = len(os.sched_getaffinity(0))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def _oracle_decode_worker(job):
    """One process of the CPU baseline's pool (spawned: it never touches the
    GPU): the oracle's decode over units of a memory-mapped sample, round robin
    from its own first unit, until its wall-clock budget is spent. Returns
    (units done, seconds)."""
    import oracle
    from threadpoolctl import threadpool_limits
    path, first, stride, budget_s, kw = job
    data = np.load(path, mmap_mode="r")          # [units, 2, R, D] fp32 K and V, then q apart
    qs = np.load(path + ".q.npy")                 # [units, g, D]
    n, i, t0 = 0, first, time.perf_counter()
    with threadpool_limits(1):
        while time.perf_counter() - t0 < budget_s:
            u = i % data.shape[0]
            oracle.decode_unit(qs[u], np.asarray(data[u, 0]), np.asarray(data[u, 1]), **kw)
            n += 1
            i += stride
    return n, time.perf_counter() - t0


def cpu_baseline_decode(inp, cfg, budget_s: float, gist_set: str = "all"):
    """The fp64 oracle (as it stands) on whole decode units: one thread, then a
    pool of processes (one thread each) over the host's cores, up to 16."""
    import concurrent.futures
    import multiprocessing
    import tempfile
    import oracle
    from threadpoolctl import threadpool_limits
    g = cfg.n_q_heads // cfg.n_kv_heads
    q = inp.q.float().cpu().numpy()
    units = [(b, j) for b in range(cfg.batch) for j in range(cfg.n_kv_heads)]
    kw = dict(n_raw=cfg.n_raw, n_gist=cfg.M, chunk=cfg.chunk, topk=cfg.topk, tail=cfg.tail, gist_set=gist_set)
    t_total, n_qh, reps = 0.0, 0, 0
    single_s = budget_s / 3
    with threadpool_limits(1):
        while t_total < single_s and reps < 1000:
            for b, j in units:
                K = inp.k_cache[b, j].float().cpu().numpy()   # host copy, not timed
                V = inp.v_cache[b, j].float().cpu().numpy()
                t0 = time.perf_counter()
                oracle.decode_unit(q[b, j * g:(j + 1) * g], K, V, **kw)
                t_total += time.perf_counter() - t0
                n_qh += g
                if t_total >= single_s:
                    break
            reps += 1
    one = n_qh / t_total
    cores, model = host_cpu()
    workers = max(1, min(16, cores))
    res = {"value": one, "unit": "query-heads/s", "cores": 1, "kind": "oracle",
           "sample": f"{n_qh // g} (batch, kv-head) units of the same workload ({n_qh} query heads), "
                     f"fp64 numpy, 1 thread, {t_total:.1f} s",
           "host_cores": cores, "cpu_model": model, "single_thread_value": one}
    if workers > 1:
        # a sample of units written once to a memory-mapped file the workers share
        pick = units[:: max(1, len(units) // (2 * workers))][: 2 * workers]
        tmp = tempfile.mkdtemp(prefix="gsa_cpu_")
        path = os.path.join(tmp, "units.npy")
        K0 = inp.k_cache[0, 0]
        arr = np.lib.format.open_memmap(path, mode="w+", dtype=np.float32,
                                        shape=(len(pick), 2, K0.shape[0], K0.shape[1]))
        for i, (b, j) in enumerate(pick):
            arr[i, 0] = inp.k_cache[b, j].float().cpu().numpy()
            arr[i, 1] = inp.v_cache[b, j].float().cpu().numpy()
        arr.flush()
        del arr
        np.save(path + ".q.npy", np.stack([q[b, j * g:(j + 1) * g] for b, j in pick]))
        pool_s = budget_s / 2
        try:
            ctx = multiprocessing.get_context("spawn")
            with concurrent.futures.ProcessPoolExecutor(workers, mp_context=ctx) as ex:
                list(ex.map(_oracle_decode_worker, [(path, w, workers, 0.2, kw) for w in range(workers)]))  # start-up
                t0 = time.perf_counter()
                done = list(ex.map(_oracle_decode_worker, [(path, w, workers, pool_s, kw) for w in range(workers)]))
                wall = time.perf_counter() - t0
        finally:
            for f in (path, path + ".q.npy"):
                try:
                    os.remove(f)
                except OSError:
                    pass
            os.rmdir(tmp)
        n_units = sum(d[0] for d in done)
        res.update({"value": n_units * g / wall, "cores": workers,
                    "sample": f"{n_units} decode units of the same workload ({n_units * g} query heads) in "
                              f"{wall:.1f} s over {workers} processes of 1 thread each (fp64 numpy), sampled "
                              f"from {len(pick)} units; one thread alone: {one:.0f} query-heads/s over "
                              f"{n_qh // g} units in {t_total:.1f} s"})
    return res


def run_decode_bench(args):
    import torch
    import decode_gsa_amd as gsa
    import gsa_inputs as gi

    cfg = gi.CONFIGS[args.config]
    dev = torch.device("cuda", 0)
    log(f"[bench] generating {cfg.name} inputs ...")
    inp = gi.make_decode(cfg, 1000 + 2, device=dev)
    stream = torch.cuda.current_stream(dev)
    step_bytes_cache = cfg.batch * cfg.n_kv_heads * cfg.R * cfg.head_dim * (2 if cfg.dtype == "bf16" else 4) * 2
    layers = args.layers or 5
    free = torch.cuda.mem_get_info(dev)[0]
    layers = max(1, min(layers, int(0.8 * free // step_bytes_cache)))
    ks = [inp.k_cache] + [inp.k_cache.clone() for _ in range(layers - 1)]
    vs = [inp.v_cache] + [inp.v_cache.clone() for _ in range(layers - 1)]
    B, Hq, D = inp.q.shape
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    sel = torch.empty(B, cfg.n_kv_heads, max(cfg.topk, 1), dtype=torch.int32, device=dev)
    p = gsa.decode_params(B, Hq, cfg.n_kv_heads, D, cfg.n_raw, cfg.M, cfg.chunk, cfg.topk,
                          cfg.tail, 0.0, gsa.GSA_BF16 if cfg.dtype == "bf16" else gsa.GSA_F32,
                          gist_set=gsa.GIST_SETS[args.gist_set])
    ws = gsa.new_workspace(gsa.decode_workspace_size(p), dev)

    def step(i):
        l = i % layers
        gsa.gsa_decode(inp.q, ks[l], vs[l], chunk=cfg.chunk, topk=cfg.topk, tail=cfg.tail,
                       n_gist=cfg.M, out=out, lse=lse, sel_idx=sel, workspace=ws, stream=stream,
                       gist_set=args.gist_set)

    # parity spot check of this exact launch configuration (selection = planted set)
    step(0)
    torch.cuda.synchronize()
    if cfg.topk > 0 and inp.planted is not None:
        assert torch.equal(sel.long(), inp.planted), "selection differs from the planted top-k"
    gist_b, unfold_b = decode_bytes(cfg, sel.cpu().numpy() if cfg.topk else [], args.gist_set)
    alg_b = gist_b + unfold_b
    # launch structure of this call (the timing hook counts the launches):
    # unit_kernel (bf16, D = 128, k <= 64, at most 16384 gists when k > 0),
    # followed by unit_unfold_kernel when a unit takes several workgroups and
    # k > 0; otherwise gist_kernel, then unfold_kernel when k > 0
    unit_path = (cfg.dtype == "bf16" and cfg.head_dim == 128 and cfg.topk <= 64
                 and (cfg.topk == 0 or cfg.M <= 16384) and cfg.M + cfg.tail <= 256 * 5120)
    n_marks = gsa.gsa_profile_marks()
    ms_per_step, per = timed_steps(gsa, step, args, n_marks)
    call_ms = float(per.sum(axis=1).mean())
    qheads = B * Hq
    sha = source_sha("gsa_decode.hip", "gsa_device.hpp")
    if args.gist_set != "all":
        # with the selection rules the scoring launch reads the gists' K rows
        # only; the set (tail included) is read by the launch that attends it
        tail_b = cfg.batch * cfg.n_kv_heads * cfg.tail * 2 * cfg.head_dim * (2 if cfg.dtype == "bf16" else 4)
        gist_b, unfold_b = gist_b - tail_b, unfold_b + tail_b
    if unit_path and n_marks == 2:
        names, nbytes = ["unit_kernel"], [alg_b]
    elif unit_path:
        names, nbytes = ["unit_kernel", "unit_unfold_kernel"], [gist_b, unfold_b]
    elif n_marks == 4:   # gist pass, per-split candidates, unfold
        names, nbytes = ["gist_kernel", "cand_kernel", "unfold_kernel"], [gist_b, 0, unfold_b]
    else:
        names, nbytes = ["gist_kernel", "unfold_kernel"][:n_marks - 1], [gist_b, unfold_b][:n_marks - 1]
    kernels = {}
    for j, (nm, nb) in enumerate(zip(names, nbytes)):
        ms = float(per[:, j].mean())
        kernels[nm] = {"ms": ms, "alg_bytes": nb, "GB_s": nb / (ms / 1e3) / 1e9, **pcts(per[:, j])}
    kernels["whole_call"] = {"ms": call_ms, "alg_bytes": alg_b, "GB_s": alg_b / (call_ms / 1e3) / 1e9,
                             **pcts(per.sum(axis=1))}
    main, main_b, main_ms = names[0], nbytes[0], kernels[names[0]]["ms"]
    achieved = main_b / (main_ms / 1e3) / 1e9
    res = {
        "metric": DECODE_METRIC,
        "value": qheads / (ms_per_step / 1e3),
        "unit": "query-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian q/K/V, planted top-k with margin >= 0.5)",
        "config": {"workload": f"{cfg.name}: GQA decode step, B={cfg.batch}, Hq={cfg.n_q_heads}, "
                               f"Hkv={cfg.n_kv_heads}, D={cfg.head_dim}, N={cfg.n_raw}, "
                               f"C={cfg.chunk}, k={cfg.topk}, T={cfg.tail}, {cfg.dtype} cache"
                               + ("" if args.gist_set == "all" else
                                  f", attention set: {GIST_SET_NAMES[args.gist_set]}"),
                   "global_batch": cfg.batch, "seq_len": cfg.n_raw, "parallelism": "none (1 GPU)",
                   "cache_layers_rotated": layers},
        "tokens_per_s": cfg.batch / (ms_per_step / 1e3),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(f"{main}/{cfg.name}"
                                                 + ("" if args.gist_set == "all" else f"/{args.gist_set}"), sha),
                     "kernel": main, "alg_bytes_per_launch": main_b,
                     "launch_ms_mean": main_ms},
        "call": {"ms_mean": call_ms, "alg_bytes": alg_b, "GB_s": alg_b / (call_ms / 1e3) / 1e9},
        "kernels": kernels,
        "source_sha": sha,
    }
    # warm cache, labelled as such: the same cache copy every step (a working
    # set under 256 MB then stays in the Infinity Cache)
    def step_warm(i):
        step(0)
    warm_ms, warm_per = timed_steps(gsa, step_warm, args, n_marks)
    res["warm_cache"] = {"ms_per_step": warm_ms, "call_ms_p50": float(np.percentile(warm_per.sum(axis=1), 50)),
                         "note": "one cache copy reused every step (not the headline: the headline rotates "
                                 f"{layers} copies so that each step reads from HBM)"}
    res["latency_us"] = {"call_p50": 1e3 * kernels["whole_call"]["ms_p50"],
                         "call_p10": 1e3 * kernels["whole_call"]["ms_p10"],
                         "call_p90": 1e3 * kernels["whole_call"]["ms_p90"],
                         "wall_per_step": 1e3 * ms_per_step,
                         "note": "device time of one call (first kernel start to last kernel end), and the "
                                 "wall clock per step including the host launch"}
    res["roofline"]["machine_stream_rates"] = hbm_stream_rates()
    if not args.no_cpu:
        log("[bench] timing the CPU oracle ...")
        res["cpu_baseline"] = cpu_baseline_decode(inp, cfg, args.cpu_seconds, args.gist_set)
    return res


# ------------------------------------------------------------- two-level ---

def hier_bytes(cfg, sel1, gist_set="all"):
    """Algorithmic bytes per two-level call: every level-2 gist row, the level-1
    gists of the candidate groups and the orphans, the raw rows of the chosen
    chunks outside the tail, the tail rows (K + V each), q, and the fp32
    out/lse and both id lists. With gist_set "selected" / "none" the level-2
    and candidate gists are read for their K rows only (they route), the tail
    moves to the set's part, and "selected" adds the chosen gists' V rows."""
    b = cfg.base
    eb = 2 if b.dtype == "bf16" else 4
    row = 2 * b.head_dim * eb
    units = b.batch * b.n_kv_heads
    n_cand = cfg.topk2 * cfg.fanout + (b.M - cfg.M2 * cfg.fanout)
    tail0 = b.n_raw - b.tail
    raw_sel = 0
    if b.topk:
        for u_sel in np.asarray(sel1).reshape(units, -1):
            for m in u_sel:
                raw_sel += max(0, min(b.chunk, tail0 - int(m) * b.chunk))
    q = b.batch * b.n_q_heads * b.head_dim * eb
    out = b.batch * b.n_q_heads * (b.head_dim + 1) * 4 + units * (b.topk + cfg.topk2) * 4
    if gist_set != "all":
        return {"l2": units * cfg.M2 * (row // 2) + q,
                "cand": units * n_cand * (row // 2),
                "unfold": raw_sel * row + units * b.tail * row
                + (units * b.topk * (row // 2) if gist_set == "selected" else 0) + out}
    return {"l2": units * cfg.M2 * row + units * b.tail * row + q,
            "cand": units * n_cand * row,
            "unfold": raw_sel * row + out}


def run_hier_bench(args):
    import torch
    import decode_gsa_amd as gsa
    import gsa_inputs as gi

    cfg = gi.CONFIGS[args.config]
    b = cfg.base
    dev = torch.device("cuda", 0)
    log(f"[bench] generating {cfg.name} inputs ...")
    inp = gi.make_hier(cfg, 1000 + 4, device=dev)
    eb = 2 if b.dtype == "bf16" else 4
    per_layer = 2 * b.batch * b.n_kv_heads * (b.R + cfg.M2) * b.head_dim * eb
    layers = args.layers or 3
    free = torch.cuda.mem_get_info(dev)[0]
    layers = max(1, min(layers, int(0.8 * free // per_layer)))
    caches = [(inp.k_cache, inp.v_cache, inp.k_l2, inp.v_l2)]
    for _ in range(layers - 1):
        caches.append(tuple(t.clone() for t in caches[0]))
    B, Hq, D = inp.q.shape
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    s2 = torch.empty(B, b.n_kv_heads, max(cfg.topk2, 1), dtype=torch.int32, device=dev)
    s1 = torch.empty(B, b.n_kv_heads, max(b.topk, 1), dtype=torch.int32, device=dev)
    base = gsa.decode_params(B, Hq, b.n_kv_heads, D, b.n_raw, b.M, b.chunk, b.topk, b.tail, 0.0,
                             gsa.GSA_BF16 if b.dtype == "bf16" else gsa.GSA_F32,
                             gist_set=gsa.GIST_SETS[args.gist_set])
    ws = gsa.new_workspace(gsa.hier_workspace_size(gsa.hier_params(base, cfg.fanout, cfg.topk2)), dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        k, v, k2, v2 = caches[i % layers]
        gsa.gsa_decode_hier(inp.q, k, v, k2, v2, chunk=b.chunk, fanout=cfg.fanout, topk1=b.topk,
                            topk2=cfg.topk2, tail=b.tail, n_gist=b.M, out=out, lse=lse, sel2=s2,
                            sel1=s1, workspace=ws, stream=stream, gist_set=args.gist_set)

    step(0)
    torch.cuda.synchronize()
    if inp.planted2 is not None:
        assert torch.equal(s2.long(), inp.planted2), "level-2 selection differs from the planted set"
        assert torch.equal(s1.long(), inp.planted1), "level-1 selection differs from the planted set"
    nb = hier_bytes(cfg, s1.cpu().numpy() if b.topk else [], args.gist_set)
    n_marks = gsa.gsa_profile_marks()
    if n_marks == 2:   # unit_kernel over level 2 + tail, its last workgroup per unit descends
        names = ["unit_kernel (level 2 + descent)"]
        nbytes = [nb["l2"] + nb["cand"] + nb["unfold"]]
    elif n_marks == 5:   # level 2, its per-split candidates, level-1 candidates, unfold
        names = ["gist_kernel (level 2)", "cand_kernel", "gist_kernel (candidates)", "unfold_kernel"]
        nbytes = [nb["l2"], 0, nb["cand"], nb["unfold"]]
    else:
        names = ["gist_kernel (level 2)", "gist_kernel (candidates)", "unfold_kernel"][:n_marks - 1]
        nbytes = [nb["l2"], nb["cand"], nb["unfold"]][:n_marks - 1]
    ms_per_step, per = timed_steps(gsa, step, args, n_marks)
    kernels = {}
    for j, (nm, b_) in enumerate(zip(names, nbytes)):
        ms = float(per[:, j].mean())
        kernels[nm] = {"ms": ms, "alg_bytes": b_, "GB_s": b_ / (ms / 1e3) / 1e9, **pcts(per[:, j])}
    call_ms = float(per.sum(axis=1).mean())
    alg_b = sum(nb.values())
    main = max(kernels, key=lambda k: kernels[k]["ms"])
    qheads = B * Hq
    return {
        "metric": "GSA two-level decode query-heads/s + achieved HBM GB/s (1M ctx, C=16, G=16, k2=8, k1=16, bf16)",
        "value": qheads / (ms_per_step / 1e3),
        "unit": "query-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": b.dtype,
        "data": "synthetic (seeded Gaussian q/K/V, planted top-k at both levels with margin >= 0.5)",
        "config": {"workload": f"{cfg.name}: two-level GQA decode step, B={b.batch}, Hq={b.n_q_heads}, "
                               f"Hkv={b.n_kv_heads}, D={b.head_dim}, N={b.n_raw}, C={b.chunk}, "
                               f"G={cfg.fanout}, k2={cfg.topk2}, k1={b.topk}, T={b.tail}"
                               + ("" if args.gist_set == "all" else
                                  f", attention set: {GIST_SET_NAMES[args.gist_set]}"),
                   "global_batch": b.batch, "seq_len": b.n_raw, "parallelism": "none (1 GPU)",
                   "cache_layers_rotated": layers},
        "roofline": {"bound": "hbm", "achieved": alg_b / (call_ms / 1e3) / 1e9, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": alg_b / (call_ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
                     "traffic": None, "kernel": f"whole call ({n_marks - 1} launches)",
                     "alg_bytes_per_launch": alg_b, "launch_ms_mean": call_ms},
        "kernels": kernels,
    }


# --------------------------------------------------------------- prefill ---

def prefill_flops(cfg):
    """Algorithmic FLOPs: 2 * D for q.k and 2 * D for p.v over every attended
    (query head, row) pair. Per query t: the eligible gists, the k*C rows of
    its chunks outside its window (planted chunks lie outside every window)
    and the window rows."""
    t = cfg.q_start + np.arange(cfg.n_q)
    elig = np.minimum(cfg.M, t // cfg.chunk)
    win = np.minimum(cfg.window, t + 1)
    rows = elig + np.minimum(elig, cfg.topk) * cfg.chunk + win
    g = cfg.n_q_heads
    total = float(rows.sum()) * g * cfg.head_dim * 4
    gist_qk = float(elig.sum()) * g * cfg.head_dim * 2      # the selection pass' group scores
    return total, gist_qk


def cpu_baseline_prefill(inp, cfg, budget_s: float):
    import oracle
    from threadpoolctl import threadpool_limits
    g = cfg.n_q_heads // cfg.n_kv_heads
    q = inp.q.float().cpu().numpy()
    K = [inp.k_cache[j].float().cpu().numpy() for j in range(cfg.n_kv_heads)]
    V = [inp.v_cache[j].float().cpu().numpy() for j in range(cfg.n_kv_heads)]
    rng = np.random.default_rng(5)
    t_total, n = 0.0, 0
    with threadpool_limits(1):
        while t_total < budget_s and n < 100000:
            i, j = int(rng.integers(cfg.n_q)), int(rng.integers(cfg.n_kv_heads))
            t0 = time.perf_counter()
            oracle.prefill_query(q[j * g:(j + 1) * g, i], K[j], V[j], t=cfg.q_start + i,
                                 n_raw=cfg.n_raw, n_gist=cfg.M, chunk=cfg.chunk, topk=cfg.topk,
                                 window=cfg.window)
            t_total += time.perf_counter() - t0
            n += 1
    # one query position = all kv-heads
    return {"value": n / cfg.n_kv_heads / t_total, "unit": "query-positions/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} random (query, kv-head) pairs of the same workload, fp64 numpy, "
                      f"1 thread, {t_total:.1f} s"}


def run_prefill_bench(args):
    import torch
    import decode_gsa_amd as gsa
    import gsa_inputs as gi

    cfg = gi.CONFIGS[args.config]
    dev = torch.device("cuda", 0)
    log(f"[bench] generating {cfg.name} inputs ...")
    inp = gi.make_prefill(cfg, 2000 + 5, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = torch.empty(cfg.n_q_heads, cfg.n_q, cfg.head_dim, dtype=torch.float32, device=dev)
    sel = torch.empty(cfg.n_kv_heads, cfg.n_q, max(cfg.topk, 1), dtype=torch.int32, device=dev)
    p = gsa.prefill_params(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.chunk, cfg.topk,
                           cfg.window, cfg.n_raw, cfg.M, cfg.q_start, cfg.n_q)
    ws = gsa.new_workspace(gsa.prefill_workspace_size(p), dev)

    def step(i):
        gsa.gsa_prefill_blocksparse(inp.q, inp.k_cache, inp.v_cache, chunk=cfg.chunk,
                                    topk=cfg.topk, window=cfg.window, q_start=cfg.q_start,
                                    n_gist=cfg.M, out=out, sel=sel, workspace=ws, stream=stream)

    step(0)
    torch.cuda.synchronize()
    if cfg.topk > 0 and inp.planted is not None:
        blk = torch.arange(cfg.n_q, device=dev) // cfg.q_block
        assert torch.equal(sel.permute(1, 0, 2).long(), inp.planted[blk]), "selection differs"
    n_marks = 3 if cfg.topk > 0 else 2
    ms_per_step, per = timed_steps(gsa, step, args, n_marks)
    att_ms = float(per[:, -1].mean())
    total_fl, sel_fl = prefill_flops(cfg)
    achieved = total_fl / (att_ms / 1e3) / 1e12
    call_ms = float(per.sum(axis=1).mean())
    kernels = {"prefill_attend": {"ms": att_ms, "alg_flops": total_fl,
                                  "TFLOP_s": total_fl / (att_ms / 1e3) / 1e12, **pcts(per[:, -1])}}
    if cfg.topk > 0:
        sel_ms = float(per[:, 0].mean())
        kernels["prefill_select"] = {"ms": sel_ms, "alg_flops": sel_fl,
                                     "TFLOP_s": sel_fl / (sel_ms / 1e3) / 1e12, **pcts(per[:, 0])}
    res = {
        "metric": PREFILL_METRIC,
        "value": cfg.n_q / (ms_per_step / 1e3),
        "unit": "query-positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian q/K/V, planted top-k per 64-query block)",
        "config": {"workload": f"{cfg.name}: causal block-sparse prefill of positions "
                               f"[{cfg.q_start}, {cfg.n_raw}), Hq={cfg.n_q_heads}, "
                               f"Hkv={cfg.n_kv_heads}, D={cfg.head_dim}, N={cfg.n_raw}, "
                               f"C={cfg.chunk}, k={cfg.topk}, W={cfg.window}, bf16",
                   "seq_len": cfg.n_raw, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / BF16_MFMA_PEAK_TFLOPS,
                     "traffic": measured_traffic(f"prefill_attend/{cfg.name}", source_sha("gsa_prefill.hip")),
                     "kernel": "prefill_attend", "alg_flops_per_launch": total_fl,
                     "launch_ms_mean": att_ms},
        "call": {"ms_mean": call_ms, "TFLOP_s": total_fl / (call_ms / 1e3) / 1e12},
        "kernels": kernels,
        "source_sha": source_sha("gsa_prefill.hip"),
    }
    if not args.no_cpu:
        log("[bench] timing the CPU oracle ...")
        res["cpu_baseline"] = cpu_baseline_prefill(inp, cfg, args.cpu_seconds)
    return res


# -------------------------------------------------------- variable length ---

def run_varlen_bench(args):
    import torch
    import decode_gsa_amd as gsa
    import gsa_inputs as gi
    import oracle

    cfg = gi.CONFIGS[args.config]
    dev = torch.device("cuda", 0)
    B, Hq, Hkv, D, C, k, T = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.chunk, cfg.topk, cfg.tail
    n, m = gi.varlen_lengths(B, cfg.n_min, cfg.n_max, C, 2000 + 9)
    N, M = max(n), max(m)
    cap = N + M
    log(f"[bench] generating {cfg.name} inputs (lengths {min(n)}..{N}) ...")
    q, kc, vc, _, _ = gi.make_levels(B, Hq, Hkv, D, N, M, C, 2, 2, 2000 + 9, device=dev, values="gauss")
    sn = torch.tensor(n, dtype=torch.int32, device=dev)
    sm = torch.tensor(m, dtype=torch.int32, device=dev)
    P = cfg.page_chunks
    p = gsa.decode_params(B, Hq, Hkv, D, N, M, C, k, T, row_capacity=cap)
    gsa.check_seq_lens(p, n, m)
    if P:
        # the caches in shuffled pages of P chunk slots; the dense copies go
        kp, vp, table_h = gi.to_pages(kc, vc, [a + b for a, b in zip(n, m)], P, C, 2000 + 10)
        del kc, vc
        torch.cuda.empty_cache()
        pp = gsa.paged_params(p, P, table_h.shape[1], kp.shape[0], 0)
        pp.base.row_capacity = 0
        gsa.check_pages(pp, table_h, n, m)
        table = torch.from_numpy(table_h).to(dev)
        ws = gsa.new_workspace(gsa.paged_workspace_size(pp), dev)
    else:
        ws = gsa.new_workspace(gsa.decode_workspace_size(p), dev)
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    sel = torch.empty(B, Hkv, k, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        if P:
            gsa.gsa_decode_paged(q, kp, vp, block_table=table, seq_n_raw=sn, seq_n_gist=sm, n_raw=N, n_gist=M,
                                 chunk=C, topk=k, tail=T, page_chunks=P, out=out, lse=lse, sel_idx=sel,
                                 workspace=ws, stream=stream)
        else:
            gsa.gsa_decode_varlen(q, kc, vc, seq_n_raw=sn, seq_n_gist=sm, n_raw=N, n_gist=M, chunk=C, topk=k,
                                  tail=T, out=out, lse=lse, sel_idx=sel, workspace=ws, stream=stream)

    def unit_rows(b, j):
        """Host fp32 copies of (q, K, V) of one unit, K/V gathered through the
        pages for a paged cache (the oracle's page gather)."""
        R = n[b] + m[b]
        qh = q[b, j * g:(j + 1) * g].float().cpu().numpy()
        if P:
            pages = [int(x) for x in table_h[b]]
            K = oracle.gather_pages(kp[:, j].float().cpu().numpy(), pages, page_chunks=P, chunk=C, n_rows=R)
            V = oracle.gather_pages(vp[:, j].float().cpu().numpy(), pages, page_chunks=P, chunk=C, n_rows=R)
            return qh, K, V
        return qh, kc[b, j, :R].float().cpu().numpy(), vc[b, j, :R].float().cpu().numpy()

    step(0)
    torch.cuda.synchronize()
    g = Hq // Hkv
    for b, j in ((int(np.argmin(n)), 0), (int(np.argmax(n)), Hkv - 1)):
        qh, Kh, Vh = unit_rows(b, j)
        r = oracle.decode_unit(qh, Kh, Vh, n_raw=n[b], n_gist=m[b], chunk=C, topk=k, tail=T)
        got = out[b, j * g:(j + 1) * g].double().cpu().numpy()
        rms = float(np.sqrt(np.mean(r["out"] ** 2)))
        if not np.array_equal(sel[b, j].cpu().numpy(), r["sel"]) or float(np.abs(got - r["out"]).max()) > 2e-3 * rms:
            raise SystemExit(f"varlen: sequence {b} kv-head {j} differs from the oracle")
    ms_per_step, per = timed_steps(gsa, step, args, 2)
    k_ms = float(per[:, 0].mean())
    row = 2 * D * 2
    sel_np = sel.cpu().numpy()
    raw_sel = sum(tail_free_rows(sel_np[b], n[b], T, C) for b in range(B))
    nb = Hkv * sum((mb + T) for mb in m) * row + raw_sel * row + B * Hq * D * 2 + B * Hq * (D + 1) * 4 + B * Hkv * k * 4
    achieved = nb / (k_ms / 1e3) / 1e9
    mean_n = float(np.mean(n))
    res = {
        "metric": PAGED_METRIC if P else VARLEN_METRIC,
        "value": B * Hq / (ms_per_step / 1e3),
        "unit": "query-heads/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian q/K/V, seeded lengths)",
        "config": {"workload": f"{cfg.name}: decode step of {B} sequences of {min(n)}..{N} tokens (mean "
                               f"{mean_n:.0f}), Hq={Hq}, Hkv={Hkv}, D={D}, C={C}, k={k}, T={T}, bf16 cache"
                               + (f" in shuffled pages of {P} chunk slots ({P * (C + 1)} rows)" if P else ""),
                   "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(f"unit_kernel/{cfg.name}", source_sha("gsa_decode.hip", "gsa_device.hpp")),
                     "kernel": "unit_kernel (VARLEN, PAGED)" if P else "unit_kernel (VARLEN)",
                     "alg_bytes_per_launch": nb, "launch_ms_mean": k_ms,
                     "longest_share": float(max(n)) / mean_n},
        "kernels": {"unit_kernel": {"ms": k_ms, "alg_bytes": nb, "GB_s": achieved, **pcts(per[:, 0])}},
        "source_sha": source_sha("gsa_decode.hip", "gsa_device.hpp"),
    }
    if not args.no_cpu:
        log("[bench] timing the CPU oracle ...")
        from threadpoolctl import threadpool_limits
        rng = np.random.default_rng(9)
        t_total, cnt, host = 0.0, 0, {}
        with threadpool_limits(1):
            while t_total < args.cpu_seconds and cnt < 100000:
                b, j = int(rng.integers(B)), int(rng.integers(Hkv))
                if (b, j) not in host:
                    host[(b, j)] = unit_rows(b, j)
                qh, Kh, Vh = host[(b, j)]
                t0 = time.perf_counter()
                oracle.decode_unit(qh, Kh, Vh, n_raw=n[b], n_gist=m[b], chunk=C, topk=k, tail=T)
                t_total += time.perf_counter() - t0
                cnt += 1
        res["cpu_baseline"] = {"value": cnt * g / t_total, "unit": "query-heads/s", "cores": 1, "kind": "oracle",
                               "sample": f"{cnt} random (sequence, kv-head) units of the same batch, fp64 numpy, "
                                         f"1 thread, {t_total:.1f} s"}
    return res


# ------------------------------------------------------------ cache build ---

def gist_flops(cfg):
    """Algorithmic FLOPs of the gist tokens: 2 * D for q.k and 2 * D for p.v
    per (query head, row); gist m attends its C raw rows and m gists."""
    rows = cfg.M * cfg.chunk + cfg.M * (cfg.M - 1) // 2
    return float(rows) * cfg.n_q_heads * cfg.head_dim * 4


def cpu_baseline_gist(q, k, v, cfg, budget_s: float):
    import oracle
    from threadpoolctl import threadpool_limits
    g = cfg.n_q_heads // cfg.n_kv_heads
    qn = q.float().cpu().numpy()
    K = [k[j].float().cpu().numpy() for j in range(cfg.n_kv_heads)]
    V = [v[j].float().cpu().numpy() for j in range(cfg.n_kv_heads)]
    rng = np.random.default_rng(6)
    t_total, n, rows = 0.0, 0, 0
    with threadpool_limits(1):
        while t_total < budget_s and n < 100000:
            m, j = int(rng.integers(cfg.M)), int(rng.integers(cfg.n_kv_heads))
            t0 = time.perf_counter()
            oracle.gist_query(qn[j * g:(j + 1) * g, m], K[j], V[j], m=m, n_raw=cfg.n_raw, n_gist=cfg.M,
                              chunk=cfg.chunk)
            t_total += time.perf_counter() - t0
            n += 1
            rows += cfg.chunk + m
    # scaled to whole gist tokens (all kv-heads) of the average length, then
    # to prompt tokens (C per gist)
    mean_rows = cfg.chunk + (cfg.M - 1) / 2
    per_token_s = t_total / n * cfg.n_kv_heads * (mean_rows / (rows / n))
    return {"value": cfg.chunk / per_token_s, "unit": "prompt-tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} random (gist token, kv-head) pairs of the same prompt, fp64 numpy, 1 thread, "
                      f"{t_total:.1f} s; the append is not timed on the CPU"}


def run_gist_bench(args):
    import torch
    import decode_gsa_amd as gsa
    import gsa_inputs as gi
    import oracle

    cfg = gi.CONFIGS[args.config]
    dev = torch.device("cuda", 0)
    C, M, N, D = cfg.chunk, cfg.M, cfg.n_raw, cfg.head_dim
    log(f"[bench] generating {cfg.name} inputs ...")
    q, k, v = gi.make_gist(cfg.n_q_heads, cfg.n_kv_heads, D, N, M, M, 2000 + 7, device=dev)
    raw_rows = torch.tensor([gi.raw_row(p, C, M) for p in range(N)], device=dev)
    gist_rows = torch.arange(M, device=dev) * (C + 1) + C
    k_raw, v_raw = k[:, raw_rows].contiguous(), v[:, raw_rows].contiguous()
    k_gist, v_gist = k[:, gist_rows].contiguous(), v[:, gist_rows].contiguous()
    kc, vc = torch.zeros_like(k), torch.zeros_like(v)
    out = torch.empty(cfg.n_q_heads, M, D, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        gsa.gsa_cache_append(kc, vc, chunk=C, n_raw=0, n_gist=0, k_raw=k_raw, v_raw=v_raw, k_gist=k_gist,
                             v_gist=v_gist, stream=stream)
        gsa.gsa_gist_prefill(q, kc, vc, chunk=C, m_start=0, n_gist=M, out=out, stream=stream)

    step(0)
    torch.cuda.synchronize()
    assert torch.equal(kc, k) and torch.equal(vc, v), "appended cache differs from the interleaved layout"
    g = cfg.n_q_heads // cfg.n_kv_heads
    for m, j in ((0, 0), (M // 2 + 3, 5), (M - 1, cfg.n_kv_heads - 1)):
        r = oracle.gist_query(q[j * g:(j + 1) * g, m].float().cpu().numpy(), k[j].float().cpu().numpy(),
                              v[j].float().cpu().numpy(), m=m, n_raw=N, n_gist=M, chunk=C)
        got = out[j * g:(j + 1) * g, m].double().cpu().numpy()
        rms = float(np.sqrt(np.mean(r["out"] ** 2)))
        assert float(np.abs(got - r["out"]).max()) <= 2e-3 * rms, f"gist token {m} differs from the oracle"
    # wall clock of uninstrumented steps, then per-call kernel times: the
    # event hook is armed per library call, so each call gets its own pair
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = 1e3 * (time.perf_counter() - t0) / args.steps
    ev = HipEvents(4 * args.steps)
    try:
        for i in range(args.steps):
            gsa.gsa_profile_events(ev.ev[4 * i:4 * i + 2])
            gsa.gsa_cache_append(kc, vc, chunk=C, n_raw=0, n_gist=0, k_raw=k_raw, v_raw=v_raw,
                                 k_gist=k_gist, v_gist=v_gist, stream=stream)
            gsa.gsa_profile_events(ev.ev[4 * i + 2:4 * i + 4])
            gsa.gsa_gist_prefill(q, kc, vc, chunk=C, m_start=0, n_gist=M, out=out, stream=stream)
            gsa.gsa_profile_events([])
        torch.cuda.synchronize()
        app_per = np.array([ev.ms(4 * i, 4 * i + 1) for i in range(args.steps)])
        att_per = np.array([ev.ms(4 * i + 2, 4 * i + 3) for i in range(args.steps)])
    finally:
        gsa.gsa_profile_events([])
        ev.close()
    app_ms = float(app_per.mean())
    att_ms = float(att_per.mean())
    fl = gist_flops(cfg)
    achieved = fl / (att_ms / 1e3) / 1e12
    row_b = D * 2
    app_bytes = 2.0 * cfg.n_kv_heads * (N + M) * row_b * 2     # K and V rows read and written
    res = {
        "metric": GIST_METRIC,
        "value": N / (ms_per_step / 1e3),
        "unit": "prompt-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian q/K/V rows)",
        "config": {"workload": f"{cfg.name}: cache build of a {N}-token prompt, append of {N} raw + {M} "
                               f"gist rows then attention of its {M} gist tokens, Hq={cfg.n_q_heads}, "
                               f"Hkv={cfg.n_kv_heads}, D={D}, C={C}, bf16",
                   "seq_len": N, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / BF16_MFMA_PEAK_TFLOPS,
                     "traffic": measured_traffic(f"prefill_attend/{cfg.name}", source_sha("gsa_prefill.hip")),
                     "kernel": "prefill_attend (gist queries)", "alg_flops_per_launch": fl,
                     "launch_ms_mean": att_ms},
        "kernels": {"prefill_attend": {"ms": att_ms, "alg_flops": fl, "TFLOP_s": achieved, **pcts(att_per)},
                    "cache_append": {"ms": app_ms, "alg_bytes": app_bytes,
                                     "GB_s": app_bytes / (app_ms / 1e3) / 1e9, **pcts(app_per)}},
        "source_sha": source_sha("gsa_prefill.hip", "gsa_cache.hip"),
    }
    if not args.no_cpu:
        log("[bench] timing the CPU oracle ...")
        res["cpu_baseline"] = cpu_baseline_gist(q, k, v, cfg, args.cpu_seconds)
    return res


# --------------------------------------------------------------- scaling ---

SCALING_N = [1 << 15, 1 << 17, 1 << 19, 1 << 21, 1 << 23, 1 << 24]


def scaling_levels(M: int, G: int = 16, top: int = 256):
    """Level sizes [M_1, ..., M_L]: levels are added until the top holds at
    most `top` gists (at least two levels)."""
    sizes = [M, M // G]
    while sizes[-1] > top:
        sizes.append(sizes[-1] // G)
    return sizes


def tail_free_rows(sel1, n_raw: int, tail: int, chunk: int) -> int:
    """Raw rows of the chosen chunks that the tail does not already hold."""
    tail0 = n_raw - tail
    return int(sum(max(0, min(chunk, tail0 - int(m) * chunk)) for m in np.asarray(sel1).ravel()))


def run_scaling(args):
    import torch
    import decode_gsa_amd as gsa
    import gsa_inputs as gi
    import oracle

    dev = torch.device("cuda", 0)
    B, Hq, Hkv, D, C, T, G = 1, 32, 8, 128, 16, 64, 16
    units, row = B * Hkv, 2 * D * 2
    k1, k_mid, k_top = 16, 8, 4
    ns = [n for n in SCALING_N if args.scaling_min <= n <= args.scaling_max]
    for N in ns:
        M = N // C
        sizes = scaling_levels(M, G)
        L = len(sizes)
        topks = [k1] + [k_mid] * (L - 2) + [k_top]
        cache_b = units * (N + M) * row
        step_b = units * (M + T) * row
        copies = int(max(1, min(16, math.ceil(2e9 / step_b), 100e9 // cache_b)))
        log(f"[scaling] N={N}: levels {sizes}, {copies} cache copies ...")
        sets = [gi.make_levels(B, Hq, Hkv, D, N, M, C, G, L, 7000 + N % 997 + i, device=dev, values="gauss")
                for i in range(copies)]
        base = gsa.decode_params(B, Hq, Hkv, D, N, M, C, k1, T)
        ws = gsa.new_workspace(max(gsa.decode_workspace_size(base),
                                   gsa.hier_workspace_size(gsa.hier_params(base, G, k_mid)),
                                   gsa.levels_workspace_size(gsa.levels_params(base, G, topks[1:]))), dev)
        stream = torch.cuda.current_stream(dev)
        # unit (0, 0) on the host for the oracle spot checks
        x0 = sets[0]
        g = Hq // Hkv
        qn = x0[0][0, :g].float().cpu().numpy()
        Kn, Vn = x0[1][0, 0].float().cpu().numpy(), x0[2][0, 0].float().cpu().numpy()
        upn = [(a[0, 0].float().cpu().numpy(), b[0, 0].float().cpu().numpy()) for a, b in zip(x0[3], x0[4])]

        def flat(x):
            return gsa.gsa_decode(x[0], x[1], x[2], chunk=C, topk=k1, tail=T, n_gist=M, workspace=ws,
                                  stream=stream)

        def two(x):
            return gsa.gsa_decode_hier(x[0], x[1], x[2], x[3][0], x[4][0], chunk=C, fanout=G, topk1=k1,
                                       topk2=k_mid, tail=T, n_gist=M, workspace=ws, stream=stream)

        def many(x):
            return gsa.gsa_decode_levels(x[0], x[1], x[2], x[3], x[4], chunk=C, fanout=G, topks=topks, tail=T,
                                         n_gist=M, workspace=ws, stream=stream)

        for name, fn in (("single-level", flat), ("two-level", two), (f"{L}-level", many)):
            if name == "two-level" and L == 2:
                continue
            res0 = fn(sets[0])
            torch.cuda.synchronize()
            if name == "single-level":
                sel1 = res0[2]
                nb = units * (M + T) * row
            elif name == "two-level":
                sel1 = res0[3]
                n_cand = k_mid * G + (M - (M // G) * G)
                nb = units * ((M // G) + T + n_cand) * row
            else:
                sel1 = res0[2][0]
                n_items = [k_mid * G + (sizes[l] - sizes[l + 1] * G) if l + 2 < L else
                           k_top * G + (sizes[l] - sizes[l + 1] * G) for l in range(L - 1)]
                nb = units * (sizes[-1] + T + sum(n_items)) * row
            nb += tail_free_rows(to_cpu(sel1), N, T, C) * row
            # oracle spot check on unit (0, 0)
            if name == "single-level":
                r = oracle.decode_unit(qn, Kn, Vn, n_raw=N, n_gist=M, chunk=C, topk=k1, tail=T)
                ok_sel = np.array_equal(to_cpu(sel1)[0, 0], r["sel"])
            elif name == "two-level":
                r = oracle.decode_hier_unit(qn, Kn, Vn, upn[0][0], upn[0][1], n_raw=N, n_gist=M, chunk=C,
                                            fanout=G, topk1=k1, topk2=k_mid, tail=T)
                ok_sel = np.array_equal(to_cpu(sel1)[0, 0], r["sel1"])
            else:
                r = oracle.decode_levels_unit(qn, Kn, Vn, upn, n_raw=N, n_gist=M, chunk=C, fanout=G, topks=topks,
                                              tail=T)
                ok_sel = np.array_equal(to_cpu(sel1)[0, 0], r["sels"][0])
            got = res0[0][0, :g].double().cpu().numpy()
            rms = float(np.sqrt(np.mean(r["out"] ** 2)))
            if not ok_sel or float(np.abs(got - r["out"]).max()) > 2e-3 * rms:
                raise SystemExit(f"[scaling] N={N} {name}: differs from the oracle")
            for i in range(3):
                fn(sets[i % copies])
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                fn(sets[i % copies])
            torch.cuda.synchronize()
            ms = 1e3 * (time.perf_counter() - t0) / args.steps
            # device time of a call: the library's event hook, first kernel's
            # start to last kernel's end
            n_marks = gsa.gsa_profile_marks()
            ev = HipEvents(n_marks * args.steps)
            try:
                for i in range(args.steps):
                    gsa.gsa_profile_events(ev.ev[i * n_marks:(i + 1) * n_marks])
                    fn(sets[i % copies])
                gsa.gsa_profile_events([])
                torch.cuda.synchronize()
                dev_ms = float(np.mean([ev.ms(i * n_marks, (i + 1) * n_marks - 1) for i in range(args.steps)]))
                # per launch: launch 0 from the call's start, launch j > 0 from the end of launch j - 1
                per_launch = [float(np.mean([ev.ms(i * n_marks + j, i * n_marks + j + 1) for i in range(args.steps)]))
                              for j in range(n_marks - 1)]
            finally:
                gsa.gsa_profile_events([])
                ev.close()
            lv, tk = {"single-level": ([M], [k1]), "two-level": ([M, M // G], [k1, k_mid])}.get(name, (sizes, topks))
            line = {"context": N, "variant": name, "levels": lv, "topks": tk,
                    "ms_per_step": ms, "device_ms_per_call": dev_ms, "launches": n_marks - 1,
                    "launch_ms": per_launch,
                    "alg_bytes_per_step": nb, "GB_s": nb / (ms / 1e3) / 1e9,
                    "cache_copies": copies, "oracle_checked_unit": [0, 0]}
            print(json.dumps(line), flush=True)
        del sets, x0, Kn, Vn, upn
        torch.cuda.empty_cache()


def to_cpu(t):
    return t.cpu().numpy()


def hbm_stream_rates(reps: int = 8) -> dict:
    """Bandwidth of a plain torch device copy of 1 GiB (bytes read + written),
    reported next to the 8 TB/s specification as what a generic streaming
    kernel reaches on this machine."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.copy_(a)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * n / (e0.elapsed_time(e1) / reps / 1e3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return {"torch_copy_1GiB_GB_s": gbs}


def run_phase_stamps(args):
    """Phase edges of the unit-path decode kernels, read from the diagnostic
    build libgsa_stamps.so (`python -m decode_gsa_amd.build --stamps`): per
    workgroup, thread 0 stamps the chip's 100 MHz clock at its phase edges
    (the slots are listed with the stamps in gsa_decode.hip). Prints one JSON
    line: for each stamped slot, the median and the maximum over the
    workgroups that stamped it of the time since the call's first start (us),
    averaged over the calls; with one workgroup per unit also the phase
    lengths and the per-XCD median end of the streaming phase (workgroup i
    runs on XCD i mod 8)."""
    import torch
    import decode_gsa_amd as gsa
    import gsa_inputs as gi
    from decode_gsa_amd import build as gb
    if not os.path.exists(gb.STAMPS_LIB):
        raise SystemExit("build the diagnostic library first: python -m decode_gsa_amd.build --stamps")
    gsa.LIB_PATH = gb.STAMPS_LIB
    L = gsa.lib()
    L.gsa_debug_phase_stamps.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    L.gsa_debug_phase_stamps.restype = ctypes.c_int
    cfg = gi.CONFIGS[args.config]
    dev = torch.device("cuda", 0)
    slots, max_wg = 16, 32768
    buf = np.zeros(max_wg * slots, dtype=np.uint64)
    if hasattr(cfg, "fanout"):
        b = cfg.base
        inp = gi.make_hier(cfg, 1000 + 4, device=dev)
        layers = [(inp.k_cache, inp.v_cache, inp.k_l2, inp.v_l2)] + [
            tuple(t.clone() for t in (inp.k_cache, inp.v_cache, inp.k_l2, inp.v_l2)) for _ in range(2)]

        def call(x):
            gsa.gsa_decode_hier(inp.q, *x, chunk=b.chunk, fanout=cfg.fanout, topk1=b.topk, topk2=cfg.topk2,
                                tail=b.tail, n_gist=b.M)
    else:
        inp = gi.make_decode(cfg, 1000 + 2, device=dev)
        layers = [(inp.k_cache, inp.v_cache)] + [(inp.k_cache.clone(), inp.v_cache.clone()) for _ in range(4)]

        def call(x):
            gsa.gsa_decode(inp.q, x[0], x[1], chunk=cfg.chunk, topk=cfg.topk, tail=cfg.tail, n_gist=cfg.M)
    rows = []
    L.gsa_debug_phase_stamps(buf.ctypes.data, buf.nbytes)   # clears the stamps
    for rep in range(args.warmup + args.steps):
        call(layers[rep % len(layers)])
        torch.cuda.synchronize()
        marks = gsa.gsa_profile_marks()
        if L.gsa_debug_phase_stamps(buf.ctypes.data, buf.nbytes) != 0:
            raise SystemExit("reading the stamps failed")
        if rep >= args.warmup:
            rows.append(buf.reshape(max_wg, slots).astype(np.int64).copy())
    res = {"metric": "decode kernel phase edges (us since the call's first workgroup start, 100 MHz clock)",
           "config": cfg.name, "calls": len(rows), "launches": marks - 1}
    for sl in range(slots):
        med, mx, n = [], [], 0
        for r in rows:
            t0 = r[:, 0][r[:, 0] > 0].min()
            v = r[:, sl][r[:, sl] > 0]
            if v.size == 0:
                continue
            d = (v - t0) / 100.0
            med.append(float(np.median(d)))
            mx.append(float(d.max()))
            n = v.size
        if med:
            res[f"slot {sl}"] = {"median": round(float(np.mean(med)), 2), "max": round(float(np.mean(mx)), 2),
                                 "workgroups": n}
    if marks == 2 and not hasattr(cfg, "fanout") and all(f"slot {i}" in res for i in range(5)):
        phases = {"stream (gists + tail)": (0, 1), "selection": (1, 2), "unfold": (2, 3),
                  "merge + output": (3, 4)}
        units = cfg.batch * cfg.n_kv_heads
        for name, (a, b2) in phases.items():
            d = np.array([(r[:units, b2] - r[:units, a]) / 100.0 for r in rows])
            res[name] = {"median": float(np.median(d)), "max_mean": float(d.max(axis=1).mean())}
        res["stream end, median per XCD"] = [
            float(np.mean([np.median((r[x:units:8, 1] - r[:units, 0].min()) / 100.0) for r in rows]))
            for x in range(8)]
    print(json.dumps(res), flush=True)


def run_copy_calibration():
    """A plain device copy of a known size (for scaling FETCH_SIZE / WRITE_SIZE
    counters: run under rocprofv3 --pmc and compare with the bytes moved)."""
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="gqa_32k")
    ap.add_argument("--layers", type=int, default=0, help="cache copies rotated per step")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--phase-stamps", action="store_true",
                    help="phase edges of the decode kernel (diagnostic library libgsa_stamps.so)")
    ap.add_argument("--scaling", action="store_true", help="decode time and bytes per step vs context length")
    ap.add_argument("--scaling-max", type=int, default=1 << 24)
    ap.add_argument("--scaling-min", type=int, default=0)
    ap.add_argument("--gist-set", default="all", choices=["all", "selected", "none"],
                    help="decode attention-set rule (slide 17 variants)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(decode units and prefill query blocks are independent; the sharding plan is "
              "written up with the design).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        run_copy_calibration()
        return
    if args.phase_stamps:
        run_phase_stamps(args)
        return
    if args.scaling:
        run_scaling(args)
        return
    import gsa_inputs as gi
    cfg = gi.CONFIGS[args.config]
    if isinstance(cfg, gi.DecodeConfig):
        res = run_decode_bench(args)
    elif isinstance(cfg, gi.PrefillConfig):
        res = run_prefill_bench(args)
    elif isinstance(cfg, gi.HierConfig):
        res = run_hier_bench(args)
    elif isinstance(cfg, gi.GistConfig):
        res = run_gist_bench(args)
    elif isinstance(cfg, gi.VarlenConfig):
        res = run_varlen_bench(args)
    else:
        raise SystemExit(f"--config {args.config}: no benchmark for this workload yet")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
