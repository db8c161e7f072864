#!/usr/bin/env python3
"""Sparse-decode benchmark on one MI355X.

A step is one decode query for every sequence of the batch through
cobs_sparse_attn_decode: block scoring + top-k, then the selected-block,
sliding-window and compressed branches with the gated combine.  Inputs are
seeded synthetic tensors resident in HBM before timing; the per-block summaries
are built once per prefix (outside the timed region), as in decoding.

Each timed step reads a different replica of every input (K, V, summaries,
pooled tokens, Q, gates), with enough replicas that a step's bytes are not
served from the 256 MB last-level cache by an earlier step; steps are issued as
HIP graph replays so host launch overhead does not bound the GPU.

Prints one JSON line (last line of stdout).  --gpus > 1 is refused: the library
runs on one GPU.
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

HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 * 2 ** 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w, lens, sel, alpha):
    """Bytes the method must move per decode step (per kernel), from the
    selection actually made: SLC blocks, the window minus its overlap with SLC,
    the pooled tokens, summaries of the candidate blocks, Q, gates, output."""
    es = 2 if w.dtype == "bf16" else 4
    d, G = w.head_dim, w.group
    vlen = -(-w.subspace // 32) * 32 if w.subspace else d      # length of a stored rank-r vector
    if w.so_kind == "lowrank_fp4":           # bf16 mean + one compressed record per block
        rec = -(-w.rank * (vlen // 2 + vlen // 32) // 16) * 16
        sum_bytes_per_block = d * 2 + (0 if alpha == 0 else rec)
    elif w.so_kind == "lowrank":
        sum_bytes_per_block = d * 4 + (0 if alpha == 0 else w.rank * vlen * 4)
    else:
        sum_bytes_per_block = d * 4 * (1 if alpha == 0 else 2)
    attn = sel_b = 0
    for b in range(w.batch):
        L = int(lens[b])
        nb = -(-L // 64)
        nc = (L - 32) // 16 + 1 if (w.cmp_len and L >= 32) else 0
        win = set(range(max(0, L - w.window), L)) if w.window else set()
        for h in range(w.n_kv_heads):
            slc = set()
            for blk in sel[b, h]:
                if blk >= 0:
                    slc.update(range(64 * blk, min(64 * blk + 64, L)))
            attn += (len(slc) + len(win - slc) + nc) * d * 2 * es
            sel_b += nb * sum_bytes_per_block
    q = w.batch * w.n_q_heads * d * es
    attn += q + w.batch * w.n_q_heads * (3 * 4 + d * 4) + sel.size * 4
    sel_b += q + sel.size * 4
    return attn, sel_b


def calibrated_subspace(w, g):
    """Query subspaces [H_kv][s][d] computed on the GPU from the workload's calibration
    queries (cobs_query_subspace), or None when the workload has no subspace."""
    if not w.subspace:
        return None
    from block_sparse_long_compressed_amd import binding as B
    from block_sparse_long_compressed_amd import runtime as U
    return B.cobs_query_subspace(U.params_for(w), g["Qcal"], w.subspace)


def counter_traffic(workload, alpha=None):
    """HBM bytes per launch of the decode kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (copy-calibrated), or None when there is no
    summary for this workload, the kernel sources changed since it was taken, or
    alpha is not the workload's own (the counters were taken at that alpha)."""
    from block_sparse_long_compressed_amd import synth
    if alpha is not None and workload in synth.WORKLOADS and alpha != synth.WORKLOADS[workload].alpha:
        return None
    import hashlib
    path = os.path.join(ROOT, "profiles", f"k_decode_{workload}_hbm_bytes.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    try:
        data = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (IndexError, ValueError):
        return None
    h = hashlib.sha256()
    for f in data.get("source_files", []):
        path_f = os.path.join(ROOT, f)
        if not os.path.exists(path_f):
            return None
        h.update(open(path_f, "rb").read())
    if h.hexdigest() != data.get("source_sha256"):
        return None
    return data.get("traffic_bytes_per_launch")


def dense_bytes(w, lens):
    """Bytes a dense decode step reads for the same queries: every key and value of
    every (sequence, kv-head), plus the same Q, gates and output traffic."""
    es = 2 if w.dtype == "bf16" else 4
    kv = int(np.asarray(lens, dtype=np.int64).sum()) * w.n_kv_heads * w.head_dim * 2 * es
    return kv + w.batch * w.n_q_heads * (w.head_dim * es + 3 * 4 + w.head_dim * 4)


def _cpu_worker(w, x, units, seconds, ready, start, results):
    """One host core of the CPU baseline: prebuild the oracle's summaries of its
    (sequence, kv-head) units (untimed, as on the GPU side), then run whole
    group queries round-robin over them until `seconds` have passed."""
    from threadpoolctl import threadpool_limits
    from oracle import cobs_oracle as O
    p = O.params_of(w)
    G = w.group
    with threadpool_limits(limits=1):
        prepared = []
        for s, h in units:
            L = int(x["lens"][s])
            keys = x["K"][s, h, :L].astype(np.float64)
            vals = x["V"][s, h, :L].astype(np.float64)
            qg = x["Q"][s, 0, h * G:(h + 1) * G].astype(np.float64)
            gt = x["gates"][s, 0, h * G:(h + 1) * G].astype(np.float64) if x["gates"] is not None else None
            prepared.append((qg, keys, vals, L, gt) + tuple(O.build_unit(p, keys, vals, L)))
        ready.put(1)
        start.wait()
        done = 0
        t0 = time.perf_counter()
        while True:
            qg, keys, vals, L, gt, summ, kc, vc = prepared[done % len(prepared)]
            O.query_group(p, qg, keys, vals, L, L - 1, summ, kc, vc, gt)
            done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    results.put((done, el))


class CpuBaseline:
    """The fp64 oracle timed on the host cores: one forked process per core, each
    owning a few (sequence, kv-head) units of the workload.  The processes are forked
    before the GPU is touched and prebuild their summaries while the GPU part runs;
    the timed region starts with finish()."""

    def __init__(self, w, x, seconds):
        import multiprocessing as mp
        self.w, self.seconds = w, seconds
        self.cores = max(1, min(16, len(os.sched_getaffinity(0))))   # one GPU's share of host cores
        nseq = min(w.batch, -(-self.cores // w.n_kv_heads))
        units = [(s, h) for s in range(nseq) for h in range(w.n_kv_heads)]
        self.cores = min(self.cores, len(units))
        self.seqs = list(range(nseq))
        ctx = mp.get_context("fork")
        self.ready, self.results, self.start = ctx.Queue(), ctx.Queue(), ctx.Event()
        self.procs = [ctx.Process(target=_cpu_worker, args=(w, x, units[i::self.cores], seconds, self.ready,
                                                            self.start, self.results), daemon=True)
                      for i in range(self.cores)]
        for pr in self.procs:
            pr.start()

    def finish(self):
        for _ in self.procs:
            self.ready.get()
        self.start.set()
        res = [self.results.get() for _ in self.procs]
        for pr in self.procs:
            pr.join()
        group_queries = sum(r[0] for r in res)
        el = max(r[1] for r in res)
        w = self.w
        return {"value": group_queries / w.n_kv_heads / el, "unit": "queries/s", "cores": self.cores,
                "kind": "oracle",
                "sample": f"{group_queries} kv-head group queries (a query = all {w.n_kv_heads} groups of one "
                          f"sequence) over sequences {self.seqs} of {w.name}, {self.cores} processes of one "
                          f"BLAS thread each for {el:.1f} s, summaries prebuilt"}


def time_decode(w, x, g0, P, alpha, steps, warmup, replicas=0, eager=False, attention_only=True):
    """Time one decode step (one launch of k_decode) on the uploaded batch g0: graph
    replays over R input replicas, HIP events on the launch stream.  Returns a dict
    with the step time and the algorithmic bytes of the selection actually made."""
    import torch
    from block_sparse_long_compressed_amd import binding as B
    from block_sparse_long_compressed_amd import runtime as U
    p = U.params_for(w, alpha=alpha, P=P)
    s0 = U.build(p, g0)
    torch.cuda.synchronize()
    # one untimed step to get the selection for the byte model
    out0, sel0 = U.decode(p, g0, s0)
    attn_bytes, sel_bytes = algorithmic_bytes(w, x["lens"], sel0, alpha)
    step_bytes = attn_bytes + sel_bytes
    R = replicas or max(3, math.ceil(2 * MALL_BYTES / step_bytes))
    reps = []
    for r in range(R):
        g = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in g0.items()} if r else g0
        s = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in s0.items()} if r else s0
        ws = B.alloc_workspace(p, w.batch, w.max_len)
        out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
        sel = torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
        reps.append((g, s, ws, out, sel))
    torch.cuda.synchronize()

    def step(i, with_sel_in=False):
        g, s, ws, out, sel = reps[i % R]
        if with_sel_in:
            B.cobs_sparse_attn_decode(p, g["lens"], g["Q"], g["K"], g["V"], s["mu"], s["so"], s["kc"], s["vc"],
                                      g["gates"], out, ws, sel_in=sel)
        else:
            B.cobs_sparse_attn_decode(p, g["lens"], g["Q"], g["K"], g["V"], s["mu"], s["so"], s["kc"], s["vc"],
                                      g["gates"], out, ws, sel_out=sel)

    def capture(fn_list):
        graph = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            for f in fn_list:          # warm the allocator-free path once outside capture
                f()
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            for f in fn_list:
                f()
        torch.cuda.synchronize()
        return graph

    full = capture([lambda i=i: step(i) for i in range(R)])
    singles = [capture([lambda i=i: step(i)]) for i in range(R)]

    def run_steps(n, with_sel_in=False, graph=None):
        if eager:
            for i in range(n):
                step(i, with_sel_in)
            return
        for _ in range(n // R):
            (graph or full).replay()
        for i in range(n % R):
            singles[i].replay()

    run_steps(warmup)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    run_steps(steps)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    res = {"us_per_step": us, "host_wall_us_per_step": wall / steps * 1e6, "step_bytes": step_bytes,
           "attn_bytes": attn_bytes, "replicas": R, "sel0": sel0}
    if attention_only:
        # the same kernel with the caller's selection (attention roles only), for reference
        attn = capture([lambda i=i: step(i, with_sel_in=True) for i in range(R)])
        n_attn = max(R, (steps // R) * R)
        for _ in range(2):
            attn.replay()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(n_attn // R):
            if eager:
                for i in range(R):
                    step(i, with_sel_in=True)
            else:
                attn.replay()
        ev1.record()
        torch.cuda.synchronize()
        res["attn_us"] = ev0.elapsed_time(ev1) * 1e3 / n_attn
        del attn
    del full, singles, reps
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def line_of(w, alpha, r):
    """Per-workload summary: step time, queries/s, algorithmic GB/s and fraction of HBM peak."""
    gbps = r["step_bytes"] / (r["us_per_step"] * 1e-6) / 1e9
    return {"workload": w.name, "alpha": alpha, "us_per_step": r["us_per_step"],
            "queries_per_s": w.batch / (r["us_per_step"] * 1e-6), "step_bytes": r["step_bytes"],
            "GBps": gbps, "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS}


EXTRA_WORKLOADS = ["decode_b1_L32k", "decode_b8_L128k_rank4", "decode_b8_L128k_rank4_fp4",
                   "decode_b8_L128k_sub85_fp4"]


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="decode_b32_L16k32k")
    ap.add_argument("--alpha", type=float, default=None)
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough to exceed 2x the last-level cache")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the alpha sweep and the other decode workloads reported beside the headline")
    ap.add_argument("--extras", default=",".join(EXTRA_WORKLOADS),
                    help="comma-separated decode workloads timed after the headline (latency, long context)")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--eager", action="store_true", help="launch steps directly instead of graph replays")
    ap.add_argument("--mode", choices=["decode", "prefill", "build", "update", "recall", "copy"], default="decode",
                    help="decode (the metric), prefill (MFMA utilisation), build (summary GB/s), "
                         "update (one appended token per sequence: incremental summaries), "
                         "recall (cumulant selections against the exact-mass selection), "
                         "copy (plain copy of known size, to calibrate HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; the library runs on one GPU "
              "(multi-GPU sharding is a design note only)", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_long_compressed_amd import binding as B
    from block_sparse_long_compressed_amd import synth
    from block_sparse_long_compressed_amd import runtime as U

    if args.mode == "copy":
        return bench_copy(args)
    if args.mode == "prefill":
        return bench_prefill(args)
    if args.mode == "build":
        return bench_build(args)
    if args.mode == "update":
        return bench_update(args)
    if args.mode == "recall":
        return bench_recall(args)
    w = synth.WORKLOADS[args.workload]
    if w.prefill:
        raise SystemExit("use --mode prefill for prefill workloads")
    alpha = w.alpha if args.alpha is None else args.alpha
    log(f"[bench] workload {w.name} alpha {alpha}: generating inputs")
    x = synth.make_inputs(w, args.seed)
    # the CPU baseline's processes are forked before anything touches the GPU
    cpu = None if args.no_cpu_baseline else CpuBaseline(w, x, args.cpu_seconds)
    B.lib()
    g0 = U.to_device(x)
    P = calibrated_subspace(w, g0)
    log(f"[bench] timing {args.steps} steps (warmup {args.warmup})")
    r = time_decode(w, x, g0, P, alpha, args.steps, args.warmup, args.replicas, args.eager)
    ms_step = r["us_per_step"] * 1e-3
    step_bytes, attn_bytes = r["step_bytes"], r["attn_bytes"]
    log(f"[bench] {r['us_per_step']:.2f} us/step (host wall {r['host_wall_us_per_step']:.2f} us/step), "
        f"step bytes {step_bytes / 2**20:.2f} MiB, replicas {r['replicas']}")
    attn_gbps = attn_bytes / (r["attn_us"] * 1e-6) / 1e9
    log(f"[bench] attention roles alone {r['attn_us']:.2f} us, {attn_gbps:.0f} GB/s")
    # the step is one launch of k_decode: its algorithmic bytes over its duration
    achieved = step_bytes / (ms_step * 1e-3) / 1e9
    qps = w.batch / (ms_step * 1e-3)
    dense = dense_bytes(w, x["lens"])
    result = {
        "metric": "sparse-decode queries/s and achieved HBM GB/s (% of peak) at 32k ctx, top-k=16",
        "value": qps,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "achieved_GBps": achieved,
        "pct_of_hbm_peak": 100.0 * achieved / HBM_PEAK_GBPS,
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.max_len,
                   "seq_len_min": w.min_len, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "block": 64, "top_k": w.top_k, "window": w.window,
                   "cmp": [w.cmp_len, w.cmp_stride], "second_order": w.so_kind, "rank": w.rank,
                   "alpha": alpha, "step_bytes": step_bytes, "replicas": r["replicas"],
                   "graph_replay": not args.eager},
        "roofline": {"bound": "hbm", "kernel": "k_decode", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": counter_traffic(w.name, alpha), "bytes_per_launch": step_bytes,
                     "avg_launch_us": r["us_per_step"],
                     "attention_only": {"avg_launch_us": r["attn_us"], "bytes_per_launch": attn_bytes,
                                        "achieved": attn_gbps}},
        # KV read traffic of this step against dense attention over the same queries
        "kv_traffic_dense_over_cobs": dense / step_bytes,
    }
    if not args.no_extras:
        # the alpha sweep of the batched workload on the same inputs (alpha = 0 is the
        # first-order mean-pool selector of NSA: its bytes give the COBS / NSA ratio)
        sweep = {}
        for a in (0.0, 0.5, 1.0, 2.0):
            if a == alpha:
                sweep[str(a)] = line_of(w, a, r)
                continue
            log(f"[bench] alpha {a}")
            ra = time_decode(w, x, g0, P, a, max(60, args.steps // 3), 10, args.replicas, args.eager,
                             attention_only=False)
            sweep[str(a)] = line_of(w, a, ra)
        result["alpha_sweep"] = sweep
        if alpha == 1.0:
            result["kv_traffic_cobs_over_alpha0"] = step_bytes / sweep["0.0"]["step_bytes"]
        result["pages_reported_kv_traffic"] = {"cobs_over_nsa": 1.21, "dense_over_cobs": 15.15,
                                               "note": "context only: the pages' own ratios, on a 32k "
                                                       "retrieval suite with unstated block size, top-k "
                                                       "and hardware"}
    del g0
    torch.cuda.empty_cache()
    if not args.no_extras:
        extras = {}
        inputs = {}
        for name in [e for e in args.extras.split(",") if e]:
            we = synth.WORKLOADS[name]
            log(f"[bench] extra workload {name}: generating inputs")
            # the rank-4 storages share one draw (the recipe does not depend on the storage)
            key = (we.batch, we.max_len, we.min_len, we.n_q_heads, we.n_kv_heads, we.head_dim, we.dtype,
                   we.needles, we.subspace)
            if key not in inputs:
                inputs.clear()
                inputs[key] = synth.make_inputs(we, args.seed)
            xe = inputs[key]
            ge = U.to_device(xe)
            Pe = calibrated_subspace(we, ge)
            re_ = time_decode(we, xe, ge, Pe, we.alpha, max(60, args.steps // 3), 10, args.replicas, args.eager,
                              attention_only=False)
            extras[name] = line_of(we, we.alpha, re_)
            extras[name]["kv_traffic_dense_over_cobs"] = dense_bytes(we, xe["lens"]) / re_["step_bytes"]
            log(f"[bench]   {name}: {re_['us_per_step']:.2f} us/step")
            del ge, Pe
            torch.cuda.empty_cache()
        result["extra_workloads"] = extras
    if cpu is not None:
        log(f"[bench] cpu baseline ({args.cpu_seconds:.0f} s on {cpu.cores} processes)")
        result["cpu_baseline"] = cpu.finish()
    print(json.dumps(result), flush=True)


def timed(fn, n, warm=2):
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e-3          # seconds per call


def bench_copy(args):
    """A plain device-to-device copy of a known size: FETCH_SIZE / WRITE_SIZE of
    this kernel against its 2 x 256 MiB gives the counters' byte scale."""
    import torch
    n = 256 * 2 ** 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src), max(args.steps, 5))
    print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n, "us": t * 1e6,
                      "GBps": 2 * n / t / 1e9}), flush=True)


def bench_build(args):
    """Summary build (mean + second-order channel + pooled tokens): K and V are
    streamed once; reported as GB/s of K+V read."""
    import torch
    from block_sparse_long_compressed_amd import binding as B
    from block_sparse_long_compressed_amd import synth
    from block_sparse_long_compressed_amd import runtime as U
    w = synth.WORKLOADS[args.workload]
    x = synth.make_inputs(w, args.seed)
    g = U.to_device(x)
    p = U.params_for(w, P=calibrated_subspace(w, g))
    s = B.alloc_summaries(p, w.batch, w.max_len)
    fn = lambda: B.cobs_build_summaries(p, g["lens"], g["K"], g["V"], s["mu"], s["so"], s["kc"], s["vc"])
    t = timed(fn, max(1, min(args.steps, 20)))
    es = 2 if w.dtype == "bf16" else 4
    kv = int(np.asarray(x["lens"], dtype=np.int64).sum()) * w.n_kv_heads * w.head_dim * es * 2
    print(json.dumps({"mode": "build", "workload": w.name, "second_order": w.so_kind, "rank": w.rank,
                      "ms": t * 1e3, "kv_bytes": kv, "GBps_streamed": kv / t / 1e9,
                      "pct_of_hbm_peak": 100 * kv / t / 1e9 / HBM_PEAK_GBPS}), flush=True)


def bench_update(args):
    """Incremental summaries for one decode step: every sequence grows by one token
    (L-1 -> L); the touched block's statistics (and rank-r vectors) are recomputed
    and the pooled token it completes, if any, is emitted."""
    import torch
    from block_sparse_long_compressed_amd import binding as B
    from block_sparse_long_compressed_amd import synth
    from block_sparse_long_compressed_amd import runtime as U
    w = synth.WORKLOADS[args.workload]
    x = synth.make_inputs(w, args.seed)
    g = U.to_device(x)
    p = U.params_for(w, P=calibrated_subspace(w, g))
    s = B.alloc_summaries(p, w.batch, w.max_len)
    new = g["lens"]
    old = (new - 1).contiguous()
    B.cobs_build_summaries(p, old, g["K"], g["V"], s["mu"], s["so"], s["kc"], s["vc"])
    fn = lambda: B.cobs_update_summaries(p, old, new, 1, g["K"], g["V"], s["mu"], s["so"], s["kc"], s["vc"])
    t = timed(fn, max(1, min(args.steps, 50)))
    print(json.dumps({"mode": "update", "workload": w.name, "second_order": w.so_kind, "rank": w.rank,
                      "units": w.batch * w.n_kv_heads, "us_per_step": t * 1e6}), flush=True)


def bench_recall(args):
    """Quality diagnostic: the share of the exact-mass top-k (every key read) that the
    cumulant selection keeps, for alpha in {0, 0.5, 1, 2}; and the time of both selectors."""
    import torch
    from block_sparse_long_compressed_amd import binding as B
    from block_sparse_long_compressed_amd import synth
    from block_sparse_long_compressed_amd import runtime as U
    w = synth.WORKLOADS[args.workload]
    x = synth.make_inputs(w, args.seed)
    g = U.to_device(x)
    Pw = calibrated_subspace(w, g)
    p = U.params_for(w, P=Pw)
    ws = B.alloc_workspace(p, w.batch, w.max_len)
    exact = torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
    fx = lambda: B.cobs_select_topk_exact(p, g["lens"], g["Q"], g["K"], exact, ws)
    t_exact = timed(fx, max(1, min(args.steps, 20)))
    ex = exact.cpu().numpy()
    res = {"mode": "recall", "workload": w.name, "us_exact_selection": t_exact * 1e6, "recall": {}}
    for alpha in (0.0, 0.5, 1.0, 2.0):
        pa = U.params_for(w, alpha=alpha, P=Pw)
        s = U.build(pa, g)
        sel = torch.empty_like(exact)
        fs = lambda: B.cobs_select_topk(pa, g["lens"], g["Q"][:, None], s["mu"], s["so"], sel, ws, max_len=w.max_len)
        t = timed(fs, max(1, min(args.steps, 20)))
        sl = sel.cpu().numpy()
        hit = sum(len(set(sl[b, h][sl[b, h] >= 0]) & set(ex[b, h][ex[b, h] >= 0]))
                  for b in range(w.batch) for h in range(w.n_kv_heads))
        tot = sum(int((ex[b, h] >= 0).sum()) for b in range(w.batch) for h in range(w.n_kv_heads))
        res["recall"][str(alpha)] = hit / max(tot, 1)
        res[f"us_cumulant_selection_alpha{alpha}"] = t * 1e6
    if w.so_kind in ("lowrank", "lowrank_fp4"):
        # the storages of the rank-r channel: fp32 vectors, bf16 mean + MX FP4 vectors, and
        # (for a subspace workload) both again in the calibrated query subspace, at the
        # workload's alpha: recall of each against the exact-mass selection, agreement
        # with the fp32 full-dimension selection, summary bytes per block
        P = Pw
        variants = [("lowrank", None), ("lowrank_fp4", None)]
        if P is not None:
            variants += [("lowrank", P), ("lowrank_fp4", P)]
        sels = {}
        for kind, Pv in variants:
            name = kind + ("" if Pv is None else f"_sub{w.subspace}")
            wk = w.scaled(so_kind=kind, subspace=0 if Pv is None else w.subspace)
            pk = U.params_for(wk, P=Pv)
            s = U.build(pk, g)
            sel = torch.empty_like(exact)
            B.cobs_select_topk(pk, g["lens"], g["Q"][:, None], s["mu"], s["so"], sel, ws, max_len=w.max_len)
            torch.cuda.synchronize()
            sels[name] = sel.cpu().numpy()
            sh = B.cobs_summary_shapes(pk, w.batch, w.max_len)
            res[f"summary_bytes_per_block_{name}"] = (sh["mu_bytes"] + sh["so_bytes"]) / (
                w.batch * w.n_kv_heads * sh["nb_max"])
        a = sels["lowrank"]
        tot_a = int((a >= 0).sum())
        for name, f in sels.items():
            hit = sum(len(set(f[b, h][f[b, h] >= 0]) & set(ex[b, h][ex[b, h] >= 0]))
                      for b in range(w.batch) for h in range(w.n_kv_heads))
            res[f"recall_{name}_alpha{w.alpha}"] = hit / max(int((ex >= 0).sum()), 1)
            if name != "lowrank":
                same = sum(len(set(a[b, h][a[b, h] >= 0]) & set(f[b, h][f[b, h] >= 0]))
                           for b in range(w.batch) for h in range(w.n_kv_heads))
                res[f"agreement_{name}_vs_lowrank"] = same / max(tot_a, 1)
        res["units"] = w.batch * w.n_kv_heads
    print(json.dumps(res), flush=True)


def prefill_flops(w, lens, sel):
    """Algorithmic FLOPs of a prefill chunk: 4d per (query head, key) of the union
    of the three branches' key sets counted per branch (QK^T and PV), plus the
    scoring contraction 2 x (d + d) per (query head, candidate block)."""
    d, G = w.head_dim, w.group
    L = int(lens[0])
    total = 0
    for i in range(w.n_q_tokens):
        t = w.q_pos0 + i
        ncand = L // 64 if t >= L - 1 else (t + 1) // 64
        nwin = min(w.window, t + 1)
        nc = (t - 31) // 16 + 1 if t >= 31 else 0
        for h in range(w.n_kv_heads):
            nslc = sum(min(64, L - 64 * b) for b in sel[i, h] if b >= 0)
            total += G * 4 * d * (nslc + nwin + nc) + G * 2 * 2 * d * ncand
    return total


def bench_prefill(args):
    import torch
    from block_sparse_long_compressed_amd import binding as B
    from block_sparse_long_compressed_amd import synth
    from block_sparse_long_compressed_amd import runtime as U
    w = synth.WORKLOADS[args.workload if args.workload.startswith("prefill") else "prefill_T8k_L32k"]
    x = synth.make_inputs(w, args.seed)
    p = U.params_for(w)
    g = U.to_device(x)
    s = U.build(p, g)
    out, sel = U.prefill(p, g, s, w.q_pos0)
    flops = prefill_flops(w, x["lens"], sel)
    K0, V0 = g["K"][0].contiguous(), g["V"][0].contiguous()
    kc, vc = s["kc"][0].contiguous(), s["vc"][0].contiguous()
    ws = B.alloc_workspace(p, 1, w.max_len, w.n_q_tokens)
    o = torch.empty((w.n_q_tokens, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    fn = lambda: B.cobs_sparse_attn_prefill(p, w.q_pos0, g["Q"], K0, V0, s["mu"], s["so"], kc, vc, g["gates"],
                                            o, ws)
    t = timed(fn, max(1, min(args.steps, 20)))
    tflops = flops / t / 1e12
    print(json.dumps({"mode": "prefill", "workload": w.name, "ms": t * 1e3, "tokens_per_s": w.n_q_tokens / t,
                      "algorithmic_flop": flops, "TFLOPs": tflops,
                      "mfma_utilisation_vs_bf16_dense": tflops / 2500.0}), flush=True)


if __name__ == "__main__":
    main()
