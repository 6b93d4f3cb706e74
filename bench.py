#!/usr/bin/env python3
"""Benchmark of the DSA decode step on one MI355X.

One step = one dsa_decode_step over the whole batch (lightning-indexer scores
for every visible token, top-2048 selection, sparse MQA-mode MLA over the
selected latent rows), inputs resident in HBM.  The default workload is the
batch-64 decode with per-request contexts drawn uniformly from [8K, 128K]
(64-token pages, shuffled page tables, fp8 index keys, bf16 latent cache).

Prints one JSON line.  `value` is decode tokens/s per layer (query rows per
second).  `roofline` covers the dominant kernel -- the lightning indexer --
with its algorithmic bytes per launch divided by its average launch time,
timed live here with HIP events on the stream it runs on.  `step_hbm` gives
the same ratio for the whole step.  `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload.  Inputs rotate over several device
copies so that the 256 MB Infinity Cache cannot serve a step from the
previous one.

Algorithmic bytes of a step (what it must read or write; workspace excluded):
  sum_r  L_r*(D_idx + 4)            fp8 keys + fp32 key scale
       + U_r*(576*e_lat + s_lat)    distinct selected latent rows
       + 4*ceil(L_r/64)             page table
       + q_r*(H_idx*D_idx + 4*H_idx + H*576*2 + H*512*2)   queries, w, out
with U_r the number of distinct tokens selected by the request's query rows.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
DEFAULT_WORKLOAD = "batched_b64_l8k_128k"


# ------------------------------------------------------------ accounting
def mla_arithmetic_intensity(H, d, r, b):
    """FLOP per byte of MQA-mode MLA decode for L >> H (MLA Modifications
    section of the GLM-5.3 article): 2H(2d+r) / (b(d+r))."""
    return 2.0 * H * (2 * d + r) / (b * (d + r))


def latent_row_bytes(wl):
    W = wl.d_latent + wl.d_rope
    return {"f32": 4 * W, "bf16": 2 * W, "e4m3": W + 4}[wl.kv_dtype]


def indexer_launch_bytes(wl):
    """Bytes one indexer launch must move: keys + scales + page table per
    visible token range, queries and weights, and the fp32 scores it writes."""
    key_row = wl.idx_dim * (1 if wl.idx_dtype == "e4m3" else 4) + (4 if wl.idx_scales is not None else 0)
    q_row = wl.idx_heads * wl.idx_dim * (1 if wl.idx_dtype == "e4m3" else 4) + 4 * wl.idx_heads
    total = 0
    for r in range(wl.batch):
        L, ql = int(wl.context_lens[r]), int(wl.q_lens[r])
        total += L * key_row + 4 * math.ceil(L / wl.block_size) + ql * q_row
    for (_, _, n) in wl.query_positions():
        total += 4 * n
    return total


def step_bytes(wl, indices):
    """Algorithmic bytes of one whole step (formula in the module docstring)."""
    import numpy as np
    key_row = wl.idx_dim * (1 if wl.idx_dtype == "e4m3" else 4) + (4 if wl.idx_scales is not None else 0)
    q_row = wl.idx_heads * wl.idx_dim * (1 if wl.idx_dtype == "e4m3" else 4) + 4 * wl.idx_heads
    e_q = 4 if wl.kv_dtype == "f32" else 2
    mla_q = wl.mla_heads * (wl.d_latent + wl.d_rope) * e_q + wl.mla_heads * wl.d_latent * e_q
    total = 0
    for r in range(wl.batch):
        L, ql = int(wl.context_lens[r]), int(wl.q_lens[r])
        q0 = int(wl.query_start_loc[r])
        sel = indices[q0:q0 + ql]
        U = len(np.unique(sel[sel >= 0]))
        total += L * key_row + U * latent_row_bytes(wl) + 4 * math.ceil(L / wl.block_size)
        total += ql * (q_row + mla_q)
    return total


def step_flops(wl, indices):
    """Indexer (2*H_idx*D_idx per visible token) + MLA (2*H*(576+512) per
    selected token) floating-point operations of one step."""
    f_idx = sum(2 * wl.idx_heads * wl.idx_dim * n for (_, _, n) in wl.query_positions())
    n_sel = int((indices >= 0).sum())
    f_mla = 2 * wl.mla_heads * ((wl.d_latent + wl.d_rope) + wl.d_latent) * n_sel
    return f_idx, f_mla


# ------------------------------------------------------------------ main
def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--copies", type=int, default=4, help="rotating device copies of the caches")
    ap.add_argument("--cpu-rows", type=int, default=24, help="query rows in the oracle CPU sample (0: skip)")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--graph", action="store_true", help="replay the step from a captured HIP graph")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the DSA step here runs on a single MI355X "
              "(no sharding or collectives); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import sparse_attention_dsa_amd as dsa
    from sparse_attention_dsa_amd import binding as B
    import workloads

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    torch.cuda.set_device(0)
    t0 = time.time()
    wl = workloads.make_workload(args.workload)
    log("[bench] workload %s: B=%d T=%d sum L=%d (generated in %.1fs)" %
        (wl.name, wl.batch, wl.total_q, int(wl.context_lens.sum()), time.time() - t0))
    d0 = workloads.to_device(wl, "cuda")
    batch = dsa.Batch(d0["context_lens"], d0["query_start_loc"], d0["page_table"], wl.block_size,
                      wl.max_q_len, wl.max_context_len)
    copies = [d0]
    for _ in range(args.copies - 1):
        dc = dict(d0)
        for key in ("idx_keys", "idx_scales", "kv", "kv_scales"):
            if d0[key] is not None:
                dc[key] = d0[key].clone()
        copies.append(dc)
    torch.cuda.synchronize()
    log("[bench] %d device copies ready" % len(copies))

    T, H, K = wl.total_q, wl.mla_heads, wl.topk
    L = B.lib()
    bst = batch.struct()
    ws_bytes = dsa.workspace_size(B.OP_DECODE_STEP, batch, K, H)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    outs = [torch.empty((T, H, wl.d_latent), dtype=torch.bfloat16 if wl.kv_dtype != "f32" else torch.float32,
                        device="cuda") for _ in copies]
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    sptr = C.c_void_p(stream.cuda_stream)

    # Prebuilt ctypes arguments per copy: the timed loop only calls into the library.
    calls = []
    for ci, dc in enumerate(copies):
        ic = B.index_cache(dc["idx_keys"], dc["idx_scales"])
        lc = B.latent_cache(dc["kv"], dc["kv_scales"], wl.d_latent)
        calls.append((C.byref(bst), C.byref(ic), C.c_void_p(dc["q_idx"].data_ptr()), C.c_void_p(dc["w"].data_ptr()),
                      wl.idx_heads, C.byref(lc), C.c_void_p(dc["q_mla"].data_ptr()), H, K,
                      C.c_float(wl.softmax_scale), C.c_void_p(outs[ci].data_ptr()), None,
                      C.c_void_p(idx.data_ptr()), C.c_void_p(ws.data_ptr()), C.c_size_t(ws_bytes), sptr, ic, lc))

    def step(i):
        a = calls[i % len(calls)]
        st = L.dsa_decode_step(*a[:16])
        if st != 0:
            raise B.DsaError("dsa_decode_step", st)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(len(calls)):
                step(i)
        torch.cuda.synchronize()

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    if graph is None:
        for i in range(args.steps):
            step(i)
    else:
        reps = max(1, args.steps // len(calls))
        for _ in range(reps):
            graph.replay()
        args.steps = reps * len(calls)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    log("[bench] step: %.1f us" % (ms_per_step * 1e3))

    # Selection of the last step (for the byte accounting only).
    step(0)
    torch.cuda.synchronize()
    indices = idx.cpu().numpy()

    # Dominant kernel: the lightning indexer, timed launch by launch.
    ld = (wl.max_context_len + 63) // 64 * 64
    scores = torch.empty((T, ld), dtype=torch.float32, device="cuda")
    icalls = []
    for dc in copies:
        ic = B.index_cache(dc["idx_keys"], dc["idx_scales"])
        icalls.append((C.byref(bst), C.byref(ic), C.c_void_p(dc["q_idx"].data_ptr()),
                       C.c_void_p(dc["w"].data_ptr()), wl.idx_heads, C.c_void_p(scores.data_ptr()), ld, sptr, ic))
    for i in range(args.warmup):
        L.dsa_indexer_scores(*icalls[i % len(icalls)][:8])
    n_idx = max(args.steps, 20)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_idx)]
    torch.cuda.synchronize()
    for i in range(n_idx):
        evs[i][0].record(stream)
        st = L.dsa_indexer_scores(*icalls[i % len(icalls)][:8])
        evs[i][1].record(stream)
        if st != 0:
            raise B.DsaError("dsa_indexer_scores", st)
    torch.cuda.synchronize()
    idx_us = 1e3 * sum(a.elapsed_time(b) for a, b in evs) / n_idx
    idx_bytes = indexer_launch_bytes(wl)
    idx_gbs = idx_bytes / (idx_us * 1e-6) / 1e9
    log("[bench] indexer kernel: %.1f us, %.1f MB -> %.0f GB/s" % (idx_us, idx_bytes / 1e6, idx_gbs))

    sb = step_bytes(wl, indices)
    f_idx, f_mla = step_flops(wl, indices)
    step_gbs = sb / (ms_per_step * 1e-3) / 1e9
    tokens_per_s = T / (ms_per_step * 1e-3)

    # CPU baseline: the oracle on a bounded sample of query rows.
    cpu = None
    if args.cpu_rows > 0:
        import oracle
        threads = args.cpu_threads or min(16, os.cpu_count() or 1)
        rng = np.random.default_rng(0)
        rows = sorted(rng.choice(T, size=min(args.cpu_rows, T), replace=False).tolist())
        tc = time.time()
        oracle.run_step(wl, rows=rows, threads=threads, keep_scores=False)
        dt = time.time() - tc
        cpu = {"value": round(len(rows) / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": "%d of %d query rows of the same workload (full contexts, fp64 C oracle), %.1f s wall"
                         % (len(rows), T, dt)}
        log("[bench] oracle: %d rows in %.1fs" % (len(rows), dt))

    res = {
        "metric": "DSA decode tokens/s per layer at 128K ctx, batch 64; HBM GB/s as % of peak",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "query_rows": T,
                   "context": "L_r ~ U[8192, 131072]" if wl.name == DEFAULT_WORKLOAD else
                   "L_r = %s" % sorted(set(wl.context_lens.tolist()))[:4],
                   "mean_context": round(float(wl.context_lens.mean()), 1), "topk": K,
                   "indexer": "%dx%d e4m3" % (wl.idx_heads, wl.idx_dim), "mla_heads": H,
                   "latent": "%d+%d %s" % (wl.d_latent, wl.d_rope, wl.kv_dtype), "block_size": wl.block_size,
                   "input_copies": len(copies), "hip_graph": bool(graph is not None)},
        "roofline": {"bound": "hbm", "kernel": "indexer_fp8_mfma", "achieved": round(idx_gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(idx_gbs / PEAK_HBM_GBS, 4),
                     "traffic": None, "bytes_per_launch": idx_bytes, "us_per_launch": round(idx_us, 2)},
        "step_hbm": {"bytes": sb, "achieved": round(step_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(step_gbs / PEAK_HBM_GBS, 4)},
        "step_tflops": {"indexer_fp8": round(f_idx / (ms_per_step * 1e-3) / 1e12, 2),
                        "mla_bf16": round(f_mla / (ms_per_step * 1e-3) / 1e12, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
