#!/usr/bin/env python3
"""Benchmark of the DSA decode step on one MI355X.

One step = one dsa_decode_step over the whole batch (lightning-indexer scores
for every visible token, top-2048 selection, sparse MQA-mode MLA over the
selected latent rows), inputs resident in HBM.  The default workload is the
batch-64 decode with per-request contexts drawn uniformly from [8K, 128K]
(64-token pages, shuffled page tables, fp8 index keys, bf16 latent cache).

Prints one JSON line.  `value` is decode tokens/s per layer (query rows per
second).  `roofline` covers the dominant kernel of the step -- the lightning
indexer as the step runs it (emitting top-K candidates instead of score
rows) -- with its algorithmic bytes per launch (the keys, scales, page-table
entries, queries and weights it must read) divided by its average launch
time, timed live here by the start and stop events that
dsa_decode_step_timed has that launch itself take; its `traffic` is the
HBM bytes per launch that rocprofv3's FETCH_SIZE and WRITE_SIZE counters
recorded (scaled by a copy-kernel calibration), read from the committed
counter summary and reported only while the indexer source is unchanged.
`step_phases_us` splits the step the same way (bound sampling, indexer,
selection, attention), and `indexer_scores_kernel` gives the standalone,
score-writing indexer (dsa_indexer_scores) timed launch by launch.
`step_hbm` gives the algorithmic-bytes ratio for the whole step.
`prefill` times the chunked prefill (4096 new query tokens on a 131072-token
context: indexer scores, top-K, then sparse MLA prefill on two layers that
share the selection) call by call, and reports each contraction as MFMA
utilisation (achieved FLOP/s over the dense fp8 / bf16 peak), since at that
shape both are compute-bound; the top-K time is reported on its own.
`hot_cache` times the two-tier latent cache (hot set in HBM, full history in
pinned host memory) on selections that drift from step to step: the fetch of
the missing rows and sparse MLA over the hot set.
`other_configs` gives the step on the other decode configurations, and
`hbm_ceiling` a plain 2 GiB streaming read as the practical bandwidth ceiling;
`page_read_ceiling` and `attention_gather_ceiling` read the indexer's pages and
the attention's selected rows in those kernels' launch shapes with no
arithmetic.
`indexshare` times groups of layers that share one selection (one full step,
then sparse MLA only on the other layers' caches) and reports the amortised
tokens/s per layer.  `all_128k` repeats the step measurement with every
context at 131072 tokens.  `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload.  Inputs rotate over several device copies so
that the 256 MB Infinity Cache cannot serve a step from the previous one.

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
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
DEFAULT_WORKLOAD = "batched_b64_l8k_128k"
PREFILL_WORKLOAD = "prefill_q4096_l131072"


# ------------------------------------------------------------ accounting
def visible_counts(wl):
    """Visible-token count of every query row, in row order: query j of a
    request with context L (new query tokens included) and q_len rows sees
    L - q_len + j + 1 tokens (inclusive causal)."""
    out = []
    for L, ql in zip(wl.context_lens.tolist(), wl.q_lens.tolist()):
        out.extend(L - ql + j + 1 for j in range(ql))
    return out


def h800_ridge():
    """The H800's practical ridge point the MLA Modifications section quotes:
    865 TFLOP/s over 3.35 TB/s, in FLOP per byte."""
    return 865e12 / 3.35e12


def mla_arithmetic_intensity(H, d, r, b):
    """FLOP per byte of MQA-mode MLA decode for L >> H (MLA Modifications
    section of the GLM-5.3 article): 2H(2d+r) / (b(d+r))."""
    return 2.0 * H * (2 * d + r) / (b * (d + r))


def latent_row_bytes(wl):
    W = wl.d_latent + wl.d_rope
    return {"f32": 4 * W, "bf16": 2 * W, "e4m3": W + 4}[wl.kv_dtype]


def key_row_bytes(wl):
    """Bytes of one token's index key: fp32 or e4m3 elements, or MXFP4 (half
    a byte an element plus one E8M0 byte per 32), and its fp32 sigma."""
    D = wl.idx_dim
    elems = {"f32": 4 * D, "e4m3": D, "mxfp4": D // 2 + D // 32}[wl.idx_dtype]
    return elems + (4 if wl.idx_scales is not None else 0)


def query_row_bytes(wl):
    """Bytes of one indexer query row (fp32, or e4m3 for e4m3 and MXFP4 keys)
    and its fp32 head weights."""
    return wl.idx_heads * wl.idx_dim * (4 if wl.idx_dtype == "f32" else 1) + 4 * wl.idx_heads


def indexer_launch_bytes(wl):
    """Bytes one indexer launch must move: keys + scales + page table per
    visible token range, queries and weights, and the fp32 scores it writes."""
    key_row, q_row = key_row_bytes(wl), query_row_bytes(wl)
    total = 0
    for r in range(wl.batch):
        L, ql = int(wl.context_lens[r]), int(wl.q_lens[r])
        total += L * key_row + 4 * math.ceil(L / wl.block_size) + ql * q_row
    for n in visible_counts(wl):
        total += 4 * n
    return total


def indexer_read_bytes(wl):
    """Bytes the candidate-emitting indexer must read: indexer_launch_bytes
    without the score rows (its candidate appends, about 8 bytes for each of a
    few thousand tokens per row, are left out)."""
    return indexer_launch_bytes(wl) - sum(4 * n for n in visible_counts(wl))


def step_bytes(wl, indices):
    """Algorithmic bytes of one whole step (formula in the module docstring)."""
    import numpy as np
    key_row, q_row = key_row_bytes(wl), query_row_bytes(wl)
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
    f_idx = sum(2 * wl.idx_heads * wl.idx_dim * n for n in visible_counts(wl))
    n_sel = int((indices >= 0).sum())
    f_mla = 2 * wl.mla_heads * ((wl.d_latent + wl.d_rope) + wl.d_latent) * n_sel
    return f_idx, f_mla


def mla_layer_bytes(wl, indices):
    """Bytes of one sparse-MLA layer that reuses a selection: distinct selected
    latent rows, the page-table entries they need, queries and outputs."""
    import numpy as np
    e_q = 4 if wl.kv_dtype == "f32" else 2
    mla_q = wl.mla_heads * (wl.d_latent + wl.d_rope) * e_q + wl.mla_heads * wl.d_latent * e_q
    total = 0
    for r in range(wl.batch):
        ql = int(wl.q_lens[r])
        q0 = int(wl.query_start_loc[r])
        sel = indices[q0:q0 + ql]
        u = np.unique(sel[sel >= 0])
        total += len(u) * latent_row_bytes(wl) + 4 * len(np.unique(u // wl.block_size))
        total += ql * mla_q
    return total


def check_against_oracle(wl, rows, ref, indices, out, oracle):
    """The timed step's selection and output for `rows` against the oracle's
    results for them: every selection holds min(K, n) distinct visible
    tokens and differs from the oracle's only at scores within 1e-4
    (relative) of the oracle's K-th score; every output is within 2e-2 max-abs
    (1e-4 for fp32) of the oracle's sparse MLA on the step's own selection."""
    import numpy as np
    atol = 1e-4 if wl.kv_dtype == "f32" else 2e-2
    diffs, worst, ok = 0, 0.0, True
    for t in rows:
        r = ref[t]
        sc, osel = r["scores"], r["indices"]
        n = len(sc)
        m = min(wl.topk, n)
        sel = indices[t][:m]
        ok &= bool((sel >= 0).all() and (indices[t][m:] == -1).all() and (np.diff(sel) > 0).all()
                   and sel[-1] < n)
        d = set(sel.tolist()) ^ set(osel.tolist())
        if d:
            kth = float(sc[osel[-1]])
            ok &= all(abs(float(sc[x]) - kth) <= 1e-4 * abs(kth) for x in d)
        diffs += len(d)
        o_ref = r["out"] if not d else oracle.query_mla(wl, t, sel)[0]
        err = float(np.abs(out[t] - o_ref).max())
        worst = max(worst, err)
        ok &= err <= atol
    return {"rows": len(rows), "selection_diffs": diffs, "max_abs_err": round(worst, 6), "atol": atol,
            "ok": bool(ok)}


# ------------------------------------------------------- measured traffic
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "indexer_fp8_persistent_b64_l8k_128k_traffic.md")
INDEXER_SOURCES = ("sparse_attention_dsa_amd/csrc/indexer.hip", "sparse_attention_dsa_amd/csrc/dsa_kernels.h")


def indexer_source_hash():
    import hashlib
    h = hashlib.sha256()
    for p in INDEXER_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, prefix=""):
    """HBM bytes per indexer launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by its copy-kernel
    calibration), or None when the summary is missing, covers another
    workload, or was taken on a different indexer source.  prefix "" is the
    score-writing instance, "emit-" the candidate-emitting one."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            fields = dict(l.strip().strip("`").split(": ", 1) for l in f if ": " in l and l.startswith("`"))
    except OSError:
        return None
    if fields.get("workload") != workload or fields.get("source-sha256") != indexer_source_hash():
        return None
    try:
        return int(fields[prefix + "fetch-bytes-per-launch"]) + int(fields[prefix + "write-bytes-per-launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ rig
class Rig:
    """One workload resident on the device in several rotating copies, with
    prebuilt ctypes argument tuples so that timed loops only call into the
    library."""

    def __init__(self, wl, ncopies, log):
        import ctypes as C
        import torch
        import sparse_attention_dsa_amd as dsa
        from sparse_attention_dsa_amd import binding as B
        import workloads

        self.wl, self.torch, self.B = wl, torch, B
        d0 = workloads.to_device(wl, "cuda")
        self.batch = dsa.Batch(d0["context_lens"], d0["query_start_loc"], d0["page_table"], wl.block_size,
                               wl.max_q_len, wl.max_context_len)
        self.copies = [d0]
        for _ in range(ncopies - 1):
            dc = dict(d0)
            for key in ("idx_keys", "idx_scales", "kv", "kv_scales", "q_mla"):
                if d0[key] is not None:
                    dc[key] = d0[key].clone()
            self.copies.append(dc)
        torch.cuda.synchronize()
        log("[bench] %s: %d device copies ready" % (wl.name, len(self.copies)))

        T, H, K = wl.total_q, wl.mla_heads, wl.topk
        self.L = B.lib()
        self.bst = self.batch.struct()
        self.ws_step = dsa.workspace_size(B.OP_DECODE_STEP, self.batch, K, H)
        self.ws_mla = dsa.workspace_size(B.OP_MLA_DECODE, self.batch, K, H)
        # (room for up to 4 layers in one dsa_sparse_mla_decode_layers call)
        self.ws = torch.empty(max(self.ws_step, 4 * self.ws_mla, 256), dtype=torch.uint8, device="cuda")
        odt = torch.bfloat16 if wl.kv_dtype != "f32" else torch.float32
        self.outs = [torch.empty((T, H, wl.d_latent), dtype=odt, device="cuda") for _ in self.copies]
        self.idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
        self.stream = torch.cuda.current_stream()
        sptr = C.c_void_p(self.stream.cuda_stream)
        self.ld = (wl.max_context_len + 63) // 64 * 64
        self.scores = torch.empty((T, self.ld), dtype=torch.float32, device="cuda")
        wsp, idxp = C.c_void_p(self.ws.data_ptr()), C.c_void_p(self.idx.data_ptr())
        self.step_args, self.mla_args, self.idx_args, self._keep = [], [], [], []
        for ci, dc in enumerate(self.copies):
            keys = B.MxFp4Keys(dc["idx_keys"], wl.idx_dim) if wl.idx_dtype == "mxfp4" else dc["idx_keys"]
            ic = B.index_cache(keys, dc["idx_scales"])
            lc = B.latent_cache(dc["kv"], dc["kv_scales"], wl.d_latent)
            self._keep += [ic, lc]
            outp, qm = C.c_void_p(self.outs[ci].data_ptr()), C.c_void_p(dc["q_mla"].data_ptr())
            self.step_args.append((C.byref(self.bst), C.byref(ic), C.c_void_p(dc["q_idx"].data_ptr()),
                                   C.c_void_p(dc["w"].data_ptr()), wl.idx_heads, C.byref(lc), qm, H, K,
                                   C.c_float(wl.softmax_scale), outp, None, idxp, wsp,
                                   C.c_size_t(self.ws_step), sptr))
            self.mla_args.append((C.byref(self.bst), C.byref(lc), qm, H, idxp, K, C.c_float(wl.softmax_scale),
                                  outp, None, wsp, C.c_size_t(self.ws_mla), sptr))
            self.idx_args.append((C.byref(self.bst), C.byref(ic), C.c_void_p(dc["q_idx"].data_ptr()),
                                  C.c_void_p(dc["w"].data_ptr()), wl.idx_heads,
                                  C.c_void_p(self.scores.data_ptr()), self.ld, sptr))
        self.lcs = [B.latent_cache(dc["kv"], dc["kv_scales"], wl.d_latent) for dc in self.copies]
        self.layers_args = {}

    def _ok(self, fn, st):
        if st != 0:
            raise self.B.DsaError(fn, st)

    def step(self, i):
        self._ok("dsa_decode_step", self.L.dsa_decode_step(*self.step_args[i % len(self.copies)]))

    def fused_ok(self):
        """Whether dsa_decode_step_fused takes this workload's shapes."""
        st = self.L.dsa_decode_step_fused(*self.step_args[0], None, 0)
        self.torch.cuda.synchronize()
        return st == 0

    def step_fused(self, i):
        self._ok("dsa_decode_step_fused", self.L.dsa_decode_step_fused(*self.step_args[i % len(self.copies)],
                                                                       None, 0))

    def fused_phases(self, iters, warmup):
        """Average µs of the one-launch step's persistent kernel (events taken
        by its launch), of its merge, and of the whole call."""
        torch, B = self.torch, self.B
        n = len(self.copies)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(B.STEP_EVENTS)] for _ in range(iters)]
        handles = [B.event_handles(e, self.stream) for e in evs]
        for i in range(warmup):
            self.step_fused(i)
        torch.cuda.synchronize()
        for i in range(iters):
            self._ok("dsa_decode_step_fused",
                     self.L.dsa_decode_step_fused(*self.step_args[i % n], handles[i], B.STEP_EVENTS))
        torch.cuda.synchronize()
        avg = lambda a, b: 1e3 * sum(e[a].elapsed_time(e[b]) for e in evs) / iters
        return {"init": avg(0, 1), "kernel": avg(1, 2), "merge": avg(3, 4), "step": avg(0, 4)}

    def group(self, i, layers):
        """One IndexShare group: the full step on one layer's caches, then
        `layers - 1` sparse-MLA layers on other caches reusing its indices,
        one dsa_sparse_mla_decode call each."""
        n = len(self.copies)
        self.step(i)
        for l in range(1, layers):
            self._ok("dsa_sparse_mla_decode", self.L.dsa_sparse_mla_decode(*self.mla_args[(i + l) % n]))

    def group_layers(self, i, layers):
        """The same group with the `layers - 1` sparse-MLA layers in one
        dsa_sparse_mla_decode_layers call."""
        import ctypes as C
        if layers - 1 > 4:   # the call takes up to 4 layers
            return self.group(i, layers)
        n, key = len(self.copies), (i % len(self.copies), layers)
        if key not in self.layers_args:
            B, wl = self.B, self.wl
            ls = [(i + l) % n for l in range(1, layers)]
            caches = (B.DsaLatentCache * len(ls))(*[self.lcs[c] for c in ls])
            qs = (C.c_void_p * len(ls))(*[self.copies[c]["q_mla"].data_ptr() for c in ls])
            outs = (C.c_void_p * len(ls))(*[self.outs[c].data_ptr() for c in ls])
            self.layers_args[key] = (C.byref(self.bst), caches, len(ls), qs, wl.mla_heads,
                                     C.c_void_p(self.idx.data_ptr()), wl.topk, C.c_float(wl.softmax_scale), outs,
                                     None, C.c_void_p(self.ws.data_ptr()), C.c_size_t(self.ws.numel()),
                                     C.c_void_p(self.stream.cuda_stream))
        self.step(i)
        self._ok("dsa_sparse_mla_decode_layers", self.L.dsa_sparse_mla_decode_layers(*self.layers_args[key]))

    def step_phases(self, iters, warmup):
        """Average µs of the step's phases (bound sampling, indexer, selection,
        attention) and of the whole step, from the events that
        dsa_decode_step_timed records on the library's stream."""
        import ctypes as C
        torch, B = self.torch, self.B
        n = len(self.copies)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(B.STEP_EVENTS)] for _ in range(iters)]
        handles = [B.event_handles(e, self.stream) for e in evs]
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        for i in range(iters):
            self._ok("dsa_decode_step_timed",
                     self.L.dsa_decode_step_timed(*self.step_args[i % n], handles[i], B.STEP_EVENTS))
        torch.cuda.synchronize()
        names = ("sampling", "indexer", "selection", "attention")
        out = {k: 1e3 * sum(e[j].elapsed_time(e[j + 1]) for e in evs) / iters for j, k in enumerate(names)}
        out["step"] = 1e3 * sum(e[0].elapsed_time(e[-1]) for e in evs) / iters
        return out

    def indexer(self, i):
        self._ok("dsa_indexer_scores", self.L.dsa_indexer_scores(*self.idx_args[i % len(self.copies)]))

    def time_loop(self, fn, iters, warmup):
        """Average ms per call of fn(i) over `iters` calls, bracketed by
        events on the library's stream after a device-wide sync."""
        torch = self.torch
        for i in range(warmup):
            fn(i)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(self.stream)
        for i in range(iters):
            fn(i)
        ev1.record(self.stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / iters

    def time_launches(self, fn, iters, warmup):
        """Average µs of single launches, each bracketed by its own events."""
        torch = self.torch
        for i in range(warmup):
            fn(i)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        torch.cuda.synchronize()
        for i in range(iters):
            evs[i][0].record(self.stream)
            fn(i)
            evs[i][1].record(self.stream)
        torch.cuda.synchronize()
        return 1e3 * sum(a.elapsed_time(b) for a, b in evs) / iters

    def selection(self):
        self.step(0)
        self.torch.cuda.synchronize()
        return self.idx.cpu().numpy()

    def free(self):
        self.copies = self.outs = self.step_args = self.mla_args = self.idx_args = self._keep = None
        self.ws = self.idx = self.scores = None
        self.torch.cuda.empty_cache()


def summarize(rig, ms_step, indices, idx_us):
    wl = rig.wl
    sb = step_bytes(wl, indices)
    ib = indexer_launch_bytes(wl)
    return {
        "ms_per_step": round(ms_step, 5),
        "tokens_per_s": round(wl.total_q / (ms_step * 1e-3), 1),
        "step_bytes": sb,
        "step_hbm_frac": round(sb / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "indexer_us": round(idx_us, 2),
        "indexer_hbm_frac": round(ib / (idx_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
    }


def prefill_flops(wl):
    """(indexer fp8 FLOPs, sparse-MLA bf16 FLOPs per layer) of one chunked
    prefill: query j of a request with context L and q new tokens sees
    L - q + j + 1 tokens and selects min(K, that) of them."""
    f_idx = f_mla = 0
    for L, q in zip(wl.context_lens.tolist(), wl.q_lens.tolist()):
        for j in range(q):
            n = L - q + j + 1
            f_idx += 2 * wl.idx_heads * wl.idx_dim * n
            f_mla += 2 * wl.mla_heads * min(wl.topk, n) * (wl.d_latent + wl.d_rope + wl.d_latent)
    return f_idx, f_mla


def prefill_leg(iters, warmup, log):
    """Chunked prefill, one call at a time: indexer scores, top-K, sparse MLA
    prefill on layer 1 and on layer 2 with layer 1's selection."""
    import torch
    import sparse_attention_dsa_amd as dsa
    import workloads

    t0 = time.time()
    wl = workloads.make_workload(PREFILL_WORKLOAD)
    d = workloads.to_device(wl, "cuda")
    log("[bench] workload %s: T=%d L=%d (generated in %.1fs)" %
        (wl.name, wl.total_q, int(wl.context_lens.max()), time.time() - t0))
    batch = dsa.Batch(d["context_lens"], d["query_start_loc"], d["page_table"], wl.block_size,
                      wl.max_q_len, wl.max_context_len)
    T, H, K = wl.total_q, wl.mla_heads, wl.topk
    ld = (wl.max_context_len + 63) // 64 * 64
    stream = torch.cuda.current_stream()
    scores = torch.empty((T, ld), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    out = torch.empty((T, H, wl.d_latent), dtype=torch.bfloat16, device="cuda")
    from sparse_attention_dsa_amd import binding as B
    ws_tk = torch.empty(max(dsa.workspace_size(B.OP_TOPK, batch, K, 0), 256), dtype=torch.uint8, device="cuda")
    ws_ml = torch.empty(max(dsa.workspace_size(B.OP_MLA_PREFILL, batch, K, H), 256), dtype=torch.uint8,
                        device="cuda")
    calls = [
        lambda: dsa.indexer_scores(batch, d["idx_keys"], d["idx_scales"], d["q_idx"], d["w"], scores=scores,
                                   ld=ld, stream=stream),
        lambda: dsa.topk(batch, scores, K, indices=idx, workspace=ws_tk, stream=stream),
        lambda: dsa.sparse_mla_prefill(batch, d["kv"], d["kv_scales"], wl.d_latent, d["q_mla"], idx,
                                       wl.softmax_scale, out=out, workspace=ws_ml, stream=stream),
        lambda: dsa.sparse_mla_prefill(batch, d["kv2"], d["kv2_scales"], wl.d_latent, d["q_mla2"], idx,
                                       wl.softmax_scale, out=out, workspace=ws_ml, stream=stream),
    ]
    for _ in range(warmup):
        for c in calls:
            c()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(iters)]
    torch.cuda.synchronize()
    for it in range(iters):
        evs[it][0].record(stream)
        for k, c in enumerate(calls):
            c()
            evs[it][k + 1].record(stream)
    torch.cuda.synchronize()
    us = [1e3 * sum(e[k].elapsed_time(e[k + 1]) for e in evs) / iters for k in range(len(calls))]
    step_us = 1e3 * sum(e[0].elapsed_time(e[-1]) for e in evs) / iters
    f_idx, f_mla = prefill_flops(wl)
    mla_us = (us[2] + us[3]) / 2
    res = {
        "workload": wl.name, "query_rows": T, "context": int(wl.context_lens.max()), "topk": K, "layers": 2,
        "ms_per_step": round(step_us * 1e-3, 4),
        "tokens_per_s": round(T / (step_us * 1e-6), 1),
        "indexer": {"us": round(us[0], 1), "tflops": round(f_idx / us[0] * 1e-6, 1),
                    "peak": PEAK_FP8_TFLOPS, "mfma_frac": round(f_idx / us[0] * 1e-6 / PEAK_FP8_TFLOPS, 4)},
        "topk": {"us": round(us[1], 1), "scores": T * int(wl.context_lens.max()) - T * (T - 1) // 2},
        "mla_prefill": {"us_per_layer": round(mla_us, 1), "tflops": round(f_mla / mla_us * 1e-6, 1),
                        "peak": PEAK_BF16_TFLOPS,
                        "mfma_frac": round(f_mla / mla_us * 1e-6 / PEAK_BF16_TFLOPS, 4)},
    }
    log("[bench] prefill: %.2f ms per step; indexer %.0f us (%.1f%% of fp8 peak), top-K %.0f us, "
        "MLA %.0f us per layer (%.1f%% of bf16 peak)" %
        (step_us * 1e-3, us[0], 100 * res["indexer"]["mfma_frac"], us[1], mla_us,
         100 * res["mla_prefill"]["mfma_frac"]))
    del d, scores, idx, out, ws_tk, ws_ml, calls
    torch.cuda.empty_cache()
    return res


def hot_cache_leg(steps, warmup, log, capacity_mult=4, keep=0.8):
    """Two-tier latent cache on the batch-64 workload: a hot set of
    capacity_mult x T x K slots in HBM in front of the full latent pool in
    pinned host memory.  Each decode step's selection keeps `keep` of every
    row's previous selection and draws the rest anew among the row's visible
    tokens (synthetic drift; random N(0,1) data has no temporal locality of
    its own).  Per step: the fetch (hits, misses, LRU victims, host reads of
    the missing rows) and sparse MLA over the hot set, timed separately."""
    import numpy as np
    import torch
    import sparse_attention_dsa_amd as dsa
    from sparse_attention_dsa_amd import binding as B
    import workloads

    wl = workloads.make_workload(DEFAULT_WORKLOAD)
    d = workloads.to_device(wl, "cuda")
    batch = dsa.Batch(d["context_lens"], d["query_start_loc"], d["page_table"], wl.block_size, wl.max_q_len,
                      wl.max_context_len)
    T, K = wl.total_q, wl.topk
    host_kv = d["kv"].cpu().pin_memory()
    cap = capacity_mult * T * K
    hot = B.HotCache(cap, wl.batch, wl.max_context_len, d["kv"].shape[-1], d["kv"].dtype)
    B.hot_cache_reset(batch, hot)
    # warm-up until the hot set is full, so that the timed steps evict
    warmup += int(np.ceil((capacity_mult - 1) / (1.0 - keep))) + 2
    sels = drifting_selections(wl, warmup + steps, keep)
    counts = torch.zeros(2, dtype=torch.int32, device="cuda")
    out = torch.empty((T, wl.mla_heads, wl.d_latent), dtype=torch.bfloat16, device="cuda")
    ws_f = None
    ws_m = torch.empty(max(dsa.workspace_size(B.OP_MLA_DECODE, batch, K, wl.mla_heads), 256), dtype=torch.uint8,
                       device="cuda")
    hb = hot.batch(batch)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        ws_f = B.hot_cache_fetch(batch, host_kv, None, wl.d_latent, sels[i], hot, counts=counts, workspace=ws_f)
        dsa.sparse_mla_decode(hb, hot.kv, None, wl.d_latent, d["q_mla"], sels[i], wl.softmax_scale, out=out,
                              workspace=ws_m)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    miss, evict = [], []
    for j in range(steps):
        i = warmup + j
        ev[j][0].record(stream)
        B.hot_cache_fetch(batch, host_kv, None, wl.d_latent, sels[i], hot, counts=counts, workspace=ws_f)
        ev[j][1].record(stream)
        dsa.sparse_mla_decode(hb, hot.kv, None, wl.d_latent, d["q_mla"], sels[i], wl.softmax_scale, out=out,
                              workspace=ws_m)
        ev[j][2].record(stream)
        miss.append(counts[0].clone())
        evict.append(counts[1].clone())
    torch.cuda.synchronize()
    f_us = 1e3 * sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    m_us = 1e3 * sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    misses = float(torch.stack(miss).float().mean().item())
    evictions = float(torch.stack(evict).float().mean().item())
    row = d["kv"].shape[-1] * d["kv"].element_size()
    res = {"workload": wl.name, "capacity_slots": cap, "hot_bytes": cap * row,
           "full_pool_bytes": int(d["kv"].numel() * d["kv"].element_size()), "selection_kept_per_step": keep,
           "fetch_us": round(f_us, 1), "mla_us": round(m_us, 1), "misses_per_step": round(misses, 1),
           "evictions_per_step": round(evictions, 1),
           "hit_rate": round(1.0 - misses / (T * K), 4),
           "host_read_gbs": round(misses * row / (f_us * 1e-6) / 1e9, 1)}
    log("[bench] two-tier cache: hot set %.2f GB of %.2f GB; fetch %.0f us (%.0f misses, %.0f evictions a step, %.1f "
        "GB/s from host), MLA %.1f us" % (res["hot_bytes"] / 1e9, res["full_pool_bytes"] / 1e9, f_us, misses,
                                          evictions, res["host_read_gbs"], m_us))
    del d, host_kv, hot, sels, out, ws_f, ws_m
    torch.cuda.empty_cache()
    return res


def drifting_selections(wl, nsteps, keep, seed=7):
    """Per step, K distinct visible tokens per query row of which `keep` of
    the row's previous selection are kept and the rest drawn anew (sorted,
    int32 on the device)."""
    import numpy as np
    import torch
    K = wl.topk
    rng = np.random.default_rng(seed)
    vis = visible_counts(wl)
    prev = [rng.choice(n, size=K, replace=False) for n in vis]
    sels = []
    for _ in range(nsteps):
        cur = []
        for t, n in enumerate(vis):
            kept = rng.choice(prev[t], size=int(keep * K), replace=False)
            new = rng.choice(n, size=2 * (K - len(kept)), replace=True)
            new = np.setdiff1d(np.unique(new), kept)[:K - len(kept)]
            while len(new) < K - len(kept):
                extra = np.setdiff1d(rng.choice(n, size=K, replace=False), np.concatenate([kept, new]))
                new = np.concatenate([new, extra])[:K - len(kept)]
            cur.append(np.concatenate([kept, new]))
        prev = cur
        sels.append(torch.from_numpy(np.sort(np.stack(cur)).astype(np.int32)).cuda())
    return sels


def hot_cache_layers_leg(steps, warmup, log, layers=4, capacity_mult=4, keep=0.8):
    """Layer-wise overlap of the two-tier cache on the batch-64 workload: a
    group of `layers` layers sharing one selection (IndexShare), each layer
    with its own hot set and its own page table into the pinned host pool (a
    permutation of the blocks, so that every layer misses on other host
    rows).  The group's step is timed with fetch and attention alternating
    on one stream, and with layer l+1's fetch on a second stream during layer
    l's attention (sparse_attention_dsa_amd.hot_layers).  Also the GPU's read
    rate from pinned host memory (dsa_read_probe over a pinned buffer), the
    floor of the fetches' host reads."""
    import torch
    import sparse_attention_dsa_amd as dsa
    from sparse_attention_dsa_amd import binding as B
    from sparse_attention_dsa_amd.hot_layers import HotLayerGroup
    import workloads

    wl = workloads.make_workload(DEFAULT_WORKLOAD)
    d = workloads.to_device(wl, "cuda")
    T, K, H = wl.total_q, wl.topk, wl.mla_heads
    nblk = d["kv"].shape[0]
    host_kv = d["kv"].cpu().pin_memory()
    g = torch.Generator().manual_seed(11)
    batches, hots = [], []
    cap = capacity_mult * T * K
    for l in range(layers):
        perm = torch.randperm(nblk, generator=g).to(torch.int32).cuda()
        pt = perm[d["page_table"].long()].contiguous()
        batches.append(dsa.Batch(d["context_lens"], d["query_start_loc"], pt, wl.block_size, wl.max_q_len,
                                 wl.max_context_len))
        hots.append(B.HotCache(cap, wl.batch, wl.max_context_len, d["kv"].shape[-1], d["kv"].dtype))
    grp = HotLayerGroup(batches, [host_kv] * layers, [None] * layers, hots, wl.d_latent, K, H)
    grp.reset()
    warmup += int(math.ceil((capacity_mult - 1) / (1.0 - keep))) + 2
    sels = drifting_selections(wl, warmup + 2 * steps, keep)
    outs = [torch.empty((T, H, wl.d_latent), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    qs = [d["q_mla"]] * layers
    counts = [torch.zeros(2, dtype=torch.int32, device="cuda") for _ in range(layers)]
    for i in range(warmup):
        grp.step(sels[i], qs, wl.softmax_scale, outs, counts=counts, overlap=(i % 2 == 0))
    torch.cuda.synchronize()
    res = {"workload": wl.name, "layers": layers, "capacity_slots": cap}
    main = torch.cuda.current_stream()
    i = warmup
    for mode in ("serial", "overlapped"):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(main)
        for j in range(steps):
            grp.step(sels[i], qs, wl.softmax_scale, outs, counts=counts, overlap=(mode == "overlapped"))
            ev[j + 1].record(main)
            i += 1
        torch.cuda.synchronize()
        res[mode + "_us_per_group"] = round(1e3 * ev[0].elapsed_time(ev[steps]) / steps, 1)
    misses = sum(float(c[0].item()) for c in counts) / layers
    row = d["kv"].shape[-1] * d["kv"].element_size()
    # read rate from pinned host memory: the library's streaming-read probe over a pinned buffer
    pin = torch.empty(256 << 20, dtype=torch.uint8).pin_memory()
    sink = torch.empty(max(int(B.lib().dsa_read_probe_sink_size()), 4), dtype=torch.uint8, device="cuda")
    for _ in range(2):
        B.read_probe(pin, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(main)
    for _ in range(5):
        B.read_probe(pin, sink)
    e1.record(main)
    torch.cuda.synchronize()
    host_gbs = 5 * pin.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    floor_us = misses * row / (host_gbs * 1e9) * 1e6
    ser, ovl = res["serial_us_per_group"], res["overlapped_us_per_group"]
    res.update({"misses_per_layer_step": round(misses, 1), "hit_rate": round(1.0 - misses / (T * K), 4),
                "host_read_probe_gbs": round(host_gbs, 1),
                "host_read_floor_us_per_layer": round(floor_us, 1),
                "overlap_saving_us_per_group": round(ser - ovl, 1),
                "overlapped_us_per_layer": round(ovl / layers, 1)})
    log("[bench] two-tier cache, %d layers sharing a selection: %.0f us per group serial, %.0f us overlapped "
        "(%.0f us per layer; host-read floor %.0f us per layer at %.1f GB/s from pinned memory)" % (
            layers, ser, ovl, ovl / layers, floor_us, host_gbs))
    del d, host_kv, hots, grp, outs, sels, pin
    torch.cuda.empty_cache()
    return res


OTHER_WORKLOADS = ("tiny_fp32_l4096", "single_b1_l32768", "mtp_b8_l202752")


def other_configs(steps, warmup, log):
    """The decode step on the other decode configurations (one request at
    4096 fp32 / 32768 tokens; 8 requests at 202752 tokens with two MTP query
    rows and an e4m3 latent cache): step time, tokens/s and the step's
    algorithmic bytes over its time."""
    import workloads
    res = {}
    for name in OTHER_WORKLOADS:
        wl = workloads.make_workload(name)
        rig = Rig(wl, 4, lambda *a: None)
        ms = rig.time_loop(rig.step, steps, warmup)
        sb = step_bytes(wl, rig.selection())
        res[name] = {"ms_per_step": round(ms, 5), "tokens_per_s": round(wl.total_q / (ms * 1e-3), 1),
                     "step_bytes": sb, "step_hbm_frac": round(sb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        if rig.fused_ok():
            msf = rig.time_loop(rig.step_fused, steps, warmup)
            res[name]["fused_ms_per_step"] = round(msf, 5)
            log("[bench] %s: step %.1f us, one-launch step %.1f us" % (name, ms * 1e3, msf * 1e3))
        else:
            log("[bench] %s: step %.1f us" % (name, ms * 1e3))
        rig.free()
        del rig
    return res


def mxfp4_leg(steps, warmup, log):
    """The default decode workload with MXFP4 index keys (E2M1 elements, one
    E8M0 scale per 32; e4m3 queries): the score-writing indexer launch and
    the decode step (which takes MXFP4 keys through score rows and the
    top-K selection)."""
    import workloads
    wl = workloads.make_workload(DEFAULT_WORKLOAD, idx_dtype="mxfp4")
    rig = Rig(wl, 4, lambda *a: None)
    ms = rig.time_loop(rig.step, steps, warmup)
    sb = step_bytes(wl, rig.selection())
    us = rig.time_launches(rig.indexer, max(steps, 20), warmup)
    ib = indexer_launch_bytes(wl)
    res = {"workload": wl.name + " (MXFP4 keys)", "key_bytes_per_token": key_row_bytes(wl),
           "ms_per_step": round(ms, 5), "tokens_per_s": round(wl.total_q / (ms * 1e-3), 1), "step_bytes": sb,
           "step_hbm_frac": round(sb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "indexer_kernel": "indexer_mxfp4<1, 4> (dsa_indexer_scores)", "indexer_us": round(us, 2),
           "indexer_bytes": ib, "indexer_hbm_frac": round(ib / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    log("[bench] MXFP4 keys: step %.1f us, indexer %.1f us (%.0f GB/s)" % (ms * 1e3, us, ib / (us * 1e-6) / 1e9))
    rig.free()
    del rig
    return res


def read_ceiling(log, nbytes=1 << 31, iters=20):
    """The library's streaming-read probe over 2 GiB (every byte read once
    with 16-byte non-temporal loads): the practical HBM read ceiling next to
    the 8 TB/s peak."""
    import torch
    from sparse_attention_dsa_amd import binding as B
    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    sink = B.read_probe(x)
    for _ in range(3):
        B.read_probe(x, sink)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(iters):
        B.read_probe(x, sink)
    ev1.record()
    torch.cuda.synchronize()
    gbs = nbytes * iters / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    log("[bench] streaming read: %.0f GB/s" % gbs)
    del x, sink
    torch.cuda.empty_cache()
    return {"kernel": "dsa_read_probe over 2 GiB", "achieved": round(gbs, 1), "unit": "GB/s",
            "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}


def page_ceiling(rig, log, iters=20):
    """dsa_page_probe over the workload's own index-key pages (every
    request's visible pages in the indexer's order, 8 KB of keys and 256 B
    of scales each, rotating the device copies as the timed loop does): the
    rate the memory system gives the indexer's access pattern without its
    arithmetic, in the indexer's launch shape."""
    import numpy as np
    import torch
    from sparse_attention_dsa_amd import binding as B
    wl = rig.wl
    bs = wl.block_size
    ids = np.concatenate([wl.page_table[r, : (int(wl.context_lens[r]) + bs - 1) // bs] for r in range(wl.batch)])
    ids_t = torch.from_numpy(ids.astype(np.int32)).cuda()
    copies = rig.copies
    pb, sb_ = bs * wl.idx_dim, (4 * bs if copies[0]["idx_scales"] is not None else 0)
    sink = B.page_probe(copies[0]["idx_keys"], pb, copies[0]["idx_scales"], sb_, ids_t)
    for i in range(3):
        B.page_probe(copies[i % len(copies)]["idx_keys"], pb, copies[i % len(copies)]["idx_scales"], sb_, ids_t, sink)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(iters):
        c = copies[i % len(copies)]
        B.page_probe(c["idx_keys"], pb, c["idx_scales"], sb_, ids_t, sink)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / iters
    nbytes = int(len(ids)) * (pb + sb_)
    gbs = nbytes / (us * 1e-6) / 1e9
    log("[bench] random-page read of the indexer's pages: %.1f us, %.1f MB -> %.0f GB/s" % (us, nbytes / 1e6, gbs))
    return {"kernel": "dsa_page_probe (the indexer's pages, its grid and depth, no arithmetic)",
            "us": round(us, 2), "pages": int(len(ids)), "bytes": nbytes, "achieved": round(gbs, 1),
            "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}


def row_ceiling(rig, indices, log, iters=20):
    """dsa_row_probe over the step's own selection (every query row's selected
    latent rows, 1152 B each, in the attention's slice order and split count,
    rotating the device copies as the timed loop does): the rate the memory
    system gives the 128-head attention tile's gather without its
    arithmetic, in that tile's launch shape."""
    import numpy as np
    import torch
    from sparse_attention_dsa_amd import binding as B
    wl = rig.wl
    bs, T, K = wl.block_size, wl.total_q, wl.topk
    if (indices < 0).any() or wl.kv_dtype != "bf16" or wl.mla_heads != 128:
        return None
    qsl = np.asarray(wl.query_start_loc)
    req = np.searchsorted(qsl, np.arange(T), side="right") - 1
    pt = np.asarray(wl.page_table)
    rows = pt[req[:, None], indices // bs].astype(np.int64) * bs + indices % bs
    # the attention's split count: enough workgroups for the chip, at least
    # 128 tokens a slice
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    S = 1
    while T * S < cus and K // (2 * S) >= 128:
        S *= 2
    per = K // S
    if per % 32:
        return None
    ids_t = torch.from_numpy(rows.astype(np.int32).ravel()).cuda()
    copies = rig.copies
    sink = B.row_probe(copies[0]["kv"], 1152, ids_t, per)
    for i in range(3):
        B.row_probe(copies[i % len(copies)]["kv"], 1152, ids_t, per, sink)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(iters):
        B.row_probe(copies[i % len(copies)]["kv"], 1152, ids_t, per, sink)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / iters
    nbytes = int(rows.size) * 1152
    gbs = nbytes / (us * 1e-6) / 1e9
    log("[bench] gather of the attention's rows: %.1f us, %.1f MB -> %.0f GB/s (%d workgroups of %d rows)" %
        (us, nbytes / 1e6, gbs, T * S, per))
    return {"kernel": "dsa_row_probe (the attention's selected rows, its grid and LDS ring, no arithmetic)",
            "us": round(us, 2), "rows": int(rows.size), "rows_per_workgroup": per, "bytes": nbytes,
            "achieved": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}


# ------------------------------------------------------------------ main
def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--copies", type=int, default=4, help="rotating device copies of the caches")
    ap.add_argument("--idx-dtype", default=None, choices=["e4m3", "mxfp4"],
                    help="index-key encoding of the workload (default: the workload's own)")
    ap.add_argument("--cpu-rows", type=int, default=64, help="query rows in the oracle CPU sample (0: skip)")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--share-layers", type=int, default=4,
                    help="layers per IndexShare group for the amortised figure (0 or 1: skip)")
    ap.add_argument("--no-128k", action="store_true",
                    help="skip the extra measurement with every context at 131072 tokens")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the chunked-prefill measurement (4096 queries on a 131072-token context)")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other decode configurations and the streaming-read ceiling")
    ap.add_argument("--no-hot-cache", action="store_true",
                    help="skip the two-tier latent cache measurement")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the DSA step here runs on a single MI355X "
              "(no sharding or collectives); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import workloads

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    torch.cuda.set_device(0)
    t0 = time.time()
    wl = (workloads.make_workload(args.workload, idx_dtype=args.idx_dtype) if args.idx_dtype
          else workloads.make_workload(args.workload))
    log("[bench] workload %s: B=%d T=%d sum L=%d (generated in %.1fs)" %
        (wl.name, wl.batch, wl.total_q, int(wl.context_lens.sum()), time.time() - t0))
    rig = Rig(wl, args.copies, log)
    T, K = wl.total_q, wl.topk

    # The timed region: exactly `steps` decode steps.
    ms_per_step = rig.time_loop(rig.step, args.steps, args.warmup)
    log("[bench] step: %.1f us" % (ms_per_step * 1e3))
    indices = rig.selection()
    out_first = rig.outs[0].float().cpu().numpy()      # the step's output on copy 0 (same inputs as every copy)

    # Dominant kernel: the lightning indexer as the step runs it, timed by the
    # events the library records around its launch.
    n_idx = max(args.steps, 20)
    phases = rig.step_phases(n_idx, args.warmup)
    # MXFP4 keys take the score-writing indexer inside the step
    emit = wl.idx_dtype == "e4m3"
    emit_us, emit_bytes = phases["indexer"], indexer_read_bytes(wl) if emit else indexer_launch_bytes(wl)
    emit_gbs = emit_bytes / (emit_us * 1e-6) / 1e9
    log("[bench] step phases (us): " + ", ".join("%s %.1f" % kv for kv in phases.items()))
    log("[bench] indexer in the step: %.1f us, %.1f MB -> %.0f GB/s" % (emit_us, emit_bytes / 1e6, emit_gbs))
    # The standalone, score-writing indexer, timed launch by launch.
    idx_us = rig.time_launches(rig.indexer, n_idx, args.warmup)
    idx_bytes = indexer_launch_bytes(wl)
    idx_gbs = idx_bytes / (idx_us * 1e-6) / 1e9
    log("[bench] standalone indexer: %.1f us, %.1f MB -> %.0f GB/s" % (idx_us, idx_bytes / 1e6, idx_gbs))

    sb = step_bytes(wl, indices)
    f_idx, f_mla = step_flops(wl, indices)
    step_gbs = sb / (ms_per_step * 1e-3) / 1e9

    # The same step as one persistent kernel (dsa_decode_step_fused).
    fused = None
    if rig.fused_ok():
        ms_f = rig.time_loop(rig.step_fused, args.steps, args.warmup)
        fp = rig.fused_phases(n_idx, args.warmup)
        k_gbs = sb / (fp["kernel"] * 1e-6) / 1e9
        fused = {"ms_per_step": round(ms_f, 5), "tokens_per_s": round(T / (ms_f * 1e-3), 1),
                 "step_hbm_frac": round(sb / (ms_f * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                 "phases_us": {k: round(v, 2) for k, v in fp.items()},
                 "kernel": "fused_decode<1, 4, false>", "kernel_achieved": round(k_gbs, 1),
                 "kernel_frac": round(k_gbs / PEAK_HBM_GBS, 4),
                 "basis": "the step's algorithmic bytes over the persistent kernel's own duration"}
        log("[bench] one-launch step: %.1f us (persistent kernel %.1f us, merge %.1f us)" %
            (ms_f * 1e3, fp["kernel"], fp["merge"]))

    # IndexShare: one full step then (layers-1) MLA-only layers on the same indices.
    share = None
    if args.share_layers >= 2:
        nl = args.share_layers
        ms_sep = rig.time_loop(lambda i: rig.group(i, nl), max(4, args.steps // nl), 2)
        ms_group = rig.time_loop(lambda i: rig.group_layers(i, nl), max(4, args.steps // nl), 2)
        gb = sb + (nl - 1) * mla_layer_bytes(wl, indices)
        share = {"layers_per_group": nl, "ms_per_group": round(ms_group, 5),
                 "tokens_per_s_per_layer": round(nl * T / (ms_group * 1e-3), 1),
                 "group_bytes": gb, "hbm_frac": round(gb / (ms_group * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                 "attention_layers": "one dsa_sparse_mla_decode_layers call",
                 "ms_per_group_one_call_per_layer": round(ms_sep, 5)}
        log("[bench] IndexShare x%d: %.1f us per group -> %.0f tok/s/layer (one call per attention layer: %.1f us)" %
            (nl, ms_group * 1e3, share["tokens_per_s_per_layer"], ms_sep * 1e3))

    traffic = measured_traffic(wl.name)
    emit_traffic = measured_traffic(wl.name, "emit-")
    pages = page_ceiling(rig, log) if wl.max_q_len == 1 and wl.idx_dtype == "e4m3" else None
    gather = row_ceiling(rig, indices, log)
    rig.free()
    del rig

    # Every context at 131072 tokens: the literal 128K point of the metric.
    at128 = None
    if not args.no_128k and args.workload == DEFAULT_WORKLOAD:
        t0 = time.time()
        wl2 = workloads.make_workload(DEFAULT_WORKLOAD, context_lens=[131072])
        log("[bench] workload all-128K generated in %.1fs" % (time.time() - t0))
        rig2 = Rig(wl2, args.copies, log)
        ms2 = rig2.time_loop(rig2.step, args.steps, args.warmup)
        ind2 = rig2.selection()
        us2 = rig2.time_launches(rig2.indexer, n_idx, args.warmup)
        at128 = dict(workload="batched_b64_l128k", **summarize(rig2, ms2, ind2, us2))
        log("[bench] all-128K step: %.1f us" % (ms2 * 1e3))
        rig2.free()
        del rig2, wl2

    # Chunked prefill: MFMA-bound, reported as utilisation per contraction.
    prefill = None
    if not args.no_prefill and args.workload == DEFAULT_WORKLOAD:
        prefill = prefill_leg(max(3, min(args.steps, 10)), 2, log)

    # Other decode configurations, and a plain streaming read as the practical HBM ceiling.
    others = ceiling = None
    if not args.no_others and args.workload == DEFAULT_WORKLOAD:
        others = other_configs(max(10, min(args.steps, 50)), 5, log)
        ceiling = read_ceiling(log)

    # MXFP4 index keys on the same workload.
    fp4 = None
    if not args.no_others and args.workload == DEFAULT_WORKLOAD:
        fp4 = mxfp4_leg(max(10, min(args.steps, 50)), 5, log)

    # Two-tier latent cache: fetch + MLA over the hot set on drifting selections.
    hot = None
    if not args.no_hot_cache and args.workload == DEFAULT_WORKLOAD:
        hot = hot_cache_leg(max(5, min(args.steps, 20)), 10, log)
        hot["layers"] = hot_cache_layers_leg(max(4, min(args.steps, 10)), 4, log)

    # CPU baseline: the oracle on a bounded sample of query rows; its results
    # also check the timed step's selection and output for those rows.
    cpu = parity = None
    if args.cpu_rows > 0:
        import oracle
        threads = args.cpu_threads or min(16, os.cpu_count() or 1)
        rng = np.random.default_rng(0)
        rows = sorted(rng.choice(T, size=min(args.cpu_rows, T), replace=False).tolist())
        tc = time.time()
        ref = oracle.run_step(wl, rows=rows, threads=threads)
        dt = time.time() - tc
        cpu = {"value": round(len(rows) / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": "%d of %d query rows of the same workload (full contexts, fp64 C oracle), %.1f s wall"
                         % (len(rows), T, dt)}
        log("[bench] oracle: %d rows in %.1fs" % (len(rows), dt))
        parity = check_against_oracle(wl, rows, ref, indices, out_first, oracle)
        log("[bench] parity of the timed step on %d rows: %s" % (len(rows), parity))

    res = {
        "metric": "DSA decode tokens/s per layer at 128K ctx, batch 64; HBM GB/s as % of peak",
        "value": round(T / (ms_per_step * 1e-3), 1),
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
                   "indexer": "%dx%d %s" % (wl.idx_heads, wl.idx_dim, wl.idx_dtype), "mla_heads": wl.mla_heads,
                   "latent": "%d+%d %s" % (wl.d_latent, wl.d_rope, wl.kv_dtype), "block_size": wl.block_size,
                   "input_copies": args.copies},
        "roofline": {"bound": "hbm",
                     "kernel": ("indexer_fp8_persistent<1, 4, true>" if emit else "indexer_%s" % wl.idx_dtype)
                               + " (in dsa_decode_step)",
                     "achieved": round(emit_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(emit_gbs / PEAK_HBM_GBS, 4), "traffic": emit_traffic,
                     "bytes_per_launch": emit_bytes, "us_per_launch": round(emit_us, 2),
                     "scope": "the dominant kernel alone; the whole step's fraction is step_frac",
                     "step_frac": round(step_gbs / PEAK_HBM_GBS, 4)},
        "step_phases_us": {k: round(v, 2) for k, v in phases.items()},
        "indexer_scores_kernel": {"kernel": "indexer_fp8_persistent<1, 4, false> (dsa_indexer_scores)",
                                  "achieved": round(idx_gbs, 1), "frac": round(idx_gbs / PEAK_HBM_GBS, 4),
                                  "traffic": traffic, "bytes_per_launch": idx_bytes,
                                  "us_per_launch": round(idx_us, 2)},
        "step_hbm": {"bytes": sb, "achieved": round(step_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(step_gbs / PEAK_HBM_GBS, 4)},
        "kernel_tflops": {"indexer_fp8": round(f_idx / (phases["indexer"] * 1e-6) / 1e12, 1),
                          "mla_bf16": round(f_mla / (phases["attention"] * 1e-6) / 1e12, 1),
                          "basis": "each contraction's FLOPs over its own phase time"},
        "fused_step": fused,
        "mxfp4_keys": fp4,
        "indexshare": share,
        "all_128k": at128,
        "prefill": prefill,
        "other_configs": others,
        "hot_cache": hot,
        "hbm_ceiling": ceiling,
        "page_read_ceiling": pages,
        "attention_gather_ceiling": gather,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
