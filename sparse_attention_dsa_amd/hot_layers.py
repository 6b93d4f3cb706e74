"""Layer-wise overlap of the two-tier latent cache (HiSparse design:
SemiAnalysis, "Sparse Savings, Persistent Demand: inside GLM-5.3", section
"How Sparse Attention Affects DRAM/NAND Memory"; remio.ai, section "HiSparse
Move o Histórico Completo para Fora da GPU"): while layer N attends over its
hot set, the host reads of layer N+1's missing rows are already running.

A group of layers shares one selection (the IndexShare pattern: the indices
of the group's first layer serve the others), so every layer's fetch can
start as soon as the selection exists.  Each fetch is taken in its two
halves (dsa_hot_cache_plan, dsa_hot_cache_copy): the plans (short kernels:
hits, misses, victims) in layer order on one stream, the copies (host reads)
in layer order on a second, attention in layer order on a third.  A copy
waits for its plan, an attention for its copy, and a plan for the previous
step's attention on the same hot set (whose slots it is about to reassign).
So later layers' plans run beside a layer's copies, and a layer's attention
beside the next layer's copies.  All streams keep the default priority.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import torch

from . import binding as B


class HotLayerGroup:
    """Layers l = 0 .. L-1, each with its own batch geometry (page table into
    its host pool), pinned host latent pool (kv, scales) and hot cache."""

    def __init__(self, batches: Sequence[B.Batch], host_kv: Sequence[torch.Tensor],
                 host_scales: Sequence[Optional[torch.Tensor]], hots: Sequence[B.HotCache], d_latent: int, k: int,
                 n_heads: int):
        if not (len(batches) == len(host_kv) == len(host_scales) == len(hots)) or not batches:
            raise ValueError("one batch, host pool and hot cache per layer")
        self.batches, self.host_kv, self.host_scales, self.hots = list(batches), list(host_kv), list(host_scales), \
            list(hots)
        self.d_latent, self.k = d_latent, k
        self.L = len(batches)
        dev = hots[0].kv.device
        self.hot_batches = [h.batch(b) for h, b in zip(hots, batches)]
        self.ws_fetch = [B.hot_cache_workspace(b, k, h, dev) for b, h in zip(batches, hots)]
        need_m = max(B.workspace_size(B.OP_MLA_DECODE, hb, k, n_heads) for hb in self.hot_batches)
        self.ws_mla = torch.empty(max(need_m, 256), dtype=torch.uint8, device=dev)
        self.plan_stream = torch.cuda.Stream(device=dev)
        self.copy_stream = torch.cuda.Stream(device=dev)
        self.mla_stream = torch.cuda.Stream(device=dev)
        self.planned = [torch.cuda.Event() for _ in range(self.L)]
        self.fetched = [torch.cuda.Event() for _ in range(self.L)]
        self.attended = [torch.cuda.Event() for _ in range(self.L)]
        self.started = False

    def reset(self):
        for b, h in zip(self.batches, self.hots):
            B.hot_cache_reset(b, h)

    def step(self, indices: torch.Tensor, qs: Sequence[torch.Tensor], scale: float, outs: Sequence[torch.Tensor],
             lses: Optional[Sequence[Optional[torch.Tensor]]] = None, counts: Optional[List[torch.Tensor]] = None,
             overlap: bool = True):
        """One decode step of the group for selection `indices` [T][k]:
        layer l's queries qs[l], outputs outs[l] (and lses[l], counts[l] when
        given).  With overlap, the three-stream schedule above; without,
        fetch and attention alternate on the current stream.  Ordered after
        the current stream's earlier work, and the current stream's later
        work is ordered after it."""
        main = torch.cuda.current_stream()
        lses = lses if lses is not None else [None] * self.L
        counts = counts if counts is not None else [None] * self.L
        fetch = lambda l, phase, stream: B.hot_cache_fetch(
            self.batches[l], self.host_kv[l], self.host_scales[l], self.d_latent, indices, self.hots[l],
            counts=counts[l], workspace=self.ws_fetch[l], stream=stream, phase=phase)
        attend = lambda l, stream: B.sparse_mla_decode(
            self.hot_batches[l], self.hots[l].kv, self.hots[l].scales, self.d_latent, qs[l], indices, scale,
            out=outs[l], lse=lses[l], workspace=self.ws_mla, stream=stream)
        if not overlap:
            for l in range(self.L):
                fetch(l, "fetch", main)
                attend(l, main)
            return
        start = torch.cuda.Event()
        start.record(main)
        P, F, M = self.plan_stream, self.copy_stream, self.mla_stream
        for st in (P, F, M):
            st.wait_event(start)
        for l in range(self.L):
            if self.started:
                P.wait_event(self.attended[l])   # the previous step is done with this hot set and workspace
            fetch(l, "plan", P)
            self.planned[l].record(P)
        for l in range(self.L):
            F.wait_event(self.planned[l])
            fetch(l, "copy", F)
            self.fetched[l].record(F)
        for l in range(self.L):
            M.wait_event(self.fetched[l])
            attend(l, M)
            self.attended[l].record(M)
        self.started = True
        main.wait_event(self.attended[self.L - 1])
