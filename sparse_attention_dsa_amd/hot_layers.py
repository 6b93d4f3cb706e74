"""Layer-wise overlap of the two-tier latent cache (HiSparse design:
SemiAnalysis, "Sparse Savings, Persistent Demand: inside GLM-5.3", section
"How Sparse Attention Affects DRAM/NAND Memory"; remio.ai, section "HiSparse
Move o Histórico Completo para Fora da GPU"): while layer N attends over its
hot set, the host reads of layer N+1's missing rows are already running.

A group of layers shares one selection (the IndexShare pattern: the indices
of the group's first layer serve the others), so every layer's fetch can
start as soon as the selection exists.  Fetches run in layer order on one
stream and attention in layer order on a second one, each attention waiting
for its own layer's fetch, each fetch waiting for the previous step's
attention on the same hot set (its slots are about to be overwritten).  Both
streams keep the default priority.  This module only orders library calls
(dsa_hot_cache_fetch, dsa_sparse_mla_decode) with streams and events; every
step runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
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
        need_f = 0
        for b, h in zip(batches, hots):
            st = b.struct()
            need_f = max(need_f, int(B.lib().dsa_hot_cache_workspace_size(ctypes.byref(st), k, h.capacity)))
        self.ws_fetch = torch.empty(max(need_f, 256), dtype=torch.uint8, device=dev)
        need_m = max(B.workspace_size(B.OP_MLA_DECODE, hb, k, n_heads) for hb in self.hot_batches)
        self.ws_mla = torch.empty(max(need_m, 256), dtype=torch.uint8, device=dev)
        self.fetch_stream = torch.cuda.Stream(device=dev)
        self.mla_stream = torch.cuda.Stream(device=dev)
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
        given).  With overlap, layer l+1's fetch runs during layer l's
        attention; without, fetch and attention alternate on the current
        stream.  Ordered after the current stream's earlier work, and the
        current stream's later work is ordered after it."""
        main = torch.cuda.current_stream()
        lses = lses if lses is not None else [None] * self.L
        counts = counts if counts is not None else [None] * self.L
        if not overlap:
            for l in range(self.L):
                B.hot_cache_fetch(self.batches[l], self.host_kv[l], self.host_scales[l], self.d_latent, indices,
                                  self.hots[l], counts=counts[l], workspace=self.ws_fetch, stream=main)
                B.sparse_mla_decode(self.hot_batches[l], self.hots[l].kv, self.hots[l].scales, self.d_latent, qs[l],
                                    indices, scale, out=outs[l], lse=lses[l], workspace=self.ws_mla, stream=main)
            return
        start = torch.cuda.Event()
        start.record(main)
        F, M = self.fetch_stream, self.mla_stream
        F.wait_event(start)
        M.wait_event(start)
        for l in range(self.L):
            if self.started:
                F.wait_event(self.attended[l])   # the previous step's attention on this hot set is done
            B.hot_cache_fetch(self.batches[l], self.host_kv[l], self.host_scales[l], self.d_latent, indices,
                              self.hots[l], counts=counts[l], workspace=self.ws_fetch, stream=F)
            self.fetched[l].record(F)
            M.wait_event(self.fetched[l])
            B.sparse_mla_decode(self.hot_batches[l], self.hots[l].kv, self.hots[l].scales, self.d_latent, qs[l],
                                indices, scale, out=outs[l], lse=lses[l], workspace=self.ws_mla, stream=M)
            self.attended[l].record(M)
        self.started = True
        main.wait_event(self.attended[self.L - 1])
        main.wait_event(self.fetched[self.L - 1])
