"""ctypes binding of libdsa.so (include/dsa.h), one function per C entry point.

Argument marshalling only: torch tensors are used for device memory and the
current stream; every step of the computation runs in the library's HIP
kernels.  The library must be built (``python -m sparse_attention_dsa_amd.build``);
loading fails loudly otherwise and there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

DSA_OK = 0
F32, BF16, E4M3 = 0, 1, 2
OP_TOPK, OP_MLA_DECODE, OP_MLA_PREFILL, OP_DECODE_STEP = 1, 2, 3, 4

EXPORTS = ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_decode", "dsa_sparse_mla_prefill",
           "dsa_decode_step", "dsa_workspace_size", "dsa_status_string", "dsa_check_device",
           "dsa_read_probe_sink_size", "dsa_read_probe", "dsa_hot_cache_reset", "dsa_hot_cache_workspace_size",
           "dsa_hot_cache_fetch", "dsa_decode_step_timed", "dsa_decode_step_noalloc",
           "dsa_decode_step_fused", "dsa_check_batch", "dsa_hot_cache_plan", "dsa_hot_cache_copy",
           "dsa_sparse_mla_decode_layers", "dsa_page_probe_sink_size", "dsa_page_probe",
           "dsa_row_probe_sink_size", "dsa_row_probe")
CHECK_QUERY_START, CHECK_CONTEXT, CHECK_PAGE, CHECK_INDEX = 1, 2, 4, 8   # dsa_check_batch's bits
ERR_BAD_DEVICE_ARG = -7
STEP_EVENTS = 5   # events of dsa_decode_step_timed: start, after sampling, indexer, selection, attention


class DsaHotCache(C.Structure):
    _fields_ = [("kv", C.c_void_p), ("scales", C.c_void_p), ("capacity", C.c_int32), ("slot_of", C.c_void_p),
                ("owner", C.c_void_p), ("last_use", C.c_void_p), ("clock", C.c_void_p)]


class DsaBatch(C.Structure):
    _fields_ = [("num_requests", C.c_int32), ("total_q", C.c_int32), ("max_q_len", C.c_int32),
                ("max_context_len", C.c_int32), ("context_lens", C.c_void_p),
                ("query_start_loc", C.c_void_p), ("page_table", C.c_void_p),
                ("max_blocks", C.c_int32), ("block_size", C.c_int32)]


class DsaIndexCache(C.Structure):
    _fields_ = [("keys", C.c_void_p), ("scales", C.c_void_p), ("dtype", C.c_int32), ("dim", C.c_int32),
                ("num_blocks", C.c_int32)]


class DsaLatentCache(C.Structure):
    _fields_ = [("kv", C.c_void_p), ("scales", C.c_void_p), ("dtype", C.c_int32),
                ("d_latent", C.c_int32), ("d_rope", C.c_int32), ("num_blocks", C.c_int32)]


_lib = None


def lib():
    """Load libdsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libdsa.so is not built; run `python -m sparse_attention_dsa_amd.build`")
        L = C.CDLL(LIB_PATH)
        P = C.POINTER
        vp, i32, i64, sz, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_float
        L.dsa_indexer_scores.argtypes = [P(DsaBatch), P(DsaIndexCache), vp, vp, i32, vp, i64, vp]
        L.dsa_topk.argtypes = [P(DsaBatch), vp, i64, i32, vp, vp, sz, vp]
        mla = [P(DsaBatch), P(DsaLatentCache), vp, i32, vp, i32, f32, vp, vp, vp, sz, vp]
        L.dsa_sparse_mla_decode.argtypes = mla
        L.dsa_sparse_mla_decode_layers.argtypes = [P(DsaBatch), P(DsaLatentCache), i32, P(vp), i32, vp, i32, f32,
                                                   P(vp), P(vp), vp, sz, vp]
        L.dsa_sparse_mla_prefill.argtypes = mla
        L.dsa_decode_step.argtypes = [P(DsaBatch), P(DsaIndexCache), vp, vp, i32, P(DsaLatentCache), vp, i32,
                                      i32, f32, vp, vp, vp, vp, sz, vp]
        L.dsa_workspace_size.argtypes = [i32, P(DsaBatch), i32, i32]
        L.dsa_workspace_size.restype = sz
        L.dsa_status_string.argtypes = [i32]
        L.dsa_status_string.restype = C.c_char_p
        L.dsa_check_device.argtypes = []
        L.dsa_read_probe_sink_size.argtypes = []
        L.dsa_read_probe_sink_size.restype = sz
        L.dsa_read_probe.argtypes = [vp, i64, vp, sz, vp]
        L.dsa_page_probe_sink_size.argtypes = []
        L.dsa_page_probe_sink_size.restype = sz
        L.dsa_page_probe.argtypes = [vp, i64, vp, i64, vp, i32, vp, sz, vp]
        L.dsa_row_probe_sink_size.argtypes = [i32, i32]
        L.dsa_row_probe_sink_size.restype = sz
        L.dsa_row_probe.argtypes = [vp, i64, vp, i32, i32, vp, sz, vp]
        L.dsa_row_probe.restype = C.c_int
        L.dsa_hot_cache_reset.argtypes = [P(DsaBatch), P(DsaHotCache), vp]
        L.dsa_hot_cache_workspace_size.argtypes = [P(DsaBatch), i32, i32]
        L.dsa_hot_cache_workspace_size.restype = sz
        L.dsa_hot_cache_fetch.argtypes = [P(DsaBatch), P(DsaLatentCache), vp, i32, P(DsaHotCache), vp, vp, sz, vp]
        L.dsa_hot_cache_plan.argtypes = [P(DsaBatch), P(DsaLatentCache), vp, i32, P(DsaHotCache), vp, sz, vp]
        L.dsa_hot_cache_copy.argtypes = [P(DsaBatch), P(DsaLatentCache), vp, i32, P(DsaHotCache), vp, vp, sz, vp]
        L.dsa_decode_step_timed.argtypes = [P(DsaBatch), P(DsaIndexCache), vp, vp, i32, P(DsaLatentCache), vp, i32,
                                            i32, f32, vp, vp, vp, vp, sz, vp, P(vp), i32]
        L.dsa_decode_step_noalloc.argtypes = [P(DsaBatch), P(DsaIndexCache), vp, vp, i32, P(DsaLatentCache), vp,
                                              i32, i32, f32, vp, vp, vp, vp]
        L.dsa_decode_step_fused.argtypes = [P(DsaBatch), P(DsaIndexCache), vp, vp, i32, P(DsaLatentCache), vp, i32,
                                            i32, f32, vp, vp, vp, vp, sz, vp, P(vp), i32]
        L.dsa_check_batch.argtypes = [P(DsaBatch), i32, vp, i32, P(C.c_uint32), vp]
        for name in ("dsa_sparse_mla_decode_layers", "dsa_check_batch", "dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_decode", "dsa_sparse_mla_prefill",
                     "dsa_decode_step", "dsa_check_device", "dsa_read_probe", "dsa_hot_cache_reset",
                     "dsa_hot_cache_fetch", "dsa_hot_cache_plan", "dsa_hot_cache_copy", "dsa_decode_step_timed", "dsa_decode_step_noalloc",
                     "dsa_decode_step_fused"):
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


class DsaError(RuntimeError):
    def __init__(self, fn, status):
        msg = lib().dsa_status_string(status).decode()
        super().__init__("%s failed: %s (%d)" % (fn, msg, status))
        self.status = status


def _check(fn, status):
    if status != DSA_OK:
        raise DsaError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libdsa must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return E4M3
    raise ValueError("unsupported cache dtype %s" % t.dtype)


class Batch:
    """Batch geometry: device int32 tensors plus the host-known maxima."""

    def __init__(self, context_lens: torch.Tensor, query_start_loc: torch.Tensor, page_table: torch.Tensor,
                 block_size: int, max_q_len: int, max_context_len: int):
        for t in (context_lens, query_start_loc, page_table):
            if t.dtype != torch.int32 or not t.is_cuda:
                raise ValueError("batch arrays must be int32 device tensors")
        self.context_lens, self.query_start_loc, self.page_table = context_lens, query_start_loc, page_table
        self.num_requests = context_lens.shape[0]
        self.total_q = int(query_start_loc[-1].item()) if query_start_loc.numel() else 0
        self.block_size, self.max_q_len, self.max_context_len = block_size, max_q_len, max_context_len

    def struct(self) -> DsaBatch:
        return DsaBatch(self.num_requests, self.total_q, self.max_q_len, self.max_context_len,
                        self.context_lens.data_ptr(), self.query_start_loc.data_ptr(),
                        self.page_table.data_ptr(), self.page_table.shape[1], self.block_size)


DSA_MXFP4 = 3


class MxFp4Keys:
    """An MXFP4 index-key cache: `data` uint8 [num_blocks][block_size *
    (dim/2 + dim/32)] (per block: packed E2M1 codes, then E8M0 scales) and
    the key dimension `dim` (a multiple of 32)."""

    def __init__(self, data: torch.Tensor, dim: int):
        if data.dtype != torch.uint8 or dim % 32:
            raise ValueError("MXFP4 keys are uint8 bytes with dim a multiple of 32")
        self.data, self.dim = data, dim

    def data_ptr(self):
        return self.data.data_ptr()


def index_cache(keys, scales: Optional[torch.Tensor]) -> DsaIndexCache:
    sp = scales.data_ptr() if scales is not None else None
    if isinstance(keys, MxFp4Keys):
        return DsaIndexCache(keys.data_ptr(), sp, DSA_MXFP4, keys.dim, keys.data.shape[0])
    return DsaIndexCache(keys.data_ptr(), sp, dtype_code(keys), keys.shape[-1], _pool_blocks(keys))


def _pool_blocks(t: torch.Tensor) -> int:
    # [num_blocks][block_size][width] pools state their block count (read by
    # the library's debug check); other views leave it unstated (0)
    return int(t.shape[0]) if t.dim() == 3 else 0


def latent_cache(kv: torch.Tensor, scales: Optional[torch.Tensor], d_latent: int) -> DsaLatentCache:
    return DsaLatentCache(kv.data_ptr(), scales.data_ptr() if scales is not None else None,
                          dtype_code(kv), d_latent, kv.shape[-1] - d_latent, _pool_blocks(kv))


def workspace_size(op: int, batch: Batch, k: int, n_heads: int = 0) -> int:
    b = batch.struct()
    return int(lib().dsa_workspace_size(op, C.byref(b), k, n_heads))


def _workspace(op, batch, k, n_heads, device, workspace):
    need = workspace_size(op, batch, k, n_heads)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace


def indexer_scores(batch: Batch, keys, key_scales, q_idx, w, scores=None, ld=None, stream=None):
    """Scores [T][ld] fp32 (-inf past each row's visible count)."""
    ld = ld or ((batch.max_context_len + 63) // 64 * 64)
    if scores is None:
        scores = torch.empty((batch.total_q, ld), dtype=torch.float32, device=q_idx.device)
    b, c = batch.struct(), index_cache(keys, key_scales)
    _check("dsa_indexer_scores", lib().dsa_indexer_scores(
        C.byref(b), C.byref(c), _ptr(q_idx), _ptr(w), q_idx.shape[1], _ptr(scores), ld, _stream(stream)))
    return scores


def topk(batch: Batch, scores, k: int, indices=None, workspace=None, stream=None):
    """Top-k logical indices [T][k] int32, ascending, -1 padded."""
    if indices is None:
        indices = torch.empty((batch.total_q, k), dtype=torch.int32, device=scores.device)
    ws = _workspace(OP_TOPK, batch, k, 0, scores.device, workspace)
    b = batch.struct()
    _check("dsa_topk", lib().dsa_topk(C.byref(b), _ptr(scores), scores.shape[1], k, _ptr(indices),
                                      _ptr(ws), ws.numel(), _stream(stream)))
    return indices


def _out_like(kv, q, d_latent):
    dt = torch.float32 if kv.dtype == torch.float32 else torch.bfloat16
    return torch.empty((q.shape[0], q.shape[1], d_latent), dtype=dt, device=q.device)


def _mla(fn, op, batch, kv, kv_scales, d_latent, q, indices, scale, out, lse, workspace, stream):
    k = indices.shape[1]
    if out is None:
        out = _out_like(kv, q, d_latent)
    ws = _workspace(op, batch, k, q.shape[1], q.device, workspace)
    b, c = batch.struct(), latent_cache(kv, kv_scales, d_latent)
    _check(fn, getattr(lib(), fn)(C.byref(b), C.byref(c), _ptr(q), q.shape[1], _ptr(indices), k,
                                  float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def sparse_mla_decode(batch: Batch, kv, kv_scales, d_latent, q, indices, scale, out=None, lse=None,
                      workspace=None, stream=None):
    return _mla("dsa_sparse_mla_decode", OP_MLA_DECODE, batch, kv, kv_scales, d_latent, q, indices,
                scale, out, lse, workspace, stream)


def sparse_mla_decode_layers(batch: Batch, kvs, kv_scales, d_latent, qs, indices, scale, outs=None, lses=None,
                             workspace=None, stream=None):
    """dsa_sparse_mla_decode_layers: layer l attends over kvs[l] (scales
    kv_scales[l]) with queries qs[l] and the shared `indices`; returns the
    list of outputs."""
    L = len(kvs)
    k = indices.shape[1]
    if outs is None:
        outs = [_out_like(kv, q, d_latent) for kv, q in zip(kvs, qs)]
    need = L * workspace_size(OP_MLA_DECODE, batch, k, qs[0].shape[1])
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=qs[0].device)
    b = batch.struct()
    caches = (DsaLatentCache * L)(*[latent_cache(kv, sc, d_latent) for kv, sc in zip(kvs, kv_scales)])
    qp = (C.c_void_p * L)(*[_ptr(q) for q in qs])
    op = (C.c_void_p * L)(*[_ptr(o) for o in outs])
    lp = None if lses is None else (C.c_void_p * L)(*[_ptr(x) for x in lses])
    _check("dsa_sparse_mla_decode_layers", lib().dsa_sparse_mla_decode_layers(
        C.byref(b), caches, L, qp, qs[0].shape[1], _ptr(indices), k, float(scale), op, lp, _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return outs


def sparse_mla_prefill(batch: Batch, kv, kv_scales, d_latent, q, indices, scale, out=None, lse=None,
                       workspace=None, stream=None):
    return _mla("dsa_sparse_mla_prefill", OP_MLA_PREFILL, batch, kv, kv_scales, d_latent, q, indices,
                scale, out, lse, workspace, stream)


def decode_step(batch: Batch, keys, key_scales, q_idx, w, kv, kv_scales, d_latent, q_mla, k, scale,
                out=None, lse=None, indices_out=None, workspace=None, stream=None):
    """Indexer + top-k + sparse MLA in one call; returns out (and fills indices_out)."""
    if out is None:
        out = _out_like(kv, q_mla, d_latent)
    ws = _workspace(OP_DECODE_STEP, batch, k, q_mla.shape[1], q_mla.device, workspace)
    b, ic, lc = batch.struct(), index_cache(keys, key_scales), latent_cache(kv, kv_scales, d_latent)
    _check("dsa_decode_step", lib().dsa_decode_step(
        C.byref(b), C.byref(ic), _ptr(q_idx), _ptr(w), q_idx.shape[1], C.byref(lc), _ptr(q_mla),
        q_mla.shape[1], k, float(scale), _ptr(out), _ptr(lse), _ptr(indices_out), _ptr(ws), ws.numel(),
        _stream(stream)))
    return out


def decode_step_fused(batch: Batch, keys, key_scales, q_idx, w, kv, kv_scales, d_latent, q_mla, k, scale,
                      out=None, lse=None, indices_out=None, workspace=None, stream=None, events=None):
    """The step as one persistent kernel (dsa_decode_step_fused); `events`
    (STEP_EVENTS torch.cuda.Event, optional) are recorded at its boundaries:
    start, persistent kernel start and end, after it, after the merge."""
    if out is None:
        out = _out_like(kv, q_mla, d_latent)
    ws = _workspace(OP_DECODE_STEP, batch, k, q_mla.shape[1], q_mla.device, workspace)
    b, ic, lc = batch.struct(), index_cache(keys, key_scales), latent_cache(kv, kv_scales, d_latent)
    h = event_handles(events, stream) if events is not None else None
    _check("dsa_decode_step_fused", lib().dsa_decode_step_fused(
        C.byref(b), C.byref(ic), _ptr(q_idx), _ptr(w), q_idx.shape[1], C.byref(lc), _ptr(q_mla),
        q_mla.shape[1], k, float(scale), _ptr(out), _ptr(lse), _ptr(indices_out), _ptr(ws), ws.numel(),
        _stream(stream), h, len(events) if events is not None else 0))
    return out


def decode_step_noalloc(batch: Batch, keys, key_scales, q_idx, w, kv, kv_scales, d_latent, q_mla, k, scale,
                        out=None, lse=None, indices_out=None, stream=None):
    """decode_step through the entry point that allocates nothing (its
    workspace is the library's per-GPU scratch)."""
    if out is None:
        out = _out_like(kv, q_mla, d_latent)
    b, ic, lc = batch.struct(), index_cache(keys, key_scales), latent_cache(kv, kv_scales, d_latent)
    _check("dsa_decode_step_noalloc", lib().dsa_decode_step_noalloc(
        C.byref(b), C.byref(ic), _ptr(q_idx), _ptr(w), q_idx.shape[1], C.byref(lc), _ptr(q_mla), q_mla.shape[1],
        k, float(scale), _ptr(out), _ptr(lse), _ptr(indices_out), _stream(stream)))
    return out


def event_handles(events, stream=None):
    """ctypes array of the raw hipEvent_t handles of torch.cuda.Event objects
    (created with enable_timing=True); torch creates an event on its first
    record, so one not yet recorded is recorded once on the stream first."""
    s = stream or torch.cuda.current_stream()
    for e in events:
        if not e.cuda_event:
            e.record(s)
    return (C.c_void_p * len(events))(*[C.c_void_p(e.cuda_event) for e in events])


def decode_step_timed(batch: Batch, keys, key_scales, q_idx, w, kv, kv_scales, d_latent, q_mla, k, scale, events,
                      out=None, lse=None, indices_out=None, workspace=None, stream=None):
    """decode_step that also records `events` (STEP_EVENTS torch.cuda.Event) at
    its phase boundaries: start, after sampling, indexer, selection, attention."""
    if out is None:
        out = _out_like(kv, q_mla, d_latent)
    ws = _workspace(OP_DECODE_STEP, batch, k, q_mla.shape[1], q_mla.device, workspace)
    b, ic, lc = batch.struct(), index_cache(keys, key_scales), latent_cache(kv, kv_scales, d_latent)
    h = event_handles(events, stream)
    _check("dsa_decode_step_timed", lib().dsa_decode_step_timed(
        C.byref(b), C.byref(ic), _ptr(q_idx), _ptr(w), q_idx.shape[1], C.byref(lc), _ptr(q_mla),
        q_mla.shape[1], k, float(scale), _ptr(out), _ptr(lse), _ptr(indices_out), _ptr(ws), ws.numel(),
        _stream(stream), h, len(events)))
    return out


class HotCache:
    """Device state of a two-tier latent cache: `capacity` slots of latent
    rows (dtype and width of the host cache) in front of a paged latent cache
    kept in pinned host memory, for batches of `num_requests` requests of at
    most `max_context_len` tokens."""

    def __init__(self, capacity, num_requests, max_context_len, row_width, dtype, device="cuda"):
        self.capacity = int(capacity)
        self.kv = torch.empty((self.capacity, row_width), dtype=dtype, device=device)
        self.scales = (torch.empty(self.capacity, dtype=torch.float32, device=device)
                       if dtype in (torch.uint8, torch.float8_e4m3fn) else None)
        self.slot_of = torch.empty((num_requests, max_context_len), dtype=torch.int32, device=device)
        self.owner = torch.empty(self.capacity, dtype=torch.int64, device=device)
        self.last_use = torch.empty(self.capacity, dtype=torch.int32, device=device)
        self.clock = torch.zeros(1, dtype=torch.int32, device=device)

    def struct(self):
        return DsaHotCache(self.kv.data_ptr(), None if self.scales is None else self.scales.data_ptr(),
                           self.capacity, self.slot_of.data_ptr(), self.owner.data_ptr(),
                           self.last_use.data_ptr(), self.clock.data_ptr())

    def batch(self, batch: "Batch") -> "Batch":
        """The geometry of MLA over the hot set: one token per block, the slot
        table as page table."""
        return Batch(batch.context_lens, batch.query_start_loc, self.slot_of, 1, batch.max_q_len,
                     batch.max_context_len)


def hot_cache_reset(batch: "Batch", hot: HotCache, stream=None):
    b, h = batch.struct(), hot.struct()
    _check("dsa_hot_cache_reset", lib().dsa_hot_cache_reset(C.byref(b), C.byref(h), _stream(stream)))


def hot_cache_workspace(batch: "Batch", k: int, hot: HotCache, device="cuda") -> torch.Tensor:
    b = batch.struct()
    need = int(lib().dsa_hot_cache_workspace_size(C.byref(b), k, hot.capacity))
    return torch.empty(max(need, 256), dtype=torch.uint8, device=device)


def hot_cache_fetch(batch: "Batch", host_kv, host_scales, d_latent, indices, hot: HotCache, counts=None,
                    workspace=None, stream=None, phase="fetch"):
    """Make every token of `indices` resident in `hot` (host_kv / host_scales:
    the paged latent cache in pinned host memory).  phase "plan" or "copy"
    runs one half (dsa_hot_cache_plan / dsa_hot_cache_copy)."""
    k = indices.shape[1]
    b = batch.struct()
    if workspace is None:
        workspace = hot_cache_workspace(batch, k, hot, indices.device)
    c, h = latent_cache(host_kv, host_scales, d_latent), hot.struct()
    if phase == "plan":
        _check("dsa_hot_cache_plan", lib().dsa_hot_cache_plan(C.byref(b), C.byref(c), _ptr(indices), k, C.byref(h),
                                                              _ptr(workspace), workspace.numel(), _stream(stream)))
    else:
        fn = "dsa_hot_cache_fetch" if phase == "fetch" else "dsa_hot_cache_copy"
        if phase not in ("fetch", "copy"):
            raise ValueError("phase is fetch, plan or copy")
        _check(fn, getattr(lib(), fn)(C.byref(b), C.byref(c), _ptr(indices), k, C.byref(h), _ptr(counts),
                                      _ptr(workspace), workspace.numel(), _stream(stream)))
    return workspace


def read_probe(buf: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Read every byte of a device buffer once (bandwidth measurement helper)."""
    n = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(max(int(lib().dsa_read_probe_sink_size()), 4), dtype=torch.uint8, device=buf.device)
    _check("dsa_read_probe", lib().dsa_read_probe(_ptr(buf), n, _ptr(sink), sink.numel(), _stream(stream)))
    return sink


def page_probe(pages: torch.Tensor, page_bytes: int, scales: Optional[torch.Tensor], scale_bytes: int,
               block_ids: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Read the listed pages of a pool the way the decode indexer does, with
    no arithmetic (measurement helper); returns the per-lane XOR sink."""
    if block_ids.dtype != torch.int32 or not block_ids.is_cuda:
        raise ValueError("block_ids must be an int32 device tensor")
    if sink is None:
        sink = torch.empty(int(lib().dsa_page_probe_sink_size()) // 4, dtype=torch.int32, device=pages.device)
    _check("dsa_page_probe", lib().dsa_page_probe(_ptr(pages), page_bytes, _ptr(scales), scale_bytes,
                                                  _ptr(block_ids), block_ids.numel(), _ptr(sink),
                                                  sink.numel() * sink.element_size(), _stream(stream)))
    return sink


def row_probe(pool: torch.Tensor, row_bytes: int, row_ids: torch.Tensor, rows_per_wg: int,
              sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Gather the listed rows of a pool the way the 128-head sparse-MLA tile
    does, with no arithmetic (measurement helper); returns the
    per-workgroup XOR sink."""
    if row_ids.dtype != torch.int32 or not row_ids.is_cuda:
        raise ValueError("row_ids must be an int32 device tensor")
    n = row_ids.numel()
    if sink is None:
        words = max(int(lib().dsa_row_probe_sink_size(n, rows_per_wg)) // 4, 1)
        sink = torch.empty(words, dtype=torch.int32, device=pool.device)
    _check("dsa_row_probe", lib().dsa_row_probe(_ptr(pool), row_bytes, _ptr(row_ids), n, rows_per_wg, _ptr(sink),
                                                sink.numel() * sink.element_size(), _stream(stream)))
    return sink


def check_device() -> int:
    return int(lib().dsa_check_device())


def check_batch(batch: "Batch", num_blocks: int = 0, indices: Optional[torch.Tensor] = None, k: int = 0,
                stream=None) -> int:
    """dsa_check_batch: waits for `stream` and returns the OR of the
    CHECK_* bits that failed (0 when the batch's device values hold)."""
    b = batch.struct()
    if indices is not None:
        k = k or indices.shape[-1]
    failed = C.c_uint32(0)
    st = lib().dsa_check_batch(C.byref(b), num_blocks, _ptr(indices), k, C.byref(failed), _stream(stream))
    if st not in (DSA_OK, ERR_BAD_DEVICE_ARG):
        raise DsaError("dsa_check_batch", st)
    return int(failed.value)
