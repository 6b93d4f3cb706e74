"""Seeded synthetic inputs for the DSA decode / prefill step.

This module only draws random numbers and encodes them into the storage
formats the caches use (fp32, bf16 bit patterns, OCP e4m3fn codes).  It holds
none of the method's arithmetic: no scores, no selection, no attention.  Both
the CPU oracle (``oracle/``) and the HIP library are fed from the arrays it
returns, so the two sides always see the same bytes.

Workloads follow the shapes of the DeepSeek Sparse Attention step as described
for the GLM-5 family ("DeepSeek Sparse Attention" section of the SemiAnalysis
GLM-5.3 article: a multi-head lightning indexer over single-head keys, top-K
selection, then MQA-mode MLA over a 512-wide latent plus a 64-wide RoPE part).

Encoding rules (readings of what the pages leave open):
  * index keys: each token's N(0,1) row is divided by sigma = amax/448 and
    rounded to e4m3fn; sigma is stored as the token's fp32 scale.
  * indexer queries: each (token, head) row is scaled the same way; the scale
    is folded into that head's weight w (exact because ReLU is positively
    homogeneous), so the kernel sees raw e4m3 q and an fp32 w.
  * latent rows: N(0,1) rounded to bf16, or for the fp8 latent cache the same
    per-token amax/448 scaling as the keys (one scale for all 576 columns).
  * pool data is drawn per slab of 64 physical blocks from its own stream
    ``default_rng([seed, tag, slab])`` so that very large pools can be drawn
    in parallel and any block can be redrawn on its own.
"""
from __future__ import annotations

import concurrent.futures as _fut
import dataclasses
import math
import os
from typing import Optional

import numpy as np
import torch

E4M3_MAX = 448.0
SLAB_BLOCKS = 64

# Stream tags for per-slab generators.
_TAG_KEYS, _TAG_KV, _TAG_KV2 = 11, 12, 13

# The five workloads.  Field meanings are in ``DSAConfig``.
CONFIGS = {
    # 1 request, 1 query, L=4096, fp32 everything, small head shapes.
    "tiny_fp32_l4096": dict(
        seed=0, batch=1, context_lens=[4096], q_len=1,
        idx_heads=4, idx_dim=32, idx_dtype="f32", topk=256,
        mla_heads=16, d_latent=64, d_rope=16, kv_dtype="f32",
        block_size=64, shuffle_pages=False, softmax_scale=1.0 / math.sqrt(80.0)),
    # one layer, batch 1, L=32768, production head shapes, paged + shuffled.
    "single_b1_l32768": dict(
        seed=1, batch=1, context_lens=[32768], q_len=1,
        idx_heads=64, idx_dim=128, idx_dtype="e4m3", topk=2048,
        mla_heads=128, d_latent=512, d_rope=64, kv_dtype="bf16",
        block_size=64, shuffle_pages=True, softmax_scale=1.0 / math.sqrt(576.0)),
    # batch 64, per-request L ~ U[8K, 128K]: the decode throughput workload.
    "batched_b64_l8k_128k": dict(
        seed=2, batch=64, context_lens=("uniform", 8192, 131072), q_len=1,
        idx_heads=64, idx_dim=128, idx_dtype="e4m3", topk=2048,
        mla_heads=128, d_latent=512, d_rope=64, kv_dtype="bf16",
        block_size=64, shuffle_pages=True, softmax_scale=1.0 / math.sqrt(576.0)),
    # batch 8 at L=202752, 2 query tokens per request (causal among them),
    # fp8 latent cache with a per-token scale.
    "mtp_b8_l202752": dict(
        seed=3, batch=8, context_lens=[202752] * 8, q_len=2,
        idx_heads=64, idx_dim=128, idx_dtype="e4m3", topk=2048,
        mla_heads=128, d_latent=512, d_rope=64, kv_dtype="e4m3",
        block_size=64, shuffle_pages=True, softmax_scale=1.0 / math.sqrt(576.0)),
    # chunked prefill: 4096 new tokens after 131072 cached ones; a second
    # layer reuses the first layer's selection on its own latent cache.
    "prefill_q4096_l131072": dict(
        seed=4, batch=1, context_lens=[131072 + 4096], q_len=4096,
        idx_heads=64, idx_dim=128, idx_dtype="e4m3", topk=2048,
        mla_heads=128, d_latent=512, d_rope=64, kv_dtype="bf16",
        block_size=64, shuffle_pages=True, softmax_scale=1.0 / math.sqrt(576.0),
        layers=2),
}

# Short aliases in file order of the workload list.
CONFIG_ORDER = list(CONFIGS)


@dataclasses.dataclass
class Workload:
    """All arrays of one synthetic step, as raw storage codes (numpy, host)."""
    name: str
    seed: int
    batch: int
    context_lens: np.ndarray      # int32 [B]  tokens in cache incl. new queries
    q_lens: np.ndarray            # int32 [B]
    query_start_loc: np.ndarray   # int32 [B+1]
    page_table: np.ndarray        # int32 [B][max_blocks]  physical block ids
    block_size: int
    num_blocks: int
    idx_heads: int
    idx_dim: int
    idx_dtype: str                # "f32" | "e4m3" | "mxfp4"
    idx_keys: np.ndarray          # [nblk][bs][dim] float32 or uint8 codes; mxfp4: [nblk][bs*(dim/2+dim/32)]
    idx_scales: Optional[np.ndarray]  # float32 [nblk][bs] or None
    q_idx: np.ndarray             # [T][H_idx][dim] float32 or uint8 codes
    w: np.ndarray                 # float32 [T][H_idx]
    topk: int
    mla_heads: int
    d_latent: int
    d_rope: int
    kv_dtype: str                 # "f32" | "bf16" | "e4m3"
    kv: np.ndarray                # [nblk][bs][d+r] float32 / uint16 bf16 bits / uint8 codes
    kv_scales: Optional[np.ndarray]   # float32 [nblk][bs] or None
    q_mla: np.ndarray             # [T][H][d+r] float32 or uint16 bf16 bits
    softmax_scale: float
    layers: int = 1
    kv2: Optional[np.ndarray] = None
    kv2_scales: Optional[np.ndarray] = None
    q_mla2: Optional[np.ndarray] = None

    @property
    def total_q(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max())

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max())

    @property
    def max_blocks(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def d_qk(self) -> int:
        return self.d_latent + self.d_rope


# ----------------------------------------------------------------- encoders
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even) bit patterns, via torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3fn codes (nearest even), saturating at +-448."""
    x = np.clip(np.asarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _rowwise_e4m3(x: np.ndarray):
    """Per-row amax/448 scaling to e4m3 codes; returns (codes, scale)."""
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)
    codes = e4m3_codes(x / scale[..., None])
    return codes, scale


# ------------------------------------------------------------ pool drawing
# Non-negative FP4 E2M1 magnitudes in code order (OCP Microscaling Formats
# v1.0), for quantising synthetic keys: codes are the generator's output,
# their decoding belongs to the oracle.
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def _mxfp4_block_codes(x: np.ndarray):
    """MX quantisation of x [..., dim] (dim % 32 == 0): per 32-element block
    a power-of-two scale 2^E with E = floor(log2 amax) - 2 (the largest E2M1
    exponent), elements rounded to the nearest E2M1 value (saturating at 6).
    Returns (packed codes [..., dim/2] uint8, E8M0 bytes [..., dim/32])."""
    sh = x.shape
    blk = x.reshape(sh[:-1] + (sh[-1] // 32, 32))
    amax = np.abs(blk).max(axis=-1)
    e = np.where(amax > 0, np.floor(np.log2(np.maximum(amax, 1e-30))) - 2, 0).astype(np.int32)
    e = np.clip(e, -126, 127)
    y = np.abs(blk) / np.exp2(e)[..., None].astype(np.float32)
    mid = (_E2M1_GRID[1:] + _E2M1_GRID[:-1]) / 2
    mag = np.searchsorted(mid, np.minimum(y, 6.0), side="left").astype(np.uint8)
    code = mag | np.where(blk < 0, 8, 0).astype(np.uint8)
    code = code.reshape(sh)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def _draw_slab(seed, tag, slab, nblk_total, bs, width, enc):
    b0 = slab * SLAB_BLOCKS
    nb = min(SLAB_BLOCKS, nblk_total - b0)
    rng = np.random.default_rng([seed, tag, slab])
    x = rng.standard_normal((nb, bs, width), dtype=np.float32)
    if enc == "f32":
        return b0, x, None
    if enc == "mxfp4":   # per block: bs rows of codes, then bs rows of E8M0 scales
        packed, exps = _mxfp4_block_codes(x)
        data = np.concatenate([packed.reshape(nb, -1), exps.reshape(nb, -1)], axis=1)
        sigma = rng.uniform(0.5, 2.0, size=(nb, bs)).astype(np.float32)
        return b0, data, sigma
    if enc == "bf16":
        return b0, bf16_bits(x), None
    codes, scale = _rowwise_e4m3(x)
    return b0, codes, scale


def draw_pool(seed, tag, nblk, bs, width, enc, threads=None):
    """Draw a [nblk][bs][width] pool in the given encoding, slab by slab."""
    dt = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8, "mxfp4": np.uint8}[enc]
    shape = (nblk, bs * (width // 2 + width // 32)) if enc == "mxfp4" else (nblk, bs, width)
    data = np.empty(shape, dtype=dt)
    scales = np.empty((nblk, bs), dtype=np.float32) if enc in ("e4m3", "mxfp4") else None
    nslab = (nblk + SLAB_BLOCKS - 1) // SLAB_BLOCKS
    threads = threads or min(16, os.cpu_count() or 1)

    def job(s):
        b0, d, sc = _draw_slab(seed, tag, s, nblk, bs, width, enc)
        data[b0:b0 + d.shape[0]] = d
        if scales is not None:
            scales[b0:b0 + d.shape[0]] = sc

    if nslab == 1 or threads == 1:
        for s in range(nslab):
            job(s)
    else:
        with _fut.ThreadPoolExecutor(threads) as ex:
            list(ex.map(job, range(nslab)))
    return data, scales


# ----------------------------------------------------------------- builder
def make_workload(name: str = "tiny_fp32_l4096", **overrides) -> Workload:
    """Build a workload from a named config, with optional field overrides.

    Overrides accept any config key (``batch``, ``context_lens`` as a list,
    ``q_len``, head shapes, ``topk``, ``kv_dtype``, ``seed``, ...).  Draw
    order from the master generator is fixed: context lengths, page-table
    permutation, indexer q, w, MLA q (layer 1), MLA q (layer 2).
    """
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    seed = int(cfg["seed"])
    rng = np.random.default_rng(seed)
    B = int(cfg["batch"])
    bs = int(cfg["block_size"])

    cl = cfg["context_lens"]
    if isinstance(cl, tuple) and cl[0] == "uniform":
        ctx = rng.integers(cl[1], cl[2], size=B, endpoint=True).astype(np.int32)
    else:
        ctx = np.asarray(cl, dtype=np.int32)
        if ctx.size == 1 and B > 1:
            ctx = np.full(B, int(ctx[0]), dtype=np.int32)
    assert ctx.shape == (B,)
    ql = cfg["q_len"]
    q_lens = (np.asarray(ql, dtype=np.int32) if np.ndim(ql)
              else np.full(B, int(ql), dtype=np.int32))
    q_lens = np.minimum(q_lens, ctx)
    qsl = np.zeros(B + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(q_lens)
    T = int(qsl[-1])

    nblocks_r = (ctx + bs - 1) // bs
    nblk = int(nblocks_r.sum())
    max_blocks = int(nblocks_r.max()) if B else 0
    order = (rng.permutation(nblk) if cfg["shuffle_pages"]
             else np.arange(nblk)).astype(np.int32)
    pt = np.zeros((B, max(max_blocks, 1)), dtype=np.int32)
    off = 0
    for r in range(B):
        pt[r, :nblocks_r[r]] = order[off:off + nblocks_r[r]]
        off += nblocks_r[r]

    Hi, Di = int(cfg["idx_heads"]), int(cfg["idx_dim"])
    idt = cfg["idx_dtype"]
    keys, kscales = draw_pool(seed, _TAG_KEYS, nblk, bs, Di, idt)

    qf = rng.standard_normal((T, Hi, Di), dtype=np.float32)
    w = rng.uniform(0.0, 1.0, size=(T, Hi)).astype(np.float32)
    if idt == "f32":
        q_idx = qf
    else:
        q_idx, qscale = _rowwise_e4m3(qf)
        w = (w * qscale).astype(np.float32)

    H, d, r_ = int(cfg["mla_heads"]), int(cfg["d_latent"]), int(cfg["d_rope"])
    kvdt = cfg["kv_dtype"]
    kv, kvs = draw_pool(seed, _TAG_KV, nblk, bs, d + r_, kvdt)
    qm = rng.standard_normal((T, H, d + r_), dtype=np.float32)
    q_mla = qm if kvdt == "f32" else bf16_bits(qm)

    wl = Workload(
        name=name, seed=seed, batch=B, context_lens=ctx, q_lens=q_lens,
        query_start_loc=qsl, page_table=pt, block_size=bs, num_blocks=nblk,
        idx_heads=Hi, idx_dim=Di, idx_dtype=idt, idx_keys=keys, idx_scales=kscales,
        q_idx=q_idx, w=w, topk=int(cfg["topk"]), mla_heads=H, d_latent=d, d_rope=r_,
        kv_dtype=kvdt, kv=kv, kv_scales=kvs, q_mla=q_mla,
        softmax_scale=float(cfg["softmax_scale"]), layers=int(cfg.get("layers", 1)))
    if wl.layers >= 2:
        wl.kv2, wl.kv2_scales = draw_pool(seed, _TAG_KV2, nblk, bs, d + r_, kvdt)
        qm2 = rng.standard_normal((T, H, d + r_), dtype=np.float32)
        wl.q_mla2 = qm2 if kvdt == "f32" else bf16_bits(qm2)
    return wl


def peaked_queries(wl: Workload, alpha: float, rows) -> np.ndarray:
    """MLA queries q[t,h] = alpha * latent row of a chosen visible token.

    ``rows`` gives, per query row t, the logical token whose latent row is
    copied (scaled by alpha) into every head's query.  Drives the softmax
    towards one-hot so outputs are O(1) rather than O(1/sqrt(K)).  Works for
    the bf16 and f32 caches.
    """
    q = np.empty((wl.total_q, wl.mla_heads, wl.d_qk), dtype=np.float32)
    t = 0
    for r in range(wl.batch):
        for j in range(int(wl.q_lens[r])):
            s = int(rows[t])
            blk = int(wl.page_table[r, s // wl.block_size])
            row = wl.kv[blk, s % wl.block_size]
            if wl.kv_dtype == "bf16":
                rowf = (row.astype(np.uint32) << 16).view(np.float32)
            elif wl.kv_dtype == "f32":
                rowf = row
            else:
                raise ValueError("peaked queries need a bf16 or f32 latent cache")
            q[t, :, :] = alpha * rowf[None, :]
            t += 1
    return q if wl.kv_dtype == "f32" else bf16_bits(q)


# ------------------------------------------------------------ device copy
def _torch_of(a: np.ndarray, device):
    """numpy storage codes -> torch tensor with the matching storage dtype."""
    if a.dtype == np.uint16:    # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_device(wl: Workload, device="cuda") -> dict:
    """Copy every array of a workload to `device` (storage dtypes kept)."""
    d = dict(
        context_lens=_torch_of(wl.context_lens, device),
        query_start_loc=_torch_of(wl.query_start_loc, device),
        page_table=_torch_of(wl.page_table, device),
        idx_keys=_torch_of(wl.idx_keys, device),
        idx_scales=None if wl.idx_scales is None else _torch_of(wl.idx_scales, device),
        q_idx=_torch_of(wl.q_idx, device),
        w=_torch_of(wl.w, device),
        kv=_torch_of(wl.kv, device),
        kv_scales=None if wl.kv_scales is None else _torch_of(wl.kv_scales, device),
        q_mla=_torch_of(wl.q_mla, device),
    )
    if wl.layers >= 2:
        d["kv2"] = _torch_of(wl.kv2, device)
        d["kv2_scales"] = None if wl.kv2_scales is None else _torch_of(wl.kv2_scales, device)
        d["q_mla2"] = _torch_of(wl.q_mla2, device)
    return d
