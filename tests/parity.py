"""Glue for the GPU parity tests: run the HIP library and the CPU oracle on the
same seeded workload and compare by the rules of the method.

Comparison rules:
  * selections: each row holds min(K, n) distinct visible indices, ascending,
    then -1 padding; the symmetric difference with the oracle's set may only
    contain tokens whose oracle score lies within 1e-4 (relative) of the
    oracle's K-th score (tokens on the selection boundary, where fp32 and
    fp64 rounding may order them differently);
  * outputs: max-abs <= 2e-2 for bf16 paths and <= 1e-4 for the fp32 path
    end to end (GPU selection vs the oracle's own selection); against the
    oracle evaluated on the GPU's own selection additionally a relative
    Frobenius bound (1e-2 bf16, 1e-5 fp32).  The Frobenius bound is not
    applied end to end: one boundary token swapped at long contexts moves an
    output by ~p*|v| ~ 5e-4 per element, about 1% of its norm.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import sparse_attention_dsa_amd as dsa
import workloads

BAND = 1e-4


def score_bound(wl, t):
    """Rounding bound of query row t's indexer scores computed in fp32.

    A score is a sum over heads of w_h * ReLU(q_h . k_s) times sigma_s: a
    dot of `dim` exact products, a head sum of `heads` terms and two
    products, i.e. at most n = dim + heads + 2 fp32 roundings in any order.
    Its error is then at most gamma_n = n u / (1 - n u) (u = 2^-24) times
    the same expression on absolute values, sigma_s * sum_h |w_h| sum_d
    |q_hd k_sd|, which the oracle evaluates on the inputs' magnitudes
    (sign bit cleared in the e4m3 codes)."""
    r, p, n = oracle.query_positions(wl)[t]
    if wl.idx_dtype == "f32":
        keys, q = np.abs(wl.idx_keys), np.abs(wl.q_idx[t])
    elif wl.idx_dtype == "mxfp4":   # both nibbles' sign bits cleared; the E8M0 bytes kept
        keys, q = wl.idx_keys.copy(), wl.q_idx[t] & np.uint8(0x7F)
        nc = wl.block_size * wl.idx_dim // 2
        keys[:, :nc] &= np.uint8(0x77)
    else:
        keys, q = wl.idx_keys & np.uint8(0x7F), wl.q_idx[t] & np.uint8(0x7F)
    mag = oracle.indexer_scores(keys, wl.idx_scales, wl.idx_dtype, wl.page_table[r], wl.block_size, q,
                                "f32" if wl.idx_dtype == "f32" else "e4m3", np.abs(wl.w[t]), n)
    m = wl.idx_dim + wl.idx_heads + 2
    u = 2.0 ** -24
    return m * u / (1.0 - m * u) * mag


def check_scores(wl, t, got):
    """GPU scores of row t (its first n entries) against the oracle, within
    the fp32 rounding bound of each score."""
    ref = oracle.query_scores(wl, t)
    assert got.shape == ref.shape
    err = np.abs(got.astype(np.float64) - ref)
    bound = score_bound(wl, t)
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, "row %d: %d scores outside the fp32 bound, first at %d: got %r ref %r bound %r" % (
        t, bad.size, bad[0], float(got[bad[0]]), float(ref[bad[0]]), float(bound[bad[0]]))


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def upload(wl, dev="cuda"):
    d = workloads.to_device(wl, dev)
    if wl.idx_dtype == "mxfp4":
        d["idx_keys"] = dsa.binding.MxFp4Keys(d["idx_keys"], wl.idx_dim)
    batch = dsa.Batch(d["context_lens"], d["query_start_loc"], d["page_table"], wl.block_size,
                      wl.max_q_len, wl.max_context_len)
    return batch, d


def gpu_step(wl, batch, d, lse=True, fused=False, events=None):
    """dsa_decode_step (or, with fused, dsa_decode_step_fused) on the device;
    returns (out f32 numpy, lse, indices)."""
    T, H = wl.total_q, wl.mla_heads
    idx = torch.empty((T, wl.topk), dtype=torch.int32, device="cuda")
    lse_t = torch.empty((T, H), dtype=torch.float32, device="cuda") if lse else None
    args = (batch, d["idx_keys"], d["idx_scales"], d["q_idx"], d["w"], d["kv"], d["kv_scales"], wl.d_latent,
            d["q_mla"], wl.topk, wl.softmax_scale)
    if fused:
        out = dsa.decode_step_fused(*args, lse=lse_t, indices_out=idx, events=events)
    else:
        out = dsa.decode_step(*args, lse=lse_t, indices_out=idx)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy(), None if lse_t is None else lse_t.cpu().numpy(), idx.cpu().numpy())


def check_selection(sel_row, scores_orc, K, band=BAND):
    """Checks one GPU selection row against the oracle's scores; returns |diff|."""
    n = scores_orc.shape[0]
    m = min(K, n)
    sel = np.asarray(sel_row)
    assert sel.shape == (K,)
    assert (sel[:m] >= 0).all(), "missing selections"
    assert (sel[m:] == -1).all(), "padding must be -1"
    s = sel[:m]
    assert (np.diff(s) > 0).all(), "indices must be unique and ascending"
    assert s[-1] < n, "non-causal index"
    ref = oracle.topk(scores_orc, K)
    diff = set(s.tolist()) ^ set(ref.tolist())
    if diff:
        assert n > K, "dense rows must select every visible token"
        kth = float(scores_orc[ref[-1]])
        bad = [x for x in diff if abs(float(scores_orc[x]) - kth) > band * abs(kth)]
        assert not bad, "selection differs outside the tie band: %s" % bad[:8]
    return len(diff)


def check_out(gpu, ref, fp32, same_selection=True):
    atol = 1e-4 if fp32 else 2e-2
    rel_bound = 1e-5 if fp32 else 1e-2
    err = np.abs(gpu - ref).max()
    rel = np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err <= atol, "max abs err %g > %g" % (err, atol)
    if same_selection:
        assert rel <= rel_bound, "relative Frobenius err %g > %g" % (rel, rel_bound)
    return err, rel


def check_step_rows(wl, rows, out, lse, idx, threads=16, layer=1):
    """Oracle-check the chosen query rows of a GPU step result."""
    fp32 = wl.kv_dtype == "f32"
    res = oracle.run_step(wl, rows=rows, threads=threads)
    worst = 0.0
    for t in rows:
        r = res[t]
        nd = check_selection(idx[t], r["scores"], wl.topk)
        # end to end against the oracle's own selection
        check_out(out[t], r["out"], fp32, same_selection=(nd == 0))
        # and against the oracle evaluated on the GPU's selection
        sel = idx[t][idx[t] >= 0]
        o2, l2 = oracle.query_mla(wl, t, sel, layer)
        err, _ = check_out(out[t], o2, fp32)
        worst = max(worst, err)
        if lse is not None:
            np.testing.assert_allclose(lse[t], l2, rtol=0, atol=1e-3 if not fp32 else 1e-5)
    return worst
