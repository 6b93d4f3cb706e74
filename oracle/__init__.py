"""CPU oracle for the DSA step (ctypes front end of ``dsa_oracle.c``).

TEST INFRASTRUCTURE ONLY: used by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg.  The product library never imports it, and it
imports nothing from the product library.  All arithmetic lives in the C file
(double precision, one query token at a time); this module only passes arrays
in and out and runs independent query rows on a thread pool (ctypes releases
the GIL during each call).

Sources: SemiAnalysis GLM-5.3 article, section "DeepSeek Sparse Attention"
(lightning indexer, top-K, dense below K) and sections "Sparse MLA" /
"MLA Modifications" (MQA-mode P = Q K^T, O = P V with V the first d columns
of the cached latent row).

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
closed forms, special cases that reduce to a library routine (numpy dot,
torch's scaled_dot_product_attention), brute force on tiny inputs and
hand-worked fixtures in ``tests/golden/``.
"""
from __future__ import annotations

import concurrent.futures as _fut
import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB = os.path.join(_HERE, "libdsa_oracle.so")

CODE = {"f32": 0, "bf16": 1, "e4m3": 2, "mxfp4": 3}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-Wall",
                               "-Wextra", "-Werror", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = C.CDLL(_LIB)
        vp, i32p, f32p, f64p = C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_float), C.POINTER(C.c_double)
        L.orc_bf16_to_f64.argtypes = [C.c_uint16]
        L.orc_bf16_to_f64.restype = C.c_double
        L.orc_e4m3_to_f64.argtypes = [C.c_uint8]
        L.orc_e4m3_to_f64.restype = C.c_double
        L.orc_e2m1_to_f64.argtypes = [C.c_uint8]
        L.orc_e2m1_to_f64.restype = C.c_double
        L.orc_e8m0_to_f64.argtypes = [C.c_uint8]
        L.orc_e8m0_to_f64.restype = C.c_double
        L.orc_indexer_scores.argtypes = [vp, f32p, C.c_int, C.c_int, i32p, C.c_int,
                                         vp, C.c_int, f32p, C.c_int, C.c_int, f64p]
        L.orc_indexer_scores.restype = None
        L.orc_topk.argtypes = [f64p, C.c_int, C.c_int, i32p]
        L.orc_topk.restype = C.c_int
        L.orc_sparse_mla.argtypes = [vp, f32p, C.c_int, C.c_int, C.c_int, i32p, C.c_int,
                                     vp, C.c_int, C.c_int, i32p, C.c_int, C.c_double, f64p, f64p]
        L.orc_sparse_mla.restype = None
        _lib = L
    return _lib


def _p(a, t):
    return None if a is None else a.ctypes.data_as(C.POINTER(t))


def _v(a):
    return C.c_void_p(a.ctypes.data)


# ------------------------------------------------------------- primitives
def decode_bf16(bits) -> np.ndarray:
    L = lib()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([L.orc_bf16_to_f64(int(x)) for x in b], dtype=np.float64)


def decode_e4m3(codes) -> np.ndarray:
    L = lib()
    c = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([L.orc_e4m3_to_f64(int(x)) for x in c], dtype=np.float64)


def decode_e2m1(codes) -> np.ndarray:
    """OCP FP4 E2M1 codes (low 4 bits of each value) to float64."""
    L = lib()
    c = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([L.orc_e2m1_to_f64(int(x) & 0xF) for x in c], dtype=np.float64)


def decode_e8m0(exps) -> np.ndarray:
    """OCP E8M0 scale bytes to float64 (2^(e-127), NaN for 255)."""
    L = lib()
    e = np.asarray(exps, dtype=np.uint8).ravel()
    return np.array([L.orc_e8m0_to_f64(int(x)) for x in e], dtype=np.float64)


def indexer_scores(keys, key_scales, key_code, page_row, block_size, q, q_code, w, n):
    """Scores of one query over its visible tokens [0, n) (float64 [n]).

    keys [nblk][bs][dim] (MXFP4: [nblk][bs * (dim/2 + dim/32)] bytes, codes
    then E8M0 scales per block); key_scales [nblk][bs] or None; q [H][dim];
    w [H].
    """
    keys = np.ascontiguousarray(keys)
    q = np.ascontiguousarray(q)
    w = np.ascontiguousarray(w, dtype=np.float32)
    page_row = np.ascontiguousarray(page_row, dtype=np.int32)
    ks = None if key_scales is None else np.ascontiguousarray(key_scales, dtype=np.float32)
    H, dim = q.shape
    if key_code == "mxfp4":
        assert dim % 32 == 0 and keys.shape[-1] == block_size * (dim // 2 + dim // 32)
    else:
        assert keys.shape[-1] == dim
    assert w.shape == (H,)
    out = np.empty(max(n, 1), dtype=np.float64)
    lib().orc_indexer_scores(_v(keys), _p(ks, C.c_float), CODE[key_code], dim,
                             _p(page_row, C.c_int32), block_size, _v(q), CODE[q_code],
                             _p(w, C.c_float), H, n, _p(out, C.c_double))
    return out[:n]


def topk(scores, k) -> np.ndarray:
    """Top-k indices (score desc, index asc) of a float64 score vector."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    n = s.shape[0]
    out = np.empty(max(min(n, k), 1), dtype=np.int32)
    cnt = lib().orc_topk(_p(s, C.c_double), n, k, _p(out, C.c_int32))
    return out[:cnt]


def sparse_mla(kv, kv_scales, kv_code, d_latent, d_rope, page_row, block_size,
               q, q_code, sel, scale):
    """Sparse MQA-mode MLA of one query: returns (out [H][d] f64, lse [H] f64)."""
    kv = np.ascontiguousarray(kv)
    q = np.ascontiguousarray(q)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    page_row = np.ascontiguousarray(page_row, dtype=np.int32)
    ks = None if kv_scales is None else np.ascontiguousarray(kv_scales, dtype=np.float32)
    H = q.shape[0]
    assert q.shape[1] == d_latent + d_rope == kv.shape[-1]
    out = np.empty((H, d_latent), dtype=np.float64)
    lse = np.empty(H, dtype=np.float64)
    lib().orc_sparse_mla(_v(kv), _p(ks, C.c_float), CODE[kv_code], d_latent, d_rope,
                         _p(page_row, C.c_int32), block_size, _v(q), CODE[q_code], H,
                         _p(sel, C.c_int32), int(sel.shape[0]), float(scale),
                         _p(out, C.c_double), _p(lse, C.c_double))
    return out, lse


# ------------------------------------------------------- workload drivers
def _q_code(wl):
    return "f32" if wl.idx_dtype == "f32" else "e4m3"


def _qm_code(wl):
    return "f32" if wl.kv_dtype == "f32" else "bf16"


def query_positions(wl):
    """(request r, position p, visible count n) of every query row, in row order.

    Reading of the pages (section "DeepSeek Sparse Attention": each query
    token is scored against the tokens before it; the MTP workload's two
    query tokens are causal among themselves): a request's context length L
    counts its q_len new query tokens, which are its last q_len positions;
    query j (0-based) sits at p = L - q_len + j and sees tokens [0, p], so
    n = p + 1.  Pinned by tests/golden/positions_hand.json."""
    out = []
    for r in range(len(wl.context_lens)):
        L, ql = int(wl.context_lens[r]), int(wl.q_lens[r])
        for j in range(ql):
            p = L - ql + j
            out.append((r, p, p + 1))
    return out


def row_position(wl, t):
    """query_positions(wl)[t] for one row, without listing every row."""
    qsl = np.asarray(wl.query_start_loc)
    r = int(np.searchsorted(qsl, t, side="right")) - 1
    while int(qsl[r + 1]) <= t:                  # requests with no query rows
        r += 1
    L, ql = int(wl.context_lens[r]), int(wl.q_lens[r])
    p = L - ql + (t - int(qsl[r]))
    return r, p, p + 1


def query_scores(wl, t):
    """Indexer scores of query row t of a workload (float64 [n_t])."""
    r, p, n = row_position(wl, t)
    return indexer_scores(wl.idx_keys, wl.idx_scales, wl.idx_dtype, wl.page_table[r],
                          wl.block_size, wl.q_idx[t], _q_code(wl), wl.w[t], n)


def query_mla(wl, t, sel, layer=1):
    """Sparse MLA of query row t over `sel` on layer 1 or 2's latent cache."""
    r, p, n = row_position(wl, t)
    kv, ks, q = (wl.kv, wl.kv_scales, wl.q_mla) if layer == 1 else (wl.kv2, wl.kv2_scales, wl.q_mla2)
    return sparse_mla(kv, ks, wl.kv_dtype, wl.d_latent, wl.d_rope, wl.page_table[r],
                      wl.block_size, q[t], _qm_code(wl), sel, wl.softmax_scale)


def run_step(wl, rows=None, threads=None, layers=1, keep_scores=True):
    """Whole DSA step for the chosen query rows of a workload.

    Returns {t: dict(scores, indices, out, lse[, out2, lse2])}.  Rows run in
    parallel on `threads` host threads.
    """
    rows = list(range(wl.total_q)) if rows is None else list(rows)
    threads = threads or min(16, os.cpu_count() or 1)

    def one(t):
        sc = query_scores(wl, t)
        idx = topk(sc, wl.topk)
        out, lse = query_mla(wl, t, idx, 1)
        res = dict(indices=idx, out=out, lse=lse)
        if keep_scores:
            res["scores"] = sc
        if layers >= 2:
            res["out2"], res["lse2"] = query_mla(wl, t, idx, 2)
        return t, res

    if threads == 1 or len(rows) == 1:
        return dict(one(t) for t in rows)
    with _fut.ThreadPoolExecutor(threads) as ex:
        return dict(ex.map(one, rows))
