"""The device-side argument check (dsa_check_batch, and every entry point
with DSA_DEBUG set): each kind of bad query start, context length, page id
and selection entry is flagged with its own bit, values outside what a
request uses are not, and in debug mode every entry point returns
DSA_ERR_BAD_DEVICE_ARG without launching its work, while valid calls give
the same results as without the check.  The bad values given to the entry
points stay inside the real buffers (a page id below the real pool's size
but at or above the stated one, an index inside a used page), so a check
that missed one would read valid memory, not fault."""
import numpy as np
import pytest
import torch

import sparse_attention_dsa_amd as dsa
import workloads
from parity import log, upload
from sparse_attention_dsa_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert B.check_device() == 0, "not a gfx950 device"


def _wl():
    return workloads.make_workload("single_b1_l32768", batch=3, context_lens=[5000, 300, 2049], seed=31)


def _batch(d, wl, ctx=None, qsl=None, pt=None, max_q_len=None):
    return dsa.Batch(d["context_lens"] if ctx is None else ctx, d["query_start_loc"] if qsl is None else qsl,
                     d["page_table"] if pt is None else pt, wl.block_size,
                     wl.max_q_len if max_q_len is None else max_q_len, wl.max_context_len)


def _selection(wl, d, batch):
    idx = torch.empty((wl.total_q, wl.topk), dtype=torch.int32, device="cuda")
    dsa.decode_step(batch, d["idx_keys"], d["idx_scales"], d["q_idx"], d["w"], d["kv"], d["kv_scales"], wl.d_latent,
                    d["q_mla"], wl.topk, wl.softmax_scale, indices_out=idx)
    torch.cuda.synchronize()
    return idx


def test_check_batch_accepts_valid_batch():
    wl = _wl()
    batch, d = upload(wl)
    assert B.check_batch(batch, wl.num_blocks) == 0
    idx = _selection(wl, d, batch)
    assert (idx[1] == -1).any()                     # the short row is padded
    assert B.check_batch(batch, wl.num_blocks, idx) == 0
    assert B.check_batch(batch, 0, idx) == 0        # pool size not stated


@pytest.mark.parametrize("case", ["qsl_start", "qsl_end", "qsl_decreasing", "q_len_over_max", "ctx_over_max",
                                  "ctx_below_q_len", "page_negative", "page_beyond_pool", "page_unused",
                                  "page_pool_unstated", "index_not_visible", "index_padding"])
def test_check_batch_flags(case):
    wl = _wl()
    batch, d = upload(wl)
    ctx, qsl, pt = d["context_lens"].clone(), d["query_start_loc"].clone(), d["page_table"].clone()
    idx = _selection(wl, d, batch)
    nblk, want, pool, max_q = wl.num_blocks, 0, wl.num_blocks, None
    used = [-(-int(L) // wl.block_size) for L in wl.context_lens]
    if case == "qsl_start":
        qsl[0] = 1
        want = B.CHECK_QUERY_START
    elif case == "qsl_end":
        qsl[-1] = wl.total_q + 1
        want = B.CHECK_QUERY_START
    elif case == "qsl_decreasing":
        qsl[1], qsl[2] = 2, 1
        want = B.CHECK_QUERY_START
    elif case == "q_len_over_max":   # rows 0..2 as [0, 2), [2, 2), [2, 3)
        qsl[1], qsl[2] = 2, 2
        want = B.CHECK_QUERY_START
    elif case == "ctx_over_max":
        ctx[2] = wl.max_context_len + 1
        want = B.CHECK_CONTEXT
    elif case == "ctx_below_q_len":
        ctx[1] = 0
        want = B.CHECK_CONTEXT
    elif case == "page_negative":
        pt[2, used[2] - 1] = -1
        want = B.CHECK_PAGE
    elif case == "page_beyond_pool":
        pt[0, 0] = nblk
        want = B.CHECK_PAGE
    elif case == "page_unused":      # past the pages request 1 uses: not read, not flagged
        pt[1, used[1]:] = -5
    elif case == "page_pool_unstated":
        pt[0, 0] = nblk
        pool = 0
    elif case == "index_not_visible":
        idx[1, 3] = int(wl.context_lens[1])      # the row sees positions [0, L)
        want = B.CHECK_INDEX
    elif case == "index_padding":
        idx[2, 5] = -7
    bad = _batch(d, wl, ctx, qsl, pt, max_q)
    got = B.check_batch(bad, pool, idx)
    log("check", case, "->", got)
    assert got == want


@pytest.fixture
def debug_env(monkeypatch):
    monkeypatch.setenv("DSA_DEBUG", "1")


def _status(fn):
    with pytest.raises(B.DsaError) as e:
        fn()
    return e.value.status


def test_debug_mode_valid_calls_unchanged(monkeypatch):
    wl = _wl()
    batch, d = upload(wl)
    args = (batch, d["idx_keys"], d["idx_scales"], d["q_idx"], d["w"], d["kv"], d["kv_scales"], wl.d_latent,
            d["q_mla"], wl.topk, wl.softmax_scale)
    res = {}
    for mode in ("0", "1"):
        monkeypatch.setenv("DSA_DEBUG", mode)
        idx = torch.empty((wl.total_q, wl.topk), dtype=torch.int32, device="cuda")
        out = dsa.decode_step(*args, indices_out=idx)
        idx_f = torch.empty_like(idx)
        out_f = dsa.decode_step_fused(*args, indices_out=idx_f)
        mla = dsa.sparse_mla_decode(batch, d["kv"], d["kv_scales"], wl.d_latent, d["q_mla"], idx, wl.softmax_scale)
        torch.cuda.synchronize()
        res[mode] = [t.cpu() for t in (out, idx, out_f, idx_f, mla)]
    for a, b in zip(res["0"], res["1"]):
        assert torch.equal(a, b)


def test_debug_mode_rejects_before_launch(debug_env):
    wl = _wl()
    batch, d = upload(wl)
    # stated pools one block short of the real ones: the request that holds
    # the last block fails the check, yet the memory behind it is valid
    keys, kv = d["idx_keys"][:-1], d["kv"][:-1]
    ks = d["idx_scales"][:-1] if d["idx_scales"] is not None else None
    kvs = d["kv_scales"][:-1] if d["kv_scales"] is not None else None
    assert int(d["page_table"].max()) == wl.num_blocks - 1
    sentinel = torch.full((wl.total_q, wl.topk), 12345, dtype=torch.int32, device="cuda")
    args = (batch, keys, ks, d["q_idx"], d["w"], kv, kvs, wl.d_latent, d["q_mla"], wl.topk, wl.softmax_scale)
    idx = sentinel.clone()
    assert _status(lambda: dsa.decode_step(*args, indices_out=idx)) == B.ERR_BAD_DEVICE_ARG
    assert _status(lambda: dsa.decode_step_fused(*args, indices_out=idx)) == B.ERR_BAD_DEVICE_ARG
    assert _status(lambda: B.decode_step_noalloc(*args, indices_out=idx)) == B.ERR_BAD_DEVICE_ARG
    scores = torch.full((wl.total_q, wl.max_context_len), 7.0, device="cuda")
    assert _status(lambda: dsa.indexer_scores(batch, keys, ks, d["q_idx"], d["w"], scores=scores)) == \
        B.ERR_BAD_DEVICE_ARG
    torch.cuda.synchronize()
    assert torch.equal(idx, sentinel)                    # nothing was launched
    assert bool((scores == 7.0).all())
    # a selection entry one past the row's visible tokens (inside a used page)
    good = _selection(wl, d, batch)
    bad_idx = good.clone()
    bad_idx[1, 0] = int(wl.context_lens[1])
    assert int(wl.context_lens[1]) // wl.block_size < -(-int(wl.context_lens[1]) // wl.block_size)
    out = torch.full((wl.total_q, wl.mla_heads, wl.d_latent), 3.0, dtype=torch.bfloat16, device="cuda")
    assert _status(lambda: dsa.sparse_mla_decode(batch, d["kv"], d["kv_scales"], wl.d_latent, d["q_mla"], bad_idx,
                                                 wl.softmax_scale, out=out)) == B.ERR_BAD_DEVICE_ARG
    assert _status(lambda: dsa.sparse_mla_prefill(batch, d["kv"], d["kv_scales"], wl.d_latent, d["q_mla"], bad_idx,
                                                  wl.softmax_scale, out=out)) == B.ERR_BAD_DEVICE_ARG
    torch.cuda.synchronize()
    assert bool((out.float() == 3.0).all())
    # a request that sees no token for its query row: selection rejects it
    ctx = d["context_lens"].clone()
    ctx[1] = 0
    sel = sentinel.clone()
    sc = torch.zeros((wl.total_q, wl.max_context_len), device="cuda")
    assert _status(lambda: dsa.topk(_batch(d, wl, ctx=ctx), sc, wl.topk, indices=sel)) == B.ERR_BAD_DEVICE_ARG
    torch.cuda.synchronize()
    assert torch.equal(sel, sentinel)


def test_debug_mode_hot_cache_fetch(debug_env):
    wl = _wl()
    batch, d = upload(wl)
    good = _selection(wl, d, batch)
    host_kv = d["kv"].cpu().pin_memory()
    host_sc = d["kv_scales"].cpu().pin_memory() if d["kv_scales"] is not None else None
    hot = B.HotCache(wl.total_q * wl.topk, wl.batch, wl.max_context_len, host_kv.shape[-1], host_kv.dtype)
    B.hot_cache_reset(batch, hot)
    B.hot_cache_fetch(batch, host_kv, host_sc, wl.d_latent, good, hot)   # valid: accepted
    torch.cuda.synchronize()
    clock = int(hot.clock.item())
    bad = good.clone()
    bad[2, 1] = int(wl.context_lens[2])
    assert _status(lambda: B.hot_cache_fetch(batch, host_kv, host_sc, wl.d_latent, bad, hot)) == \
        B.ERR_BAD_DEVICE_ARG
    torch.cuda.synchronize()
    assert int(hot.clock.item()) == clock                # the rejected fetch changed nothing
