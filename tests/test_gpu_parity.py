"""GPU parity: every C entry point against the CPU oracle on seeded inputs
small enough for the oracle (several tiles and ragged tails), plus the edge
cases of the method (empty/short contexts, n around K, ties, MTP rows,
fp8 latent, cross-layer index reuse)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_dsa_amd as dsa
import workloads
from parity import BAND, check_out, check_scores, check_selection, check_step_rows, gpu_step, log, upload

pytestmark = pytest.mark.gpu

PROD = dict(idx_heads=64, idx_dim=128, mla_heads=128, d_latent=512, d_rope=64)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert dsa.binding.check_device() == 0, "not a gfx950 device"


def _ragged(**kw):
    # lengths straddle page (64) and K (2048) boundaries
    return workloads.make_workload("single_b1_l32768", batch=8, seed=11,
                                   context_lens=[1, 63, 64, 65, 2047, 2048, 2049, 5000], **kw)


def test_indexer_scores_fp8_ragged():
    wl = _ragged()
    log("indexer fp8 ragged", wl.context_lens.tolist())
    batch, d = upload(wl)
    # a row stride past the longest row: every row has a tail of -inf
    ld = 5000 + 200
    sc = dsa.indexer_scores(batch, d["idx_keys"], d["idx_scales"], d["q_idx"], d["w"], ld=ld)
    torch.cuda.synchronize()
    sc = sc.cpu().numpy()
    for t, (r, p, n) in enumerate(oracle.query_positions(wl)):
        check_scores(wl, t, sc[t, :n])
        assert np.all(np.isneginf(sc[t, n:])), "row %d: entries past the visible tokens must be -inf" % t


@pytest.mark.parametrize("heads,scaled", [(64, True), (32, True), (16, True), (64, False)])
def test_indexer_scores_query_blocks(heads, scaled):
    """Long query chunks take the query-blocked indexer (8 rows per
    workgroup, 128-page ranges): ragged query counts (one row, a block plus
    one row, several blocks), contexts across a page range, causal rows."""
    wl = workloads.make_workload("single_b1_l32768", batch=4, seed=21, idx_heads=heads,
                                 context_lens=[70, 700, 3000, 8300], q_len=[1, 9, 17, 40])
    if not scaled:
        wl.idx_scales = None
    log("indexer query blocks", heads, scaled, wl.context_lens.tolist(), wl.q_lens.tolist())
    batch, d = upload(wl)
    sc = dsa.indexer_scores(batch, d["idx_keys"], d["idx_scales"] if scaled else None, d["q_idx"], d["w"])
    torch.cuda.synchronize()
    sc = sc.cpu().numpy()
    for t, (r, p, n) in enumerate(oracle.query_positions(wl)):
        check_scores(wl, t, sc[t, :n])
        assert np.all(np.isneginf(sc[t, n:]))


def test_indexer_scores_f32_tiny():
    wl = workloads.make_workload("tiny_fp32_l4096")
    batch, d = upload(wl)
    sc = dsa.indexer_scores(batch, d["idx_keys"], None, d["q_idx"], d["w"], ld=4096 + 37).cpu().numpy()
    ref = oracle.query_scores(wl, 0)
    np.testing.assert_allclose(sc[0, :4096], ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())
    assert np.all(np.isneginf(sc[0, 4096:]))


@pytest.mark.parametrize("dup", [False, True])
def test_topk_exact_on_identical_scores(dup):
    """Both sides select from the same fp32 scores: the sets must be identical,
    ties (duplicated values) included."""
    rng = np.random.default_rng(5)
    lens = [1, 100, 2048, 2049, 9000, 40000]
    wl = workloads.make_workload("single_b1_l32768", batch=len(lens), context_lens=lens, seed=3)
    batch, d = upload(wl)
    ld = (max(lens) + 63) // 64 * 64
    scores = np.full((len(lens), ld), np.nan, dtype=np.float32)
    for t, n in enumerate(lens):
        v = rng.standard_normal(n).astype(np.float32)
        if dup:   # few distinct values -> massive ties around the threshold
            v = np.round(v * 4).astype(np.float32) / 4
        scores[t, :n] = v
    idx = dsa.topk(batch, torch.from_numpy(scores).cuda(), 2048).cpu().numpy()
    for t, n in enumerate(lens):
        ref = oracle.topk(scores[t, :n].astype(np.float64), 2048)
        m = min(n, 2048)
        assert idx[t, :m].tolist() == sorted(ref.tolist())
        assert (idx[t, m:] == -1).all()


def test_topk_all_equal_takes_lowest_indices():
    """One bucket holds the whole row (more members than the candidate list
    keeps), so the selection rescans the row; one row spans 9 chunks."""
    lens = [5000, 3000, 70000]
    wl = workloads.make_workload("single_b1_l32768", batch=3, context_lens=lens, seed=3)
    batch, _ = upload(wl)
    scores = torch.zeros((3, 70016), dtype=torch.float32, device="cuda")
    idx = dsa.topk(batch, scores, 2048).cpu().numpy()
    for t in range(3):
        assert idx[t].tolist() == list(range(2048))


def test_mla_decode_on_oracle_selection():
    wl = _ragged()
    batch, d = upload(wl)
    T = wl.total_q
    sel = np.full((T, wl.topk), -1, dtype=np.int32)
    for t in range(T):
        s = oracle.topk(oracle.query_scores(wl, t), wl.topk)
        sel[t, :len(s)] = np.sort(s)
    lse = torch.empty((T, wl.mla_heads), dtype=torch.float32, device="cuda")
    out = dsa.sparse_mla_decode(batch, d["kv"], None, wl.d_latent, d["q_mla"], torch.from_numpy(sel).cuda(),
                                wl.softmax_scale, lse=lse)
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    for t in range(T):
        s = sel[t][sel[t] >= 0]
        ref, rlse = oracle.query_mla(wl, t, s)
        check_out(out[t], ref, fp32=False)
        np.testing.assert_allclose(lse[t], rlse, rtol=0, atol=1e-3)


@pytest.mark.parametrize("k", [1024, 2048])
def test_mla_single_slice(k):
    """One slice per row (the prefill entry point), so the tile stores its
    normalised rows itself instead of split partials; K = 1024 and 2048,
    rows in descending score order, against the oracle."""
    wl = _ragged()
    batch, d = upload(wl)
    T = wl.total_q
    sel = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        s = oracle.topk(oracle.query_scores(wl, t), k)
        sel[t, :len(s)] = s[::-1]
    lse = torch.empty((T, wl.mla_heads), dtype=torch.float32, device="cuda")
    out = dsa.sparse_mla_prefill(batch, d["kv"], None, wl.d_latent, d["q_mla"], torch.from_numpy(sel).cuda(),
                                 wl.softmax_scale, lse=lse)
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    for t in range(T):
        s = sel[t][sel[t] >= 0]
        ref, rlse = oracle.query_mla(wl, t, s)
        check_out(out[t], ref, fp32=False)
        np.testing.assert_allclose(lse[t], rlse, rtol=0, atol=1e-3)


def test_mla_decode_unsorted_and_holey_indices():
    """Indices in any order with -1 holes anywhere give the same result."""
    wl = workloads.make_workload("single_b1_l32768", batch=1, context_lens=[3000], seed=4)
    batch, d = upload(wl)
    rng = np.random.default_rng(0)
    s = rng.choice(3000, size=1500, replace=False).astype(np.int32)
    sel = np.full((1, 2048), -1, dtype=np.int32)
    pos = np.sort(rng.choice(2048, size=1500, replace=False))
    sel[0, pos] = s
    out = dsa.sparse_mla_decode(batch, d["kv"], None, 512, d["q_mla"], torch.from_numpy(sel).cuda(),
                                wl.softmax_scale).float().cpu().numpy()
    ref, _ = oracle.query_mla(wl, 0, s)
    check_out(out[0], ref, fp32=False)


@pytest.mark.parametrize("case", ["tiny_f32", "ragged_bf16", "mtp_fp8", "mtp_bf16", "peaked"])
def test_decode_step(case):
    if case == "tiny_f32":
        wl = workloads.make_workload("tiny_fp32_l4096")
    elif case == "ragged_bf16":
        wl = _ragged()
    elif case == "mtp_fp8":
        wl = workloads.make_workload("mtp_b8_l202752", batch=3, context_lens=[2, 2049, 7001], seed=12)
    elif case == "mtp_bf16":
        wl = workloads.make_workload("mtp_b8_l202752", batch=3, context_lens=[2050, 130, 4099], seed=13,
                                     kv_dtype="bf16")
    else:
        wl = workloads.make_workload("single_b1_l32768", batch=2, context_lens=[3000, 6000], seed=14)
        # copy (scaled) a selected token's latent row into every head's query
        rows = [int(np.sort(oracle.topk(oracle.query_scores(wl, t), wl.topk))[100 + 7 * t])
                for t in range(wl.total_q)]
        wl.q_mla = workloads.peaked_queries(wl, 1.0, rows)
    log("decode_step", case, wl.context_lens.tolist(), "q_len", wl.q_lens.tolist())
    batch, d = upload(wl)
    out, lse, idx = gpu_step(wl, batch, d)
    worst = check_step_rows(wl, list(range(wl.total_q)), out, lse, idx)
    if case == "peaked":
        assert np.abs(out).max() > 0.5      # outputs really are O(1)
    log("  worst abs err", worst)


@pytest.mark.parametrize("q_len", [[2, 0, 1], [0, 9, 1]])
def test_decode_step_request_without_queries(q_len):
    """A request with no new query rows in the batch (its pages are in the
    page table but nothing reads them) between requests that have some: every
    row still matches the oracle.  The second case also takes the
    query-blocked indexer (9 rows in one request)."""
    wl = workloads.make_workload("single_b1_l32768", batch=3, context_lens=[5000, 14000, 3000], q_len=q_len,
                                 seed=23)
    assert wl.total_q == sum(q_len)
    log("decode_step request without queries", wl.context_lens.tolist(), wl.q_lens.tolist())
    batch, d = upload(wl)
    out, lse, idx = gpu_step(wl, batch, d)
    check_step_rows(wl, list(range(wl.total_q)), out, lse, idx)
    sc = dsa.indexer_scores(batch, d["idx_keys"], d["idx_scales"], d["q_idx"], d["w"])
    torch.cuda.synchronize()
    sc = sc.cpu().numpy()
    for t, (r, p, n) in enumerate(oracle.query_positions(wl)):
        check_scores(wl, t, sc[t, :n])


def test_decode_step_zero_query_ties():
    """All indexer scores tie at 0 -> the lowest K indices, bit-exact."""
    wl = workloads.make_workload("single_b1_l32768", batch=2, context_lens=[4000, 2100], seed=15)
    wl.q_idx[:] = 0
    batch, d = upload(wl)
    out, lse, idx = gpu_step(wl, batch, d)
    assert idx[0].tolist() == list(range(2048))
    assert idx[1].tolist() == list(range(2048))
    check_step_rows(wl, [0, 1], out, lse, idx)


def test_prefill_with_index_reuse():
    """Chunked prefill: 96 new tokens after 3000 cached; top-K per query; the
    second layer reuses the first layer's selection on its own cache."""
    wl = workloads.make_workload("prefill_q4096_l131072", context_lens=[3096], q_len=96, seed=16)
    batch, d = upload(wl)
    T = wl.total_q
    sc = dsa.indexer_scores(batch, d["idx_keys"], d["idx_scales"], d["q_idx"], d["w"])
    idx = dsa.topk(batch, sc, wl.topk)
    lse1 = torch.empty((T, wl.mla_heads), dtype=torch.float32, device="cuda")
    out1 = dsa.sparse_mla_prefill(batch, d["kv"], None, 512, d["q_mla"], idx, wl.softmax_scale, lse=lse1)
    out2 = dsa.sparse_mla_prefill(batch, d["kv2"], None, 512, d["q_mla2"], idx, wl.softmax_scale)
    torch.cuda.synchronize()
    sc, idx = sc.cpu().numpy(), idx.cpu().numpy()
    out1, out2, lse1 = out1.float().cpu().numpy(), out2.float().cpu().numpy(), lse1.cpu().numpy()
    rows = [0, 1, 47, 94, 95]
    res = oracle.run_step(wl, rows=rows, layers=2)
    for t in rows:
        r = res[t]
        np.testing.assert_allclose(sc[t, :len(r["scores"])], r["scores"], rtol=1e-5,
                                   atol=1e-5 * np.abs(r["scores"]).max())
        nd = check_selection(idx[t], r["scores"], wl.topk)
        sel = idx[t][idx[t] >= 0]
        for layer, out in ((1, out1), (2, out2)):
            ref, rl = oracle.query_mla(wl, t, sel, layer)
            check_out(out[t], ref, fp32=False)
        check_out(out1[t], r["out"], fp32=False, same_selection=(nd == 0))
        check_out(out2[t], r["out2"], fp32=False, same_selection=(nd == 0))
    # the decode entry point agrees with the prefill one on the same selection
    out_dec = dsa.sparse_mla_decode(batch, d["kv"], None, 512, d["q_mla"], torch.from_numpy(idx).cuda(),
                                    wl.softmax_scale).float().cpu().numpy()
    np.testing.assert_allclose(out_dec, out1, rtol=0, atol=2e-2)


def test_band_is_rarely_used():
    """Selections differ from the oracle's only at genuine near-ties."""
    wl = workloads.make_workload("single_b1_l32768", batch=4, context_lens=[9000, 12000, 3000, 20000], seed=17)
    batch, d = upload(wl)
    out, lse, idx = gpu_step(wl, batch, d, lse=False)
    total = 0
    for t in range(wl.total_q):
        total += check_selection(idx[t], oracle.query_scores(wl, t), wl.topk, band=BAND)
    assert total <= 4


@pytest.mark.parametrize("dup", [False, True])
def test_topk_rows_beyond_single_kernel(dup):
    """Rows of 600000 and 530000 tokens (73 and 65 chunk workgroups per row)
    next to a short one; same exact-set rule as above."""
    lens = [600000, 530000, 5000]
    bs = 64
    maxb = (max(lens) + bs - 1) // bs
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    qsl = torch.tensor([0, 1, 2, 3], dtype=torch.int32, device="cuda")
    pt = torch.zeros((3, maxb), dtype=torch.int32, device="cuda")
    batch = dsa.Batch(ctx, qsl, pt, bs, 1, max(lens))
    rng = np.random.default_rng(9)
    ld = maxb * bs
    scores = np.zeros((3, ld), dtype=np.float32)
    for t, n in enumerate(lens):
        v = rng.standard_normal(n).astype(np.float32)
        if dup:
            v = np.round(v * 8).astype(np.float32) / 8
        scores[t, :n] = v
    idx = dsa.topk(batch, torch.from_numpy(scores).cuda(), 2048).cpu().numpy()
    for t, n in enumerate(lens):
        ref = oracle.topk(scores[t, :n].astype(np.float64), 2048)
        assert sorted(ref.tolist()) == idx[t].tolist()


@pytest.mark.parametrize("case", ["bf16", "mtp_fp8"])
def test_indexshare_decode_group(case):
    """IndexShare decode: the full layer runs the whole step and hands its
    indices to a shared layer, whose sparse MLA runs on its own latent cache
    and queries with those indices unchanged."""
    if case == "bf16":
        wl = workloads.make_workload("single_b1_l32768", batch=4, context_lens=[3000, 9000, 2048, 20000],
                                     seed=18, layers=2)
    else:
        wl = workloads.make_workload("mtp_b8_l202752", batch=2, context_lens=[5000, 2100], seed=19, layers=2)
    log("indexshare", case, wl.context_lens.tolist(), "q_len", wl.q_lens.tolist())
    batch, d = upload(wl)
    T, H = wl.total_q, wl.mla_heads
    idx = torch.empty((T, wl.topk), dtype=torch.int32, device="cuda")
    lse2 = torch.empty((T, H), dtype=torch.float32, device="cuda")
    out1 = dsa.decode_step(batch, d["idx_keys"], d["idx_scales"], d["q_idx"], d["w"], d["kv"], d["kv_scales"],
                           wl.d_latent, d["q_mla"], wl.topk, wl.softmax_scale, indices_out=idx)
    out2 = dsa.sparse_mla_decode(batch, d["kv2"], d["kv2_scales"], wl.d_latent, d["q_mla2"], idx,
                                 wl.softmax_scale, lse=lse2)
    torch.cuda.synchronize()
    out1, out2 = out1.float().cpu().numpy(), out2.float().cpu().numpy()
    idx, lse2 = idx.cpu().numpy(), lse2.cpu().numpy()
    res = oracle.run_step(wl, rows=list(range(T)), layers=2)
    for t in range(T):
        r = res[t]
        nd = check_selection(idx[t], r["scores"], wl.topk)
        sel = idx[t][idx[t] >= 0]
        check_out(out1[t], r["out"], fp32=False, same_selection=(nd == 0))
        check_out(out2[t], r["out2"], fp32=False, same_selection=(nd == 0))
        ref2, rl2 = oracle.query_mla(wl, t, sel, 2)
        check_out(out2[t], ref2, fp32=False)
        np.testing.assert_allclose(lse2[t], rl2, rtol=0, atol=1e-3)


@pytest.mark.parametrize("case", ["bf16", "mtp_fp8", "h64"])
def test_mla_decode_layers_matches_per_layer_calls(case):
    """Three layers sharing one selection in one dsa_sparse_mla_decode_layers
    call (one launch on the 128-head path, one call per layer on the 64-head
    one): every layer's output and lse equal its own dsa_sparse_mla_decode
    bit for bit, and the second layer's output matches the oracle."""
    if case == "bf16":
        wl = workloads.make_workload("single_b1_l32768", batch=3, context_lens=[3000, 9000, 2100], seed=51,
                                     layers=2)
    elif case == "mtp_fp8":
        wl = workloads.make_workload("mtp_b8_l202752", batch=2, context_lens=[5000, 2100], seed=52, layers=2)
    else:
        wl = workloads.make_workload("single_b1_l32768", batch=2, context_lens=[4000, 2500], mla_heads=64, seed=53,
                                     layers=2)
    log("mla layers", case, wl.context_lens.tolist(), "heads", wl.mla_heads)
    batch, d = upload(wl)
    T, H = wl.total_q, wl.mla_heads
    idx = torch.empty((T, wl.topk), dtype=torch.int32, device="cuda")
    dsa.decode_step(batch, d["idx_keys"], d["idx_scales"], d["q_idx"], d["w"], d["kv"], d["kv_scales"], wl.d_latent,
                    d["q_mla"], wl.topk, wl.softmax_scale, indices_out=idx)
    roll = lambda x, dim: None if x is None else x.roll(1, dims=dim).contiguous()
    kvs = [d["kv"], d["kv2"], roll(d["kv"], 0)]
    scs = [d["kv_scales"], d["kv2_scales"], roll(d["kv_scales"], 0)]
    qs = [d["q_mla"], d["q_mla2"], roll(d["q_mla"], 1)]
    lses = [torch.empty((T, H), dtype=torch.float32, device="cuda") for _ in kvs]
    outs = dsa.sparse_mla_decode_layers(batch, kvs, scs, wl.d_latent, qs, idx, wl.softmax_scale, lses=lses)
    for l in range(len(kvs)):
        lse1 = torch.empty((T, H), dtype=torch.float32, device="cuda")
        one = dsa.sparse_mla_decode(batch, kvs[l], scs[l], wl.d_latent, qs[l], idx, wl.softmax_scale, lse=lse1)
        torch.cuda.synchronize()
        assert torch.equal(outs[l], one), (case, l)
        assert torch.equal(lses[l], lse1), (case, l)
    out2, ix = outs[1].float().cpu().numpy(), idx.cpu().numpy()
    for t in range(T):
        ref, _ = oracle.query_mla(wl, t, ix[t][ix[t] >= 0], 2)
        check_out(out2[t], ref, fp32=False)


def _sample_positions(n, m=1024):
    """Token positions of the sample the decode step's top-K bound is drawn
    from (m per 128K tokens of the row): m / 16 runs of 16 consecutive tokens,
    run j starting at floor(j n / (m / 16)) rounded down to a multiple of 16,
    at most n - 16 rounded down likewise."""
    nrun, last = m // 16, (n - 16) & ~15
    return [min((j * n // nrun) & ~15, last) + c for j in range(nrun) for c in range(16)]


def test_decode_step_bound_fallbacks():
    """Rows where the sample bound cannot hold the top K: one whose scores all
    tie (every token is a candidate: the list overflows) and one whose sampled
    tokens score far above the rest (the bound leaves fewer than K
    candidates).  Both must still match the oracle exactly."""
    wl = workloads.make_workload("single_b1_l32768", batch=3, context_lens=[20000, 30000, 9000], seed=21)
    wl.q_idx[0] = 0                                   # row 0: all scores 0
    n1 = 30000
    for s in _sample_positions(n1):                  # row 1: sampled tokens x1000
        blk = int(wl.page_table[1, s // wl.block_size])
        wl.idx_scales[blk, s % wl.block_size] *= 1000.0
    batch, d = upload(wl)
    out, lse, idx = gpu_step(wl, batch, d)
    assert idx[0].tolist() == list(range(2048))
    check_step_rows(wl, [0, 1, 2], out, lse, idx)


@pytest.mark.parametrize("case", ["list_edge", "k4096", "idx32", "idx16_h64"])
def test_decode_step_shapes(case):
    """The candidate-emitting step across its shape switches: rows exactly at
    and one past the length where the sample bound starts (12288), the
    largest K, 32- and 16-head indexers, and 64 MLA heads (the GLM-5 shape)."""
    if case == "list_edge":
        wl = workloads.make_workload("single_b1_l32768", batch=3, context_lens=[12288, 12289, 12352], seed=22)
    elif case == "k4096":
        wl = workloads.make_workload("single_b1_l32768", batch=2, context_lens=[4096, 30000], topk=4096, seed=23)
    elif case == "idx32":
        wl = workloads.make_workload("single_b1_l32768", batch=2, context_lens=[20000, 3000], idx_heads=32, seed=24)
    else:
        wl = workloads.make_workload("single_b1_l32768", batch=2, context_lens=[15000, 2500], idx_heads=16,
                                     mla_heads=64, seed=25)
    log("decode_step shape", case, wl.context_lens.tolist(), "K", wl.topk, "H_idx", wl.idx_heads, "H", wl.mla_heads)
    batch, d = upload(wl)
    out, lse, idx = gpu_step(wl, batch, d)
    check_step_rows(wl, list(range(wl.total_q)), out, lse, idx)


@pytest.mark.parametrize("case", ["vec", "odd_widths", "wide_rows"])
def test_generic_fp32_shapes(case):
    """The generic fp32 kernels on both sides of their register-row path:
    key and latent rows of at most 128 values that are multiples of 4 (rows
    read by 16-byte loads), widths that are not (element loads), and latent
    rows wider than 128 values; several rows, ragged contexts, pages
    shuffled, every row against the oracle."""
    kw = dict(batch=3, context_lens=[700, 4096, 2500], shuffle_pages=True, seed=31)
    if case == "vec":
        kw.update(idx_heads=3, idx_dim=36, mla_heads=8, d_latent=60, d_rope=8, topk=300)
    elif case == "odd_widths":
        kw.update(idx_heads=4, idx_dim=30, mla_heads=8, d_latent=62, d_rope=9, topk=256)
    else:
        kw.update(idx_heads=2, idx_dim=132, mla_heads=4, d_latent=192, d_rope=16, topk=512)
    wl = workloads.make_workload("tiny_fp32_l4096", **kw)
    log("generic fp32", case, "idx", wl.idx_heads, wl.idx_dim, "mla", wl.mla_heads, wl.d_latent, wl.d_rope)
    batch, d = upload(wl)
    out, lse, idx = gpu_step(wl, batch, d)
    check_step_rows(wl, list(range(wl.total_q)), out, lse, idx)
    sc = dsa.indexer_scores(batch, d["idx_keys"], d["idx_scales"], d["q_idx"], d["w"])
    torch.cuda.synchronize()
    sc = sc.cpu().numpy()
    for t, (r, p, n) in enumerate(oracle.query_positions(wl)):
        check_scores(wl, t, sc[t, :n])


@pytest.mark.parametrize("q_len", [1, 2])
def test_many_requests(q_len):
    """More than 4096 (request, query-group) items: 4200 short requests (16 to
    300 tokens) plus a few long ones.  Standalone scores on sampled rows
    element by element (with the -inf tail), and the whole decode step's
    selections and outputs on sampled rows."""
    rng = np.random.default_rng(77)
    lens = rng.integers(16, 300, size=4200).tolist() + [3000, 9000, 14000, 20000, 2049, 2500]
    kw = dict(batch=len(lens), context_lens=lens, q_len=q_len, seed=78)
    if q_len == 2:   # the indexer with two query rows per item; small MLA shapes keep the arrays small
        kw.update(mla_heads=16, d_latent=64, d_rope=16, kv_dtype="f32")
    wl = workloads.make_workload("single_b1_l32768", **kw)
    T = wl.total_q
    log("many requests: B", wl.batch, "T", T, "q_len", q_len, "sum L", int(wl.context_lens.sum()))
    batch, d = upload(wl)
    ld = (max(lens) + 63) // 64 * 64
    sc = dsa.indexer_scores(batch, d["idx_keys"], d["idx_scales"], d["q_idx"], d["w"], ld=ld)
    out, lse, idx = gpu_step(wl, batch, d)
    pos = oracle.query_positions(wl)
    rows = sorted(set(list(range(12)) + list(range(T - 2 * 6 - 4, T)) + rng.choice(T, 24, replace=False).tolist()))
    sc_rows = sc[rows].cpu().numpy()
    for i, t in enumerate(rows):
        n = pos[t][2]
        check_scores(wl, t, sc_rows[i, :n])
        assert np.all(np.isneginf(sc_rows[i, n:]))
    check_step_rows(wl, rows, out, lse, idx)
