"""Pins for the oracle's lightning-indexer scores.

Definition (SemiAnalysis GLM-5.3 article, "DeepSeek Sparse Attention" /
"Lightning Indexer"): I[s] = sigma_s * sum_h w_h * ReLU(q_h . k_s).
Pins: a hand-worked fixture (negative weight, negative dots, per-token
scales, shuffled pages), the single-head special case (numpy dot + max),
zero query, positive homogeneity, and page-table permutation invariance.
"""
import json
import os

import numpy as np
import pytest

import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _hand():
    with open(os.path.join(GOLD, "indexer_hand.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("code", ["f32", "e4m3"])
def test_hand_fixture(orc, code):
    g = _hand()
    keys = np.array(g["physical_keys"], dtype=np.float32)
    q = np.array(g["q"], dtype=np.float32)
    if code == "e4m3":  # every fixture value is exact in e4m3
        keys, q = workloads.e4m3_codes(keys), workloads.e4m3_codes(q)
    sc = orc.indexer_scores(keys, np.array(g["physical_scales"], np.float32), code,
                            np.array(g["page_row"], np.int32), g["block_size"], q, code,
                            np.array(g["w"], np.float32), g["n"])
    assert sc.tolist() == g["expected_scores"]
    for k, exp in g["expected_topk"].items():
        assert sorted(orc.topk(sc, int(k)).tolist()) == exp


def test_single_head_is_relu_dot(orc):
    rng = np.random.default_rng(5)
    n, dim, bs = 37, 16, 8
    keys = rng.standard_normal((5, bs, dim)).astype(np.float32)
    q = rng.standard_normal((1, dim)).astype(np.float32)
    pr = np.arange(5, dtype=np.int32)
    sc = orc.indexer_scores(keys, None, "f32", pr, bs, q, "f32", np.ones(1, np.float32), n)
    flat = keys.reshape(-1, dim)[:n].astype(np.float64)
    ref = np.maximum(flat @ q[0].astype(np.float64), 0.0)
    np.testing.assert_allclose(sc, ref, rtol=1e-12, atol=1e-12)


def test_zero_query_gives_zero_scores(orc):
    wl = workloads.make_workload("tiny_fp32_l4096", context_lens=[300])
    sc = orc.indexer_scores(wl.idx_keys, None, "f32", wl.page_table[0], wl.block_size,
                            np.zeros_like(wl.q_idx[0]), "f32", wl.w[0], 300)
    assert np.all(sc == 0.0)
    # all scores tie, so the lowest indices win
    assert sorted(orc.topk(sc, 17).tolist()) == list(range(17))


def test_positive_homogeneity(orc):
    wl = workloads.make_workload("single_b1_l32768", context_lens=[200], idx_heads=4,
                                 mla_heads=4, d_latent=16, d_rope=8)
    base = orc.query_scores(wl, 0)
    sc2 = orc.indexer_scores(wl.idx_keys, wl.idx_scales * 4.0, "e4m3", wl.page_table[0],
                             wl.block_size, wl.q_idx[0], "e4m3", wl.w[0], 200)
    np.testing.assert_array_equal(sc2, base * 4.0)   # power-of-two scale is exact
    sc3 = orc.indexer_scores(wl.idx_keys, wl.idx_scales, "e4m3", wl.page_table[0],
                             wl.block_size, wl.q_idx[0], "e4m3", wl.w[0] * 0.5, 200)
    np.testing.assert_array_equal(sc3, base * 0.5)


def test_page_table_permutation_invariance(orc):
    wl = workloads.make_workload("single_b1_l32768", context_lens=[700], idx_heads=8,
                                 mla_heads=4, d_latent=16, d_rope=8)
    pr = wl.page_table[0]
    nb = (700 + 63) // 64
    contiguous_keys = wl.idx_keys[pr[:nb]]
    contiguous_scales = wl.idx_scales[pr[:nb]]
    a = orc.query_scores(wl, 0)
    b = orc.indexer_scores(contiguous_keys, contiguous_scales, "e4m3",
                           np.arange(nb, dtype=np.int32), 64, wl.q_idx[0], "e4m3", wl.w[0], 700)
    assert not np.array_equal(pr[:nb], np.arange(nb))  # the table really is shuffled
    np.testing.assert_array_equal(a, b)


def test_head_order_does_not_matter(orc):
    wl = workloads.make_workload("tiny_fp32_l4096", context_lens=[129])
    perm = np.array([2, 0, 3, 1])
    a = orc.query_scores(wl, 0)
    b = orc.indexer_scores(wl.idx_keys, None, "f32", wl.page_table[0], 64,
                           wl.q_idx[0][perm], "f32", wl.w[0][perm], 129)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)
