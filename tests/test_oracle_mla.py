"""Pins for the oracle's sparse MQA-mode MLA and the whole oracle step.

Definition (SemiAnalysis GLM-5.3 article, "MLA Modifications"): in MQA mode
P = Q[H, d+r] K^T[d+r, L], O = P[H, L] V[L, d], with K and V the same cached
latent row (V = its first d columns); softmax with the given logit scale.
Pins: a hand-worked fixture (rope column in the logits, V excluding it, the
scale, an unselected row), zero query -> mean of selected rows (closed form),
one selected token -> its row, torch's scaled_dot_product_attention on the
gathered rows (library routine, float64), top-K >= n -> sparse equals dense,
a peaked query -> the chosen row, per-row fp8 scales, page-table invariance.
"""
import json
import math
import os

import numpy as np

import oracle
import pytest
import torch

import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _num(v):
    table = {"ln3": math.log(3.0), "ln4": math.log(4.0), "ln(e+1)": math.log(math.e + 1),
             "e/(e+1)": math.e / (math.e + 1), "2/(e+1)": 2 / (math.e + 1)}
    return table[v] if isinstance(v, str) else float(v)


def _tree(x):
    return [_tree(v) for v in x] if isinstance(x, list) else _num(x)


def test_hand_fixture(orc):
    with open(os.path.join(GOLD, "mla_hand.json")) as f:
        g = json.load(f)
    kv = np.array(_tree(g["physical_kv"]), dtype=np.float64)
    q = np.array(g["q"], dtype=np.float64)
    for order in (g["sel"], g["sel"][::-1]):
        out, lse = orc.sparse_mla(kv.astype(np.float32), None, "f32", g["d_latent"], g["d_rope"],
                                  np.array(g["page_row"], np.int32), g["block_size"],
                                  q.astype(np.float32), "f32", np.array(order, np.int32), g["scale"])
        np.testing.assert_allclose(out, np.array(_tree(g["expected_out"])), rtol=0, atol=1e-7)
        np.testing.assert_allclose(lse, np.array(_tree(g["expected_lse"])), rtol=0, atol=1e-7)


def _small(seed=0, n=150, kv_dtype="bf16", H=4, d=32, r=8):
    return workloads.make_workload("single_b1_l32768", seed=seed, context_lens=[n], idx_heads=4,
                                   mla_heads=H, d_latent=d, d_rope=r, kv_dtype=kv_dtype, topk=64)


def _gathered(wl, orc, sel):
    """Decoded selected rows [n_sel][d+r] via the oracle's own decoders."""
    pr = wl.page_table[0]
    rows = []
    for s in sel:
        raw = wl.kv[pr[s // 64], s % 64]
        if wl.kv_dtype == "bf16":
            v = orc.decode_bf16(raw)
        elif wl.kv_dtype == "e4m3":
            v = orc.decode_e4m3(raw) * float(wl.kv_scales[pr[s // 64], s % 64])
        else:
            v = raw.astype(np.float64)
        rows.append(v)
    return np.array(rows)


def test_zero_query_is_mean_of_selected_rows(orc):
    wl = _small()
    sel = np.array([3, 140, 77, 0, 64], dtype=np.int32)
    q0 = np.zeros_like(wl.q_mla[0])
    out, lse = orc.sparse_mla(wl.kv, None, "bf16", 32, 8, wl.page_table[0], 64, q0, "bf16",
                              sel, wl.softmax_scale)
    rows = _gathered(wl, orc, sel)
    np.testing.assert_allclose(out, np.broadcast_to(rows[:, :32].mean(0), out.shape), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, np.full(4, math.log(5)), rtol=0, atol=1e-14)


def test_single_token_returns_its_row(orc):
    wl = _small()
    sel = np.array([99], dtype=np.int32)
    out, lse = orc.query_mla(wl, 0, sel)
    rows = _gathered(wl, orc, sel)
    np.testing.assert_array_equal(out, np.broadcast_to(rows[0, :32], out.shape))


@pytest.mark.parametrize("kv_dtype", ["bf16", "e4m3", "f32"])
def test_matches_torch_sdpa(orc, kv_dtype):
    wl = _small(seed=7, kv_dtype=kv_dtype)
    rng = np.random.default_rng(1)
    sel = rng.choice(150, size=41, replace=False).astype(np.int32)
    out, lse = orc.query_mla(wl, 0, sel)
    rows = torch.from_numpy(_gathered(wl, orc, sel))
    if kv_dtype == "f32":
        q = torch.from_numpy(wl.q_mla[0].astype(np.float64))
    else:
        q = torch.from_numpy(orc.decode_bf16(wl.q_mla[0]).reshape(4, 40))
    H = q.shape[0]
    K = rows[None, None].expand(1, H, -1, -1)
    V = rows[None, None, :, :32].expand(1, H, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(q[None, :, None, :], K, V,
                                                           scale=wl.softmax_scale)
    np.testing.assert_allclose(out, ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-13)
    ref_lse = torch.logsumexp(wl.softmax_scale * (q @ rows.T), dim=-1)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def test_topk_at_least_n_equals_dense(orc):
    wl = _small(n=50)            # topk=64 >= n=50
    res = orc.run_step(wl, threads=1)[0]
    assert res["indices"].tolist() == list(range(50))
    dense_out, dense_lse = orc.query_mla(wl, 0, np.arange(50, dtype=np.int32))
    np.testing.assert_array_equal(res["out"], dense_out)
    np.testing.assert_array_equal(res["lse"], dense_lse)


def test_peaked_query_picks_the_row(orc):
    wl = _small(n=150)
    s_star = 121
    wl.q_mla = workloads.peaked_queries(wl, 20.0, [s_star])
    sel = np.array([5, s_star, 60, 149], dtype=np.int32)
    out, _ = orc.query_mla(wl, 0, sel)
    rows = _gathered(wl, orc, sel)
    # the chosen row's logit leads by ~20*|row|^2*scale ~ 30 nats: the result is that row
    np.testing.assert_allclose(out, np.broadcast_to(rows[1, :32], out.shape), atol=1e-6)


def test_fp8_row_scale_covers_all_columns(orc):
    wl = _small(kv_dtype="e4m3")
    sel = np.arange(0, 150, 3, dtype=np.int32)
    base_out, base_lse = orc.query_mla(wl, 0, sel)
    # doubling a row's scale equals doubling the decoded row (rope part included)
    ks2 = wl.kv_scales.copy()
    s = int(sel[4])
    ks2[wl.page_table[0][s // 64], s % 64] *= 2.0
    out2, lse2 = orc.sparse_mla(wl.kv, ks2, "e4m3", 32, 8, wl.page_table[0], 64, wl.q_mla[0], "bf16",
                                sel, wl.softmax_scale)
    rows = _gathered(wl, orc, sel)
    rows[4] *= 2.0
    q = orc.decode_bf16(wl.q_mla[0]).reshape(4, 40)
    z = wl.softmax_scale * (q @ rows.T)
    p = np.exp(z - z.max(1, keepdims=True))
    ref = (p / p.sum(1, keepdims=True)) @ rows[:, :32]
    np.testing.assert_allclose(out2, ref, rtol=1e-12, atol=1e-13)
    assert not np.allclose(out2, base_out)


def test_page_table_invariance(orc):
    wl = _small(n=150)
    sel = np.array([0, 63, 64, 65, 127, 128, 149], dtype=np.int32)
    a, la = orc.query_mla(wl, 0, sel)
    nb = 3
    kvc = wl.kv[wl.page_table[0][:nb]]
    b, lb = orc.sparse_mla(kvc, None, "bf16", 32, 8, np.arange(nb, dtype=np.int32), 64, wl.q_mla[0],
                           "bf16", sel, wl.softmax_scale)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def test_mtp_queries_are_causal(orc):
    wl = workloads.make_workload("single_b1_l32768", context_lens=[90], q_len=2, idx_heads=4,
                                 mla_heads=2, d_latent=16, d_rope=8, topk=200)
    pos = oracle.query_positions(wl)
    assert [p for (_, p, _) in pos] == [88, 89]
    res = orc.run_step(wl, threads=1)
    assert res[0]["indices"].tolist() == list(range(89))
    assert res[1]["indices"].tolist() == list(range(90))
