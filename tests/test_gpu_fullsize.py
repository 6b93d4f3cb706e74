"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (one dsa_decode_step per batch; indexer + top-K + prefill MLA
for the chunked-prefill workload).  The oracle checks sampled query rows one
by one; every row's selection is also checked for the structural properties
(count, -1 padding, causal, unique, ascending)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_dsa_amd as dsa
import workloads
from parity import check_out, check_selection, check_step_rows, gpu_step, log, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _structural(wl, idx):
    for t, (r, p, n) in enumerate(oracle.query_positions(wl)):
        m = min(n, wl.topk)
        s = idx[t, :m]
        assert (s >= 0).all() and (idx[t, m:] == -1).all()
        assert (np.diff(s) > 0).all() and s[-1] < n


@pytest.mark.parametrize("name,rows", [
    ("single_b1_l32768", [0]),
    ("batched_b64_l8k_128k", [0, 17, 40, 63]),
    ("mtp_b8_l202752", [0, 1, 14, 15]),
])
def test_decode_full_size(name, rows):
    wl = workloads.make_workload(name)
    log(name, "T", wl.total_q, "sum L", int(wl.context_lens.sum()))
    batch, d = upload(wl)
    out, lse, idx = gpu_step(wl, batch, d)
    _structural(wl, idx)
    worst = check_step_rows(wl, rows, out, lse, idx)
    log("  rows", rows, "worst abs err", worst)


def test_decode_all_128k_full_size():
    """Batch 64 with every context at 131072 tokens (10.8 GB latent pool)."""
    wl = workloads.make_workload("batched_b64_l8k_128k", context_lens=[131072])
    log("all-128K T", wl.total_q, "sum L", int(wl.context_lens.sum()))
    batch, d = upload(wl)
    out, lse, idx = gpu_step(wl, batch, d)
    _structural(wl, idx)
    worst = check_step_rows(wl, [0, 31, 63], out, lse, idx)
    log("  worst abs err", worst)


def test_chunked_prefill_full_size():
    wl = workloads.make_workload("prefill_q4096_l131072")
    log("prefill T", wl.total_q, "L", int(wl.context_lens[0]))
    batch, d = upload(wl)
    sc = dsa.indexer_scores(batch, d["idx_keys"], d["idx_scales"], d["q_idx"], d["w"])
    idx = dsa.topk(batch, sc, wl.topk)
    out1 = dsa.sparse_mla_prefill(batch, d["kv"], None, 512, d["q_mla"], idx, wl.softmax_scale)
    out2 = dsa.sparse_mla_prefill(batch, d["kv2"], None, 512, d["q_mla2"], idx, wl.softmax_scale)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    _structural(wl, idx)
    rows = [0, 1, 2047, 4095]
    sc_rows = sc[rows].cpu().numpy()
    out1, out2 = out1[rows].float().cpu().numpy(), out2[rows].float().cpu().numpy()
    del sc
    res = oracle.run_step(wl, rows=rows, layers=2)
    for i, t in enumerate(rows):
        r = res[t]
        n = len(r["scores"])
        np.testing.assert_allclose(sc_rows[i, :n], r["scores"], rtol=1e-5, atol=1e-5 * np.abs(r["scores"]).max())
        nd = check_selection(idx[t], r["scores"], wl.topk)
        log("  row", t, "selection diff", nd)
        check_out(out1[i], r["out"], fp32=False, same_selection=(nd == 0))
        check_out(out2[i], r["out2"], fp32=False, same_selection=(nd == 0))
        sel = idx[t][idx[t] >= 0]
        for layer, out in ((1, out1), (2, out2)):
            ref, _ = oracle.query_mla(wl, t, sel, layer)
            check_out(out[i], ref, fp32=False)
