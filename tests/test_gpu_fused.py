"""The step as one persistent kernel (dsa_decode_step_fused): the same
parity cases as dsa_decode_step through the kernel's paths (rows at and
around K, dense requests, two query rows a request, requests without query
rows, mass ties that defeat the per-chunk candidate quotas, K = 4096, more
than 1024 requests, full-size batches), plus its own properties: the same
selection as dsa_decode_step, bit-identical results from run to run and
with events, and DSA_ERR_UNSUPPORTED outside its shapes."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_dsa_amd as dsa
import workloads
from parity import check_step_rows, gpu_step, log, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(name):
    if name == "ragged_bf16":   # lengths straddle page (64) and K (2048) boundaries
        return workloads.make_workload("single_b1_l32768", batch=8, seed=11,
                                       context_lens=[1, 63, 64, 65, 2047, 2048, 2049, 5000])
    if name == "mtp_fp8":
        return workloads.make_workload("mtp_b8_l202752", batch=3, context_lens=[2, 2049, 7001], seed=12)
    if name == "mtp_bf16":
        return workloads.make_workload("mtp_b8_l202752", batch=3, context_lens=[2050, 130, 4099], seed=13,
                                       kv_dtype="bf16")
    if name == "no_queries":    # a request with no query rows between two that have some
        return workloads.make_workload("single_b1_l32768", batch=3, context_lens=[5000, 14000, 3000],
                                       q_len=[2, 0, 1], seed=23)
    if name == "k4096":
        return workloads.make_workload("single_b1_l32768", batch=2, context_lens=[4096, 30000], topk=4096, seed=23)
    if name == "idx32":
        return workloads.make_workload("single_b1_l32768", batch=2, context_lens=[20000, 3000], idx_heads=32,
                                       seed=24)
    if name == "idx16":
        return workloads.make_workload("single_b1_l32768", batch=2, context_lens=[15000, 2500], idx_heads=16,
                                       seed=25)
    if name == "long_rows":     # many chunks a row, rows of very different length
        return workloads.make_workload("batched_b64_l8k_128k", batch=5, context_lens=[131072, 8192, 70001, 9000,
                                                                                       40000], seed=26)
    raise ValueError(name)


@pytest.mark.parametrize("name", ["ragged_bf16", "mtp_fp8", "mtp_bf16", "no_queries", "k4096", "idx32", "idx16",
                                  "long_rows"])
def test_fused_step_parity(name):
    wl = _case(name)
    log("fused step", name, wl.context_lens.tolist(), "q_len", wl.q_lens.tolist(), "K", wl.topk)
    batch, d = upload(wl)
    out, lse, idx = gpu_step(wl, batch, d, fused=True)
    worst = check_step_rows(wl, list(range(wl.total_q)), out, lse, idx)
    log("  worst abs err", worst)
    # the same selection as the multi-kernel step (both are exact)
    _, _, idx2 = gpu_step(wl, batch, d)
    assert (idx == idx2).all()


def test_fused_step_ties_defeat_quotas():
    """Rows whose scores all tie (every chunk's quota cuts through the tie, so
    the candidates cannot be shown to hold the top K and the row is scored
    again in full) and rows whose top K sits in one chunk (far above the
    quota that chunk is given): both must still match the oracle exactly."""
    wl = workloads.make_workload("single_b1_l32768", batch=3, context_lens=[20000, 30000, 9000], seed=21)
    wl.q_idx[0] = 0                                    # row 0: every score 0
    blk = wl.page_table[1, :48]                        # row 1: tokens 0 .. 3071 scaled x1000
    wl.idx_scales[blk] *= 1000.0
    batch, d = upload(wl)
    out, lse, idx = gpu_step(wl, batch, d, fused=True)
    assert idx[0].tolist() == list(range(2048))
    check_step_rows(wl, [0, 1, 2], out, lse, idx)


def test_fused_step_many_requests():
    """More than 1024 requests (stream in request order, not by length)."""
    rng = np.random.default_rng(79)
    lens = rng.integers(16, 300, size=1500).tolist() + [3000, 9000, 20000, 2049]
    wl = workloads.make_workload("single_b1_l32768", batch=len(lens), context_lens=lens, seed=80)
    log("fused step, %d requests" % len(lens))
    batch, d = upload(wl)
    out, lse, idx = gpu_step(wl, batch, d, fused=True)
    rows = [0, 1, 700, 1499, 1500, 1501, 1502, 1503]
    check_step_rows(wl, rows, out, lse, idx)


def test_fused_step_deterministic_with_events():
    """Two runs, the second recording events, give identical bits; the events
    are ordered."""
    wl = workloads.make_workload("single_b1_l32768", batch=4, context_lens=[30000, 5000, 12000, 2100], seed=27)
    batch, d = upload(wl)
    o1, l1, i1 = gpu_step(wl, batch, d, fused=True)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    o2, l2, i2 = gpu_step(wl, batch, d, fused=True, events=evs)
    assert (i1 == i2).all()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    t = [evs[0].elapsed_time(e) for e in evs]
    assert all(b >= a for a, b in zip(t, t[1:])), t


def test_fused_step_unsupported_shapes():
    """fp32 keys and latents (the generic shapes) are left to dsa_decode_step."""
    wl = workloads.make_workload("tiny_fp32_l4096")
    batch, d = upload(wl)
    with pytest.raises(dsa.DsaError) as e:
        gpu_step(wl, batch, d, fused=True)
    assert e.value.status == -2   # DSA_ERR_UNSUPPORTED


@pytest.mark.parametrize("name,rows", [
    ("single_b1_l32768", [0]),
    ("batched_b64_l8k_128k", [0, 17, 40, 63]),
    ("mtp_b8_l202752", [0, 1, 14, 15]),
])
def test_fused_step_full_size(name, rows):
    wl = workloads.make_workload(name)
    log("fused full size", name, "T", wl.total_q)
    batch, d = upload(wl)
    out, lse, idx = gpu_step(wl, batch, d, fused=True)
    for t, (r, p, n) in enumerate(oracle.query_positions(wl)):
        m = min(n, wl.topk)
        assert (idx[t, :m] >= 0).all() and (idx[t, m:] == -1).all()
        assert (np.diff(idx[t, :m]) > 0).all() and idx[t, m - 1] < n
    worst = check_step_rows(wl, rows, out, lse, idx)
    log("  rows", rows, "worst abs err", worst)
