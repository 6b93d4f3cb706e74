"""MXFP4 index keys (FP4 E2M1 elements, one E8M0 scale per 32; e4m3
queries) on the GPU against the oracle: scores element by element within
their fp32 rounding bound (the fast 16/32/64-head kernel, one and two query
rows a request, and the generic kernel), the -inf tail, and the whole decode
step (selection and output) on ragged and full-size batches."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_dsa_amd as dsa
import workloads
from parity import check_scores, check_step_rows, gpu_step, log, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _scores(wl, ld=None):
    batch, d = upload(wl)
    sc = dsa.indexer_scores(batch, d["idx_keys"], d["idx_scales"], d["q_idx"], d["w"], ld=ld)
    torch.cuda.synchronize()
    return sc.cpu().numpy()


@pytest.mark.parametrize("heads,q_len", [(64, 1), (32, 1), (16, 1), (64, 2)])
def test_mxfp4_scores_fast(heads, q_len):
    wl = workloads.make_workload("single_b1_l32768", batch=8, seed=31, idx_dtype="mxfp4", idx_heads=heads,
                                 q_len=q_len, context_lens=[2, 63, 64, 65, 2047, 2048, 2049, 9000])
    log("mxfp4 scores", heads, "heads, q_len", q_len, wl.context_lens.tolist())
    ld = 9000 + 96
    sc = _scores(wl, ld)
    for t, (r, p, n) in enumerate(oracle.query_positions(wl)):
        check_scores(wl, t, sc[t, :n])
        assert np.isneginf(sc[t, n:]).all()


def test_mxfp4_scores_generic():
    """dim 64 and block size 32: the generic kernel's MXFP4 decoding."""
    wl = workloads.make_workload("single_b1_l32768", batch=3, seed=32, idx_dtype="mxfp4", idx_dim=64,
                                 block_size=32, idx_heads=8, context_lens=[5, 700, 1333])
    sc = _scores(wl)
    for t, (r, p, n) in enumerate(oracle.query_positions(wl)):
        check_scores(wl, t, sc[t, :n])


@pytest.mark.parametrize("q_len", [1, 2])
def test_mxfp4_decode_step(q_len):
    wl = workloads.make_workload("single_b1_l32768", batch=5, seed=33, idx_dtype="mxfp4", q_len=q_len,
                                 context_lens=[300, 2049, 5000, 12000, 30000])
    log("mxfp4 decode step q_len", q_len, wl.context_lens.tolist())
    batch, d = upload(wl)
    out, lse, idx = gpu_step(wl, batch, d)
    worst = check_step_rows(wl, list(range(wl.total_q)), out, lse, idx)
    log("  worst abs err", worst)
    with pytest.raises(dsa.DsaError) as e:   # the one-launch step takes e4m3 keys only
        gpu_step(wl, batch, d, fused=True)
    assert e.value.status == -2


def test_mxfp4_decode_step_full_size():
    wl = workloads.make_workload("batched_b64_l8k_128k", idx_dtype="mxfp4")
    log("mxfp4 full size T", wl.total_q)
    batch, d = upload(wl)
    out, lse, idx = gpu_step(wl, batch, d)
    worst = check_step_rows(wl, [0, 21, 63], out, lse, idx)
    log("  worst abs err", worst)
