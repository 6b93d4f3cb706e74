"""The no-allocation decode step (dsa_decode_step_noalloc), called through the
C ABI: on two calls in a row, the second with a smaller batch, its
selection, output and lse equal those of dsa_decode_step (same kernels,
caller workspace) bit for bit, and match the CPU oracle on every row."""
import numpy as np
import pytest
import torch

import sparse_attention_dsa_amd as dsa
import workloads
from parity import check_step_rows, log, upload
from sparse_attention_dsa_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert B.check_device() == 0, "not a gfx950 device"


def _run(wl):
    batch, d = upload(wl)
    T, H, K = wl.total_q, wl.mla_heads, wl.topk
    args = (batch, d["idx_keys"], d["idx_scales"], d["q_idx"], d["w"], d["kv"], d["kv_scales"], wl.d_latent,
            d["q_mla"], K, wl.softmax_scale)
    i_ref, i_na = (torch.full((T, K), -7, dtype=torch.int32, device="cuda") for _ in range(2))
    l_ref, l_na = (torch.empty((T, H), dtype=torch.float32, device="cuda") for _ in range(2))
    o_ref = dsa.decode_step(*args, lse=l_ref, indices_out=i_ref)
    o_na = B.decode_step_noalloc(*args, lse=l_na, indices_out=i_na)
    torch.cuda.synchronize()
    assert torch.equal(i_na, i_ref)
    assert torch.equal(o_na, o_ref)
    assert torch.equal(l_na, l_ref)
    check_step_rows(wl, list(range(T)), o_na.float().cpu().numpy(), l_na.cpu().numpy(), i_na.cpu().numpy())


def test_noalloc_matches_decode_step_twice():
    big = workloads.make_workload("batched_b64_l8k_128k", batch=6, context_lens=[20000, 3000, 45000, 12289, 9000, 700],
                                  seed=51)
    small = workloads.make_workload("mtp_b8_l202752", batch=2, context_lens=[5000, 2100], seed=52)
    log("noalloc: first call B", big.batch, "T", big.total_q, "; second call B", small.batch, "T", small.total_q)
    _run(big)
    _run(small)
