"""The measurement variant of the decode step (dsa_decode_step_timed): the same
results as dsa_decode_step, bit for bit, with its five events recorded in
order on the stream -- on the candidate-emitting path (fp8 keys, 64 heads) and
on the score-row path (fp32 keys)."""
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


CASES = {
    "emit_fp8": dict(name="batched_b64_l8k_128k", batch=3, context_lens=[20000, 9000, 15000], seed=41),
    "scores_f32": dict(name="tiny_fp32_l4096"),
}


@pytest.mark.parametrize("case", list(CASES))
def test_timed_step_matches_and_orders_events(case):
    kw = dict(CASES[case])
    wl = workloads.make_workload(kw.pop("name"), **kw)
    log("timed step", case, "T", wl.total_q, "K", wl.topk)
    batch, d = upload(wl)
    args = (batch, d["idx_keys"], d["idx_scales"], d["q_idx"], d["w"], d["kv"], d["kv_scales"], wl.d_latent,
            d["q_mla"], wl.topk, wl.softmax_scale)
    i1 = torch.empty((wl.total_q, wl.topk), dtype=torch.int32, device="cuda")
    i2 = torch.empty_like(i1)
    lse1 = torch.empty((wl.total_q, wl.mla_heads), dtype=torch.float32, device="cuda")
    lse2 = torch.empty_like(lse1)
    out1 = dsa.decode_step(*args, lse=lse1, indices_out=i1)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(B.STEP_EVENTS)]
    out2 = dsa.decode_step_timed(*args, evs, lse=lse2, indices_out=i2)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(out1, out2)
    assert torch.equal(lse1, lse2)
    phases = [evs[j].elapsed_time(evs[j + 1]) for j in range(B.STEP_EVENTS - 1)]
    log("  phases (ms):", ["%.4f" % p for p in phases])
    assert all(p >= 0.0 for p in phases)
    assert phases[1] > 0.0 and phases[3] > 0.0          # the indexer and attention take time
    assert evs[0].elapsed_time(evs[-1]) >= max(phases)
