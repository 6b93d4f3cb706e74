"""GPU parity of the two-tier latent cache: after every fetch the device state
(slot table, owners, last uses, clock, counts) equals the reference model's
(oracle/hot_cache.py) exactly, and sparse MLA over the hot set gives the same
output and LSE bit for bit as over the full cache."""
import numpy as np
import pytest
import torch

import sparse_attention_dsa_amd as dsa
import workloads
from oracle.hot_cache import HotCacheModel
from parity import log, upload
from sparse_attention_dsa_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert B.check_device() == 0, "not a gfx950 device"


def _selections(wl, K, steps, keep, seed):
    """Per step, K distinct visible tokens per query row, about `keep` of them
    carried over from the row's previous selection (a decode sequence whose
    selection drifts)."""
    rng = np.random.default_rng(seed)
    pos = wl.query_positions()
    prev = [rng.choice(n, size=K, replace=False) for (_, _, n) in pos]
    out = []
    for _ in range(steps):
        cur = []
        for t, (_, _, n) in enumerate(pos):
            kept = rng.choice(prev[t], size=int(keep * K), replace=False)
            rest = np.setdiff1d(np.arange(n), kept)
            cur.append(np.concatenate([kept, rng.choice(rest, size=K - len(kept), replace=False)]))
        prev = cur
        out.append(np.sort(np.stack(cur)).astype(np.int32))
    return out


@pytest.mark.parametrize("case,capacity_extra", [("bf16", 0), ("bf16", 300), ("e4m3", 64)])
def test_hot_cache_matches_model_and_full_cache(case, capacity_extra):
    if case == "bf16":
        wl = workloads.make_workload("single_b1_l32768", batch=3, context_lens=[3000, 5000, 2000], q_len=[1, 2, 1],
                                     topk=256, seed=31)
    else:
        wl = workloads.make_workload("mtp_b8_l202752", batch=3, context_lens=[3000, 5000, 2000], topk=256, seed=32)
    K, T = wl.topk, wl.total_q
    cap = T * K + capacity_extra
    log("hot cache", case, "capacity", cap, "T", T, "K", K)
    batch, d = upload(wl)
    host_kv = d["kv"].cpu().pin_memory()
    host_sc = d["kv_scales"].cpu().pin_memory() if d["kv_scales"] is not None else None
    hot = B.HotCache(cap, wl.batch, wl.max_context_len, d["kv"].shape[-1], d["kv"].dtype)
    B.hot_cache_reset(batch, hot)
    model = HotCacheModel(cap)
    counts = torch.zeros(2, dtype=torch.int32, device="cuda")
    ws = None
    req = [r for (r, _, _) in wl.query_positions()]
    for step, sel in enumerate(_selections(wl, K, steps=6, keep=0.6, seed=33)):
        idx = torch.from_numpy(sel).cuda()
        ws = B.hot_cache_fetch(batch, host_kv, host_sc, wl.d_latent, idx, hot, counts=counts, workspace=ws)
        misses, victims, evicted = model.step({(req[t], int(s)) for t in range(T) for s in sel[t]})
        torch.cuda.synchronize()
        assert counts.tolist() == [len(misses), len(evicted)], step
        slot_of = hot.slot_of.cpu().numpy()
        want = np.full_like(slot_of, -1)
        for (r, s), v in model.slot_of.items():
            want[r, s] = v
        assert np.array_equal(slot_of, want), step
        owner = hot.owner.cpu().numpy()
        want_owner = np.array([-1 if o is None else (o[0] << 32) | o[1] for o in model.owner], dtype=np.int64)
        assert np.array_equal(owner, want_owner), step
        assert hot.last_use.cpu().tolist() == model.last_use, step
        assert int(hot.clock.item()) == model.clock
        # MLA over the hot set == MLA over the full cache, bit for bit
        lse_h = torch.empty((T, wl.mla_heads), dtype=torch.float32, device="cuda")
        lse_f = torch.empty_like(lse_h)
        out_h = dsa.sparse_mla_decode(hot.batch(batch), hot.kv, hot.scales, wl.d_latent, d["q_mla"], idx,
                                      wl.softmax_scale, lse=lse_h)
        out_f = dsa.sparse_mla_decode(batch, d["kv"], d["kv_scales"], wl.d_latent, d["q_mla"], idx,
                                      wl.softmax_scale, lse=lse_f)
        torch.cuda.synchronize()
        assert torch.equal(out_h, out_f), step
        assert torch.equal(lse_h, lse_f), step
        log("  step", step + 1, "misses", len(misses), "evictions", len(evicted))


def test_hot_cache_rejects_small_capacity():
    wl = workloads.make_workload("single_b1_l32768", batch=2, context_lens=[3000, 4000], topk=256, seed=34)
    batch, d = upload(wl)
    hot = B.HotCache(wl.total_q * wl.topk - 1, wl.batch, wl.max_context_len, d["kv"].shape[-1], d["kv"].dtype)
    B.hot_cache_reset(batch, hot)
    idx = torch.zeros((wl.total_q, wl.topk), dtype=torch.int32, device="cuda")
    with pytest.raises(B.DsaError):
        B.hot_cache_fetch(batch, d["kv"].cpu().pin_memory(), None, wl.d_latent, idx, hot)
