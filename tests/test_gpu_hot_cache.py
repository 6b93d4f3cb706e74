"""GPU parity of the two-tier latent cache against the LRU model
(oracle/hot_cache.py): after every fetch the misses and victims are the
model's, the kernel's placement of misses into victims is a one-to-one map
(the model then takes it over: the pages leave placement open), and the whole
device state (slot table, owners, last uses, clock, counts) equals the
model's.  Sparse MLA over the hot set matches the CPU oracle on the full
cache, and the full-cache MLA bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_dsa_amd as dsa
import workloads
from oracle.hot_cache import HotCacheModel
from parity import check_out, log, upload
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
    pos = oracle.query_positions(wl)
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


def _state_matches(hot, model, step):
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


@pytest.mark.parametrize("case,capacity_extra,jumps", [("bf16", 0, False), ("bf16", 300, False),
                                                       ("e4m3", 64, False), ("bf16", 500, True)])
def test_hot_cache_matches_model_and_oracle(case, capacity_extra, jumps):
    if case == "bf16":
        wl = workloads.make_workload("single_b1_l32768", batch=3, context_lens=[3000, 5000, 2000], q_len=[1, 2, 1],
                                     topk=256, seed=31)
    else:
        wl = workloads.make_workload("mtp_b8_l202752", batch=3, context_lens=[3000, 5000, 2000], topk=256, seed=32)
    K, T = wl.topk, wl.total_q
    cap = T * K + capacity_extra
    log("hot cache", case, "capacity", cap, "T", T, "K", K, "clock jumps", jumps)
    batch, d = upload(wl)
    host_kv = d["kv"].cpu().pin_memory()
    host_sc = d["kv_scales"].cpu().pin_memory() if d["kv_scales"] is not None else None
    hot = B.HotCache(cap, wl.batch, wl.max_context_len, d["kv"].shape[-1], d["kv"].dtype)
    B.hot_cache_reset(batch, hot)
    model = HotCacheModel(cap)
    counts = torch.zeros(2, dtype=torch.int32, device="cuda")
    ws = None
    pos = oracle.query_positions(wl)
    req = [r for (r, _, _) in pos]
    sels = _selections(wl, K, steps=8, keep=0.6, seed=33)
    for step, sel in enumerate(sels):
        if jumps and step in (3, 5):
            # ages beyond 16 bits: the clock moves 70000 steps on (the slots
            # keep their last uses), on the device and in the model alike
            model.clock += 70000
            hot.clock.fill_(model.clock)
        idx = torch.from_numpy(sel).cuda()
        ws = B.hot_cache_fetch(batch, host_kv, host_sc, wl.d_latent, idx, hot, counts=counts, workspace=ws)
        torch.cuda.synchronize()
        selected = {(req[t], int(s)) for t in range(T) for s in sel[t]}
        before = set(model.slot_of)
        slot_of = hot.slot_of.cpu().numpy()
        # the kernel's placement of this step's misses, checked and adopted by the model
        assign = {(r, s): int(slot_of[r, s]) for (r, s) in selected if (r, s) not in before}
        misses, victims, evicted = model.step(selected, assign=assign)
        assert counts.tolist() == [len(misses), len(evicted)], step
        _state_matches(hot, model, step)
        # MLA over the hot set: the oracle on the full cache, and the full-cache MLA bit for bit
        lse_h = torch.empty((T, wl.mla_heads), dtype=torch.float32, device="cuda")
        lse_f = torch.empty_like(lse_h)
        out_h = dsa.sparse_mla_decode(hot.batch(batch), hot.kv, hot.scales, wl.d_latent, d["q_mla"], idx,
                                      wl.softmax_scale, lse=lse_h)
        out_f = dsa.sparse_mla_decode(batch, d["kv"], d["kv_scales"], wl.d_latent, d["q_mla"], idx,
                                      wl.softmax_scale, lse=lse_f)
        torch.cuda.synchronize()
        assert torch.equal(out_h, out_f), step
        assert torch.equal(lse_h, lse_f), step
        if step in (0, len(sels) - 1):
            oh, lh = out_h.float().cpu().numpy(), lse_h.cpu().numpy()
            for t in range(T):
                ref, rlse = oracle.query_mla(wl, t, sel[t])
                check_out(oh[t], ref, fp32=False)
                np.testing.assert_allclose(lh[t], rlse, rtol=0, atol=1e-3)
        log("  step", step + 1, "misses", len(misses), "evictions", len(evicted))


def test_hot_cache_rejects_small_capacity():
    wl = workloads.make_workload("single_b1_l32768", batch=2, context_lens=[3000, 4000], topk=256, seed=34)
    batch, d = upload(wl)
    hot = B.HotCache(wl.total_q * wl.topk - 1, wl.batch, wl.max_context_len, d["kv"].shape[-1], d["kv"].dtype)
    B.hot_cache_reset(batch, hot)
    idx = torch.zeros((wl.total_q, wl.topk), dtype=torch.int32, device="cuda")
    with pytest.raises(B.DsaError):
        B.hot_cache_fetch(batch, d["kv"].cpu().pin_memory(), None, wl.d_latent, idx, hot)


def test_layer_group_overlap_matches_serial_and_full_cache():
    """Three layers sharing a selection, each with its own page table into
    the pinned pool and its own hot set: with layer l+1's fetch on a second
    stream during layer l's attention, every layer's output equals the
    serial schedule's and the full-cache MLA of that layer, bit for bit,
    step after step."""
    from sparse_attention_dsa_amd.hot_layers import HotLayerGroup
    wl = workloads.make_workload("single_b1_l32768", batch=3, context_lens=[3000, 5000, 2000], q_len=[1, 2, 1],
                                 topk=256, seed=41)
    K, T, H, L = wl.topk, wl.total_q, wl.mla_heads, 3
    batch, d = upload(wl)
    nblk = d["kv"].shape[0]
    host_kv = d["kv"].cpu().pin_memory()
    g = torch.Generator().manual_seed(5)
    batches = []
    for _ in range(L):
        perm = torch.randperm(nblk, generator=g).to(torch.int32).cuda()
        batches.append(dsa.Batch(d["context_lens"], d["query_start_loc"], perm[d["page_table"].long()].contiguous(),
                                 wl.block_size, wl.max_q_len, wl.max_context_len))
    qs = [d["q_mla"].roll(l, dims=1).contiguous() for l in range(L)]

    def group():
        hots = [B.HotCache(T * K + 100, wl.batch, wl.max_context_len, d["kv"].shape[-1], d["kv"].dtype)
                for _ in range(L)]
        grp = HotLayerGroup(batches, [host_kv] * L, [None] * L, hots, wl.d_latent, K, H)
        grp.reset()
        return grp

    ovl, ser = group(), group()
    for step, sel in enumerate(_selections(wl, K, steps=6, keep=0.5, seed=42)):
        idx = torch.from_numpy(sel).cuda()
        out_o = [torch.empty((T, H, wl.d_latent), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
        out_s = [torch.empty_like(o) for o in out_o]
        ovl.step(idx, qs, wl.softmax_scale, out_o, overlap=True)
        ser.step(idx, qs, wl.softmax_scale, out_s, overlap=False)
        full = [dsa.sparse_mla_decode(batches[l], d["kv"], None, wl.d_latent, qs[l], idx, wl.softmax_scale)
                for l in range(L)]
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(out_o[l], out_s[l]), (step, l)
            assert torch.equal(out_o[l], full[l]), (step, l)
        log("  layer group step", step + 1, "ok")
