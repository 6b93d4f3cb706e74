"""Pins of the oracle's MXFP4 index keys (FP4 E2M1 elements, E8M0 block
scales; OCP Microscaling Formats v1.0), without retyping its decoder:

  * E8M0: every byte against torch's float8_e8m0fnu decoding;
  * E2M1: every code against the specification's value table
    (tests/golden/e2m1_values.json), against torch's e4m3 decoding of the
    same value rebuilt bit field by bit field (E2M1 normal exponent e,
    mantissa m -> e4m3 exponent e + 6, mantissa 4m; the one subnormal 0.5 ->
    e4m3 exponent 6), and ordered / sign-symmetric;
  * the key layout (nibble order, block-scale placement, per-block scales)
    by hand-worked one-hot cases;
  * whole-row scoring: an MXFP4 key cache scores exactly like the e4m3 cache
    holding the same values (every E2M1 value times the workloads' scales is
    an e4m3 value), which the e4m3 pins already cover.
"""
import json
import os

import numpy as np
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.json")


def test_e8m0_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e8m0(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])


def _e2m1_via_e4m3(code):
    """E2M1 code -> the e4m3 code of the same value, by bit fields only."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    if e == 0 and m == 0:
        return s << 7
    if e == 0:                      # 0.5 = 2^-1: e4m3 biased exponent 6
        return (s << 7) | (6 << 3)
    return (s << 7) | ((e + 6) << 3) | (m << 2)


def test_e2m1_table_and_library():
    ours = oracle.decode_e2m1(np.arange(16, dtype=np.uint8))
    mags = json.load(open(GOLDEN))["magnitudes"]
    assert ours[:8].tolist() == mags
    assert (ours[8:] == -np.array(mags)).all() and np.signbit(ours[8])
    via = np.array([_e2m1_via_e4m3(c) for c in range(16)], dtype=np.uint8)
    ref = torch.from_numpy(via).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(ours, ref)
    assert (np.diff(ours[:8]) > 0).all()
    assert oracle.decode_e2m1([0x12]) == oracle.decode_e2m1([0x02])   # only the low nibble


def _one_token_cache(codes_row, exps_row, dim=128, bs=4):
    """A one-block MXFP4 cache whose slot 1 holds the given key."""
    keys = np.zeros((1, bs * (dim // 2 + dim // 32)), dtype=np.uint8)
    keys[0, 1 * (dim // 2):2 * (dim // 2)] = codes_row
    keys[0, bs * (dim // 2) + 1 * (dim // 32):bs * (dim // 2) + 2 * (dim // 32)] = exps_row
    return keys


def _score_slot1(keys, q_codes, sigma=1.0, dim=128, bs=4):
    H = q_codes.shape[0]
    scales = np.full((1, bs), sigma, dtype=np.float32)
    w = np.ones(H, dtype=np.float32)
    return oracle.indexer_scores(keys, scales, "mxfp4", np.array([0], np.int32), bs, q_codes, "e4m3", w, 2)[1]


def test_mxfp4_layout_hand_cases():
    dim = 128
    one = 0x38                                       # e4m3 1.0
    codes = np.zeros(dim // 2, dtype=np.uint8)
    exps = np.full(dim // 32, 127, dtype=np.uint8)
    codes[0] = 0x72                                  # element 0: 1.0 (low nibble), element 1: 6.0 (high)
    codes[20] = 0x0D                                 # element 40: -3.0 (0b1101)
    exps[1] = 129                                    # block 1 (elements 32..63): x4
    keys = _one_token_cache(codes, exps)
    for d, want in [(0, 1.0), (1, 6.0), (40, 0.0), (2, 0.0)]:   # element 40 negative: ReLU -> 0
        q = np.zeros((1, dim), dtype=np.uint8)
        q[0, d] = one
        assert _score_slot1(keys, q) == want, d
    q = np.zeros((1, dim), dtype=np.uint8)
    q[0, 40] = 0xB8                                  # e4m3 -1.0: (-1) * (-3.0 * 4) = 12
    assert _score_slot1(keys, q) == 12.0
    assert _score_slot1(keys, q, sigma=0.5) == 6.0   # sigma multiplies the head sum
    q[0, 0] = one                                    # 1.0 + 12.0 on one head
    assert _score_slot1(keys, q) == 13.0


def test_mxfp4_scores_equal_e4m3_cache():
    """Workload keys decoded independently (E2M1 via e4m3 bit fields and
    torch, E8M0 via torch) into an e4m3 cache score exactly like the MXFP4
    cache, with the same queries, weights and sigma."""
    wl = workloads.make_workload("single_b1_l32768", batch=2, context_lens=[200, 700], idx_dtype="mxfp4", seed=5)
    dim, bs, nblk = wl.idx_dim, wl.block_size, wl.num_blocks
    codes = wl.idx_keys[:, :bs * dim // 2].reshape(nblk, bs, dim // 2)
    exps = wl.idx_keys[:, bs * dim // 2:].reshape(nblk, bs, dim // 32)
    nib = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(nblk, bs, dim)
    via = np.vectorize(_e2m1_via_e4m3)(nib).astype(np.uint8)
    elem = torch.from_numpy(via).view(torch.float8_e4m3fn).float()
    scale = torch.from_numpy(exps).view(torch.float8_e8m0fnu).float().repeat_interleave(32, dim=-1)
    e4 = (elem * scale).to(torch.float8_e4m3fn)
    assert torch.equal(e4.float(), elem * scale)     # exactly representable
    e4_codes = e4.view(torch.uint8).numpy()
    for t, (r, p, n) in enumerate(oracle.query_positions(wl)):
        got = oracle.query_scores(wl, t)
        ref = oracle.indexer_scores(e4_codes, wl.idx_scales, "e4m3", wl.page_table[r], bs, wl.q_idx[t], "e4m3",
                                    wl.w[t], n)
        assert np.array_equal(got, ref)
