"""Pins of the benchmark's byte and FLOP accounting, on which every reported
HBM fraction rests: the arithmetic-intensity closed form and the ridge point
that the SemiAnalysis article prints (section "MLA Modifications"), and the
per-step byte counts against a hand count on a two-request fixture."""
import types

import numpy as np

import bench
import workloads


def test_mla_intensity_matches_the_printed_values():
    # the article prints 120.8 FLOP/B for H = 64 heads, d = 512, r = 64, b = 2
    # (bf16), and about 2H for large H
    assert abs(bench.mla_arithmetic_intensity(64, 512, 64, 2) - 120.8) < 0.1
    assert abs(bench.mla_arithmetic_intensity(128, 512, 64, 2) - 241.8) < 0.1
    # ... and the H800 ridge point it compares against: 865 TFLOP/s / 3.35 TB/s
    assert abs(bench.h800_ridge() - 258.2) < 0.05


def _fixture():
    """Two requests: L = 100 with one query row, L = 3000 with two (MTP).
    Production shapes: 64 x 128 e4m3 indexer with fp32 key scales, 128 MLA
    heads, 512 + 64 bf16 latent, 64-token pages."""
    wl = types.SimpleNamespace(
        batch=2, context_lens=np.array([100, 3000], dtype=np.int32), q_lens=np.array([1, 2], dtype=np.int32),
        query_start_loc=np.array([0, 1, 3], dtype=np.int32), block_size=64,
        idx_heads=64, idx_dim=128, idx_dtype="e4m3", idx_scales=np.ones(1, dtype=np.float32),
        mla_heads=128, d_latent=512, d_rope=64, kv_dtype="bf16")
    K = 200
    idx = np.full((3, K), -1, dtype=np.int32)
    idx[0, :100] = np.arange(100)                 # dense row: all 100 tokens
    idx[1, :] = np.arange(0, 200)                 # row 1 of request 1: tokens 0..199
    idx[2, :] = np.arange(150, 350)               # row 2: tokens 150..349 (50 shared with row 1)
    return wl, idx


def test_visible_counts_hand():
    wl, _ = _fixture()
    assert bench.visible_counts(wl) == [100, 2999, 3000]


def test_indexer_bytes_hand_count():
    wl, _ = _fixture()
    # request 0: 100 keys x (128 B + 4 B scale) = 13200; 2 page-table entries
    # = 8; one query row: 64 x 128 B of q + 64 x 4 B of w = 8448
    # request 1: 3000 x 132 = 396000; 47 entries = 188; two rows = 16896
    read = 13200 + 8 + 8448 + 396000 + 188 + 16896
    assert bench.indexer_read_bytes(wl) == read == 434740
    # the score-writing launch also writes 4 B per visible token of each row
    assert bench.indexer_launch_bytes(wl) == read + 4 * (100 + 2999 + 3000)


def test_step_bytes_hand_count():
    wl, idx = _fixture()
    # per query row: indexer q and w 8448, MLA q 128 x 576 x 2 = 147456,
    # output 128 x 512 x 2 = 131072  ->  286976
    # request 0: keys 13200 + pages 8 + 100 distinct latent rows x 1152
    # = 115200 + one row 286976
    # request 1: keys 396000 + pages 188 + 350 distinct rows (0..349) x 1152
    # = 403200 + two rows 573952
    want = (13200 + 8 + 115200 + 286976) + (396000 + 188 + 403200 + 573952)
    assert bench.step_bytes(wl, idx) == want == 1788724


def test_step_flops_hand_count():
    wl, idx = _fixture()
    f_idx, f_mla = bench.step_flops(wl, idx)
    # indexer: 2 x 64 x 128 = 16384 FLOP per visible token, 6099 tokens
    assert f_idx == 16384 * 6099
    # MLA: 2 x 128 x (576 + 512) = 278528 FLOP per selected token, 500 of them
    assert f_mla == 278528 * 500


def test_mxfp4_key_bytes_hand_count():
    """MXFP4 keys: 128 elements x half a byte + 4 E8M0 bytes + 4 B sigma = 72
    bytes a token; queries stay e4m3 (64 x 128 B + 64 x 4 B of w = 8448)."""
    wl = workloads.make_workload("single_b1_l32768", batch=1, context_lens=[100], idx_dtype="mxfp4", seed=1)
    assert bench.key_row_bytes(wl) == 64 + 4 + 4 == 72
    assert bench.query_row_bytes(wl) == 8448
    # 100 keys x 72 + 2 page-table entries x 4 + one query row
    assert bench.indexer_read_bytes(wl) == 7200 + 8 + 8448
