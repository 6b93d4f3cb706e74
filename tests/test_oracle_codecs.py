"""Oracle decoders, pinned exhaustively against torch's own casts.

The oracle decodes every stored code itself (bf16 bit patterns, OCP e4m3fn
codes).  torch's dtype conversion is an independent library routine, so an
exhaustive sweep over all codes pins the decoders completely.
"""
import numpy as np
import torch


def test_e4m3_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_bf16_all_codes(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
