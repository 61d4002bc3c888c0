"""The oracle's decoder of quantized K/V caches (llama.cpp's q8_0 / q4_0 blocks).

The pages name the cache types but not their byte layout; the layout pinned here is
the public ggml block definition (fp16 scale, then 32 int8 codes / 16 bytes of
nibbles with element i in the low and element i + 16 in the high nibble of byte i).
Hand-built blocks fix every field; round trips through the input generator's
quantizer bound the decode error by the quantization step.
"""
import numpy as np
import torch

import oracle
import synth


def _block(scale, payload):
    return np.concatenate([np.array([scale], dtype=np.float16).view(np.uint8), np.asarray(payload, dtype=np.uint8)])


def test_q8_0_hand_block():
    codes = np.array([-128, -1, 0, 1, 127] + list(range(-13, 14)) * 1, dtype=np.int8)[:32]
    raw = _block(0.5, codes.view(np.uint8))[None, :]
    vals = oracle.dequantize_rows(raw, "q8_0")
    assert vals.shape == (1, 32)
    np.testing.assert_array_equal(vals[0], 0.5 * codes.astype(np.float64))


def test_q4_0_hand_block_nibble_order():
    payload = np.zeros(16, dtype=np.uint8)
    payload[0] = 0x21   # element 0 = low nibble 1, element 16 = high nibble 2
    payload[1] = 0xF0   # element 1 = 0, element 17 = 15
    payload[15] = 0x8A  # element 15 = 10, element 31 = 8
    raw = _block(2.0, payload)[None, :]
    v = oracle.dequantize_rows(raw, "q4_0")[0]
    assert v[0] == 2.0 * (1 - 8) and v[16] == 2.0 * (2 - 8)
    assert v[1] == 2.0 * (0 - 8) and v[17] == 2.0 * (15 - 8)
    assert v[15] == 2.0 * (10 - 8) and v[31] == 0.0
    assert all(v[i] == -16.0 for i in range(2, 15))


def test_multi_block_rows_and_lead_dims():
    x = torch.randn(2, 3, 4, 256, generator=torch.Generator().manual_seed(3))
    for fmt, bb in (("q8_0", 34), ("q4_0", 18)):
        raw = synth.quantize_rows(x, fmt)
        assert tuple(raw.shape) == (2, 3, 4, 8 * bb)
        y = oracle.dequantize_rows(raw, fmt)
        assert y.shape == (2, 3, 4, 256)
        # block b of a row decodes from bytes [b*bb, (b+1)*bb) only
        raw2 = raw.clone()
        raw2[..., 3 * bb:4 * bb] = 0
        y2 = oracle.dequantize_rows(raw2, fmt)
        keep = np.ones(256, dtype=bool)
        keep[96:128] = False
        np.testing.assert_array_equal(y[..., keep], y2[..., keep])


def test_round_trip_within_one_step():
    x = torch.randn(64, 128, generator=torch.Generator().manual_seed(5)) * 3
    xb = x.numpy().reshape(64, 4, 32)
    y8 = oracle.dequantize_rows(synth.quantize_rows(x, "q8_0"), "q8_0").reshape(64, 4, 32)
    step8 = np.abs(xb).max(axis=2, keepdims=True) / 127
    assert (np.abs(y8 - xb) <= 0.5 * step8 * 1.01 + 1e-6).all()
    y4 = oracle.dequantize_rows(synth.quantize_rows(x, "q4_0"), "q4_0").reshape(64, 4, 32)
    step4 = np.abs(xb).max(axis=2, keepdims=True) / 8
    assert (np.abs(y4 - xb) <= step4 * 1.01 + 1e-6).all()


# ---------------------------------------------------------------------------- fp8 (OCP E4M3) pool rows
FP8_CASES = [(0x38, 1.0), (0x7E, 448.0), (0x01, 2.0 ** -9), (0x08, 2.0 ** -6), (0xB8, -1.0), (0x3C, 1.5),
             (0x07, 7 / 8 * 2.0 ** -6), (0x00, 0.0), (0x46, 3.5), (0xFE, -448.0)]


def test_fp8_decode_closed_forms():
    """Values the E4M3 definition fixes: bias 7, subnormals below 2^-6, 448 the largest
    finite value, S.1111.111 NaN."""
    got = oracle.decode_fp8_e4m3(np.array([c for c, _ in FP8_CASES]))
    assert np.array_equal(got, np.array([v for _, v in FP8_CASES]))
    assert np.isnan(oracle.decode_fp8_e4m3(np.array([0x7F, 0xFF]))).all()


def test_fp8_decode_equals_library():
    """All 256 codes against torch's float8_e4m3fn (the same OCP format)."""
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_fp8_e4m3(codes.numpy())
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])


def test_fp8_rows_blocks_and_quantizer():
    """Each 128-column block takes its own scale; the quantizer's round trip stays within
    half an E4M3 step (2^-4 relative) of the input."""
    x = torch.randn(6, 512, generator=torch.Generator().manual_seed(3)) * torch.tensor([1.0, 10.0, 0.01, 3.0]
                                                                                      ).repeat_interleave(128)
    codes, scales = synth.quantize_fp8_rows(x)
    y = oracle.dequantize_fp8_rows(codes.numpy(), scales.numpy())
    for blk in range(4):
        cols = slice(128 * blk, 128 * blk + 128)
        assert np.allclose(y[:, cols], oracle.decode_fp8_e4m3(codes[:, cols].numpy()) * scales[:, blk:blk + 1].numpy())
    err = np.abs(y - x.double().numpy())
    assert (err <= np.abs(x.double().numpy()) * 2.0 ** -4 + scales.repeat_interleave(128, 1).double().numpy()
            * 2.0 ** -10).all()
