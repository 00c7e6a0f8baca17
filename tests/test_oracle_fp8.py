"""Pins for the oracle's E4M3 codec (CPU only): torch's float8_e4m3fn cast
(an independent library routine) for decode and for in-range encode, the
round trip of every code, ties to even, saturation and NaN."""
import numpy as np
import torch

from oracle import fp8


def test_decode_table_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.DECODE_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2  # 0x7f and 0xff
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = fp8.decode(codes).astype(np.float32)
    assert np.array_equal(fp8.encode_rne_sat(vals), codes)


def test_midpoints_round_to_even_code():
    vals = fp8.DECODE_TABLE[:0x7F]
    for c in range(0x7E):
        mid = np.float32((vals[c] + vals[c + 1]) / 2)  # exact in fp32
        assert float(mid) == (vals[c] + vals[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert fp8.encode_rne_sat(np.array([mid]))[0] == want
        assert fp8.encode_rne_sat(np.array([-mid]))[0] == want | 0x80


def test_in_range_values_match_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.1, 1, 30, 200)])
    x = x[np.abs(x) < 448].astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.encode_rne_sat(x), ref)


def test_saturation_nan_and_signed_zero():
    x = np.array([448.0, 449.0, 464.0, 1e9, np.inf, -np.inf, -500.0, np.nan, -0.0, 0.0], np.float32)
    got = fp8.encode_rne_sat(x).tolist()
    assert got == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x80, 0x00]


def test_quantize_uses_fp32_reciprocal_multiply():
    x = np.array([1.0, -2.5, 3.14159], np.float32)
    scale = np.float32(0.0123)
    inv = np.float32(1.0) / scale
    assert np.array_equal(fp8.quantize(x, scale), fp8.encode_rne_sat(x * inv))
    back = fp8.dequantize(fp8.quantize(x, scale), scale)
    assert np.abs(back - x).max() <= 0.0625 * np.abs(x).max()  # 3-bit mantissa
