"""Oracle number formats pinned to the format definitions and to torch's casts."""
import math

import numpy as np
import pytest
import torch

import oracle as O


def test_bf16_decode_all_codes():
    codes = np.arange(65536, dtype=np.uint16)
    ours = O.bf16_bits_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_landmarks():
    # OCP 8-bit floating point spec, E4M3: bias 7, max normal 448 (S.1111.110),
    # min normal 2^-6 (S.0001.000), min subnormal 2^-9, S.1111.111 = NaN.
    v = O.e4m3_to_f64(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x7E, 0x80, 0xFE, 0x3C], np.uint8))
    assert list(v) == [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 448.0, -0.0, -448.0, 1.5]
    assert math.isnan(O.e4m3_to_f64(np.array([0x7F], np.uint8))[0])
    assert math.isnan(O.e4m3_to_f64(np.array([0xFF], np.uint8))[0])


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_encode_vs_torch():
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.normal(size=2000) * 50,
        rng.normal(size=500) * 2.0 ** -7,                       # subnormal range
        O.e4m3_to_f64(np.arange(0, 0x7F, dtype=np.uint8)),      # exact codes
        # midpoints between neighbouring positive codes: ties to even
        0.5 * (O.e4m3_to_f64(np.arange(0, 0x7E, dtype=np.uint8))
               + O.e4m3_to_f64(np.arange(1, 0x7F, dtype=np.uint8))),
        [464.0, -464.0, 0.0, -0.0],
    ])
    vals = vals[np.abs(vals) <= 464.0]                          # torch turns > 464 into NaN
    ours = O.f64_to_e4m3(vals)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # -0.0 vs +0.0 codes both decode to zero; compare values, then codes elsewhere
    assert np.array_equal(O.e4m3_to_f64(ours), O.e4m3_to_f64(ref))
    nz = vals != 0
    assert np.array_equal(ours[nz], ref[nz])


def test_e4m3_encode_saturates():
    # Reading adopted for the cache format: values past the largest finite
    # code saturate to +-448 rather than becoming NaN.
    assert list(O.f64_to_e4m3(np.array([500.0, -1e9, 448.0]))) == [0x7E, 0xFE, 0x7E]


def test_e5m2_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e5m2_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e5m2).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e5m2_landmarks_and_saturation():
    # OCP E5M2: bias 15, max normal 57344 (S.11110.11), min subnormal 2^-16,
    # S.11111.00 = inf, other exponent-31 codes NaN
    v = O.e5m2_to_f64(np.array([0x01, 0x04, 0x3C, 0x7B, 0x7C, 0xFC], np.uint8))
    assert list(v) == [2.0 ** -16, 2.0 ** -14, 1.0, 57344.0, math.inf, -math.inf]
    assert list(O.f64_to_e5m2(np.array([1e9, -60000.0, 57344.0, math.nan]))) == [0x7B, 0xFB, 0x7B, 0x7F]


def test_e5m2_encode_vs_torch():
    rng = np.random.default_rng(8)
    vals = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-6, 5, 3000),
                           O.e5m2_to_f64(np.arange(0x7B, dtype=np.uint8)) * 1.0000001,
                           (O.e5m2_to_f64(np.arange(0x7A, dtype=np.uint8)) +
                            O.e5m2_to_f64(np.arange(1, 0x7B, dtype=np.uint8))) / 2])   # exact ties
    vals = vals[np.abs(vals) < 57344.0].astype(np.float32).astype(np.float64)
    ours = O.f64_to_e5m2(vals)
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_f16_decode_all_codes_and_encode():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.f16_bits_to_f64(codes)
    ref = codes.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 5, 20000)).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f64_to_f16(x.astype(np.float64)), want)
