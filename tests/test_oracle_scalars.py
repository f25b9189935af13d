"""Pins for the oracle's scalar conversions: bf16 decode, OCP e4m3 decode/encode, the fp8
quantiser.  Each is checked against facts outside the oracle: torch's own dtype conversions
(an independent library routine) and values fixed by the formats' definitions."""
import numpy as np
import pytest
import torch

from oracle import oracle


def test_bf16_decode_all_patterns(oracle_lib):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros are kept
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_e4m3_decode_all_codes(oracle_lib):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_to_f64(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # only S.1111.111
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_decode_format_facts(oracle_lib):
    # Values fixed by the OCP e4m3 definition (bias 7, 3 mantissa bits, no infinities).
    assert oracle.e4m3_to_f64(0x7E) == 448.0          # largest finite
    assert oracle.e4m3_to_f64(0xFE) == -448.0
    assert oracle.e4m3_to_f64(0x38) == 1.0            # exponent field 7 = bias
    assert oracle.e4m3_to_f64(0x08) == 2.0 ** -6      # smallest normal
    assert oracle.e4m3_to_f64(0x01) == 2.0 ** -9      # smallest subnormal
    assert oracle.e4m3_to_f64(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert np.isnan(oracle.e4m3_to_f64(0x7F))


def _torch_e4m3(x: np.ndarray) -> np.ndarray:
    """torch's fp32 -> e4m3fn cast (round to nearest even); torch does not saturate, so clamp first."""
    t = torch.from_numpy(np.clip(x.astype(np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _encode_cases():
    finite = np.array([oracle.e4m3_to_f64(c) for c in range(0x7F)], dtype=np.float64)
    mids = (finite[:-1] + finite[1:]) / 2  # exact ties
    vals = np.concatenate([finite, mids]).astype(np.float32)
    up = np.nextafter(vals, np.float32(np.inf))
    down = np.nextafter(vals, np.float32(0))
    rng = np.random.default_rng(5)
    rand = (rng.standard_normal(20000) * np.exp2(rng.uniform(-12, 10, 20000))).astype(np.float32)
    big = np.array([448.0, 449.0, 463.9, 464.0, 470.0, 1e4, 3e38], dtype=np.float32)
    x = np.concatenate([vals, up, down, rand, big, np.float32([0.0, 1e-30, 2.0 ** -10, 2.0 ** -11])])
    return np.concatenate([x, -x])


def test_e4m3_encode_matches_torch(oracle_lib):
    x = _encode_cases()
    got = np.array([oracle.f32_to_e4m3(float(v)) for v in x], dtype=np.uint8)
    assert np.array_equal(got, _torch_e4m3(x))


def test_e4m3_encode_ties_to_even(oracle_lib):
    # midpoint between 1.0 (0x38) and 1.125 (0x39) rounds to the even code 0x38;
    # midpoint between 1.125 and 1.25 (0x3A) rounds to 0x3A.
    assert oracle.f32_to_e4m3(1.0625) == 0x38
    assert oracle.f32_to_e4m3(1.1875) == 0x3A
    assert oracle.f32_to_e4m3(2.0 ** -10) == 0x00       # half the smallest subnormal -> 0 (even)
    assert oracle.f32_to_e4m3(3 * 2.0 ** -10) == 0x02   # 1.5 * 2^-9 -> 2 * 2^-9 (even)
    assert oracle.f32_to_e4m3(1e6) == 0x7E             # saturates
    assert oracle.f32_to_e4m3(-1e6) == 0xFE


def test_quantizer_matches_torch(oracle_lib):
    rng = np.random.default_rng(9)
    x = torch.from_numpy(rng.standard_normal(4000).astype(np.float32)).to(torch.bfloat16).to(torch.float32)
    for s in (0.015625, 0.03125, 0.0173, 0.041, 1.0):
        q_ref = _torch_e4m3((x / torch.tensor(s, dtype=torch.float32)).numpy())
        q = np.array([oracle.quantize_e4m3(float(v), s) for v in x.numpy()], dtype=np.uint8)
        assert np.array_equal(q, q_ref), s
