"""Pins of the oracle's element formats (FP8 E4M3FN, bf16) and of the
generator's encoders, against the format definitions and torch's CPU casts."""
import math

import numpy as np
import pytest
import torch

import oracle
import workload


# OCP 8-bit floating point specification, E4M3 encodings (values fixed by
# the format, not by the oracle): code -> value
E4M3_POINTS = {
    0x00: 0.0,
    0x01: 2.0 ** -9,            # smallest subnormal
    0x07: 7 * 2.0 ** -9,        # largest subnormal
    0x08: 2.0 ** -6,            # smallest normal
    0x30: 0.5,
    0x38: 1.0,
    0x39: 1.125,
    0x40: 2.0,
    0x7E: 448.0,                # largest finite
    0x81: -(2.0 ** -9),
    0xB8: -1.0,
    0xFE: -448.0,
}


def test_fp8_spec_points():
    for code, val in E4M3_POINTS.items():
        assert oracle.fp8_e4m3_value(code) == val, hex(code)
    assert math.isnan(oracle.fp8_e4m3_value(0x7F))
    assert math.isnan(oracle.fp8_e4m3_value(0xFF))
    z = oracle.fp8_e4m3_value(0x80)
    assert z == 0.0 and math.copysign(1.0, z) < 0


def test_fp8_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.fp8_e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(mine))
    assert np.array_equal(ref[~nan], mine[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(mine[~nan]))


def test_fp8_monotone_positive_codes():
    vals = [oracle.fp8_e4m3_value(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(vals, vals[1:]))


def test_bf16_all_codes_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = np.array([oracle.bf16_value(int(b)) for b in bits[::97]])
    r = ref[::97]
    nan = np.isnan(r)
    assert np.array_equal(nan, np.isnan(mine))
    assert np.array_equal(r[~nan], mine[~nan])


def test_round_bf16_matches_torch_rne():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(4000).astype(np.float32)
    # exact halfway cases: bf16 value + half an ulp, both parities
    base = np.array([1.0, 1.0078125, 3.0, -2.015625], np.float32)
    ulp = np.array([2 ** -7, 2 ** -7, 2 ** -6, 2 ** -6], np.float32)
    x = np.concatenate([x, base + ulp / 2, base - ulp / 2])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    mine = np.array([oracle.round_bf16(v) for v in x], np.float32)
    assert np.array_equal(ref, mine)


def test_generator_fp8_encoder_roundtrip_and_torch():
    L = workload.lib()
    # every finite code decodes then re-encodes to itself (except -0 -> 0x80)
    for c in range(256):
        v = oracle.fp8_e4m3_value(c)
        if math.isnan(v):
            continue
        assert L.wl_fp8_e4m3_rne(v) == c, hex(c)
    # in-range values round like torch's cast (round to nearest even)
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(5000) * 60).astype(np.float32)
    x = x[np.abs(x) < 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([L.wl_fp8_e4m3_rne(float(v)) for v in x], np.uint8)
    assert np.array_equal(ref, mine)
    # saturation instead of NaN above the largest finite value
    assert L.wl_fp8_e4m3_rne(1e6) == 0x7E and L.wl_fp8_e4m3_rne(-500.0) == 0xFE


def test_generator_is_seeded_and_order_independent():
    a = workload.normal_f32(11, 1, (4, 8))
    b = workload.normal_f32(11, 1, (32,))
    assert np.array_equal(a.ravel(), b)
    c = workload.normal_f32(12, 1, (32,))
    assert not np.array_equal(b, c)
    big = workload.normal_f32(5, 2, (200_000,))
    assert abs(big.mean()) < 0.01 and abs(big.std() - 1) < 0.01
    u = workload.uniform_f32(5, 3, (200_000,))
    assert u.min() >= 0 and u.max() < 1 and abs(u.mean() - 0.5) < 0.01
    p = workload.permutation(5, 4, 1000)
    assert np.array_equal(np.sort(p), np.arange(1000))
