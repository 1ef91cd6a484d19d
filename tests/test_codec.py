"""Pins for the oracle's codecs: e4m3fn and e5m2 decoding, fp64 -> bf16 rounding.

The fp8 decodes are checked against values fixed by the OCP 8-bit format definitions
and against torch's own float8_e4m3fn / float8_e5m2 conversions; the bf16 rounding
against torch's fp32 -> bfloat16 rounding (an independent implementation) and
hand-made ties."""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import f32_to_bf16_bits_torch


def test_e4m3fn_decode_matches_format_definition():
    expect = {
        0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
        0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0x7D: 416.0, 0x77: 240.0,
        0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9),
    }
    got = oracle.decode_e4m3fn(np.array(list(expect), dtype=np.uint8))
    assert np.array_equal(got, np.array(list(expect.values())))
    z = oracle.decode_e4m3fn(np.array([0x80], np.uint8))[0]
    assert z == 0.0 and math.copysign(1.0, z) == -1.0
    nan = oracle.decode_e4m3fn(np.array([0x7F, 0xFF], np.uint8))
    assert np.all(np.isnan(nan))


def test_e4m3fn_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert int(np.isnan(ours).sum()) == 2   # only S.1111.111


def test_e5m2_decode_matches_format_definition():
    expect = {
        0x00: 0.0, 0x01: 2.0 ** -16, 0x03: 3 * 2.0 ** -16, 0x04: 2.0 ** -14,
        0x3C: 1.0, 0x3D: 1.25, 0x3E: 1.5, 0x3F: 1.75, 0x40: 2.0, 0x7B: 57344.0,
        0x7A: 49152.0, 0xBC: -1.0, 0xFB: -57344.0, 0x81: -(2.0 ** -16),
    }
    got = oracle.decode_e5m2(np.array(list(expect), dtype=np.uint8))
    assert np.array_equal(got, np.array(list(expect.values())))
    z = oracle.decode_e5m2(np.array([0x80], np.uint8))[0]
    assert z == 0.0 and math.copysign(1.0, z) == -1.0
    inf = oracle.decode_e5m2(np.array([0x7C, 0xFC], np.uint8))
    assert inf[0] == math.inf and inf[1] == -math.inf
    nan = oracle.decode_e5m2(np.array([0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF], np.uint8))
    assert np.all(np.isnan(nan))


def test_e5m2_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e5m2(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert int(np.isnan(ours).sum()) == 6 and int(np.isinf(ours).sum()) == 2


def test_bf16_rne_matches_torch_on_fp32_values():
    rng = np.random.default_rng(123)
    # wide exponent range, subnormals, values near the overflow threshold
    with np.errstate(over="ignore"):
        x = (rng.standard_normal(200000) * np.exp2(rng.integers(-140, 128, 200000))).astype(np.float32)
    x = x[np.isfinite(x)]
    bits = rng.integers(0, 2 ** 32, 100000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    bits = bits[np.isfinite(bits)]
    x = np.concatenate([x, bits, np.float32([0.0, -0.0, 1.0, 3.3895314e38, -3.3895314e38,
                                             1e-45, -1e-45, 1.1754944e-38])])
    ours = oracle.bf16_rne(x.astype(np.float64))
    ref = f32_to_bf16_bits_torch(x)
    assert np.array_equal(ours, ref)


def test_bf16_rne_ties_and_direct_rounding():
    cases = [
        (1.0 + 2.0 ** -8, 0x3F80),              # tie between 1 and 1+2^-7 -> even (1)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),          # tie -> even (1+2^-6)
        (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81), # just above the tie: must round up; a
                                                # detour through fp32 would lose 2^-40
        (-(1.0 + 2.0 ** -8 + 2.0 ** -40), 0xBF81),
        (255.5 * 2.0 ** -7, 0x4000),            # carry into the exponent: 1.99609375 -> 2
        (2.0 ** -133, 0x0001),                  # smallest bf16 subnormal
        (2.0 ** -134, 0x0000),                  # tie with zero -> even (0)
        (1.5 * 2.0 ** -134, 0x0001),
        (3.0e38, 0x7F62),
        (3.5e38, 0x7F80),                       # rounds past the largest finite -> inf
        (float("nan"), 0x7FC0),
        (-0.0, 0x8000),
    ]
    x = np.array([c[0] for c in cases], dtype=np.float64)
    got = oracle.bf16_rne(x)
    for (v, want), g in zip(cases, got):
        assert int(g) == want, (v, hex(int(g)), hex(want))
