"""Pins for the oracle's fp8 quantiser (per-token 1x128 and per-block 128x128 scales).

The encoder (an exhaustive nearest-code search in C) is checked against torch's own
float8_e4m3fn / float8_e5m2 rounding, an independent implementation, on values over
the whole range including exact midpoints; the two block quantisers are checked bit for
bit against the input generator's torch-based quantisation (amax over the block,
scale = amax / FMAX in fp32, codes of x / scale rounded to nearest-even, saturating),
and against invariants fixed by that definition."""
import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_lhs_amd import inputs as I

FMTS = ["e4m3", "e5m2"]
FMAX = {"e4m3": 448.0, "e5m2": 57344.0}
TDT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def torch_encode(x, fmt):
    t = torch.from_numpy(np.asarray(x, np.float32)).clamp(-FMAX[fmt], FMAX[fmt])
    return t.to(TDT[fmt]).view(torch.uint8).numpy()


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_matches_torch_over_the_range(fmt):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(400000) * np.exp2(rng.integers(-26, 20, 400000))).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, FMAX[fmt], -FMAX[fmt], 1e30, -1e30])])
    assert np.array_equal(oracle.encode_fp8(x.astype(np.float64), fmt), torch_encode(x, fmt))


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_midpoints_round_to_even(fmt):
    dec = oracle.decode_e4m3fn if fmt == "e4m3" else oracle.decode_e5m2
    codes = np.arange(0, 127, dtype=np.uint8)
    vals = dec(codes)
    fin = np.isfinite(vals)
    lo, hi = vals[:-1][fin[:-1] & fin[1:]], vals[1:][fin[:-1] & fin[1:]]
    c_lo = codes[:-1][fin[:-1] & fin[1:]]
    mid = (lo + hi) / 2                     # exact in fp64 and in fp32
    got = oracle.encode_fp8(mid, fmt)
    want = np.where(c_lo % 2 == 0, c_lo, c_lo + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    assert np.array_equal(got, torch_encode(mid.astype(np.float32), fmt))
    assert np.array_equal(oracle.encode_fp8(-mid, fmt), want | 0x80)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("outliers", [False, True])
def test_1x128_matches_the_input_generator(fmt, outliers):
    x = I.normal_matrix(11, 1, 37, 1024, outliers)
    q, s = oracle.quantize_1x128(x, fmt)
    q_ref, s_ref = I.quantize_1x128(x, fmt)
    assert np.array_equal(s, s_ref)
    assert np.array_equal(q, q_ref)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows", [128, 300, 1])
def test_128x128_matches_the_input_generator(fmt, rows):
    x = I.normal_matrix(12, 2, rows, 512, True)
    q, s = oracle.quantize_128x128(x, fmt)
    q_ref, s_ref = I.quantize_128x128(x, fmt)
    assert np.array_equal(s, s_ref)
    assert np.array_equal(q, q_ref)


@pytest.mark.parametrize("fmt", FMTS)
def test_block_invariants(fmt):
    rng = np.random.default_rng(13)
    x = rng.standard_normal((8, 256)).astype(np.float32) * 3
    x[2, :128] = 0.0                              # an all-zero block: scale 1, codes 0
    x[3, 128:] = -0.0
    x[5, 7] = 1e4                                 # one large element sets the scale
    q, s = oracle.quantize_1x128(x, fmt)
    dec = oracle.decode_e4m3fn if fmt == "e4m3" else oracle.decode_e5m2
    assert s[2, 0] == 1.0 and not q[2, :128].any()
    assert s[3, 1] == 1.0 and np.all(q[3, 128:] == 0x80)
    assert s[5, 0] == np.float32(np.float32(1e4) / np.float32(FMAX[fmt]))
    for r in range(8):
        for kb in range(2):
            blk = x[r, kb * 128:(kb + 1) * 128]
            if not np.any(blk):
                continue
            j = int(np.argmax(np.abs(blk)))
            # the block's largest element maps to +-FMAX exactly
            assert abs(dec(q[r, kb * 128 + j:kb * 128 + j + 1])[0]) == FMAX[fmt]
    # bf16 inputs are the same values: quantising their fp32 expansion is identical
    xb = torch.from_numpy(x).to(torch.bfloat16)
    qb, sb = oracle.quantize_1x128(xb.view(torch.int16).numpy().view(np.uint16), fmt)
    q2, s2 = oracle.quantize_1x128(xb.float().numpy(), fmt)
    assert np.array_equal(qb, q2) and np.array_equal(sb, s2)


def test_rejects_ragged_k():
    with pytest.raises(ValueError):
        oracle.quantize_1x128(np.zeros((2, 100), np.float32))
