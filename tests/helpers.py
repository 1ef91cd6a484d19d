"""Helpers shared by the tests: fixture parsing, bf16 bit conversions and the parity
tolerance.  None of this is GEMM arithmetic."""
from __future__ import annotations

import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Per written element: |C_gpu - C_ref| <= REL * |C_ref| + ABS_FRAC * max|C_ref|, where
# the max runs over the written elements of the whole output of that call.
REL = 2.0 ** -7
ABS_FRAC = 1e-3

SENTINEL = 0xDEAD  # finite bf16 (about -6.2e18) that pre-fills outputs in routing tests


def read_sections(name: str) -> dict:
    """Parse a golden text fixture made of '# section <name>' blocks of numbers."""
    out, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line:
                continue
            if line.startswith("# section"):
                cur = line.split()[2]
                out[cur] = []
                continue
            if line.startswith("#"):
                continue
            if cur is not None:
                out[cur].append([float(v) for v in line.split()])
    return {k: np.array(v) for k, v in out.items()}


def read_table(name: str) -> list:
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def bf16_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits_torch(x) -> np.ndarray:
    """torch's own fp32 -> bf16 rounding, as uint16 bits."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


FP8_TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def fp8_codes_of(values, fmt: str = "e4m3") -> np.ndarray:
    """fp8 codes (E4M3 or E5M2) of values that are exactly representable (used to build
    integer test inputs); raises if a value is not exact."""
    v = torch.as_tensor(np.asarray(values, dtype=np.float32))
    codes = v.to(FP8_TORCH[fmt])
    back = codes.to(torch.float32)
    assert torch.equal(back, v), f"value not exact in {fmt}"
    return codes.view(torch.uint8).numpy()


def e4m3_codes_of(values) -> np.ndarray:
    """e4m3fn codes of values that are exactly representable."""
    return fp8_codes_of(values, "e4m3")


def assert_within_tolerance(c_test_bits, c_ref_bits, written, what=""):
    """Compare two bf16 outputs: written elements within the tolerance, unwritten
    elements bit-identical (the caller pre-fills both with the same bits)."""
    c_test_bits = np.asarray(c_test_bits, dtype=np.uint16)
    c_ref_bits = np.asarray(c_ref_bits, dtype=np.uint16)
    written = np.asarray(written, dtype=bool)
    assert c_test_bits.shape == c_ref_bits.shape == written.shape
    un = ~written
    if un.any():
        bad = np.argwhere(un & (c_test_bits != c_ref_bits))
        assert bad.size == 0, f"{what}: {len(bad)} unwritten elements changed, first at {bad[:5]}"
    if written.any():
        t = bf16_to_f64(c_test_bits[written])
        r = bf16_to_f64(c_ref_bits[written])
        assert np.all(np.isfinite(r)), f"{what}: reference has non-finite values"
        assert np.all(np.isfinite(t)), f"{what}: non-finite values in the tested output"
        amax = float(np.max(np.abs(r))) if r.size else 0.0
        err = np.abs(t - r)
        lim = REL * np.abs(r) + ABS_FRAC * amax
        nbad = int(np.sum(err > lim))
        if nbad:
            i = int(np.argmax(err - lim))
            raise AssertionError(
                f"{what}: {nbad}/{r.size} elements out of tolerance; worst got {t[i]!r} "
                f"want {r[i]!r} (limit {lim[i]!r})")


def rows_written_contiguous(group_idx, G) -> np.ndarray:
    gi = np.asarray(group_idx, dtype=np.int64)
    lead = gi[(np.arange(gi.size) // 128) * 128]
    return (gi >= 0) & (gi < G) & (gi == lead)


def rows_written_masked(masked_m, cap) -> np.ndarray:
    mm = np.clip(np.asarray(masked_m, dtype=np.int64), 0, cap)
    return (np.arange(cap)[None, :] < mm[:, None]).reshape(-1)
