"""CPU model of how the GPU quantiser forms each quotient x / scale, checked against the
IEEE fp32 division that the quantisation's definition asks for (scale = amax / FMAX in
fp32, codes of x / scale rounded to nearest-even; casting is left to the caller by the
pages, turtlesai.it summary, technical paragraph).

The kernel takes one correctly rounded reciprocal r = 1/scale per block and forms
y = x*r, the fma residual e = x - y*scale and q = y + e*r (Markstein's correction),
for blocks whose scale is at least 2^-64, and a plain IEEE division below that.  Here
every fp32 step is modelled exactly: products and fmas in rational arithmetic, rounded
once to fp32 with ties to even (subnormals included).  The model must give the same
fp8 code as the IEEE quotient on ordinary blocks and on tiny and subnormal ones, and
the reciprocal path alone (no guard) must fail on tiny blocks, which is what the guard
is there for."""
from fractions import Fraction

import numpy as np
import pytest

import oracle

FMAX = {"e4m3": 448.0, "e5m2": 57344.0}
MIN_RECIPROCAL_SCALE = 2.0 ** -64


def rn32(v: Fraction) -> np.float32:
    """Round a rational exactly to the nearest fp32 value, ties to even (subnormals and
    overflow to infinity included)."""
    if v == 0:
        return np.float32(0.0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = Fraction(2) ** (max(e, -126) - 23)           # spacing of fp32 values near a
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * q
    if r >= Fraction(2) ** 128:
        return np.float32(sign * np.inf)
    return np.float32(sign * float(r))               # exact: r is an fp32 value


def ieee_quotient(x: np.float32, scale: np.float32) -> np.float32:
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.float32(x) / np.float32(scale)
    return np.copysign(np.float32(0.0), x) if np.isnan(q) else q


def kernel_quotient(x: np.float32, scale: np.float32, guard: bool = True) -> np.float32:
    """The GPU's quotient, step by step in exact fp32 arithmetic."""
    if guard and not scale >= MIN_RECIPROCAL_SCALE:
        return ieee_quotient(x, scale)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        r = np.float32(1.0) / scale                  # correctly rounded reciprocal
        y = np.float32(x) * r
    if not (np.isfinite(r) and np.isfinite(y)):
        return np.float32(np.nan)                    # what the hardware produces there
    e = rn32(Fraction(float(x)) - Fraction(float(y)) * Fraction(float(scale)))
    q = rn32(Fraction(float(e)) * Fraction(float(r)) + Fraction(float(y)))
    return np.copysign(q, x)


def codes(q, fmt):
    q = np.asarray(q, np.float64)
    m = FMAX[fmt]
    # the kernel saturates with fmin/fmax, which map NaN to -FMAX
    q = np.where(np.isnan(q), -m, np.clip(q, -m, m))
    return oracle.encode_fp8(q, fmt)


def block(rng, amax, n=64, subnormal_fill=False):
    x = (rng.uniform(-1.0, 1.0, n) * amax).astype(np.float32)
    x[0] = np.float32(amax)
    x[1] = np.float32(0.0)
    x[2] = np.float32(-0.0)
    if subnormal_fill:
        x[3:8] = np.float32([1e-45, -3e-45, 1e-42, -7e-40, 2e-39])
    return x


def scale_of(x, fmt):
    amax = np.float32(np.max(np.abs(x)))
    return np.float32(1.0) if amax == 0 else np.float32(amax) / np.float32(FMAX[fmt])


# amax of each block: ordinary, near the guard, tiny (1/scale overflows), subnormal
# bf16 and fp32 values, and fp32 blocks whose scale underflows to zero
AMAXES = [3.7, 1e-3, 1e-15, 1e-18, 448 * 2.0 ** -64 * 1.5, 448 * 2.0 ** -64 * 0.75, 1e-30,
          3e-36, 1e-36, 5e-37, 1e-38, 1e-40, 1e-42, 4e-43, 2e-45]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("amax", AMAXES)
def test_kernel_quotient_gives_the_ieee_codes(fmt, amax):
    rng = np.random.default_rng(int(abs(np.log2(amax))) * 7 + len(fmt))
    x = block(rng, amax, subnormal_fill=amax > 1e-30)
    s = scale_of(x, fmt)
    want = codes([ieee_quotient(v, s) for v in x], fmt)
    got = codes([kernel_quotient(v, s) for v in x], fmt)
    assert np.array_equal(got, want), f"amax {amax}: {np.nonzero(got != want)[0][:5]}"
    # the quotients themselves agree wherever they can reach a non-zero code
    for v in x:
        qi, qk = ieee_quotient(v, s), kernel_quotient(v, s)
        if abs(qi) >= 2.0 ** -18:
            assert qk == qi, f"amax {amax}: x={v!r} gives {qk!r}, want {qi!r}"


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_reciprocal_path_alone_breaks_on_tiny_blocks(fmt):
    """Without the guard, a block with amax 1e-36 (scale subnormal, 1/scale infinite)
    gets the wrong codes; the guard is what makes those blocks right."""
    rng = np.random.default_rng(3)
    x = block(rng, 1e-36)
    s = scale_of(x, fmt)
    want = codes([ieee_quotient(v, s) for v in x], fmt)
    bad = codes([kernel_quotient(v, s, guard=False) for v in x], fmt)
    assert not np.array_equal(bad, want)


def test_zero_scale_block_definition():
    """An fp32 block whose amax / FMAX underflows to zero: the oracle saturates x / 0 to
    +-FMAX and gives 0 / 0 a zero code with the sign of x."""
    x = np.zeros((1, 128), np.float32)
    x[0, :4] = np.float32([2e-45, -2e-45, 0.0, -0.0])
    q, s = oracle.quantize_1x128(x, "e4m3")
    assert s[0, 0] == 0.0
    assert q[0, :4].tolist() == [0x7E, 0xFE, 0x00, 0x80]
    assert np.all(q[0, 4:] == 0x00)
