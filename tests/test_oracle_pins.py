"""Pins for the CPU oracle against what the DeepGEMM pages and mathematics fix.

Each test checks the oracle against something other than itself:
  P1  the worked 3x2 . 2x4 example (senqingzn.com article, GEMM introduction; values
      are this repository's choice, the page prints shapes only)
  P2  exact rational arithmetic on tiny shapes (the exact result, and that the oracle
      returns the nearest bf16 with ties to even)
  P3  integer-valued e4m3 inputs with unit scales against int64 products
  P4  exact power-of-two scaling of rows/columns when a scale is multiplied by 2^k
  P5  group-order independence of both grouped layouts
  P6  masked rows never written; NaN bytes in masked-off A rows change nothing
  P7  reductions between the three forms (masked at full capacity = G dense calls,
      contiguous with G=1 = dense, contiguous = per-segment dense calls)
  P8  NumPy fp64 matmul of torch-decoded values with unit scales, and a blockwise
      einsum with scales
P2 and P3 also run with E5M2 operands (either or both), the other input format the
aisharenet.com/ja usage guide names (main functions, section 1); one pin plants a block
whose exact partial needs more than fp64's 53 bits.
A plausible mistake in the oracle (dropped K block, wrong scale index, transposed
operand, wrong sign, double rounding, wrong group) fails at least one of these."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_lhs_amd import inputs as I
from tests.helpers import (FP8_TORCH, SENTINEL, bf16_to_f64, e4m3_codes_of, fp8_codes_of,
                           read_sections, rows_written_contiguous, rows_written_masked)

FMT_PAIRS = [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")]
LSB_EXP = {"e4m3": 9, "e5m2": 16}   # every finite value is an integer times 2^-LSB_EXP


def torch_decode(codes, fmt: str = "e4m3") -> np.ndarray:
    """Independent fp8 decoding through torch (not the oracle's table)."""
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(
        FP8_TORCH[fmt]).to(torch.float64).numpy()


def random_codes(rng, shape, fmt: str = "e4m3"):
    """Random fp8 bytes, excluding the NaN (and, for E5M2, infinity) codes."""
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    if fmt == "e4m3":
        c[(c & 0x7F) == 0x7F] = 0x7E
    else:
        c[(c & 0x7C) == 0x7C] = (c[(c & 0x7C) == 0x7C] & 0x80) | 0x7B
    return c


def random_scales(rng, shape):
    return np.exp2(rng.uniform(-12, 6, size=shape)).astype(np.float32)


# ---------------------------------------------------------------------------- P1
def test_p1_worked_example():
    fx = read_sections("worked_example_3x2x4.txt")
    A, Bt, Cw = fx["A"], fx["Bt"], fx["C"]
    assert A.shape == (3, 2) and Bt.shape == (4, 2) and Cw.shape == (3, 4)
    C = oracle.gemm_fp8_nt(e4m3_codes_of(A), np.ones((3, 1), np.float32),
                           e4m3_codes_of(Bt), np.ones((1, 1), np.float32))
    assert C.shape == (3, 4)
    assert np.array_equal(bf16_to_f64(C), Cw)
    # the same example padded with zeros to one full 128-deep K block
    Ap = np.zeros((3, 128)); Ap[:, :2] = A
    Bp = np.zeros((4, 128)); Bp[:, :2] = Bt
    C2 = oracle.gemm_fp8_nt(e4m3_codes_of(Ap), np.ones((3, 1), np.float32),
                            e4m3_codes_of(Bp), np.ones((1, 1), np.float32))
    assert np.array_equal(bf16_to_f64(C2), Cw)


# ---------------------------------------------------------------------------- P2
def _bf16_fraction(bits: int) -> Fraction:
    return Fraction(float(bf16_to_f64(np.array([bits], np.uint16))[0]))


def _exact_results(A, sA, B, sB, a_fmt="e4m3", b_fmt="e4m3"):
    """Exact rational C (list of lists) and the sum of |terms| per element."""
    M, K = A.shape
    N = B.shape[0]
    nkb = -(-K // 128)
    la, lb = LSB_EXP[a_fmt], LSB_EXP[b_fmt]
    ia = [[int(round(v * 2 ** la)) for v in row] for row in torch_decode(A, a_fmt)]
    ib = [[int(round(v * 2 ** lb)) for v in row] for row in torch_decode(B, b_fmt)]
    out, mag = [], []
    for m in range(M):
        row, mrow = [], []
        for n in range(N):
            tot, tmag = Fraction(0), Fraction(0)
            for kb in range(nkb):
                k0, k1 = kb * 128, min(K, kb * 128 + 128)
                p = Fraction(sum(x * y for x, y in zip(ia[m][k0:k1], ib[n][k0:k1])),
                             1 << (la + lb))
                s = Fraction(float(sA[m, kb])) * Fraction(float(sB[n // 128, kb]))
                tot += p * s
                tmag += abs(p * s)
            row.append(tot)
            mrow.append(tmag)
        out.append(row)
        mag.append(mrow)
    return out, mag


def _check_nearest(bits: int, exact: Fraction, err: Fraction) -> bool:
    """True if `bits` is the nearest bf16 to `exact` (ties to even).  Returns False
    (ambiguous) when `exact` lies within `err` of a rounding midpoint."""
    b = _bf16_fraction(bits)
    mag = bits & 0x7FFF
    sign = -1 if bits & 0x8000 else 1
    if exact != 0:
        assert (exact > 0) == (sign > 0) or mag == 0
    nbrs = [(mag + d) for d in (-1, 1) if 0 <= mag + d < 0x7F80]
    for nm in nbrs:
        nb = _bf16_fraction(nm | (bits & 0x8000))
        mid = (b + nb) / 2
        if abs(exact - mid) <= err:
            return False
        d_self, d_n = abs(exact - b), abs(exact - nb)
        assert d_self <= d_n, (bits, float(exact))
        if d_self == d_n:
            assert (mag & 1) == 0
    return True


@pytest.mark.parametrize("M,N,K,seed", [(5, 7, 384, 1), (2, 260, 200, 2), (8, 8, 128, 3),
                                        (3, 130, 256, 4)])
@pytest.mark.parametrize("a_fmt,b_fmt", FMT_PAIRS)
def test_p2_exact_rational_brute_force(M, N, K, seed, a_fmt, b_fmt):
    rng = np.random.default_rng(seed)
    nkb = -(-K // 128)
    A = random_codes(rng, (M, K), a_fmt)
    B = random_codes(rng, (N, K), b_fmt)
    sA = random_scales(rng, (M, nkb))
    sB = random_scales(rng, (-(-N // 128), nkb))
    C, acc = oracle.gemm_fp8_nt(A, sA, B, sB, want_acc=True, a_fmt=a_fmt, b_fmt=b_fmt)
    exact, mag = _exact_results(A, sA, B, sB, a_fmt, b_fmt)
    ambiguous = 0
    for m in range(M):
        for n in range(N):
            # fp64 error bound of the oracle's scaled-term rounding and kb summation
            err = Fraction((nkb + 1) * 2.0 ** -52) * mag[m][n]
            assert abs(Fraction(float(acc[m, n])) - exact[m][n]) <= err
            if not _check_nearest(int(C[m, n]), exact[m][n], err):
                ambiguous += 1
    assert ambiguous == 0, f"{ambiguous} elements lie within fp64 error of a bf16 midpoint"


def test_p2_wide_partial_is_exact():
    """E5M2 x E5M2: a block holding 57344^2, then 2^-32, then -57344^2 sums exactly to
    2^-32 (a left-to-right fp64 sum would return 0); the same with the tiny product in
    each of 128 positions of one block and 2^-32 scaled into the bf16 range."""
    K = 128
    big, tiny = 0x7B, 0x01                      # 57344 and 2^-16 in E5M2
    for pos in (1, 5, 127):
        a = np.zeros((1, K), np.uint8)
        b = np.zeros((1, K), np.uint8)
        a[0, 0], b[0, 0] = big, big
        a[0, pos], b[0, pos] = tiny, tiny
        neg = 2 if pos != 2 else 3
        a[0, neg], b[0, neg] = big | 0x80, big  # -57344 * 57344
        C, acc = oracle.gemm_fp8_nt(a, np.ones((1, 1), np.float32), b,
                                    np.ones((1, 1), np.float32), want_acc=True,
                                    a_fmt="e5m2", b_fmt="e5m2")
        assert acc[0, 0] == 2.0 ** -32
        C2 = oracle.gemm_fp8_nt(a, np.full((1, 1), 2.0 ** 30, np.float32), b,
                                np.full((1, 1), 2.0 ** 2, np.float32), a_fmt="e5m2",
                                b_fmt="e5m2")
        assert bf16_to_f64(C2)[0, 0] == 1.0


# ---------------------------------------------------------------------------- P3
def _sparse_int_rows(rng, rows, K, nnz, lo=-4, hi=4):
    v = np.zeros((rows, K))
    for r in range(rows):
        pos = rng.choice(K, size=nnz, replace=False)
        v[r, pos] = rng.integers(lo, hi + 1, size=nnz)
    return v


@pytest.mark.parametrize("a_fmt,b_fmt", FMT_PAIRS)
def test_p3_integer_inputs_exact(a_fmt, b_fmt):
    rng = np.random.default_rng(7)
    M, N, K = 37, 300, 384
    a = _sparse_int_rows(rng, M, K, 8)
    b = rng.integers(-4, 5, size=(N, K)).astype(np.float64)
    ref = a.astype(np.int64) @ b.astype(np.int64).T
    assert np.abs(ref).max() <= 256
    C = oracle.gemm_fp8_nt(fp8_codes_of(a, a_fmt), np.ones((M, 3), np.float32),
                           fp8_codes_of(b, b_fmt), np.ones((3, 3), np.float32),
                           a_fmt=a_fmt, b_fmt=b_fmt)
    assert np.array_equal(bf16_to_f64(C), ref.astype(np.float64))


def test_p3_integer_routing_contiguous_and_masked():
    rng = np.random.default_rng(8)
    G, N, K = 3, 136, 256
    sizes = [256, 128, 384]
    a = _sparse_int_rows(rng, sum(sizes), K, 6)
    bs = [rng.integers(-4, 5, size=(N, K)).astype(np.float64) for _ in range(G)]
    gi = I.group_sizes_to_idx(sizes)
    ones_a = np.ones((sum(sizes), 2), np.float32)
    ones_b = np.ones((G * 2, 2), np.float32)
    C = oracle.grouped_contiguous(e4m3_codes_of(a), ones_a, e4m3_codes_of(np.concatenate(bs)),
                                  ones_b, gi, G)
    ref = np.concatenate([a[gi == g].astype(np.int64) @ bs[g].astype(np.int64).T
                          for g in range(G)])
    assert np.array_equal(bf16_to_f64(C), ref.astype(np.float64))
    # masked: 3 groups of capacity 200, counts 200, 0, 57
    cap, mm = 200, np.array([200, 0, 57], np.int32)
    am = _sparse_int_rows(rng, G * cap, K, 6)
    Cm = np.full((G * cap, N), SENTINEL, np.uint16)
    oracle.grouped_masked(e4m3_codes_of(am), np.ones((G * cap, 2), np.float32),
                          e4m3_codes_of(np.concatenate(bs)), ones_b, mm, G, cap, C=Cm)
    for g in range(G):
        blk = Cm[g * cap:(g + 1) * cap]
        r = am[g * cap:g * cap + mm[g]].astype(np.int64) @ bs[g].astype(np.int64).T
        assert np.array_equal(bf16_to_f64(blk[:mm[g]]), r.astype(np.float64))
        assert np.all(blk[mm[g]:] == SENTINEL)


# ---------------------------------------------------------------------------- P4
def test_p4_power_of_two_scaling():
    p = I.make_dense(40, 300, 384, seed=11)
    C0 = oracle.gemm_fp8_nt(p.A, p.sA, p.B, p.sB)
    sA = p.sA.copy(); sA[5, :] *= 8.0; sA[17, :] *= 0.25
    C1 = oracle.gemm_fp8_nt(p.A, sA, p.B, p.sB)
    f0, f1 = bf16_to_f64(C0), bf16_to_f64(C1)
    assert np.array_equal(f1[5], 8.0 * f0[5])
    assert np.array_equal(f1[17], 0.25 * f0[17])
    keep = np.ones(40, bool); keep[[5, 17]] = False
    assert np.array_equal(C1[keep], C0[keep])
    sB = p.sB.copy(); sB[1, :] *= 16.0          # columns 128..255
    C2 = bf16_to_f64(oracle.gemm_fp8_nt(p.A, p.sA, p.B, sB))
    assert np.array_equal(C2[:, 128:256], 16.0 * f0[:, 128:256])
    assert np.array_equal(C2[:, :128], f0[:, :128]) and np.array_equal(C2[:, 256:], f0[:, 256:])
    # a single K block's scale: scaling only that block must change the result
    sA3 = p.sA.copy(); sA3[:, 2] *= 2.0
    assert not np.array_equal(oracle.gemm_fp8_nt(p.A, sA3, p.B, p.sB), C0)


# ---------------------------------------------------------------------------- P5
def test_p5_group_order_independence_contiguous():
    sizes = [128, 384, 256]
    p = I.make_contiguous(sizes, 200, 256, seed=12)
    C = oracle.grouped_contiguous(p.A, p.sA, p.B, p.sB, p.group_idx, p.G)
    starts = np.cumsum([0] + sizes)
    order = [2, 0, 1]
    rows = np.concatenate([np.arange(starts[g], starts[g + 1]) for g in order])
    Cp = oracle.grouped_contiguous(p.A[rows], p.sA[rows], p.B, p.sB, p.group_idx[rows], p.G)
    assert np.array_equal(Cp, C[rows])


def test_p5_group_order_independence_masked():
    G, cap, N, K = 3, 160, 200, 256
    p = I.make_masked(G, cap, N, K, seed=13, masked_m=[160, 31, 97])
    C = oracle.grouped_masked(p.A, p.sA, p.B, p.sB, p.masked_m, G, cap)
    perm = [1, 2, 0]
    nnb = -(-N // 128)
    ra = np.concatenate([np.arange(g * cap, (g + 1) * cap) for g in perm])
    rb = np.concatenate([np.arange(g * N, (g + 1) * N) for g in perm])
    rs = np.concatenate([np.arange(g * nnb, (g + 1) * nnb) for g in perm])
    Cp = oracle.grouped_masked(p.A[ra], p.sA[ra], p.B[rb], p.sB[rs], p.masked_m[perm], G, cap)
    assert np.array_equal(Cp, C[ra])


# ---------------------------------------------------------------------------- P6
def test_p6_masked_rows_untouched_and_nan_rows_ignored():
    G, cap, N, K = 4, 96, 150, 384
    mm = np.array([96, 0, 1, 50], np.int32)
    p = I.make_masked(G, cap, N, K, seed=14, masked_m=mm)
    C = np.full((G * cap, N), SENTINEL, np.uint16)
    oracle.grouped_masked(p.A, p.sA, p.B, p.sB, mm, G, cap, C=C)
    w = rows_written_masked(mm, cap)
    assert np.all(C[~w] == SENTINEL)
    assert not np.any(C[w] == SENTINEL)
    A2 = p.A.copy()
    A2[~w] = 0x7F                                   # NaN codes in every masked-off row
    C2 = np.full_like(C, SENTINEL)
    oracle.grouped_masked(A2, p.sA, p.B, p.sB, mm, G, cap, C=C2)
    assert np.array_equal(C2, C)
    # out-of-range counts are clamped to [0, cap]
    C3 = np.full_like(C, SENTINEL)
    oracle.grouped_masked(p.A, p.sA, p.B, p.sB, np.array([500, -3, 1, 50], np.int32), G, cap, C=C3)
    assert np.array_equal(C3, C)


def test_p6_contiguous_malformed_rows_untouched():
    sizes = [256, 128]
    p = I.make_contiguous(sizes, 130, 256, seed=15)
    gi = p.group_idx.copy()
    gi[250:256] = -1        # padding rows at the tail of a segment
    gi[300] = 0             # disagrees with its 128-row block's leading index (1)
    gi[130] = 7             # out of range
    C = np.full((p.rows, p.N), SENTINEL, np.uint16)
    oracle.grouped_contiguous(p.A, p.sA, p.B, p.sB, gi, p.G, C=C)
    w = rows_written_contiguous(gi, p.G)
    assert not w[250] and not w[300] and not w[130] and w[129] and w[299]
    assert np.all(C[~w] == SENTINEL)
    Cref = oracle.grouped_contiguous(p.A, p.sA, p.B, p.sB, p.group_idx, p.G)
    assert np.array_equal(C[w], Cref[w])


# ---------------------------------------------------------------------------- P7
def test_p7_masked_full_equals_dense_calls():
    G, cap, N, K = 3, 70, 260, 256
    p = I.make_masked(G, cap, N, K, seed=16, masked_m=[cap] * G)
    C = oracle.grouped_masked(p.A, p.sA, p.B, p.sB, p.masked_m, G, cap)
    nnb = -(-N // 128)
    for g in range(G):
        Cd = oracle.gemm_fp8_nt(p.A[g * cap:(g + 1) * cap], p.sA[g * cap:(g + 1) * cap],
                                p.B[g * N:(g + 1) * N], p.sB[g * nnb:(g + 1) * nnb])
        assert np.array_equal(C[g * cap:(g + 1) * cap], Cd)


def test_p7_contiguous_equals_dense():
    p = I.make_contiguous([384], 200, 384, seed=17)
    C = oracle.grouped_contiguous(p.A, p.sA, p.B, p.sB, p.group_idx, 1)
    assert np.array_equal(C, oracle.gemm_fp8_nt(p.A, p.sA, p.B, p.sB))
    sizes = [128, 256]
    q = I.make_contiguous(sizes, 140, 256, seed=18)
    Cq = oracle.grouped_contiguous(q.A, q.sA, q.B, q.sB, q.group_idx, 2)
    nnb = -(-140 // 128)
    for g, (r0, r1) in enumerate([(0, 128), (128, 384)]):
        Cd = oracle.gemm_fp8_nt(q.A[r0:r1], q.sA[r0:r1], q.B[g * 140:(g + 1) * 140],
                                q.sB[g * nnb:(g + 1) * nnb])
        assert np.array_equal(Cq[r0:r1], Cd)


# ---------------------------------------------------------------------------- P8
def test_p8_numpy_fp64_matmul_unit_scales():
    rng = np.random.default_rng(19)
    M, N, K = 33, 270, 640
    A, B = random_codes(rng, (M, K)), random_codes(rng, (N, K))
    C, acc = oracle.gemm_fp8_nt(A, np.ones((M, 5), np.float32), B,
                                np.ones((3, 5), np.float32), want_acc=True)
    ref = torch_decode(A) @ torch_decode(B).T        # exact in fp64 (< 53 bits)
    assert np.array_equal(acc, ref)
    assert np.array_equal(C, oracle.bf16_rne(ref))
    # torch's float64 -> bfloat16 goes through fp32 (two roundings): within 1 ulp
    tb = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.all(np.abs(tb.astype(np.int32) - C.astype(np.int32)) <= 1)


def test_p8_blockwise_einsum_with_scales():
    p = I.make_dense(24, 300, 512, seed=20, outliers=True)
    C, acc = oracle.gemm_fp8_nt(p.A, p.sA, p.B, p.sB, want_acc=True)
    a = torch_decode(p.A).reshape(24, 4, 128)
    b = torch_decode(p.B).reshape(300, 4, 128)
    part = np.einsum("mkc,nkc->mnk", a, b)                         # exact block partials
    s = p.sA.astype(np.float64)[:, None, :] * p.sB.astype(np.float64)[np.arange(300) // 128][None]
    ref = (part * s).sum(axis=2)
    assert np.allclose(acc, ref, rtol=1e-14, atol=0)
    assert np.all(np.abs(bf16_to_f64(C) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)


@pytest.mark.parametrize("a_fmt,b_fmt", FMT_PAIRS[1:])
def test_p7_grouped_forms_with_e5m2_equal_dense_calls(a_fmt, b_fmt):
    """The grouped forms' operand formats: with E5M2 for either or both operands
    (random codes over the whole range, random scales), masked at full counts and
    contiguous both equal per-group dense calls, which P2 pins for every format pair;
    a swapped or dropped format in a grouped form changes the decoded values."""
    rng = np.random.default_rng(29)
    G, cap, N, K = 3, 40, 150, 256
    nnb, nkb = -(-N // 128), K // 128
    A = random_codes(rng, (G * cap, K), a_fmt)
    B = random_codes(rng, (G * N, K), b_fmt)
    sA = random_scales(rng, (G * cap, nkb))
    sB = random_scales(rng, (G * nnb, nkb))
    fm = dict(a_fmt=a_fmt, b_fmt=b_fmt)
    dense = [oracle.gemm_fp8_nt(A[g * cap:(g + 1) * cap], sA[g * cap:(g + 1) * cap],
                                B[g * N:(g + 1) * N], sB[g * nnb:(g + 1) * nnb], **fm)
             for g in range(G)]
    Cm = oracle.grouped_masked(A, sA, B, sB, np.full(G, cap, np.int32), G, cap, **fm)
    # contiguous: the same rows, padded to 128-row segments with rows marked -1
    rows = 128 * G
    Ac = np.zeros((rows, K), np.uint8)
    sAc = np.ones((rows, nkb), np.float32)
    gi = np.full(rows, -1, np.int32)
    for g in range(G):
        Ac[128 * g:128 * g + cap] = A[g * cap:(g + 1) * cap]
        sAc[128 * g:128 * g + cap] = sA[g * cap:(g + 1) * cap]
        gi[128 * g:128 * g + cap] = g
    Cc = oracle.grouped_contiguous(Ac, sAc, B, sB, gi, G, **fm)
    for g in range(G):
        assert np.array_equal(Cm[g * cap:(g + 1) * cap], dense[g])
        assert np.array_equal(Cc[128 * g:128 * g + cap], dense[g])
    # and the formats matter: reading the operands as E4M3 gives other values
    other = oracle.gemm_fp8_nt(A[:cap], sA[:cap], B[:N], sB[:nnb])
    assert not np.array_equal(other, dense[0])
