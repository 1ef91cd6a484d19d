"""GPU parity of the fp8 block quantisers (dg_quantize_fp8_1x128 / _128x128) against the
CPU oracle: codes and scales must match bit for bit (fp32 and bf16 inputs, E4M3 and
E5M2, ragged row counts, exact rounding ties, all-zero blocks, saturation), and
quantise-then-GEMM on the GPU must agree with the oracle doing both steps.  Also the
byte transposition (dg_transpose_fp8) against NumPy's transpose, bit for bit."""
import numpy as np
import pytest

from moe_grouped_gemm_lhs_amd import inputs as I
from tests.helpers import assert_within_tolerance

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import oracle  # noqa: E402
from moe_grouped_gemm_lhs_amd import binding as dg  # noqa: E402
from tests import gpu_util as gu  # noqa: E402

FMTS = ["e4m3", "e5m2"]
FMAX = {"e4m3": 448.0, "e5m2": 57344.0}


def gpu_quant(x, fmt, kind, dtype):
    X = torch.from_numpy(x).to(gu.DEV).to(dtype)
    f = dg.dg_quantize_fp8_1x128 if kind == "1x128" else dg.dg_quantize_fp8_128x128
    Q, S = f(X, fmt)
    torch.cuda.synchronize()
    return Q.view(torch.uint8).cpu().numpy(), S.cpu().numpy(), X


def oracle_quant(X, fmt, kind):
    if X.dtype == torch.bfloat16:
        xin = X.cpu().view(torch.int16).numpy().view(np.uint16)
    else:
        xin = X.cpu().numpy()
    f = oracle.quantize_1x128 if kind == "1x128" else oracle.quantize_128x128
    return f(xin, fmt)


def check(x, fmt, kind, dtype, what):
    gu.say(f"[case] quant {kind} {fmt} {dtype} {what}")
    q, s, X = gpu_quant(x, fmt, kind, dtype)
    q_ref, s_ref = oracle_quant(X, fmt, kind)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32)), f"{what}: scales differ"
    bad = np.nonzero(q != q_ref)
    assert bad[0].size == 0, f"{what}: {bad[0].size} codes differ, first at {bad[0][0]},{bad[1][0]}"


@pytest.mark.parametrize("kind,shapes", [("1x128", [(1, 128), (37, 1024), (1000, 4096)]),
                                         ("128x128", [(1, 128), (300, 512), (2112, 2048)])])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_quantize_bit_exact(kind, shapes, fmt, dtype):
    for i, (rows, K) in enumerate(shapes):
        x = I.normal_matrix(70 + i, 1, rows, K, outliers=True)
        check(x, fmt, kind, getattr(torch, dtype), f"{rows}x{K}")


@pytest.mark.parametrize("kind,rows,K", [("1x128", 600, 16384), ("128x128", 1100, 16384)])
@pytest.mark.parametrize("fmt,dtype", [("e4m3", "bfloat16"), ("e5m2", "float32")])
def test_quantize_large_shapes(kind, rows, K, fmt, dtype):
    """Larger shapes: for 128x128 blocks more blocks than the persistent grid has
    workgroups, so each workgroup loads its next block while it quantises the current
    one (with a ragged row count)."""
    x = I.normal_matrix(90 + rows, 1, rows, K, outliers=True)
    check(x, fmt, kind, getattr(torch, dtype), f"{rows}x{K} several pieces")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("kind", ["1x128", "128x128"])
def test_quantize_ties_zeros_saturation(fmt, kind):
    """A block whose amax is FMAX has scale 1, so its other values are rounded as given:
    exact midpoints between fp8 neighbours must go to the even code.  Also an all-zero
    block (scale 1, codes 0 / 0x80 for -0) and a block with one huge element."""
    dec = oracle.decode_e4m3fn if fmt == "e4m3" else oracle.decode_e5m2
    vals = dec(np.arange(0, 127, dtype=np.uint8))
    vals = vals[np.isfinite(vals)]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.zeros((256, 512), np.float32)
    row = np.resize(mids, 127)
    for r in range(128):
        x[r, :127] = row * (1 if r % 2 else -1)
        x[r, 127] = FMAX[fmt]                    # sets scale 1 for 1x128 blocks
    x[:128, 128:256] = 0.0
    x[128:, 128:256] = -0.0
    x[:, 256:384] = np.linspace(-3, 3, 128, dtype=np.float32)
    x[5, 300] = 3e4 if fmt == "e4m3" else 3e8   # one huge element sets the scale
    check(x, fmt, kind, torch.float32, "ties/zeros/saturation")


# amax per block: ordinary, either side of the 2^-64 scale below which the kernel divides
# instead of multiplying by 1/scale, tiny (1/scale overflows), bf16 subnormal; fp32 adds
# subnormal blocks and blocks whose scale underflows to zero
TINY_AMAX = [3.0, 1e-15, 448 * 2.0 ** -64 * 1.5, 448 * 2.0 ** -64 * 0.75, 1e-30, 3e-36, 1e-36,
             5e-37, 1e-38, 1e-40]
TINY_AMAX_F32 = [1e-42, 4e-43, 2e-45]


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
@pytest.mark.parametrize("kind", ["1x128", "128x128"])
@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_tiny_blocks(fmt, kind, dtype):
    """Blocks whose amax is tiny or subnormal, codes and scales bit for bit against the
    oracle (a subnormal scale overflows 1/scale; the kernel divides there)."""
    amaxes = TINY_AMAX + (TINY_AMAX_F32 if dtype == "float32" else [])
    rng = np.random.default_rng(17)
    x = np.zeros((200, 128 * len(amaxes)), np.float32)
    for j, a in enumerate(amaxes):
        blk = (rng.uniform(-1.0, 1.0, (200, 128)) * a).astype(np.float32)
        blk[::7, 5] = np.float32(a)
        blk[::5, 9] = -np.float32(a)
        blk[::3, 11] = 0.0
        blk[1::3, 12] = -0.0
        x[:, 128 * j:128 * (j + 1)] = blk
    check(x, fmt, kind, getattr(torch, dtype), "tiny and subnormal blocks")


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_then_gemm(fmt):
    """X -> 1x128 codes, W -> 128x128 codes on the GPU, then the GEMM: codes identical to
    the oracle's, output within the GEMM tolerance of the oracle's GEMM."""
    M, N, K = 200, 300, 1024
    x = I.normal_matrix(80, 1, M, K, outliers=True)
    w = I.normal_matrix(81, 2, N, K, outliers=True)
    Xd = torch.from_numpy(x).to(gu.DEV).to(torch.bfloat16)
    Wd = torch.from_numpy(w).to(gu.DEV)
    A, sA = dg.dg_quantize_fp8_1x128(Xd, fmt)
    B, sB = dg.dg_quantize_fp8_128x128(Wd, fmt)
    C = dg.dg_gemm_fp8_nt(A, sA, B, sB)
    torch.cuda.synchronize()
    qa, sa = oracle.quantize_1x128(Xd.cpu().view(torch.int16).numpy().view(np.uint16), fmt)
    qb, sb = oracle.quantize_128x128(w, fmt)
    assert np.array_equal(A.view(torch.uint8).cpu().numpy(), qa)
    assert np.array_equal(B.view(torch.uint8).cpu().numpy(), qb)
    assert np.array_equal(sA.cpu().numpy(), sa) and np.array_equal(sB.cpu().numpy(), sb)
    c_ref = oracle.gemm_fp8_nt(qa, sa, qb, sb, a_fmt=fmt, b_fmt=fmt)
    c_gpu = C.view(torch.int16).cpu().numpy().view(np.uint16)
    assert_within_tolerance(c_gpu, c_ref, np.ones((M, N), bool), f"quantise+gemm {fmt}")


@pytest.mark.parametrize("rows,cols", [(16, 16), (64, 64), (112, 2112), (2048, 7168),
                                       (48, 80)])
def test_transpose_bit_exact(rows, cols):
    rng = np.random.default_rng(rows + cols)
    x = rng.integers(0, 256, (rows, cols), dtype=np.uint8)
    gu.say(f"[case] transpose {rows}x{cols}")
    Y = dg.dg_transpose_fp8(torch.from_numpy(x).to(gu.DEV))
    torch.cuda.synchronize()
    assert np.array_equal(Y.cpu().numpy(), x.T)


def test_transpose_then_gemm():
    """B stored K x N (the layout the NT calls do not take), transposed on the GPU, then
    the GEMM: equal to the oracle on the N x K operand."""
    M, N, K = 130, 2112, 512
    p = I.make_dense(M, N, K, seed=85)
    Bkn = torch.from_numpy(np.ascontiguousarray(p.B.T)).to(gu.DEV)        # K x N
    B = dg.dg_transpose_fp8(Bkn)
    A, sA, _, sB = gu.device_operands(p)
    C = dg.dg_gemm_fp8_nt(A, sA, B, sB)
    torch.cuda.synchronize()
    c_gpu = C.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(B.cpu().numpy(), p.B)
    assert_within_tolerance(c_gpu, oracle.gemm_fp8_nt(p.A, p.sA, p.B, p.sB),
                            np.ones((M, N), bool), "transpose+gemm")
