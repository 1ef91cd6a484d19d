"""GPU check at the largest K the C ABI admits (2^22), where the kernels' 32-bit byte
offsets inside a tile's rows of A and B are largest and the scale matrices are 32768
blocks wide.

Inputs are fp8 codes of -1, 0 and +1 with power-of-two scales (sA = 2 in the last K block,
sB = 4 in the first, 1 elsewhere), so every block partial, every promoted term and every
partial sum is an integer below 2^23: exact in fp32 whatever the summation order.  The
expected output is therefore the closed form

    C = bf16_rne( A B^T + A_last B_last^T + 3 A_first B_first^T )

with A_first / A_last the first / last 128 columns, computed here in float64 (exact for
these integers) and compared bit for bit, on the dense stream-K and tiled paths and on
both grouped forms."""
import numpy as np
import pytest

from moe_grouped_gemm_lhs_amd import inputs as I
from tests.helpers import SENTINEL, bf16_to_f64, e4m3_codes_of, f32_to_bf16_bits_torch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from tests import gpu_util as gu  # noqa: E402

K = 1 << 22
NKB = K // 128
ROWS, N = 256, 256


def _draw(rng, rows):
    """Values -1, 0, +1 (int8) and their e4m3 codes."""
    v = rng.integers(-1, 2, size=(rows, K), dtype=np.int8)
    lut = e4m3_codes_of(np.array([-1.0, 0.0, 1.0]))
    return v, lut[v + 1]


def _closed_form(a, bs, chunk=1 << 16):
    """For each b in bs: A B^T + A_last B_last^T + 3 A_first B_first^T, in float64 over
    K in chunks (exact: integer sums below 2^53)."""
    accs = [np.zeros((a.shape[0], b.shape[0]), np.float64) for b in bs]
    for k0 in range(0, K, chunk):
        ac = a[:, k0:k0 + chunk].astype(np.float64)
        for acc, b in zip(accs, bs):
            acc += ac @ b[:, k0:k0 + chunk].astype(np.float64).T
    for acc, b in zip(accs, bs):
        acc += a[:, -128:].astype(np.float64) @ b[:, -128:].astype(np.float64).T
        acc += 3.0 * (a[:, :128].astype(np.float64) @ b[:, :128].astype(np.float64).T)
    return accs


@pytest.fixture(scope="module")
def operands():
    gu.say(f"[case] drawing integer operands, K={K}")
    rng = np.random.default_rng(77)
    va, a = _draw(rng, ROWS)
    vb0, b0 = _draw(rng, N)
    vb1, b1 = _draw(rng, N)
    want0, want1 = _closed_form(va, [vb0, vb1])
    del va, vb0, vb1
    assert np.abs(want0).max() < 2 ** 23 and np.abs(want1).max() < 2 ** 23
    return a, b0, b1, want0, want1


def _scales(rows, groups):
    sA = np.ones((rows, NKB), np.float32)
    sA[:, -1] = 2.0
    sB = np.ones((groups * ((N + 127) // 128), NKB), np.float32)
    sB[:, 0] = 4.0
    return sA, sB


def _bits(want):
    return f32_to_bf16_bits_torch(want.astype(np.float32))


def _force(monkeypatch, kind, rows, G, inst):
    """Pin the kernel instance (None: the library's own choice); returns its name."""
    if inst:
        monkeypatch.setenv("DG_FORCE_INSTANCE", inst)
    name = gu.dg.dg_instance_name(kind, rows, N, K, G)
    assert not inst or name == inst, f"{inst} not selected ({name})"
    return name


@pytest.mark.parametrize("M,inst", [(64, None), (256, None), (256, "dense_256x256"),
                                    (256, "dense_256x224"), (256, "dense_256x160")])
def test_dense_largest_k(operands, M, inst, monkeypatch):
    a, b0, _, want0, _ = operands
    sA, sB = _scales(M, 1)
    p = I.Problem("dense", M, N, K, 1, a[:M], sA, b0, sB)
    gu.say(f"[case] dense {M}x{N}x{K} ({_force(monkeypatch, 0, M, 1, inst)})")
    got = gu.run_gpu(p)
    assert np.array_equal(got, _bits(want0[:M])), "dense result differs from the closed form"


@pytest.mark.parametrize("inst", [None, "contig_256x256", "contig_256x224"])
def test_contiguous_largest_k(operands, inst, monkeypatch):
    a, b0, b1, want0, want1 = operands
    sA, sB = _scales(ROWS, 2)
    gi = I.group_sizes_to_idx([128, 128])
    p = I.Problem("contiguous", ROWS, N, K, 2, a, sA, np.concatenate([b0, b1]), sB,
                  group_idx=gi)
    gu.say(f"[case] contiguous 2x128 x{N}x{K} ({_force(monkeypatch, 1, ROWS, 2, inst)})")
    got = gu.run_gpu(p)
    want = np.concatenate([want0[:128], want1[128:]])
    assert np.array_equal(got, _bits(want)), "contiguous result differs from the closed form"


@pytest.mark.parametrize("inst", [None, "masked_128x128", "masked_256x256", "masked_64x128"])
def test_masked_largest_k(operands, inst, monkeypatch):
    a, b0, b1, want0, want1 = operands
    cap, mm = 128, np.array([128, 77], np.int32)
    sA, sB = _scales(2 * cap, 2)
    p = I.Problem("masked", cap, N, K, 2, a, sA, np.concatenate([b0, b1]), sB, masked_m=mm)
    gu.say(f"[case] masked 2x{cap} x{N}x{K} ({_force(monkeypatch, 2, cap, 2, inst)})")
    got = gu.run_gpu(p)
    assert np.array_equal(got[:128], _bits(want0[:128])), "group 0 differs"
    assert np.array_equal(got[128:128 + 77], _bits(want1[128:128 + 77])), "group 1 differs"
    assert np.all(got[128 + 77:] == SENTINEL), "rows past masked_m were written"
    assert np.all(np.isfinite(bf16_to_f64(got[:128 + 77])))
