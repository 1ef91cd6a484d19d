"""Seeded random sweep of the three GEMM forms through the C ABI, every output element
against the CPU oracle: shapes from one row to a few tiles with ragged edges (so both
the stream-K and the tiled kernels and their edge paths run), every operand-format pair,
empty and misaligned-count groups.  Routing (which rows are written, the untouched bits
of the rest) must be exact; values within the parity tolerance."""
import numpy as np
import pytest

from moe_grouped_gemm_lhs_amd import inputs as I
from tests.helpers import SENTINEL, assert_within_tolerance

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from tests import gpu_util as gu  # noqa: E402

FMTS = ["e4m3", "e5m2"]


def _check(p, what):
    gu.say(f"[case] {what}")
    c_gpu = gu.run_gpu(p)
    c_ref = gu.oracle_full(p)
    w = gu.written_rows(p)
    assert np.all(c_gpu[~w] == SENTINEL), f"{what}: rows outside the routing were written"
    assert_within_tolerance(c_gpu, c_ref, np.repeat(w[:, None], p.N, axis=1), what)


@pytest.mark.parametrize("seed", range(40))
def test_fuzz_dense(seed):
    rng = np.random.default_rng(1000 + seed)
    M = int(rng.choice([int(rng.integers(1, 129)), int(rng.integers(129, 1100))]))
    N = int(rng.integers(1, 1500))
    K = 128 * int(rng.integers(1, 17))
    fa, fb = (FMTS[int(v)] for v in rng.integers(0, 2, size=2))
    p = I.make_dense(M, N, K, seed=2000 + seed, outliers=bool(rng.integers(0, 2)),
                     a_fmt=fa, b_fmt=fb)
    _check(p, f"fuzz dense {M}x{N}x{K} {fa}/{fb}")


@pytest.mark.parametrize("seed", range(20))
def test_fuzz_contiguous(seed):
    rng = np.random.default_rng(3000 + seed)
    G = int(rng.integers(1, 7))
    sizes = [128 * int(v) for v in rng.integers(0, 7, size=G)]
    if sum(sizes) == 0:
        sizes[0] = 128
    N = int(rng.integers(1, 700))
    K = 128 * int(rng.integers(1, 7))
    fa, fb = (FMTS[int(v)] for v in rng.integers(0, 2, size=2))
    p = I.make_contiguous(sizes, N, K, seed=4000 + seed, a_fmt=fa, b_fmt=fb)
    _check(p, f"fuzz contiguous sizes={sizes} N={N} K={K} {fa}/{fb}")


@pytest.mark.parametrize("seed", range(20))
def test_fuzz_masked(seed):
    rng = np.random.default_rng(5000 + seed)
    G = int(rng.integers(1, 9))
    cap = int(rng.integers(1, 600))
    mm = rng.integers(-3, cap + 4, size=G).astype(np.int32)
    N = int(rng.integers(1, 1000))
    K = 128 * int(rng.integers(1, 9))
    fa, fb = (FMTS[int(v)] for v in rng.integers(0, 2, size=2))
    p = I.make_masked(G, cap, N, K, seed=6000 + seed, masked_m=mm, a_fmt=fa, b_fmt=fb)
    _check(p, f"fuzz masked G={G} cap={cap} masked_m={mm.tolist()} N={N} K={K} {fa}/{fb}")
