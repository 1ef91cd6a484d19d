"""Seeded synthetic inputs for the FP8 block-scaled NT GEMM (dense, contiguous-grouped,
masked-grouped).

This module is shared by the GPU path's tests and benchmark and by the CPU oracle's
tests.  It holds no GEMM arithmetic: it draws normal samples, quantises them to
e4m3fn bytes with fp32 block scales (the casting step that the DeepGEMM pages leave
to the user, turtlesai.it summary page, technical paragraph), and builds the routing
metadata (per-row group indices, per-group valid-row counts).

Workload shapes are the DeepSeek-V3/R1 matrix shapes that the flashmla.org/zh page
benchmarks (its dense, contiguous-grouped and masked-grouped tables).

Recipe (identical for every consumer):
  * Scalars that pick the routing (group sizes, masked_m) come from
    ``numpy.random.default_rng(seed)`` in a fixed order: contiguous sizes first, then
    masked_m.
  * Each large fp32 tensor is drawn in row chunks; chunk ``c`` of tensor ``tag`` uses
    its own PCG64 stream ``default_rng([seed, tag, c])``, so chunks can be drawn in
    parallel threads and the result does not depend on the thread count.  Values are
    standard normal float32; with ``outliers`` each entry is replaced, with
    probability 0.01, by 30 times a fresh standard normal (a heavy-tailed
    population that exercises per-block scaling).
  * Quantisation: per block, amax = max |x| (fp32), scale = amax / FMAX (fp32;
    1 when amax == 0), code = fp8(x / scale) with round-to-nearest-even, saturating
    at +-FMAX; the 8-bit format is E4M3 ("fn", FMAX = 448) by default, or E5M2
    (FMAX = 57344), the other input format the aisharenet.com/ja usage guide names
    (main functions, section 1).  A uses 1x128 blocks along K (one scale per row and K block);
    B uses 128x128 blocks (one scale per 128 rows of B, i.e. 128 output columns, and K
    block).  A final partial block (N not a multiple of 128) takes its amax over the
    rows that exist.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np
import torch

E4M3_MAX = 448.0
E5M2_MAX = 57344.0
BLOCK = 128
FP8_MAX = {"e4m3": E4M3_MAX, "e5m2": E5M2_MAX}
FP8_DTYPE = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}

# tensor tags for the per-tensor random streams
_TAG_A = 1
_TAG_B = 2


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_chunk(seed: int, tag: int, chunk: int, shape, outliers: bool) -> np.ndarray:
    rng = np.random.default_rng([seed, tag, chunk])
    x = rng.standard_normal(shape, dtype=np.float32)
    if outliers:
        mask = rng.random(shape, dtype=np.float32) < 0.01
        cnt = int(mask.sum())
        if cnt:
            x[mask] = np.float32(30.0) * rng.standard_normal(cnt, dtype=np.float32)
    return x


def normal_matrix(seed: int, tag: int, rows: int, cols: int, outliers: bool = False,
                  chunk_elems: int = 1 << 23) -> np.ndarray:
    """Draw a rows x cols float32 matrix by row chunks (see the module recipe)."""
    out = np.empty((rows, cols), dtype=np.float32)
    if rows == 0 or cols == 0:
        return out
    rows_per = max(1, chunk_elems // max(cols, 1))
    starts = list(range(0, rows, rows_per))

    def work(ci: int) -> None:
        r0 = starts[ci]
        r1 = min(rows, r0 + rows_per)
        out[r0:r1] = _normal_chunk(seed, tag, ci, (r1 - r0, cols), outliers)

    if len(starts) == 1:
        work(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(len(starts))))
    return out


def fp8_encode(x: torch.Tensor, fmt: str = "e4m3") -> torch.Tensor:
    """fp32 -> fp8 bytes (E4M3 or E5M2), round-to-nearest-even, saturating."""
    m = FP8_MAX[fmt]
    return x.clamp(-m, m).to(FP8_DTYPE[fmt]).view(torch.uint8)


def e4m3fn_encode(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> e4m3fn bytes, round-to-nearest-even, saturating at +-448."""
    return fp8_encode(x, "e4m3")


def _pad_to(t: torch.Tensor, rows: int, cols: int) -> torch.Tensor:
    if t.shape[0] == rows and t.shape[1] == cols:
        return t
    out = torch.zeros((rows, cols), dtype=t.dtype)
    out[: t.shape[0], : t.shape[1]] = t
    return out


def _scale_of(amax: torch.Tensor, fmt: str = "e4m3") -> torch.Tensor:
    return torch.where(amax == 0, torch.ones_like(amax), amax / FP8_MAX[fmt])


def quantize_1x128(x: np.ndarray, fmt: str = "e4m3"):
    """Per-row, per-128-wide-K-block quantisation of a rows x K float32 matrix.

    Returns (codes uint8 rows x K, scales float32 rows x ceil(K/128))."""
    rows, K = x.shape
    nkb = -(-K // BLOCK)
    t = _pad_to(torch.from_numpy(x), rows, nkb * BLOCK).view(rows, nkb, BLOCK)
    scales = _scale_of(t.abs().amax(dim=2), fmt)                   # rows x nkb
    codes = fp8_encode(t / scales[:, :, None], fmt).view(rows, nkb * BLOCK)[:, :K]
    return np.ascontiguousarray(codes.numpy()), scales.numpy()


def quantize_128x128(x: np.ndarray, fmt: str = "e4m3"):
    """Per 128x128 block quantisation of an N x K float32 matrix (B stored N x K).

    Returns (codes uint8 N x K, scales float32 ceil(N/128) x ceil(K/128))."""
    N, K = x.shape
    nnb, nkb = -(-N // BLOCK), -(-K // BLOCK)
    t = _pad_to(torch.from_numpy(x), nnb * BLOCK, nkb * BLOCK).view(nnb, BLOCK, nkb, BLOCK)
    scales = _scale_of(t.abs().amax(dim=(1, 3)), fmt)              # nnb x nkb
    codes = fp8_encode(t / scales[:, None, :, None], fmt).view(nnb * BLOCK, nkb * BLOCK)
    return np.ascontiguousarray(codes[:N, :K].numpy()), scales.numpy()


def group_sizes_to_idx(sizes) -> np.ndarray:
    """Expand a list of contiguous group sizes into the per-row int32 group index."""
    sizes = [int(s) for s in sizes]
    return np.repeat(np.arange(len(sizes), dtype=np.int32), sizes)


@dataclass
class Problem:
    """One call's operands.  kind is 'dense', 'contiguous' or 'masked'."""
    kind: str
    M: int          # dense: M; contiguous: total rows; masked: capacity per group
    N: int
    K: int
    G: int
    A: np.ndarray   # uint8, rows x K  (masked: G*cap x K)
    sA: np.ndarray  # float32, rows x K/128
    B: np.ndarray   # uint8, G*N x K
    sB: np.ndarray  # float32, G*ceil(N/128) x K/128
    group_idx: np.ndarray | None = None   # int32 per row (contiguous)
    masked_m: np.ndarray | None = None    # int32 per group (masked)
    sizes: list | None = None
    seed: int = 0
    meta: dict = field(default_factory=dict)
    a_fmt: str = "e4m3"     # operand formats: "e4m3" or "e5m2"
    b_fmt: str = "e4m3"

    @property
    def rows(self) -> int:
        return self.A.shape[0]


def _quant_B(seed: int, G: int, N: int, K: int, outliers: bool, fmt: str = "e4m3"):
    Bs, sBs = [], []
    for g in range(G):
        b = normal_matrix(seed, _TAG_B + 16 * g, N, K, outliers)
        q, s = quantize_128x128(b, fmt)
        Bs.append(q)
        sBs.append(s)
    return np.concatenate(Bs, 0), np.concatenate(sBs, 0)


def make_dense(M: int, N: int, K: int, seed: int, outliers: bool = False,
               a_fmt: str = "e4m3", b_fmt: str = "e4m3") -> Problem:
    a = normal_matrix(seed, _TAG_A, M, K, outliers)
    A, sA = quantize_1x128(a, a_fmt)
    del a
    B, sB = _quant_B(seed, 1, N, K, outliers, b_fmt)
    return Problem("dense", M, N, K, 1, A, sA, B, sB, seed=seed, a_fmt=a_fmt, b_fmt=b_fmt)


def make_contiguous(sizes, N: int, K: int, seed: int, a_fmt: str = "e4m3",
                    b_fmt: str = "e4m3") -> Problem:
    sizes = [int(s) for s in sizes]
    G = len(sizes)
    rows = sum(sizes)
    a = normal_matrix(seed, _TAG_A, rows, K)
    A, sA = quantize_1x128(a, a_fmt)
    del a
    B, sB = _quant_B(seed, G, N, K, False, b_fmt)
    gi = group_sizes_to_idx(sizes)
    return Problem("contiguous", rows, N, K, G, A, sA, B, sB, group_idx=gi, sizes=sizes,
                   seed=seed, a_fmt=a_fmt, b_fmt=b_fmt)


def random_contiguous_sizes(seed: int, G: int = 8, align: int = 128, max_blocks: int = 64):
    """Group sizes drawn uniformly from the multiples of `align` in [align, align*max_blocks]."""
    rng = np.random.default_rng(seed)
    return [int(v) * align for v in rng.integers(1, max_blocks + 1, size=G)]


def masked_counts(G: int, cap: int, seed: int) -> np.ndarray:
    """The masked workload's per-group valid-row counts, uniform on [0, cap]."""
    return np.random.default_rng(seed).integers(0, cap + 1, size=G).astype(np.int32)


def make_masked(G: int, cap: int, N: int, K: int, seed: int, masked_m=None,
                a_fmt: str = "e4m3", b_fmt: str = "e4m3") -> Problem:
    if masked_m is None:
        masked_m = masked_counts(G, cap, seed)
    masked_m = np.asarray(masked_m, dtype=np.int32)
    a = normal_matrix(seed, _TAG_A, G * cap, K)
    A, sA = quantize_1x128(a, a_fmt)
    del a
    B, sB = _quant_B(seed, G, N, K, False, b_fmt)
    return Problem("masked", cap, N, K, G, A, sA, B, sB, masked_m=masked_m, seed=seed,
                   a_fmt=a_fmt, b_fmt=b_fmt)


# --------------------------------------------------------------------------------------
# The workloads: the shapes of the flashmla.org/zh page's three benchmark tables.

DECODE_NK = [(2112, 7168), (24576, 1536), (32768, 512), (7168, 16384), (4096, 7168),
             (7168, 2048)]
GROUPED_NK = [(4096, 7168), (7168, 2048)]
MASKED_GC = [(1, 1024), (2, 512), (4, 256)]


def small_case():
    """128x256x512 dense, seed 0: the smallest instance."""
    return [dict(kind="dense", M=128, N=256, K=512, seed=0, outliers=False)]


def decode_cases():
    """Dense decode shapes: M in {64,128} x the six (N,K) pairs; seed = shape index."""
    out = []
    for mi, M in enumerate((64, 128)):
        for j, (N, K) in enumerate(DECODE_NK):
            out.append(dict(kind="dense", M=M, N=N, K=K, seed=6 * mi + j, outliers=False))
    return out


def prefill_cases():
    """Dense prefill shapes: M=4096 x the six (N,K) pairs, 1% N(0,30) outliers."""
    return [dict(kind="dense", M=4096, N=N, K=K, seed=12 + j, outliers=True)
            for j, (N, K) in enumerate(DECODE_NK)]


def contiguous_cases():
    """4x8192 rows, 8x4096 rows, 8 random multiples of 128 in [128, 8192]."""
    out = []
    for c, (N, K) in enumerate(GROUPED_NK):
        for t, kind in enumerate(("4x8192", "8x4096", "8xrand")):
            seed = 18 + 3 * c + t
            if kind == "4x8192":
                sizes = [8192] * 4
            elif kind == "8x4096":
                sizes = [4096] * 8
            else:
                sizes = random_contiguous_sizes(seed)
            out.append(dict(kind="contiguous", sizes=sizes, N=N, K=K, seed=seed, name=kind))
    return out


def masked_cases():
    out = []
    for c, (N, K) in enumerate(GROUPED_NK):
        for t, (G, cap) in enumerate(MASKED_GC):
            out.append(dict(kind="masked", G=G, cap=cap, N=N, K=K, seed=24 + 3 * c + t))
    return out


def make(case: dict) -> Problem:
    k = case["kind"]
    fmts = dict(a_fmt=case.get("a_fmt", "e4m3"), b_fmt=case.get("b_fmt", "e4m3"))
    if k == "dense":
        return make_dense(case["M"], case["N"], case["K"], case["seed"],
                          case.get("outliers", False), **fmts)
    if k == "contiguous":
        return make_contiguous(case["sizes"], case["N"], case["K"], case["seed"], **fmts)
    if k == "masked":
        return make_masked(case["G"], case["cap"], case["N"], case["K"], case["seed"],
                           case.get("masked_m"), **fmts)
    raise ValueError(k)


def with_formats(cases, a_fmt: str, b_fmt: str):
    """The same cases with other operand formats (the draws are unchanged)."""
    return [dict(c, a_fmt=a_fmt, b_fmt=b_fmt) for c in cases]


def case_name(case: dict) -> str:
    k = case["kind"]
    fm = ""
    if case.get("a_fmt", "e4m3") != "e4m3" or case.get("b_fmt", "e4m3") != "e4m3":
        fm = f"_{case.get('a_fmt', 'e4m3')}x{case.get('b_fmt', 'e4m3')}"
    if k == "dense":
        return f"dense_{case['M']}x{case['N']}x{case['K']}{fm}"
    if k == "contiguous":
        return f"contig_{case.get('name', len(case['sizes']))}_{case['N']}x{case['K']}{fm}"
    return f"masked_{case['G']}x{case['cap']}_{case['N']}x{case['K']}{fm}"
