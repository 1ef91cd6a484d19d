"""Glue for the GPU parity tests: move a generated Problem to the device, run it through
the C ABI binding, and compute the oracle's answer (whole output or sampled rows)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from moe_grouped_gemm_lhs_amd import binding as dg
from tests.helpers import SENTINEL, rows_written_contiguous, rows_written_masked

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device_operands(p):
    nkb, nnb = -(-p.K // 128), -(-p.N // 128)
    A = torch.from_numpy(p.A).to(DEV)
    sA = torch.from_numpy(p.sA).to(DEV)
    B = torch.from_numpy(p.B).to(DEV)
    sB = torch.from_numpy(p.sB).to(DEV)
    if p.kind == "dense":
        return A, sA, B.view(p.N, p.K), sB.view(nnb, nkb)
    B = B.view(p.G, p.N, p.K)
    sB = sB.view(p.G, nnb, nkb)
    if p.kind == "masked":
        A = A.view(p.G, p.M, p.K)
        sA = sA.view(p.G, p.M, nkb)
    return A, sA, B, sB


def out_shape(p):
    return (p.rows, p.N)


def run_gpu(p, c_init_bits=None, group_idx=None, masked_m=None, ops=None, workspace=None):
    """Run the problem on the GPU; returns C as uint16 bits (rows x N)."""
    A, sA, B, sB = ops if ops is not None else device_operands(p)
    if c_init_bits is None:
        c_init_bits = np.full(out_shape(p), SENTINEL, np.uint16)
    C = torch.from_numpy(c_init_bits.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    fm = dict(a_format=p.a_fmt, b_format=p.b_fmt)
    if p.kind == "dense":
        dg.dg_gemm_fp8_nt(A, sA, B, sB, C, workspace=workspace, **fm)
    elif p.kind == "contiguous":
        gi = group_idx if group_idx is not None else p.group_idx
        dg.dg_grouped_gemm_fp8_contiguous(A, sA, B, sB, torch.from_numpy(gi).to(DEV), C, **fm)
    else:
        mm = masked_m if masked_m is not None else p.masked_m
        Cv = C.view(p.G, p.M, p.N)
        dg.dg_grouped_gemm_fp8_masked(A, sA, B, sB, torch.from_numpy(np.asarray(mm, np.int32)).to(DEV), Cv,
                                      workspace=workspace, **fm)
    torch.cuda.synchronize()
    return C.view(torch.int16).cpu().numpy().view(np.uint16).reshape(out_shape(p))


def written_rows(p, group_idx=None, masked_m=None):
    if p.kind == "dense":
        return np.ones(p.rows, bool)
    if p.kind == "contiguous":
        return rows_written_contiguous(group_idx if group_idx is not None else p.group_idx, p.G)
    return rows_written_masked(masked_m if masked_m is not None else p.masked_m, p.M)


def row_group(p, m, group_idx=None):
    if p.kind == "dense":
        return 0
    if p.kind == "contiguous":
        gi = group_idx if group_idx is not None else p.group_idx
        return int(gi[m])
    return m // p.M


def oracle_rows(p, rows, group_idx=None):
    """Oracle output for the given (written) rows, computed group by group with the
    dense oracle on that group's B (the definition restricted to those rows)."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, p.N), np.uint16)
    nnb = -(-p.N // 128)
    groups = np.array([row_group(p, int(m), group_idx) for m in rows])
    for g in np.unique(groups):
        sel = np.nonzero(groups == g)[0]
        r = rows[sel]
        Bg = p.B[g * p.N:(g + 1) * p.N]
        sBg = p.sB[g * nnb:(g + 1) * nnb]
        out[sel] = oracle.gemm_fp8_nt(p.A[r], p.sA[r], Bg, sBg, a_fmt=p.a_fmt, b_fmt=p.b_fmt)
    return out


def oracle_full(p, c_init_bits=None, group_idx=None, masked_m=None):
    if c_init_bits is None:
        c_init_bits = np.full(out_shape(p), SENTINEL, np.uint16)
    C = c_init_bits.copy()
    fm = dict(a_fmt=p.a_fmt, b_fmt=p.b_fmt)
    if p.kind == "dense":
        oracle.gemm_fp8_nt(p.A, p.sA, p.B, p.sB, C=C, **fm)
    elif p.kind == "contiguous":
        gi = group_idx if group_idx is not None else p.group_idx
        oracle.grouped_contiguous(p.A, p.sA, p.B, p.sB, gi, p.G, C=C, **fm)
    else:
        mm = masked_m if masked_m is not None else p.masked_m
        oracle.grouped_masked(p.A, p.sA, p.B, p.sB, np.asarray(mm, np.int32), p.G, p.M, C=C,
                              **fm)
    return C


def sample_rows(p, written, per_group=24, seed=0):
    """Rows to check at full size: the first and the last written row of every 128-row
    block that has written rows (routing goes by 128-row blocks, so a block computed
    with the wrong group's B, or not at all, shows in them), plus random written rows."""
    rng = np.random.default_rng(seed)
    w = np.nonzero(written)[0]
    if w.size <= 4 * per_group:
        return w
    picks = set()
    blocks = w // 128
    first = np.r_[True, blocks[1:] != blocks[:-1]]
    last = np.r_[blocks[1:] != blocks[:-1], True]
    picks.update(w[first].tolist())
    picks.update(w[last].tolist())
    picks.update(rng.choice(w, size=min(w.size, 4 * per_group), replace=False).tolist())
    return np.array(sorted(picks), dtype=np.int64)
