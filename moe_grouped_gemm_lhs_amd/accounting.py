"""Algorithmic work of one call: FLOPs and HBM bytes the method must move.

FLOPs = 2 * (written rows) * N * K.  Bytes count each operand once: e4m3 A rows that
are computed, B (N*K) of every group with at least one written row, fp32 scales of
those rows/groups, bf16 C of the written rows, and the routing metadata.  Padded
capacity rows and skipped groups count nothing.

``pages_bytes`` is the convention behind the GB/s column of the flashmla.org/zh
page's three tables: FP8 A and B plus BF16 C, scales ignored, every row counted.
"""
from __future__ import annotations

BLOCK = 128


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def flops(rows: int, N: int, K: int) -> int:
    return 2 * int(rows) * int(N) * int(K)


def algorithmic_bytes(rows: int, N: int, K: int, active_groups: int = 1,
                      meta_bytes: int = 0) -> int:
    nkb = _cdiv(K, BLOCK)
    nnb = _cdiv(N, BLOCK)
    a = rows * K + 4 * rows * nkb
    b = active_groups * (N * K + 4 * nnb * nkb)
    c = 2 * rows * N
    return int(a + b + c + meta_bytes)


def pages_bytes(groups: int, m_per_group: int, N: int, K: int) -> int:
    rows = groups * m_per_group
    return int(rows * K + groups * N * K + 2 * rows * N)


def dense_work(M: int, N: int, K: int):
    return flops(M, N, K), algorithmic_bytes(M, N, K, 1)


def contiguous_work(sizes, N: int, K: int):
    rows = sum(sizes)
    active = sum(1 for s in sizes if s > 0)
    return flops(rows, N, K), algorithmic_bytes(rows, N, K, active, meta_bytes=4 * rows)


def masked_work(masked_m, cap: int, N: int, K: int):
    valid = [min(max(int(v), 0), cap) for v in masked_m]
    rows = sum(valid)
    active = sum(1 for v in valid if v > 0)
    return flops(rows, N, K), algorithmic_bytes(rows, N, K, active, meta_bytes=4 * len(valid))
