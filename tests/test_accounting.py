"""The byte/FLOP accounting used by the benchmark reproduces the GB/s column of the
flashmla.org/zh page's three tables from their TFLOPS column (the pages round TFLOPS
to integers, so a few GB/s of difference is expected)."""
from moe_grouped_gemm_lhs_amd import accounting as acc
from tests.helpers import read_table


def test_pages_gbs_column_reproduced():
    rows = read_table("h800_tables.txt")
    assert len(rows) == 28
    for kind, g, m, n, k, tf, gbs, _ in rows:
        g, m, n, k, tf, gbs = int(g), int(m), int(n), int(k), float(tf), float(gbs)
        t = acc.flops(g * m, n, k) / (tf * 1e12)
        derived = acc.pages_bytes(g, m, n, k) / t / 1e9
        assert abs(derived - gbs) <= max(3.5, 0.003 * gbs), (kind, g, m, n, k, derived, gbs)


def test_algorithmic_bytes_counts_only_written_rows():
    f_full, b_full = acc.masked_work([256] * 4, 256, 4096, 7168)
    f_half, b_half = acc.masked_work([128, 0, 256, 300], 256, 4096, 7168)
    assert f_full == 2 * 1024 * 4096 * 7168
    assert f_half == 2 * (128 + 256 + 256) * 4096 * 7168
    # the empty group's B is not counted; every written row's A, sA and C are
    nkb, nnb = 56, 32
    per_row = 7168 + 4 * nkb + 2 * 4096
    per_group = 4096 * 7168 + 4 * nnb * nkb
    assert b_half == 640 * per_row + 3 * per_group + 16
    assert b_full == 1024 * per_row + 4 * per_group + 16
    f, b = acc.dense_work(64, 2112, 7168)
    assert f == 2 * 64 * 2112 * 7168
    assert b == 64 * 7168 + 4 * 64 * 56 + 2112 * 7168 + 4 * 17 * 56 + 2 * 64 * 2112
