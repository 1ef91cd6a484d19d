"""Host-side checks of libdg that need no GPU: the library loads, exports every symbol
that include/dg.h declares, and its argument validation returns each documented error
code before touching any device state."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")


@pytest.fixture(scope="module")
def lib():
    from moe_grouped_gemm_lhs_amd import build, binding
    if not os.path.exists(binding.LIB_PATH):
        if not os.path.exists(build.HIPCC):
            pytest.skip("libdg.so not built and hipcc unavailable")
        build.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"dg_gemm_fp8_nt", "dg_grouped_gemm_fp8_contiguous", "dg_grouped_gemm_fp8_masked",
            "dg_get_m_alignment_for_contiguous_layout", "dg_workspace_bytes",
            "dg_status_string", "dg_instance_name"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_constants_and_strings(lib):
    from moe_grouped_gemm_lhs_amd import binding as b
    assert b.dg_get_m_alignment_for_contiguous_layout() == 128
    want = ["DG_OK", "DG_ERR_NULL", "DG_ERR_SHAPE", "DG_ERR_ALIGN", "DG_ERR_WORKSPACE",
            "DG_ERR_DEVICE", "DG_ERR_HIP", "DG_ERR_FORMAT"]
    assert [b.dg_status_string(i) for i in range(8)] == want
    assert b.dg_status_string(99) == "DG_ERR_UNKNOWN"


A16 = 0x10000        # fake, 16-byte aligned addresses: validation never dereferences
A4 = 0x20004
BAD16 = 0x10008


def dense(lib, A=A16, sA=A4, B=A16, sB=A4, C=A16, M=64, N=256, K=512):
    return lib.dg_gemm_fp8_nt(A, sA, B, sB, C, M, N, K, None, 0, None)


def test_dense_validation_codes(lib):
    assert dense(lib, K=100) == 2
    assert dense(lib, K=0) == 2
    assert dense(lib, M=-1) == 2
    assert dense(lib, M=0) == 0          # empty output: nothing to do, pointers unused
    assert dense(lib, N=0, A=None) == 0
    assert dense(lib, A=None) == 1
    assert dense(lib, sB=None) == 1
    assert dense(lib, C=None) == 1
    assert dense(lib, A=BAD16) == 3
    assert dense(lib, C=A16 + 2) == 3
    assert dense(lib, sA=A4 + 1) == 3
    assert dense(lib, M=1 << 31) == 2
    assert dense(lib, K=1 << 23) == 2     # 32-bit offsets within a tile's rows of A and B
    assert dense(lib, M=1 << 30, N=1 << 30) == 2   # more tiles than 32-bit tile indices


def test_format_validation_codes(lib):
    f = lib.dg_gemm_fp8_nt_ex
    # formats are checked right after the shapes, before the empty-output shortcut
    assert f(A16, 2, A4, A16, 0, A4, A16, 64, 256, 512, None, 0, None) == 7
    assert f(A16, 0, A4, A16, -1, A4, A16, 64, 256, 512, None, 0, None) == 7
    assert f(A16, 5, A4, A16, 0, A4, A16, 0, 256, 512, None, 0, None) == 7
    assert f(A16, 5, A4, A16, 0, A4, A16, 64, 256, 100, None, 0, None) == 2    # shape first
    for fa in (0, 1):
        for fb in (0, 1):
            assert f(A16, fa, A4, A16, fb, A4, A16, 0, 256, 512, None, 0, None) == 0
            assert f(None, fa, A4, A16, fb, A4, A16, 64, 256, 512, None, 0, None) == 1
    c = lib.dg_grouped_gemm_fp8_contiguous_ex
    assert c(A16, 0, A4, A16, 3, A4, A4, A16, 256, 128, 128, 2, None, 0, None) == 7
    assert c(A16, 1, A4, A16, 1, A4, None, A16, 256, 128, 128, 2, None, 0, None) == 1
    m = lib.dg_grouped_gemm_fp8_masked_ex
    assert m(A16, 7, A4, A16, 0, A4, A4, A16, 2, 64, 128, 128, None, 0, None) == 7
    assert m(A16, 1, A4, A16, 0, A4, None, A16, 2, 64, 128, 128, None, 0, None) == 1


def test_quantize_validation_codes(lib):
    for f in (lib.dg_quantize_fp8_1x128, lib.dg_quantize_fp8_128x128):
        assert f(A16, 0, A16, A4, 64, 100, 0, None) == 2      # K % 128
        assert f(A16, 0, A16, A4, -1, 128, 0, None) == 2
        assert f(A16, 0, A16, A4, 64, 128, 2, None) == 7      # format
        assert f(A16, 2, A16, A4, 64, 128, 0, None) == 7      # input dtype
        assert f(None, 0, A16, A4, 0, 128, 1, None) == 0      # nothing to do
        assert f(None, 0, A16, A4, 64, 128, 0, None) == 1
        assert f(A16, 1, A16, None, 64, 128, 0, None) == 1
        assert f(A16 + 8, 0, A16, A4, 64, 128, 0, None) == 3  # 16-byte input loads
        assert f(A16 + 8, 1, A16, A4, 64, 128, 0, None) == 3  # bf16 too
        assert f(A16, 0, A16 + 4, A4, 64, 128, 0, None) == 3  # 8-byte code stores
        assert f(A16, 0, A16, A4 + 1, 64, 128, 0, None) == 3


def test_transpose_validation_codes(lib):
    f = lib.dg_transpose_fp8
    assert f(A16, A16, 64, 100, None) == 2
    assert f(A16, A16, 8, 64, None) == 2
    assert f(A16, A16, -16, 64, None) == 2
    assert f(None, A16, 0, 64, None) == 0
    assert f(None, A16, 64, 64, None) == 1
    assert f(A16, None, 64, 64, None) == 1
    assert f(A16 + 4, A16, 64, 64, None) == 3
    assert f(A16, A16 + 8, 64, 64, None) == 3


def test_grouped_validation_codes(lib):
    c = lib.dg_grouped_gemm_fp8_contiguous
    assert c(A16, A4, A16, A4, A4, A16, 256, 128, 128, 0, None, 0, None) == 2   # G < 1
    assert c(A16, A4, A16, A4, None, A16, 256, 128, 128, 2, None, 0, None) == 1
    assert c(A16, A4, A16, A4, A4 + 2, A16, 256, 128, 128, 2, None, 0, None) == 3
    assert c(A16, A4, A16, A4, A4, A16, 0, 128, 128, 2, None, 0, None) == 0
    m = lib.dg_grouped_gemm_fp8_masked
    assert m(A16, A4, A16, A4, A4, A16, 2, 64, 128, 96, None, 0, None) == 2     # K % 128
    assert m(A16, A4, A16, A4, None, A16, 2, 64, 128, 128, None, 0, None) == 1
    assert m(A16, A4, A16, A4, A4, BAD16, 2, 64, 128, 128, None, 0, None) == 3
    assert m(A16, A4, A16, A4, A4, A16, 2, 0, 128, 128, None, 0, None) == 0
    assert m(A16, A4, A16, A4, A4, A16, 1 << 16, 1 << 16, 128, 128, None, 0, None) == 2


def test_workspace_validation(lib):
    from moe_grouped_gemm_lhs_amd import binding as b
    need = b.dg_workspace_bytes(0, 64, 256, 512, 1)
    assert need >= 256 * 2 * 64 * 64 * 4   # stream-K decode instance: two partial tiles per workgroup
    f = lib.dg_gemm_fp8_nt
    assert f(A16, A4, A16, A4, A16, 64, 256, 512, None, need, None) == 4
    assert f(A16, A4, A16, A4, A16, 64, 256, 512, A16, need - 1, None) == 4
    assert f(A16, A4, A16, A4, A16, 64, 256, 512, A16 + 8, need, None) == 4   # alignment
    assert b.dg_workspace_bytes(0, 4096, 4096, 7168, 1) == 0                  # tiled: none


def test_device_check_without_gpu(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: valid-looking fake pointers would be launched")
    from moe_grouped_gemm_lhs_amd import binding as b
    need = b.dg_workspace_bytes(0, 64, 256, 512, 1)
    assert lib.dg_gemm_fp8_nt(A16, A4, A16, A4, A16, 64, 256, 512, A16, need, None) == 5
    assert lib.dg_gemm_fp8_nt(A16, A4, A16, A4, A16, 4096, 4096, 512, None, 0, None) == 5
    # aligned fake pointers pass validation; the device check then fails
    assert lib.dg_quantize_fp8_1x128(A16, 1, A16 + 8, A4 + 4, 64, 128, 1, None) == 5
    assert lib.dg_quantize_fp8_128x128(A16, 1, A16 + 8, A4 + 4, 64, 128, 1, None) == 5


def test_instance_selection_is_host_logic(lib):
    from moe_grouped_gemm_lhs_amd import binding as b
    assert b.dg_instance_name(0, 0, 128, 128) == "none"
    assert b.dg_instance_name(0, 64, 128, 100) == "none"
    for kind, rows, n, k, g in [(0, 64, 2112, 7168, 1), (0, 4096, 7168, 16384, 1),
                                (1, 32768, 4096, 7168, 4), (2, 256, 7168, 2048, 4)]:
        name = b.dg_instance_name(kind, rows, n, k, g)
        assert name != "none"
        assert ("dense", "contig", "masked")[kind] in name
        ws = b.dg_workspace_bytes(kind, rows, n, k, g)
        assert ws >= 0
    assert b.dg_workspace_bytes(0, 64, 2112, 100, 1) == 0


def test_tiled_selection_uses_measured_tile_efficiency(lib):
    """The tile-shape heuristic (full rounds of tiles over 256 CUs, divided by each shape's
    measured per-area efficiency) on the bench's prefill and contiguous shapes: the
    narrower 256x224 / 256x160 tiles only where they save a whole round of tiles, never
    for the contiguous form."""
    from moe_grouped_gemm_lhs_amd import binding as b
    dense = {(2112, 7168): "dense_256x160", (24576, 1536): "dense_256x256",
             (32768, 512): "dense_256x256", (7168, 16384): "dense_256x224",
             (4096, 7168): "dense_256x256", (7168, 2048): "dense_256x224"}
    for (n, k), name in dense.items():
        assert b.dg_instance_name(0, 4096, n, k, 1) == name, (n, k)
    for rows, n, k, g in [(32768, 4096, 7168, 4), (30592, 4096, 7168, 8),
                          (32768, 7168, 2048, 8), (24448, 7168, 2048, 8)]:
        assert b.dg_instance_name(1, rows, n, k, g) == "contig_256x256", (rows, n, k)


def test_decode_selection(lib):
    """Decode shapes (all rows in one tile) take the split-K instances: 128-column tiles
    unless their grid would leave more than a quarter of the CUs idle, and the 4-wave
    build of the 128-column tile when the ranges average 16 K blocks or more."""
    from moe_grouped_gemm_lhs_amd import binding as b
    want = {(64, 2112, 7168): "dense_64x64_stream", (64, 24576, 1536): "dense_64x128_stream",
            (64, 7168, 16384): "dense_64x128_stream_4w", (64, 4096, 7168): "dense_64x128_stream",
            (128, 2112, 7168): "dense_128x64_stream", (128, 32768, 512): "dense_128x128_stream",
            (128, 7168, 16384): "dense_128x128_stream_4w",
            (128, 4096, 7168): "dense_128x128_stream", (128, 7168, 2048): "dense_128x64_stream"}
    for (m, n, k), name in want.items():
        assert b.dg_instance_name(0, m, n, k, 1) == name, (m, n, k)


def test_masked_selection(lib):
    """Masked calls whose groups each fit one 128-row tile (at most 64 groups) and whose
    column tiles are fewer than the CUs take the split-K instances that schedule on the
    device; otherwise the tiled ones."""
    from moe_grouped_gemm_lhs_amd import binding as b
    assert b.dg_instance_name(2, 128, 4096, 7168, 4) == "masked_128x128_stream"
    assert b.dg_instance_name(2, 128, 4096, 7168, 8) == "masked_128x128"     # 256 tiles
    assert b.dg_instance_name(2, 64, 4096, 7168, 32) == "masked_64x128"
    assert b.dg_instance_name(2, 100, 256, 512, 2) == "masked_128x64_stream"
    assert b.dg_instance_name(2, 64, 512, 512, 100) == "masked_64x128"
    assert b.dg_instance_name(2, 256, 4096, 7168, 4) == "masked_128x128"
    assert b.dg_instance_name(2, 128, 4096, 7168, 65).startswith("masked_") and \
        "stream" not in b.dg_instance_name(2, 128, 4096, 7168, 65)
    assert b.dg_workspace_bytes(2, 128, 4096, 7168, 4) > 0
    assert b.dg_workspace_bytes(2, 256, 4096, 7168, 4) == 0


def test_selection_is_reentrant_across_host_threads(lib):
    """dg_instance_name and dg_workspace_bytes called from 8 host threads at once give the
    same answers as single-threaded calls (ctypes releases the GIL around each call)."""
    import threading
    shapes = []
    for kind in (0, 1, 2):
        for rows in (64, 128, 1024, 4096, 32768):
            for n, k in ((2112, 7168), (7168, 2048), (4096, 7168), (24576, 1536)):
                shapes.append((kind, rows, n, k, 4))
    want = [(lib.dg_instance_name(*s), lib.dg_workspace_bytes(*s)) for s in shapes]
    errors = []

    def worker(t):
        for rep in range(40):
            order = shapes[t::3] + shapes
            for s in order:
                got = (lib.dg_instance_name(*s), lib.dg_workspace_bytes(*s))
                if got != want[shapes.index(s)]:
                    errors.append((s, got))
                    return

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]
