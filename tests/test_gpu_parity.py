"""GPU parity of libdg against the CPU oracle (needs an MI355X and the built library).

Small cases compare every element; the workload shapes compare sampled rows (the
oracle computes them one by one) plus the exact set of written rows over the whole
output.  Floating-point results must satisfy, per written element,
|C_gpu - C_ref| <= 2^-7 |C_ref| + 1e-3 max|C_ref|; routing and masking (which rows are
written, and the untouched bits of the others) must match exactly; integer-valued
inputs must match bit for bit."""
import os

import numpy as np
import pytest

from moe_grouped_gemm_lhs_amd import inputs as I
from tests.helpers import (SENTINEL, assert_within_tolerance, bf16_to_f64, e4m3_codes_of,
                           fp8_codes_of, read_sections)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from tests import gpu_util as gu  # noqa: E402


def check_full(p, what, group_idx=None, masked_m=None):
    gu.say(f"[case] {what}")
    c_gpu = gu.run_gpu(p, group_idx=group_idx, masked_m=masked_m)
    c_ref = gu.oracle_full(p, group_idx=group_idx, masked_m=masked_m)
    w = gu.written_rows(p, group_idx, masked_m)
    written = np.repeat(w[:, None], p.N, axis=1)
    assert_within_tolerance(c_gpu, c_ref, written, what)
    return c_gpu


def check_sampled(p, what, seed=0):
    gu.say(f"[case] {what} (sampled rows)")
    c_gpu = gu.run_gpu(p)
    w = gu.written_rows(p)
    # routing: exactly the written rows changed; every other row keeps the sentinel
    untouched = c_gpu[~w]
    assert np.all(untouched == SENTINEL), f"{what}: rows outside the routing were written"
    # and every written row was written in full (no output value is near -6.2e18)
    missed = np.argwhere(c_gpu[w] == SENTINEL)
    assert missed.size == 0, f"{what}: {len(missed)} written elements still hold the sentinel"
    rows = gu.sample_rows(p, w, seed=seed)
    if rows.size == 0:
        return
    c_ref = gu.oracle_rows(p, rows)
    assert_within_tolerance(c_gpu[rows], c_ref, np.ones_like(c_ref, bool), what)


# ----------------------------------------------------------------------- small cases
def test_smallest_instance_128x256x512():
    p = I.make_dense(128, 256, 512, seed=0)
    check_full(p, "dense 128x256x512 seed 0")


def test_worked_example_padded_to_one_k_block():
    fx = read_sections("worked_example_3x2x4.txt")
    Ap = np.zeros((3, 128)); Ap[:, :2] = fx["A"]
    Bp = np.zeros((4, 128)); Bp[:, :2] = fx["Bt"]
    p = I.Problem("dense", 3, 4, 128, 1, e4m3_codes_of(Ap), np.ones((3, 1), np.float32),
                  e4m3_codes_of(Bp), np.ones((1, 1), np.float32))
    gu.say("[case] worked example")
    c = gu.run_gpu(p)
    assert np.array_equal(bf16_to_f64(c), fx["C"])


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (17, 200, 384), (130, 300, 256),
                                   (64, 16, 128), (257, 520, 1024), (300, 2112, 640),
                                   (129, 130, 128), (1000, 1100, 384)])
def test_dense_ragged(M, N, K):
    p = I.make_dense(M, N, K, seed=M * 7 + N, outliers=True)
    check_full(p, f"dense ragged {M}x{N}x{K}")


@pytest.mark.parametrize("kind", ["dense", "contiguous", "masked"])
def test_every_instance_on_ragged_problem(kind, monkeypatch):
    """Force each compiled instance of a kind on one ragged problem."""
    from moe_grouped_gemm_lhs_amd import binding as b
    names = set()
    for rows in (1, 16, 64, 65, 96, 128, 200, 256, 1024, 2000, 4096, 32768):
        for n, k in ((256, 512), (2112, 7168), (7168, 2048), (24576, 1536), (32768, 512),
                     (7168, 16384), (4096, 7168)):
            names.add(b.dg_instance_name(("dense", "contiguous", "masked").index(kind), rows, n, k, 4))
    names.discard("none")
    for name in sorted(names):
        monkeypatch.setenv("DG_FORCE_INSTANCE", name)
        if kind == "dense":
            p = I.make_dense(333, 400, 512, seed=5)
        elif kind == "contiguous":
            p = I.make_contiguous([256, 128, 384], 400, 384, seed=6)
        else:
            p = I.make_masked(3, 200, 400, 384, seed=7, masked_m=[200, 37, 0])
        check_full(p, f"{kind} forced {name}")
    monkeypatch.delenv("DG_FORCE_INSTANCE")


# tiled instances and problems with more tiles than workgroups (several work items per
# workgroup, so the copy pipeline crosses item boundaries); K = 128 / 256 gives items
# shorter than the 3- and 4-stage pipelines (each item then fills and drains its own)
TILED_CASES = [
    # (instance, kind, rows or group sizes / (G, cap), tile columns, K values)
    ("dense_256x256", "dense", 4096, 17 * 256, (128, 384)),
    ("dense_256x224", "dense", 4096, 17 * 224, (128, 384)),
    ("dense_256x160", "dense", 4096, 17 * 160, (256,)),
    ("dense_128x128", "dense", 2048, 17 * 128, (128, 256)),
    ("contig_256x256", "contiguous", [1152, 896, 2048], 17 * 256, (128, 384)),
    ("contig_256x224", "contiguous", [1152, 896, 2048], 17 * 224, (256,)),
    ("contig_128x128", "contiguous", [640, 384, 1024], 17 * 128, (128, 256)),
    ("masked_256x256", "masked", (2, 2048), 17 * 256, (128,)),
    ("masked_128x128", "masked", (2, 1024), 17 * 128, (128, 256)),
    ("masked_64x128", "masked", (4, 512), 9 * 128, (128, 256, 384)),
]


@pytest.mark.parametrize("case", TILED_CASES, ids=[c[0] for c in TILED_CASES])
@pytest.mark.parametrize("ragged_n", [False, True], ids=["n8", "nodd"])
def test_tiled_pipeline_across_items(case, ragged_n, monkeypatch):
    """Each tiled instance on a problem with more tiles than the persistent grid, for
    short and longer K, with N a multiple of 8 (fixed-count stores) and not (element-wise
    stores at the right edge); every row checked for routing, sampled rows against the
    oracle."""
    name, kind, rows, n, ks = case
    n = n - 3 if ragged_n else n
    monkeypatch.setenv("DG_FORCE_INSTANCE", name)
    for K in ks:
        seed = len(name) + K // 128 + (1 if ragged_n else 0)
        if kind == "dense":
            p = I.make_dense(rows, n, K, seed=seed)
        elif kind == "contiguous":
            p = I.make_contiguous(rows, n, K, seed=seed)
        else:
            G, cap = rows
            p = I.make_masked(G, cap, n, K, seed=seed,
                              masked_m=[cap - 1 - 300 * g for g in range(G)])
        check_sampled(p, f"{name} N={n} K={K} across items", seed=K)
    monkeypatch.delenv("DG_FORCE_INSTANCE")


STREAM_INSTANCES = ["dense_64x64_stream", "dense_64x128_stream", "dense_64x128_stream_4w",
                    "dense_128x64_stream", "dense_128x128_stream", "dense_128x128_stream_4w"]


@pytest.mark.parametrize("M,N,K", [(64, 64, 128 * 200), (128, 200, 16384), (1, 130, 128 * 64),
                                   (100, 1000, 128 * 40), (128, 4100, 1024), (37, 640, 128)])
def test_stream_k_shared_tiles(M, N, K, monkeypatch):
    """Split-K decode instances: tiles shared by up to ~200 workgroups (one 64-column tile
    over 200 K blocks), ragged N, a single row, every stream instance that fits the rows;
    the workspace's arrival counters must be zero again after every call, and two calls
    give identical bits."""
    from moe_grouped_gemm_lhs_amd import binding as b
    p = I.make_dense(M, N, K, seed=M + N + K // 128)
    A, sA, B, sB = gu.device_operands(p)
    c_ref = gu.oracle_full(p)
    written = np.ones((M, N), bool)
    for name in STREAM_INSTANCES:
        if M > int(name.split("_")[1].split("x")[0]):
            continue
        monkeypatch.setenv("DG_FORCE_INSTANCE", name)
        assert b.dg_instance_name(0, M, N, K, 1) == name
        need = b.dg_workspace_bytes(0, M, N, K, 1)
        ws = torch.zeros(need, dtype=torch.uint8, device=gu.DEV)
        first = None
        for rep in range(2):     # the second call reuses the workspace the first left
            gu.say(f"[case] stream {name} {M}x{N}x{K} call {rep}")
            c_gpu = gu.run_gpu(p, ops=(A, sA, B, sB), workspace=ws)
            assert_within_tolerance(c_gpu, c_ref, written, f"{name} {M}x{N}x{K}")
            assert not ws.cpu().numpy().any(), f"{name}: workspace not left zero filled"
            if first is None:
                first = c_gpu
            assert np.array_equal(c_gpu, first), f"{name}: two calls differ"
    monkeypatch.delenv("DG_FORCE_INSTANCE")


@pytest.mark.parametrize("M,N,K", [(64, 64, 128 * 200), (128, 200, 16384), (100, 1000, 128 * 40)])
def test_stream_k_owners_give_up(M, N, K, monkeypatch):
    """The hand-over of a shared tile's parts: with the owners' poll bound forced to 0 or 1
    (DG_HELPER_POLLS, set from the host) owners give up at once and the last contributor
    to arrive reduces what is left.  Every part is summed in the same order whoever
    reduces it, so the output is bit-identical to the default run; the workspace is left
    zero filled."""
    from moe_grouped_gemm_lhs_amd import binding as b
    p = I.make_dense(M, N, K, seed=M + N + K // 128 + 1)
    A, sA, B, sB = gu.device_operands(p)
    c_ref = gu.oracle_full(p)
    written = np.ones((M, N), bool)
    for name in ["dense_64x128_stream", "dense_128x128_stream_4w", "dense_128x64_stream"]:
        if M > int(name.split("_")[1].split("x")[0]):
            continue
        monkeypatch.setenv("DG_FORCE_INSTANCE", name)
        ws = torch.zeros(b.dg_workspace_bytes(0, M, N, K, 1), dtype=torch.uint8, device=gu.DEV)
        monkeypatch.delenv("DG_HELPER_POLLS", raising=False)
        gu.say(f"[case] stream {name} {M}x{N}x{K} default poll bound")
        base = gu.run_gpu(p, ops=(A, sA, B, sB), workspace=ws)
        assert_within_tolerance(base, c_ref, written, f"{name} {M}x{N}x{K}")
        for polls in ("0", "1"):
            monkeypatch.setenv("DG_HELPER_POLLS", polls)
            gu.say(f"[case] stream {name} {M}x{N}x{K} poll bound {polls}")
            c_gpu = gu.run_gpu(p, ops=(A, sA, B, sB), workspace=ws)
            diff = np.argwhere(c_gpu != base)
            if diff.size:
                gu.say(f"[diag] {len(diff)} elements differ, first {diff[:4].tolist()}: "
                       f"{c_gpu[tuple(diff[0])]:#06x} vs {base[tuple(diff[0])]:#06x}; "
                       f"workspace zero: {not ws.cpu().numpy().any()}")
            assert_within_tolerance(c_gpu, c_ref, written, f"{name} poll bound {polls}")
            assert np.array_equal(c_gpu, base), f"{name}: poll bound {polls} changed the output"
            assert not ws.cpu().numpy().any(), f"{name}: workspace not left zero filled"
        monkeypatch.delenv("DG_HELPER_POLLS")
    monkeypatch.delenv("DG_FORCE_INSTANCE")


MASKED_STREAM_INSTANCES = ["masked_128x128_stream", "masked_128x64_stream"]


@pytest.mark.parametrize("G,cap,N,K,mm", [(2, 128, 130, 128 * 60, [128, 70]),
                                         (4, 512, 256, 2048, [512, 0, 300, 129])])
def test_masked_stream_k_owners_give_up(G, cap, N, K, mm, monkeypatch):
    """The masked split-K instances with the owners' poll bound forced to 0: every part of
    every shared tile falls to its last contributor; the output is bit-identical to the
    default run and the workspace is left zero filled."""
    from moe_grouped_gemm_lhs_amd import binding as b
    p = I.make_masked(G, cap, N, K, seed=G * 11 + cap, masked_m=mm)
    ops = gu.device_operands(p)
    for name in MASKED_STREAM_INSTANCES:
        monkeypatch.setenv("DG_FORCE_INSTANCE", name)
        ws = torch.zeros(b.dg_workspace_bytes(2, cap, N, K, G), dtype=torch.uint8, device=gu.DEV)
        monkeypatch.delenv("DG_HELPER_POLLS", raising=False)
        gu.say(f"[case] {name} G={G} cap={cap} default poll bound")
        base = gu.run_gpu(p, ops=ops, workspace=ws)
        monkeypatch.setenv("DG_HELPER_POLLS", "0")
        gu.say(f"[case] {name} G={G} cap={cap} poll bound 0")
        c_gpu = gu.run_gpu(p, ops=ops, workspace=ws)
        assert np.array_equal(c_gpu, base), f"{name}: poll bound 0 changed the output"
        assert not ws.cpu().numpy().any(), f"{name}: workspace not left zero filled"
        monkeypatch.delenv("DG_HELPER_POLLS")
    monkeypatch.delenv("DG_FORCE_INSTANCE")




@pytest.mark.parametrize("G,cap,N,K,mm", [
    (3, 200, 400, 384, [200, 37, 0]),                      # ragged rows, an empty group
    (6, 96, 300, 512, [0, 96, 1, 95, -5, 103]),            # counts outside [0, cap]
    (2, 128, 130, 128 * 60, [128, 70]),                    # tiles shared by many workgroups
    (64, 16, 256, 1024, None),                             # the 64-group limit
    (4, 512, 256, 2048, [512, 0, 300, 129]),               # several row tiles per group
])
def test_masked_stream_k(G, cap, N, K, mm, monkeypatch):
    """Split-K masked instances (the schedule is built on the device from masked_m): every
    written row within tolerance, every other row untouched, the workspace's arrival
    counters zero again after each of two calls; all-zero counts write nothing."""
    from moe_grouped_gemm_lhs_amd import binding as b
    if mm is None:
        mm = np.random.default_rng(G + cap).integers(0, cap + 1, size=G)
    p = I.make_masked(G, cap, N, K, seed=G * 7 + cap, masked_m=mm)
    ops = gu.device_operands(p)
    c_ref = gu.oracle_full(p)
    w = np.repeat(gu.written_rows(p)[:, None], N, axis=1)
    for name in MASKED_STREAM_INSTANCES:
        monkeypatch.setenv("DG_FORCE_INSTANCE", name)
        assert b.dg_instance_name(2, cap, N, K, G) == name
        ws = torch.zeros(b.dg_workspace_bytes(2, cap, N, K, G), dtype=torch.uint8,
                         device=gu.DEV)
        for rep in range(2):
            gu.say(f"[case] {name} G={G} cap={cap} N={N} K={K} call {rep}")
            mmv = torch.from_numpy(np.asarray(p.masked_m, np.int32)).to(gu.DEV)
            C = torch.from_numpy(np.full((G * cap, N), SENTINEL, np.uint16).view(np.int16)
                                 ).to(gu.DEV).view(torch.bfloat16)
            b.dg_grouped_gemm_fp8_masked(*ops[:4], mmv, C.view(G, cap, N), workspace=ws)
            torch.cuda.synchronize()
            c_gpu = C.view(torch.int16).cpu().numpy().view(np.uint16)
            assert_within_tolerance(c_gpu, c_ref, w, f"{name} masked G={G}")
            assert np.all(c_gpu[~w] == SENTINEL), f"{name}: rows past masked_m written"
            assert not ws.cpu().numpy().any(), f"{name}: workspace not left zero filled"
        gu.say(f"[case] {name} all-zero counts")
        z = torch.zeros(G, dtype=torch.int32, device=gu.DEV)
        C = torch.from_numpy(np.full((G * cap, N), SENTINEL, np.uint16).view(np.int16)
                             ).to(gu.DEV).view(torch.bfloat16)
        b.dg_grouped_gemm_fp8_masked(*ops[:4], z, C.view(G, cap, N), workspace=ws)
        torch.cuda.synchronize()
        assert np.all(C.view(torch.int16).cpu().numpy().view(np.uint16) == SENTINEL)
    monkeypatch.delenv("DG_FORCE_INSTANCE")


# ------------------------------------------------------- E5M2 operands (either or both)
FMT_PAIRS = [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")]


@pytest.mark.parametrize("a_fmt,b_fmt", FMT_PAIRS)
def test_formats_every_form(a_fmt, b_fmt):
    """E5M2 for either or both operands, in every form: a decode shape (stream-K), a
    ragged tiled dense shape, contiguous and masked grouped shapes."""
    fm = dict(a_fmt=a_fmt, b_fmt=b_fmt)
    cases = [I.make_dense(64, 600, 1024, seed=60, **fm),
             I.make_dense(300, 520, 640, seed=61, outliers=True, **fm),
             I.make_contiguous([256, 128, 384], 400, 384, seed=62, **fm),
             I.make_masked(3, 200, 400, 384, seed=63, masked_m=[200, 37, 0], **fm)]
    for p in cases:
        check_full(p, f"{p.kind} {p.rows}x{p.N}x{p.K} {a_fmt}x{b_fmt}")


@pytest.mark.parametrize("a_fmt,b_fmt", FMT_PAIRS)
def test_formats_every_instance(a_fmt, b_fmt, monkeypatch):
    """Each dense instance forced with E5M2 operands."""
    from moe_grouped_gemm_lhs_amd import binding as b
    for name in ["dense_256x256", "dense_256x224", "dense_256x160", "dense_128x128",
                 "dense_64x128_stream",
                 "dense_64x64_stream", "dense_128x128_stream", "dense_128x64_stream",
                 "dense_128x128_stream_4w", "dense_64x128_stream_4w"]:
        monkeypatch.setenv("DG_FORCE_INSTANCE", name)
        M = 333 if "stream" not in name else (50 if name.startswith("dense_64x") else 100)
        assert b.dg_instance_name(0, M, 400, 512, 1) == name
        p = I.make_dense(M, 400, 512, seed=64, a_fmt=a_fmt, b_fmt=b_fmt)
        check_full(p, f"dense forced {name} {a_fmt}x{b_fmt}")
    monkeypatch.delenv("DG_FORCE_INSTANCE")


@pytest.mark.parametrize("a_fmt,b_fmt", FMT_PAIRS)
def test_formats_every_grouped_instance(a_fmt, b_fmt, monkeypatch):
    """Each contiguous and masked instance forced with E5M2 operands (the split-K masked
    instances too, on groups of several 128-row tiles)."""
    from moe_grouped_gemm_lhs_amd import binding as b
    fm = dict(a_fmt=a_fmt, b_fmt=b_fmt)
    for name in ["contig_256x256", "contig_256x224", "contig_128x128"]:
        monkeypatch.setenv("DG_FORCE_INSTANCE", name)
        p = I.make_contiguous([256, 128, 384], 400, 384, seed=65, **fm)
        assert b.dg_instance_name(1, p.rows, p.N, p.K, p.G) == name
        check_full(p, f"contiguous forced {name} {a_fmt}x{b_fmt}")
    for name in ["masked_256x256", "masked_128x128", "masked_64x128", "masked_128x128_stream",
                 "masked_128x64_stream"]:
        monkeypatch.setenv("DG_FORCE_INSTANCE", name)
        p = I.make_masked(3, 200, 400, 384, seed=66, masked_m=[200, 37, 130], **fm)
        assert b.dg_instance_name(2, 200, 400, 384, 3) == name
        check_full(p, f"masked forced {name} {a_fmt}x{b_fmt}")
    monkeypatch.delenv("DG_FORCE_INSTANCE")


@pytest.mark.parametrize("a_fmt,b_fmt", FMT_PAIRS)
def test_formats_integer_inputs_bit_exact(a_fmt, b_fmt):
    rng = np.random.default_rng(41)
    M, N, K = 130, 300, 384
    a = np.zeros((M, K))
    for r in range(M):
        pos = rng.choice(K, 8, replace=False)
        a[r, pos] = rng.integers(-4, 5, 8)
    b = rng.integers(-4, 5, (N, K)).astype(np.float64)
    ref = (a.astype(np.int64) @ b.astype(np.int64).T).astype(np.float64)
    p = I.Problem("dense", M, N, K, 1, fp8_codes_of(a, a_fmt), np.ones((M, 3), np.float32),
                  fp8_codes_of(b, b_fmt), np.ones((3, 3), np.float32), a_fmt=a_fmt,
                  b_fmt=b_fmt)
    gu.say(f"[case] integer dense {a_fmt}x{b_fmt}")
    assert np.array_equal(bf16_to_f64(gu.run_gpu(p)), ref)


def test_formats_decode_shape_full():
    case = dict(I.decode_cases()[3], a_fmt="e5m2", b_fmt="e5m2")   # 64x7168x16384
    p = I.make(case)
    check_sampled(p, I.case_name(case))


def test_integer_inputs_bit_exact():
    rng = np.random.default_rng(40)
    M, N, K = 200, 300, 384
    a = np.zeros((M, K))
    for r in range(M):
        pos = rng.choice(K, 8, replace=False)
        a[r, pos] = rng.integers(-4, 5, 8)
    b = rng.integers(-4, 5, (N, K)).astype(np.float64)
    ref = (a.astype(np.int64) @ b.astype(np.int64).T).astype(np.float64)
    p = I.Problem("dense", M, N, K, 1, e4m3_codes_of(a), np.ones((M, 3), np.float32),
                  e4m3_codes_of(b), np.ones((3, 3), np.float32))
    gu.say("[case] integer dense")
    assert np.array_equal(bf16_to_f64(gu.run_gpu(p)), ref)
    # grouped: a wrong group gives a wrong integer
    G = 3
    bs = [rng.integers(-4, 5, (N, K)).astype(np.float64) for _ in range(G)]
    sizes = [128, 256, 128]
    ac = a[:512] if a.shape[0] >= 512 else np.concatenate([a, a, a])[:512]
    gi = I.group_sizes_to_idx(sizes)
    pc = I.Problem("contiguous", 512, N, K, G, e4m3_codes_of(ac), np.ones((512, 3), np.float32),
                   e4m3_codes_of(np.concatenate(bs)), np.ones((G * 3, 3), np.float32),
                   group_idx=gi)
    gu.say("[case] integer contiguous")
    got = bf16_to_f64(gu.run_gpu(pc))
    want = np.concatenate([ac[gi == g].astype(np.int64) @ bs[g].astype(np.int64).T
                           for g in range(G)]).astype(np.float64)
    assert np.array_equal(got, want)
    cap = 160
    mm = np.array([160, 3, 77], np.int32)
    am = np.concatenate([a, a, a])[:G * cap]
    pm = I.Problem("masked", cap, N, K, G, e4m3_codes_of(am), np.ones((G * cap, 3), np.float32),
                   e4m3_codes_of(np.concatenate(bs)), np.ones((G * 3, 3), np.float32),
                   masked_m=mm)
    gu.say("[case] integer masked")
    got = gu.run_gpu(pm)
    for g in range(G):
        blk = got[g * cap:(g + 1) * cap]
        want = am[g * cap:g * cap + mm[g]].astype(np.int64) @ bs[g].astype(np.int64).T
        assert np.array_equal(bf16_to_f64(blk[:mm[g]]), want.astype(np.float64))
        assert np.all(blk[mm[g]:] == SENTINEL)


def test_power_of_two_scaling_and_determinism():
    p = I.make_dense(256, 384, 768, seed=41)
    gu.say("[case] 2^k scaling")
    c0 = gu.run_gpu(p)
    c0b = gu.run_gpu(p)
    assert np.array_equal(c0, c0b), "two runs differ"
    sA = p.sA.copy(); sA[7] *= 8.0; sA[200] *= 0.5
    sB = p.sB.copy(); sB[1] *= 4.0
    q = I.Problem("dense", p.M, p.N, p.K, 1, p.A, sA, p.B, sB)
    c1 = bf16_to_f64(gu.run_gpu(q))
    f0 = bf16_to_f64(c0)
    f0[7] *= 8.0; f0[200] *= 0.5; f0[:, 128:256] *= 4.0
    assert np.array_equal(c1, f0)


def test_masked_edge_counts_nan_rows_and_sentinel():
    G, cap, N, K = 6, 96, 300, 512
    mm = np.array([0, cap, 1, cap - 1, -5, cap + 7], np.int32)
    p = I.make_masked(G, cap, N, K, seed=42, masked_m=mm)
    valid = np.clip(mm, 0, cap)
    A = p.A.copy()
    for g in range(G):
        A[g * cap + valid[g]:(g + 1) * cap] = 0x7F       # NaN bytes that must never be read
    p.A = A
    check_full(p, "masked edge counts")
    gu.say("[case] masked all-zero counts")
    z = gu.run_gpu(p, masked_m=np.zeros(G, np.int32))
    assert np.all(z == SENTINEL)


def test_masked_group_permutation_bit_exact():
    G, cap, N, K = 4, 128, 256, 384
    p = I.make_masked(G, cap, N, K, seed=43, masked_m=[128, 50, 0, 77])
    c = gu.run_gpu(p)
    perm = [2, 0, 3, 1]
    nnb = 2
    ra = np.concatenate([np.arange(g * cap, (g + 1) * cap) for g in perm])
    rb = np.concatenate([np.arange(g * N, (g + 1) * N) for g in perm])
    rs = np.concatenate([np.arange(g * nnb, (g + 1) * nnb) for g in perm])
    q = I.Problem("masked", cap, N, K, G, p.A[ra], p.sA[ra], p.B[rb], p.sB[rs],
                  masked_m=p.masked_m[perm])
    gu.say("[case] masked permutation")
    assert np.array_equal(gu.run_gpu(q), c[ra])


def test_contiguous_malformed_rows_and_permutation():
    sizes = [256, 128, 384, 128]
    p = I.make_contiguous(sizes, 300, 384, seed=44)
    gi = p.group_idx.copy()
    gi[250:256] = -1
    gi[300] = 0
    gi[130] = 9
    gi[640:768] = -1
    check_full(p, "contiguous malformed rows", group_idx=gi)
    c = gu.run_gpu(p)
    starts = np.cumsum([0] + sizes)
    order = [3, 1, 0, 2]
    rows = np.concatenate([np.arange(starts[g], starts[g + 1]) for g in order])
    q = I.Problem("contiguous", p.rows, p.N, p.K, p.G, p.A[rows], p.sA[rows], p.B, p.sB,
                  group_idx=p.group_idx[rows])
    gu.say("[case] contiguous permutation")
    assert np.array_equal(gu.run_gpu(q), c[rows])


def test_contiguous_single_group_matches_dense():
    p = I.make_contiguous([512], 384, 512, seed=45)
    d = I.Problem("dense", 512, 384, 512, 1, p.A, p.sA, p.B, p.sB)
    c1 = gu.run_gpu(p)
    c2 = gu.run_gpu(d)
    assert_within_tolerance(c1, c2, np.ones_like(c1, bool), "contiguous G=1 vs dense")


def test_empty_calls_are_noops():
    from moe_grouped_gemm_lhs_amd import binding as b
    A = torch.zeros((0, 128), dtype=torch.uint8, device=gu.DEV)
    sA = torch.zeros((0, 1), dtype=torch.float32, device=gu.DEV)
    B = torch.zeros((16, 128), dtype=torch.uint8, device=gu.DEV)
    sB = torch.ones((1, 1), dtype=torch.float32, device=gu.DEV)
    C = b.dg_gemm_fp8_nt(A, sA, B, sB)
    assert C.shape == (0, 16)


# ------------------------------------------------------------- the workload shapes
@pytest.mark.parametrize("case", I.decode_cases(), ids=I.case_name)
def test_decode_shapes_full(case):
    p = I.make(case)
    check_full(p, I.case_name(case))


@pytest.mark.parametrize("case", I.prefill_cases(), ids=I.case_name)
def test_prefill_shapes_sampled(case):
    p = I.make(case)
    check_sampled(p, I.case_name(case))


@pytest.mark.parametrize("case", I.contiguous_cases(), ids=I.case_name)
def test_contiguous_shapes_sampled(case):
    p = I.make(case)
    check_sampled(p, I.case_name(case))


@pytest.mark.parametrize("case", I.masked_cases(), ids=I.case_name)
def test_masked_shapes_sampled(case):
    p = I.make(case)
    check_sampled(p, I.case_name(case) + f" masked_m={p.masked_m.tolist()}")


def test_graph_capture_replays_with_new_counts():
    """The masked call (and a stream-K decode call that uses the workspace)
    captured once in a HIP graph and replayed with new masked_m values written between
    replays: every replay matches the oracle, rows past the counts stay untouched."""
    from moe_grouped_gemm_lhs_amd import binding as dg
    G, cap, N, K = 3, 128, 512, 1024
    p = I.make_masked(G, cap, N, K, seed=46, masked_m=[128, 40, 0])
    A, sA, B, sB = gu.device_operands(p)
    mm = torch.tensor([128, 40, 0], dtype=torch.int32, device=gu.DEV)
    C = torch.empty((G, cap, N), dtype=torch.bfloat16, device=gu.DEV)
    d = I.make_dense(64, 2112, 1024, seed=47)
    dA, dsA, dB, dsB = gu.device_operands(d)
    dC = torch.empty((64, 2112), dtype=torch.bfloat16, device=gu.DEV)
    ws = torch.zeros(dg.dg_workspace_bytes(0, 64, 2112, 1024, 1) + 16, dtype=torch.uint8,
                     device=gu.DEV)
    sentinel = int(np.uint16(SENTINEL).view(np.int16))
    gu.say("[case] graph capture")
    dg.dg_grouped_gemm_fp8_masked(A, sA, B, sB, mm, C)
    dg.dg_gemm_fp8_nt(dA, dsA, dB, dsB, dC, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        dg.dg_grouped_gemm_fp8_masked(A, sA, B, sB, mm, C)
        dg.dg_gemm_fp8_nt(dA, dsA, dB, dsB, dC, workspace=ws)
    torch.cuda.synchronize()
    ref_dense = gu.oracle_full(d)
    for counts in ([128, 40, 0], [5, 128, 77], [0, 0, 1], [128, 128, 128]):
        gu.say(f"[case] graph replay masked_m={counts}")
        mm.copy_(torch.tensor(counts, dtype=torch.int32))
        C.view(torch.int16).fill_(sentinel)
        dC.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = C.view(torch.int16).cpu().numpy().view(np.uint16).reshape(G * cap, N)
        ref = gu.oracle_full(p, masked_m=np.array(counts, np.int32))
        w = np.repeat(gu.written_rows(p, masked_m=np.array(counts))[:, None], N, axis=1)
        assert_within_tolerance(got, ref, w, f"graph replay {counts}")
        got_d = dC.view(torch.int16).cpu().numpy().view(np.uint16)
        assert_within_tolerance(got_d, ref_dense, np.ones_like(got_d, bool), "graph replay dense")


def test_graph_capture_contiguous_new_routing():
    """The contiguous call captured once in a HIP graph and replayed with new group
    indices written between replays (groups of other sizes and order, 256-row tiles that
    straddle two groups, a padding block of index -1, one group for every row): every
    replay matches the oracle and leaves the padding rows untouched."""
    from moe_grouped_gemm_lhs_amd import binding as dg
    G, M, N, K = 4, 1024, 384, 1024
    p = I.make_contiguous([256, 128, 384, 256], N, K, seed=48)
    A, sA, B, sB = gu.device_operands(p)
    gi = torch.from_numpy(p.group_idx.copy()).to(gu.DEV)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=gu.DEV)
    sentinel = int(np.uint16(SENTINEL).view(np.int16))
    gu.say("[case] graph capture contiguous")
    dg.dg_grouped_gemm_fp8_contiguous(A, sA, B, sB, gi, C)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        dg.dg_grouped_gemm_fp8_contiguous(A, sA, B, sB, gi, C)
    torch.cuda.synchronize()
    layouts = [I.group_sizes_to_idx([256, 128, 384, 256]),
               np.repeat(np.array([2, 0, 3, 1], np.int32), [128, 512, 128, 256]),
               np.repeat(np.array([1, -1, 0, 3], np.int32), [256, 128, 384, 256]),
               np.full(M, 3, np.int32)]
    for gl in layouts:
        gl = np.ascontiguousarray(gl, dtype=np.int32)
        gu.say(f"[case] graph replay contiguous, groups {np.unique(gl).tolist()}")
        gi.copy_(torch.from_numpy(gl))
        C.view(torch.int16).fill_(sentinel)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = C.view(torch.int16).cpu().numpy().view(np.uint16)
        ref = gu.oracle_full(p, group_idx=gl)
        w = np.repeat(gu.written_rows(p, group_idx=gl)[:, None], N, axis=1)
        assert_within_tolerance(got, ref, w, f"graph replay contiguous {np.unique(gl)}")


def test_auto_workspace_on_side_streams():
    """Split-K decode calls without a workspace argument, launched on two side streams
    (neither the current stream) back to back and concurrently: each stream gets its own
    workspace, zero filled on that stream before the call; every result matches the
    oracle."""
    from moe_grouped_gemm_lhs_amd import binding as dg
    probs = [I.make_dense(64, 2112, 2048, seed=48), I.make_dense(128, 4096, 1024, seed=49)]
    assert all("stream" in dg.dg_instance_name(0, p.M, p.N, p.K, 1) for p in probs)
    refs = [gu.oracle_full(p) for p in probs]
    ops = [gu.device_operands(p) for p in probs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        gu.say(f"[case] auto workspace on side streams, round {rep}")
        outs = []
        for p, o, s in zip(probs, ops, streams):
            s.wait_stream(torch.cuda.current_stream())
            C = torch.empty((p.M, p.N), dtype=torch.bfloat16, device=gu.DEV)
            with torch.cuda.stream(s):
                C.zero_()
            dg.dg_gemm_fp8_nt(*o, C, stream=s)
            dg.dg_gemm_fp8_nt(*o, C, stream=s)      # the second call reuses the workspace
            outs.append(C)
        torch.cuda.synchronize()
        for p, C, ref in zip(probs, outs, refs):
            got = C.view(torch.int16).cpu().numpy().view(np.uint16)
            assert_within_tolerance(got, ref, np.ones_like(got, bool), f"side stream {p.M}")


# --------------------------------------------- routing at workload size, every row exact
_SMALL_INTS = np.arange(-4, 5)


def _one_hot_problem(case):
    """The case's routing (group sizes or masked_m) and shapes with integer-valued inputs:
    A entries uniform on {-4..4}, unit scales, and for group g a one-hot B_g whose row n
    has its 1 at column p_g(n) = (7n + 131g + 1) mod K.  Then C[m, n] = A[m, p_g(n)]
    exactly, for the group g that row m belongs to; p_g(n) differs between groups for
    every n, so a row computed with another group's B gets other integers."""
    N, K = case["N"], case["K"]
    if case["kind"] == "contiguous":
        G, rows = len(case["sizes"]), sum(case["sizes"])
    else:
        G, rows = case["G"], case["G"] * case["cap"]
    rng = np.random.default_rng(case["seed"] + 500)
    a_codes = e4m3_codes_of(_SMALL_INTS.astype(np.float64))
    A = a_codes[rng.integers(0, 9, size=(rows, K), dtype=np.uint8)]
    cols = np.stack([(7 * np.arange(N) + 131 * g + 1) % K for g in range(G)])
    B = np.zeros((G * N, K), np.uint8)
    B[np.arange(G * N), cols.reshape(-1)] = e4m3_codes_of(np.ones(1))[0]
    nkb, nnb = K // 128, -(-N // 128)
    sA = np.ones((rows, nkb), np.float32)
    sB = np.ones((G * nnb, nkb), np.float32)
    if case["kind"] == "contiguous":
        p = I.Problem("contiguous", rows, N, K, G, A, sA, B, sB,
                      group_idx=I.group_sizes_to_idx(case["sizes"]), sizes=case["sizes"])
    else:
        p = I.Problem("masked", case["cap"], N, K, G, A, sA, B, sB,
                      masked_m=I.masked_counts(G, case["cap"], case["seed"]))
    return p, cols


@pytest.mark.parametrize("case", I.contiguous_cases() + I.masked_cases(), ids=I.case_name)
def test_routing_full_size_every_row(case):
    """Grouped routing at the workload's full size: every written row bit-exact against
    its integer product, every other row untouched."""
    p, cols = _one_hot_problem(case)
    gu.say(f"[case] one-hot routing {I.case_name(case)} rows={p.rows}")
    got = gu.run_gpu(p)
    w = gu.written_rows(p)
    assert np.all(got[~w] == SENTINEL), "rows outside the routing were written"
    # code -> bf16 bits of the decoded integer (exact)
    lut = np.zeros(256, np.uint16)
    codes = e4m3_codes_of(_SMALL_INTS.astype(np.float64))
    lut[codes] = torch.tensor(_SMALL_INTS, dtype=torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if p.kind == "contiguous":
        grp = p.group_idx
    else:
        grp = np.repeat(np.arange(p.G), p.M)
    rows = np.nonzero(w)[0]
    for r0 in range(0, rows.size, 4096):
        r = rows[r0:r0 + 4096]
        want = lut[p.A[r[:, None], cols[grp[r]]]]
        bad = np.argwhere(got[r] != want)
        assert bad.size == 0, f"{bad.shape[0]} elements differ, first at row {r[bad[0][0]]}"


@pytest.mark.parametrize("sizes,N,K,full,what", [
    # every third 128-row block starts a new group: a third of the 256-row tiles straddle
    # two groups; their second passes are appended to the work list
    ([384] * 40, 512, 256, True, "appended second passes"),
    # 128-row groups: every tile straddles, more second passes than four per workgroup of a
    # full-chip grid, so each runs right after its first pass (checked on the first and last
    # row of every group, and on random rows)
    ([128] * 128, 4352, 128, False, "second passes in place"),
])
def test_contiguous_straddling_tiles(sizes, N, K, full, what, monkeypatch):
    """256-row contiguous tiles that hold two groups run once per group; both ways of
    scheduling the second passes write every row of both groups, and nothing else."""
    monkeypatch.setenv("DG_FORCE_INSTANCE", "contig_256x256")
    p = I.make_contiguous(sizes, N, K, seed=len(sizes) + N)
    label = f"contiguous {what} ({len(sizes)} groups, N={N})"
    if full:
        check_full(p, label)
    else:
        check_sampled(p, label, seed=len(sizes))
    monkeypatch.delenv("DG_FORCE_INSTANCE")
