"""Host-side logic of bench.py (no GPU): the number of operand sets the dominant call's
timing rotates over, so that no launch can find its inputs left in the 256 MB Infinity
Cache by an earlier one."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(spec)
spec.loader.exec_module(bench)


def test_rotation_copies_cover_twice_the_cache():
    mall = bench.MALL_BYTES
    for nbytes in (1, 4096, 1 << 20, 121_466_880, 235_000_000, mall, 2 * mall, 3 * mall):
        r = bench.rotation_copies(nbytes)
        assert 1 <= r <= 16
        # between two uses of one set, the other r - 1 sets are read
        assert (r - 1) * nbytes >= 2 * mall or r == 16, (nbytes, r)
        # and no more sets than that needs
        assert r == 16 or r == 2 or (r - 2) * nbytes < 2 * mall, (nbytes, r)


def test_rotation_copies_examples():
    assert bench.rotation_copies(121_466_880) == 6     # decode 128x7168x16384
    assert bench.rotation_copies(750_000_000) == 2     # a call larger than the cache
    assert bench.rotation_copies(300_000) == 16        # tiny calls: capped


def test_pages_gbs_convention_reproduces_the_tables():
    """The pages' GB/s column (FP8 A and B plus BF16 C, scales ignored, every capacity row
    counted) from the bytes convention and their TFLOPS: three rows, one per table."""
    class P:
        pass

    def gbs(p, rows, tflops):
        return bench.pages_bytes_of(p) / (2 * rows * p.N * p.K / (tflops * 1e12)) / 1e9

    d = P(); d.kind, d.M, d.N, d.K = "dense", 64, 2112, 7168
    assert abs(gbs(d, 64, 206) - 1688) < 3
    c = P(); c.kind, c.rows, c.G, c.N, c.K = "contiguous", 4 * 8192, 4, 4096, 7168
    assert abs(gbs(c, 4 * 8192, 1297) - 418) < 3
    m = P(); m.kind, m.G, m.M, m.N, m.K = "masked", 4, 256, 4096, 7168
    assert abs(gbs(m, 4 * 256, 932) - 2064) < 3


def test_traffic_summaries_match_the_kernel_sources():
    """Every dominant kernel the bench maps to a committed HBM traffic summary has one, it
    parses, and its source hash matches the kernel sources as they stand (bench.py reports
    `traffic` only then); the algorithmic bytes recorded with it are the bench's own."""
    for (inst, shape), rel in bench._TRAFFIC_FILES.items():
        path = os.path.join(ROOT, rel)
        assert os.path.exists(path), rel
        t = bench._profiled_traffic(inst, shape)
        assert t is not None and t > 0, f"{rel}: stale or unparsable"
        fields = dict(l.split(":", 1) for l in open(path) if ":" in l)
        assert inst in fields["kernel"] and shape in fields["kernel"], rel
        assert int(fields["traffic_bytes_per_launch"].strip()) == t


def test_traffic_is_withheld_when_the_sources_change(tmp_path, monkeypatch):
    """A kernel source that no longer hashes to the recorded value switches `traffic` off."""
    (inst, shape), rel = next(iter(bench._TRAFFIC_FILES.items()))
    srcs = []
    for s in bench._KERNEL_SOURCES:
        dst = tmp_path / os.path.basename(s)
        dst.write_bytes(open(os.path.join(ROOT, s), "rb").read())
        srcs.append(str(dst))
    (tmp_path / "profiles").mkdir()
    (tmp_path / rel).write_text(open(os.path.join(ROOT, rel)).read())
    monkeypatch.setattr(bench, "_ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "_KERNEL_SOURCES", srcs)
    assert bench._profiled_traffic(inst, shape) is not None
    with open(srcs[0], "ab") as f:
        f.write(b"\n// changed\n")
    assert bench._profiled_traffic(inst, shape) is None
