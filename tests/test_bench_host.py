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
