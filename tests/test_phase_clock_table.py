"""The phase-clock tool's arithmetic on synthetic clock arrays (CPU): each
interval is the difference of its two marks, an item is the distance to the
next item's top mark, and items a later launch overwrote are left out."""
import numpy as np

from linear_attention_prefill_amd import phase_clocks as P


def _intra_item(t0, widths):
    """Marks 0..10 of one intra-chunk item starting at t0 with the given
    interval widths (10 intervals)."""
    m = np.zeros(16, dtype=np.int64)
    m[0] = t0
    for i, w in enumerate(widths):
        m[i + 1] = m[i] + w
    return m


def test_intervals_and_item_lengths():
    clk = np.zeros((8, 64, 16), dtype=np.int64)
    widths = [400, 30, 350, 20, 100, 60, 150, 40, 250, 10]
    for w in range(8):
        for i in range(5):
            clk[w, i] = _intra_item(10_000 + 2_000 * i + w, widths)
    lines = P.table(clk, fused=False)
    assert len(lines) == 1 + 8
    for w in range(8):
        f = lines[1 + w].split()
        assert int(f[0]) == w and int(f[1]) == 4          # the fifth item has no next top mark
        assert float(f[2]) == 2000.0
        assert [float(x) for x in f[3:]] == [float(x) for x in widths]


def test_items_left_from_an_earlier_launch_are_skipped():
    """A later launch rewrote items 0..2; items 3 and 4 are left from an
    earlier one (item 3's top mark is earlier than item 2's), so item 2,
    whose successor is not its launch's, gives no row."""
    clk = np.zeros((8, 64, 16), dtype=np.int64)
    widths = [100] * 10
    for i in range(3):
        clk[0, i] = _intra_item(50_000 + 3_000 * i, widths)
    clk[0, 3] = _intra_item(1_000, widths)
    clk[0, 4] = _intra_item(4_000, widths)
    lines = P.table(clk, fused=False)
    f = lines[1].split()
    assert int(f[1]) == 3                                 # items 0, 1 and 3
    assert float(f[2]) == (3000 + 3000 + 3000) / 3


def test_scan_intervals():
    clk = np.zeros((8, 64, 16), dtype=np.int64)
    for w in range(4):
        for i in range(10):
            t = 100_000 + 5_000 * i
            clk[w, i, :5] = [t, t + 900, t + 1700, t + 2700, t + 4600]
    lines = P.table(clk, fused=False, intervals=P.SCAN_INTERVALS)
    assert len(lines) == 1 + 4
    f = lines[1].split()
    assert int(f[1]) == 9 and float(f[2]) == 5000.0
    assert [float(x) for x in f[3:]] == [900.0, 800.0, 1000.0, 1900.0]
