"""The plain statement of the log-decay contract (tests/gdr_testlib.py,
gate_check_bits) that the GPU gate-status test compares the kernels' bits
with, checked on hand-made cases: 16-token windows spanning 15 steps of a
constant decay (15 * 12 = 180 > 160 is out, 15 * 10 = 150 is in), a single
positive decay, a NaN, and a ragged chunk."""
import numpy as np

from tests import gdr_testlib as tl


def test_constant_decays_across_the_window_limit():
    g = np.full((1, 128, 2, 8), -12.0)
    assert tl.gate_check_bits(g) == tl.GATE_RANGE
    g[:] = -10.0
    assert tl.gate_check_bits(g) == 0
    # a scalar gate has no window contract
    assert tl.gate_check_bits(np.full((1, 128, 2), -50.0)) == 0


def test_single_positive_nan_and_strong_entries():
    g = np.full((1, 100, 1, 4), -1.0)
    g[0, 70, 0, 3] = 0.5
    assert tl.gate_check_bits(g) == tl.GATE_POSITIVE
    g[0, 10, 0, 1] = np.nan
    assert tl.gate_check_bits(g) == tl.GATE_POSITIVE | tl.GATE_NONFINITE
    h = np.full((1, 100, 1, 4), -1.0)
    # token 81 is row 17 of the ragged chunk 1, the second row of its window
    # 16..31: the window spans that step plus 14 more of -1
    h[0, 81, 0, 2] = -170.0
    assert tl.gate_check_bits(h) == tl.GATE_RANGE
    h[0, 81, 0, 2] = -140.0
    assert tl.gate_check_bits(h) == 0
    # at the window's first row the step is inside every row's value: no range
    h2 = np.full((1, 100, 1, 4), -1.0)
    h2[0, 80, 0, 2] = -170.0
    assert tl.gate_check_bits(h2) == 0


def test_window_boundaries_follow_the_chunk():
    # a large step at token 64 (first row of chunk 1) spans no window of
    # chunk 0, and inside chunk 1 it is the window's first row (range 0 from it)
    g = np.full((1, 128, 1, 2), -1.0)
    g[0, 64, 0, 0] = -200.0
    assert tl.gate_check_bits(g) == 0
    g[0, 65, 0, 0] = -200.0   # second row of a window: the window spans 200 + 14
    assert tl.gate_check_bits(g) == tl.GATE_RANGE
