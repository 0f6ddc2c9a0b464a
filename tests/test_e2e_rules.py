"""The comparison rule of the end-to-end GPU tests (CPU only): a greedy pick other than
the oracle's argmax passes only when its oracle logit is within near_tie() of the largest
(twice the average per-element deviation the relative-L2 bar of 1e-3 allows)."""
import numpy as np

from e2e import REL_L2, compare, failures, near_tie


def test_near_tie_threshold_and_greedy_rule():
    ref = np.zeros(1000, np.float32)
    ref[::2] = 3.0
    ref[1::2] = -3.0                                  # rms 3: near_tie = 2 * 1e-3 * 3
    assert np.isclose(near_tie(ref), 2 * REL_L2 * 3.0)
    ref[10] = 5.0
    ref[20] = 5.0 - 0.5 * near_tie(ref)               # within the near-tie band
    ref[30] = 5.0 - 2.0 * near_tie(ref)               # outside it
    got = ref.copy()
    assert compare(0, 0, got, ref).argmax_ok
    got[20] = 5.001
    s = compare(0, 0, got, ref)
    assert s.argmax_ok and not failures([s])
    got = ref.copy()
    got[30] = 5.001
    s = compare(0, 0, got, ref)
    assert not s.argmax_ok and failures([s]) and not failures([s], greedy=False)
