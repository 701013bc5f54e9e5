"""The near-tie acceptance rule for GPU top-k rows (oracle/acceptance.py):
rows may differ from the oracle's only on a near tie, and then only by blocks
inside the 1e-5 tie window at the cut, with a well-formed row.  Wrong sets are
planted here on the CPU and must be rejected."""
import numpy as np
import pytest

import oracle
from oracle.acceptance import check_topk_rows

K = 3


def _scores():
    """Two sequences (1024 and 200 tokens: 8 and 2 blocks), two KV heads.
    Head 0 of sequence 0 has a near tie at the cut: the 3rd and 4th largest
    scores differ by 2e-6 relative; head 1 has a clear cut."""
    s = np.zeros((2, 2, 8))
    s[0, 0] = [0.9, 0.1, 0.5, 0.5 * (1 - 3e-6), 0.2, 0.05, 0.01, 0.5 * (1 - 5e-6)]
    s[0, 1] = [0.1, 0.8, 0.05, 0.6, 0.3, 0.02, 0.01, 0.2]
    s[1, 0, :2] = [0.4, 0.6]
    s[1, 1, :2] = [0.7, 0.3]
    ctx = np.array([1024, 200], np.int32)
    want, margin = oracle.topk(s, ctx, K)
    return s, ctx, want, margin


def test_oracle_rows_and_margins():
    s, ctx, want, margin = _scores()
    assert want[0, 0].tolist() == [0, 2, 3]
    assert margin[0, 0] < 1e-5 <= margin[0, 1]
    assert want[1, 0].tolist() == [0, 1, -1] and np.isinf(margin[1, 0])


def test_identical_rows_pass():
    s, ctx, want, margin = _scores()
    assert check_topk_rows(want.copy(), want, s, margin, ctx, K) == 0


@pytest.mark.parametrize("row", [[0, 2, 7], [0, 3, 7]])
def test_swap_inside_tie_window_is_excused(row):
    s, ctx, want, margin = _scores()
    got = want.copy()
    got[0, 0] = row
    assert check_topk_rows(got, want, s, margin, ctx, K) == 1


@pytest.mark.parametrize("b,g,row,msg", [
    (0, 0, [0, 2, 4], "outside the tie window"),   # block 4 scores 0.2, far below the cut
    (0, 0, [1, 2, 3], "outside the tie window"),   # dropped the top block
    (0, 0, [0, 7, 2], "not strictly ascending"),
    (0, 0, [0, 2, 2], "not strictly ascending"),
    (0, 0, [2, 7, -1], "outside"),                 # padding inside the first k_eff slots
    (0, 0, [0, 2, 8], "outside"),                  # id past the context
    (0, 1, [1, 3, 7], "away from a near tie"),     # clear cut: no excuse at all
    (1, 0, [1, 0, -1], "away from a near tie"),    # k >= N: the set is every block
])
def test_planted_wrong_sets_are_rejected(b, g, row, msg):
    s, ctx, want, margin = _scores()
    got = want.copy()
    got[b, g] = row
    with pytest.raises(AssertionError, match=msg):
        check_topk_rows(got, want, s, margin, ctx, K)
