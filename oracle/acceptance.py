"""Acceptance rule for top-k index sets -- TEST INFRASTRUCTURE ONLY.

Compares a GPU top-k row with the oracle's (``oracle.topk`` on the oracle's
float64 block scores).  The rule: indices match bit for bit, except on a
(sequence, KV head) row whose oracle cut margin (k-th vs (k+1)-th block
score, relative to the k-th) is below 1e-5.  Such a near-tie row is still
held to everything a correct answer must satisfy:

  * it holds k_eff = min(k, N_b) distinct block ids in ascending order, all in
    [0, N_b), followed by -1 padding up to k;
  * every block that is in one set and not in the other has an oracle score
    within 1e-5 (relative) of the oracle's k-th score -- i.e. the two sets
    differ only by blocks inside the tie window at the cut.

Only ``tests/`` and the smoke check use this module.
"""
from __future__ import annotations

import numpy as np

BLOCK = 128
MARGIN = 1e-5


def _row_blocks(ctx_b, max_blocks):
    T = min(max(int(ctx_b), 0), BLOCK * int(max_blocks))
    return (T + BLOCK - 1) // BLOCK


def check_topk_rows(got, want, score, margin, ctx, k, what="top-k"):
    """Checks GPU index rows ``got`` against the oracle's ``want`` (both
    [B][Hkv][k] int) under the near-tie rule above; ``score`` is the oracle's
    [B][Hkv][max_blocks] float64 score array and ``margin`` its [B][Hkv] cut
    margins.  Raises AssertionError naming the first failing row.  Returns
    the number of rows excused as near ties (their sets differ within the
    tie window)."""
    got = np.asarray(got)
    want = np.asarray(want)
    score = np.asarray(score, dtype=np.float64)
    margin = np.asarray(margin, dtype=np.float64)
    B, Hkv, kk = want.shape
    assert got.shape == want.shape == (B, Hkv, k), (got.shape, want.shape, k)
    max_blocks = score.shape[-1]
    excused = 0
    for b in range(B):
        N = _row_blocks(ctx[b], max_blocks)
        keff = min(k, N)
        for g in range(Hkv):
            gr, wr = got[b, g], want[b, g]
            if np.array_equal(gr, wr):
                continue
            where = "%s row (seq %d, KV head %d)" % (what, b, g)
            mg = margin[b, g]
            assert mg < MARGIN, "%s differs from the oracle away from a near tie " \
                                "(cut margin %.3g): got %s want %s" % (where, mg, gr, wr)
            sel = gr[:keff]
            assert np.all(gr[keff:] == -1), "%s: padding is not -1 after %d ids: %s" % (
                where, keff, gr)
            assert np.all((sel >= 0) & (sel < N)), "%s: ids outside [0, %d): %s" % (
                where, N, sel)
            assert np.all(np.diff(sel) > 0), "%s: ids not strictly ascending: %s" % (where, sel)
            s = score[b, g]
            kth = min(s[int(n)] for n in wr[:keff])
            for n in sorted(set(sel.tolist()) ^ set(wr[:keff].tolist())):
                assert abs(s[n] - kth) <= MARGIN * kth, (
                    "%s: block %d (oracle score %.17g) lies outside the tie window of the "
                    "k-th score %.17g" % (where, n, s[n], kth))
            excused += 1
    return excused

