"""Pins of the oracle's offline similarity matrix (HyLRA technical summary
2.2: M from the overlap ratio of logged top-k index sets), against a
hand-derived example and closed forms."""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "overlap_worked.json")


def test_overlap_golden():
    g = json.load(open(GOLDEN))
    M = oracle.overlap_matrix(np.array(g["idx_log"], dtype=np.int32))
    assert M.dtype == np.float32
    np.testing.assert_array_equal(M, np.array(g["M"], dtype=np.float32))


def windows(L, S, k, shift, pad=0):
    """Layer l selects the window [l*shift, l*shift + k - pad) in every slice."""
    idx = np.full((1, L, S, k), -1, np.int32)
    for l in range(L):
        idx[0, l, :, :k - pad] = l * shift + np.arange(k - pad)
    return idx


def test_overlap_sliding_windows_closed_form():
    # windows of k ids shifted by d per layer overlap in max(0, k - (j - i) d) ids
    for k, d in [(8, 1), (16, 3), (5, 5), (32, 7)]:
        L = 9
        M = oracle.overlap_matrix(windows(L, 3, k, d))
        for j in range(L):
            for i in range(L):
                want = max(0, k - (j - i) * d) / k if i <= j else 0.0
                assert M[j, i] == np.float32(want), (k, d, j, i)


def test_overlap_padding_and_empty_slices():
    # 4 valid ids of 6 slots; slice 1 of the last layer empty (skipped)
    idx = windows(4, 2, 6, 1, pad=2)
    idx[0, 3, 1, :] = -1
    M = oracle.overlap_matrix(idx)
    assert M[1, 0] == np.float32(3 / 4) and M[2, 0] == np.float32(2 / 4)
    assert M[3, 0] == np.float32(1 / 4)   # only slice 0 counts for target layer 3
    assert M[3, 3] == np.float32(1.0)
    none = np.full((1, 3, 2, 4), -1, np.int32)
    np.testing.assert_array_equal(oracle.overlap_matrix(none), np.zeros((3, 3), np.float32))


def test_overlap_ratio_is_over_the_target_set():
    # reading of the overlap ratio: shared ids over the target layer's set.
    # Layer 0 selects {3, 8}, layer 1 {1, 3, 5, 8}, layer 2 {3, 8} (-1 padded);
    # over the source's set instead, M[1][0] would be 1 and M[2][1] 1/2.
    idx = np.array([[[[3, 8, -1, -1]], [[1, 3, 5, 8]], [[3, 8, -1, -1]]]], np.int32)
    M = oracle.overlap_matrix(idx)
    assert M[1, 0] == np.float32(2 / 4)
    assert M[2, 1] == np.float32(2 / 2)
    assert M[2, 0] == np.float32(1.0)


def test_overlap_identical_and_disjoint_layers():
    rng = np.random.default_rng(3)
    base = np.sort(rng.choice(100, size=(2, 1, 5, 10), replace=False, axis=-1), axis=-1)
    same = np.repeat(base, 6, axis=1).astype(np.int32)
    M = oracle.overlap_matrix(same)
    np.testing.assert_array_equal(M, np.tril(np.ones((6, 6), np.float32)))
    disjoint = windows(5, 2, 10, 10)
    np.testing.assert_array_equal(oracle.overlap_matrix(disjoint), np.eye(5, dtype=np.float32))


def test_overlap_averages_steps():
    # step 0: windows shifted by 1, step 1: shifted by 2 -> mean of both ratios
    k, L = 10, 4
    idx = np.concatenate([windows(L, 1, k, 1), windows(L, 1, k, 2)], axis=0)
    M = oracle.overlap_matrix(idx)
    for j in range(L):
        for i in range(j + 1):
            r1, r2 = max(0, k - (j - i)) / k, max(0, k - 2 * (j - i)) / k
            assert M[j, i] == np.float32((r1 + r2) / 2)
