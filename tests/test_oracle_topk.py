"""Pins of the top-k selection oracle (oracle/topk.py): brute force with
Python's own ordering, the library selection on distinct scores, ties, the
total order of signed zeros and infinities, NaN, short rows and padding."""
import numpy as np
import pytest

import oracle


def _brute(row, k, n=None):
    n = len(row) if n is None else n
    vals = [(float(row[p]), p) for p in range(n)]
    # Python float order, NaN lowest; -0.0 below +0.0
    def rank(v):
        x, p = v
        if np.isnan(x):
            return (0, 0.0, 0, -p)
        return (1, x, 1 if np.copysign(1.0, x) > 0 else 0, -p)
    top = sorted(vals, key=rank, reverse=True)[:min(k, n)]
    sel = sorted(p for _, p in top)
    return sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("seed", range(5))
def test_bruteforce_with_ties(seed):
    rng = np.random.default_rng(seed)
    s = rng.integers(-3, 4, size=(4, 40)).astype(np.float32)  # many ties
    s[0, 5] = -0.0
    s[0, 6] = 0.0
    got = oracle.select_topk(s, 11)
    for r in range(4):
        assert got[r].tolist() == _brute(s[r], 11)


def test_distinct_scores_match_argpartition():
    rng = np.random.default_rng(10)
    s = rng.standard_normal((3, 5000)).astype(np.float32)
    got = oracle.select_topk(s, 300)
    for r in range(3):
        ref = np.sort(np.argpartition(-s[r].astype(np.float64), 300)[:300])
        assert np.array_equal(got[r], ref)


def test_all_equal_takes_the_first_positions():
    got = oracle.select_topk(np.full((2, 50), 1.5, np.float32), 7)
    assert got.tolist() == [list(range(7))] * 2


def test_special_values():
    s = np.array([[np.nan, -np.inf, 0.0, -0.0, np.inf, 1.0, np.nan]], np.float32)
    assert oracle.select_topk(s, 3).tolist() == [[2, 4, 5]]          # inf, 1, +0
    assert oracle.select_topk(s, 5).tolist() == [[1, 2, 3, 4, 5]]    # ... then -0, -inf
    assert oracle.select_topk(s, 7).tolist() == [[0, 1, 2, 3, 4, 5, 6]]


def test_short_rows_and_padding():
    s = np.arange(20, dtype=np.float32)[None].repeat(3, axis=0)
    got = oracle.select_topk(s, 8, row_lens=np.array([20, 5, 0]))
    assert got[0].tolist() == list(range(12, 20))
    assert got[1].tolist() == [0, 1, 2, 3, 4, -1, -1, -1]
    assert got[2].tolist() == [-1] * 8


def test_permutation_moves_the_selection():
    rng = np.random.default_rng(11)
    s = rng.standard_normal((1, 200)).astype(np.float32)
    perm = rng.permutation(200)
    a = set(oracle.select_topk(s, 17)[0].tolist())
    b = set(oracle.select_topk(s[:, perm], 17)[0].tolist())
    assert {int(perm[p]) for p in b} == a
