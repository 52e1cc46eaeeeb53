"""The comparison rules of the parity tests, checked on hand-built cases
(CPU only): a selection the oracle would not make must fail, a selection that
differs only in candidates within 1e-5 (relative) of a cut must pass.  The
rule is the one every selection test uses (top-k rows, column lists, the
LoSA Active set and page unions)."""

import numpy as np
import pytest

from gpu_util import CUT_REL, check_topk_rows, check_topk_set, check_union_of_topk, near_cut_topk


def test_near_cut_sets():
    s = np.array([5.0, 3.0, 3.0 * (1 + 0.5 * CUT_REL), 1.0, -2.0])
    req, alw = near_cut_topk(s, 2)
    # top-2 by (score desc, index asc) is {0, 2}; 1 and 2 straddle the cut
    assert req.tolist() == [0] and alw.tolist() == [0, 1, 2]


def test_negative_cut_uses_its_magnitude():
    s = np.array([-1.0, -2.0, -2.0 * (1 + 0.5 * CUT_REL), -3.0])
    req, alw = near_cut_topk(s, 2)
    assert req.tolist() == [0] and alw.tolist() == [0, 1, 2]
    check_topk_set([0, 2], s, 2)      # the near-cut swap passes
    with pytest.raises(AssertionError):
        check_topk_set([0, 3], s, 2)  # a candidate far below the cut fails


def test_topk_set_rejects_wrong_count_and_far_candidates():
    s = np.arange(10, dtype=np.float64)
    check_topk_set([7, 8, 9], s, 3)
    for bad in ([6, 8, 9], [8, 9], [7, 8, 9, 9], [0, 8, 9]):
        with pytest.raises(AssertionError):
            check_topk_set(bad, s, 3)


def test_union_requires_every_row_pick_and_allows_only_row_picks():
    rows = np.array([[9.0, 1.0, 8.0, 0.0, 0.5, 0.2],
                     [0.0, 7.0, 1.0, 6.0, 0.3, 0.1]])
    # exact per-row top-2: {0, 2} and {1, 3}; union {0, 1, 2, 3}
    assert check_union_of_topk([0, 1, 2, 3], rows, 2) == 0
    with pytest.raises(AssertionError):
        check_union_of_topk([0, 1, 2], rows, 2)         # misses row 1's page 3
    with pytest.raises(AssertionError):
        check_union_of_topk([0, 1, 2, 3, 4], rows, 2)   # page 4 is no row's pick
    with pytest.raises(AssertionError):
        check_union_of_topk([0, 2, 1, 3], rows, 2)      # not ascending


def test_union_near_cut_page_may_go_either_way():
    tie = 8.0 * (1 - 0.5 * CUT_REL)
    rows = np.array([[9.0, 1.0, 8.0, tie, 0.5]])
    # page 3 scores within CUT_REL of the cut (page 2): either may be kept
    assert check_union_of_topk([0, 2], rows, 2) == 0
    assert check_union_of_topk([0, 3], rows, 2) == 2
    assert check_union_of_topk([0, 2, 3], rows, 2) == 1  # one row may take 2, another 3
    with pytest.raises(AssertionError):
        check_union_of_topk([0, 4], rows, 2)


def test_topk_rows_rule_matches_the_set_rule():
    rng = np.random.default_rng(5)
    A = rng.random((20, 16))
    sets = [np.sort(np.lexsort((np.arange(16), -a))[:4]) for a in A]
    assert check_topk_rows(sets, A, 4) == 0
    bad = [s.copy() for s in sets]
    order = np.lexsort((np.arange(16), -A[3]))
    bad[3] = np.sort(np.concatenate([order[:3], order[10:11]]))
    with pytest.raises(AssertionError):
        check_topk_rows(bad, A, 4)
