"""CPU tests of the index-match rule used by every GPU parity test
(tests/gpu_util.check_indices): rows whose oracle K-boundary gap is below
1e-6 may hold another top-K, but only a valid one. A wrong selection in such
a row, a non-candidate, a duplicate, an unsorted row or a difference in a row
with a clear gap must each fail; a valid alternative must pass and yield the
oracle's log gates for that set."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests.gpu_util import check_indices


def _ora(rows, K):
    """Oracle selection (top-K, gate, gap) of each score vector in rows."""
    out = dict(idx=np.full((1, 1, len(rows), K), -1, np.int32), logg=np.zeros((1, 1, len(rows), K)),
               gap=np.zeros((1, 1, len(rows))), k_eff=np.zeros((1, 1, len(rows)), np.int32))
    for r, s in enumerate(rows):
        idx, logg, ke, gap, _ = oracle.select_from_scores(s[np.isfinite(s)] if np.isinf(s).any() else s, K)
        out["idx"][0, 0, r], out["logg"][0, 0, r] = idx, logg
        out["gap"][0, 0, r], out["k_eff"][0, 0, r] = gap, ke
    return out


# row 0: cells 1, 2 and 4 tie for two places (gap 0); row 1: a clear gap
ROWS = [np.array([1.0, 2.0, 2.0, 0.5, 2.0]), np.array([0.1, 3.0, 2.0, 0.5, 1.0])]


def _fn(rows):
    return lambda pos: rows[pos[2]]


def _gpu(*rows):
    return np.array(rows, np.int32).reshape(1, 1, len(rows), -1)


def test_oracle_tie_rule_and_gap():
    ora = _ora(ROWS, 2)
    assert ora["idx"][0, 0, 0].tolist() == [1, 2] and ora["gap"][0, 0, 0] == 0.0
    assert ora["idx"][0, 0, 1].tolist() == [1, 2] and ora["gap"][0, 0, 1] == pytest.approx(1.0)


def test_identical_selection_passes():
    ora = _ora(ROWS, 2)
    chk = check_indices(_gpu([1, 2], [1, 2]), ora, _fn(ROWS))
    assert chk.n_exempt == 1 and chk.alt == []
    assert np.array_equal(chk.idx, ora["idx"]) and np.array_equal(chk.logg, ora["logg"])


def test_valid_alternative_in_an_exempt_row_passes_with_its_gates():
    ora = _ora(ROWS, 2)
    chk = check_indices(_gpu([1, 4], [1, 2]), ora, _fn(ROWS))
    assert chk.alt == [(0, 0, 0)]
    assert chk.idx[0, 0, 0].tolist() == [1, 4]
    s = ROWS[0]
    lse = np.log(np.exp(s).sum())
    assert np.allclose(chk.logg[0, 0, 0], [s[1] - lse, s[4] - lse], rtol=0, atol=1e-15)
    # the alternative's gates are the oracle's gates of the same set
    assert np.allclose(chk.logg[0, 0, 0], ora["logg"][0, 0, 0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("row0,what", [
    ([1, 3], "keeps"),                 # a cell 1.5 below the K-th score
    ([0, 1], "keeps"),
    ([2, 1], "ascending"),             # order
    ([2, 2], "ascending"),             # duplicate
    ([1, -1], "pads"),                 # K_eff = 2 but one entry
    ([1, 5], "non-candidate"),         # past the candidates
])
def test_wrong_selection_in_an_exempt_row_fails(row0, what):
    ora = _ora(ROWS, 2)
    with pytest.raises(AssertionError, match=what):
        check_indices(_gpu(row0, [1, 2]), ora, _fn(ROWS))


def test_difference_in_a_row_with_a_clear_gap_fails():
    ora = _ora(ROWS, 2)
    with pytest.raises(AssertionError, match="select different blocks"):
        check_indices(_gpu([1, 2], [1, 4]), ora, _fn(ROWS))


def test_non_candidate_marked_minus_inf_fails():
    # cell 4 ties with the winners but is not a candidate of the row (a
    # subset selection lists only kept cells)
    s = np.array([1.0, 2.0, 2.0, 0.5, 2.0])
    masked = s.copy()
    masked[4] = -np.inf
    ora = _ora([s[:4]], 2)
    ora["gap"][:] = 0.0
    with pytest.raises(AssertionError, match="non-candidate"):
        check_indices(_gpu([1, 4]), ora, lambda pos: masked)


def test_within_the_band_passes_and_below_fails():
    # the oracle's K-th (cell 2) leads cell 3 by 4e-7: an exempt row, and
    # cell 3 in its place is a valid top-K
    s_ok = np.array([0.0, 2.0, 1.0, 1.0 - 4e-7])
    ora = _ora([s_ok], 2)
    assert ora["idx"][0, 0, 0].tolist() == [1, 2] and ora["gap"][0, 0, 0] < 1e-6
    chk = check_indices(_gpu([1, 3]), ora, lambda pos: s_ok)
    assert chk.n_exempt == 1 and chk.alt == [(0, 0, 0)]
    # 3e-6 below the K-th is outside the band even if the row were exempt
    s_bad = np.array([0.0, 2.0, 1.0, 1.0 - 3e-6])
    ora = _ora([s_bad], 2)
    ora["gap"][:] = 0.0
    with pytest.raises(AssertionError, match="keeps"):
        check_indices(_gpu([1, 3]), ora, lambda pos: s_bad)
