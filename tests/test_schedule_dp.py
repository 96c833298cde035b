"""Anchor selection: overlap metric on hand-made sets, dynamic program against
exhaustive search (host logic, no GPU)."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from long_context_amd import schedule as S  # noqa: E402


def test_overlap_by_hand():
    a = np.array([[0, 1, 2, 3], [5, 6, -1, -1]])
    l = np.array([[2, 3, 4, 5], [6, 7, 8, -1]])
    # unit 0: {2,3} of {2,3,4,5} -> 1/2; unit 1: {6} of {6,7,8} -> 1/3
    assert S.topk_overlap(a, l) == pytest.approx((0.5 + 1 / 3) / 2)
    assert S.topk_overlap(a, a) == 1.0
    assert S.topk_overlap(np.full((1, 3), -1), np.array([[1, 2, 3]])) == 0.0


def test_similarity_matrix_shape_and_diagonal():
    rng = np.random.default_rng(0)
    layers = [np.sort(rng.choice(50, 10, replace=False))[None, None] for _ in range(4)]
    sim = S.similarity_matrix(layers)
    assert np.allclose(np.diag(sim), 1.0) and np.all(np.tril(sim, -1) == 0.0)
    assert np.all((sim >= 0) & (sim <= 1))


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("first", [0, 2])
def test_dp_matches_exhaustive_search(seed, first):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(4, 10))
    sim = np.triu(rng.uniform(0.0, 1.0, (n, n)), 1) + np.eye(n)
    for m in range(1, n - first + 1):
        got, score = S.dp_anchor_schedule(sim, m, first)
        ref_arg, ref = S.brute_force_schedule(sim, m, first)
        assert score == pytest.approx(ref, abs=1e-12)
        assert S.schedule_score(sim, got) == pytest.approx(ref, abs=1e-12)
        assert len(got) == m and got == sorted(set(got)) and got[0] == first


def test_decaying_similarity_spreads_anchors_evenly():
    # similarity falls with distance the same way everywhere: equal spacing wins
    n = 12
    sim = np.array([[0.8 ** (l - a) if l >= a else 0.0 for l in range(n)] for a in range(n)])
    anchors, _ = S.dp_anchor_schedule(sim, 3)
    assert anchors == [0, 4, 8]
    anchors, _ = S.dp_anchor_schedule(sim, 3, first=2)   # layers 0-1 dense
    spans = np.diff(anchors + [n])
    assert anchors[0] == 2 and spans.max() - spans.min() <= 1


def test_all_anchors_is_exact():
    sim = np.triu(np.full((5, 5), 0.3), 1) + np.eye(5)
    anchors, score = S.dp_anchor_schedule(sim, 5)
    assert anchors == [0, 1, 2, 3, 4] and score == pytest.approx(5.0)


def test_bad_requests():
    sim = np.eye(4)
    with pytest.raises(ValueError):
        S.dp_anchor_schedule(sim, 0)
    with pytest.raises(ValueError):
        S.dp_anchor_schedule(sim, 4, first=1)
