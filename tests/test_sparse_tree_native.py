"""The native calibrated sparse-tree builder (medusa_sparse_tree, host code in
the library) against the printed worked example of "Medusa 深读" §6.2 and the
oracle's greedy builder: the chosen paths, their canonical order, the pick
order and every weight must be identical (the weights bit for bit: both take
the product of the rank probabilities in path order)."""

import json
import os

import numpy as np
import pytest

from oracle import sparse_tree as OS
from oracle import tree as OT

import medusa_tree_verification_forward_amd._lib as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _paths(ranks):
    return [tuple(int(x) for x in row if x >= 0) for row in ranks]


def test_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "sparse_tree_worked_example.json")))
    a = np.array(g["a"], dtype=np.float64)
    ranks, w, order = L.sparse_tree(a, g["budget"])
    picks = [_paths(ranks)[i] for i in order]
    assert [[r + 1 for r in p] for p in picks] == g["order"]   # the page's ranks are 1-based
    assert np.allclose([w[i] for i in order], g["weights"], rtol=0, atol=1e-12)
    assert abs(float(w.sum()) - g["expected_cover"]) < 1e-12
    assert OT.check_spec(_paths(ranks), a.shape[0]) is None


def _table(rng, K, S, ties):
    if ties:
        # few distinct values: many equal weights, so the lexicographic rule decides
        return rng.choice([0.0, 0.05, 0.1, 0.25, 0.5], size=(K, S))
    # decaying by rank like a calibrated head, with noise
    return np.sort(rng.random((K, S)), axis=1)[:, ::-1] * rng.random((K, 1))


@pytest.mark.parametrize("seed", range(48))
def test_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    K = int(rng.integers(1, 7))
    S = int(rng.integers(1, 9))
    a = _table(rng, K, S, ties=seed % 3 == 0)
    full = sum(S ** k for k in range(1, K + 1))
    budget = int(rng.integers(0, min(255, full + 3) + 1))
    picks = OS.greedy_tree(a, budget)
    ranks, w, order = L.sparse_tree(a, budget)
    assert np.array_equal(ranks, OS.to_spec(picks, K).reshape(-1, K))
    assert [_paths(ranks)[i] for i in order] == picks
    assert np.array_equal(w, np.array([OS.path_weight(a, p) for p in _paths(ranks)]))
    assert OT.check_spec(_paths(ranks), K) is None
    assert len(ranks) == min(budget, full)


def test_budget_beyond_the_full_tree():
    a = np.array([[0.6, 0.3], [0.5, 0.4]])
    ranks, w, order = L.sparse_tree(a, 50)
    assert len(ranks) == 2 + 4
    assert sorted(order.tolist()) == list(range(6))


def test_empty_budget():
    ranks, w, order = L.sparse_tree(np.full((3, 2), 0.5), 0)
    assert ranks.shape == (0, 3) and w.size == 0 and order.size == 0


@pytest.mark.parametrize("bad", [-0.1, np.nan, np.inf])
def test_rejects_bad_probabilities(bad):
    a = np.full((2, 3), 0.2)
    a[1, 2] = bad
    with pytest.raises(L.MedusaError) as e:
        L.sparse_tree(a, 4)
    assert e.value.code == L.ERR_ARG


@pytest.mark.parametrize("K,S,budget,code", [(9, 2, 4, "UNSUPPORTED"), (2, 17, 4, "UNSUPPORTED"),
                                             (2, 2, 256, "UNSUPPORTED"), (2, 2, -1, "ARG")])
def test_rejects_limits(K, S, budget, code):
    with pytest.raises(L.MedusaError) as e:
        L.sparse_tree(np.full((K, S), 0.1), budget)
    assert e.value.code == getattr(L, "ERR_" + code)
