"""Pins for the oracle's router top-K, gates and load matrix (CPU only)."""
import math

import numpy as np
import pytest

import oracle
from tests.brute_force import topk_by_sorting
from workloads import WORKLOADS, router_logits


def _quantised_logits(rng, N, E, levels):
    """Logits on a coarse grid so that ties are frequent; includes -0.0."""
    v = rng.integers(-levels, levels + 1, size=(N, E)).astype(np.float32) * np.float32(0.5)
    neg0 = rng.random((N, E)) < 0.1
    v[neg0 & (v == 0)] = np.float32(-0.0)
    return v


@pytest.mark.parametrize("E,K", [(4, 1), (4, 4), (8, 2), (16, 5), (33, 8), (64, 8)])
def test_topk_matches_sorting_brute_force(E, K):
    rng = np.random.default_rng(E * 100 + K)
    logits = _quantised_logits(rng, 200, E, 3)
    ids, _ = oracle.route_topk(logits, K, oracle.SIGMOID)
    for t in range(logits.shape[0]):
        assert list(ids[t]) == topk_by_sorting(logits[t], K)


def test_topk_with_selection_bias_matches_sorting():
    rng = np.random.default_rng(5)
    E, K = 16, 4
    logits = _quantised_logits(rng, 100, E, 4)
    bias = (rng.integers(-2, 3, size=E) * 0.25).astype(np.float32)
    ids, gates = oracle.route_topk(logits, K, oracle.SIGMOID, sel_bias=bias)
    for t in range(logits.shape[0]):
        key = [np.float32(logits[t, e]) + np.float32(bias[e]) for e in range(E)]
        assert list(ids[t]) == topk_by_sorting(key, K)
        # the bias steers selection only: gates come from the raw logits
        for k in range(K):
            x = float(logits[t, ids[t, k]])
            assert gates[t, k] == pytest.approx(1.0 / (1.0 + math.exp(-x)), rel=1e-15)


def test_special_cases():
    E = 8
    # all-equal logits -> experts 0..K-1
    ids, _ = oracle.route_topk(np.zeros((3, E), np.float32), 3, oracle.SIGMOID)
    assert (ids == np.array([0, 1, 2])).all()
    # K = 1 -> argmax with the lowest index among equals
    lg = np.array([[1, 3, 3, 0, 2, 3, 0, 0]], np.float32)
    ids, _ = oracle.route_topk(lg, 1, oracle.SIGMOID)
    assert ids[0, 0] == int(np.argmax(lg[0]))
    # K = E -> full order, descending key, ascending index among equals
    ids, _ = oracle.route_topk(lg, E, oracle.SIGMOID)
    assert list(ids[0]) == [1, 2, 5, 4, 0, 3, 6, 7]
    # -0.0 and +0.0 tie -> the lower index first, whichever is negative
    lg = np.array([[-1, 0.0, -0.0, -2], [-1, -0.0, 0.0, -2]], np.float32)
    ids, _ = oracle.route_topk(lg, 2, oracle.SIGMOID)
    assert (ids == np.array([[1, 2], [1, 2]])).all()


def test_gates_closed_forms():
    # sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4
    lg = np.array([[0.0, math.log(3.0), -50.0, -60.0]], np.float32)
    _, g = oracle.route_topk(lg, 2, oracle.SIGMOID)
    assert g[0, 0] == pytest.approx(0.75, rel=2e-7)
    assert g[0, 1] == 0.5
    # softmax of equal logits = 1/E
    _, g = oracle.route_topk(np.full((2, 8), 0.3, np.float32), 3, oracle.SOFTMAX)
    assert np.all(g == pytest.approx(1.0 / 8, rel=1e-15))
    # softmax of log(1..4) = (1..4)/10 (up to the fp32 rounding of the logs)
    lg = np.log(np.array([[1.0, 2.0, 3.0, 4.0]])).astype(np.float32)
    ids, g = oracle.route_topk(lg, 4, oracle.SOFTMAX)
    assert list(ids[0]) == [3, 2, 1, 0]
    assert g[0] == pytest.approx([0.4, 0.3, 0.2, 0.1], rel=3e-7)
    # renormalisation over the chosen K sums to one, ratios kept
    ids, g = oracle.route_topk(lg, 2, oracle.SOFTMAX, renorm=True)
    assert g[0] == pytest.approx([4 / 7, 3 / 7], rel=3e-7)
    # softmax is shift invariant: a large common offset changes nothing
    _, g2 = oracle.route_topk(lg + np.float32(80.0), 4, oracle.SOFTMAX)
    assert g2[0] == pytest.approx([0.4, 0.3, 0.2, 0.1], rel=1e-5)


def test_load_matrix_against_bincount_and_closed_forms():
    rng = np.random.default_rng(1)
    R, S, E, K = 4, 50, 16, 3
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(R * S)])
    counts = oracle.load_matrix(ids, R, S, E)
    for r in range(R):
        assert (counts[r] == np.bincount(ids[r * S:(r + 1) * S].ravel(), minlength=E)).all()
    assert counts.sum() == R * S * K
    # round robin over all experts: perfectly balanced, max_vio = 0
    N, K, E = 32, 2, 8
    ids = np.array([[(t * K + k) % E for k in range(K)] for t in range(N)])
    st = oracle.imbalance(oracle.load_matrix(ids, 4, 8, E), 8, K)
    assert st["max_vio"] == 0.0
    # every token on experts 0..K-1: max_vio = E/K - 1
    ids = np.tile(np.arange(K), (N, 1))
    st = oracle.imbalance(oracle.load_matrix(ids, 4, 8, E), 8, K)
    assert st["max_vio"] == pytest.approx(E / K - 1)


def test_workload_generators_are_seeded_and_shaped():
    w = WORKLOADS["tiny"]
    a = router_logits(w, 0)
    b = router_logits(w, 0)
    assert a.dtype == np.float32 and a.shape == (w.N, w.E)
    assert (a.view(np.uint32) == b.view(np.uint32)).all()
    assert not np.array_equal(router_logits(w, 1), a)
