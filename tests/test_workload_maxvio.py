"""The max_vio sweep workload: routings built so that max_vio (the MoonEP
article's imbalance measure, max_e T_e / mean_e T_e - 1) takes a chosen value.

Pins: top-K of the generated logits (the oracle's router) selects exactly the
constructed expert sets; the realised max_vio equals the construction's
closed form round((1 + v) N K / E) * E / (N K) - 1, within half a pair of the
target; every other expert's load is within one pair of the others."""
import numpy as np
import pytest

import oracle
from workloads import WORKLOADS
from workloads.gen import MAXVIO_SWEEP, hot_pair_count, maxvio_choice, maxvio_logits


@pytest.mark.parametrize("vio", MAXVIO_SWEEP)
def test_topk_selects_the_constructed_sets_and_hits_max_vio(vio):
    w = WORKLOADS["moonep"].with_(vio=vio, S=512)
    hot, choice = maxvio_choice(w)
    ids, _ = oracle.route_topk(maxvio_logits(w), w.K, oracle.SIGMOID)
    picked = np.zeros_like(choice)
    np.put_along_axis(picked, ids, True, axis=1)
    assert np.array_equal(picked, choice)
    st = oracle.imbalance(oracle.load_matrix(ids, w.R, w.S, w.E), w.S, w.K)
    T = st["T"]
    assert T.argmax() == hot and T[hot] == hot_pair_count(w)
    assert st["max_vio"] == pytest.approx(hot_pair_count(w) * w.E / (w.N * w.K) - 1, abs=1e-12)
    assert abs(st["max_vio"] - vio) <= 0.5 * w.E / (w.N * w.K) + 1e-12
    rest = np.delete(T, hot)
    assert rest.max() - rest.min() <= 1


def test_full_size_loads_without_routing():
    """At the article's bench shape (S=8192, E=384, K=8, EP8) the constructed
    loads give max_vio within 1e-3 of each target."""
    for vio in MAXVIO_SWEEP:
        w = WORKLOADS["moonep"].with_(vio=vio)
        hot, choice = maxvio_choice(w)
        assert (choice.sum(axis=1) == w.K).all()
        T = choice.sum(axis=0)
        assert T.argmax() == hot
        assert abs(T[hot] * w.E / (w.N * w.K) - 1 - vio) < 1e-3


def test_vio_out_of_range_is_refused():
    w = WORKLOADS["moonep"]
    with pytest.raises(ValueError):
        maxvio_choice(w.with_(vio=w.E / w.K))
