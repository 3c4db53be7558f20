"""Pins for the oracle's quota planner with a searched threshold (CPU only).

Hand-derived examples (tests/golden/Q*.json), brute-force enumeration of the
quota rule stated declaratively (tests/brute_force.py), closed forms (no slots,
enough slots, one expert per rank) and invariants.
"""
import glob
import json
import os

import numpy as np
import pytest

import oracle
from oracle import path as oracle_path
from tests import brute_force as bf
from tests.test_oracle_plan import _tiny_cases, check_invariants
from workloads import WORKLOADS, router_logits

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "Q*.json")))


def _quota(ids, E, R, S, K, B, blk, tau_max=0):
    counts = oracle.load_matrix(ids, R, S, E)
    plan = oracle.plan_quota(counts, K, S, B, blk, tau_max)
    return counts, plan, oracle.align_sort(ids, plan)


def _ids_of(w, layer=0):
    score = oracle.SOFTMAX if w.score == "softmax" else oracle.SIGMOID
    ids, _ = oracle.route_topk(router_logits(w, layer), w.K, score)
    return ids


@pytest.mark.parametrize("path", GOLDEN, ids=[os.path.basename(p) for p in GOLDEN])
def test_hand_examples(path):
    g = json.load(open(path))
    sh = g["shape"]
    E, R, S, K, blk = (sh[k] for k in ("E", "R", "S", "K", "blk"))
    ids, _ = oracle.route_topk(np.array(g["logits"], np.float32), K, oracle.SIGMOID)
    assert ids.tolist() == g["ids"]
    for c in g["cases"]:
        counts, plan, al = _quota(ids, E, R, S, K, c["B"], blk, c["tau_max"])
        assert counts.tolist() == g["counts"]
        assert plan["tau"] == c["tau"] and plan["feasible"] == c["feasible"]
        for key in ("T", "L", "deficit", "h", "o", "O", "D", "n_rows_padded", "n_slots",
                    "n_remote", "home_row", "home_local"):
            assert plan[key].tolist() == c[key], key
        assert plan["C"] == c["C"]
        assert plan["replicas"] == c["replicas"]
        assert plan["segments"] == c["segments"]
        assert al["slot"].tolist() == c["slot"]
        C = plan["C"]
        for r in range(R):
            got = al["sorted_ids"][r * C:(r + 1) * C].tolist()
            for w_, x_ in zip(c["sorted_ids"][r], got):
                assert x_ == (oracle.UNSPECIFIED if w_ is None else w_)
        assert al["block_wrow"].tolist() == c["block_wrow"]
        assert al["block_expert"].tolist() == c["block_expert"]
        if "fixed_replicas" in c:
            fixed = oracle.plan_balance(counts, K, S, c["B"], blk, tau_max=c["tau_max"])
            assert fixed["replicas"] == c["fixed_replicas"]


def _small_cases():
    return [c for c in _tiny_cases() if len(c[0]) * c[4] <= 9]


@pytest.mark.parametrize("B", [0, 1, 2])
def test_brute_force_threshold_and_assignment(B):
    cases = _small_cases()
    assert len(cases) >= 10
    for ids, E, R, S, K in cases:
        counts = oracle.load_matrix(ids, R, S, E)
        maxL = int(oracle.imbalance(counts, S, K)["L"].max())
        plan = oracle.plan_quota(counts, K, S, B, 1, tau_max=maxL)
        al = oracle.align_sort(ids, plan)
        tau, asg = bf.quota_threshold(ids.tolist(), E, R, S, B)
        assert plan["tau"] == tau and plan["feasible"]
        assert tuple(int(s) // plan["C"] for s in al["slot"]) == asg
        reps = bf.replicas_of(asg, ids.tolist(), E, R)
        assert reps == {(rp["expert"], rp["rank"]) for rp in plan["replicas"]}


def test_brute_force_every_threshold_below():
    """At every tau the declarative rule admits one assignment, the oracle's,
    before and after the locality step."""
    for ids, E, R, S, K in _small_cases()[:8]:
        counts = oracle.load_matrix(ids, R, S, E)
        maxL = int(oracle.imbalance(counts, S, K)["L"].max())
        for tau in range(S * K, maxL + 1):
            plan = oracle_path._place(counts, K, S, 9, 1, oracle.capacity(E, K, S, 1, 0, maxL),
                                      tau, oracle_path._split_hot_first)
            al = oracle.align_sort(ids, plan)
            plans = bf.quota_conforming_plans(ids.tolist(), E, R, S, tau)
            assert len(plans) == 1
            assert tuple(int(s) // plan["C"] for s in al["slot"]) == plans[0]
            # the locality step on the same quotas
            oracle_path._local_counts(plan, counts)
            al = oracle.align_sort(ids, plan)
            local = bf.local_conforming_assignments(ids.tolist(), E, R, S, plans[0])
            assert len(local) == 1
            assert tuple(int(s) // plan["C"] for s in al["slot"]) == local[0]


def test_no_slots_means_nothing_moves():
    """B = 0: every replica would be remote, so the threshold rises to the
    largest home load and every pair stays home (closed form)."""
    for name in ("tiny", "decode16"):
        w = WORKLOADS[name]
        ids = _ids_of(w)
        counts = oracle.load_matrix(ids, w.R, w.S, w.E)
        L = oracle.imbalance(counts, w.S, w.K)["L"]
        plan = oracle.plan_quota(counts, w.K, w.S, 0, w.blk, tau_max=int(L.max()))
        assert plan["tau"] == L.max() and plan["replicas"] == []
        assert plan["h"].tolist() == plan["T"].tolist()


def test_enough_slots_means_exact_balance():
    """B >= E - E/R: no rank can hold more replicas than that, so tau = S*K
    and every rank holds exactly S*K pairs."""
    w = WORKLOADS["tiny"]
    ids = _ids_of(w)
    counts = oracle.load_matrix(ids, w.R, w.S, w.E)
    B = w.E - w.E // w.R
    plan = oracle.plan_quota(counts, w.K, w.S, B, 1, tau_max=4 * w.SK)
    al = oracle.align_sort(ids, plan)
    assert plan["tau"] == w.SK and plan["feasible"]
    rank_of = al["slot"] // plan["C"]
    assert np.bincount(rank_of, minlength=w.R).tolist() == [w.SK] * w.R


@pytest.mark.parametrize("seed", range(6))
def test_one_expert_per_rank_reduces_to_fixed_rule(seed):
    """With E = R the hottest expert of a rank is its only one, so shedding
    hot-first and shedding the stream tail coincide: at tau = S*K the quota
    plan is the fixed rule's plan."""
    rng = np.random.default_rng(seed)
    R = int(rng.integers(2, 9))
    S, K = int(rng.integers(1, 20)), int(rng.integers(1, R + 1))
    p = np.exp(-0.7 * rng.permutation(R))
    ids = np.array([rng.choice(R, K, replace=False, p=p / p.sum()) for _ in range(R * S)])
    counts = oracle.load_matrix(ids, R, S, R)
    a = oracle.plan_quota(counts, K, S, 1, 4)
    b = oracle.plan_balance(counts, K, S, 1, 4)
    assert a["tau"] == S * K
    for key in ("h", "o", "O", "D", "n_rows_padded", "n_slots", "n_remote", "home_row"):
        assert a[key].tolist() == b[key].tolist(), key
    # the same instances; only the quota plan adds its locality counts
    assert [{k: v for k, v in rp.items() if k != "local"} for rp in a["replicas"]] == b["replicas"]
    assert a["segments"] == b["segments"]


def check_quota_invariants(ids, plan, al, B):
    """Properties the quota rule fixes at any size."""
    E, R, tau, nh = plan["E"], plan["R"], plan["tau"], plan["E"] // plan["R"]
    T, L, h, o = plan["T"], plan["L"], plan["h"], plan["o"]
    rank_of = al["slot"] // plan["C"]
    load = np.bincount(rank_of, minlength=R)
    assert (load <= tau).all()
    assert np.array_equal(load[L >= tau], np.full(int((L >= tau).sum()), tau))
    assert np.array_equal(h + o, T)
    for r in range(R):
        mine = sorted(range(r * nh, (r + 1) * nh), key=lambda e: (-T[e], e))
        shedding = [o[e] > 0 for e in mine]
        for i, e in enumerate(mine):       # hot first
            if shedding[i]:
                assert all(h[x] == 0 for x in mine[:i])
        assert int(h[mine].sum()) == min(int(L[r]), tau)
    assert all(rp["count"] > 0 for rp in plan["replicas"])
    per_rank = np.bincount([rp["rank"] for rp in plan["replicas"]], minlength=R)
    if plan["feasible"]:
        assert per_rank.max(initial=0) <= B and plan["n_remote"].sum() == 0
    SK = plan["SK"]
    counts = oracle.load_matrix(ids, R, plan["S"], E)
    if plan["feasible"] and tau > SK:     # the threshold below did not qualify
        assert oracle.replicas_per_rank(counts, plan["K"], plan["S"], tau - 1,
                                        oracle_path._split_hot_first).max() > B


@pytest.mark.parametrize("name,B,tau_max_x", [("tiny", 1, 2), ("tiny", 0, 4), ("decode16", 1, 2),
                                              ("decode16", 3, 1), ("decode128", 1, 2),
                                              ("decode128", 3, 1), ("wideep", 2, 2)])
def test_invariants_on_workloads(name, B, tau_max_x):
    w = WORKLOADS[name]
    ids = _ids_of(w)
    counts = oracle.load_matrix(ids, w.R, w.S, w.E)
    plan = oracle.plan_quota(counts, w.K, w.S, B, w.blk, tau_max=tau_max_x * w.SK)
    al = oracle.align_sort(ids, plan)
    check_invariants(ids, plan, al) if plan["tau"] == w.SK else None
    check_quota_invariants(ids, plan, al, B)


def test_threshold_never_rises_with_more_slots():
    w = WORKLOADS["decode128"]
    ids = _ids_of(w)
    counts = oracle.load_matrix(ids, w.R, w.S, w.E)
    taus = [oracle.plan_quota(counts, w.K, w.S, B, w.blk, tau_max=2 * w.SK)["tau"]
            for B in range(0, 5)]
    assert all(a >= b for a, b in zip(taus, taus[1:]))
    assert taus[0] == oracle.imbalance(counts, w.S, w.K)["L"].max()


def test_quota_fits_the_pages_slot_counts():
    """On the decode workload with B = 3 the fixed rule needs remote replicas
    while hot-first shedding balances exactly inside the slots."""
    w = WORKLOADS["decode128"]
    ids = _ids_of(w)
    counts = oracle.load_matrix(ids, w.R, w.S, w.E)
    fixed = oracle.plan_balance(counts, w.K, w.S, w.B, w.blk)
    quota = oracle.plan_quota(counts, w.K, w.S, w.B, w.blk)
    assert fixed["n_remote"].sum() > 0
    assert quota["tau"] == w.SK and quota["feasible"] and quota["n_remote"].sum() == 0
