"""Pins for the oracle's replica weight prefetch, the unpermute backward
(combine and dispatch gradients) and reduce_grad (CPU only).

Prefetch and reduce_grad are checked against the replica lists of the
hand-derived plans (tests/golden/W*.json, Q*.json), not the oracle's own plan;
the backward against adjoint identities, central differences and exactly
representable cases; reduce_grad against exact integer conservation.
"""
import glob
import json
import os

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, router_logits, random_expert_out

GOLD = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "*.json")))


def _golden_plans():
    """(E, R, B, replicas) of every hand-derived plan."""
    out = []
    for path in GOLD:
        g = json.load(open(path))
        sh = g["shape"]
        if "cases" in g:
            for c in g["cases"]:
                out.append((sh["E"], sh["R"], c["B"], c["replicas"]))
        else:
            out.append((sh["E"], sh["R"], sh["B"], g["replicas"]))
    return out


def _plan_stub(E, R, B, replicas):
    return {"E": E, "R": R, "B": B, "replicas": replicas}


# --------------------------------------------------------------------------- prefetch
def check_prefetch_follows_the_hand_derived_slot_tables(o=oracle):
    rng = np.random.default_rng(0)
    seen_remote = False
    for E, R, B, reps in _golden_plans():
        W = rng.integers(0, 2 ** 16, size=(E, 24), dtype=np.uint16)
        slots = rng.integers(0, 2 ** 16, size=(R, max(B, 1), 24), dtype=np.uint16)
        got = o.prefetch_weights(_plan_stub(E, R, B, reps), W, slots)
        want = slots.copy()
        for rp in reps:
            if rp["wrow"] >= E:                      # a slot row: copy home weights
                want[rp["rank"], rp["wrow"] - E] = W[rp["expert"]]
            else:                                    # remote: read from home, no copy
                assert rp["wrow"] == rp["expert"]
                seen_remote = True
        assert np.array_equal(got, want)
    assert seen_remote


def check_prefetch_on_a_workload_plan(o=oracle):
    w = WORKLOADS["decode128"]
    ids, _ = o.route_topk(router_logits(w, 0), w.K, o.SIGMOID)
    plan = o.plan_balance(o.load_matrix(ids, w.R, w.S, w.E), w.K, w.S, w.B, w.blk)
    m = o.prefetch_slots(plan)
    assert len(m) == int(plan["n_slots"].sum())
    for (d, j), e in m.items():
        assert 0 <= j < w.B and e // (w.E // w.R) != d      # never the rank's own expert


# --------------------------------------------------------------------------- backward
def _small_case(seed=0, N=12, K=3, H=40, rows=64):
    rng = np.random.default_rng(seed)
    slot = rng.permutation(rows)[: N * K]
    out = rng.integers(0, 2 ** 15, size=(rows, H)).astype(np.uint16)     # finite bf16
    out = np.where(rng.random((rows, H)) < 0.5, out | 0x8000, out).astype(np.uint16)
    out = np.where((out & 0x7F80) == 0x7F80, out & 0xBFFF, out).astype(np.uint16)
    gates = rng.random((N, K)).astype(np.float32)
    dy = rng.standard_normal((N, H)).astype(np.float32)
    return slot, out, gates, dy


def check_gate_gradient_matches_central_differences(o=oracle):
    slot, out, gates, dy = _small_case()
    N, K = gates.shape
    _, d_g, mag = o.combine_bwd(lambda r: out[r], slot, gates, dy, K)
    loss = lambda g: (dy.astype(np.float64) * o.combine(lambda r: out[r], slot, g, K)[0]).sum()  # noqa
    for t, k in [(0, 0), (3, 2), (11, 1)]:
        gp = gates.astype(np.float64).copy()
        gm = gates.astype(np.float64).copy()
        eps = 2.0 ** -10
        gp[t, k] += eps
        gm[t, k] -= eps
        # combine takes fp32 gates; keep the perturbed values exact in fp32
        fd = (loss(gp.astype(np.float32)) - loss(gm.astype(np.float32))) / (2 * eps)
        assert abs(fd - d_g[t, k]) <= 1e-9 * mag[t, k]


def check_expert_output_gradient_is_exact_when_representable(o=oracle):
    """Gates that are powers of two and dy that is bf16-representable make
    g * dy exact, so d_out must equal it bit for bit, and the adjoint
    identity <dy, combine(out)> = <d_out, out> holds to fp64 rounding."""
    slot, out, gates, dy = _small_case(1)
    N, K = gates.shape
    rng = np.random.default_rng(5)
    gates = (2.0 ** -rng.integers(0, 4, size=(N, K))).astype(np.float32)
    dy = o.bf16_to_f64(o.f32_to_bf16_rne(dy)).astype(np.float32)
    d_out, _, _ = o.combine_bwd(lambda r: out[r], slot, gates, dy, K)
    want = gates.reshape(-1)[:, None].astype(np.float64) * dy[np.arange(N * K) // K]
    assert np.array_equal(o.bf16_to_f64(d_out), want)
    y, _ = o.combine(lambda r: out[r], slot, gates, K)
    lhs = (dy.astype(np.float64) * y).sum()
    rhs = (o.bf16_to_f64(d_out) * o.bf16_to_f64(out[slot])).sum()
    assert abs(lhs - rhs) <= 1e-12 * np.abs(dy.astype(np.float64) * y).sum()


def check_bf16_rounding_ties_to_even(o=oracle):
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5,
                     3.0e38, 1e-40], dtype=np.float32)
    got = o.bf16_to_f64(o.f32_to_bf16_rne(vals))
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even (1);
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to 1 + 2^-6
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == 1.0 + 2 ** -6
    assert got[3] == 1.0 + 2 ** -7 and got[4] == -2.5
    assert np.isfinite(got[5]) and got[6] >= 0


def check_dispatch_gradient_is_the_adjoint_of_dispatch(o=oracle):
    slot, out, gates, dy = _small_case(2)
    N, K = gates.shape
    rows, H = out.shape
    rng = np.random.default_rng(3)
    x = o.f32_to_bf16_rne(rng.standard_normal((N, H)).astype(np.float32))
    recv = np.zeros((rows, H), np.uint16)
    recv[slot] = x[np.arange(N * K) // K]
    d_recv = out                                   # any bf16 rows
    dx, _ = o.dispatch_bwd(lambda r: d_recv[r], slot, K, N)
    lhs = (o.bf16_to_f64(d_recv) * o.bf16_to_f64(recv)).sum()
    rhs = (dx * o.bf16_to_f64(x)).sum()
    assert abs(lhs - rhs) <= 1e-12 * (np.abs(o.bf16_to_f64(d_recv)).sum() * 4)
    # unit gates: dispatch_bwd is combine with every gate 1
    y, _ = o.combine(lambda r: d_recv[r], slot, np.ones((N, K), np.float32), K)
    assert np.array_equal(y, dx)


# --------------------------------------------------------------------------- reduce_grad
def check_reduce_grad_on_hand_derived_plans_conserves_exactly(o=oracle):
    rng = np.random.default_rng(4)
    for E, R, B, reps in _golden_plans():
        Bs = max(B, 1)
        G = rng.integers(-50, 50, size=(E, 6)).astype(np.float32)       # exact in fp32
        SG = rng.integers(-50, 50, size=(R, Bs, 6)).astype(np.float32)
        g2, sg2 = o.reduce_grad(_plan_stub(E, R, B, reps), SG, G)
        want = G.astype(np.int64)
        used = set()
        for rp in reps:
            if rp["wrow"] >= E:
                want[rp["expert"]] += SG[rp["rank"], rp["wrow"] - E].astype(np.int64)
                used.add((rp["rank"], rp["wrow"] - E))
        assert np.array_equal(g2.astype(np.int64), want)
        for d in range(R):
            for j in range(Bs):
                if (d, j) in used:
                    assert (sg2[d, j] == 0).all()
                else:
                    assert np.array_equal(sg2[d, j], SG[d, j])


def check_reduce_grad_adds_in_line_order(o=oracle):
    """fp32 addition is not associative: the order is part of the result.
    Three replicas of one expert, values chosen so every other order of
    the three additions gives a different fp32 sum."""
    E, R, B = 4, 4, 1
    reps = [{"expert": 0, "rank": 1, "count": 1, "line": 0, "wrow": 4, "row": 0},
            {"expert": 0, "rank": 2, "count": 1, "line": 1, "wrow": 4, "row": 0},
            {"expert": 0, "rank": 3, "count": 1, "line": 2, "wrow": 4, "row": 0}]
    G = np.zeros((E, 1), np.float32)
    G[0] = 1.0
    SG = np.zeros((R, B, 1), np.float32)
    SG[1, 0], SG[2, 0], SG[3, 0] = 2.0 ** 24, -(2.0 ** 24), 1.0
    g2, _ = o.reduce_grad(_plan_stub(E, R, B, reps), SG, G)
    # ((1 + 2^24) + -2^24) + 1 = (2^24 - 2^24) + 1 = 1 (1 + 2^24 rounds to 2^24 in fp32)
    assert g2[0, 0] == 1.0


def test_prefetch_follows_the_hand_derived_slot_tables():
    check_prefetch_follows_the_hand_derived_slot_tables()


def test_prefetch_on_a_workload_plan():
    check_prefetch_on_a_workload_plan()


def test_gate_gradient_matches_central_differences():
    check_gate_gradient_matches_central_differences()


def test_expert_output_gradient_is_exact_when_representable():
    check_expert_output_gradient_is_exact_when_representable()


def test_bf16_rounding_ties_to_even():
    check_bf16_rounding_ties_to_even()


def test_dispatch_gradient_is_the_adjoint_of_dispatch():
    check_dispatch_gradient_is_the_adjoint_of_dispatch()


def test_reduce_grad_on_hand_derived_plans_conserves_exactly():
    check_reduce_grad_on_hand_derived_plans_conserves_exactly()


def test_reduce_grad_adds_in_line_order():
    check_reduce_grad_adds_in_line_order()
