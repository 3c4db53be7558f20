"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a private copy of the oracle's source (on the
CPU; the real oracle is untouched), runs the pin checks against the copy, and
requires that at least one of them fails.
"""
import glob
import importlib.util
import json
import os
import sys
import types

import numpy as np
import pytest

import oracle
from oracle import path as oracle_path
from tests import brute_force as bf
from tests.test_oracle_plan import check_invariants, _tiny_cases

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "W*.json")))
QGOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "Q*.json")))

MUTATIONS = {
    "tie_to_higher_index": ("np.lexsort((expert, -key)", "np.lexsort((-expert, -key)"),
    "sigmoid_sign": ("np.exp(-l64)", "np.exp(l64)"),
    "source_rank_modulo": ("np.arange(N, dtype=np.int64) // S", "np.arange(N, dtype=np.int64) % S"),
    "home_keep_off_by_one": ("h[e] = min(max(tau - Pe, 0), T[e])", "h[e] = min(max(tau - Pe - 1, 0), T[e])"),
    "inclusive_overflow_prefix": ("        O[e] = acc\n        acc += o[e]", "        acc += o[e]\n        O[e] = acc"),
    "intersection_min_for_max": ("lo = np.maximum(O[:, None], D[None, :R])", "lo = np.minimum(O[:, None], D[None, :R])"),
    "slot_bound_inclusive": ("if j < B:", "if j <= B:"),
    "remote_row_wrong": ("wrow = e\n", "wrow = E + j\n"),
    "pad_always_adds_block": ("pad = lambda c: ((c + blk - 1) // blk) * blk",
                              "pad = lambda c: (c // blk + 1) * blk"),
    "overflow_offset_drops_h": ("o_pos = O[e_ov] + (q[ov] - h[e_ov])", "o_pos = O[e_ov] + q[ov]"),
    "replica_row_offset": ("(o_pos - np.maximum(O[e_ov], D[d_ov]))", "(o_pos - O[e_ov])"),
    "sentinel_minus_one": ("= P                 # padding sentinel", "= P - 1             # padding sentinel"),
    "combine_subtracts": ("y = term if y is None else y + term", "y = term if y is None else y - term"),
    "stable_rank_unstable": ('order = np.argsort(flat, kind="stable")', 'order = np.argsort(-flat, kind="stable")[::-1]'),
    # quota planner
    "quota_coldest_first": ("key=lambda e: (-int(T[e]), e))", "key=lambda e: (int(T[e]), e))"),
    "quota_tie_to_higher_index": ("key=lambda e: (-int(T[e]), e))", "key=lambda e: (-int(T[e]), -e))"),
    "quota_sheds_one_extra": ("shed = max(int(sum(T[e] for e in mine)) - tau, 0)",
                              "shed = max(int(sum(T[e] for e in mine)) - tau + 1, 0)"),
    "quota_line_in_index_order": ("order.extend(hot)", "order.extend(mine)"),
    "quota_search_skips_SK": ("for t in range(SK, hi + 1):", "for t in range(SK + 1, hi + 1):"),
    "quota_slot_bound_strict": ("_split_hot_first).max() <= B:", "_split_hot_first).max() < B:"),
    "quota_fallback_at_SK": ("tau, feasible = t_max, False", "tau, feasible = SK, False"),
    "quota_deficit_from_SK": ("    deficit = tau - keep\n", "    deficit = S * K - np.minimum(L, S * K)\n"),
    # locality of the quota plan
    "locality_off": ('    if plan.get("local", False):\n        d, row = _place_local', '    if False:\n        d, row = _place_local'),
    "locality_takes_latest": ("mine = np.nonzero((src[fs] == rank) & ~taken)[0][:quota]",
                              "mine = np.nonzero((src[fs] == rank) & ~taken)[0][::-1][:quota][::-1]"),
    "locality_rest_replicas_first": ("for (rank, quota, row0), nl in zip(inst, n_local):",
                                     "for (rank, quota, row0), nl in list(zip(inst, n_local))[::-1]:"),
    "locality_rest_before_local": ("row[fs[sel]] = row0 + nl + np.arange(sel.size)",
                                   "row[fs[sel]] = row0 + np.arange(sel.size); row[fs[taken & (src[fs] == rank)]] += sel.size"),
    "locality_home_count_from_rank0": ("counts[e_all // nh, e_all])", "counts[0, e_all])"),
}


def _mutant(old, new):
    src = open(oracle_path.__file__).read()
    assert src.count(old) >= 1, old
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pins(o):
    """Run the pin checks against oracle module ``o``; return failures."""
    failures = 0
    for path in GOLDEN:
        g = json.load(open(path))
        sh = g["shape"]
        E, R, S, K, B, blk = (sh[k] for k in ("E", "R", "S", "K", "B", "blk"))
        try:
            ids, _ = o.route_topk(np.array(g["logits"], np.float32), K, o.SIGMOID)
            counts = o.load_matrix(ids, R, S, E)
            plan = o.plan_balance(counts, K, S, B, blk)
            al = o.align_sort(ids, plan)
            ok = (ids.tolist() == g["ids"] and counts.tolist() == g["counts"]
                  and plan["segments"] == g["segments"] and plan["replicas"] == g["replicas"]
                  and al["slot"].tolist() == g["slot"])
            C = plan["C"]
            for r in range(R):
                for w_, x_ in zip(g["sorted_ids"][r], al["sorted_ids"][r * C:(r + 1) * C].tolist()):
                    ok = ok and (w_ is None or w_ == x_)
        except Exception:
            ok = False
        failures += not ok
    for case in range(0, 40, 5):
        ids, E, R, S, K = _tiny_cases()[case]
        try:
            counts = o.load_matrix(ids, R, S, E)
            plan = o.plan_balance(counts, K, S, 1, 1)
            al = o.align_sort(ids, plan)
            check_invariants(ids, plan, al)
            plans = bf.rule_conforming_plans(ids.tolist(), E, R, S)
            ok = len(plans) == 1 and tuple(int(s) // plan["C"] for s in al["slot"]) == plans[0]
        except Exception:
            ok = False
        failures += not ok
    for path in QGOLDEN:
        g = json.load(open(path))
        sh = g["shape"]
        E, R, S, K, blk = (sh[k] for k in ("E", "R", "S", "K", "blk"))
        for c in g["cases"]:
            try:
                ids = np.array(g["ids"])
                counts = o.load_matrix(ids, R, S, E)
                plan = o.plan_quota(counts, K, S, c["B"], blk, c["tau_max"])
                al = o.align_sort(ids, plan)
                ok = (plan["tau"] == c["tau"] and plan["feasible"] == c["feasible"]
                      and all(plan[k].tolist() == c[k] for k in ("h", "O", "D", "deficit", "home_local"))
                      and plan["segments"] == c["segments"] and plan["replicas"] == c["replicas"]
                      and al["slot"].tolist() == c["slot"])
            except Exception:
                ok = False
            failures += not ok
    for case in (0, 3, 6, 9):
        ids, E, R, S, K = [c for c in _tiny_cases() if len(c[0]) * c[4] <= 9][case]
        try:
            counts = o.load_matrix(ids, R, S, E)
            maxL = int(o.imbalance(counts, S, K)["L"].max())
            plan = o.plan_quota(counts, K, S, 1, 1, tau_max=maxL)
            al = o.align_sort(ids, plan)
            tau, asg = bf.quota_threshold(ids.tolist(), E, R, S, 1)
            ok = plan["tau"] == tau and tuple(int(s) // plan["C"] for s in al["slot"]) == asg
        except Exception:
            ok = False
        failures += not ok
    # closed forms: sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4; identity combine
    try:
        _, gg = o.route_topk(np.array([[0.0, np.log(3.0)]], np.float32), 2, o.SIGMOID)
        ok = abs(gg[0, 0] - 0.75) < 1e-6 and gg[0, 1] == 0.5
        rng = np.random.default_rng(0)
        out = rng.integers(0, 2 ** 15, size=(6, 4)).astype(np.uint16)
        gt = rng.random((3, 2)).astype(np.float32)
        y, _ = o.combine(lambda rows: out[rows], np.arange(6), gt, 2)
        o64 = oracle.bf16_to_f64(out)
        ok = ok and np.allclose(y[1], gt[1, 0] * o64[2] + gt[1, 1] * o64[3], rtol=1e-15)
    except Exception:
        ok = False
    failures += not ok
    return failures


TRAIN_MUTATIONS = {
    "prefetch_slot_is_weight_row": ('return {(rp["rank"], rp["wrow"] - E): rp["expert"]',
                                    'return {(rp["rank"], rp["wrow"]): rp["expert"]'),
    "prefetch_takes_remote_too": ('for rp in plan["replicas"] if rp["wrow"] >= E}',
                                  'for rp in plan["replicas"] if rp["wrow"] >= 0}'),
    "reduce_grad_reverse_order": ("    for rp in plan[\"replicas\"]:                 # line order",
                                  "    for rp in plan[\"replicas\"][::-1]:           # line order"),
    "reduce_grad_keeps_slots": ("        slot_grads[d, j] = 0.0", "        slot_grads[d, j] = slot_grads[d, j]"),
    "reduce_grad_clears_all": ("    for d, j in used:\n        slot_grads[d, j] = 0.0",
                               "    for d, j in used:\n        slot_grads[d, j] = 0.0\n    slot_grads[:] = 0.0"),
    "combine_bwd_wrong_token": ("t = f // K\n", "t = f % N\n"),
    "combine_bwd_no_gate": ("prod = (g32.reshape(-1)[:, None].astype(np.float64) * dy32[t].astype(np.float64))",
                            "prod = (1.0 * dy32[t].astype(np.float64))"),
    "bf16_ties_up": ("((drop == 0x8000) & ((keep & np.uint32(1)) == 1))", "(drop == 0x8000)"),
    "dispatch_bwd_drops_last_k": ("    for k in range(K):\n        v = bf16_to_f64(d_recv_rows_of",
                                  "    for k in range(K - 1):\n        v = bf16_to_f64(d_recv_rows_of"),
}


def _pins_train(o):
    from tests import test_oracle_train as tt
    failures = 0
    for name in dir(tt):
        if name.startswith("check_"):
            try:
                getattr(tt, name)(o)
            except Exception:
                failures += 1
    return failures


def test_unmutated_oracle_passes_the_train_pins():
    assert _pins_train(oracle_path) == 0


@pytest.mark.parametrize("name", sorted(TRAIN_MUTATIONS))
def test_train_pins_catch_planted_mistake(name):
    old, new = TRAIN_MUTATIONS[name]
    assert _pins_train(_mutant(old, new)) > 0, f"planted mistake {name!r} went unnoticed"


def test_unmutated_oracle_passes_the_pins():
    assert _pins(oracle_path) == 0


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    old, new = MUTATIONS[name]
    assert _pins(_mutant(old, new)) > 0, f"planted mistake {name!r} went unnoticed"
