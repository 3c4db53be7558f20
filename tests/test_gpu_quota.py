"""GPU parity of the quota planner (lbt_plan_quota): threshold search and plan
against the oracle's plan_quota, bit-exact, followed by the unchanged align,
dispatch and combine."""
import glob
import json
import os

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, router_logits, activations
from tests import gpu_util as gu
from tests.test_gpu_parity import _full_move_check

pytestmark = pytest.mark.gpu

QGOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "Q*.json")))


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _quota_pair(w, B, tau_max, layer=0):
    w = w.with_(B=B)
    logits = router_logits(w, layer)
    res = gu.run_front(gu.shape_of(w, tau_max=tau_max), logits, planner="quota")
    ref = gu.run_oracle(w, logits, planner="quota", tau_max=tau_max)
    return w, res, ref


@pytest.mark.parametrize("path", QGOLDEN, ids=[os.path.basename(p) for p in QGOLDEN])
def test_gpu_quota_matches_hand_examples(path):
    import load_balanced_token_amd as lbt
    g = json.load(open(path))
    sh = g["shape"]
    for c in g["cases"]:
        shape = lbt.Shape(E=sh["E"], K=sh["K"], R=sh["R"], S=sh["S"], H=8, B=c["B"],
                          blk=sh["blk"], tau_max=c["tau_max"])
        res = gu.run_front(shape, np.array(g["logits"], np.float32), planner="quota")
        assert res["ids"].tolist() == g["ids"]
        assert res["counts"].tolist() == g["counts"]
        pf = res["plan_fields"]
        assert pf["hdr"][gu.HDR_TAU] == c["tau"]
        assert pf["hdr"][gu.HDR_FEASIBLE] == int(c["feasible"])
        for key in ("T", "h", "O", "L", "D", "n_rows_padded", "n_slots", "n_remote",
                    "home_row"):
            assert pf[key].tolist() == c[key], key
        assert pf["def"].tolist() == c["deficit"]
        assert res["sizes"]["C"] == c["C"]
        assert res["slot"].tolist() == c["slot"]
        C = c["C"]
        for r in range(sh["R"]):
            for want, got in zip(c["sorted_ids"][r], res["sorted_ids"][r * C:(r + 1) * C].tolist()):
                if want is not None:
                    assert got == want
        assert res["block_wrow"].tolist() == c["block_wrow"]
        assert res["block_expert"].tolist() == c["block_expert"]


# (workload, B, tau_max in units of S*K): the pages' own B (exact S*K holds),
# smaller B that makes the threshold rise, and a fallback case.
QUOTA_CASES = [("tiny", 0, 4), ("tiny", 1, 2), ("decode1", 1, 4), ("decode16", 1, 2),
               ("decode128", 1, 2), ("decode128", 3, 1), ("wideep", 1, 2), ("wideep", 2, 2),
               ("dsv3", 2, 2), ("dsv3", 32, 1), ("kimi", 4, 1)]


@pytest.mark.parametrize("name,B,x", QUOTA_CASES)
def test_quota_plan_parity(name, B, x):
    w = WORKLOADS[name]
    print(f"[quota] {name} B={B} tau_max={x}*SK", flush=True)
    w, res, ref = _quota_pair(w, B, x * w.SK)
    gu.check_route(res, ref)
    gu.check_plan(res["plan_fields"], ref["plan"], w.P)
    gu.check_align(res, ref, w.R, res["sizes"]["C"])
    # every rank holds at most tau pairs
    load = np.bincount(res["slot"][:w.P] // res["sizes"]["C"], minlength=w.R)
    assert load.max() <= ref["plan"]["tau"]


@pytest.mark.parametrize("B,x", [(2, 2), (1, 1)])
def test_quota_ragged_tiles(B, x):
    """Several tiles per rank with a ragged last one (S = 300): the locality
    step's per-rank pair offsets come from rank r's first tile."""
    w = WORKLOADS["dsv3"].with_(S=300, H=64)
    w, res, ref = _quota_pair(w, B, x * w.SK)
    gu.check_plan(res["plan_fields"], ref["plan"], w.P)
    gu.check_align(res, ref, w.R, res["sizes"]["C"])
    _full_move_check(w, res, ref, activations(w, 0))


def test_quota_plan_parity_more_layers():
    w = WORKLOADS["decode128"]
    for layer in (1, 2, 3):
        _, res, ref = _quota_pair(w, 1, 2 * w.SK, layer)
        gu.check_plan(res["plan_fields"], ref["plan"], w.P)
        gu.check_align(res, ref, w.R, res["sizes"]["C"])


@pytest.mark.parametrize("name,S,B", [("tiny", None, 1), ("dsv3", 256, 2), ("wideep", 64, 1)])
def test_quota_dispatch_combine_full_rows(name, S, B):
    w = WORKLOADS[name]
    if S is not None:
        w = w.with_(S=S)
    print(f"[quota] move {name} S={w.S} B={B}", flush=True)
    w, res, ref = _quota_pair(w, B, 2 * w.SK)
    gu.check_align(res, ref, w.R, res["sizes"]["C"])
    _full_move_check(w, res, ref, activations(w, 0))


def test_quota_deterministic_rerun():
    w = WORKLOADS["dsv3"].with_(B=2)
    logits = router_logits(w, 0)
    a = gu.run_front(gu.shape_of(w, tau_max=2 * w.SK), logits, planner="quota")
    b = gu.run_front(gu.shape_of(w, tau_max=2 * w.SK), logits, planner="quota")
    assert np.array_equal(a["plan"], b["plan"])
    assert np.array_equal(a["slot"], b["slot"])
    C = a["sizes"]["C"]
    for r, n in enumerate(a["plan_fields"]["n_rows_padded"]):   # rows past n are unspecified
        assert np.array_equal(a["sorted_ids"][r * C: r * C + n], b["sorted_ids"][r * C: r * C + n])


def test_quota_degenerate_shapes():
    """One expert per rank (the quota plan equals the fixed rule's at S*K),
    no slots with room to keep everything home, and an empty batch."""
    t = gu.torch()
    base = WORKLOADS["tiny"]
    # E = R
    w = base.with_(E=4, R=4, K=2)
    logits = router_logits(w, 0)
    q = gu.run_front(gu.shape_of(w), logits, planner="quota")
    f = gu.run_front(gu.shape_of(w), logits, planner="fixed")
    # the same plan; only the quota plan carries the locality words
    z = q["sizes"]
    skip = np.zeros(q["plan"].size, bool)
    skip[z["off_hdr"] + gu.HDR_LOCAL] = True
    skip[z["off_home_local"]: z["off_home_local"] + w.E] = True
    skip[z["off_piece_local"]: z["off_piece_local"] + z["max_pieces"]] = True
    assert np.array_equal(q["plan"][~skip], f["plan"][~skip])
    ref = gu.run_oracle(w, logits, planner="quota")
    gu.check_plan(q["plan_fields"], ref["plan"], w.P)
    gu.check_align(q, ref, w.R, q["sizes"]["C"])
    # B = 0 with room: tau = max load, nothing moves
    w, res, ref = _quota_pair(base, 0, 8 * base.SK)
    assert ref["plan"]["tau"] == ref["plan"]["L"].max() and ref["plan"]["replicas"] == []
    gu.check_plan(res["plan_fields"], ref["plan"], w.P)
    gu.check_align(res, ref, w.R, res["sizes"]["C"])
    # S = 0
    w = base.with_(S=0)
    shape = gu.shape_of(w, tau_max=0)
    import load_balanced_token_amd as lbt
    path = lbt.Path(shape)
    buf = path.alloc()
    counts = t.zeros(w.R, w.E, dtype=t.int32, device="cuda")
    path.plan_quota(counts, buf["plan"], buf["status"])
    t.cuda.synchronize()
    pf = lbt.plan_fields(gu.d2h(buf["plan"]), path.sizes, w.R, w.E)
    assert pf["hdr"][gu.HDR_TAU] == 0 and pf["hdr"][gu.HDR_N_PIECES] == 0
    assert int(buf["status"].item()) == 0


def test_quota_inconsistent_counts_flagged():
    import load_balanced_token_amd as lbt
    t = gu.torch()
    w = WORKLOADS["tiny"]
    path = lbt.Path(gu.shape_of(w, tau_max=2 * w.SK))
    buf = path.alloc()
    counts = t.ones(w.R, w.E, dtype=t.int32, device="cuda")     # sums to R*E != R*S*K
    path.plan_quota(counts, buf["plan"], buf["status"])
    t.cuda.synchronize()
    assert int(buf["status"].item()) & lbt.ST_BADCOUNT


@pytest.mark.parametrize("E,R,S,B,x,layer", [
    (130, 65, 24, 2, 4, 0),    # tau* = 470 > S*K = 192: found inside the first batch
    (130, 65, 24, 1, 8, 0),    # tau* = 1353: more than 1024 candidates, found in the second batch
    (130, 65, 24, 1, 8, 1),    # no qualifying tau up to 8*S*K: both batches, tau = tau_max
    (256, 128, 16, 2, 2, 0),   # R = 128: tau* = 142
    (256, 128, 16, 2, 2, 1),   # tau* = 210
    (256, 128, 16, 1, 2, 0),   # infeasible: the whole range searched, remote fallback
])
def test_quota_search_past_one_wave_of_ranks(E, R, S, B, x, layer):
    """More than 64 ranks, where the wave-per-candidate first stage is skipped
    and the per-thread batches walk the ranks: thresholds above S*K, a search
    longer than one batch of 1024 candidates, and a range with no qualifying
    threshold; plan and placement bit-exact with the oracle."""
    w = WORKLOADS["dsv3"].with_(E=E, R=R, K=8, S=S, H=64, blk=8)
    w, res, ref = _quota_pair(w, B, x * w.SK, layer)
    print(f"[quota] R={R} B={B} tau_max={x}SK layer={layer}: tau={ref['plan']['tau']}", flush=True)
    assert ref["plan"]["tau"] > w.SK
    gu.check_route(res, ref)
    gu.check_plan(res["plan_fields"], ref["plan"], w.P)
    gu.check_align(res, ref, w.R, res["sizes"]["C"])
    _full_move_check(w, res, ref, activations(w, layer))
