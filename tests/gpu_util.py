"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare every output with the oracle run on the same seeded inputs."""
import numpy as np

import oracle
import load_balanced_token_amd as lbt
from load_balanced_token_amd.binding import (HDR_N_PIECES, HDR_MAX_T, HDR_MAX_L,
                                             HDR_TOTAL_OVERFLOW, HDR_N_DEFICIT_RANKS,
                                             HDR_N_OVERFLOW_RANKS, HDR_N_OVERFLOW_EXPERTS,
                                             HDR_STATUS, HDR_P, HDR_TAU, HDR_MAX_REPLICAS,
                                             HDR_FEASIBLE, HDR_LOCAL)

GATE_RTOL = 1e-6       # gates vs the fp64 oracle (relative)
COMBINE_RTOL = 1e-6    # |y - y_ref| <= 1e-6 * sum_k |g * out|


def torch():
    import torch as _t
    return _t


def shape_of(w, cap=0, renorm=0, tau_max=0):
    return lbt.Shape(E=w.E, K=w.K, R=w.R, S=w.S, H=w.H, B=w.B, blk=w.blk,
                     score_fn=lbt.SOFTMAX if w.score == "softmax" else lbt.SIGMOID,
                     renorm=renorm, cap=cap, tau_max=tau_max)


def oracle_score(w):
    return oracle.SOFTMAX if w.score == "softmax" else oracle.SIGMOID


def h2d(a):
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return t.from_numpy(a).cuda()


def d2h(t_):
    a = t_.cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a


def run_front(shape, logits, sel_bias=None, planner="fixed"):
    """route_topk + plan (plan_balance or plan_quota) + align_sort on the GPU;
    host copies."""
    t = torch()
    path = lbt.Path(shape)
    buf = path.alloc()
    del buf["recv"], buf["y"]
    buf["status"].zero_()
    lg = h2d(logits)
    sb = None if sel_bias is None else h2d(np.asarray(sel_bias, np.float32))
    path.route_topk(lg, buf["ids"], buf["gates"], buf["counts"], buf["work"], sel_bias=sb)
    plan = path.plan_balance if planner == "fixed" else path.plan_quota
    plan(buf["counts"], buf["plan"], buf["status"])
    path.align_sort(buf["ids"], buf["work"], buf["plan"], buf["slot"], buf["sorted_ids"],
                    buf["block_wrow"], buf["block_expert"], buf["status"])
    t.cuda.synchronize()
    out = {k: d2h(v) for k, v in buf.items()}
    out["plan_fields"] = lbt.plan_fields(out["plan"], path.sizes, shape.R, shape.E)
    out["sizes"] = path.sizes
    out["path"] = path
    out["dev"] = buf
    return out


def run_oracle(w, logits, sel_bias=None, B=None, blk=None, cap=0, renorm=False, planner="fixed",
               tau_max=0):
    ids, gates = oracle.route_topk(logits, w.K, oracle_score(w), sel_bias=sel_bias, renorm=renorm)
    counts = oracle.load_matrix(ids, w.R, w.S, w.E)
    B_ = w.B if B is None else B
    blk_ = w.blk if blk is None else blk
    if planner == "fixed":
        plan = oracle.plan_balance(counts, w.K, w.S, B_, blk_, cap, tau_max)
    else:
        plan = oracle.plan_quota(counts, w.K, w.S, B_, blk_, tau_max, cap)
    al = oracle.align_sort(ids, plan)
    return {"ids": ids, "gates": gates, "counts": counts, "plan": plan, "align": al}


def check_route(g, o):
    assert np.array_equal(g["ids"], o["ids"]), "ids differ"
    ref = o["gates"]
    err = np.abs(g["gates"].astype(np.float64) - ref)
    assert (err <= GATE_RTOL * np.abs(ref)).all(), f"gates: max rel err {(err / np.abs(ref)).max()}"
    assert np.array_equal(g["counts"], o["counts"]), "counts differ"


def check_plan(pf, op, P):
    E, R, SK = op["E"], op["R"], op["SK"]
    nh = E // R
    for gk, ok in (("T", "T"), ("h", "h"), ("O", "O"), ("home_row", "home_row"), ("L", "L"),
                   ("def", "deficit"), ("D", "D"), ("n_rows_padded", "n_rows_padded"),
                   ("n_slots", "n_slots"), ("n_remote", "n_remote")):
        assert np.array_equal(pf[gk], op[ok]), f"plan field {gk} differs"
    assert np.array_equal(pf["n_seg"], nh + op["n_slots"] + op["n_remote"])
    for r in range(R):
        segs = op["segments"][r]
        n = len(segs)
        assert pf["seg_expert"][r, :n].tolist() == [s["expert"] for s in segs], f"rank {r}"
        assert pf["seg_wrow"][r, :n].tolist() == [s["wrow"] for s in segs], f"rank {r}"
        assert pf["seg_count"][r, :n].tolist() == [s["count"] for s in segs], f"rank {r}"
        assert pf["seg_start"][r, :n].tolist() == [s["start"] for s in segs], f"rank {r}"
        assert (pf["seg_expert"][r, n:] == -1).all() and (pf["seg_wrow"][r, n:] == -1).all()
        assert (pf["seg_count"][r, n:] == 0).all()
        assert (pf["seg_start"][r, n:] == op["n_rows_padded"][r]).all()
    reps = op["replicas"]
    nP = len(reps)
    hdr = pf["hdr"]
    assert hdr[HDR_N_PIECES] == nP
    for key, field in (("expert", "piece_expert"), ("rank", "piece_rank"), ("count", "piece_count"),
                       ("line", "piece_line"), ("row", "piece_row")):
        assert pf[field][:nP].tolist() == [rp[key] for rp in reps], field
    assert (pf["piece_expert"][nP:] == -1).all() and (pf["piece_count"][nP:] == 0).all()
    assert hdr[HDR_MAX_T] == op["T"].max()
    assert hdr[HDR_MAX_L] == op["L"].max()
    assert hdr[HDR_TOTAL_OVERFLOW] == op["o"].sum()
    assert hdr[HDR_N_DEFICIT_RANKS] == (op["deficit"] > 0).sum()
    assert hdr[HDR_N_OVERFLOW_RANKS] == (op["L"] > op["tau"]).sum()
    assert hdr[HDR_N_OVERFLOW_EXPERTS] == (op["o"] > 0).sum()
    assert hdr[HDR_P] == P
    assert hdr[HDR_STATUS] == 0
    assert hdr[HDR_TAU] == op["tau"]
    assert hdr[HDR_MAX_REPLICAS] == op["max_replicas"]
    assert hdr[HDR_FEASIBLE] == int(op["max_replicas"] <= op["B"])
    # locality counts (quota plans; zero under the fixed rule)
    assert hdr[HDR_LOCAL] == int(op.get("local", False))
    assert np.array_equal(pf["home_local"], op["home_local"]), "home_local differs"
    assert pf["piece_local"][:nP].tolist() == [rp.get("local", 0) for rp in reps], "piece_local"
    assert (pf["piece_local"][nP:] == 0).all()


def check_align(g, o, R, C):
    al = o["align"]
    assert np.array_equal(g["slot"][: al["slot"].size], al["slot"]), "slot differs"
    nrp = o["plan"]["n_rows_padded"]
    for r in range(R):
        lo = r * C
        assert np.array_equal(g["sorted_ids"][lo: lo + nrp[r]], al["sorted_ids"][lo: lo + nrp[r]]), \
            f"sorted_ids rank {r}"
    assert np.array_equal(g["block_wrow"], al["block_wrow"]), "block_wrow differs"
    assert np.array_equal(g["block_expert"], al["block_expert"]), "block_expert differs"
    assert g["status"][0] == 0
