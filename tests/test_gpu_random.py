"""Seeded random small shapes through the whole path (route, either planner,
align, dispatch, combine) against the oracle: integer outputs bit-exact,
gates and combine within their tolerances.  The shapes mix what the named
workloads keep fixed: ranks 1-16, 1-32 home experts per rank, K up to 24,
ragged S, alignment blocks 1-128, 0-4 slots, softmax or sigmoid gates,
renormalisation, a selection bias, skewed or flat routing, tau_max = S*K or
2*S*K."""
import numpy as np
import pytest

from workloads import WORKLOADS, activations
from tests import gpu_util as gu
from tests.test_gpu_parity import _full_move_check

pytestmark = pytest.mark.gpu
N_CASES = 600


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    R = int(rng.choice([1, 2, 3, 4, 8, 16]))
    wide = rng.random() < 0.1                      # now and then many experts and a large K
    E = R * int(rng.integers(9, 33) if wide else rng.integers(1, 9))
    K = int(rng.integers(1, min(E, 24 if wide else 8) + 1))
    S = int(rng.integers(1, 300))
    blk = int(rng.choice([1, 2, 4, 8, 16, 64, 128]))
    B = int(rng.integers(0, 5))
    H = int(rng.choice([8, 64, 136]))
    score = "softmax" if rng.random() < 0.3 else "sigmoid"
    renorm = int(rng.random() < 0.3)
    skew = float(rng.random() * 3.0)
    hot = -np.log(np.arange(1, E + 1, dtype=np.float64))[rng.permutation(E)]
    logits = (rng.standard_normal((R * S, E)) + skew * hot).astype(np.float32)
    sel_bias = (0.5 * rng.standard_normal(E)).astype(np.float32) if rng.random() < 0.3 else None
    planner = "quota" if seed % 2 else "fixed"
    tau_max = int(rng.choice([1, 2])) * S * K
    w = WORKLOADS["tiny"].with_(E=E, K=K, R=R, S=S, H=H, B=B, blk=blk, score=score)
    return w, logits, sel_bias, renorm, planner, tau_max


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shapes(seed):
    w, logits, sb, renorm, planner, tau_max = random_case(seed)
    print(f"[random] seed {seed}: E={w.E} R={w.R} K={w.K} S={w.S} blk={w.blk} B={w.B} H={w.H} "
          f"{w.score} renorm={renorm} bias={sb is not None} {planner} tau_max={tau_max}", flush=True)
    res = gu.run_front(gu.shape_of(w, renorm=renorm, tau_max=tau_max), logits, sel_bias=sb,
                       planner=planner)
    ref = gu.run_oracle(w, logits, sel_bias=sb, renorm=bool(renorm), planner=planner,
                        tau_max=tau_max)
    gu.check_route(res, ref)
    gu.check_plan(res["plan_fields"], ref["plan"], w.P)
    gu.check_align(res, ref, w.R, res["sizes"]["C"])
    _full_move_check(w, res, ref, activations(w, 0))


@pytest.mark.parametrize("seed", range(0, N_CASES, 4))
def test_random_shapes_training(seed):
    """The training-side kernels on the same random shapes: prefetch and
    reduce_grad bit-exact, the combine and dispatch gradients within their
    tolerances."""
    import oracle
    from tests.test_gpu_train import _check_combine_bwd, DX_RTOL
    from workloads import random_expert_out
    t = gu.torch()
    w, logits, sb, renorm, planner, tau_max = random_case(seed)
    res = gu.run_front(gu.shape_of(w, renorm=renorm, tau_max=tau_max), logits, sel_bias=sb,
                       planner=planner)
    ref = gu.run_oracle(w, logits, sel_bias=sb, renorm=bool(renorm), planner=planner,
                        tau_max=tau_max)
    rng = np.random.default_rng(seed)
    path, C = res["path"], res["sizes"]["C"]
    if w.B > 0:
        row_bytes = 16 * int(rng.integers(1, 300))
        W = rng.integers(0, 256, size=(w.E, row_bytes), dtype=np.uint8)
        slots0 = np.full((w.R, w.B, row_bytes), 0x3C, np.uint8)
        Sd = t.from_numpy(slots0).cuda()
        path.prefetch_weights(res["dev"]["plan"], t.from_numpy(W).cuda(), Sd)
        row = 4 * int(rng.integers(1, 300))
        G = rng.standard_normal((w.E, row)).astype(np.float32)
        SG = rng.standard_normal((w.R, w.B, row)).astype(np.float32)
        Gd, SGd = t.from_numpy(G).cuda(), t.from_numpy(SG).cuda()
        path.reduce_grad(res["dev"]["plan"], SGd, Gd)
        t.cuda.synchronize()
        assert np.array_equal(Sd.cpu().numpy(), oracle.prefetch_weights(ref["plan"], W, slots0))
        g2, sg2 = oracle.reduce_grad(ref["plan"], SG, G)
        assert np.array_equal(Gd.cpu().numpy(), g2) and np.array_equal(SGd.cpu().numpy(), sg2)
    _check_combine_bwd(w, res, ref, bool(seed % 8 == 4))
    d_recv = random_expert_out(w, w.R * C, seed=seed)
    dx = t.empty((w.N, w.H), dtype=t.float32, device="cuda")
    path.dispatch_bwd(gu.h2d(d_recv), res["dev"]["slot"], dx)
    t.cuda.synchronize()
    want, mag = oracle.dispatch_bwd(lambda r: d_recv[r], ref["align"]["slot"], w.K, w.N)
    assert (np.abs(dx.cpu().numpy().astype(np.float64) - want) <= DX_RTOL * mag + 1e-30).all()


def small_case(seed):
    """At most 32 tokens (the single-launch route with its own tile scan)."""
    rng = np.random.default_rng(5000 + seed)
    R = int(rng.choice([1, 2, 4, 8, 16, 32]))
    S = int(rng.integers(1, 32 // R + 1))
    E = R * int(rng.integers(1, 512 // R + 1)) if rng.random() < 0.5 else R * int(rng.integers(1, 9))
    E = min(E, 512)
    K = int(rng.integers(1, min(E, 64) + 1))
    blk = int(rng.choice([1, 3, 4, 16, 128]))
    B = int(rng.integers(0, 4))
    score = "softmax" if rng.random() < 0.3 else "sigmoid"
    logits = rng.standard_normal((R * S, E)).astype(np.float32)
    planner = "quota" if seed % 2 else "fixed"
    w = WORKLOADS["tiny"].with_(E=E, K=K, R=R, S=S, H=64, B=B, blk=blk, score=score)
    return w, logits, planner


def _front_matches_separate_calls(w, logits, sel_bias=None):
    """lbt_front (route, fixed-rule plan and align in one launch: one token
    per wave up to 16 tokens, four per wave above; padding sentinels four
    rows per store when blk is a multiple of 4, else one) against
    lbt_route_topk + lbt_plan_balance + lbt_align_sort, every output word."""
    import load_balanced_token_amd as lbt
    t = gu.torch()
    path = lbt.Path(gu.shape_of(w))
    a, b = path.alloc(), path.alloc()
    for buf in (a, b):
        del buf["recv"], buf["y"]
        buf["sorted_ids"].fill_(-5)
        buf["slot"].fill_(-5)
        buf["status"].zero_()
    lg = gu.h2d(logits)
    sb = None if sel_bias is None else gu.h2d(np.asarray(sel_bias, np.float32))
    path.route_topk(lg, a["ids"], a["gates"], a["counts"], a["work"], sel_bias=sb)
    path.plan_balance(a["counts"], a["plan"], a["status"])
    path.align_sort(a["ids"], a["work"], a["plan"], a["slot"], a["sorted_ids"], a["block_wrow"],
                    a["block_expert"], a["status"])
    path.front(lg, b, sel_bias=sb)
    t.cuda.synchronize()
    for k in ("ids", "gates", "counts", "plan", "status", "slot", "sorted_ids", "block_wrow",
              "block_expert"):
        assert t.equal(a[k], b[k]), f"front: {k}"


@pytest.mark.parametrize("seed", range(24))
def test_small_batches(seed):
    w, logits, planner = small_case(seed)
    assert 1 <= w.N <= 32 and w.R * w.E <= 16384
    print(f"[small] seed {seed}: E={w.E} R={w.R} K={w.K} S={w.S} blk={w.blk} B={w.B} {planner}",
          flush=True)
    res = gu.run_front(gu.shape_of(w), logits, planner=planner)
    ref = gu.run_oracle(w, logits, planner=planner)
    gu.check_route(res, ref)
    gu.check_plan(res["plan_fields"], ref["plan"], w.P)
    gu.check_align(res, ref, w.R, res["sizes"]["C"])
    _full_move_check(w, res, ref, activations(w, 0))
    _front_matches_separate_calls(w, logits)


def medium_case(seed):
    """33 to 1024 tokens (past the one-launch front) with at most 8192 pairs
    and R * ceil(S / 32) * E <= 8192, blocks that are not all powers of
    two."""
    rng = np.random.default_rng(7000 + seed)
    while True:
        R = int(rng.choice([1, 2, 4, 8, 16, 32]))
        S = int(rng.integers(max(1, 33 // R + 1), 1024 // R + 1))
        n_sub = R * -(-S // 32)
        e_max = min(512, 8192 // n_sub) // R
        if e_max < 1:
            continue
        E = R * int(rng.integers(1, e_max + 1))
        K = int(rng.integers(1, min(E, 64, 8192 // (R * S)) + 1))
        break
    blk = int(rng.choice([12, 16, 64, 96, 128]))
    B = int(rng.integers(0, 4))
    score = "softmax" if rng.random() < 0.3 else "sigmoid"
    logits = rng.standard_normal((R * S, E)).astype(np.float32)
    w = WORKLOADS["tiny"].with_(E=E, K=K, R=R, S=S, H=64, B=B, blk=blk, score=score)
    return w, logits


@pytest.mark.parametrize("seed", range(40))
def test_medium_batches(seed):
    """Batches just past the one-launch front, whose sub-tile histograms fit
    the fused column scan + plan launch (lbt_front: route, scan + plan,
    align): against the oracle, and lbt_front word for word against the
    separate calls (route + column scan, plan, align)."""
    w, logits = medium_case(seed)
    assert 33 <= w.N <= 1024 and w.N * w.K <= 8192
    print(f"[medium] seed {seed}: E={w.E} R={w.R} K={w.K} S={w.S} blk={w.blk} B={w.B}",
          flush=True)
    res = gu.run_front(gu.shape_of(w), logits)
    ref = gu.run_oracle(w, logits)
    gu.check_route(res, ref)
    gu.check_plan(res["plan_fields"], ref["plan"], w.P)
    gu.check_align(res, ref, w.R, res["sizes"]["C"])
    _front_matches_separate_calls(w, logits)


@pytest.mark.parametrize("E,K,S,score,bias", [
    (256, 8, 40, "sigmoid", False), (256, 8, 2, "sigmoid", True), (384, 8, 40, "sigmoid", True),
    (256, 24, 40, "softmax", False), (512, 64, 4, "sigmoid", True), (384, 16, 1, "softmax", False),
    (256, 5, 3, "sigmoid", False)])
def test_ties_wide_rows(E, K, S, score, bias):
    """Rows of 256-512 experts whose keys take a few values (many exact ties,
    signed zeros, also in the selection bias), so equal keys meet inside
    one lane's run of experts and across lanes; every third row has its
    K + 4 first experts tied at the top, and every third row K distinct top
    keys on consecutive experts, so one lane wins every round and its short
    sorted list runs dry and refills.  ids must follow the oracle's order
    (key descending, lower expert on equal keys) exactly; up to 32 tokens the
    fused front must match the separate calls word for word."""
    w = WORKLOADS["dsv3"].with_(E=E, K=K, R=8, S=S, H=64, B=4, blk=16, score=score)
    print(f"[ties] E={E} K={K} S={S} {score} bias={bias}", flush=True)
    rng = np.random.default_rng(E * 1000 + K * 10 + S)
    logits = (rng.integers(-2, 3, size=(w.N, E)) * 0.5).astype(np.float32)
    logits[rng.random(logits.shape) < 0.2] = np.float32(-0.0)
    logits[0::3, :K + 4] = 3.0
    logits[1::3, 20:20 + K] = 2.0 + 0.125 * np.arange(K, dtype=np.float32)
    sb = None
    if bias:
        sb = (rng.integers(-1, 2, size=E) * 0.5).astype(np.float32)
        sb[rng.random(E) < 0.2] = np.float32(-0.0)
    res = gu.run_front(gu.shape_of(w), logits, sel_bias=sb)
    ref = gu.run_oracle(w, logits, sel_bias=sb)
    gu.check_route(res, ref)
    gu.check_plan(res["plan_fields"], ref["plan"], w.P)
    gu.check_align(res, ref, w.R, res["sizes"]["C"])
    if w.N <= 32:
        _front_matches_separate_calls(w, logits, sb)


@pytest.mark.parametrize("planner", ["fixed", "quota"])
@pytest.mark.parametrize("blk", [3, 12, 96])
def test_block_sizes_not_powers_of_two(blk, planner):
    """Alignment blocks that are not powers of two (segment padding by
    division rather than by mask), DSV3 routing at S = 100."""
    from workloads import router_logits
    w = WORKLOADS["dsv3"].with_(S=100, H=64, blk=blk, B=4)
    tau_max = 2 * w.SK if planner == "quota" else 0
    print(f"[random] blk={blk} {planner}", flush=True)
    logits = router_logits(w, 0)
    res = gu.run_front(gu.shape_of(w, tau_max=tau_max), logits, planner=planner)
    ref = gu.run_oracle(w, logits, planner=planner, tau_max=tau_max)
    gu.check_route(res, ref)
    gu.check_plan(res["plan_fields"], ref["plan"], w.P)
    gu.check_align(res, ref, w.R, res["sizes"]["C"])
    _full_move_check(w, res, ref, activations(w, 0))
