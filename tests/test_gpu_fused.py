"""The fused calls against the calls they replace, every output word:
lbt_align_dispatch against lbt_align_sort + lbt_dispatch (both planners,
the quota plan's locality step, ragged tiles, dropped pairs, batches past
the one-launch limit) and lbt_front_dispatch against lbt_front +
lbt_dispatch (the one-launch front and dispatch up to 16 tokens, the front
then the dispatch up to 32, the fused scan + plan and align + dispatch
past that); the align outputs also against the oracle."""
import numpy as np
import pytest

from workloads import WORKLOADS, router_logits, activations
from tests import gpu_util as gu
from tests.test_gpu_random import medium_case

pytestmark = pytest.mark.gpu

SENT_ROW = 0x7F7F        # recv rows no call writes keep this pattern
SENT_ID = -5             # sorted_ids / slot words no call writes keep this


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _fresh(path, t):
    buf = path.alloc()
    del buf["y"]
    buf["recv"].fill_(SENT_ROW)
    buf["sorted_ids"].fill_(SENT_ID)
    buf["slot"].fill_(SENT_ID)
    buf["block_wrow"].fill_(SENT_ID)
    buf["block_expert"].fill_(SENT_ID)
    buf["status"].zero_()
    return buf


def _align_dispatch_case(w, logits, planner="fixed", tau_max=0, cap=0, check_oracle=True):
    import load_balanced_token_amd as lbt
    t = gu.torch()
    shape = gu.shape_of(w, cap=cap, tau_max=tau_max)
    path = lbt.Path(shape)
    a, b = _fresh(path, t), _fresh(path, t)
    lg = gu.h2d(logits)
    x = gu.h2d(activations(w, 0))
    path.route_topk(lg, a["ids"], a["gates"], a["counts"], a["work"])
    plan_fn = path.plan_balance if planner == "fixed" else path.plan_quota
    plan_fn(a["counts"], a["plan"], a["status"])
    b["status"].copy_(a["status"])
    path.align_sort(a["ids"], a["work"], a["plan"], a["slot"], a["sorted_ids"], a["block_wrow"],
                    a["block_expert"], a["status"])
    path.dispatch(x, a["slot"], a["recv"])
    path.align_dispatch(a["ids"], a["work"], a["plan"], x, b["slot"], b["sorted_ids"],
                        b["block_wrow"], b["block_expert"], b["recv"], b["status"])
    t.cuda.synchronize()
    for k in ("slot", "sorted_ids", "block_wrow", "block_expert", "status"):
        assert t.equal(a[k], b[k]), f"align_dispatch: {k}"
    assert t.equal(a["recv"], b["recv"]), "align_dispatch: recv"
    if check_oracle:
        ref = gu.run_oracle(w, logits, planner=planner, tau_max=tau_max, cap=cap)
        out = {k: gu.d2h(b[k]) for k in ("slot", "sorted_ids", "block_wrow", "block_expert",
                                          "status")}
        gu.check_align(out, ref, w.R, path.sizes["C"])
    return a, b


@pytest.mark.parametrize("case", [
    ("decode1", {}), ("decode16", {}), ("decode128", {}),
    ("decode16", {"H": 512, "S": 33}), ("decode16", {"H": 512, "S": 130}),
    ("decode16", {"H": 512, "S": 300, "R": 2}), ("tiny", {}), ("tiny", {"S": 5}),
    ("decode16", {"H": 136, "K": 3, "E": 40, "R": 4}),
    ("decode1", {"H": 512, "S": 64, "E": 512, "R": 16, "K": 16}),
    ("dsv3", {"S": 256, "H": 512}),          # 2048 tokens: the two launches
])
@pytest.mark.parametrize("planner", ["fixed", "quota"])
def test_align_dispatch_matches_separate_calls(case, planner):
    name, over = case
    w = WORKLOADS[name].with_(**over)
    print(f"[fused] align_dispatch {name} {over} {planner}", flush=True)
    _align_dispatch_case(w, router_logits(w, 1), planner=planner,
                         tau_max=2 * w.S * w.K if planner == "quota" else 0)


@pytest.mark.parametrize("seed", range(12))
def test_align_dispatch_medium_batches(seed):
    w, logits = medium_case(seed)
    planner = "quota" if seed % 2 else "fixed"
    print(f"[fused] medium seed {seed}: E={w.E} R={w.R} K={w.K} S={w.S} blk={w.blk} B={w.B} "
          f"{planner}", flush=True)
    _align_dispatch_case(w, logits, planner=planner,
                         tau_max=2 * w.S * w.K if planner == "quota" else 0)


def test_align_dispatch_dropped_pairs():
    """A capacity below the plan's need: pairs that do not fit get slot -1
    and no row, in both forms alike."""
    w = WORKLOADS["decode16"].with_(H=512)
    logits = router_logits(w, 0)
    ref = gu.run_oracle(w, logits)
    need = int(ref["plan"]["n_rows_padded"].max())
    cap = (need // w.blk - 1) * w.blk
    print(f"[fused] dropped pairs cap={cap}", flush=True)
    a, b = _align_dispatch_case(w, logits, cap=cap, check_oracle=False)
    slot = gu.d2h(b["slot"])
    assert (slot == -1).any() and (slot >= 0).any()


@pytest.mark.parametrize("case", [
    ("decode1", {}), ("decode1", {"S": 2}), ("decode1", {"E": 384}),
    ("decode1", {"S": 1, "R": 4, "E": 40, "K": 6, "H": 136}),
    ("decode1", {"S": 1, "R": 16, "E": 512, "K": 16, "H": 512}),
    ("tiny", {"S": 4}), ("tiny", {"S": 5, "R": 2}), ("tiny", {"S": 8}),
    ("decode16", {}), ("decode128", {}), ("tiny", {}),
    ("decode16", {"S": 40}), ("decode16", {"S": 33, "R": 4, "E": 40, "K": 6, "H": 136}),
    ("decode1", {"S": 100, "E": 512, "R": 16, "H": 512}),
    ("dsv3", {"S": 64}), ("dsv3", {"S": 160, "H": 512}),
])
def test_front_dispatch_matches_separate_calls(case):
    import load_balanced_token_amd as lbt
    t = gu.torch()
    name, over = case
    w = WORKLOADS[name].with_(**over)
    print(f"[fused] front_dispatch {name} {over}", flush=True)
    logits = router_logits(w, 2)
    path = lbt.Path(gu.shape_of(w))
    a, b = _fresh(path, t), _fresh(path, t)
    lg = gu.h2d(logits)
    x = gu.h2d(activations(w, 0))
    path.front(lg, a)
    path.dispatch(x, a["slot"], a["recv"])
    path.front_dispatch(lg, x, b)
    t.cuda.synchronize()
    for k in ("ids", "gates", "counts", "plan", "status", "slot", "sorted_ids", "block_wrow",
              "block_expert", "recv"):
        assert t.equal(a[k], b[k]), f"front_dispatch: {k}"
    ref = gu.run_oracle(w, logits)
    out = {k: gu.d2h(b[k]) for k in ("slot", "sorted_ids", "block_wrow", "block_expert",
                                      "status")}
    gu.check_align(out, ref, w.R, path.sizes["C"])


def test_front_dispatch_dropped_pairs():
    """The one-launch front + dispatch with a capacity below the plan's
    need: the same slots (-1 where a pair does not fit) and rows as lbt_front
    + lbt_dispatch."""
    import load_balanced_token_amd as lbt
    t = gu.torch()
    w = WORKLOADS["decode1"].with_(H=512)
    logits = router_logits(w, 0)
    ref = gu.run_oracle(w, logits)
    need = int(ref["plan"]["n_rows_padded"].max())
    cap = max(w.blk, (need // w.blk - 1) * w.blk)
    print(f"[fused] front_dispatch dropped pairs cap={cap}", flush=True)
    path = lbt.Path(gu.shape_of(w, cap=cap))
    a, b = _fresh(path, t), _fresh(path, t)
    lg = gu.h2d(logits)
    x = gu.h2d(activations(w, 0))
    path.front(lg, a)
    path.dispatch(x, a["slot"], a["recv"])
    path.front_dispatch(lg, x, b)
    t.cuda.synchronize()
    for k in ("ids", "gates", "counts", "plan", "status", "slot", "sorted_ids", "block_wrow",
              "block_expert", "recv"):
        assert t.equal(a[k], b[k]), f"front_dispatch: {k}"
    slot = gu.d2h(b["slot"])
    assert (slot == -1).any() and (slot >= 0).any()
