"""lbt_align_sort_noalloc (the align step with the library's static workspace,
for callers that cannot allocate) against lbt_histogram + lbt_align_sort with
a caller workspace: bit for bit on two calls in a row, the second on a
smaller input, and its size limit."""
import ctypes

import numpy as np
import pytest

from workloads import WORKLOADS, router_logits
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _compare(w, layer, planner):
    """Route and plan with a caller workspace, then align both ways into
    outputs pre-filled alike; every output word must agree."""
    import load_balanced_token_amd as lbt
    t = gu.torch()
    path = lbt.Path(gu.shape_of(w, tau_max=2 * w.SK if planner == "quota" else 0))
    buf = path.alloc()
    del buf["recv"], buf["y"]
    buf["status"].zero_()
    lg = gu.h2d(router_logits(w, layer))
    path.route_topk(lg, buf["ids"], buf["gates"], buf["counts"], buf["work"])
    (path.plan_balance if planner == "fixed" else path.plan_quota)(buf["counts"], buf["plan"],
                                                                   buf["status"])
    outs = []
    for mode in ("workspace", "noalloc"):
        o = {k: t.full_like(buf[k], -7) for k in ("slot", "sorted_ids", "block_wrow",
                                                   "block_expert")}
        o["status"] = t.zeros(1, dtype=t.int32, device="cuda")
        if mode == "workspace":
            counts = t.empty_like(buf["counts"])
            work = t.full_like(buf["work"], -3)
            path.histogram(buf["ids"], counts, work, o["status"])
            path.align_sort(buf["ids"], work, buf["plan"], o["slot"], o["sorted_ids"],
                            o["block_wrow"], o["block_expert"], o["status"])
        else:
            path.align_sort_noalloc(buf["ids"], buf["plan"], o["slot"], o["sorted_ids"],
                                    o["block_wrow"], o["block_expert"], o["status"])
        outs.append(o)
    t.cuda.synchronize()
    for k in ("slot", "sorted_ids", "block_wrow", "block_expert", "status"):
        assert t.equal(outs[0][k], outs[1][k]), f"{w.name} S={w.S} {planner}: {k} differs"
    assert outs[1]["status"].item() == 0
    # and the oracle's placement
    ref = gu.run_oracle(w, router_logits(w, layer), planner=planner,
                        tau_max=2 * w.SK if planner == "quota" else 0)
    assert np.array_equal(gu.d2h(outs[1]["slot"]), ref["align"]["slot"])


def test_noalloc_matches_workspace_call_twice():
    """Two calls in a row on one GPU: the full DSV3 shape with the fixed
    rule, then a smaller input (S = 1000) with the quota planner's locality
    placement, which reuses the same static array."""
    print("[noalloc] dsv3 S=4096 fixed", flush=True)
    _compare(WORKLOADS["dsv3"], 0, "fixed")
    print("[noalloc] dsv3 S=1000 quota", flush=True)
    _compare(WORKLOADS["dsv3"].with_(S=1000), 1, "quota")


def test_noalloc_rejects_shapes_past_its_array():
    """A shape whose workspace exceeds the static array is refused on the
    host with LBT_EUNSUPPORTED, before any launch."""
    import load_balanced_token_amd as lbt
    L = lbt.lib()
    sh = lbt.Shape(E=512, K=8, R=64, S=8192, H=64, B=1, blk=1).c()
    P = ctypes.c_void_p
    rc = L.lbt_align_sort_noalloc(ctypes.byref(sh), P(0x1000), P(0x2000), P(0x3000), P(0x4000),
                                  P(0x5000), P(0x6000), None, None)
    from load_balanced_token_amd import binding
    assert rc == binding.EUNSUPPORTED
