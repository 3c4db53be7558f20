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
N_CASES = 120


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
