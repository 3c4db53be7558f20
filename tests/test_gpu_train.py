"""GPU parity of the training side: replica weight prefetch, reduce_grad,
combine backward and dispatch backward against the oracle.

Bit-exact: prefetched slots, reduce_grad (same fp32 additions in the same
order), the bf16 expert-output gradient rows.  Gate gradients: the device sums
in fp64 and rounds once to fp32, so |got - ref| <= 2^-24 |ref| + 1e-12 *
sum_h |dy * out| (fp64 error of a 7168-term sum is below 1e-12 of that
scale).  Dispatch backward: fp32 sum of K rows, |got - ref| <= 1e-6 *
sum_k |d_recv| (K - 1 roundings of 2^-24 each)."""
import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, router_logits, random_expert_out
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

GG_REL = 2.0 ** -24
GG_ABS = 1e-12
DX_RTOL = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _front(w, planner="fixed", tau_max=0, cap=0):
    logits = router_logits(w, 0)
    res = gu.run_front(gu.shape_of(w, cap=cap, tau_max=tau_max), logits, planner=planner)
    ref = gu.run_oracle(w, logits, planner=planner, tau_max=tau_max, cap=cap)
    gu.check_align(res, ref, w.R, res["sizes"]["C"]) if cap == 0 else None
    return res, ref


# --------------------------------------------------------------------------- prefetch
@pytest.mark.parametrize("name,B,planner,row_bytes", [
    ("tiny", 2, "fixed", 3072), ("decode128", 3, "fixed", 32768 * 3 + 16),
    ("decode128", 3, "quota", 1040), ("dsv3", 32, "fixed", 4096), ("wideep", 4, "fixed", 65552)])
def test_prefetch_parity(name, B, planner, row_bytes):
    t = gu.torch()
    w = WORKLOADS[name].with_(B=B)
    res, ref = _front(w, planner)
    rng = np.random.default_rng(1)
    W = rng.integers(0, 256, size=(w.E, row_bytes), dtype=np.uint8)
    slots0 = np.full((w.R, w.B, row_bytes), 0xA5, np.uint8)
    Wd, Sd = t.from_numpy(W).cuda(), t.from_numpy(slots0).cuda()
    res["path"].prefetch_weights(res["dev"]["plan"], Wd, Sd)
    t.cuda.synchronize()
    want = oracle.prefetch_weights(ref["plan"], W, slots0)
    assert np.array_equal(Sd.cpu().numpy(), want)
    n_slotted = len(oracle.prefetch_slots(ref["plan"]))
    assert n_slotted == int(res["plan_fields"]["n_slots"].sum()) and n_slotted > 0
    pw = res["plan_fields"]["piece_wrow"][: len(ref["plan"]["replicas"])]
    assert pw.tolist() == [rp["wrow"] for rp in ref["plan"]["replicas"]]


def test_prefetch_full_size_weight_rows():
    """DSV3 shape, H' = 2048 bf16 weights (29.4 MB per expert): every slotted
    replica's slot equals its home row, compared on the device."""
    t = gu.torch()
    w = WORKLOADS["dsv3"]
    res, ref = _front(w)
    row = 7168 * 2048
    W = t.randint(-32768, 32767, (w.E, row), dtype=t.int16, device="cuda")
    S = t.zeros((w.R, w.B, row), dtype=t.int16, device="cuda")
    res["path"].prefetch_weights(res["dev"]["plan"], W, S)
    t.cuda.synchronize()
    m = oracle.prefetch_slots(ref["plan"])
    assert len(m) == 38
    for (d, j), e in m.items():
        assert t.equal(S[d, j], W[e]), (d, j, e)
    used = np.zeros((w.R, w.B), bool)
    for (d, j) in m:
        used[d, j] = True
    for d, j in zip(*np.nonzero(~used)):
        assert int(S[d, j].abs().max().item()) == 0
    del W, S


# --------------------------------------------------------------------------- reduce_grad
@pytest.mark.parametrize("name,B,planner,row", [
    ("tiny", 2, "fixed", 1000), ("decode128", 3, "fixed", 4100), ("decode128", 1, "quota", 256),
    ("dsv3", 32, "fixed", 9000), ("wideep", 4, "fixed", 64)])
def test_reduce_grad_parity(name, B, planner, row):
    t = gu.torch()
    w = WORKLOADS[name].with_(B=B)
    res, ref = _front(w, planner, tau_max=2 * w.SK if planner == "quota" else 0)
    rng = np.random.default_rng(2)
    G = rng.standard_normal((w.E, row)).astype(np.float32)
    SG = rng.standard_normal((w.R, w.B, row)).astype(np.float32) * 1e3
    Gd, SGd = t.from_numpy(G).cuda(), t.from_numpy(SG).cuda()
    res["path"].reduce_grad(res["dev"]["plan"], SGd, Gd)
    t.cuda.synchronize()
    g2, sg2 = oracle.reduce_grad(ref["plan"], SG, G)
    assert np.array_equal(Gd.cpu().numpy(), g2)
    assert np.array_equal(SGd.cpu().numpy(), sg2)
    # a second call finds the used slots already cleared: grads unchanged
    res["path"].reduce_grad(res["dev"]["plan"], SGd, Gd)
    t.cuda.synchronize()
    assert np.array_equal(Gd.cpu().numpy(), g2)


# --------------------------------------------------------------------------- backward
def _check_combine_bwd(w, res, ref, dy_bf16):
    t = gu.torch()
    path, C = res["path"], res["sizes"]["C"]
    rows = w.R * C
    out_h = random_expert_out(w, rows)
    rng = np.random.default_rng(3)
    dy32 = rng.standard_normal((w.N, w.H)).astype(np.float32)
    if dy_bf16:
        dy_bits = oracle.f32_to_bf16_rne(dy32)
        dy32 = oracle.bf16_to_f64(dy_bits).astype(np.float32)
        dy_d = gu.h2d(dy_bits)
    else:
        dy_d = gu.h2d(dy32)
    gates32 = ref["gates"].astype(np.float32)
    d_out = t.full((rows, w.H), 0x7F7F, dtype=t.int16, device="cuda")
    d_g = t.empty((w.N, w.K), dtype=t.float32, device="cuda")
    path.combine_bwd(gu.h2d(out_h), res["dev"]["slot"], gu.h2d(gates32), dy_d, d_out, d_g)
    t.cuda.synchronize()
    slot = ref["align"]["slot"]
    want_rows, want_g, mag = oracle.combine_bwd(lambda r: out_h[r], slot, gates32, dy32, w.K)
    got = gu.d2h(d_out)
    ok = slot >= 0
    assert np.array_equal(got[slot[ok]], want_rows[ok]), "d_out rows differ"
    untouched = np.ones(rows, bool)
    untouched[slot[ok]] = False
    assert (got[untouched] == 0x7F7F).all(), "rows no pair maps to were written"
    gg = d_g.cpu().numpy().astype(np.float64)
    err = np.abs(gg - want_g)
    assert (err <= GG_REL * np.abs(want_g) + GG_ABS * mag).all(), \
        f"d_gates max err {err.max()}"


@pytest.mark.parametrize("name,S,dy_bf16", [("tiny", None, False), ("tiny", None, True),
                                            ("dsv3", 256, False), ("dsv3", 128, True),
                                            ("decode16", None, False)])
def test_combine_bwd_parity(name, S, dy_bf16):
    w = WORKLOADS[name]
    if S is not None:
        w = w.with_(S=S)
    print(f"[train] combine_bwd {name} S={w.S} dy_bf16={dy_bf16}", flush=True)
    res, ref = _front(w)
    _check_combine_bwd(w, res, ref, dy_bf16)


def test_combine_bwd_ragged_H_and_K3():
    w = WORKLOADS["tiny"].with_(H=7176, K=3)
    res, ref = _front(w)
    _check_combine_bwd(w, res, ref, False)


def test_combine_bwd_with_dropped_pairs():
    """A capacity too small for the plan: dropped pairs (slot -1) get gate
    gradient 0 and write no row."""
    t = gu.torch()
    w = WORKLOADS["tiny"]
    logits = router_logits(w, 0)
    res = gu.run_front(gu.shape_of(w, cap=128), logits)
    slot = res["slot"][: w.P].astype(np.int64)     # the slot map is combine_bwd's input
    assert (slot < 0).any()
    path, C = res["path"], res["sizes"]["C"]
    rows = w.R * C
    out_h = random_expert_out(w, rows)
    dy32 = np.random.default_rng(4).standard_normal((w.N, w.H)).astype(np.float32)
    _, gates = oracle.route_topk(logits, w.K, gu.oracle_score(w))
    gates32 = gates.astype(np.float32)
    d_out = t.full((rows, w.H), 0x7F7F, dtype=t.int16, device="cuda")
    d_g = t.empty((w.N, w.K), dtype=t.float32, device="cuda")
    path.combine_bwd(gu.h2d(out_h), res["dev"]["slot"], gu.h2d(gates32), gu.h2d(dy32), d_out, d_g)
    t.cuda.synchronize()
    gg = d_g.cpu().numpy().reshape(-1)
    assert (gg[slot < 0] == 0).all()
    rows_of = lambda r: out_h[np.where(r < 0, 0, r)]  # noqa: E731
    want_rows, want_g, mag = oracle.combine_bwd(rows_of, slot, gates32, dy32, w.K)
    ok = slot >= 0
    got = gu.d2h(d_out)
    assert np.array_equal(got[slot[ok]], want_rows[ok])
    wg = want_g.reshape(-1)[ok]
    assert (np.abs(gg[ok] - wg) <= GG_REL * np.abs(wg) + GG_ABS * mag.reshape(-1)[ok]).all()


@pytest.mark.parametrize("name,S", [("tiny", None), ("dsv3", 256), ("decode128", None)])
def test_dispatch_bwd_parity(name, S):
    t = gu.torch()
    w = WORKLOADS[name]
    if S is not None:
        w = w.with_(S=S)
    res, ref = _front(w)
    path, C = res["path"], res["sizes"]["C"]
    d_recv = random_expert_out(w, w.R * C, seed=11)
    dx = t.empty((w.N, w.H), dtype=t.float32, device="cuda")
    path.dispatch_bwd(gu.h2d(d_recv), res["dev"]["slot"], dx)
    dxb = t.empty((w.N, w.H), dtype=t.int16, device="cuda")
    path.dispatch_bwd(gu.h2d(d_recv), res["dev"]["slot"], dxb)
    t.cuda.synchronize()
    want, mag = oracle.dispatch_bwd(lambda r: d_recv[r], ref["align"]["slot"], w.K, w.N)
    got = dx.cpu().numpy().astype(np.float64)
    assert (np.abs(got - want) <= DX_RTOL * mag + 1e-30).all()
    assert np.array_equal(gu.d2h(dxb), oracle.f32_to_bf16_rne(dx.cpu().numpy()))


@pytest.mark.parametrize("planner", ["fixed", "quota"])
def test_prefetch_and_reduce_grad_at_limits(planner):
    """R = E = 512 (one expert per rank, 510 replica segments, B = 2): the
    slot table at the library's size limits through prefetch and reduce_grad."""
    t = gu.torch()
    w = WORKLOADS["dsv3"].with_(E=512, R=512, K=8, S=4, H=64, B=2, blk=4)
    res, ref = _front(w, planner)
    rng = np.random.default_rng(5)
    W = rng.integers(0, 256, size=(w.E, 1040), dtype=np.uint8)
    slots0 = np.full((w.R, w.B, 1040), 0x5A, np.uint8)
    Sd = t.from_numpy(slots0).cuda()
    res["path"].prefetch_weights(res["dev"]["plan"], t.from_numpy(W).cuda(), Sd)
    G = rng.standard_normal((w.E, 260)).astype(np.float32)
    SG = rng.standard_normal((w.R, w.B, 260)).astype(np.float32)
    Gd, SGd = t.from_numpy(G).cuda(), t.from_numpy(SG).cuda()
    res["path"].reduce_grad(res["dev"]["plan"], SGd, Gd)
    t.cuda.synchronize()
    assert np.array_equal(Sd.cpu().numpy(), oracle.prefetch_weights(ref["plan"], W, slots0))
    g2, sg2 = oracle.reduce_grad(ref["plan"], SG, G)
    assert np.array_equal(Gd.cpu().numpy(), g2) and np.array_equal(SGd.cpu().numpy(), sg2)
    assert len(oracle.prefetch_slots(ref["plan"])) > 0
