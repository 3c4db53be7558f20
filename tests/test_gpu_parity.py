"""GPU parity: the HIP path through the C ABI against the CPU oracle, element
by element on the same seeded inputs.  Integer outputs must be bit-exact;
gates within 1e-6 relative of the fp64 oracle; combine within
1e-6 * sum_k |g * out| (fp32 accumulation of K terms)."""
import glob
import json
import os

import numpy as np
import pytest

import oracle
from workloads import (WORKLOADS, router_logits, activations, activation_rows,
                       random_expert_out, f32_to_bf16_bits)
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "W*.json")))


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# --------------------------------------------------------------------------- golden
@pytest.mark.parametrize("path", GOLDEN, ids=[os.path.basename(p) for p in GOLDEN])
def test_gpu_matches_hand_examples(path):
    g = json.load(open(path))
    sh = g["shape"]
    import load_balanced_token_amd as lbt
    shape = lbt.Shape(E=sh["E"], K=sh["K"], R=sh["R"], S=sh["S"], H=8, B=sh["B"], blk=sh["blk"])
    res = gu.run_front(shape, np.array(g["logits"], np.float32))
    assert res["ids"].tolist() == g["ids"]
    assert res["counts"].tolist() == g["counts"]
    pf = res["plan_fields"]
    for key in ("T", "h", "O", "L", "D", "n_rows_padded", "n_slots", "n_remote", "home_row"):
        assert pf[key].tolist() == g[key], key
    assert pf["def"].tolist() == g["deficit"]
    assert res["sizes"]["C"] == g["C"]
    assert res["slot"].tolist() == g["slot"]
    C = g["C"]
    for r in range(sh["R"]):
        for want, got in zip(g["sorted_ids"][r], res["sorted_ids"][r * C:(r + 1) * C].tolist()):
            if want is not None:
                assert got == want
    assert res["block_wrow"].tolist() == g["block_wrow"]
    assert res["block_expert"].tolist() == g["block_expert"]


# --------------------------------------------------------------------------- configs
FRONT_CONFIGS = ["tiny", "dsv3", "wideep", "decode1", "decode16", "decode128", "kimi"]


@pytest.mark.parametrize("name", FRONT_CONFIGS)
def test_route_plan_align_parity(name):
    """Full-size route + plan + align against the oracle: ids, counts, the
    whole plan, slot, sorted_ids and block tables bit-exact."""
    w = WORKLOADS[name]
    print(f"[parity] {name} E={w.E} K={w.K} R={w.R} S={w.S}", flush=True)
    logits = router_logits(w, 0)
    res = gu.run_front(gu.shape_of(w), logits)
    ref = gu.run_oracle(w, logits)
    gu.check_route(res, ref)
    gu.check_plan(res["plan_fields"], ref["plan"], w.P)
    gu.check_align(res, ref, w.R, res["sizes"]["C"])


@pytest.mark.parametrize("name", ["dsv3", "decode128"])
def test_route_plan_align_parity_more_layers(name):
    w = WORKLOADS[name]
    for layer in (1, 2, 3):
        logits = router_logits(w, layer)
        res = gu.run_front(gu.shape_of(w), logits)
        ref = gu.run_oracle(w, logits)
        gu.check_route(res, ref)
        gu.check_plan(res["plan_fields"], ref["plan"], w.P)
        gu.check_align(res, ref, w.R, res["sizes"]["C"])


def _full_move_check(w, res, ref, x_bits, out_bits=None):
    """Dispatch + combine with every row compared (sizes that fit the host)."""
    t = gu.torch()
    path = res["path"]
    C = res["sizes"]["C"]
    recv = t.full((w.R * C, w.H), 0x7F7F, dtype=t.int16, device="cuda")   # sentinel fill
    x = gu.h2d(x_bits)
    path.dispatch(x, res["dev"]["slot"], recv)
    slot = ref["align"]["slot"]
    recv_h = gu.d2h(recv)
    want = oracle.dispatch(x_bits, slot, w.K, w.R, C)
    used = np.zeros(w.R * C, bool)
    used[slot] = True
    assert np.array_equal(recv_h[used], want[used]), "dispatched rows differ"
    assert (recv_h[~used] == 0x7F7F).all(), "dispatch touched rows it does not own"
    # combine of the identity expert and of a random expert output
    gates32 = ref["gates"].astype(np.float32)
    for src in ("identity", "random"):
        if src == "identity":
            out_d, out_h = recv, want
        else:
            out_h = random_expert_out(w, w.R * C) if out_bits is None else out_bits
            out_d = gu.h2d(out_h)
        y = t.empty((w.N, w.H), dtype=t.float32, device="cuda")
        path.combine(out_d, res["dev"]["slot"], gu.h2d(gates32), y)
        yref, mag = oracle.combine(lambda rows: out_h[rows], slot, gates32, w.K)
        err = np.abs(y.cpu().numpy().astype(np.float64) - yref)
        assert (err <= gu.COMBINE_RTOL * mag + 1e-30).all(), \
            f"combine ({src}) max err/mag {(err / np.maximum(mag, 1e-30)).max()}"
        if src == "identity":
            xs = oracle.bf16_to_f64(x_bits) * gates32.astype(np.float64).sum(axis=1)[:, None]
            assert (np.abs(y.cpu().numpy() - xs) <= gu.COMBINE_RTOL * np.abs(xs) + 1e-30).all()
    # bf16 output is the round-to-nearest-even of the fp32 accumulator
    yb = t.empty((w.N, w.H), dtype=t.int16, device="cuda")
    yf = t.empty((w.N, w.H), dtype=t.float32, device="cuda")
    path.combine(recv, res["dev"]["slot"], gu.h2d(gates32), yb)
    path.combine(recv, res["dev"]["slot"], gu.h2d(gates32), yf)
    assert np.array_equal(gu.d2h(yb), f32_to_bf16_bits(yf.cpu().numpy()))


@pytest.mark.parametrize("name,S", [("tiny", None), ("dsv3", 256), ("wideep", 64), ("kimi", 64)])
def test_dispatch_combine_parity_full_rows(name, S):
    w = WORKLOADS[name]
    if S is not None:
        w = w.with_(S=S)
    print(f"[parity] move {name} S={w.S} H={w.H}", flush=True)
    logits = router_logits(w, 0)
    res = gu.run_front(gu.shape_of(w), logits)
    ref = gu.run_oracle(w, logits)
    gu.check_align(res, ref, w.R, res["sizes"]["C"])
    _full_move_check(w, res, ref, activations(w, 0))


@pytest.mark.parametrize("name", ["dsv3", "wideep", "kimi", "moonep"])
def test_dispatch_combine_full_size_every_row(name):
    """Full-size dispatch + combine in the launch configuration the benchmark
    times.  Every one of the P dispatched rows is compared bitwise with its
    source row x[f // K] by device-side gathers (torch's, not the library's),
    every padding row below a rank's padded end keeps its sentinel, and every
    one of the N*H combine outputs (identity expert) is checked against
    x * sum_k g within 1e-6 * sum_k |g * out|; 256 sampled tokens are also
    recomputed by the oracle from the host.  At the DSV3 shape the combine
    is repeated on a random expert-output buffer, checked against the
    oracle's combine on sampled tokens."""
    t = gu.torch()
    w = WORKLOADS[name]
    print(f"[parity] full-size move {name}", flush=True)
    logits = router_logits(w, 0)
    res = gu.run_front(gu.shape_of(w), logits)
    ref = gu.run_oracle(w, logits)
    gu.check_align(res, ref, w.R, res["sizes"]["C"])
    path, C = res["path"], res["sizes"]["C"]
    x = t.empty((w.N, w.H), dtype=t.int16, device="cuda")
    from workloads.gen import X_CHUNK, x_chunk, device_normal_bf16
    for c in range((w.N + X_CHUNK - 1) // X_CHUNK):
        blk = x_chunk(w, 0, c)
        x[c * X_CHUNK: c * X_CHUNK + blk.shape[0]] = gu.h2d(blk)
    recv = t.full((w.R * C, w.H), 0x7F7F, dtype=t.int16, device="cuda")
    slot_d = res["dev"]["slot"]
    path.dispatch(x, slot_d, recv)
    y = t.empty((w.N, w.H), dtype=t.float32, device="cuda")
    gates32 = ref["gates"].astype(np.float32)
    g_d = gu.h2d(gates32)
    path.combine(recv, slot_d, g_d, y)
    t.cuda.synchronize()
    slot = ref["align"]["slot"]
    assert (slot >= 0).all()
    # every dispatched row, bitwise, in chunks of pairs
    step = 8192
    for f0 in range(0, w.P, step):
        f1 = min(w.P, f0 + step)
        got = recv.index_select(0, slot_d[f0:f1].long())
        src = t.arange(f0, f1, device="cuda", dtype=t.int64) // w.K
        assert t.equal(got, x.index_select(0, src)), f"dispatch rows of pairs [{f0}, {f1})"
    # every padding row below a rank's padded end is untouched
    sid = ref["align"]["sorted_ids"]
    pad_rows = np.nonzero(sid == w.P)[0]
    for i0 in range(0, pad_rows.size, step):
        rows = t.from_numpy(pad_rows[i0: i0 + step]).cuda()
        assert bool((recv.index_select(0, rows) == 0x7F7F).all()), "padding row written"
    assert (ref["plan"]["n_rows_padded"] <= C).all()
    # every combine output: y = x * sum_k g (gates are sigmoid or softmax, so positive)
    gsum = g_d.double().sum(dim=1)
    for t0 in range(0, w.N, 2048):
        t1 = min(w.N, t0 + 2048)
        xb = (x[t0:t1].int() & 0xFFFF) << 16
        want = xb.view(t.float32).double() * gsum[t0:t1, None]
        err = (y[t0:t1].double() - want).abs()
        assert bool((err <= gu.COMBINE_RTOL * want.abs() + 1e-30).all()), \
            f"combine tokens [{t0}, {t1})"
    # sampled tokens recomputed by the oracle from host copies of x
    rng = np.random.default_rng(123)
    tokens = np.sort(rng.choice(w.N, size=256, replace=False))
    xs = activation_rows(w, tokens, 0)
    for i, tok in enumerate(tokens):
        rows = slot[tok * w.K:(tok + 1) * w.K]
        got = gu.d2h(recv[t.from_numpy(rows).cuda()])
        assert (got == xs[i][None, :]).all(), f"token {tok}"
    yh = y[t.from_numpy(tokens).cuda()].cpu().numpy().astype(np.float64)
    want = oracle.bf16_to_f64(xs) * gates32[tokens].astype(np.float64).sum(axis=1)[:, None]
    assert (np.abs(yh - want) <= gu.COMBINE_RTOL * np.abs(want) + 1e-30).all()
    if name == "dsv3":
        # a random expert output in the receive layout, drawn on the device
        del x
        out = device_normal_bf16((w.R * C, w.H), 11, "cuda")
        path.combine(out, slot_d, g_d, y)
        t.cuda.synchronize()
        yref, mag = oracle.combine(lambda rows: gu.d2h(out[t.from_numpy(rows).cuda()]), slot,
                                   gates32, w.K, tokens=tokens)
        err = np.abs(y[t.from_numpy(tokens).cuda()].cpu().numpy().astype(np.float64) - yref)
        assert (err <= gu.COMBINE_RTOL * mag + 1e-30).all(), \
            f"combine (random out) max err/mag {(err / np.maximum(mag, 1e-30)).max()}"


def test_recv_views_zero_copy_and_clones():
    """Zero-copy views alias the receive buffer (the next dispatch changes
    them); zero_copy=False clones keep the rows."""
    t = gu.torch()
    w = WORKLOADS["tiny"]
    logits = router_logits(w, 0)
    res = gu.run_front(gu.shape_of(w), logits)
    path, C = res["path"], res["sizes"]["C"]
    recv = t.zeros((w.R * C, w.H), dtype=t.int16, device="cuda")
    x = gu.h2d(activations(w, 0))
    path.dispatch(x, res["dev"]["slot"], recv)
    nrp = res["plan_fields"]["n_rows_padded"]
    views = path.recv_views(recv, nrp)
    kept = path.recv_views(recv, nrp, zero_copy=False)
    assert all(v.data_ptr() == recv[r * C:].data_ptr() for r, v in enumerate(views))
    before = [k.clone() for k in kept]
    path.dispatch(t.zeros_like(x), res["dev"]["slot"], recv)
    t.cuda.synchronize()
    assert any(int(v.abs().sum().item()) != int(b.abs().sum().item()) for v, b in zip(views, before))
    assert all(t.equal(k, b) for k, b in zip(kept, before))


# --------------------------------------------------------------------------- max_vio sweep
@pytest.mark.parametrize("vio", [0.2, 1.0, 10.0, 20.0])
@pytest.mark.parametrize("planner", ["fixed", "quota"])
def test_maxvio_routing_parity(vio, planner):
    """The sweep's routings (MoonEP's bench shape with S cut to 1024 tokens
    per rank) through route, either planner and align, bit-exact."""
    w = WORKLOADS["moonep"].with_(vio=vio, S=1024)
    print(f"[parity] moonep vio={vio} {planner}", flush=True)
    logits = router_logits(w, 0)
    res = gu.run_front(gu.shape_of(w), logits, planner=planner)
    ref = gu.run_oracle(w, logits, planner=planner)
    gu.check_route(res, ref)
    gu.check_plan(res["plan_fields"], ref["plan"], w.P)
    gu.check_align(res, ref, w.R, res["sizes"]["C"])


# --------------------------------------------------------------------------- edge cases
def _edge(w, logits=None, sel_bias=None, cap=0, renorm=0, move=True):
    logits = router_logits(w, 0) if logits is None else logits
    res = gu.run_front(gu.shape_of(w, cap=cap, renorm=renorm), logits, sel_bias=sel_bias)
    ref = gu.run_oracle(w, logits, sel_bias=sel_bias, cap=cap, renorm=bool(renorm))
    gu.check_route(res, ref)
    gu.check_plan(res["plan_fields"], ref["plan"], w.P)
    gu.check_align(res, ref, w.R, res["sizes"]["C"])
    if move:
        _full_move_check(w, res, ref, activations(w, 0))
    return res, ref


TINY = WORKLOADS["tiny"]


@pytest.mark.parametrize("case", [
    "S1", "S300_ragged", "K1", "K3", "KeqE", "B0", "E_eq_R", "H_ragged", "H8", "renorm",
    "softmax_big_E", "sel_bias"])
def test_edge_cases(case):
    print(f"[parity] edge {case}", flush=True)
    w = TINY
    kw = {}
    if case == "S1":
        w = w.with_(S=1)
    elif case == "S300_ragged":
        w = w.with_(S=300, H=64)
    elif case == "K1":
        w = w.with_(K=1)
    elif case == "K3":
        w = w.with_(K=3)
    elif case == "KeqE":
        w = w.with_(K=w.E)
    elif case == "B0":
        w = WORKLOADS["wideep"].with_(S=16, H=64, B=0)
    elif case == "E_eq_R":
        w = w.with_(E=8, R=8, S=16)
    elif case == "H_ragged":
        w = w.with_(H=7176, S=8)
    elif case == "H8":
        w = w.with_(H=8)
    elif case == "renorm":
        kw["renorm"] = 1
    elif case == "softmax_big_E":
        w = WORKLOADS["dsv3"].with_(S=64, H=64, score="softmax")
    elif case == "sel_bias":
        kw["sel_bias"] = np.linspace(-1, 1, w.E).astype(np.float32)
    _edge(w, **kw)


def test_ties_and_signed_zero():
    w = TINY.with_(S=16)
    rng = np.random.default_rng(4)
    logits = (rng.integers(-2, 3, size=(w.N, w.E)) * 0.5).astype(np.float32)
    logits[rng.random(logits.shape) < 0.2] = np.float32(-0.0)
    logits[0] = 0.0
    _edge(w, logits=logits)


def test_all_equal_logits():
    w = TINY.with_(S=32)
    _edge(w, logits=np.zeros((w.N, w.E), np.float32))


def test_balanced_routing_no_replicas():
    w = TINY.with_(S=32, H=64)
    # token t of rank r picks rank r's two home experts with the largest keys
    logits = np.full((w.N, w.E), -5.0, np.float32)
    nh = w.E // w.R
    for t_ in range(w.N):
        r = t_ // w.S
        logits[t_, r * nh:(r + 1) * nh] = [1.0, 0.5]
    res, ref = _edge(w, logits=logits)
    assert ref["plan"]["replicas"] == []
    assert res["plan_fields"]["hdr"][0] == 0


def test_one_overloaded_rank():
    w = TINY.with_(S=32, H=64, B=1)
    logits = router_logits(w, 0)
    logits[:, 0] += 10.0   # expert 0 (rank 0) chosen by every token
    res, ref = _edge(w, logits=logits)
    assert ref["plan"]["over"][0] > 0


def test_empty_input():
    import load_balanced_token_amd as lbt
    t = gu.torch()
    shape = lbt.Shape(E=8, K=2, R=4, S=0, H=64, B=2, blk=16)
    path = lbt.Path(shape)
    buf = path.alloc()
    lg = t.empty((0, 8), dtype=t.float32, device="cuda")
    path.route_topk(lg, buf["ids"], buf["gates"], buf["counts"], buf["work"])
    path.plan_balance(buf["counts"], buf["plan"], buf["status"])
    path.align_sort(buf["ids"], buf["work"], buf["plan"], buf["slot"], buf["sorted_ids"],
                    buf["block_wrow"], buf["block_expert"], buf["status"])
    t.cuda.synchronize()
    pf = lbt.plan_fields(buf["plan"].cpu().numpy(), path.sizes, 4, 8)
    assert (buf["counts"].cpu().numpy() == 0).all()
    assert (pf["n_rows_padded"] == 0).all() and pf["hdr"][0] == 0
    assert (buf["block_wrow"].cpu().numpy() == -1).all()
    assert buf["status"].item() == 0


def test_capacity_too_small_sets_status():
    import load_balanced_token_amd as lbt
    t = gu.torch()
    w = WORKLOADS["dsv3"].with_(S=64, H=64)
    logits = router_logits(w, 0)
    ref = gu.run_oracle(w, logits)
    need = int(ref["plan"]["n_rows_padded"].max())
    cap = (need // w.blk - 1) * w.blk
    res = gu.run_front(gu.shape_of(w, cap=cap), logits)
    assert res["status"][0] & lbt.ST_CAPACITY
    assert res["plan_fields"]["hdr"][7] & lbt.ST_CAPACITY
    ok = res["slot"] >= 0
    assert (~ok).any()
    # pairs that fit land where the uncapped plan puts them (same rows, new C)
    full = ref["align"]["slot"]
    C0 = ref["plan"]["C"]
    assert np.array_equal(res["slot"][ok], (full[ok] // C0) * cap + full[ok] % C0)


def test_histogram_of_caller_ids_and_bad_ids():
    import load_balanced_token_amd as lbt
    t = gu.torch()
    w = TINY
    ids, _ = oracle.route_topk(router_logits(w, 0), w.K, oracle.SOFTMAX)
    path = lbt.Path(gu.shape_of(w))
    buf = path.alloc()
    buf["status"].zero_()
    path.histogram(gu.h2d(ids.astype(np.int32)), buf["counts"], buf["work"], buf["status"])
    t.cuda.synchronize()
    assert np.array_equal(buf["counts"].cpu().numpy(), oracle.load_matrix(ids, w.R, w.S, w.E))
    assert buf["status"].item() == 0
    bad = ids.astype(np.int32).copy()
    bad[3, 1] = w.E + 5
    path.histogram(gu.h2d(bad), buf["counts"], buf["work"], buf["status"])
    t.cuda.synchronize()
    assert buf["status"].item() & lbt.ST_BADID


@pytest.mark.parametrize("S", [1, 33, 100, 300])
def test_histogram_path_ragged_sizes(S):
    """Caller-supplied ids through lbt_histogram (one workgroup per 32-token
    sub-tile), the plan and align, at sizes with a ragged last sub-tile and
    several 128-token tiles per rank: load matrix, plan and placement equal
    the oracle's."""
    import load_balanced_token_amd as lbt
    t = gu.torch()
    w = WORKLOADS["dsv3"].with_(S=S, H=64)
    logits = router_logits(w, 0)
    ref = gu.run_oracle(w, logits)
    path = lbt.Path(gu.shape_of(w))
    buf = path.alloc()
    buf["status"].zero_()
    d = gu.h2d(ref["ids"].astype(np.int32))
    path.histogram(d, buf["counts"], buf["work"], buf["status"])
    path.plan_balance(buf["counts"], buf["plan"], buf["status"])
    path.align_sort(d, buf["work"], buf["plan"], buf["slot"], buf["sorted_ids"],
                    buf["block_wrow"], buf["block_expert"], buf["status"])
    t.cuda.synchronize()
    got = {k: gu.d2h(v) for k, v in buf.items()}
    assert np.array_equal(got["counts"], ref["counts"])
    pf = lbt.plan_fields(got["plan"], path.sizes, w.R, w.E)
    gu.check_plan(pf, ref["plan"], w.P)
    gu.check_align(got, ref, w.R, path.sizes["C"])


def test_duplicate_ids_flagged():
    import load_balanced_token_amd as lbt
    t = gu.torch()
    w = TINY
    ids, _ = oracle.route_topk(router_logits(w, 0), w.K, oracle.SOFTMAX)
    dup = ids.astype(np.int32).copy()
    dup[5, 1] = dup[5, 0]
    path = lbt.Path(gu.shape_of(w))
    buf = path.alloc()
    buf["status"].zero_()
    d = gu.h2d(dup)
    path.histogram(d, buf["counts"], buf["work"], buf["status"])
    path.plan_balance(buf["counts"], buf["plan"], buf["status"])
    path.align_sort(d, buf["work"], buf["plan"], buf["slot"], buf["sorted_ids"],
                    buf["block_wrow"], buf["block_expert"], buf["status"])
    t.cuda.synchronize()
    assert buf["status"].item() & lbt.ST_DUPID


def test_inconsistent_counts_flagged():
    import load_balanced_token_amd as lbt
    t = gu.torch()
    w = TINY
    path = lbt.Path(gu.shape_of(w))
    buf = path.alloc()
    counts = np.ones((w.R, w.E), np.int32)
    path.plan_balance(gu.h2d(counts), buf["plan"], buf["status"])
    t.cuda.synchronize()
    assert buf["status"].item() & lbt.ST_BADCOUNT


def test_bad_arguments_rejected():
    import load_balanced_token_amd as lbt
    t = gu.torch()
    with pytest.raises(lbt.LbtError):
        lbt.Path(lbt.Shape(E=10, K=2, R=4, S=8, H=64, B=1, blk=16))   # E % R != 0
    with pytest.raises(lbt.LbtError):
        lbt.Path(lbt.Shape(E=8, K=9, R=4, S=8, H=64, B=1, blk=16))    # K > E
    with pytest.raises(lbt.LbtError):
        lbt.Path(lbt.Shape(E=8, K=2, R=4, S=8, H=60, B=1, blk=16))    # H % 8
    path = lbt.Path(lbt.Shape(E=8, K=2, R=4, S=8, H=64, B=1, blk=16))
    buf = path.alloc()
    xs = t.zeros(32 * 64 + 1, dtype=t.int16, device="cuda")[1:]        # misaligned
    with pytest.raises(lbt.LbtError):
        path.dispatch(xs, buf["slot"], buf["recv"])


def test_stale_hip_error_is_not_reported_by_a_later_call():
    """An error left in the thread's HIP last-error state by an earlier,
    unrelated HIP call (here hipSetDevice on a device that does not exist,
    made through the same HIP runtime the library uses) is not returned by
    the next lbt call: route (two launches), plan and align launch and return
    LBT_OK, and their outputs equal the oracle's.  Every buffer is allocated
    before the error is left behind, so the library's call is the first HIP
    call after it."""
    import ctypes
    t = gu.torch()
    import load_balanced_token_amd as lbt
    lbt.lib()
    paths = sorted({l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l})
    assert len(paths) == 1, paths
    hip = ctypes.CDLL(paths[0])
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    w = WORKLOADS["dsv3"].with_(S=64, H=64)             # 16 sub-tiles: the two-launch route
    logits = router_logits(w, 0)
    path = lbt.Path(gu.shape_of(w))
    buf = path.alloc()
    buf["status"].zero_()
    lg = gu.h2d(logits)
    stream = t.cuda.current_stream()
    t.cuda.synchronize()
    assert hip.hipSetDevice(9999) != 0                  # leaves hipErrorInvalidDevice behind
    path.route_topk(lg, buf["ids"], buf["gates"], buf["counts"], buf["work"], stream=stream)
    path.plan_balance(buf["counts"], buf["plan"], buf["status"], stream=stream)
    path.align_sort(buf["ids"], buf["work"], buf["plan"], buf["slot"], buf["sorted_ids"],
                    buf["block_wrow"], buf["block_expert"], buf["status"], stream=stream)
    t.cuda.synchronize()
    assert lbt.lib().lbt_last_hip_error().decode() == "hipSuccess"
    ref = gu.run_oracle(w, logits)
    assert np.array_equal(gu.d2h(buf["ids"]), ref["ids"])
    assert np.array_equal(gu.d2h(buf["counts"]), ref["counts"])
    assert np.array_equal(gu.d2h(buf["slot"]), ref["align"]["slot"])
    assert buf["status"].item() == 0


def test_deterministic_rerun():
    t = gu.torch()
    w = WORKLOADS["wideep"]
    logits = router_logits(w, 0)
    a = gu.run_front(gu.shape_of(w), logits)
    b = gu.run_front(gu.shape_of(w), logits)
    for k in ("ids", "gates", "counts", "plan", "slot", "block_wrow", "block_expert"):
        assert np.array_equal(a[k], b[k]), k
    C = a["sizes"]["C"]
    nrp = a["plan_fields"]["n_rows_padded"]
    for r in range(w.R):
        assert np.array_equal(a["sorted_ids"][r * C: r * C + nrp[r]],
                              b["sorted_ids"][r * C: r * C + nrp[r]])


def test_graph_capture_replays_match_eager():
    """The whole step captured in a HIP graph on a fixed input buffer: every
    replay (fresh routing copied in before it, outside the graph, with eager
    work and syncs in between) equals the eager run.  The routing of each
    replay is chosen on the host, so no device-side index is involved."""
    import load_balanced_token_amd as lbt
    t = gu.torch()
    w = WORKLOADS["decode16"].with_(H=512)
    path = lbt.Path(gu.shape_of(w))
    buf = path.alloc()
    buf["status"].zero_()
    n = 4
    all_logits = [gu.h2d(router_logits(w, i)) for i in range(n)]
    x = gu.h2d(activations(w, 0))
    cur = t.empty((w.N, w.E), dtype=t.float32, device="cuda")
    cur.copy_(all_logits[0])
    keys = ("ids", "gates", "counts", "plan", "slot", "block_wrow", "y")

    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        path.step(cur, x, buf)                          # warm-up outside the graph
    t.cuda.current_stream().wait_stream(s)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g, stream=s):
        path.step(cur, x, buf)
    t.cuda.synchronize()
    ref_path = lbt.Path(gu.shape_of(w))
    for i in range(n):
        cur.copy_(all_logits[i])                        # host-chosen routing, outside the graph
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        got = {k: buf[k].clone() for k in keys}
        ref = ref_path.alloc()
        ref["status"].zero_()
        ref_path.step(all_logits[i], x, ref)            # eager work between replays
        t.cuda.synchronize()
        for k in keys:
            assert t.equal(got[k], ref[k]), f"replay {i}: {k}"
        assert buf["status"].item() == 0


@pytest.mark.parametrize("H,S", [(7168, 32), (7168, 33), (512, 32), (512, 33)])
def test_dispatch_combine_with_dropped_pairs(H, S):
    """A capacity below the plan's need drops pairs (slot -1): dispatch skips
    them and combine sums only the pairs that fit (both row widths; N = 256
    takes the small-batch kernels, N = 264 the row-per-workgroup ones)."""
    t = gu.torch()
    w = WORKLOADS["dsv3"].with_(S=S, H=H)
    logits = router_logits(w, 0)
    ref = gu.run_oracle(w, logits)
    need = int(ref["plan"]["n_rows_padded"].max())
    cap = (need // w.blk - 1) * w.blk
    res = gu.run_front(gu.shape_of(w, cap=cap), logits)
    slot = res["slot"]
    assert (slot < 0).any() and (slot >= 0).any()
    path = res["path"]
    x_bits = activations(w, 0)
    recv = t.zeros((w.R * cap, w.H), dtype=t.int16, device="cuda")
    path.dispatch(gu.h2d(x_bits), res["dev"]["slot"], recv)
    gates32 = ref["gates"].astype(np.float32)
    y = t.empty((w.N, w.H), dtype=t.float32, device="cuda")
    path.combine(recv, res["dev"]["slot"], gu.h2d(gates32), y)
    t.cuda.synchronize()
    recv_h = gu.d2h(recv)
    ok = slot >= 0
    f = np.nonzero(ok)[0]
    assert np.array_equal(recv_h[slot[f]], x_bits[f // w.K])
    g_fit = np.where(ok.reshape(w.N, w.K), gates32, 0).astype(np.float64)
    want = oracle.bf16_to_f64(x_bits) * g_fit.sum(axis=1)[:, None]
    got = y.cpu().numpy().astype(np.float64)
    assert (np.abs(got - want) <= gu.COMBINE_RTOL * np.abs(want) + 1e-30).all()



@pytest.mark.parametrize("H,K", [(7168, 8), (512, 8), (136, 3), (64, 4)])
def test_small_batch_kernels_bitwise_equal_row_kernels(H, K):
    """Batches of up to 256 tokens move rows with one wave per slice of a row;
    larger ones with one workgroup per row.  The same pairs through both (256
    tokens vs the same 256 plus 8 more) give bit-identical recv rows,
    combine outputs (fp32 and bf16) and dispatch gradients."""
    import load_balanced_token_amd as lbt
    t = gu.torch()
    R, E, cap = 8, 64, 512
    small = lbt.Path(lbt.Shape(E=E, K=K, R=R, S=32, H=H, B=2, blk=128, cap=cap))
    large = lbt.Path(lbt.Shape(E=E, K=K, R=R, S=33, H=H, B=2, blk=128, cap=cap))
    Ns, Nl = R * 32, R * 33
    rng = np.random.default_rng(7 + H + K)
    rows = rng.permutation(R * cap)[: Nl * K].astype(np.int32)
    rows[rng.random(Nl * K) < 0.05] = -1               # some pairs did not fit
    slot_l = gu.h2d(rows)
    slot_s = gu.h2d(rows[: Ns * K].copy())
    gates = gu.h2d(rng.random((Nl, K)).astype(np.float32))
    gates_s = gates[:Ns].contiguous()
    bf16 = lambda n: t.randn(n, H, device="cuda").to(t.bfloat16).view(t.int16)
    out = bf16(R * cap)
    x = bf16(Nl)
    for y_dtype in (t.float32, t.int16):
        ys = t.empty(Ns, H, dtype=y_dtype, device="cuda")
        yl = t.empty(Nl, H, dtype=y_dtype, device="cuda")
        small.combine(out, slot_s, gates_s, ys)
        large.combine(out, slot_l, gates, yl)
        assert t.equal(ys.view(t.int32) if y_dtype == t.float32 else ys,
                       (yl.view(t.int32) if y_dtype == t.float32 else yl)[:Ns])
        small.dispatch_bwd(out, slot_s, ys)
        large.dispatch_bwd(out, slot_l, yl)
        assert t.equal(ys.view(t.int32) if y_dtype == t.float32 else ys,
                       (yl.view(t.int32) if y_dtype == t.float32 else yl)[:Ns])
    rs = t.zeros(R * cap, H, dtype=t.int16, device="cuda")
    rl = t.zeros(R * cap, H, dtype=t.int16, device="cuda")
    small.dispatch(x[:Ns].contiguous(), slot_s, rs)
    large.dispatch(x, slot_l, rl)
    t.cuda.synchronize()
    mine = rows[: Ns * K]
    mine = mine[mine >= 0]
    idx = t.from_numpy(mine.astype(np.int64)).cuda()
    assert t.equal(rs[idx], rl[idx])
    assert t.equal(rs[idx], x[t.from_numpy(np.nonzero(rows[: Ns * K] >= 0)[0] // K).cuda()])
    untouched = np.ones(R * cap, bool)
    untouched[mine] = False
    assert not rs[t.from_numpy(np.nonzero(untouched)[0]).cuda()].any()


# --------------------------------------------------------------------------- widths and limits
@pytest.mark.parametrize("E,K,R", [(24, 4, 4), (40, 6, 8), (64, 8, 8), (128, 8, 16), (200, 8, 8),
                                   (512, 8, 8)])
def test_route_width_ladder(E, K, R):
    """Every compiled route width (a lane holds V = ceil(E/16) experts: V = 2,
    3 -> 4, 4, 8, 13 -> 16, 32), with ragged last lanes where E is not a
    multiple of 16; the DSV3 generator at that E, full rows moved."""
    w = WORKLOADS["dsv3"].with_(E=E, K=K, R=R, S=64, H=64, B=4, blk=16)
    print(f"[parity] width E={E} K={K} R={R}", flush=True)
    _edge(w)


@pytest.mark.parametrize("E,R,S", [(60, 5, 7000), (66, 3, 27000), (96, 2, 33000)])
def test_column_scan_batches(E, R, S):
    """Columns of more than 1024 sub-tiles, where the column scan spreads a
    column's batches over several waves, with a ragged last batch and ranks
    that end inside a batch: four columns per workgroup (E a multiple of
    4) and one (E = 66); load matrix, plan and placement equal the
    oracle's, full rows moved."""
    w = WORKLOADS["dsv3"].with_(E=E, K=4, R=R, S=S, H=64, B=4, blk=16)
    n_sub = R * -(-S // 32)
    print(f"[parity] column scan E={E} R={R} S={S}: {n_sub} sub-tiles", flush=True)
    assert n_sub > 1024
    _edge(w)


@pytest.mark.parametrize("case,planner", [("E512_K64", "fixed"), ("E512_K64", "quota"),
                                          ("R512", "fixed"), ("R512", "quota"),
                                          ("R65", "fixed"), ("R65", "quota"),
                                          ("R128", "fixed"), ("R128", "quota")])
def test_maximum_sizes(case, planner):
    """The library's limits: E = 512 with K = 64 (64 top-K rounds per token,
    every lane list refilled many times), and R = E = 512 (one expert per
    rank, up to E + R replica pieces), through either planner; and rank
    counts past one wave (65, 128), where the plan's per-rank prefixes come
    from LDS scans instead of one lane per rank."""
    if case == "E512_K64":
        w = WORKLOADS["dsv3"].with_(E=512, K=64, R=8, S=64, H=64, B=4, blk=16)
    elif case == "R512":
        w = WORKLOADS["dsv3"].with_(E=512, R=512, K=8, S=4, H=64, B=2, blk=4)
    elif case == "R65":
        w = WORKLOADS["dsv3"].with_(E=130, R=65, K=8, S=24, H=64, B=3, blk=8)
    else:
        w = WORKLOADS["dsv3"].with_(E=256, R=128, K=8, S=16, H=64, B=2, blk=16)
    print(f"[parity] limits {case} {planner}", flush=True)
    logits = router_logits(w, 0)
    res = gu.run_front(gu.shape_of(w), logits, planner=planner)
    ref = gu.run_oracle(w, logits, planner=planner)
    gu.check_route(res, ref)
    gu.check_plan(res["plan_fields"], ref["plan"], w.P)
    gu.check_align(res, ref, w.R, res["sizes"]["C"])
    _full_move_check(w, res, ref, activations(w, 0))


@pytest.mark.parametrize("planner", ["fixed", "quota"])
def test_corrupt_plan_is_flagged_not_followed(planner):
    """A plan blob whose replica segments name a rank past R and rows past C
    (as a caller's corrupted buffer might): align raises LBT_ST_CAPACITY and
    gives those pairs slot -1; every other slot stays in range."""
    t = gu.torch()
    from load_balanced_token_amd.binding import ST_CAPACITY
    w = TINY.with_(S=32, B=1)
    logits = router_logits(w, 0)
    res = gu.run_front(gu.shape_of(w), logits, planner=planner)
    assert res["plan_fields"]["hdr"][gu.HDR_N_PIECES] > 0
    path, z = res["path"], res["sizes"]
    plan = res["dev"]["plan"].clone()
    nP = int(res["plan_fields"]["hdr"][gu.HDR_N_PIECES])
    plan[z["off_piece_rank"]: z["off_piece_rank"] + nP] = w.R + 3
    plan[z["off_piece_row"]: z["off_piece_row"] + nP] = z["C"] + 100
    slot = t.empty(w.P, dtype=t.int32, device="cuda")
    sid = t.empty(w.R * z["C"], dtype=t.int32, device="cuda")
    bw = t.empty(w.R * z["n_blocks"], dtype=t.int32, device="cuda")
    be = t.empty_like(bw)
    st = t.zeros(1, dtype=t.int32, device="cuda")
    path.align_sort(res["dev"]["ids"], res["dev"]["work"], plan, slot, sid, bw, be, st)
    t.cuda.synchronize()
    s = slot.cpu().numpy()
    assert int(st.item()) & ST_CAPACITY
    assert ((s == -1) | ((s >= 0) & (s < w.R * z["C"]))).all()
    assert (s == -1).any()


# --------------------------------------------------------------------------- fused front
@pytest.mark.parametrize("case", [
    ("decode1", {}), ("decode1", {"E": 384, "R": 8}), ("decode1", {"E": 512, "R": 16, "K": 16}),
    ("decode1", {"S": 4}), ("decode1", {"S": 3, "R": 4, "E": 40, "K": 6}),
    ("tiny", {"S": 8}), ("tiny", {"S": 5, "R": 2}),
    # past 32 tokens: the separate launches
    ("decode16", {}), ("tiny", {}), ("decode128", {}), ("decode16", {"S": 40}),
    ("decode16", {"S": 33, "R": 4, "E": 40, "K": 6}), ("tiny", {"S": 300}),
    ("tiny", {"S": 2100}), ("decode1", {"S": 100, "E": 512, "R": 16}),
    ("decode1", {"S": 64, "E": 512, "R": 16, "K": 4}),
])
@pytest.mark.parametrize("variant", ["plain", "bias_renorm"])
def test_route_plan_matches_separate_calls(case, variant):
    """lbt_route_plan gives bit for bit the outputs of lbt_route_topk followed
    by lbt_plan_balance (ids, gates, counts, the tile offsets align reads,
    the whole plan blob and the status), and lbt_front those plus
    lbt_align_sort's (slots, sorted ids, block tables), for batches that take
    the one-launch small-batch kernel and for larger ones; all equal the
    oracle."""
    import load_balanced_token_amd as lbt
    t = gu.torch()
    name, over = case
    w = WORKLOADS[name].with_(**over)
    renorm = 1 if variant == "bias_renorm" else 0
    logits = router_logits(w, 3)
    rng = np.random.default_rng(5)
    bias = rng.standard_normal(w.E).astype(np.float32) if variant == "bias_renorm" else None
    shape = gu.shape_of(w, renorm=renorm)
    path = lbt.Path(shape)
    a, b = path.alloc(), path.alloc()
    for k in ("recv", "y"):
        del a[k], b[k]
    a["status"].zero_()
    b["status"].fill_(-1)
    lg = gu.h2d(logits)
    sb = None if bias is None else gu.h2d(bias)
    path.route_topk(lg, a["ids"], a["gates"], a["counts"], a["work"], sel_bias=sb)
    path.plan_balance(a["counts"], a["plan"], a["status"])
    path.route_plan(lg, b["ids"], b["gates"], b["counts"], b["work"], b["plan"], b["status"],
                    sel_bias=sb)
    t.cuda.synchronize()
    for k in ("ids", "gates", "counts", "plan", "status"):
        assert t.equal(a[k], b[k]), k
    z = path.sizes
    lo = w.E * w.R * -(-w.S // 32)                      # tile offsets follow the sub-tile counts
    assert t.equal(a["work"][lo: lo + z["n_tiles"] * w.E], b["work"][lo: lo + z["n_tiles"] * w.E])
    ref = gu.run_oracle(w, logits, sel_bias=bias, renorm=bool(renorm))
    res = {"ids": gu.d2h(b["ids"]), "gates": gu.d2h(b["gates"]), "counts": gu.d2h(b["counts"])}
    gu.check_route(res, ref)
    pf = lbt.plan_fields(gu.d2h(b["plan"]), z, w.R, w.E)
    gu.check_plan(pf, ref["plan"], w.P)
    # and align on the fused outputs
    for k in ("sorted_ids", "slot"):
        b[k].fill_(-5)
    path.align_sort(b["ids"], b["work"], b["plan"], b["slot"], b["sorted_ids"], b["block_wrow"],
                    b["block_expert"], b["status"])
    t.cuda.synchronize()
    out = {k: gu.d2h(b[k]) for k in ("slot", "sorted_ids", "block_wrow", "block_expert", "status")}
    gu.check_align(out, ref, w.R, z["C"])
    # lbt_front: route, plan and align in one call, every output word equal
    c = path.alloc()
    del c["recv"], c["y"]
    for k in ("sorted_ids", "slot"):
        c[k].fill_(-5)
    c["status"].fill_(-1)
    path.front(lg, c, sel_bias=sb)
    t.cuda.synchronize()
    for k in ("ids", "gates", "counts", "plan", "status", "slot", "sorted_ids", "block_wrow",
              "block_expert"):
        assert t.equal(b[k], c[k]), f"front: {k}"
    assert t.equal(b["work"][lo: lo + z["n_tiles"] * w.E], c["work"][lo: lo + z["n_tiles"] * w.E])
