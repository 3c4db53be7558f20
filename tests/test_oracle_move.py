"""Pins for the oracle's dispatch and combine (CPU only)."""
import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, activations, router_logits, f32_to_bf16_bits, bf16_bits_to_f32


def _tiny_path():
    w = WORKLOADS["tiny"]
    ids, gates = oracle.route_topk(router_logits(w, 0), w.K, oracle.SOFTMAX)
    counts = oracle.load_matrix(ids, w.R, w.S, w.E)
    plan = oracle.plan_balance(counts, w.K, w.S, w.B, w.blk)
    al = oracle.align_sort(ids, plan)
    return w, ids, gates.astype(np.float32), plan, al


def test_dispatch_is_a_bit_copy_to_each_slot():
    w, ids, gates, plan, al = _tiny_path()
    x = activations(w, 0)
    recv = oracle.dispatch(x, al["slot"], w.K, w.R, plan["C"])
    for f in range(w.P):
        assert (recv[al["slot"][f]] == x[f // w.K]).all()
    # rows no pair maps to are untouched (zero here)
    used = np.zeros(w.R * plan["C"], bool)
    used[al["slot"]] = True
    assert (recv[~used] == 0).all()


def test_combine_of_identity_expert_is_x_times_gate_sum():
    """combine(dispatch(x)) = x * sum_k gates (closed form)."""
    w, ids, gates, plan, al = _tiny_path()
    x = activations(w, 0)
    recv = oracle.dispatch(x, al["slot"], w.K, w.R, plan["C"])
    y, mag = oracle.combine(lambda rows: recv[rows], al["slot"], gates, w.K)
    want = bf16_bits_to_f32(x).astype(np.float64) * gates.astype(np.float64).sum(axis=1)[:, None]
    assert np.allclose(y, want, rtol=1e-15, atol=0)
    assert (mag >= np.abs(y) * (1 - 1e-15)).all()


def test_combine_is_linear_and_ordered_by_k():
    rng = np.random.default_rng(0)
    K, H, N = 3, 16, 5
    out = f32_to_bf16_bits(rng.standard_normal((N * K, H)).astype(np.float32))
    slot = rng.permutation(N * K)
    g = rng.random((N, K)).astype(np.float32)
    y, _ = oracle.combine(lambda rows: out[rows], slot, g, K)
    o64 = bf16_bits_to_f32(out).astype(np.float64)
    for t in range(N):
        acc = np.zeros(H)
        for k in range(K):
            acc = acc + np.float64(g[t, k]) * o64[slot[t * K + k]]
        assert np.array_equal(y[t], acc)
    # doubling the gates doubles y exactly
    y2, _ = oracle.combine(lambda rows: out[rows], slot, g * np.float32(2), K)
    assert np.array_equal(y2, 2 * y)


@pytest.mark.parametrize("v", [1.0, -2.5, 3.140625, 1e-3])
def test_bf16_widening_is_exact(v):
    b = f32_to_bf16_bits(np.array([v], np.float32))
    assert oracle.bf16_to_f64(b)[0] == float(bf16_bits_to_f32(b)[0])
