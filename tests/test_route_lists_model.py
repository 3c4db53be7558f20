"""A CPU model of the GPU route's top-K selection procedure, checked against
brute-force sorting on rows full of ties (CPU only).

The route kernel gives each token a 16-lane row; lane j holds experts
[j*V, j*V + V), V = ceil(E / 16).  A lane keeps only the values of its best
T = min(V, 4) keys (as order-preserving integers, -0.0 and +0.0 equal), a
round takes the largest list head and the lowest lane holding it, the
winner pops, a lane whose full list runs dry refills from the values after
the ones it gave up, and after the K rounds the expert of a lane's i-th win
of a value is the lane's i-th expert (in expert order) holding that value.
This model restates that procedure step by step so the argument that it
equals "largest untaken key, lowest expert on ties" can be checked on the
CPU; the GPU parity tests check the kernel itself against the oracle.
"""
import math
import struct

import numpy as np
import pytest

from tests.brute_force import topk_by_sorting

LANES = 16


def _ordered(x):
    """Order-preserving u32 of an fp32 value, -0.0 mapped with +0.0."""
    u = struct.unpack("<I", struct.pack("<f", float(np.float32(x) + np.float32(0.0))))[0]
    return u ^ (0xFFFFFFFF if u >> 31 else 0x80000000)


def _insert(lst, x):
    """Keep lst (descending, fixed length) the largest values seen, repeats
    included: each position takes the median of (value above, x, itself)."""
    for j in range(len(lst) - 1, 0, -1):
        lst[j] = sorted((lst[j - 1], x, lst[j]))[1]
    lst[0] = max(lst[0], x)


def model_topk(keys, K):
    E = len(keys)
    V = -(-E // LANES)
    T = min(V, 4)
    ok = [[_ordered(keys[j * V + v]) if j * V + v < E else 0 for v in range(V)]
          for j in range(LANES)]
    lists, more = [], []
    for j in range(LANES):
        lst = [0] * T
        for v in range(V):
            _insert(lst, ok[j][v])
        lists.append(lst)
        more.append(V > T and lst[T - 1] != 0)
    last, eq = [0] * LANES, [0] * LANES
    wins = []
    for _ in range(K):
        heads = [lst[0] for lst in lists]
        top = max(heads)
        w = heads.index(top)                      # the lowest lane holding it
        eq[w] = eq[w] + 1 if top == last[w] else 1
        last[w] = top
        wins.append((w, eq[w] - 1, top))
        lists[w] = lists[w][1:] + [0]
        if V > T and more[w] and lists[w][0] == 0:
            lst, seen = [0] * T, 0
            for v in range(V):
                same = ok[w][v] == last[w]
                _insert(lst, ok[w][v] if ok[w][v] < last[w] or (same and seen >= eq[w]) else 0)
                seen += same
            lists[w], more[w] = lst, lst[T - 1] != 0
    out = []
    for w, occ, val in wins:
        hits = [w * V + v for v in range(V) if w * V + v < E and ok[w][v] == val]
        out.append(hits[occ])
    return out


def _tie_rows(rng, n, E, K):
    rows = (rng.integers(-2, 3, size=(n, E)) * 0.5).astype(np.float32)
    rows[rng.random(rows.shape) < 0.2] = np.float32(-0.0)
    rows[0::4, :K + 4] = 3.0                                   # a tied block in the first lanes
    rows[1::4, 20:20 + K] = 2.0 + 0.125 * np.arange(K)[: len(rows[0, 20:20 + K])]
    rows[2::4] = 0.0                                           # every key equal
    return rows


@pytest.mark.parametrize("E,K", [(8, 2), (33, 8), (64, 8), (256, 8), (256, 24), (384, 8),
                                 (512, 64), (200, 13)])
def test_model_equals_sorting_on_ties(E, K):
    rng = np.random.default_rng(E * 64 + K)
    for row in _tie_rows(rng, 48, E, K):
        assert model_topk(row, K) == topk_by_sorting(row, K)


def test_model_equals_sorting_on_random_rows():
    rng = np.random.default_rng(11)
    for _ in range(200):
        E = int(rng.choice([16, 100, 256, 384]))
        K = int(rng.integers(1, min(E, 16) + 1))
        row = rng.standard_normal(E).astype(np.float32)
        assert model_topk(row, K) == topk_by_sorting(row, K)


def test_ordered_key_is_monotone_and_merges_zeros():
    vals = np.array([-math.inf, -3.5, -1e-38, -0.0, 0.0, 1e-45, 2.0, math.inf], np.float32)
    keys = [_ordered(v) for v in vals]
    assert keys[3] == keys[4]
    assert all(a < b for a, b in zip(keys[:3], keys[1:4]))
    assert all(a < b for a, b in zip(keys[4:], keys[5:]))
    assert min(keys) > 0                                       # 0 stays free as "no key"
