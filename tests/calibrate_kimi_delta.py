"""Recompute KIMI_DELTA: the logit offset of the 19 hot experts (5% of 384)
that makes them draw 30% of all (token, expert) assignments in the Kimi-K3-
scale workload.  Bisection on [0, 4] over a 16,384-token sample of layer 0,
routed by the CPU oracle.  Prints the offset, rounded to a multiple of 2^-10,
and the share it reaches on the full layer-0 routing.

    python tests/calibrate_kimi_delta.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from workloads.gen import WORKLOADS, router_logits, expert_bias, n_hot  # noqa: E402
from oracle import route_topk, SIGMOID  # noqa: E402


def hot_share(w, delta, rows):
    logits = router_logits(w, 0, delta=delta, rows=rows)
    ids, _ = route_topk(logits, w.K, SIGMOID)
    hot = np.nonzero(expert_bias(w, 0, delta=1.0))[0]
    assert hot.size == n_hot(w)
    return np.isin(ids, hot).mean()


def main():
    w = WORKLOADS["kimi"]
    lo, hi = 0.0, 4.0
    sample = slice(0, 16384)
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        if hot_share(w, mid, sample) < 0.30:
            lo = mid
        else:
            hi = mid
    delta = round(0.5 * (lo + hi) * 1024) / 1024
    print(f"KIMI_DELTA = {delta!r}  (sample share {hot_share(w, delta, sample):.4f}, "
          f"full share {hot_share(w, delta, None):.4f})")


if __name__ == "__main__":
    main()
