"""Brute-force enumerators used to pin the oracle on tiny inputs.

They state the plan rule declaratively and search every assignment of
(token, expert) pairs to ranks; they share nothing with the oracle's interval
arithmetic (prefix offsets and intersections).
"""
import itertools


def pair_list(ids):
    """[(f, e)] in ascending flat index f = t*K + k."""
    out = []
    for t, row in enumerate(ids):
        for k, e in enumerate(row):
            out.append((t * len(row) + k, int(e)))
    return out


def _assignments(P, R, SK):
    """Every map pair -> rank that gives each rank exactly SK pairs."""
    load = [0] * R
    cur = [0] * P

    def rec(i):
        if i == P:
            yield tuple(cur)
            return
        for d in range(R):
            if load[d] < SK:
                load[d] += 1
                cur[i] = d
                yield from rec(i + 1)
                load[d] -= 1

    yield from rec(0)


def rule_conforming_plans(ids, E, R, S):
    """All assignments meeting the fixed rule, stated declaratively:
      (a) every rank holds exactly S*K pairs;
      (b) rank r keeps exactly min(L_r, S*K) of the pairs whose expert is
          home to r, where L_r counts those pairs;
      (c) the kept pairs are the earliest of r's home stream (experts
          ascending, then flat index ascending);
      (d) the pairs that leave their home rank, taken in (expert, flat index)
          order, go to ranks in non-decreasing rank order.
    Returns the list of assignments (tuples rank-of-pair in f order)."""
    K = len(ids[0])
    SK = S * K
    nh = E // R
    pairs = pair_list(ids)
    P = len(pairs)
    home = [e // nh for (_, e) in pairs]
    streams = []
    for r in range(R):
        st = sorted((e, f) for (f, e) in pairs if e // nh == r)
        streams.append([f for (_, f) in st])
    moved_order = [f for (e, f) in sorted((e, f) for (f, e) in pairs)]
    found = []
    for asg in _assignments(P, R, SK):
        ok = True
        for r in range(R):
            kept = [asg[f] == r for f in streams[r]]
            nkeep = min(len(streams[r]), SK)
            if sum(kept) != nkeep or not all(kept[:nkeep]):
                ok = False
                break
        if not ok:
            continue
        moved = [asg[f] for f in moved_order if asg[f] != home[f]]
        if any(moved[i] > moved[i + 1] for i in range(len(moved) - 1)):
            continue
        found.append(asg)
    return found


def replicas_of(asg, ids, E, R):
    """Distinct (expert, rank) pairs that place an expert away from home."""
    nh = E // R
    return {(e, asg[f]) for (f, e) in pair_list(ids) if asg[f] != e // nh}


def min_replicas(ids, E, R, S):
    """Fewest replicas over every exact-S*K assignment (no rule imposed)."""
    K = len(ids[0])
    best = None
    for asg in _assignments(len(ids) * K, R, S * K):
        n = len(replicas_of(asg, ids, E, R))
        best = n if best is None else min(best, n)
    return best


def topk_by_sorting(key_row, K):
    """Top-K of one row by Python's sort on (-key, index)."""
    return sorted(range(len(key_row)), key=lambda e: (-float(key_row[e]), e))[:K]


def ordered_rows_per_rank(asg, ids, R):
    """Multiset of experts each rank serves under an assignment."""
    out = [[] for _ in range(R)]
    for (f, e) in pair_list(ids):
        out[asg[f]].append(e)
    return [sorted(x) for x in out]


def all_small_routings(E, K, N):
    """Every routing of N tokens to K distinct experts each (tiny sizes)."""
    combos = list(itertools.combinations(range(E), K))
    for choice in itertools.product(combos, repeat=N):
        yield [list(c) for c in choice]
