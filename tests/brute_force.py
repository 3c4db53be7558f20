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


def _capped_assignments(P, R, cap):
    """Every map pair -> rank that gives no rank more than cap pairs."""
    load = [0] * R
    cur = [0] * P

    def rec(i):
        if i == P:
            yield tuple(cur)
            return
        for d in range(R):
            if load[d] < cap:
                load[d] += 1
                cur[i] = d
                yield from rec(i + 1)
                load[d] -= 1

    yield from rec(0)


def quota_conforming_plans(ids, E, R, S, tau):
    """All assignments meeting the quota rule at threshold tau, stated
    declaratively (no prefix offsets, no intervals):
      (a) no rank holds more than tau pairs;
      (b) rank r keeps exactly min(L_r, tau) of the pairs of its home experts;
      (c) hot first: list r's experts by load descending, ties by lower
          index; if an expert sends any pair away, every expert listed before
          it sends all of its pairs away;
      (d) an expert keeps its earliest pairs (ascending flat index);
      (e) the pairs that leave home, taken rank by rank, in the hot-first
          list inside a rank, then by flat index, go to non-decreasing ranks;
      (f) a rank receives a pair from another rank only if every lower rank
          holds exactly tau pairs."""
    nh = E // R
    pairs = pair_list(ids)
    P = len(pairs)
    expert_of = {f: e for (f, e) in pairs}
    T = [0] * E
    for (_, e) in pairs:
        T[e] += 1
    hot = {}
    for r in range(R):
        for pos, e in enumerate(sorted(range(r * nh, (r + 1) * nh), key=lambda x: (-T[x], x))):
            hot[e] = pos
    by_expert = {e: sorted(f for (f, x) in pairs if x == e) for e in range(E)}
    leave_order = sorted(range(P), key=lambda f: (expert_of[f] // nh, hot[expert_of[f]], f))
    found = []
    for asg in _capped_assignments(P, R, tau):
        ok = True
        load = [0] * R
        for f in range(P):
            load[asg[f]] += 1
        for r in range(R):
            mine = [e for e in range(r * nh, (r + 1) * nh)]
            L = sum(T[e] for e in mine)
            kept = sum(1 for e in mine for f in by_expert[e] if asg[f] == r)
            if kept != min(L, tau):
                ok = False
                break
            order = sorted(mine, key=lambda x: hot[x])
            sheds = [any(asg[f] != r for f in by_expert[e]) for e in order]
            alls = [all(asg[f] != r for f in by_expert[e]) for e in order]
            for i in range(len(order)):
                if sheds[i] and not all(alls[:i]):
                    ok = False
            for e in mine:
                flags = [asg[f] == r for f in by_expert[e]]
                nk = sum(flags)
                if flags != [True] * nk + [False] * (len(flags) - nk):
                    ok = False
            if not ok:
                break
        if not ok:
            continue
        moved = [asg[f] for f in leave_order if asg[f] != expert_of[f] // nh]
        if any(moved[i] > moved[i + 1] for i in range(len(moved) - 1)):
            continue
        if any(not all(load[x] == tau for x in range(d)) for d in set(moved)):
            continue
        found.append(asg)
    return found


def quota_threshold(ids, E, R, S, B):
    """Smallest tau >= S*K whose quota-rule assignment puts no more than B
    replicas (distinct away-from-home experts) on any rank; with the
    assignment after the locality step (local_conforming_assignments, same
    quotas).  Every tau is tried in ascending order."""
    K = len(ids[0])
    nh = E // R
    T = [0] * E
    for (_, e) in pair_list(ids):
        T[e] += 1
    maxL = max(sum(T[r * nh:(r + 1) * nh]) for r in range(R))
    for tau in range(S * K, maxL + 1):
        plans = quota_conforming_plans(ids, E, R, S, tau)
        assert len(plans) == 1, (tau, len(plans))
        reps = replicas_of(plans[0], ids, E, R)
        if all(len([x for x in reps if x[1] == r]) <= B for r in range(R)):
            local = local_conforming_assignments(ids, E, R, S, plans[0])
            assert len(local) == 1, (tau, len(local))
            return tau, local[0]
    raise AssertionError("tau = max load always qualifies")


def local_conforming_assignments(ids, E, R, S, base):
    """Every map pair -> rank that keeps the instance quotas of `base` (the
    number of pairs of each expert on each rank) and meets the locality
    rule stated declaratively:
      (a) an instance (e, d) holds, of the pairs of e whose token comes from
          rank d, exactly the earliest min(quota, their number);
      (b) the pairs of e placed away from their own token's rank, taken by
          ascending flat index, go to instances in non-decreasing order
          (home first, then replicas by ascending rank).
    Returns the assignments found (the rule admits exactly one)."""
    K = len(ids[0])
    nh = E // R
    pairs = pair_list(ids)
    src = {f: (f // K) // S for (f, _) in pairs}
    quota = {}
    for (f, e) in pairs:
        quota[(e, base[f])] = quota.get((e, base[f]), 0) + 1
    ranks_of = {e: sorted({d for (x, d) in quota if x == e}, key=lambda d: (d != e // nh, d))
                for e in range(E)}
    found = []
    for asg in itertools.product(*[ranks_of[e] for (_, e) in pairs]):
        asg = dict(zip([f for (f, _) in pairs], asg))
        got = {}
        for (f, e) in pairs:
            got[(e, asg[f])] = got.get((e, asg[f]), 0) + 1
        if got != quota:
            continue
        ok = True
        for e in range(E):
            fs = [f for (f, x) in pairs if x == e]
            for d in ranks_of[e]:
                own = [f for f in fs if src[f] == d]
                if [f for f in own if asg[f] == d] != own[:min(quota[(e, d)], len(own))]:
                    ok = False
            order = [ranks_of[e].index(asg[f]) for f in fs if asg[f] != src[f]]
            if order != sorted(order):
                ok = False
        if ok:
            found.append(tuple(asg[f] for (f, _) in pairs))
    return found
