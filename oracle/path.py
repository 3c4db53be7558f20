"""Plain, slow CPU oracle of the load-balanced MoE token path.

TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and imports nothing from it; the product path never calls it.

Every step is written from the pages' description, in their notation:

  S tokens per rank, K experts per token, E routed experts, R ranks (each
  owning E/R "home" experts), B prefetch slots per rank, T_e pairs routed to
  expert e, T̄ = mean of T_e, max_vio = max_e T_e/T̄ - 1.

Sources (page title, then section):
  [MoonEP-GR]  TWO DOTS, "MoonEP: πώς η εξισορρόπηση των AI experts αλλάζει
               την υποδομή των MoE μοντέλων"
  [MoonEP-FR]  hamidun.com news, "Moonshot AI открыла код MoonEP ..."
  [UltraEP]    remio.ai, "Xiaohongshuと北京大学がUltraEPを発表、静的MoE負荷分散に挑戦"
  [AlignSort]  新智元 article on SGLang's MoE Align & Sort kernel

Where the pages leave a step open, the plain reading taken is stated at the
function.  Floating point is fp64 except where the method itself fixes fp32
(the top-K key is an fp32 value; bf16 rows widen exactly to fp32).

Parity pins (see tests/test_oracle_*.py): brute-force top-K, closed-form gates,
numpy bincount, hand-derived plans W1-W3 (fixed rule) and Q1-Q4 (quota rule,
with its locality step), brute-force enumeration of rule-conforming plans
under both rules and of the locality rule stated declaratively, the
balanced-routing special case (textbook stable counting sort), the
one-expert-per-rank reduction of the quota rule to the fixed rule, invariants,
the identity-expert closed form for combine; for the training side the
hand-derived replica lists (prefetch, reduce_grad), exact integer
conservation and line-order sensitivity of reduce_grad, central differences
and adjoint identities for the backward.
Gate values' last fp32 bit is pinned only to 1e-6 relative (parity partially
unpinned there); rows past each rank's padded end are unspecified.
"""
from __future__ import annotations

import numpy as np

SOFTMAX = 0
SIGMOID = 1
UNSPECIFIED = -2          # marker for sorted_ids rows the method leaves undefined


# --------------------------------------------------------------------------- O1
def route_topk(logits, K, score_fn, sel_bias=None, renorm=False):
    """Router top-K.  [AlignSort] (the MoE layer gates each token to its Top-K
    experts by gate score, with DeepSeek's per-expert gating bias) and
    [MoonEP-GR] section "Γιατί τα Mixture-of-Experts δημιουργούν πρόβλημα
    κατανομής" (the router picks each token's top K experts).

    Readings: the selection key is the fp32 value logit[t,e] (+ sel_bias[e],
    one fp32 round-to-nearest-even add); experts are ordered by key
    descending, ties (IEEE equality, so -0.0 == +0.0) to the lower expert
    index; the output keeps that order.  The gating bias only steers
    selection: gates are score_fn of the raw logit (sigmoid, or softmax over
    all E raw logits), optionally renormalised over the K chosen.  NaN keys
    are not allowed.

    Returns ids int32 [N,K] and gates fp64 [N,K].
    """
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    N, E = logits.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    key = logits
    if sel_bias is not None:
        key = logits + np.asarray(sel_bias, dtype=np.float32)[None, :]
    expert = np.broadcast_to(np.arange(E, dtype=np.int64), (N, E))
    # lexsort: last key is primary -> descending key, then ascending expert
    order = np.lexsort((expert, -key), axis=-1)
    ids = order[:, :K].astype(np.int32)

    l64 = logits.astype(np.float64)
    if score_fn == SIGMOID:
        score = 1.0 / (1.0 + np.exp(-l64))
    elif score_fn == SOFTMAX:
        m = l64.max(axis=1, keepdims=True)
        ex = np.exp(l64 - m)
        score = ex / ex.sum(axis=1, keepdims=True)
    else:
        raise ValueError("score_fn")
    gates = np.take_along_axis(score, ids.astype(np.int64), axis=1)
    if renorm:
        gates = gates / gates.sum(axis=1, keepdims=True)
    return ids, gates


# --------------------------------------------------------------------------- O2
def load_matrix(ids, R, S, E):
    """Exact post-routing load matrix counts[src][e]: how many of source rank
    src's (token, expert) pairs chose expert e.  [UltraEP] section
    "その仕組みは高速なエキスパート複製に依存する" (the runtime starts from the
    exact load matrix of per-source-rank token counts per logical expert).
    Reading: token t belongs to source rank t // S."""
    ids = np.asarray(ids)
    N, K = ids.shape
    if N != R * S:
        raise ValueError("N != R*S")
    if ids.size and (ids.min() < 0 or ids.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.zeros((R, E), dtype=np.int64)
    src = np.repeat(np.arange(N, dtype=np.int64) // S, K)
    np.add.at(counts, (src, ids.reshape(-1).astype(np.int64)), 1)
    return counts


def imbalance(counts, S, K):
    """max_vio = max_e(T_e / T̄) - 1 with T̄ the mean per-expert load
    ([MoonEP-FR] "Pourquoi le parallélisme d'experts est-il nécessaire";
    [MoonEP-GR] maxvio, zero = perfect balance) and the per-rank view
    max_r L_r / (S K) - 1 of the same skew before balancing."""
    counts = np.asarray(counts, dtype=np.int64)
    R, E = counts.shape
    T = counts.sum(axis=0)
    P = int(T.sum())
    nh = E // R
    L = T.reshape(R, nh).sum(axis=1)
    Tbar = P / E
    return {
        "T": T,
        "L": L,
        "max_vio": float(T.max() / Tbar - 1.0) if P else 0.0,
        "rank_imbalance": float(L.max() / (S * K) - 1.0) if P else 0.0,
    }


# --------------------------------------------------------------------------- O3
def capacity(E, K, S, blk, cap=0, tau_max=0):
    """Static rows per rank of the receive buffer.  A plan gives each rank at
    most tau_max real rows (tau_max = S*K, the exact-balance contract, unless
    the caller allows more), in at most min(E, tau_max) non-empty expert
    segments, each padded to a multiple of blk; so tau_max + min(E, tau_max)
    * (blk-1) rows, rounded up to blk, always suffice.  Static shapes:
    [MoonEP-GR] section "Online planning, zero copy και στατικά σχήματα".  A
    caller may ask for a smaller cap."""
    if cap:
        return int(cap)
    t = int(tau_max) if tau_max else S * K
    need = t + min(E, t) * (blk - 1)
    return ((need + blk - 1) // blk) * blk


def _split_stream_tail(T, R, tau):
    """Fixed rule: rank r keeps the first min(L_r, tau) pairs of its home
    stream (its experts ascending, each expert's pairs by ascending flat index
    f), so the overflow is the stream's tail.  The overflow line lists the
    experts in ascending order.  Returns (h, o, line order of experts)."""
    E = len(T)
    nh = E // R
    h = np.zeros(E, dtype=np.int64)
    o = np.zeros(E, dtype=np.int64)
    for r in range(R):
        Pe = 0
        for e in range(r * nh, (r + 1) * nh):
            h[e] = min(max(tau - Pe, 0), T[e])
            o[e] = T[e] - h[e]
            Pe += T[e]
    return h, o, list(range(E))


def _split_hot_first(T, R, tau):
    """Quota rule ([UltraEP] section "その仕組みは高速なエキスパート複製に依存する":
    the quota planner decides which hot experts get copies and how many tokens
    each instance takes).  Reading: an overloaded rank r sheds L_r - tau
    pairs, taking them from its hottest experts first (load descending, ties
    to the lower expert index), each expert shedding all it has before the
    next one sheds any; each expert keeps its first h_e pairs (by f).  The
    overflow line lists the experts rank by rank (ascending), in that
    shedding order inside a rank."""
    E = len(T)
    nh = E // R
    h = np.zeros(E, dtype=np.int64)
    o = np.zeros(E, dtype=np.int64)
    order = []
    for r in range(R):
        mine = list(range(r * nh, (r + 1) * nh))
        shed = max(int(sum(T[e] for e in mine)) - tau, 0)
        hot = sorted(mine, key=lambda e: (-int(T[e]), e))
        for e in hot:
            o[e] = min(int(T[e]), shed)
            shed -= o[e]
            h[e] = T[e] - o[e]
        order.extend(hot)
    return h, o, order


def _place(counts, K, S, B, blk, C, tau, split):
    """Lay the overflow and the deficits on one line and build the plan.

    [MoonEP-GR] sections "Η βασική υπόσχεση του MoonEP: σταθερό φορτίο S × K"
    (a few temporary expert copies on other ranks, planned online from the
    current router output) and "Το memory contract ..." (weight rows 0..E-1
    hold the ranks' experts, rows E..E+B-1 are local prefetch slots found by
    row index; when remote experts exceed the slots they are read from the
    home rank, still correct).  [UltraEP] "その仕組みは..." (replicas exist only
    when the plan gives them work; per-token destinations come from
    cumulative quotas).

    Rank r keeps min(L_r, tau) pairs (which ones: `split`) and has deficit
    def_r = tau - min(L_r, tau).  Readings taken:
      * home experts of rank r are [r*E/R, (r+1)*E/R);
      * the overflow stream lists (expert e, o_e) for o_e > 0 in the split's
        line order; the deficit stream lists ranks with def_r > 0 in
        ascending r; both are laid on one line (O_e = start of e's overflow,
        D_r = start of r's deficit) and every non-empty intersection
        [O_e, O_e+o_e) ∩ [D_d, D_d+def_d) is one replica segment (e, d,
        count); with tau > S*K the deficit line is longer than the overflow
        line and its tail stays unused;
      * on rank d the replica segments, in line order, take prefetch slots
        0..B-1 (weight row E+j); further ones are remote (weight row e);
      * the segment table of rank r is its E/R home experts ascending (count
        h_e, possibly 0) then its replica segments in line order; each count
        is padded up to a multiple of blk and the padded starts are the
        exclusive prefix sums (the cu_seqlens of the grouped GEMM).
    """
    counts = np.asarray(counts, dtype=np.int64)
    R, E = counts.shape
    if E % R:
        raise ValueError("E must be a multiple of R")
    nh = E // R
    SK = S * K

    T = counts.sum(axis=0)
    if int(T.sum()) != R * SK:
        raise ValueError("counts do not sum to R*S*K")

    # per-rank load and the keep / overflow / deficit split
    L = np.array([T[r * nh:(r + 1) * nh].sum() for r in range(R)], dtype=np.int64)
    keep = np.minimum(L, tau)
    over = L - keep
    deficit = tau - keep
    h, o, order = split(T, R, tau)

    # overflow line offsets O_e (in line order) and deficit offsets D_r
    O = np.zeros(E, dtype=np.int64)
    acc = 0
    for e in order:
        O[e] = acc
        acc += o[e]
    D = np.zeros(R + 1, dtype=np.int64)
    acc = 0
    for r in range(R):
        D[r] = acc
        acc += deficit[r]
    D[R] = acc

    # replica segments = non-empty intersections, in line order
    lo = np.maximum(O[:, None], D[None, :R])
    hi = np.minimum((O + o)[:, None], (D[:R] + deficit)[None, :])
    ee, dd = np.nonzero((hi > lo) & (o[:, None] > 0) & (deficit[None, :] > 0))
    reps = sorted(zip(lo[ee, dd].tolist(), ee.tolist(), dd.tolist(), (hi - lo)[ee, dd].tolist()))

    # per-rank segment tables
    segs = [[(e, e, int(h[e]), None) for e in range(r * nh, (r + 1) * nh)] for r in range(R)]
    n_slots = np.zeros(R, dtype=np.int64)
    n_remote = np.zeros(R, dtype=np.int64)
    replicas = []
    for (lo, e, d, c) in reps:
        j = n_slots[d] + n_remote[d]
        if j < B:
            wrow = E + j
            n_slots[d] += 1
        else:
            wrow = e
            n_remote[d] += 1
        segs[d].append((e, wrow, c, lo))
        replicas.append({"expert": e, "rank": d, "count": c, "line": lo, "wrow": wrow})

    pad = lambda c: ((c + blk - 1) // blk) * blk  # noqa: E731
    seg_tables = []
    n_rows_padded = np.zeros(R, dtype=np.int64)
    home_row = np.zeros(E, dtype=np.int64)
    rep_row = {}
    for r in range(R):
        start = 0
        table = []
        for (e, wrow, c, lo) in segs[r]:
            table.append({"expert": e, "wrow": wrow, "count": c, "start": start})
            if lo is None:
                home_row[e] = start
            else:
                rep_row[(e, r)] = start
            start += pad(c)
        n_rows_padded[r] = start
        seg_tables.append(table)
    for rp in replicas:
        rp["row"] = rep_row[(rp["expert"], rp["rank"])]

    n_rep = n_slots + n_remote
    return {
        "E": E, "K": K, "R": R, "S": S, "B": B, "blk": blk, "C": C, "SK": SK, "tau": int(tau),
        "T": T, "L": L, "keep": keep, "over": over, "deficit": deficit,
        "h": h, "o": o, "O": O, "D": D, "line_order": order,
        "replicas": replicas, "segments": seg_tables,
        "n_rows_padded": n_rows_padded, "n_slots": n_slots, "n_remote": n_remote,
        "max_replicas": int(n_rep.max()) if R else 0,
        "home_row": home_row,
        "capacity_ok": bool(n_rows_padded.max() <= C) if R else True,
    }


def plan_balance(counts, K, S, B, blk, cap=0, tau_max=0):
    """Online redundant-expert plan giving every rank exactly S*K pairs
    (MoonEP's contract, [MoonEP-GR] "Η βασική υπόσχεση του MoonEP: σταθερό
    φορτίο S × K").  The fixed rule: home rank r keeps min(L_r, S*K) of its
    pairs, the first ones of its home stream; the overflow segments (experts
    ascending) fill deficit ranks in ascending order; see _place for the
    readings.  tau_max only sizes the static capacity C."""
    counts = np.asarray(counts, dtype=np.int64)
    R, E = counts.shape
    C = capacity(E, K, S, blk, cap, tau_max)
    p = _place(counts, K, S, B, blk, C, S * K, _split_stream_tail)
    p["rule"] = "fixed"
    p["feasible"] = p["max_replicas"] <= B
    p["home_local"] = np.zeros(E, dtype=np.int64)    # the fixed rule has no locality step
    p["local"] = False
    return p


def replicas_per_rank(counts, K, S, tau, split):
    """Replica segments each rank would hold at threshold tau (the same line
    construction as _place, counting only)."""
    counts = np.asarray(counts, dtype=np.int64)
    R, E = counts.shape
    T = counts.sum(axis=0)
    nh = E // R
    L = T.reshape(R, nh).sum(axis=1)
    deficit = tau - np.minimum(L, tau)
    h, o, order = split(T, R, tau)
    O = np.zeros(E, dtype=np.int64)
    acc = 0
    for e in order:
        O[e] = acc
        acc += o[e]
    D = np.concatenate([[0], np.cumsum(deficit)])
    lo = np.maximum(O[:, None], D[None, :R])
    hi = np.minimum((O + o)[:, None], (D[:R] + deficit)[None, :])
    return ((hi > lo) & (o[:, None] > 0) & (deficit[None, :] > 0)).sum(axis=0)


def plan_quota(counts, K, S, B, blk, tau_max=0, cap=0):
    """UltraEP-style quota plan with a searched threshold.

    [UltraEP] section "その仕組みは高速なエキスパート複製に依存する": from the
    exact post-routing load matrix the runtime searches a target workload
    threshold that keeps every rank under it within the available replica
    slots; a quota-driven planner decides which hot experts get copies, where
    they run and how many tokens each instance takes, creating a replica only
    when it gets work; per-token destinations come from a lookup against the
    cumulative quotas (align_sort, unchanged).

    Readings taken:
      * instances and quotas: at threshold tau every overloaded rank keeps
        tau pairs and sheds the rest from its hottest experts first
        (_split_hot_first); the deficit ranks (ascending) absorb the overflow
        up to tau each (_place), each intersection being one instance;
      * "within the replica slots" = no rank holds more than B replica
        segments, so no weight is read from a remote home;
      * the threshold is the smallest integer tau in [S*K, min(max_r L_r,
        tau_max)] meeting that (at tau = max_r L_r nothing moves, so the
        range always holds one when max_r L_r <= tau_max); the search is
        exhaustive because the condition is not monotone in tau;
      * if no tau <= tau_max qualifies, the plan at tau_max is used with the
        remote fallback for replicas beyond B ("feasible" False);
      * locality: the instance quotas above are split into pairs from the
        instance's own rank first (_local_counts); align_sort places them.
    tau_max = 0 means S*K (exact balance).
    """
    counts = np.asarray(counts, dtype=np.int64)
    R, E = counts.shape
    SK = S * K
    t_max = int(tau_max) if tau_max else SK
    if t_max < SK:
        raise ValueError("tau_max must be at least S*K")
    C = capacity(E, K, S, blk, cap, t_max)
    T = counts.sum(axis=0)
    L = T.reshape(R, E // R).sum(axis=1)
    hi = min(int(L.max()), t_max) if R else SK
    tau, feasible = t_max, False
    for t in range(SK, hi + 1):
        if replicas_per_rank(counts, K, S, t, _split_hot_first).max() <= B:
            tau, feasible = t, True
            break
    p = _place(counts, K, S, B, blk, C, tau, _split_hot_first)
    p["rule"] = "quota"
    p["feasible"] = feasible
    p["tau_max"] = t_max
    _local_counts(p, counts)
    return p


def _local_counts(plan, counts):
    """Locality of the quota plan ([UltraEP] "その仕組みは...": tokens use the
    capacity of local expert instances before the rest of the demand goes
    elsewhere).  Every instance of an expert (its home, then its replicas in
    line order) first serves the pairs that come from its own rank, up to
    its quota: home_local[e] = min(h_e, pairs of e from e's home rank), and
    each replica's "local" = min(count, pairs of e from the replica's rank).
    Reading: only an instance on the token's own rank counts as local (the
    pages give no node topology to rank other ranks as nearer)."""
    counts = np.asarray(counts, dtype=np.int64)
    R, E = counts.shape
    nh = E // R
    e_all = np.arange(E)
    plan["home_local"] = np.minimum(plan["h"], counts[e_all // nh, e_all])
    for rp in plan["replicas"]:
        rp["local"] = int(min(rp["count"], counts[rp["rank"], rp["expert"]]))
    plan["local"] = True


# --------------------------------------------------------------------------- O4
def align_sort(ids, plan):
    """Block-aligned sort of the (token, expert) pairs into each rank's expert
    segments.  [AlignSort]: pairs are sorted by expert id with every expert's
    share padded to the GEMM block so the grouped GEMM takes whole blocks; the
    permutation records the source -> destination map.  [UltraEP]: per-token
    destinations follow from a local lookup against cumulative quotas.

    For pair f = t*K + k with e = ids[t,k] and q = #{f' < f : ids[f'] = e}:
      q < h_e  -> home rank of e, row = home start of e + q
      q >= h_e -> o = O_e + (q - h_e); d is the rank with D_d <= o < D_d+def_d;
                  row = start of e's replica segment on d + (o - max(O_e, D_d)).
    Under a quota plan (plan["local"]) the destinations follow its locality
    step instead (_place_local).
    slot[f] = d*C + row and sorted_ids[d*C + row] = f.  Readings: padding rows
    below a rank's padded end hold the sentinel P (one past the last pair);
    rows at or past the padded end are left unspecified (UNSPECIFIED here);
    block tables give, per blk-row block, the weight row and expert of the
    segment covering it, or -1 past the padded end.
    """
    ids = np.asarray(ids)
    N, K = ids.shape
    P = N * K
    E, R, C, blk = plan["E"], plan["R"], plan["C"], plan["blk"]
    nh = E // R
    h, O, D, deficit = plan["h"], plan["O"], plan["D"], plan["deficit"]
    flat = ids.reshape(-1).astype(np.int64)

    # q: stable rank of each pair inside its expert (library stable sort)
    order = np.argsort(flat, kind="stable")
    sorted_e = flat[order]
    group_start = np.searchsorted(sorted_e, sorted_e, side="left")
    q = np.empty(P, dtype=np.int64)
    q[order] = np.arange(P, dtype=np.int64) - group_start

    rep_start = np.full((E, R), -1, dtype=np.int64)
    for rp in plan["replicas"]:
        rep_start[rp["expert"], rp["rank"]] = rp["row"]

    if plan.get("local", False):
        d, row = _place_local(flat, plan, K)
        ov = np.zeros(P, dtype=bool)
    else:
        at_home = q < h[flat]
        d = np.where(at_home, flat // nh, 0)
        row = np.where(at_home, plan["home_row"][flat] + q, 0)
        ov = ~at_home
    if ov.any():
        e_ov = flat[ov]
        o_pos = O[e_ov] + (q[ov] - h[e_ov])
        # the deficit rank whose interval holds o_pos (ranks without deficit
        # have empty intervals and are never the last with D_d <= o_pos)
        d_ov = np.searchsorted(D[:R], o_pos, side="right") - 1
        assert np.all(D[d_ov] <= o_pos) and np.all(o_pos < D[d_ov] + deficit[d_ov])
        start = rep_start[e_ov, d_ov]
        assert np.all(start >= 0)
        d[ov] = d_ov
        row[ov] = start + (o_pos - np.maximum(O[e_ov], D[d_ov]))
    slot = d * C + row

    sorted_ids = np.full(R * C, UNSPECIFIED, dtype=np.int64)
    nb = C // blk
    block_wrow = np.full((R, nb), -1, dtype=np.int64)
    block_expert = np.full((R, nb), -1, dtype=np.int64)
    for r in range(R):
        for sg in plan["segments"][r]:
            plen = ((sg["count"] + blk - 1) // blk) * blk
            lo = r * C + sg["start"]
            sorted_ids[lo: lo + plen] = P                 # padding sentinel
            for b in range(sg["start"] // blk, (sg["start"] + plen) // blk):
                block_wrow[r, b] = sg["wrow"]
                block_expert[r, b] = sg["expert"]
    sorted_ids[slot] = np.arange(P, dtype=np.int64)
    return {"slot": slot, "sorted_ids": sorted_ids,
            "block_wrow": block_wrow, "block_expert": block_expert, "q": q}


# --------------------------------------------------------------------------- O5
def _place_local(flat, plan, K):
    """Per-pair (rank, row) of a quota plan with locality ([UltraEP]
    "その仕組みは...": tokens first use the capacity of local instances, then
    the remaining demand goes elsewhere; per-token destinations are a lookup
    against the cumulative quotas).  For expert e, with instances I_0 = home
    (quota h_e) and I_1.. = its replicas in line order (quota = count):
      1. each instance takes, up to its quota, the earliest (ascending f)
         pairs of e whose token comes from the instance's own rank;
      2. the pairs of e not taken in step 1, in ascending f, fill the
         instances' remaining quotas in instance order (home first);
      3. inside an instance's segment its step-1 pairs come first, then its
         step-2 pairs, each in ascending f.
    The token of pair f comes from rank (f // K) // S."""
    E, R, S = plan["E"], plan["R"], plan["S"]
    nh = E // R
    P = flat.size
    src = (np.arange(P) // K) // S
    d = np.zeros(P, dtype=np.int64)
    row = np.zeros(P, dtype=np.int64)
    reps_of = {e: [] for e in range(E)}
    for rp in plan["replicas"]:                       # line order
        reps_of[rp["expert"]].append(rp)
    for e in range(E):
        fs = np.nonzero(flat == e)[0]                 # ascending f
        if fs.size == 0:
            continue
        inst = [(e // nh, int(plan["h"][e]), int(plan["home_row"][e]))]
        inst += [(rp["rank"], int(rp["count"]), int(rp["row"])) for rp in reps_of[e]]
        taken = np.zeros(fs.size, dtype=bool)
        n_local = []
        for (rank, quota, row0) in inst:              # step 1
            mine = np.nonzero((src[fs] == rank) & ~taken)[0][:quota]
            taken[mine] = True
            d[fs[mine]] = rank
            row[fs[mine]] = row0 + np.arange(mine.size)
            n_local.append(mine.size)
        rest = np.nonzero(~taken)[0]                  # step 2, ascending f
        pos = 0
        for (rank, quota, row0), nl in zip(inst, n_local):
            sel = rest[pos:pos + quota - nl]
            d[fs[sel]] = rank
            row[fs[sel]] = row0 + nl + np.arange(sel.size)
            pos += quota - nl
        assert pos == rest.size, "instance quotas must add up to the expert's pairs"
    return d, row


def dispatch_rows(x_bits, slot, K):
    """Zero-copy dispatch: pair f's token row is written straight to its final
    expert-grouped row slot[f] of the static receive buffer ([MoonEP-GR]
    "Online planning, zero copy ..."; tokens land in their final positions,
    grouped per expert, and the caller gets views of that buffer).
    Returns {row: bf16 bits} as (rows, data) with data[i] = x[f // K]."""
    slot = np.asarray(slot, dtype=np.int64)
    f = np.arange(slot.size, dtype=np.int64)
    return slot, np.asarray(x_bits)[f // K]


def dispatch(x_bits, slot, K, R, C):
    """Full receive buffer [R*C, H] (bit copy); rows no pair maps to stay 0."""
    x_bits = np.asarray(x_bits)
    recv = np.zeros((R * C, x_bits.shape[1]), dtype=np.uint16)
    rows, data = dispatch_rows(x_bits, slot, K)
    recv[rows] = data
    return recv


# --------------------------------------------------------------------------- O6
def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)) \
        .view(np.float32).astype(np.float64)


def combine(out_rows_of, slot, gates, K, tokens=None):
    """Inverse of dispatch: y[t] = sum_k gates[t,k] * out[slot[t*K+k]] in
    ascending k ([MoonEP-GR]: combine returns the experts' results to their
    source tokens; [UltraEP]: tokens come back after expert compute).
    Computed in fp64 from the bf16 rows (exact widening) and the fp32 gates.
    ``out_rows_of(rows)`` returns bf16 bits of the requested rows of the
    expert-output buffer.  Returns fp64 y [len(tokens), H] and the fp64 sum
    of |g * out| per element (the scale of the rounding-error bound)."""
    slot = np.asarray(slot, dtype=np.int64)
    gates = np.asarray(gates, dtype=np.float32)
    N = gates.shape[0]
    tokens = np.arange(N) if tokens is None else np.asarray(tokens, dtype=np.int64)
    y = None
    mag = None
    for k in range(K):
        rows = slot[tokens * K + k]
        v = bf16_to_f64(out_rows_of(rows))
        g = gates[tokens, k].astype(np.float64)[:, None]
        term = g * v
        y = term if y is None else y + term
        mag = np.abs(term) if mag is None else mag + np.abs(term)
    return y, mag


# --------------------------------------------------------------------------- O7
def prefetch_slots(plan):
    """Which expert's weights every used prefetch slot must hold.

    [MoonEP-GR] section "Το memory contract ...": one contiguous weight tensor
    [E+B, H, H'] per expert projection; rows 0..E-1 hold the ranks' experts,
    rows E..E+B-1 are the rank's local prefetch slots, found by row index;
    the prefetch pool is process-global (shared by the layers); replicas
    beyond the slots read their weights from the home rank.  A replica
    segment of expert e on rank d with weight row E + j therefore needs
    slot j of rank d to hold e's weights; remote replicas need no slot.
    Returns {(d, j): e}."""
    E = plan["E"]
    return {(rp["rank"], rp["wrow"] - E): rp["expert"]
            for rp in plan["replicas"] if rp["wrow"] >= E}


def prefetch_weights(plan, weights, slots):
    """Copy home weight rows into the prefetch slots: slots[d, j] =
    weights[e] for every (d, j) -> e of prefetch_slots (a bit copy); slots
    the plan does not use are left as they were.  weights [E, ...],
    slots [R, B, ...] of the same element type.  Returns a new array."""
    slots = np.array(slots, copy=True)
    for (d, j), e in prefetch_slots(plan).items():
        slots[d, j] = weights[e]
    return slots


# --------------------------------------------------------------------------- O8
def f32_to_bf16_rne(a):
    """bf16 bits nearest to each finite fp32 value, ties to an even last bit:
    keep the upper 16 bits and round up when the dropped 16 bits exceed half
    a bf16 unit, or equal half with the kept last bit odd."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    keep = bits >> np.uint32(16)
    drop = bits & np.uint32(0xFFFF)
    up = (drop > 0x8000) | ((drop == 0x8000) & ((keep & np.uint32(1)) == 1))
    return (keep + up.astype(np.uint32)).astype(np.uint16)


def combine_bwd(out_rows_of, slot, gates, dy, K):
    """Gradient of combine, y[t] = sum_k g[t,k] out[slot[t*K+k]], with respect
    to the expert outputs and the gates.  [AlignSort]: permute records the
    source -> destination map and the gradient of unpermute is a permute
    (the same map run forward); [MoonEP-GR]: combine is the inverse of the
    zero-copy dispatch.  So

      d_out[slot[t*K+k]] = g[t,k] * dy[t]      (a dispatch of the scaled
                                                output gradient into the
                                                expert-grouped rows)
      d_g[t,k]          = sum_h dy[t,h] * out[slot[t*K+k], h]

    Precision readings: d_out rows are bf16, like the expert outputs: the
    fp32 product of the fp32 gate and the fp32 output gradient, rounded to
    nearest even; d_g is computed in fp64 (then rounded once to fp32 by the
    caller) with sum_h |dy * out| returned as the scale of its error bound.
    dy is fp32 [N, H] (bf16 inputs widen to it exactly).
    Returns (d_out bits [P, H] in pair order, d_g fp64 [N, K], mag [N, K])."""
    slot = np.asarray(slot, dtype=np.int64)
    g32 = np.asarray(gates, dtype=np.float32)
    dy32 = np.asarray(dy, dtype=np.float32)
    N = g32.shape[0]
    f = np.arange(N * K, dtype=np.int64)
    t = f // K
    # one fp32 product (the exact product of two fp32 numbers fits in fp64)
    prod = (g32.reshape(-1)[:, None].astype(np.float64) * dy32[t].astype(np.float64)).astype(np.float32)
    d_out = f32_to_bf16_rne(prod)
    d_g = np.empty((N, K), dtype=np.float64)
    mag = np.empty((N, K), dtype=np.float64)
    for k in range(K):
        v = bf16_to_f64(out_rows_of(slot[np.arange(N) * K + k]))
        terms = dy32.astype(np.float64) * v
        d_g[:, k] = terms.sum(axis=1)
        mag[:, k] = np.abs(terms).sum(axis=1)
    return d_out, d_g, mag


def dispatch_bwd(d_recv_rows_of, slot, K, N):
    """Gradient of dispatch, recv[slot[t*K+k]] = x[t], with respect to x:
    dx[t] = sum_k d_recv[slot[t*K+k]] ([AlignSort]: the backward of a permute
    gathers the K copies back to their token), in ascending k, fp64 from the
    bf16 rows.  Returns fp64 dx [N, H] and sum_k |d_recv| (error-bound
    scale)."""
    slot = np.asarray(slot, dtype=np.int64)
    dx = None
    mag = None
    for k in range(K):
        v = bf16_to_f64(d_recv_rows_of(slot[np.arange(N) * K + k]))
        dx = v if dx is None else dx + v
        mag = np.abs(v) if mag is None else mag + np.abs(v)
    return dx, mag


# --------------------------------------------------------------------------- O9
def reduce_grad(plan, slot_grads, grads):
    """Fold the replicas' weight gradients back into their home experts.

    [MoonEP-GR] section "Τι συμβαίνει στους gradients κατά την εκπαίδευση":
    training keeps an fp32 gradient buffer laid out like the weights
    ([E+B, H, H']); the prefetched slots do not write into the parameter
    gradients but into a separate reduce buffer, seen over all ranks as
    [R, B, H, H']; reduce_grad reads the slots that belong to each rank's
    own experts, adds them to the parameter gradient and clears the used
    slots before the next micro-batch.

    Readings: for expert e its used slots are added in line order
    (ascending rank), one fp32 addition each: G[e] = ((G[e] + s_1) + s_2)...;
    remote replicas hold no slot (their gradient is the caller's to route);
    unused slots are left as they were.
    slot_grads fp32 [R, B, ...], grads fp32 [E, ...].  Returns new arrays
    (grads', slot_grads')."""
    E = plan["E"]
    grads = np.array(grads, dtype=np.float32, copy=True)
    slot_grads = np.array(slot_grads, dtype=np.float32, copy=True)
    used = []
    for rp in plan["replicas"]:                 # line order
        if rp["wrow"] >= E:
            d, j = rp["rank"], rp["wrow"] - E
            grads[rp["expert"]] = grads[rp["expert"]] + slot_grads[d, j]
            used.append((d, j))
    for d, j in used:
        slot_grads[d, j] = 0.0
    return grads, slot_grads
