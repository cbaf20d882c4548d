"""CPU oracle for the redistribution of kept pairs onto replicas -- TEST
INFRASTRUCTURE ONLY.

Only the test suite may import this module; the product path never calls it,
and it imports nothing from the product package.

Source: the bullet on redistribution in the section on what LRMoE does, on the
Russian page ("Перераспределение") and the French page ("Redistribution").
After selection, an integer algorithm spreads each expert's remaining pairs
over the admissible copies of that expert, with the aim of minimising the peak
load on any single GPU; no new replica is created during the backward pass.
The kept rows are then packed into dense blocks per receiver and expert
(bullet on physical compaction, same section).

Reading of the pages (they give no formula):
  * GPUs g = 0..G-1; expert e has M_e kept pairs and a fixed admissible set
    R_e (the GPUs holding a copy of e, planned by the controller before the
    backward pass).
  * An assignment is a set of integers x[e][g] >= 0 with x[e][g] = 0 for g not
    in R_e and sum_g x[e][g] = M_e.
  * The load of GPU g is base[g] + sum_e x[e][g], in pairs (the experts of one
    layer have equal shapes, so a pair costs the same work on any replica);
    base[g] >= 0 is load the GPU already carries (zero by default).
  * Capacity-aware: GPU g may take at most cap[g] pairs (unlimited by default).
  * Objective: the minimum over assignments of max_g load(g).
  * This is a transportation problem, so integral optima exist.  The optimal
    peak is unique; the assignment reaching it generally is not.
  * Receiver-major packing: receiver g's block holds experts e = 0..E-1 in
    order, x[e][g] rows each; an expert's kept rows (in packed order) go to its
    replicas in ascending g, the first x[e][g0] rows to the lowest g0, and so
    on.

Everything here is plain Python on small integer arrays.
"""

from __future__ import annotations

import itertools
from collections import deque

import numpy as np


class Infeasible(ValueError):
    """Some kept pairs cannot be placed (no replica, or capacities too small)."""


def _norm(M, R, base, cap):
    M = np.asarray(M, dtype=np.int64)
    R = np.asarray(R, dtype=bool)
    E, G = R.shape
    assert M.shape == (E,) and (M >= 0).all()
    base = np.zeros(G, np.int64) if base is None else np.asarray(base, dtype=np.int64)
    cap = None if cap is None else np.asarray(cap, dtype=np.int64)
    return M, R, base, cap, E, G


def _max_flow(n, edges, s, t):
    """Edmonds-Karp maximum flow on a small graph.  edges: list of (u, v,
    capacity).  Returns (flow value, flow on each edge in input order)."""
    graph = [[] for _ in range(n)]
    to, capr, rev = [], [], []

    def add(u, v, c):
        graph[u].append(len(to)); to.append(v); capr.append(c); rev.append(len(to))
        graph[v].append(len(to)); to.append(u); capr.append(0); rev.append(len(to) - 2)

    for u, v, c in edges:
        add(u, v, c)
    orig = list(capr)
    total = 0
    while True:
        prev = [-1] * n
        prev[s] = -2
        q = deque([s])
        while q and prev[t] == -1:
            u = q.popleft()
            for a in graph[u]:
                if capr[a] > 0 and prev[to[a]] == -1:
                    prev[to[a]] = a
                    q.append(to[a])
        if prev[t] == -1:
            break
        # bottleneck along the path
        f, v = None, t
        while v != s:
            a = prev[v]
            f = capr[a] if f is None else min(f, capr[a])
            v = to[rev[a]]
        v = t
        while v != s:
            a = prev[v]
            capr[a] -= f
            capr[rev[a]] += f
            v = to[rev[a]]
        total += f
    return total, [orig[2 * i] - capr[2 * i] for i in range(len(edges))]


def _feasible(M, R, base, cap, T):
    """Max flow source -> expert e (M_e) -> GPU g in R_e -> sink
    (min(cap_g, T - base_g)); feasible iff it carries every kept pair."""
    E, G = R.shape
    s, t = E + G, E + G + 1
    edges = [(s, e, int(M[e])) for e in range(E)]
    pair_edges = [(e, g) for e in range(E) for g in range(G) if R[e, g]]
    big = int(M.sum()) + 1
    edges += [(e, E + g, big) for e, g in pair_edges]
    for g in range(G):
        room = max(0, int(T - base[g]))
        if cap is not None:
            room = min(room, int(cap[g]))
        edges.append((E + g, t, room))
    value, flows = _max_flow(E + G + 2, edges, s, t)
    x = np.zeros((E, G), np.int64)
    for (e, g), f in zip(pair_edges, flows[E:E + len(pair_edges)]):
        x[e, g] = f
    return value == int(M.sum()), x


def min_peak(M, R, base=None, cap=None):
    """Optimal peak load and one assignment reaching it (binary search on the
    peak T, each T checked by a maximum flow)."""
    M, R, base, cap, E, G = _norm(M, R, base, cap)
    for e in range(E):
        if M[e] > 0 and not R[e].any():
            raise Infeasible(f"expert {e} keeps {M[e]} pairs but has no replica")
    lo = int(base.max()) if G else 0
    hi = lo + int(M.sum())
    ok, x = _feasible(M, R, base, cap, hi)
    if not ok:
        raise Infeasible("capacities cannot hold the kept pairs")
    while lo < hi:
        mid = (lo + hi) // 2
        ok, xm = _feasible(M, R, base, cap, mid)
        if ok:
            hi, x = mid, xm
        else:
            lo = mid + 1
    if hi != lo or not _feasible(M, R, base, cap, lo)[0]:
        raise AssertionError("binary search invariant")
    ok, x = _feasible(M, R, base, cap, lo)
    return lo, x


def hall_peak(M, R, base=None, cap=None):
    """The optimal peak from the cut condition alone (no flow): for every
    non-empty GPU subset S, the pairs of experts whose replicas all lie in S
    must fit into S, sum_{g in S} min(cap_g, max(0, T - base_g)) >= D(S); the
    optimum is the largest over S of the smallest such T (and at least the
    largest base load).  Exponential in G: for small cases."""
    M, R, base, cap, E, G = _norm(M, R, base, cap)
    best = int(base.max()) if G else 0
    for k in range(1, G + 1):
        for S in itertools.combinations(range(G), k):
            inS = np.zeros(G, bool)
            inS[list(S)] = True
            D = int(sum(M[e] for e in range(E) if R[e].any() and not (R[e] & ~inS).any()))
            if D == 0:
                continue

            def room(T):
                r = 0
                for g in S:
                    v = max(0, T - int(base[g]))
                    r += v if cap is None else min(v, int(cap[g]))
                return r

            hi = int(base.max()) + D
            if room(hi) < D:
                raise Infeasible("capacities cannot hold the kept pairs")
            lo = 0
            while lo < hi:
                mid = (lo + hi) // 2
                if room(mid) >= D:
                    hi = mid
                else:
                    lo = mid + 1
            best = max(best, lo)
    return best


def brute_force_peak(M, R, base=None, cap=None):
    """The optimal peak by enumerating every assignment (tiny cases only)."""
    M, R, base, cap, E, G = _norm(M, R, base, cap)

    def splits(m, gs):
        if not gs:
            if m == 0:
                yield ()
            return
        if len(gs) == 1:
            yield (m,)
            return
        for a in range(m + 1):
            for rest in splits(m - a, gs[1:]):
                yield (a,) + rest

    per_expert = []
    for e in range(E):
        gs = [g for g in range(G) if R[e, g]]
        if M[e] > 0 and not gs:
            raise Infeasible(f"expert {e} has no replica")
        per_expert.append([(gs, sp) for sp in splits(int(M[e]), gs)] if gs else [([], ())])
    best = None
    for choice in itertools.product(*per_expert):
        load = base.copy()
        for gs, sp in choice:
            for g, a in zip(gs, sp):
                load[g] += a
        if cap is not None and ((load - base) > cap).any():
            continue
        peak = int(load.max()) if G else 0
        best = peak if best is None else min(best, peak)
    if best is None:
        raise Infeasible("capacities cannot hold the kept pairs")
    return best


def check_assignment(M, R, x, base=None, cap=None):
    """Peak load of a valid assignment x (raises AssertionError if invalid)."""
    M, R, base, cap, E, G = _norm(M, R, base, cap)
    x = np.asarray(x, dtype=np.int64)
    assert x.shape == (E, G)
    assert (x >= 0).all(), "negative share"
    assert (x[~R] == 0).all(), "pairs on a GPU without a replica"
    assert (x.sum(axis=1) == M).all(), "an expert's shares do not add up to its kept pairs"
    if cap is not None:
        assert (x.sum(axis=0) <= cap).all(), "capacity exceeded"
    return int((base + x.sum(axis=0)).max()) if G else 0


def receiver_layout(offsets, x):
    """Receiver-major packing of expert-major packed rows.

    offsets[E+1]: expert e's kept rows are offsets[e] .. offsets[e+1]-1.
    x[E][G]: the assignment (row sums equal the kept counts).
    Returns send_off[G+1] (first row of receiver g's block), blk_off[G][E+1]
    (first row of expert e's block inside receiver g's block, relative to
    send_off[g]) and dst[M] (receiver-major row of each expert-major row)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    x = np.asarray(x, dtype=np.int64)
    E, G = x.shape
    M = int(offsets[-1])
    assert (x.sum(axis=1) == np.diff(offsets)).all()
    send_off = np.zeros(G + 1, np.int64)
    blk_off = np.zeros((G, E + 1), np.int64)
    for g in range(G):
        for e in range(E):
            blk_off[g, e + 1] = blk_off[g, e] + x[e, g]
        send_off[g + 1] = send_off[g] + blk_off[g, E]
    dst = np.full(M, -1, np.int64)
    for e in range(E):
        j = int(offsets[e])
        for g in range(G):
            for k in range(int(x[e, g])):
                dst[j] = send_off[g] + blk_off[g, e] + k
                j += 1
    return send_off, blk_off, dst
