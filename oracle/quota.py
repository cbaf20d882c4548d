"""CPU oracle for the quota controller -- TEST INFRASTRUCTURE ONLY.

Only the test suite may import this module; the product path never calls it.

Source: the bullet on quotas in the section on what LRMoE does, on the Russian
page ("Квоты до вычислений") and the French page ("Des quotas avant le
calcul"): before the backward pass a controller sees how many tokens reached
each expert and, given the memory and network limits, decides how many pairs
of each expert to keep; the quota is fixed for the whole layer call.

Reading (the pages give no formula): the limits are one budget B of pairs this
GPU may carry through the backward pass.  Quotas are water-filling caps, which
trim the most loaded experts first:
  * tau is the largest integer with sum_e min(n_e, tau) <= B;
  * q_e = min(n_e, tau), plus one for the first r experts (lowest index) with
    n_e > tau, where r = B - sum_e min(n_e, tau);
  * so sum_e q_e = min(B, N), every q_e <= n_e, and an expert that is cut
    keeps at least as many pairs as any other expert, minus one.
"""

from __future__ import annotations

import itertools

import numpy as np


def waterfill(counts, budget):
    """Quotas q[E] for candidate counts n[E] and a pair budget B >= 0."""
    n = np.asarray(counts, dtype=np.int64)
    assert (n >= 0).all() and budget >= 0
    if budget >= n.sum():
        return n.copy()
    # largest tau with sum(min(n, tau)) <= budget, by bisection on tau
    lo, hi = 0, int(n.max())
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if np.minimum(n, mid).sum() <= budget:
            lo = mid
        else:
            hi = mid - 1
    tau = lo
    q = np.minimum(n, tau)
    r = int(budget - q.sum())
    for e in range(len(n)):
        if r == 0:
            break
        if n[e] > tau:
            q[e] += 1
            r -= 1
    return q


def brute_force_min_max(counts, budget):
    """Smallest possible max_e q_e over all q with 0 <= q_e <= n_e and
    sum q = min(B, N) (tiny cases only)."""
    n = [int(v) for v in counts]
    total = min(budget, sum(n))
    best = None
    for q in itertools.product(*[range(v + 1) for v in n]):
        if sum(q) == total:
            m = max(q) if q else 0
            best = m if best is None else min(best, m)
    return best
