"""Pure-Python brute force for tiny heads (test infrastructure only).

Written independently of ``rkv_oracle`` from the same passages and readings
(see that module's header): explicit loops, ``math.exp`` and ``math.fsum``,
no numpy. It pins the numpy oracle on small inputs, and its selection is an
exhaustive search over every subset of the budget's size, so it checks the
top-k by a route that does not sort.
"""
from __future__ import annotations

import itertools
import math


def _dot(a, b):
    return math.fsum(x * y for x, y in zip(a, b))


def importance_bf(K, Q, window, causal=True, pool="max"):
    """K: list of N rows; Q: [G][w] rows. Returns list of N floats.
    causal=False: every window query sees all keys; pool="mean": mean over
    the G heads instead of max."""
    n = len(K)
    d = len(K[0])
    G = len(Q)
    scale = 1.0 / math.sqrt(d)
    per_head = []
    for g in range(G):
        acc = [0.0] * n
        for r in range(window):
            # last visible key of window query r
            last = n - window + r if causal else n - 1
            logits = [_dot(Q[g][r], K[j]) * scale for j in range(last + 1)]
            m = max(logits)
            ex = [math.exp(v - m) for v in logits]
            tot = math.fsum(ex)
            for j in range(last + 1):
                acc[j] += ex[j] / tot
        per_head.append([a / window for a in acc])
    if pool == "mean":
        return [math.fsum(per_head[g][j] for g in range(G)) / G for j in range(n)]
    return [max(per_head[g][j] for g in range(G)) for j in range(n)]


def redundancy_bf(K, symmetric=False):
    """R_i = max of cos(k_i, k_j) over j < i (symmetric: over j != i); 0 when
    there is no such j."""
    n = len(K)
    norms = [math.sqrt(_dot(k, k)) for k in K]
    R = [0.0] * n
    for i in range(n):
        others = [j for j in range(n) if j != i] if symmetric else list(range(i))
        if not others:
            continue
        best = -math.inf
        for j in others:
            den = norms[i] * norms[j]
            c = _dot(K[i], K[j]) / den if den > 0 else 0.0
            best = max(best, c)
        R[i] = best
    return R


def select_bf(Z, n, budget, window):
    """Exhaustive: among (B-w)-subsets of the non-window candidates, the one with
    the largest exact sum of Z; among equal sums, the lexicographically
    smallest ascending index tuple. The window is added back."""
    if n <= budget:
        return list(range(n))
    cand = n - window
    best_sum = None
    best = None
    for combo in itertools.combinations(range(cand), budget - window):
        s = math.fsum(Z[i] for i in combo)
        if best_sum is None or s > best_sum or (s == best_sum and combo < best):
            best_sum, best = s, combo
    return sorted(list(best) + list(range(cand, n)))


def compress_head_bf(K, V, Q, budget, window, lam, symmetric=False, causal=True, pool="max"):
    n = len(K)
    if n <= budget:
        kept = list(range(n))
        return dict(kept=kept, I=None, R=None, Z=None,
                    K_out=[K[i] for i in kept], V_out=[V[i] for i in kept])
    I = importance_bf(K, Q, window, causal=causal, pool=pool)
    R = redundancy_bf(K, symmetric=symmetric)
    Z = [lam * a - (1.0 - lam) * b for a, b in zip(I, R)]
    kept = select_bf(Z, n, budget, window)
    return dict(kept=kept, I=I, R=R, Z=Z, K_out=[K[i] for i in kept],
                V_out=[V[i] for i in kept])


def select_shared_bf(Zs, n, budget, window):
    """Head-shared selection by exhaustive search: the (B-w)-subset S of the
    non-window candidates with the largest sum over heads h and members i of
    Z[h][i]; among equal sums the lexicographically smallest index tuple."""
    if n <= budget:
        return list(range(n))
    cand = n - window
    best_sum = None
    best = None
    for combo in itertools.combinations(range(cand), budget - window):
        s = math.fsum(Z[i] for Z in Zs for i in combo)
        if best_sum is None or s > best_sum or (s == best_sum and combo < best):
            best_sum, best = s, combo
    return sorted(list(best) + list(range(cand, n)))


def compress_shared_bf(Ks, Vs, Qs, budget, window, lam, **variant):
    """Ks, Vs: [H] lists of N rows; Qs: [H][G][w] rows."""
    n = len(Ks[0])
    if n <= budget:
        return dict(kept=list(range(n)), Z=None)
    Zs = [compress_head_bf(K, V, Q, budget, window, lam, **variant)["Z"]
          for K, V, Q in zip(Ks, Vs, Qs)]
    return dict(kept=select_shared_bf(Zs, n, budget, window), Z=Zs)
