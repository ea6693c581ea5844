"""GOOSE's adaptive spine topology, step by step (GOOSE page, section 2, A-C).

Test infrastructure: this is the oracle's own reading of the policy, written apart from the
device path's host policy; the tests check that both give the same topologies.

Per step, with a budget of B draft nodes:
1. if the moving average of the spine acceptance rate is at least the bypass level, the
   step is a chain of B spine tokens and no branches (bypass mode);
2. otherwise the spine takes round(r * B) nodes (at least 1), r being the average held
   within [r_min, r_max] (dynamic spine ratio);
3. the remaining B - L nodes are branches whose widths fall linearly with depth
   (Proposition 2): fork j (0 = root) is weighted L - j; each fork first gets the whole
   part of its share, then the leftover nodes go one each to the forks with the largest
   fractional parts, shallower first on ties;
4. after verification, a spine whose first k tokens were accepted and then broke suggests a
   per-token rate k/(k+1) (1 if none broke); the batch's mean rate enters the average with
   weight 1 - beta.
"""
from __future__ import annotations

import math


def branch_widths(L, nodes):
    if L < 1 or nodes < 1:
        return [0] * max(L, 0)
    tot = L * (L + 1) // 2          # sum of the weights L, L-1, ..., 1
    exact = [nodes * (L - j) / tot for j in range(L)]
    w = [math.floor(x) for x in exact]
    left = nodes - sum(w)
    ranked = sorted(range(L), key=lambda j: (w[j] - exact[j], j))   # largest fraction first
    for j in ranked[:left]:
        w[j] += 1
    return w


def plan(avg, B, r_min=0.1, r_max=0.9, bypass=0.9):
    if avg >= bypass:
        return B, [0] * B
    r = r_min if avg < r_min else (r_max if avg > r_max else avg)
    L = int(round(r * B))
    L = 1 if L < 1 else (B if L > B else L)
    return L, branch_widths(L, B - L)


def update(avg, spine_runs, L, beta=0.8):
    rates = []
    for k in spine_runs:
        rates.append(1.0 if k >= L else k / (k + 1.0))
    return beta * avg + (1.0 - beta) * (sum(rates) / len(rates))


def spine_run(path, L):
    """Accepted spine tokens: the path's nodes among the spine slots 1..L."""
    n = 0
    for v in path[1:]:
        if 1 <= v <= L:
            n += 1
    return n
