"""Verification of a draft tree: greedy matching and Leviathan rejection sampling.

Both walk the tree from the root. ``target(r)`` and ``draft(r)`` return float64 logit
rows; node i reads row ``row[i]`` of each table. Every result is a path (slots, root
first), the number of accepted draft tokens A = len(path) - 1, and the bonus token
emitted after the path (the target's correction or continuation, which becomes the
next root and is not written to the cache).
"""
from __future__ import annotations

import numpy as np

from .mask import ancestors
from .rows import row_max_argmax, row_softmax


def greedy(parent, token, row, target) -> dict:
    """Greedy verification (OPT-Tree summary, section 2; GOOSE page, section 2C).

    Under greedy decoding the accepted branch is the longest one that agrees with the
    target's highest-probability token at every step:

    * a[v] = argmax of the target row at v (lowest index on ties);
    * node c matches when token[c] == a[parent[c]];
    * a node is valid when every node on its path below the root matches;
    * the accepted node v* is the deepest valid node, the lowest slot among equals
      (GOOSE's unified walk prefers the spine, which holds the lowest slots);
    * A = depth(v*), path = root .. v*, bonus = a[v*].
    """
    N = len(parent)
    a = [row_max_argmax(target(int(row[v])))[1] for v in range(N)]
    best, best_depth = 0, 0
    for v in range(1, N):
        path = ancestors(parent, v)
        if all(int(token[c]) == a[int(parent[c])] for c in path[1:]):
            d = len(path) - 1
            if d > best_depth:
                best, best_depth = v, d
    path = ancestors(parent, best)
    return {"path": path, "A": len(path) - 1, "bonus": a[best], "argmax": a}


def uniform(u32) -> float:
    """A 32-bit draw k as the open-interval uniform (k + 1/2) * 2^-32."""
    return (float(int(u32)) + 0.5) * 2.0 ** -32


def inverse_cdf(p: np.ndarray, u32) -> int:
    """Smallest k with sum_{j<=k} p_j > u * sum_j p_j (ascending float64 prefix sums)."""
    c = np.cumsum(p)
    return int(np.argmax(c > uniform(u32) * c[-1]))


def sample(parent, token, row, target, draft, u_acc, u_res, margins: list | None = None) -> dict:
    """Rejection-sampling verification (concept page, "The protocol", steps 3-4).

    The chain rule of the page: accept a drafted token x with probability
    min(1, p(x)/q(x)); on rejection draw the correction from (p - q)+ normalised.
    Readings for a tree (the pages state only the chain rule):

    * at node v, p = softmax(target row of v) and q = softmax(draft row of v), the
      distribution that proposed v's children;
    * v's children are tried in slot order with u = (u_acc[c] + 1/2) 2^-32: accept c when
      q(x_c) > 0 and u < p(x_c)/q(x_c), or when q(x_c) = 0 < p(x_c);
    * after each rejected child, p <- (p - q)+ / sum (p - q)+ (q unchanged); if that sum
      is 0 the current p is kept;
    * on acceptance the walk moves to c; when no child is accepted, or v is a leaf, the
      bonus is drawn from the current p by inverse CDF with u_res[v].

    With ``margins`` (a list), every decision that depends on the rows' normalisers
    appends (kind, relative margin): each acceptance test |u - p/q| / (p/q), and the bonus
    draw's distance from the nearer boundary of the drawn entry's cumulative interval,
    over the total mass. They are reported, not used.
    """
    N = len(parent)
    children = [[] for _ in range(N)]
    for c in range(1, N):
        children[int(parent[c])].append(c)
    v = 0
    path = [0]
    decisions = []  # (child, u, ratio) of every test, for margin reports
    while True:
        p = row_softmax(target(int(row[v])))
        accepted = None
        if children[v]:
            q = row_softmax(draft(int(row[v])))
            for c in children[v]:
                x = int(token[c])
                u = uniform(u_acc[c])
                if q[x] > 0.0:
                    ratio = p[x] / q[x]
                    ok = u < ratio
                else:
                    ratio = np.inf
                    ok = p[x] > 0.0
                decisions.append((c, u, ratio))
                if margins is not None and np.isfinite(ratio) and ratio > 0.0:
                    margins.append(("sample_accept", abs(u - ratio) / ratio))
                if ok:
                    accepted = c
                    break
                r = np.maximum(p - q, 0.0)
                z = float(np.sum(r))
                if z > 0.0:
                    p = r / z
        if accepted is None:
            bonus = inverse_cdf(p, u_res[v])
            if margins is not None:
                c = np.cumsum(p)
                tgt = uniform(u_res[v]) * c[-1]
                lo = c[bonus - 1] if bonus > 0 else 0.0
                margins.append(("sample_bonus", min(tgt - lo, c[bonus] - tgt) / c[-1]))
            break
        v = accepted
        path.append(v)
    return {"path": path, "A": len(path) - 1, "bonus": bonus, "decisions": decisions}
