"""Draft-tree builders: given trees, TALON, GOOSE spine trees, OPT-Tree.

Every builder returns a ``Tree`` in slot numbering: slot 0 is the root, parents come
before children, ``row[i]`` is the index of node i's row in the draft and target
logit tables (the draft row that proposes i's children, and the target row that scores
them), and ``score[i]`` is the log path score log prod p_d along the root path
(0 for the root; 0 for nodes of a given tree, which carries no scores).

Draft rows are read through ``draft(r) -> float64 row`` so that a builder touches only
the rows it expands.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable

import numpy as np

from .rows import row_logp, topk

RowFn = Callable[[int], np.ndarray]


@dataclasses.dataclass
class Tree:
    parent: list
    token: list
    depth: list
    row: list
    score: list
    layers: int = 0        # draft forward passes the build spent (rows expanded per layer)
    rows_read: int = 0     # draft rows expanded
    expected: list = dataclasses.field(default_factory=list)  # OPT-Tree E_l per layer

    @property
    def N(self) -> int:
        return len(self.parent)

    def add(self, parent: int, token: int, row: int, score: float) -> int:
        self.parent.append(int(parent))
        self.token.append(int(token))
        self.depth.append(self.depth[parent] + 1)
        self.row.append(int(row))
        self.score.append(float(score))
        return len(self.parent) - 1


def _root() -> Tree:
    return Tree(parent=[-1], token=[-1], depth=[0], row=[0], score=[0.0])


def given_tree(parent, token) -> Tree:
    """A tree whose shape and tokens come from the drafter as data (random trees).

    Slot i's row is row i. No scores: the drafter that made it is outside the step.
    """
    t = _root()
    for i in range(1, len(parent)):
        p = int(parent[i])
        if not (0 <= p < i):
            raise ValueError(f"parent[{i}] = {p} is not an earlier slot")
        t.add(p, int(token[i]), i, 0.0)
    return t


def _boundary_margin(ranked, k: int, score, group) -> float:
    """Smallest score gap between a kept and a dropped candidate of different groups, when
    `ranked` (best first) keeps its first k: the decision that two rows' normalisers could
    flip. Candidates of one group (one parent row) differ by their logits alone, exactly,
    so their order is not a cross-row decision. inf when no such pair exists."""
    kept_min, drop_max = {}, {}
    for i, c in enumerate(ranked):
        g, sc = group(c), score(c)
        if i < k:
            kept_min[g] = min(kept_min.get(g, math.inf), sc)
        else:
            drop_max[g] = max(drop_max.get(g, -math.inf), sc)
    m = math.inf
    for ga, lo in kept_min.items():
        for gb, hi in drop_max.items():
            if ga != gb:
                m = min(m, lo - hi)
    return m


def talon(draft: RowFn, B: int, K: int, alpha: float, margins: list | None = None) -> Tree:
    """TALON budget-driven hybrid expansion (TALON page, sections 5.1 and 5.2).

    * Budget (5.1): B is the largest number of draft nodes; the root is extra (slot 0).
    * Robust initialisation (5.2.2): layer 1 is TopK(p_d(x_1 | x_0), K), with no gate;
      if K exceeds B only the best B are kept.
    * Confidence-gated expansion (5.2.1), for every later layer l:
      - the candidate pool is the union over the previous layer's nodes v of Expand(v),
        read here as the K most probable children of v under v's draft row;
      - each candidate carries the path score s(c) = prod_t p_d(x_t | x_<t), kept as a
        sum of logs: log s(c) = log s(v) + log p_d(token | v);
      - anchor = max over the pool of s(c); keep c when s(c) >= alpha * anchor, i.e.
        log s(c) >= log(alpha) + log anchor;
      - budget respect: if more candidates pass than budget remains, keep the best
        remaining-budget of them by path score (ties: lower parent slot, then lower
        rank within the parent's row).
    * New nodes take the next slots in (parent slot, rank in the parent's row) order,
      so scores only decide which nodes exist, never how they are numbered.
    * The loop ends when B nodes exist; the anchor always passes, so every layer adds
      at least one node.
    * Rows are keyed by slot: node i expands with draft row i.

    With ``margins`` (a list), every cross-row decision appends (kind, margin): for the
    gate, |log s(c) - (log alpha + log anchor)| of every candidate whose parent differs
    from the anchor's; for the budget cut, the smallest score gap between a kept and a
    dropped candidate of different parents. Margins are in log units (relative
    differences of the path probabilities); they are reported, not used.
    """
    if B < 1 or K < 1 or not (0.0 <= alpha <= 1.0):
        raise ValueError("need B >= 1, K >= 1 and 0 <= alpha <= 1")
    log_alpha = -math.inf if alpha == 0.0 else math.log(alpha)
    t = _root()
    x0 = draft(0)
    lp0 = row_logp(x0)
    for r, tok in enumerate(topk(x0, min(K, B))):
        t.add(0, int(tok), len(t.parent), lp0[tok])
    t.layers, t.rows_read = 1, 1
    prev = list(range(1, t.N))
    while t.N - 1 < B:
        pool = []  # (log score, parent slot, rank, token)
        for v in prev:
            x = draft(t.row[v])
            lp = row_logp(x)
            for r, tok in enumerate(topk(x, K)):
                pool.append((t.score[v] + lp[tok], v, r, int(tok)))
        t.layers += 1
        t.rows_read += len(prev)
        anchor = max(c[0] for c in pool)
        kept = [c for c in pool if c[0] >= log_alpha + anchor]
        room = B - (t.N - 1)
        if margins is not None and alpha > 0.0:
            a_par = next(c[1] for c in pool if c[0] == anchor)
            for c in pool:
                if c[1] != a_par:
                    margins.append(("talon_gate", abs(c[0] - (log_alpha + anchor))))
        if len(kept) > room:
            ranked = sorted(kept, key=lambda c: (-c[0], c[1], c[2]))
            if margins is not None:
                margins.append(("talon_cap", _boundary_margin(ranked, room, lambda c: c[0], lambda c: c[1])))
            kept = ranked[:room]
        kept.sort(key=lambda c: (c[1], c[2]))
        prev = []
        for s, v, r, tok in kept:
            prev.append(t.add(v, tok, t.N, s))
    return t


def spine(draft: RowFn, spine_tokens, widths) -> Tree:
    """GOOSE anisotropic spine tree (GOOSE page, section 2A, and 2C unified walk).

    * The spine is a chain of the given context-match tokens: slot k+1 holds
      spine_tokens[k] with parent slot k (slot 0 is the root).
    * Forks are slots 0 .. len(widths)-1 (the root and the first spine nodes). Fork f
      carries widths[f] depth-1 branch nodes whose tokens are the most probable tokens
      of fork f's draft row, skipping the token of f's spine child (slot f+1), which is
      already in the tree. Branches follow the spine in (fork, rank) order, so the spine
      holds the lowest slots and a greedy walk that prefers low slots prefers the spine.
    * Rows are keyed by slot.
    """
    sp = [int(x) for x in spine_tokens]
    t = _root()
    for k, tok in enumerate(sp):
        t.add(k, tok, k + 1, 0.0)
    for f, w in enumerate(widths):
        w = int(w)
        if w <= 0:
            continue
        if f > len(sp):
            raise ValueError("a fork must be the root or a spine node")
        x = draft(f)
        lp = row_logp(x)
        skip = sp[f] if f < len(sp) else None
        picked = [int(tok) for tok in topk(x, w + 1) if int(tok) != skip][:w]
        for tok in picked:
            t.add(f, tok, t.N, t.score[f] + lp[tok])
    t.layers, t.rows_read = 1, sum(1 for w in widths if int(w) > 0)
    return t


def opt_tree(draft: RowFn, n: int, delta: float, max_layers: int, margins: list | None = None) -> Tree:
    """OPT-Tree greedy construction (OPT-Tree summary, section 3).

    * A node's score is the product of draft probabilities along its parent path, kept
      as a sum of logs.
    * Layer by layer, every frontier node takes its next draft row and proposes its n
      most probable children; the layer keeps the n candidates of largest score (ties:
      lower frontier position, then lower rank), which become the next frontier. The
      frontier is ordered by (parent's frontier position, rank), so scores decide
      membership only.
    * Expected acceptance length after layer l, E_l, is the sum of the scores of the
      best n-node subtree among all nodes drafted so far. Because a child never scores
      above its parent, the n best nodes (ties: earlier layer first) form a subtree that
      contains the root's children, so E_l is the sum of exp(score) over those n nodes.
    * Drafting stops when E_l - E_{l-1} < delta (E_0 = 0) or after max_layers layers.
      The last drafted layer is kept.
    * The final tree is the n best nodes of all layers, renumbered layer by layer in
      frontier order.
    * Row identity: the node at frontier position p of layer l uses row
      1 + (l-1)*n + p of the tables (the root uses row 0).

    With ``margins`` (a list), every cross-row decision appends (kind, margin): the layer's
    selection and the best-n set (smallest score gap between a kept and a dropped
    candidate of different parents, log units) and the stop test (|E_l - E_{l-1} - delta|).
    They are reported, not used.
    """
    if n < 1 or max_layers < 1:
        raise ValueError("need n >= 1 and max_layers >= 1")
    # node records: (score, layer, position, parent index in `nodes` or -1, rank, token, row)
    nodes = []
    frontier = [-1]          # -1 stands for the root
    root_score, root_row = 0.0, 0
    E_prev = 0.0
    expected = []
    layers = rows_read = 0
    for layer in range(1, max_layers + 1):
        pool = []  # (score, frontier position, rank, token)
        for pos, ni in enumerate(frontier):
            s_v = root_score if ni < 0 else nodes[ni][0]
            r_v = root_row if ni < 0 else nodes[ni][6]
            x = draft(r_v)
            lp = row_logp(x)
            for r, tok in enumerate(topk(x, n)):
                pool.append((s_v + lp[tok], pos, r, int(tok)))
        layers += 1
        rows_read += len(frontier)
        ranked = sorted(pool, key=lambda c: (-c[0], c[1], c[2]))
        if margins is not None and len(ranked) > n:
            margins.append(("opt_layer", _boundary_margin(ranked, n, lambda c: c[0], lambda c: c[1])))
        best = ranked[:n]
        best.sort(key=lambda c: (c[1], c[2]))
        new_frontier = []
        for p_new, (s, pos, r, tok) in enumerate(best):
            nodes.append((s, layer, p_new, frontier[pos], r, tok, 1 + (layer - 1) * n + p_new))
            new_frontier.append(len(nodes) - 1)
        frontier = new_frontier
        allr = sorted(nodes, key=lambda c: (-c[0], c[1], c[2]))
        if margins is not None and len(allr) > n:
            margins.append(("opt_best", _boundary_margin(allr, n, lambda c: c[0], lambda c: (c[1], c[3]))))
        top = allr[:n]
        E_l = float(sum(math.exp(c[0]) for c in top))
        expected.append(E_l)
        if margins is not None and layer < max_layers:
            margins.append(("opt_stop", abs((E_l - E_prev) - delta)))
        if E_l - E_prev < delta:
            break
        E_prev = E_l
    chosen = sorted(range(len(nodes)), key=lambda i: (-nodes[i][0], nodes[i][1], nodes[i][2]))[:n]
    chosen.sort(key=lambda i: (nodes[i][1], nodes[i][2]))
    t = _root()
    slot_of = {-1: 0}
    for i in chosen:
        s, layer, pos, par, r, tok, row = nodes[i]
        if par not in slot_of:
            raise AssertionError("final OPT-Tree node set is not root-closed")
        slot_of[i] = t.add(slot_of[par], tok, row, s)
    t.layers, t.rows_read, t.expected = layers, rows_read, expected
    return t
