"""Pins of the oracle's tree builders (CPU only).

* TALON: hand-derived trees (tests/golden/talon_hand.json); on random rows, an
  independent checker of the page's rules (Top-K root layer; every later node is a
  top-K child of a previous-layer node; every node passes the gate against its
  layer's anchor; the budget cap keeps the best scores; exactly B nodes); alpha = 1
  gives one node per layer after the root layer.
* GOOSE: hand-derived tree (tests/golden/goose_hand.json) and structural invariants.
* OPT-Tree: hand-derived tree (tests/golden/opt_hand.json); with delta = 0 the result
  equals brute force over the full depth-D tree (top-n nodes of all V + V^2 + ...);
  root-closure and monotone E_l on random rows.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import log_softmax

from oracle import build, mask

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _table(prob_rows):
    return [np.log(np.asarray(r, dtype=np.float64)) for r in prob_rows]


# ----------------------------------------------------------------------------- TALON

def test_talon_hand_cases():
    g = _load("talon_hand.json")
    rows = _table(g["rows_prob"])
    for c in g["cases"]:
        t = build.talon(lambda r: rows[r], c["B"], c["K"], c["alpha"])
        assert t.parent == c["parent"], c["why"]
        assert t.token == c["token"], c["why"]
        assert t.depth == c["depth"], c["why"]
        assert t.row == list(range(len(c["parent"])))


def _topk_ref(lp, K):
    # order by (log-prob desc, index asc) with a lexsort on an independent key
    idx = np.lexsort((np.arange(len(lp)), -lp))
    return [int(i) for i in idx[:K]]


def check_talon(t, rows, B, K, alpha):
    """Independent check of a TALON tree against the page's rules."""
    N = t.N
    assert N == B + 1
    lp = {}

    def lsm(r):
        if r not in lp:
            lp[r] = log_softmax(rows[r])
        return lp[r]

    # path scores recomputed by walking each root path
    score = [0.0] * N
    for i in range(1, N):
        path = mask.ancestors(t.parent, i)
        score[i] = sum(lsm(path[k - 1])[t.token[path[k]]] for k in range(1, len(path)))
        assert score[i] == pytest.approx(t.score[i], abs=1e-12)
    depth = mask.depths(t.parent)
    L = int(depth.max())
    layer1 = [i for i in range(N) if depth[i] == 1]
    assert [t.token[i] for i in layer1] == _topk_ref(lsm(0), min(K, B))
    count = len(layer1)
    for l in range(2, L + 1):
        prev = [i for i in range(N) if depth[i] == l - 1]
        cur = [i for i in range(N) if depth[i] == l]
        assert cur == list(range(min(cur), max(cur) + 1))   # a layer is a contiguous slot range
        pool = []
        for v in prev:
            for r, tok in enumerate(_topk_ref(lsm(v), K)):
                pool.append((score[v] + lsm(v)[tok], v, r, tok))
        anchor = max(c[0] for c in pool)
        thr = (-math.inf if alpha == 0 else math.log(alpha)) + anchor
        passing = [c for c in pool if c[0] >= thr]
        kept = [(t.parent[i], t.token[i]) for i in cur]
        # every node is a pool member that passes the gate
        keyed = {(c[1], c[3]): c for c in passing}
        assert all(k in keyed for k in kept)
        room = B - count
        assert len(kept) == min(len(passing), room)
        if len(passing) > room:
            kept_scores = [keyed[k][0] for k in kept]
            dropped = [c[0] for c in passing if (c[1], c[3]) not in set(kept)]
            assert max(dropped) <= min(kept_scores)
        # numbering: parent slot, then rank in the parent's row
        ranks = [(t.parent[i], _topk_ref(lsm(t.parent[i]), K).index(t.token[i])) for i in cur]
        assert ranks == sorted(ranks)
        count += len(cur)
    assert count == B


@pytest.mark.parametrize("seed", range(40))
def test_talon_random_rows_follow_the_rules(seed):
    rng = np.random.default_rng(100 + seed)
    V = int(rng.integers(3, 12))
    K = int(rng.integers(1, 5))
    B = int(rng.integers(1, 13))
    alpha = [0.0, 0.05, 0.3, 0.7, 1.0][seed % 5]
    rows = [rng.standard_normal(V) * 2 for _ in range(B + 1)]
    t = build.talon(lambda r: rows[r], B, K, alpha)
    check_talon(t, rows, B, K, alpha)


def test_talon_alpha_one_is_a_chain_after_the_root_layer():
    rng = np.random.default_rng(7)
    B, K = 12, 3
    rows = [rng.standard_normal(20) for _ in range(B + 1)]
    t = build.talon(lambda r: rows[r], B, K, 1.0)
    d = mask.depths(t.parent)
    assert list(np.bincount(d)[1:]) == [K] + [1] * (B - K)


def test_talon_alpha_zero_keeps_best_of_pool():
    rng = np.random.default_rng(8)
    B, K = 11, 3
    rows = [rng.standard_normal(15) for _ in range(B + 1)]
    t = build.talon(lambda r: rows[r], B, K, 0.0)
    check_talon(t, rows, B, K, 0.0)
    # layer 2 is the best (B - K) of the K*K pool, i.e. 8 of 9 candidates
    assert list(np.bincount(mask.depths(t.parent))[1:]) == [3, 8]


# ----------------------------------------------------------------------------- GOOSE

def test_goose_hand_case():
    g = _load("goose_hand.json")
    rows = _table(g["draft_prob"])
    t = build.spine(lambda r: rows[r], g["spine"], g["widths"])
    assert t.parent == g["parent"] and t.token == g["token"]


def test_goose_structure_invariants():
    rng = np.random.default_rng(9)
    V, n_spine = 40, 24
    rows = [rng.standard_normal(V) * 3 for _ in range(n_spine + 1)]
    sp = rng.integers(0, V, size=n_spine)
    widths = [4] * 24
    t = build.spine(lambda r: rows[r], sp, widths)
    assert t.N == 1 + 24 + 96
    assert t.parent[1:25] == list(range(24)) and t.token[1:25] == list(sp)
    for f in range(24):
        kids = [i for i in range(25, t.N) if t.parent[i] == f]
        assert len(kids) == 4
        toks = [t.token[i] for i in kids]
        want = [x for x in _topk_ref(log_softmax(rows[f]), 5) if x != sp[f]][:4]
        assert toks == want
    # without branches the tree is the spine chain
    t2 = build.spine(lambda r: rows[r], sp, [0] * 24)
    assert t2.parent == [-1] + list(range(24))


# ----------------------------------------------------------------------------- OPT-Tree

def test_opt_hand_case():
    g = _load("opt_hand.json")
    rows = _table(g["rows_prob"])
    t = build.opt_tree(lambda r: rows[r], g["n"], g["delta"], g["max_layers"])
    assert t.parent == g["parent"] and t.token == g["token"] and t.row == g["row"]
    assert t.layers == g["layers"]
    np.testing.assert_allclose(t.expected, g["expected_E"], rtol=1e-12)
    np.testing.assert_allclose(np.exp(t.score), g["score_prob"], rtol=1e-12)


@pytest.mark.parametrize("V,D,n", [(4, 4, 1), (4, 4, 3), (4, 4, 10), (4, 4, 40), (4, 4, 100),
                                   (3, 5, 25), (5, 3, 60)])
def test_opt_equals_brute_force_with_delta_zero(V, D, n):
    rng = np.random.default_rng(V * 100 + D * 10 + n)
    per_depth = [rng.standard_normal(V) * 2 for _ in range(D)]   # row depends on depth only

    def draft(r):
        return per_depth[0 if r == 0 else 1 + (r - 1) // n]

    t = build.opt_tree(draft, n, 0.0, D)
    lps = [log_softmax(x) for x in per_depth]
    nodes = []
    for d in range(1, D + 1):
        for path in itertools.product(range(V), repeat=d):
            nodes.append((sum(lps[k][path[k]] for k in range(d)), d, path))
    nodes.sort(key=lambda c: (-c[0], c[1]))
    best = nodes[:n]
    got = set()
    for i in range(1, t.N):
        got.add(tuple(t.token[j] for j in mask.ancestors(t.parent, i)[1:]))
    assert got == {c[2] for c in best}
    assert t.layers == D


@pytest.mark.parametrize("seed", range(10))
def test_opt_random_rows_invariants(seed):
    rng = np.random.default_rng(500 + seed)
    V, n, L = int(rng.integers(4, 30)), int(rng.integers(2, 40)), 5
    table = [rng.standard_normal(V) * 3 for _ in range(1 + L * n)]
    t = build.opt_tree(lambda r: table[r], n, 0.05, L)
    assert t.N - 1 == min(n, sum(V ** d for d in range(1, L + 1)))
    d = mask.depths(t.parent)
    for i in range(1, t.N):
        p = t.parent[i]
        assert t.score[i] <= t.score[p]
        assert 1 + (d[i] - 1) * n <= t.row[i] < 1 + d[i] * n
        assert t.score[i] == pytest.approx(t.score[p] + log_softmax(table[t.row[p]])[t.token[i]], abs=1e-12)
    E = t.expected
    assert all(b >= a - 1e-15 for a, b in zip(E, E[1:]))
    gains = [E[0]] + [b - a for a, b in zip(E, E[1:])]
    assert all(gn >= 0.05 for gn in gains[:-1])
    assert gains[-1] < 0.05 or t.layers == L
    # the final tree is the best n nodes by score among everything kept: its smallest
    # score is at least E's last term, and the sum of its probabilities is E_last
    assert float(np.sum(np.exp(t.score[1:]))) == pytest.approx(E[-1], rel=1e-12)


def test_given_tree_rejects_bad_parents():
    with pytest.raises(ValueError):
        build.given_tree([-1, 1], [-1, 3])
