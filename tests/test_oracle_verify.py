"""Pins of the oracle's verification, compaction and bookkeeping (CPU only).

* Greedy: hand-derived GOOSE walk (tests/golden/goose_hand.json); equality with a
  brute-force depth-first search over all matching branches on random tiny trees;
  all-match chains and no-match trees.
* Sampling: hand-derived decisions (tests/golden/sample_hand.json); single-draft
  acceptance probability equals sum_x min(p(x), q(x)) (Leviathan et al., named on the
  concept page); p = q always accepts; losslessness: the emitted tokens follow the
  target distribution (chi-square, a single chain, i.i.d. siblings, and a depth-2 tree
  under a Markov target).
* Compaction: gather identity. Bookkeeping: closed forms.
"""
import json
import os

import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

from oracle import bookkeeping, compact, mask, verify

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_greedy_hand_goose_walk():
    g = _load("goose_hand.json")
    V = g["V"]
    N = len(g["parent"])
    rows = []
    for a in g["target_argmax"]:
        r = np.zeros(V)
        r[a] = 1.0
        rows.append(r)
    out = verify.greedy(g["parent"], g["token"], list(range(N)), lambda r: rows[r])
    assert out["path"] == g["path"] and out["A"] == g["A"] and out["bonus"] == g["bonus"]


def _dfs_longest(parent, token, tgt_rows):
    """Explore every branch that keeps matching the target argmax; deepest, then lowest slot."""
    N = len(parent)
    kids = [[] for _ in range(N)]
    for c in range(1, N):
        kids[parent[c]].append(c)
    best = (0, 0)  # (depth, -slot) maximised ... store as (depth, slot)
    best_node, best_depth = 0, 0
    stack = [(0, 0)]
    while stack:
        v, dep = stack.pop()
        if dep > best_depth or (dep == best_depth and v < best_node):
            best_node, best_depth = v, dep
        a = int(np.argmax(tgt_rows[v]))
        for c in kids[v]:
            if token[c] == a:
                stack.append((c, dep + 1))
    return best_node, best_depth


@pytest.mark.parametrize("seed", range(60))
def test_greedy_equals_brute_force_search(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 4))
    N = int(rng.integers(1, 25))
    parent = [-1] + [int(rng.integers(0, i)) for i in range(1, N)]
    token = [-1] + [int(rng.integers(0, V)) for _ in range(1, N)]
    rows = [rng.integers(0, 3, size=V).astype(float) for _ in range(N)]   # many argmax ties
    out = verify.greedy(parent, token, list(range(N)), lambda r: rows[r])
    node, depth = _dfs_longest(parent, token, rows)
    assert out["A"] == depth
    assert out["path"] == mask.ancestors(parent, node)
    assert out["bonus"] == int(np.argmax(rows[node]))


def test_greedy_all_match_chain_and_no_match():
    V, N = 6, 9
    rows = [np.eye(V)[(i * 5) % V] for i in range(N)]
    parent = [-1] + list(range(N - 1))
    token = [-1] + [int(np.argmax(rows[i - 1])) for i in range(1, N)]
    out = verify.greedy(parent, token, list(range(N)), lambda r: rows[r])
    assert out["A"] == N - 1 and out["path"] == list(range(N))
    assert out["bonus"] == int(np.argmax(rows[N - 1]))
    bad = [-1] + [(t + 1) % V for t in token[1:]]
    out = verify.greedy(parent, bad, list(range(N)), lambda r: rows[r])
    assert out["A"] == 0 and out["path"] == [0] and out["bonus"] == int(np.argmax(rows[0]))


def test_sample_hand_cases():
    g = _load("sample_hand.json")
    tr = [np.log(np.asarray(r)) for r in g["target_prob"]]
    dr = [np.log(np.asarray(r)) for r in g["draft_prob"]]
    for c in g["cases"]:
        u_acc = [0, c["u_acc"]]
        u_res = [c.get("u_res_root", 0), c.get("u_res_child", 0)]
        out = verify.sample([-1, 0], [-1, c["token"]], [0, 1], lambda r: tr[r], lambda r: dr[r],
                            u_acc, u_res)
        assert out["path"] == c["path"] and out["bonus"] == c["bonus"], c["why"]


def _u32(rng, n):
    return rng.integers(0, 2 ** 32, size=n, dtype=np.uint64)


def test_single_draft_acceptance_probability_closed_form():
    rng = np.random.default_rng(20)
    V = 5
    t = rng.standard_normal(V)
    d = rng.standard_normal(V)
    p, q = softmax(t), softmax(d)
    T = 40000
    acc = 0
    toks = rng.choice(V, size=T, p=q)
    ua = _u32(rng, T)
    for k in range(T):
        out = verify.sample([-1, 0], [-1, int(toks[k])], [0, 1], lambda r: [t, t][r],
                            lambda r: [d, d][r], [0, ua[k]], [0, 0])
        acc += out["A"]
    want = float(np.minimum(p, q).sum())
    se = np.sqrt(want * (1 - want) / T)
    assert abs(acc / T - want) < 5 * se


def test_p_equals_q_always_accepts():
    rng = np.random.default_rng(21)
    t = rng.standard_normal(7)
    for k in range(200):
        tok = int(rng.integers(0, 7))
        out = verify.sample([-1, 0], [-1, tok], [0, 1], lambda r: t, lambda r: t,
                            [0, int(_u32(rng, 1)[0])], [0, 0])
        assert out["A"] == 1


def test_disjoint_support_always_resamples_from_p():
    # q puts no mass where p lives: every draft is rejected, the bonus is drawn from p
    with np.errstate(divide="ignore"):
        t = np.log(np.array([0.5, 0.5, 0.0, 0.0]))
        d = np.log(np.array([0.0, 0.0, 0.5, 0.5]))
    rng = np.random.default_rng(22)
    for k in range(200):
        tok = int(rng.integers(2, 4))
        out = verify.sample([-1, 0, 0], [-1, tok, 5 - tok], [0, 1, 2], lambda r: t, lambda r: d,
                            [0] + [int(x) for x in _u32(rng, 2)], [int(_u32(rng, 1)[0]), 0, 0])
        assert out["A"] == 0 and out["bonus"] in (0, 1)


def _chi2_ok(counts, probs):
    T = counts.sum()
    exp = probs * T
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    return stats.chi2.sf(chi2, len(probs) - 1) > 1e-4


@pytest.mark.parametrize("m", [1, 3])
def test_lossless_first_token(m):
    """Root with m i.i.d. children drawn from q: the first emitted token follows p."""
    rng = np.random.default_rng(30 + m)
    V = 5
    t = rng.standard_normal(V)
    d = rng.standard_normal(V)
    p, q = softmax(t), softmax(d)
    T = 30000
    counts = np.zeros(V)
    parent = [-1] + [0] * m
    rows = list(range(m + 1))
    for k in range(T):
        tok = [-1] + [int(x) for x in rng.choice(V, size=m, p=q)]
        out = verify.sample(parent, tok, rows, lambda r: t, lambda r: d,
                            [0] + [int(x) for x in _u32(rng, m)], [int(x) for x in _u32(rng, m + 1)])
        first = tok[out["path"][1]] if out["A"] >= 1 else out["bonus"]
        counts[first] += 1
    assert _chi2_ok(counts, p)


def test_lossless_depth_two_markov_target():
    """Depth-2 tree, 2 i.i.d. children per node; target and draft depend on the last token.

    The first token follows p0 and, after an accepted first token x1, the second
    emitted token follows the target row of x1.
    """
    rng = np.random.default_rng(40)
    V = 4
    T0, D0 = rng.standard_normal(V), rng.standard_normal(V)
    Tm, Dm = rng.standard_normal((V, V)) * 1.5, rng.standard_normal((V, V)) * 1.5
    trials = 30000
    c1 = np.zeros(V)
    c2 = np.zeros((V, V))
    parent = [-1, 0, 0, 1, 1, 2, 2]
    for k in range(trials):
        tok = [-1] * 7
        tok[1], tok[2] = [int(x) for x in rng.choice(V, 2, p=softmax(D0))]
        tok[3], tok[4] = [int(x) for x in rng.choice(V, 2, p=softmax(Dm[tok[1]]))]
        tok[5], tok[6] = [int(x) for x in rng.choice(V, 2, p=softmax(Dm[tok[2]]))]
        trows = [T0] + [Tm[tok[i]] for i in range(1, 7)]
        drows = [D0] + [Dm[tok[i]] for i in range(1, 7)]
        out = verify.sample(parent, tok, list(range(7)), lambda r: trows[r], lambda r: drows[r],
                            [int(x) for x in _u32(rng, 7)], [int(x) for x in _u32(rng, 7)])
        emitted = [tok[i] for i in out["path"][1:]] + [out["bonus"]]
        c1[emitted[0]] += 1
        if out["A"] >= 1:
            c2[emitted[0], emitted[1]] += 1
    assert _chi2_ok(c1, softmax(T0))
    for x in range(V):
        if c2[x].sum() > 2000:
            assert _chi2_ok(c2[x], softmax(Tm[x]))


def test_inverse_cdf_boundaries():
    p = np.array([0.25, 0.0, 0.5, 0.25])
    assert verify.inverse_cdf(p, 0) == 0
    assert verify.inverse_cdf(p, 2 ** 30) == 2          # u just above .25 skips the empty bin
    assert verify.inverse_cdf(p, 2 ** 32 - 1) == 3


def test_compaction_gather_identity():
    rng = np.random.default_rng(50)
    H, P, N, D = 3, 10, 12, 4
    k = rng.standard_normal((H, P + N + 2, D))
    v = rng.standard_normal((H, P + N + 2, D))
    path = [0, 3, 7, 11]
    k2, v2, Pn = compact.kv_compact(k, v, P, path)
    assert Pn == P + 4
    for kk, node in enumerate(path):
        np.testing.assert_array_equal(k2[:, P + kk], k[:, P + node])
        np.testing.assert_array_equal(v2[:, P + kk], v[:, P + node])
    np.testing.assert_array_equal(k2[:, :P], k[:, :P])
    np.testing.assert_array_equal(k2[:, P + 4:], k[:, P + 4:])


def test_bookkeeping_closed_forms():
    out = bookkeeping.bookkeeping([3, 0, 5], draft_steps=6, gamma=0.0)
    assert out["L"] == (3 + 1) + (0 + 1) + (5 + 1) and out["E_A"] == pytest.approx(11 / 3)
    assert out["speedup"] == pytest.approx(out["E_A"])
    out = bookkeeping.bookkeeping([0, 0, 0, 0], draft_steps=0, gamma=0.3)
    assert out["speedup"] == 1.0 and out["eta"] == 0.0
    out = bookkeeping.bookkeeping([2, 4], draft_steps=8, gamma=0.1)
    assert out["eta"] == 4.0 and out["speedup"] == pytest.approx(4.0 / 1.4)
    # the concept page's L/(1 + L c) is the same number when eta equals E[A]
    out = bookkeeping.bookkeeping([2, 2], draft_steps=6, gamma=0.05)
    assert out["speedup"] == pytest.approx(3.0 / (1 + 3.0 * 0.05))
