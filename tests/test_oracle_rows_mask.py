"""Pins of the oracle's row primitives and tree mask (CPU only).

Row primitives are checked against library routines (scipy's logsumexp, numpy's
stable argsort on an independent key) and brute force; the mask against closed forms
for chains and stars and against invariants of random trees.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import mask, rows


def test_bf16_decode_known_patterns():
    # bf16 bit patterns with known values (sign/exponent/mantissa written out)
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3FC0, 0x7F7F, 0x0080, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 1.5, 3.3895313892515355e38, 2.0 ** -126, 3.140625]
    got = rows.decode(bits, "bf16")
    assert got.dtype == np.float64
    assert list(got) == want


def test_argmax_brute_force_ties():
    rng = np.random.default_rng(0)
    for _ in range(200):
        x = rng.integers(-3, 3, size=rng.integers(1, 12)).astype(np.float64)
        m, a = rows.row_max_argmax(x)
        best = 0
        for j in range(len(x)):
            if x[j] > x[best]:
                best = j
        assert a == best and m == x[best]


def test_topk_brute_force_ties():
    rng = np.random.default_rng(1)
    for _ in range(200):
        V = int(rng.integers(1, 15))
        x = rng.integers(-2, 3, size=V).astype(np.float64)
        K = int(rng.integers(1, V + 3))
        got = list(rows.topk(x, K))
        # selection by repeated scans: largest value, lowest index first
        left = list(range(V))
        want = []
        while left and len(want) < K:
            b = left[0]
            for j in left:
                if x[j] > x[b]:
                    b = j
            want.append(b)
            left.remove(b)
        assert got == want


def test_lse_matches_scipy_and_closed_form():
    rng = np.random.default_rng(2)
    for V in (1, 2, 7, 1000, 128256):
        x = rng.standard_normal(V) * 3
        assert rows.row_lse(x) == pytest.approx(float(logsumexp(x)), rel=1e-14, abs=1e-13)
    x = np.full(50, 1.25)
    assert rows.row_lse(x) == pytest.approx(1.25 + math.log(50), rel=1e-15)
    p = rows.row_softmax(rng.standard_normal(300))
    assert p.sum() == pytest.approx(1.0, abs=1e-14)
    m, a = rows.row_max_argmax(np.full(9, -0.5))
    assert a == 0 and list(rows.topk(np.full(9, -0.5), 4)) == [0, 1, 2, 3]


def test_lse_handles_minus_inf_entries():
    x = np.array([0.0, -np.inf, np.log(3.0)])
    assert rows.row_lse(x) == pytest.approx(math.log(4.0), rel=1e-15)


def _chain(n):
    return [-1] + list(range(n - 1))


def test_mask_chain_is_causal():
    for n in (1, 2, 17, 64, 65, 130):
        anc = mask.ancestor_matrix(_chain(n))
        assert (anc == np.tril(np.ones((n, n), dtype=bool))).all()
        assert list(mask.depths(_chain(n))) == list(range(n))


def test_mask_star():
    n = 70
    par = [-1] + [0] * (n - 1)
    anc = mask.ancestor_matrix(par)
    want = np.eye(n, dtype=bool)
    want[:, 0] = True
    assert (anc == want).all()


def test_pack_words_word_boundary():
    n = 65
    w = mask.pack_words(mask.ancestor_matrix(_chain(n)), 2)
    assert w[63, 0] == np.uint64(0xFFFFFFFFFFFFFFFF) and w[63, 1] == 0
    assert w[64, 0] == np.uint64(0xFFFFFFFFFFFFFFFF) and w[64, 1] == 1
    assert w[0, 0] == 1 and w[5, 0] == 0x3F


def test_mask_random_tree_invariants():
    rng = np.random.default_rng(3)
    for _ in range(30):
        n = int(rng.integers(1, 140))
        par = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
        anc = mask.ancestor_matrix(par)
        d = mask.depths(par)
        for i in range(n):
            assert anc[i].sum() == d[i] + 1          # popcount = depth + 1
            assert anc[i, i] and anc[i, 0]
            if i:
                p = par[i]
                assert (anc[i] >= anc[p]).all()      # anc(parent) is a subset of anc(i)
                assert (anc[i] & ~anc[p]).sum() == 1


def test_mask_rejects_bad_parent():
    with pytest.raises(ValueError):
        mask.depths([-1, 0, 2])
