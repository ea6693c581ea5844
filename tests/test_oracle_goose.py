"""GOOSE's adaptive spine topology (GOOSE page, section 2): the oracle's policy against what
the page fixes, and the device path's host policy against the oracle's.

Pinned: a step spends exactly its budget; branch widths never grow with depth and stay
within one node of the linear profile of Proposition 2; bypass drafts a bare chain; the
moving average of a constant rate rho follows its closed form rho + beta^n (avg_0 - rho);
the accepted spine run of a path is the number of its spine slots.
"""
from __future__ import annotations

import numpy as np
import pytest

from draft_tree_verification_build_amd import goose as dgoose
from oracle import goose as og


@pytest.mark.parametrize("L,nodes", [(1, 0), (1, 5), (5, 7), (24, 96), (72, 48), (10, 3), (7, 100), (120, 0)])
def test_branch_widths_linear_profile(L, nodes):
    w = og.branch_widths(L, nodes)
    assert len(w) == L and sum(w) == nodes and min(w) >= 0
    assert all(w[j] >= w[j + 1] for j in range(L - 1))
    tot = L * (L + 1) / 2
    for j in range(L):
        assert abs(w[j] - nodes * (L - j) / tot) < 1.0


@pytest.mark.parametrize("avg", [0.0, 0.05, 0.3, 0.6, 0.89, 0.9, 0.97])
def test_plan_spends_the_budget(avg):
    B = 120
    L, w = og.plan(avg, B)
    assert L + sum(w) == B and len(w) == L
    if avg >= 0.9:
        assert L == B and not any(w)
    else:
        r = min(max(avg, 0.1), 0.9)
        assert L == max(1, min(B, int(round(r * B))))


def test_average_closed_form():
    rho_k, L = 3, 10            # a spine that always breaks after 3 accepted tokens: rate 3/4
    avg0, beta = 0.5, 0.8
    avg = avg0
    for n in range(1, 30):
        avg = og.update(avg, [rho_k], L, beta)
        assert avg == pytest.approx(0.75 + beta ** n * (avg0 - 0.75), rel=1e-12)
    assert og.update(0.5, [10], 10, beta) == pytest.approx(0.8 * 0.5 + 0.2 * 1.0)   # unbroken spine


def test_spine_run_counts_spine_slots():
    L = 6
    assert og.spine_run([0], L) == 0
    assert og.spine_run([0, 1, 2, 3], L) == 3
    assert og.spine_run([0, 1, 2, 9], L) == 2          # left the spine for a branch of node 2
    assert og.spine_run([0, 7, 12], L) == 0            # a branch of the root
    assert dgoose.spine_accepted([0, 1, 2, 9], L) == 2


def test_host_policy_equals_oracle_policy():
    rng = np.random.default_rng(5)
    B = 120
    pol = dgoose.SpineTopology(B)
    avg = 0.5
    bypassed = 0
    for t in range(200):
        L, w = pol.plan()
        assert (L, list(w)) == og.plan(avg, B), t
        S = int(rng.integers(1, 4))
        # mostly long runs later on, so that the average also crosses the bypass level
        ks = [int(min(L, rng.geometric(0.5 if t < 100 else 0.02) - 1)) for _ in range(S)]
        pol.observe(ks, L)
        avg = og.update(avg, ks, L)
        assert pol.ema == avg
        bypassed += L == B
    assert bypassed > 0
