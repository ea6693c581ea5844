"""Decision margins of the oracle on the measured workloads (CPU only).

Several decisions of the step compare values computed from different logit rows, so
they depend on those rows' normalisers (log-sum-exp), which two float64
implementations round differently in the last bits: TALON's gate and budget cut, OPT-Tree's
per-layer selection, best-n set and stop test, and rejection sampling's acceptance tests
and bonus draw. The oracle reports each decision's margin (its distance from flipping);
this records the smallest on every measured workload's seed and checks that it exceeds,
by orders of magnitude, the 1e-12 by which the GPU's float64 normalisers may differ from
the oracle's (they are compared at 1e-12 in the parity tests): no tree or path here rests
on a near tie. A plausible mistake in the margin code (a missing term, a sign) shows up as
a margin of 0 or a negative one.
"""
from __future__ import annotations

import math

import pytest

from oracle import step as ostep
from workloads import make_workload
from workloads.configs import CONFIG_ORDER

GPU_NORMALISER_TOL = 1e-12


def _smallest(margins):
    out = {}
    for kind, m in margins:
        out[kind] = min(out.get(kind, math.inf), m)
    return out


@pytest.mark.parametrize("name", ["c2_talon_llama3_8b", "c4_opt_llama2_7b", "c5_batched_llama2_70b",
                                  "c6_ragged_serving"])
def test_margins_on_measured_seed(name):
    seed = CONFIG_ORDER.index(name) + 1
    # the keys and values play no part in these decisions: a one-key prefix keeps the
    # workload small where the prefix length is a single setting (every other input is
    # drawn from streams of its own, so trees, logits and uniforms are the measured ones)
    wl = make_workload(name, seed) if name.startswith("c6") else make_workload(name, seed, P=1)
    margins = []
    ostep.run_step(wl, with_attention=False, margins=margins)
    small = _smallest(margins)
    print(f"decision margins {name} seed {seed}: " + ", ".join(f"{k} {v:.3e} ({sum(1 for kk, _ in margins if kk == k)})"
                                                               for k, v in sorted(small.items())))
    assert small, "the workload takes cross-row decisions"
    for kind, m in small.items():
        assert m > 1e3 * GPU_NORMALISER_TOL, (kind, m)


def test_margin_of_a_planted_tie_is_zero():
    """Two candidates of different parents with equal path scores at the budget cut: the
    oracle reports a margin of 0 (the tie is then broken by parent slot, on both sides)."""
    from oracle import build
    import numpy as np
    # root row: tokens 0 and 1 with equal logits become slots 1 and 2; their rows are equal,
    # so their best children tie across the two parents, and one slot of budget remains
    rows = {0: np.array([2.0, 2.0, -9.0, -9.0]), 1: np.array([1.0, -9.0, -9.0, -9.0]),
            2: np.array([1.0, -9.0, -9.0, -9.0])}
    margins = []
    t = build.talon(lambda r: rows[r], B=3, K=2, alpha=0.0, margins=margins)
    assert t.parent == [-1, 0, 0, 1]   # the tie goes to the lower parent slot
    caps = [m for k, m in margins if k == "talon_cap"]
    assert caps and min(caps) == 0.0
