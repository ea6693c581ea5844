"""The oracle's decoding loop (several draft-tree steps on one KV cache) against what the
loop must do, checked from the step inputs and the accepted paths alone:

* prefix lengths: P_T = P_0 + sum over steps of (A_t + 1) (TALON page, section 5.3: every
  verification pass emits its accepted tokens plus one);
* the cache: the prefix is untouched, and the rows a step appends are that step's tree
  keys and values at the accepted path's slots, in path order (concept page, "The
  protocol", step 4), one step after another;
* bookkeeping: L = sum of (A_t + 1), E[A] = L / N_v with N_v the number of steps.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import step as ostep
from workloads import make_step_inputs

CASES = [
    ("c1_tiny", 1, {}, 5),
    ("c5_batched_llama2_70b", 5, {"S": 2, "P": 40, "V": 60, "Hq": 4, "Hkv": 2, "D": 64, "B": 20}, 4),
    ("c6_ragged_serving", 6, {"S": 3, "P": 50, "V": 60, "Hq": 4, "Hkv": 2, "D": 64, "B": 24, "P_min": 0}, 4),
]


@pytest.mark.parametrize("name,seed,ov,steps", CASES)
def test_decode_loop_cache_and_lengths(name, seed, ov, steps):
    inputs = lambda t: make_step_inputs(name, seed, t, planted=0.7, **ov)
    out = ostep.run_decode(inputs, steps)
    wl0 = inputs(0)
    cfg = wl0.cfg
    N = cfg.N
    total_accepted = 0
    for s in range(cfg.S):
        p = int(wl0.P[s])
        np.testing.assert_array_equal(out["k"][s, :, :p], wl0.k[s, :, :p])
        np.testing.assert_array_equal(out["v"][s, :, :p], wl0.v[s, :, :p])
        L = 0
        for t, res in enumerate(out["steps"]):
            ver = res[s]["verify"]
            A, path = ver["A"], ver["path"]
            assert len(path) == A + 1 and path[0] == 0
            if t == 0:
                tk = wl0.k[s, :, p:p + N]
                tv = wl0.v[s, :, p:p + N]
            else:
                w = inputs(t)
                tk, tv = w.k[s, :, :N], w.v[s, :, :N]
            np.testing.assert_array_equal(out["k"][s, :, p:p + A + 1], tk[:, path])
            np.testing.assert_array_equal(out["v"][s, :, p:p + A + 1], tv[:, path])
            p += A + 1
            L += A + 1
            total_accepted += A
        assert p == int(out["P"][s])
        bk = out["bookkeeping"][s]
        assert bk["N_v"] == steps and bk["L"] == L and bk["E_A"] == L / steps
    assert total_accepted > 0   # the planted tokens make some drafts acceptable
