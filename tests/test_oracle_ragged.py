"""Ragged batches (per-request prefix lengths and tree sizes): the oracle's step on one
request of a batch equals its step on that request alone.

A request alone is built from the batch's arrays, cut to its own sizes: its queries, the
cache up to its prefix plus its tree, its draft and target rows, its tree and its uniforms.
Equality (exact: the same float64 arithmetic on the same numbers) pins that nothing of the
batch's padding (slots past a request's tree, cache positions past its keys, other
requests) reaches a request's result, and that the generator places each tree's keys right
after that request's own prefix.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

from oracle import step as ostep
from workloads import make_workload
from workloads.configs import Workload


def _alone(wl, s):
    cfg = wl.cfg
    n = int(wl.n_nodes[s])
    P = int(wl.P[s])
    c1 = dataclasses.replace(cfg, S=1, P=P, B=n - 1, P_min=-1, B_min=-1)
    sl = slice(s, s + 1)
    return Workload(cfg=c1, seed=wl.seed, P=np.array([P], dtype=np.int32), P_cap=P + n,
                    q=wl.q[sl, :n], k=wl.k[sl, :, :P + n], v=wl.v[sl, :, :P + n],
                    draft=wl.draft[sl, :n], target=wl.target[sl, :n],
                    parent=wl.parent[sl, :n], token=wl.token[sl, :n],
                    u_acc=wl.u_acc[sl, :n], u_res=wl.u_res[sl, :n])


@pytest.mark.parametrize("seed,ov", [
    (7, {"S": 4, "P": 300, "P_min": 0, "B_min": 0, "V": 500, "Hq": 8, "Hkv": 2, "D": 64}),
    (8, {"S": 3, "P": 130, "P_min": 100, "B_min": 30, "V": 300, "Hq": 4, "Hkv": 4, "D": 64,
         "dtype": "f32"}),
])
def test_request_alone_equals_request_in_batch(seed, ov):
    wl = make_workload("c6_ragged_serving", seed, **ov)
    assert len(set(wl.n_nodes.tolist())) > 1 or len(set(wl.P.tolist())) > 1   # really ragged
    batch = ostep.run_step(wl)
    for s in range(wl.cfg.S):
        one = ostep.run_step(_alone(wl, s))[0]
        b = batch[s]
        n = int(wl.n_nodes[s])
        assert b["tree"].N == n == one["tree"].N
        assert list(b["tree"].parent) == list(one["tree"].parent)
        assert list(b["tree"].token) == list(one["tree"].token)
        for key in ("A", "path", "bonus"):
            assert b["verify"][key] == one["verify"][key], (s, key)
        np.testing.assert_array_equal(b["o"], one["o"])
        assert b["P_new"] == one["P_new"] == int(wl.P[s]) + b["verify"]["A"] + 1
        P = int(wl.P[s])
        np.testing.assert_array_equal(b["k"][:, :P + n], one["k"])
        np.testing.assert_array_equal(b["v"][:, :P + n], one["v"])


def test_ragged_sizes_follow_the_config():
    wl = make_workload("c6_ragged_serving", 9, S=40, P=500, P_min=200, B_min=5, V=50, Hq=4, Hkv=4, D=64)
    cfg = wl.cfg
    assert wl.P.min() >= 200 and wl.P.max() <= 500
    assert wl.n_nodes.min() >= 6 and wl.n_nodes.max() <= cfg.N
    for s in range(cfg.S):
        n = int(wl.n_nodes[s])
        assert (wl.parent[s, n:] == -1).all() and (wl.token[s, n:] == -1).all()
        assert (wl.parent[s, 1:n] >= 0).all()
