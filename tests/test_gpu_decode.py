"""The device decoding loop (several draft-tree steps on one growing KV cache) equals the
oracle's loop: per step and sequence the accepted length, path and bonus token exactly,
the final prefix lengths, the whole final cache bit for bit, and the bookkeeping."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from draft_tree_verification_build_amd import goose as dgoose
from draft_tree_verification_build_amd.decode import DraftTreeDecoder
from oracle import goose as og
from oracle import step as ostep
from tests.gpu_common import need_gpu
from workloads import config_by_name, make_step_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


@pytest.mark.parametrize("name,seed,ov,steps", [
    ("c1_tiny", 1, {}, 6),
    ("c2_talon_llama3_8b", 2, {"P": 64, "V": 3000}, 3),
    ("c3_goose_spine", 3, {"P": 64, "V": 2000}, 3),
    ("c4_opt_llama2_7b", 4, {"P": 64, "V": 2000, "n": 64, "max_layers": 4}, 3),
    ("c5_batched_llama2_70b", 5, {"S": 3, "P": 200, "V": 500}, 4),
    ("c6_ragged_serving", 6, {"S": 4, "P": 300, "V": 400}, 4),
])
def test_decode_loop_matches_oracle(name, seed, ov, steps):
    need_gpu()
    inputs = lambda t: make_step_inputs(name, seed, t, planted=0.7, **ov)
    dec = DraftTreeDecoder(inputs, steps, DEV)
    log = dec.run()
    ref = ostep.run_decode(inputs, steps)
    S = dec.S
    for t in range(steps):
        for s in range(S):
            r = ref["steps"][t][s]["verify"]
            A = int(log[t]["A"][s])
            assert A == r["A"], (t, s)
            assert list(log[t]["path"][s, :A + 1]) == r["path"], (t, s)
            assert int(log[t]["bonus"][s]) == r["bonus"], (t, s)
    np.testing.assert_array_equal(dec.P_host, ref["P"])
    k, v = _bits(dec.k), _bits(dec.v)
    for s in range(S):
        p = int(ref["P"][s])
        np.testing.assert_array_equal(k[s, :, :p], ref["k"][s, :, :p])
        np.testing.assert_array_equal(v[s, :, :p], ref["v"][s, :, :p])
    if dec.cfg.build == "opt":   # OPT-Tree's forecast E[A] = sum of exp(score) over the tree
        for t in range(steps):
            for s in range(S):
                tr = ref["steps"][t][s]["tree"]
                want = float(np.exp(np.asarray(tr.score[1:tr.N], dtype=np.float64)).sum())
                assert log[t]["E_A_predicted"][s] == pytest.approx(want, rel=1e-9)
    books = dec.bookkeeping(1.0)
    for s in range(S):
        for key in ("E_A", "eta", "speedup"):
            assert books[s][key] == pytest.approx(ref["bookkeeping"][s][key], rel=1e-12, abs=1e-12), key


@pytest.mark.parametrize("seed,ov,steps", [
    (3, {"P": 64, "V": 2000, "spine_p": 0.8}, 6),
    (31, {"P": 64, "V": 1500, "spine_p": 0.4, "S": 2}, 5),
])
def test_goose_adaptive_decode_matches_oracle(seed, ov, steps):
    """GOOSE's adaptive topology over a decoding loop: the host policy plans each step's
    spine length and branch widths from the previous steps' spine acceptance; the oracle
    loop runs its own policy. Both must plan the same topologies and give the same steps."""
    need_gpu()
    name = "c3_goose_spine"
    B = config_by_name(name, **ov).N - 1

    def inputs_for(topo):
        return lambda t: make_step_inputs(name, seed, t, n_spine=topo[t][0], n_forks=len(topo[t][1]),
                                          spine_widths=tuple(topo[t][1]), **ov)

    pol = dgoose.SpineTopology(B)
    topo = {0: pol.plan()}
    dec = DraftTreeDecoder(inputs_for(topo), steps, DEV)
    for t in range(steps):
        if t > 0:
            topo[t] = pol.plan()
        rec = dec.step(t)
        L = topo[t][0]
        pol.observe([dgoose.spine_accepted(rec["path"][s][:int(rec["A"][s]) + 1], L) for s in range(dec.S)], L)

    state = {"avg": 0.5}
    otopo = {0: og.plan(0.5, B)}

    def after(t, res):
        L = otopo[t][0]
        state["avg"] = og.update(state["avg"], [og.spine_run(r["verify"]["path"], L) for r in res], L)
        otopo[t + 1] = og.plan(state["avg"], B)

    ref = ostep.run_decode(inputs_for(otopo), steps, after_step=after)
    for t in range(steps):
        assert (topo[t][0], list(topo[t][1])) == (otopo[t][0], list(otopo[t][1])), t
        assert sum(topo[t][1]) + topo[t][0] == B
        for s in range(dec.S):
            r = ref["steps"][t][s]["verify"]
            A = int(dec.log[t]["A"][s])
            assert A == r["A"] and list(dec.log[t]["path"][s, :A + 1]) == r["path"], (t, s)
            assert int(dec.log[t]["bonus"][s]) == r["bonus"], (t, s)
    np.testing.assert_array_equal(dec.P_host, ref["P"])
    k = _bits(dec.k)
    for s in range(dec.S):
        p = int(ref["P"][s])
        np.testing.assert_array_equal(k[s, :, :p], ref["k"][s, :, :p])
    assert len({topo[t][0] for t in range(steps)}) > 1   # the topology did adapt
