"""A whole step captured as a HIP graph gives, on every replay, exactly what the eager step gives.

The step's kernels keep state between calls in their workspaces (result slots that the
consumer clears again), so each replay is checked, with eager steps and synchronisations of
the program's own between replays, against an eager step on the same inputs. The KV cache is
restored before every step because the compaction rewrites it in place.
"""
from __future__ import annotations

import pytest
import torch

from draft_tree_verification_build_amd.step import DraftTreeStep
from tests.gpu_common import need_gpu
from workloads import make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _outputs(step):
    t = step.tree
    out = {"n_nodes": t.n_nodes, "parent": t.parent, "token": t.token, "depth": t.depth,
           "row": t.row, "score": t.score, "anc": t.anc, "o": step.o, "P_new": step.P_new,
           "k": step.k, "v": step.v}
    for i, x in enumerate(step.verify_out):
        out[f"verify{i}"] = x
    torch.cuda.synchronize()
    return {name: x.detach().clone() for name, x in out.items()}


def _assert_same(got, want, label):
    for name, w in want.items():
        assert torch.equal(got[name], w), f"{label}: {name} differs from the eager step"


@pytest.mark.parametrize("name,seed,ov", [
    ("c1_tiny", 1, {}),
    ("c2_talon_llama3_8b", 2, {}),
    ("c3_goose_spine", 3, {}),
    ("c4_opt_llama2_7b", 4, {"P": 512}),
    ("c5_batched_llama2_70b", 5, {"P": 1024}),
])
def test_graph_replay_matches_eager(name, seed, ov):
    need_gpu()
    wl = make_workload(name, seed, **ov)
    step = DraftTreeStep(wl, DEV)
    k0, v0 = step.k.clone(), step.v.clone()

    def restore():
        step.k.copy_(k0)
        step.v.copy_(v0)

    step.run()            # warm: workspaces allocated outside the capture
    restore()
    step.run()
    want = _outputs(step)
    assert all(v == 0 for v in step.ws_status().values())

    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run()
    for r in range(3):
        restore()
        graph.replay()
        got = _outputs(step)
        _assert_same(got, want, f"replay {r}")
        restore()
        step.run()        # eager work between replays
        _assert_same(_outputs(step), want, f"eager step after replay {r}")
    assert all(v == 0 for v in step.ws_status().values())


def test_graph_replay_matches_oracle_c2():
    """The headline step (TALON tree on the Llama-3-8B shape) captured as a HIP graph: every
    replay against the float64 oracle directly, not only against the eager step: tree arrays
    and masks, path and bonus, new prefix length and compacted cache bit-exact, attention
    outputs (every row) within 2e-2."""
    need_gpu()
    import numpy as np
    from oracle import step as ostep
    from tests.gpu_common import assert_tree_equal, tree_to_numpy
    from tests.test_gpu_parity import attn_compare, attn_reference
    wl = make_workload("c2_talon_llama3_8b", 2)
    step = DraftTreeStep(wl, DEV)
    k0, v0 = step.k.clone(), step.v.clone()
    step.run()            # warm: workspaces allocated outside the capture
    assert all(v == 0 for v in step.ws_status().values())
    res = ostep.run_step(wl, with_attention=False)[0]
    graph = torch.cuda.CUDAGraph()
    step.k.copy_(k0)
    step.v.copy_(v0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step.run()
    refs = None
    for r in range(3):
        step.k.copy_(k0)
        step.v.copy_(v0)
        step.o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert all(v == 0 for v in step.ws_status().values())
        g = tree_to_numpy(step.tree)
        assert_tree_equal(g, 0, res["tree"], step.tree.words)
        if refs is None:
            refs = attn_reference(wl, g)
        attn_compare(step.o.float().cpu().numpy(), refs, 2e-2, f"c2 graph replay {r}")
        path, plen, bonus, _ = [t.cpu() for t in step.verify_out]
        A = int(plen[0]) - 1
        assert A == res["verify"]["A"] and list(path[0, :A + 1].numpy()) == res["verify"]["path"]
        assert int(bonus[0]) == res["verify"]["bonus"]
        assert int(step.P_new[0]) == res["P_new"]
        kk = step.k.view(torch.int16).cpu().numpy().view(np.uint16)
        vv = step.v.view(torch.int16).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(kk[0], res["k"])
        np.testing.assert_array_equal(vv[0], res["v"])
