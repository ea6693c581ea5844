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
