"""Seeded sweep of rejection-sampling verification against the oracle (run with -m sweep).

Evidence for the walk's cross-workgroup exchanges beyond the parity cases: many distinct
seeds of the batched shape (8 sequences of 65-node random trees, vocabulary 32000, target
3 randn, draft = target + 1.5 randn), every sequence's accepted path and bonus token
compared with the float64 oracle's, the workspace reused from seed to seed, stopping at the
first mismatch or device error. DTV_SWEEP_SEEDS sets the number of seeds (default 500).
"""
from __future__ import annotations

import os
import time

import numpy as np
import pytest
import torch

import draft_tree_verification_build_amd as dtv
from draft_tree_verification_build_amd.step import to_device
from oracle import rows as orows
from oracle import step as ostep
from oracle import verify as overify
from tests.gpu_common import need_gpu
from workloads import make_workload

pytestmark = pytest.mark.sweep
DEV = "cuda"


def test_sample_walk_seed_sweep():
    need_gpu()
    from tests.test_gpu_parity import _upload_tree_with_rows
    seeds = int(os.environ.get("DTV_SWEEP_SEEDS", "500"))
    ws = dtv.Workspace(DEV)
    t0 = time.time()
    rejections = accepted = 0
    for i in range(seeds):
        seed = 1000 + i
        wl = make_workload("c5_batched_llama2_70b", seed, P=16)
        cfg = wl.cfg
        otrees = [ostep.build_tree(wl, s) for s in range(cfg.S)]
        tree = _upload_tree_with_rows(otrees, cfg.N)
        path, plen, bonus = dtv.tree_verify_sample(
            tree, to_device(wl.target, cfg.dtype, DEV), to_device(wl.draft, cfg.dtype, DEV),
            torch.from_numpy(wl.u_acc.view(np.int32)).to(DEV), torch.from_numpy(wl.u_res.view(np.int32)).to(DEV), ws)
        assert ws.status("verify_sample") == 0, f"seed {seed}: device status"
        path, plen, bonus = path.cpu().numpy(), plen.cpu().numpy(), bonus.cpu().numpy()
        for s in range(cfg.S):
            t = otrees[s]
            ref = overify.sample(t.parent, t.token, t.row, lambda r: orows.decode(wl.target[s, r], cfg.dtype),
                                 lambda r: orows.decode(wl.draft[s, r], cfg.dtype), wl.u_acc[s], wl.u_res[s])
            A = int(plen[s]) - 1
            assert A == ref["A"] and list(path[s, :A + 1]) == ref["path"] and int(bonus[s]) == ref["bonus"], \
                f"seed {seed} sequence {s}: GPU A={A} bonus={int(bonus[s])}, oracle A={ref['A']} bonus={ref['bonus']}"
            accepted += A
            rejections += sum(1 for c, u, r in ref["decisions"] if not u < r)
        if (i + 1) % 25 == 0:
            print(f"sweep: {i + 1}/{seeds} seeds agree ({accepted} accepted tokens, {rejections} rejections, "
                  f"{time.time() - t0:.0f} s)", flush=True)
