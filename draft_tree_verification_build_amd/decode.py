"""A multi-step speculative decoding loop on one KV cache, through libdtv.

Each step builds a draft tree, attends with the tree mask, verifies and compacts the
accepted path into the cache in the verification launch, so that the prefix grows by
A_t + 1 per step (the bonus token is the next step's root and is not written). The inputs
of a step stand in for the draft and target models' outputs: ``inputs(t)`` returns them
(any object with the fields of ``workloads.Workload``); step 0 carries the prefix, and a
later step only its tree's keys and values at slots 0..N-1, which the loop writes at each
sequence's current prefix length, as a target forward over the tree would.

The host reads the accepted lengths after every step (one synchronisation per step), which
is what a decoding loop needs to emit tokens and to size the next step's attention launch.
"""
from __future__ import annotations

import numpy as np
import torch

from . import api
from .step import to_device


class DraftTreeDecoder:
    def __init__(self, inputs, steps: int, device="cuda"):
        self.inputs = inputs
        self.steps = steps
        self.device = torch.device(device)
        wl0 = inputs(0)
        cfg = wl0.cfg
        self.cfg = cfg
        self.S, self.N = cfg.S, cfg.N
        self.cap = cfg.P + (steps + 1) * cfg.N      # each step appends at most N rows
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self.k = torch.zeros((cfg.S, cfg.Hkv, self.cap, cfg.D), dtype=dt, device=self.device)
        self.v = torch.zeros_like(self.k)
        n0 = wl0.k.shape[2]
        self.k[:, :, :n0] = to_device(wl0.k, cfg.dtype, self.device)
        self.v[:, :, :n0] = to_device(wl0.v, cfg.dtype, self.device)
        self.P_host = np.asarray(wl0.P, dtype=np.int64).copy()
        self.P = torch.from_numpy(self.P_host.astype(np.int32)).to(self.device)
        self.P_new = torch.zeros_like(self.P)
        self.ws = api.Workspace(self.device)
        self.tree = api.Tree(cfg.S, cfg.N, self.device)
        self.o = None
        self.log = []
        self._wl0 = wl0

    def upload(self, t: int) -> dict:
        """Device copies of step t's inputs (the loop can upload every step before timing)."""
        cfg, dev = self.cfg, self.device
        wl = self._wl0 if t == 0 else self.inputs(t)
        d = {"q": to_device(wl.q, cfg.dtype, dev), "draft": to_device(wl.draft, cfg.dtype, dev),
             "target": to_device(wl.target, cfg.dtype, dev), "tree_k": None, "tree_v": None}
        if t > 0:
            d["tree_k"] = to_device(wl.k, cfg.dtype, dev)
            d["tree_v"] = to_device(wl.v, cfg.dtype, dev)
        if cfg.build == "given":
            d["parent"] = torch.from_numpy(np.asarray(wl.parent, dtype=np.int32)).to(dev)
            d["token"] = torch.from_numpy(np.asarray(wl.token, dtype=np.int32)).to(dev)
            n = np.full(cfg.S, cfg.N, dtype=np.int32) if wl.n_nodes is None else np.asarray(wl.n_nodes, np.int32)
            d["n_nodes"] = torch.from_numpy(n).to(dev)
        if cfg.build == "spine":
            d["spine"] = torch.from_numpy(np.asarray(wl.spine, dtype=np.int32)).to(dev)
            d["widths"] = np.asarray(wl.widths, dtype=np.int32)
        if cfg.verify == "sample":
            d["u_acc"] = torch.from_numpy(np.asarray(wl.u_acc, dtype=np.uint32).view(np.int32)).to(dev)
            d["u_res"] = torch.from_numpy(np.asarray(wl.u_res, dtype=np.uint32).view(np.int32)).to(dev)
        return d

    def step(self, t: int, d: dict | None = None, stream=None) -> dict:
        """Step t; returns per sequence the accepted length A, the path and the bonus token."""
        cfg = self.cfg
        d = self.upload(t) if d is None else d
        N = self.N
        if t > 0:   # the step's tree keys and values follow each sequence's prefix
            for s in range(self.S):
                p = int(self.P_host[s])
                self.k[s, :, p:p + N] = d["tree_k"][s, :, :N]
                self.v[s, :, p:p + N] = d["tree_v"][s, :, :N]
        tree, ws = self.tree, self.ws
        if cfg.build == "given":
            tree.parent.copy_(d["parent"])
            tree.token.copy_(d["token"])
            tree.n_nodes.copy_(d["n_nodes"])
            api.tree_build_given(tree, ws, stream=stream)
        elif cfg.build == "talon":
            api.tree_build_talon(tree, d["draft"], cfg.B, cfg.K, cfg.alpha, ws, stream=stream)
        elif cfg.build == "opt":
            api.tree_build_opt(tree, d["draft"], cfg.n, cfg.delta, cfg.max_layers, ws, stream=stream)
        elif cfg.build == "spine":
            api.tree_build_spine(tree, d["spine"], d["widths"], d["draft"], ws, stream=stream)
        else:
            raise NotImplementedError(cfg.build)
        if self.o is None:
            self.o = torch.zeros_like(d["q"])
        api.tree_attn(d["q"], self.k, self.v, self.P, int(self.P_host.max()), tree, ws, o=self.o, stream=stream)
        kv = (self.k, self.v, self.P, self.P_new)
        if cfg.verify == "greedy":
            path, plen, bonus = api.tree_verify_greedy(tree, d["target"], ws, stream=stream, kv=kv)[:3]
        else:
            path, plen, bonus = api.tree_verify_sample(tree, d["target"], d["draft"], d["u_acc"], d["u_res"],
                                                       ws, stream=stream, kv=kv)[:3]
        # the step's results in one read: path length, bonus, new prefix, layers, path and the
        # status word of every workspace (a kernel that refused or timed out records it there)
        S = self.S
        words = ws.status_words()
        res = torch.cat([plen, bonus, self.P_new, tree.layers, path.reshape(-1), *words.values()]).cpu().numpy()
        if (res[len(res) - len(words):] != 0).any():
            ws.check(stream)   # raises with the library's message
        res = res[:len(res) - len(words)]
        plen_h, bonus_h = res[:S], res[S:2 * S]
        P_new = res[2 * S:3 * S].astype(np.int64)
        if (P_new < 0).any():
            raise RuntimeError(f"step {t}: the cache cannot hold the step (P_new {P_new})")
        rec = {"A": (plen_h - 1).astype(np.int64), "path": res[4 * S:].reshape(S, -1), "bonus": bonus_h,
               "layers": res[3 * S:4 * S], "P": self.P_host.copy()}
        if cfg.build == "opt":
            # OPT-Tree's own forecast: the expected number of accepted draft tokens, the sum
            # of the draft path probabilities exp(score) over the tree's non-root nodes
            sc = tree.score.cpu().numpy()
            nn = tree.n_nodes.cpu().numpy()
            rec["E_A_predicted"] = np.array([float(np.exp(sc[s, 1:int(nn[s])]).sum()) for s in range(S)])
        self.P_host = P_new
        self.P.copy_(self.P_new)
        self.log.append(rec)
        return rec

    def run(self) -> list:
        for t in range(self.steps):
            self.step(t)
        return self.log

    def bookkeeping(self, gamma: float = 1.0) -> list:
        """Per sequence: N_v, N_d, L, E[A], eta and Speedup over the loop (libdtv's host call)."""
        out = []
        for s in range(self.S):
            acc = [int(r["A"][s]) for r in self.log]
            nd = sum(int(r["layers"][s]) for r in self.log)
            out.append(api.bookkeeping(acc, nd, gamma))
        return out
