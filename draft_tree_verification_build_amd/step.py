"""One draft-tree step on the GPU: build -> tree attention -> verify -> compact.

``DraftTreeStep`` uploads the inputs of a synthetic workload once (any object with the
fields of ``workloads.Workload``), allocates every output and workspace, and then runs
the four stages through libdtv on one stream with no host synchronisation; with
``fuse_compact`` (the default) the verification launch also compacts the cache. The step is
re-runnable: the build, attention and verification read only inputs; the compaction
writes the new prefix length to a separate ``P_new`` and moves cache rows inside the
tree block, which changes attention outputs of later repetitions but not their work.
"""
from __future__ import annotations

import numpy as np
import torch

from . import api


def to_device(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Stored numpy array -> device tensor (bf16 arrives as uint16 bit patterns)."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


class DraftTreeStep:
    def __init__(self, wl, device="cuda", fuse_compact=True):
        cfg = wl.cfg
        self.fuse_compact = fuse_compact
        self.cfg = cfg
        self.device = torch.device(device)
        dev = self.device
        dt = cfg.dtype
        self.S, self.N = cfg.S, cfg.N
        self.P_max = int(np.max(wl.P))
        self.q = to_device(wl.q, dt, dev)
        self.k = to_device(wl.k, dt, dev)
        self.v = to_device(wl.v, dt, dev)
        self.P = torch.from_numpy(np.asarray(wl.P, dtype=np.int32)).to(dev)
        self.draft = to_device(wl.draft, dt, dev)
        self.target = to_device(wl.target, dt, dev)
        self.ws = api.Workspace(dev)
        if cfg.build == "given":
            parent = torch.from_numpy(np.asarray(wl.parent, dtype=np.int32)).to(dev)
            token = torch.from_numpy(np.asarray(wl.token, dtype=np.int32)).to(dev)
            self.tree = api.Tree(self.S, self.N, dev, parent=parent, token=token)
            if wl.n_nodes is None:
                self.tree.n_nodes.fill_(self.N)
            else:   # a ragged batch: each request's own tree size
                self.tree.n_nodes.copy_(torch.from_numpy(np.asarray(wl.n_nodes, dtype=np.int32)))
        else:
            self.tree = api.Tree(self.S, self.N, dev)
        if cfg.build == "spine":
            self.spine = torch.from_numpy(np.asarray(wl.spine, dtype=np.int32)).to(dev)
            self.widths = np.asarray(wl.widths, dtype=np.int32)
        self.o = torch.zeros_like(self.q)
        self.verify_out = (torch.full((self.S, self.N), -1, dtype=torch.int32, device=dev),
                           torch.zeros(self.S, dtype=torch.int32, device=dev),
                           torch.zeros(self.S, dtype=torch.int32, device=dev),
                           torch.zeros((self.S, self.N), dtype=torch.int32, device=dev))
        self.P_new = torch.zeros_like(self.P)
        if cfg.verify == "sample":
            self.u_acc = torch.from_numpy(np.asarray(wl.u_acc, dtype=np.uint32).view(np.int32)).to(dev)
            self.u_res = torch.from_numpy(np.asarray(wl.u_res, dtype=np.uint32).view(np.int32)).to(dev)

    # -- stages ---------------------------------------------------------------------
    def build(self, stream=None):
        cfg = self.cfg
        if cfg.build == "given":
            api.tree_build_given(self.tree, self.ws, stream=stream)
        elif cfg.build == "talon":
            api.tree_build_talon(self.tree, self.draft, cfg.B, cfg.K, cfg.alpha, self.ws, stream=stream)
        elif cfg.build == "opt":
            api.tree_build_opt(self.tree, self.draft, cfg.n, cfg.delta, cfg.max_layers, self.ws, stream=stream)
        elif cfg.build == "spine":
            api.tree_build_spine(self.tree, self.spine, self.widths, self.draft, self.ws, stream=stream)
        else:
            raise NotImplementedError(f"build mode {cfg.build!r} is not built yet")

    def attention(self, stream=None):
        api.tree_attn(self.q, self.k, self.v, self.P, self.P_max, self.tree, self.ws, o=self.o,
                      stream=stream)

    def verify(self, stream=None):
        if self.cfg.verify == "greedy":
            api.tree_verify_greedy(self.tree, self.target, self.ws, out=self.verify_out, stream=stream)
        else:
            api.tree_verify_sample(self.tree, self.target, self.draft, self.u_acc, self.u_res, self.ws,
                                   out=self.verify_out, stream=stream)

    def verify_compact(self, stream=None):
        """Verification that compacts the KV cache along its path in the same launch."""
        kv = (self.k, self.v, self.P, self.P_new)
        if self.cfg.verify == "greedy":
            api.tree_verify_greedy(self.tree, self.target, self.ws, out=self.verify_out, stream=stream, kv=kv)
        else:
            api.tree_verify_sample(self.tree, self.target, self.draft, self.u_acc, self.u_res, self.ws,
                                   out=self.verify_out, stream=stream, kv=kv)

    def compact(self, stream=None):
        path, plen = self.verify_out[0], self.verify_out[1]
        api.kv_compact(self.k, self.v, self.P, path, plen, P_new=self.P_new, stream=stream)

    def stages(self):
        """(name, callable) of every launch group of a step, in order."""
        if self.fuse_compact:
            return [("build", self.build), ("attention", self.attention), ("verify_compact", self.verify_compact)]
        return [("build", self.build), ("attention", self.attention), ("verify", self.verify),
                ("compact", self.compact)]

    def run(self, stream=None):
        for _, fn in self.stages():
            fn(stream)

    def ws_status(self) -> dict:
        """Synchronise and collect the device status of every workspace used so far."""
        return {k: self.ws.status(k) for k in list(self.ws._bufs)}
