"""One whole draft-tree step: build, tree attention, verification, compaction.

The concept page ("The protocol") drafts, verifies in one target pass, accepts and
appends; the OPT-Tree summary (section 2) does the same for a tree with a tree mask.
This chains the oracle's stages in that order for every sequence of a workload.

``wl`` is any object with the fields of a synthetic workload (cfg, P, q, k, v, draft,
target, and parent/token, spine/widths or u_acc/u_res as the configuration needs);
arrays hold stored values (float32, or bf16 bit patterns as uint16).
"""
from __future__ import annotations

import time

import numpy as np

from . import attention, bookkeeping, build, compact, mask, verify
from .rows import decode


def build_tree(wl, s: int) -> build.Tree:
    cfg = wl.cfg
    draft = lambda r: decode(wl.draft[s, r], cfg.dtype)
    if cfg.build == "given":
        n = cfg.N if getattr(wl, "n_nodes", None) is None else int(wl.n_nodes[s])
        return build.given_tree(wl.parent[s][:n], wl.token[s][:n])
    if cfg.build == "talon":
        return build.talon(draft, cfg.B, cfg.K, cfg.alpha)
    if cfg.build == "spine":
        return build.spine(draft, wl.spine[s], wl.widths)
    if cfg.build == "opt":
        return build.opt_tree(draft, cfg.n, cfg.delta, cfg.max_layers)
    raise ValueError(cfg.build)


def run_step(wl, attn_pairs=None, sequences=None, with_attention=True, timings=None) -> list:
    """Per sequence: tree, mask words, attention output, verification and compaction.

    ``attn_pairs`` restricts attention to the listed (node, head) pairs; ``sequences``
    restricts the step to some sequences. ``timings`` (a dict) receives seconds per stage.
    """
    cfg = wl.cfg
    out = []
    seqs = range(cfg.S) if sequences is None else sequences
    tm = timings if timings is not None else {}
    for s in seqs:
        t0 = time.perf_counter()
        tree = build_tree(wl, s)
        anc = mask.ancestor_matrix(tree.parent)
        words = (cfg.N + 63) // 64
        anc_words = mask.pack_words(anc, words)
        t1 = time.perf_counter()
        P = int(wl.P[s])
        o = None
        if with_attention:
            q = decode(wl.q[s], cfg.dtype).reshape(wl.q.shape[1:])
            k = decode(wl.k[s], cfg.dtype).reshape(wl.k.shape[1:])
            v = decode(wl.v[s], cfg.dtype).reshape(wl.v.shape[1:])
            o = attention.tree_attention(q[:tree.N], k, v, P, tree.parent, pairs=attn_pairs)
        t2 = time.perf_counter()
        target = lambda r: decode(wl.target[s, r], cfg.dtype)
        draft = lambda r: decode(wl.draft[s, r], cfg.dtype)
        if cfg.verify == "greedy":
            ver = verify.greedy(tree.parent, tree.token, tree.row, target)
        else:
            ver = verify.sample(tree.parent, tree.token, tree.row, target, draft,
                                wl.u_acc[s], wl.u_res[s])
        t3 = time.perf_counter()
        k2, v2, P_new = compact.kv_compact(wl.k[s], wl.v[s], P, ver["path"])
        t4 = time.perf_counter()
        for key, dt in (("build", t1 - t0), ("attention", t2 - t1), ("verify", t3 - t2),
                        ("compact", t4 - t3)):
            tm[key] = tm.get(key, 0.0) + dt
        out.append({"tree": tree, "anc_words": anc_words, "o": o, "verify": ver,
                    "k": k2, "v": v2, "P_new": P_new})
    return out


def step_bookkeeping(results, gamma: float) -> dict:
    """Bookkeeping over the sequences of one step, each counted as a verification pass."""
    return bookkeeping.bookkeeping([r["verify"]["A"] for r in results],
                                   sum(r["tree"].layers for r in results), gamma)
