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


def build_tree(wl, s: int, margins: list | None = None) -> build.Tree:
    """Sequence s's tree; ``margins`` (a list) receives the build's cross-row decision margins."""
    cfg = wl.cfg
    draft = lambda r: decode(wl.draft[s, r], cfg.dtype)
    if cfg.build == "given":
        n = cfg.N if getattr(wl, "n_nodes", None) is None else int(wl.n_nodes[s])
        return build.given_tree(wl.parent[s][:n], wl.token[s][:n])
    if cfg.build == "talon":
        return build.talon(draft, cfg.B, cfg.K, cfg.alpha, margins=margins)
    if cfg.build == "spine":
        return build.spine(draft, wl.spine[s], wl.widths)
    if cfg.build == "opt":
        return build.opt_tree(draft, cfg.n, cfg.delta, cfg.max_layers, margins=margins)
    raise ValueError(cfg.build)


def run_step(wl, attn_pairs=None, sequences=None, with_attention=True, timings=None, margins=None) -> list:
    """Per sequence: tree, mask words, attention output, verification and compaction.

    ``attn_pairs`` restricts attention to the listed (node, head) pairs; ``sequences``
    restricts the step to some sequences. ``timings`` (a dict) receives seconds per stage;
    ``margins`` (a list) receives every cross-row decision margin of the build and the
    verification.
    """
    cfg = wl.cfg
    out = []
    seqs = range(cfg.S) if sequences is None else sequences
    tm = timings if timings is not None else {}
    for s in seqs:
        t0 = time.perf_counter()
        tree = build_tree(wl, s, margins=margins)
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
                                wl.u_acc[s], wl.u_res[s], margins=margins)
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


def decode_capacity(cfg, steps: int) -> int:
    """Cache rows per (sequence, KV head) for ``steps`` steps: each step appends at most N
    rows (path plus the next tree block), after a prefix of at most cfg.P."""
    return cfg.P + (steps + 1) * cfg.N


def run_decode(inputs, steps: int, with_attention=False, attn_pairs=None, after_step=None) -> dict:
    """A decoding loop of ``steps`` draft-tree steps on one KV cache.

    ``inputs(t)`` gives step t's workload: step 0 with the prefix and the first tree in its
    cache; later steps with only their tree's keys and values (slots 0..N-1), which are
    written at each sequence's current prefix length P_t. Each step is ``run_step`` on the
    cache as it stands; its compaction leaves the accepted path's rows at P_t .. P_t + A_t
    and P_{t+1} = P_t + A_t + 1 (the bonus token becomes the next step's root and is not
    written). Returns the per-step results, the final cache and prefix lengths, and per
    sequence the bookkeeping of the TALON page, section 5.3, over the loop (N_v = steps
    verification passes, N_d = the draft layers the builds spent, L = sum of A_t + 1).
    ``after_step(t, results)``, if given, sees every step's results before step t + 1's
    inputs are asked for (an adaptive drafting policy observes the step there).
    """
    import dataclasses
    wl0 = inputs(0)
    cfg = wl0.cfg
    N, S = cfg.N, cfg.S
    cap = decode_capacity(cfg, steps)
    shape = (S, cfg.Hkv, cap, cfg.D)
    k = np.zeros(shape, dtype=wl0.k.dtype)
    v = np.zeros(shape, dtype=wl0.v.dtype)
    k[:, :, :wl0.k.shape[2]] = wl0.k
    v[:, :, :wl0.v.shape[2]] = wl0.v
    P = np.asarray(wl0.P, dtype=np.int64).copy()
    log = []
    for t in range(steps):
        wl = wl0 if t == 0 else inputs(t)
        if t > 0:
            for s in range(S):
                k[s, :, P[s]:P[s] + N] = wl.k[s, :, :N]
                v[s, :, P[s]:P[s] + N] = wl.v[s, :, :N]
        view = dataclasses.replace(wl, P=P.astype(np.int32), P_cap=cap, k=k, v=v)
        res = run_step(view, attn_pairs=attn_pairs, with_attention=with_attention)
        for s in range(S):
            k[s] = res[s]["k"]
            v[s] = res[s]["v"]
            P[s] = res[s]["P_new"]
        log.append(res)
        if after_step is not None:
            after_step(t, res)
    books = [bookkeeping.bookkeeping([log[t][s]["verify"]["A"] for t in range(steps)],
                                     sum(log[t][s]["tree"].layers for t in range(steps)), 1.0)
             for s in range(S)]
    return {"steps": log, "k": k, "v": v, "P": P, "bookkeeping": books}
