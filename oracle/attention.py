"""Tree-masked attention, float64.

The OPT-Tree summary (section 2) verifies all tree tokens in one target pass with a
tree attention mask; the concept page ("Why it is a win") notes that the verifier
processes the k+1 positions in one pass. For node i and query head h:

    o[i, h] = sum_j softmax_j(q[i, h] . k[j, kv] * scale) v[j, kv]

over the key set J(i) = {0 .. P-1} (the whole committed prefix) united with
{P + j : j an ancestor-or-self of i} (the tree block sits at cache positions P + slot).

Readings: scale = 1/sqrt(D); grouped-query heads map query head h to KV head
h // (Hq / Hkv); no positional encoding is applied here (Q and K arrive rotated).
"""
from __future__ import annotations

import numpy as np

from .mask import ancestor_matrix, ancestors


def node_head(q_ih: np.ndarray, k_kv: np.ndarray, v_kv: np.ndarray, P: int,
              anc_slots, scale: float) -> np.ndarray:
    """One output row. q_ih [D]; k_kv, v_kv [P_cap][D] (float64)."""
    keys = list(range(P)) + [P + j for j in anc_slots]
    kk = k_kv[keys]
    vv = v_kv[keys]
    s = (kk @ q_ih) * scale
    w = np.exp(s - np.max(s))
    w = w / np.sum(w)
    return w @ vv


def tree_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, P: int, parent,
                   scale: float | None = None, pairs=None) -> np.ndarray:
    """All outputs of one sequence (or only ``pairs`` = [(i, h), ...]).

    q [N][Hq][D], k and v [Hkv][P_cap][D], all float64. Returns o [N][Hq][D] (rows not
    in ``pairs`` are NaN).
    """
    N, Hq, D = q.shape
    Hkv = k.shape[0]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.full((N, Hq, D), np.nan)
    if pairs is None:
        pairs = [(i, h) for i in range(N) for h in range(Hq)]
    anc = {}
    for i, h in pairs:
        if i not in anc:
            anc[i] = ancestors(parent, i)
        o[i, h] = node_head(q[i, h], k[h // g], v[h // g], P, anc[i], scale)
    return o


def tree_attention_dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, P: int, parent,
                         scale: float | None = None) -> np.ndarray:
    """All outputs of one sequence, the same definition with one matrix product per KV head.

    For KV head kv the query rows of its g heads meet every key of the prefix and of the
    tree block at once: scores = q k^T * scale, tree keys that are not an ancestor-or-self
    of the query's node are excluded (their weight is exactly 0), then a softmax over each
    row and a product with v. q [N][Hq][D], k and v [Hkv][P_cap][D], float64; returns
    o [N][Hq][D]. This is the per-row definition of ``tree_attention`` evaluated for all
    rows at once, for full-size checks that the per-row loop would take minutes over.
    """
    N, Hq, D = q.shape
    Hkv = k.shape[0]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    visible = np.ones((N, P + N), dtype=bool)
    visible[:, P:] = ancestor_matrix(parent)          # row i: prefix, then anc(i) in the tree block
    o = np.empty((N, Hq, D))
    for kv in range(Hkv):
        qg = q[:, kv * g:(kv + 1) * g, :].reshape(N * g, D)   # row n*g + h' = (node n, head kv*g + h')
        s = (qg @ k[kv, :P + N].T) * scale                       # [N*g][P+N]
        s = np.where(np.repeat(visible, g, axis=0), s, -np.inf)
        w = np.exp(s - np.max(s, axis=1, keepdims=True))
        w = w / np.sum(w, axis=1, keepdims=True)
        o[:, kv * g:(kv + 1) * g, :] = (w @ v[kv, :P + N]).reshape(N, g, D)
    return o
