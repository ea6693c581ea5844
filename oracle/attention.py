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

from .mask import ancestors


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
