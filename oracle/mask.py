"""Depth and tree-attention mask of a draft tree.

The OPT-Tree summary (section 2, Preliminaries) has the target model verify every
tree token in parallel "using a tree attention mask"; the Medusa paragraph of the
speculative-decoding concept page verifies the candidate set with tree attention in
one forward pass. A node's query may see the committed prefix and the tree tokens on
its own root path, itself included.

Conventions (slot numbering): slot 0 is the root (the last committed token, whose key
and value are not yet cached), draft nodes follow in topological order, so
parent[i] < i for i >= 1 and parent[0] = -1.
"""
from __future__ import annotations

import numpy as np


def depths(parent) -> np.ndarray:
    """depth[0] = 0 and depth[i] = depth[parent[i]] + 1."""
    N = len(parent)
    d = np.zeros(N, dtype=np.int64)
    for i in range(1, N):
        p = int(parent[i])
        if not (0 <= p < i):
            raise ValueError(f"parent[{i}] = {p} is not an earlier slot")
        d[i] = d[p] + 1
    return d


def ancestors(parent, i: int) -> list[int]:
    """Slots on the path from the root to node i, root first, i last."""
    path = []
    j = int(i)
    while j >= 0:
        path.append(j)
        j = int(parent[j]) if j > 0 else -1
    return path[::-1]


def ancestor_matrix(parent) -> np.ndarray:
    """anc[i, j] is True when j is i or an ancestor of i (ancestor-or-self)."""
    N = len(parent)
    anc = np.zeros((N, N), dtype=bool)
    for i in range(N):
        for j in ancestors(parent, i):
            anc[i, j] = True
    return anc


def pack_words(anc: np.ndarray, words: int) -> np.ndarray:
    """Pack rows of a boolean mask into little-endian 64-bit words: bit j%64 of word j//64."""
    N, M = anc.shape
    out = np.zeros((N, words), dtype=np.uint64)
    for i in range(N):
        for j in range(M):
            if anc[i, j]:
                out[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return out
