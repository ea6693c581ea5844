"""Committing the accepted path to the KV cache.

The concept page ("The protocol", step 4) appends the accepted tokens and loops. The
tree's keys and values were written at cache positions P + slot by the verification
pass; after acceptance the root and the accepted nodes must sit right behind the
prefix, in path order:

    cache[P + k] <- cache[P + path[k]]  for k = 0 .. A,  then P <- P + A + 1.

The bonus token is the next step's root and has no cache row yet.
"""
from __future__ import annotations

import numpy as np


def kv_compact(k: np.ndarray, v: np.ndarray, P: int, path) -> tuple[np.ndarray, np.ndarray, int]:
    """k, v [Hkv][P_cap][D]. Returns new copies and the new prefix length."""
    k2, v2 = k.copy(), v.copy()
    for kk, node in enumerate(path):
        k2[:, P + kk] = k[:, P + int(node)]
        v2[:, P + kk] = v[:, P + int(node)]
    return k2, v2, P + len(path)
