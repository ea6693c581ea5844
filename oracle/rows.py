"""Row primitives over one vocabulary row of logits (float64).

The TALON page (section 5.2.1, path score formula) multiplies draft probabilities
p_d(x_t | x_<t); its root initialisation (section 5.2.2) takes TopK of p_d. The
OPT-Tree summary (section 2, Preliminaries) accepts the branch that matches the
target's highest-probability token. The speculative-decoding concept page (section
"The protocol", step 3) compares p(x) with q(x). All of these need, per row: the
maximum, the index of the maximum, the normaliser log sum exp, and the K largest
entries.

Readings:
* values are compared as stored (bf16 or fp32 logits, decoded exactly to float64);
  probabilities are never used to rank tokens, so the order of a row is exact;
* ties go to the lowest index, for argmax and for top-K;
* the softmax has temperature 1.
"""
from __future__ import annotations

import math

import numpy as np


def decode(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Stored row -> float64, exactly. bf16 rows arrive as uint16 bit patterns."""
    if dtype == "bf16":
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def row_max_argmax(x: np.ndarray) -> tuple[float, int]:
    """Largest value and the lowest index that holds it."""
    m = float(np.max(x))
    return m, int(np.argmax(x))  # numpy returns the first occurrence


def row_lse(x: np.ndarray) -> float:
    """log sum_j exp(x_j) in float64, shifted by the maximum."""
    m = float(np.max(x))
    return m + math.log(float(np.sum(np.exp(x - m))))


def row_logp(x: np.ndarray) -> np.ndarray:
    """log softmax(x) = x - lse(x)."""
    return x - row_lse(x)


def row_softmax(x: np.ndarray) -> np.ndarray:
    """softmax(x) = exp(x - lse(x))."""
    return np.exp(x - row_lse(x))


def topk(x: np.ndarray, K: int) -> np.ndarray:
    """Indices of the K largest values, largest first, ties by lowest index.

    A stable sort of -x keeps equal values in index order.
    """
    K = min(int(K), x.shape[0])
    return np.argsort(-x, kind="stable")[:K].astype(np.int64)
