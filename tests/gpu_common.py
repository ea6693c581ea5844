"""Shared pieces of the GPU parity tests: device checks and oracle/GPU comparisons."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import mask as omask


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def tree_to_numpy(tree):
    torch.cuda.synchronize()
    return {name: getattr(tree, name).cpu().numpy() for name in
            ("n_nodes", "parent", "token", "depth", "row", "score", "anc", "layers")}


def assert_tree_equal(gpu: dict, s: int, otree, words: int, check_scores=True, check_row=True):
    """Tree structure bit-exact, scores to 1e-12 (float64 sums of exp/log differ in the last bits)."""
    N = otree.N
    assert int(gpu["n_nodes"][s]) == N
    np.testing.assert_array_equal(gpu["parent"][s, :N], np.asarray(otree.parent))
    np.testing.assert_array_equal(gpu["token"][s, :N], np.asarray(otree.token))
    np.testing.assert_array_equal(gpu["depth"][s, :N], np.asarray(otree.depth))
    if check_row:
        np.testing.assert_array_equal(gpu["row"][s, :N], np.asarray(otree.row))
    anc = omask.pack_words(omask.ancestor_matrix(otree.parent), words)
    np.testing.assert_array_equal(gpu["anc"][s, :N].view(np.uint64), anc)
    if check_scores:
        np.testing.assert_allclose(gpu["score"][s, :N], np.asarray(otree.score), rtol=0, atol=1e-12)
