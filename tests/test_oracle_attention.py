"""Pins of the oracle's tree attention (CPU only).

* A chain tree is ordinary causal attention over prefix + chain: checked against
  torch's scaled_dot_product_attention (float64, CPU) with an explicit
  bottom-right-aligned boolean mask.
* A star tree sees prefix + root + itself.
* Grouped-query attention equals multi-head attention with each KV head repeated.
* With no prefix, the root attends only to itself: its output is its own value row.
* Relabelling the nodes of a tree permutes the outputs the same way.
"""
import numpy as np
import torch

from oracle import attention


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa(q, k, v, allowed, scale):
    # q [Hq][Lq][D], k/v [Hq][Lk][D], allowed [Lq][Lk] bool
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(allowed), scale=scale)
    return out.numpy()


def test_chain_equals_causal_attention():
    rng = np.random.default_rng(10)
    for P, N, Hq, Hkv, D in ((0, 5, 2, 2, 8), (37, 17, 4, 2, 16), (64, 65, 2, 1, 8)):
        q = _rand(rng, N, Hq, D)
        k = _rand(rng, Hkv, P + N + 3, D)
        v = _rand(rng, Hkv, P + N + 3, D)
        parent = [-1] + list(range(N - 1))
        o = attention.tree_attention(q, k, v, P, parent)
        g = Hq // Hkv
        kk = np.repeat(k[:, :P + N], g, axis=0)
        vv = np.repeat(v[:, :P + N], g, axis=0)
        # query i sits at absolute position P + i and sees keys 0 .. P + i
        allowed = np.arange(P + N)[None, :] <= (P + np.arange(N))[:, None]
        ref = _sdpa(np.transpose(q, (1, 0, 2)).copy(), kk, vv, allowed, 1.0 / np.sqrt(D))
        np.testing.assert_allclose(o, np.transpose(ref, (1, 0, 2)), rtol=1e-12, atol=1e-12)


def test_star_sees_prefix_root_and_self():
    rng = np.random.default_rng(11)
    P, N, H, D = 20, 9, 3, 8
    q, k, v = _rand(rng, N, H, D), _rand(rng, H, P + N, D), _rand(rng, H, P + N, D)
    parent = [-1] + [0] * (N - 1)
    o = attention.tree_attention(q, k, v, P, parent)
    allowed = np.zeros((N, P + N), dtype=bool)
    allowed[:, :P] = True
    allowed[:, P] = True
    allowed[np.arange(N), P + np.arange(N)] = True
    ref = _sdpa(np.transpose(q, (1, 0, 2)).copy(), k, v, allowed, 1.0 / np.sqrt(D))
    np.testing.assert_allclose(o, np.transpose(ref, (1, 0, 2)), rtol=1e-12, atol=1e-12)


def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(12)
    P, N, Hq, Hkv, D = 15, 11, 8, 2, 8
    parent = [-1] + [int(rng.integers(0, i)) for i in range(1, N)]
    q, k, v = _rand(rng, N, Hq, D), _rand(rng, Hkv, P + N, D), _rand(rng, Hkv, P + N, D)
    o1 = attention.tree_attention(q, k, v, P, parent)
    o2 = attention.tree_attention(q, np.repeat(k, Hq // Hkv, 0), np.repeat(v, Hq // Hkv, 0), P, parent)
    np.testing.assert_array_equal(o1, o2)


def test_single_root_without_prefix_returns_its_value():
    rng = np.random.default_rng(13)
    q, k, v = _rand(rng, 1, 2, 4), _rand(rng, 2, 1, 4), _rand(rng, 2, 1, 4)
    o = attention.tree_attention(q, k, v, 0, [-1])
    np.testing.assert_allclose(o[0], v[:, 0], rtol=0, atol=1e-15)


def test_relabelling_nodes_permutes_outputs():
    rng = np.random.default_rng(14)
    P, H, D = 10, 2, 4
    # tree 0 -> {1, 2}, 1 -> 3 ; relabel by swapping slots 1 and 2 (keeps parents earlier)
    parent = [-1, 0, 0, 1]
    q, k, v = _rand(rng, 4, H, D), _rand(rng, H, P + 4, D), _rand(rng, H, P + 4, D)
    o = attention.tree_attention(q, k, v, P, parent)
    perm = [0, 2, 1, 3]                  # new slot j holds old node perm[j]
    parent2 = [-1, 0, 0, 2]
    q2 = q[perm]
    k2, v2 = k.copy(), v.copy()
    k2[:, P:P + 4] = k[:, P + np.array(perm)]
    v2[:, P:P + 4] = v[:, P + np.array(perm)]
    o2 = attention.tree_attention(q2, k2, v2, P, parent2)
    np.testing.assert_allclose(o2, o[perm], rtol=1e-13, atol=1e-13)


# The all-rows form used by the full-size GPU checks: the same pins, plus agreement with
# the per-row form on random trees with grouped-query heads and a ragged prefix.

def test_dense_chain_equals_causal_attention():
    rng = np.random.default_rng(20)
    for P, N, Hq, Hkv, D in ((0, 5, 2, 2, 8), (37, 17, 4, 2, 16), (64, 65, 2, 1, 8)):
        q = _rand(rng, N, Hq, D)
        k = _rand(rng, Hkv, P + N + 3, D)
        v = _rand(rng, Hkv, P + N + 3, D)
        o = attention.tree_attention_dense(q, k, v, P, [-1] + list(range(N - 1)))
        g = Hq // Hkv
        allowed = np.arange(P + N)[None, :] <= (P + np.arange(N))[:, None]
        ref = _sdpa(np.transpose(q, (1, 0, 2)).copy(), np.repeat(k[:, :P + N], g, axis=0),
                    np.repeat(v[:, :P + N], g, axis=0), allowed, 1.0 / np.sqrt(D))
        np.testing.assert_allclose(o, np.transpose(ref, (1, 0, 2)), rtol=1e-12, atol=1e-12)


def test_dense_star_sees_prefix_root_and_self():
    rng = np.random.default_rng(21)
    P, N, H, D = 20, 9, 3, 8
    q, k, v = _rand(rng, N, H, D), _rand(rng, H, P + N, D), _rand(rng, H, P + N, D)
    o = attention.tree_attention_dense(q, k, v, P, [-1] + [0] * (N - 1))
    allowed = np.zeros((N, P + N), dtype=bool)
    allowed[:, :P + 1] = True
    allowed[np.arange(N), P + np.arange(N)] = True
    ref = _sdpa(np.transpose(q, (1, 0, 2)).copy(), k, v, allowed, 1.0 / np.sqrt(D))
    np.testing.assert_allclose(o, np.transpose(ref, (1, 0, 2)), rtol=1e-12, atol=1e-12)


def test_dense_gqa_equals_repeated_mha_and_per_row_form():
    rng = np.random.default_rng(22)
    for P, N, Hq, Hkv, D in ((15, 11, 8, 2, 8), (0, 30, 4, 4, 16), (130, 70, 16, 2, 8)):
        parent = [-1] + [int(rng.integers(0, i)) for i in range(1, N)]
        q, k, v = _rand(rng, N, Hq, D), _rand(rng, Hkv, P + N + 5, D), _rand(rng, Hkv, P + N + 5, D)
        o1 = attention.tree_attention_dense(q, k, v, P, parent)
        o2 = attention.tree_attention_dense(q, np.repeat(k, Hq // Hkv, 0), np.repeat(v, Hq // Hkv, 0), P, parent)
        np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(o1, attention.tree_attention(q, k, v, P, parent), rtol=1e-12, atol=1e-12)
