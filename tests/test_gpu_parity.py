"""GPU parity: every stage of the step through the C ABI against the float64 oracle.

Bars: tree arrays, masks, argmax/top-K indices, paths and bonus tokens bit-exact;
log-sum-exp and path scores to 1e-12 absolute; attention within 2e-2 (bf16) and 1e-4
(fp32) max-abs error of the float64 oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import draft_tree_verification_build_amd as dtv
from draft_tree_verification_build_amd.step import DraftTreeStep, to_device
from oracle import attention as oattn
from oracle import build as obuild
from oracle import compact as ocompact
from oracle import mask as omask
from oracle import rows as orows
from oracle import step as ostep
from oracle import verify as overify
from workloads import f32_to_bf16_bits, make_workload
from tests.gpu_common import assert_tree_equal, need_gpu, tree_to_numpy

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rows(kind, R, V, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        x = rng.standard_normal((R, V), dtype=np.float32) * 3
    elif kind == "ties":          # few distinct values: heavy ties everywhere
        x = rng.integers(-3, 4, size=(R, V)).astype(np.float32)
    elif kind == "equal":
        x = np.full((R, V), 0.5, dtype=np.float32)
    elif kind == "signed_zero":
        x = np.where(rng.random((R, V)) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        x[:, V // 3] = -1.0
    else:
        raise ValueError(kind)
    return x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kind,R,V,K", [
    ("normal", 5, 128256, 10), ("normal", 7, 32000, 512), ("normal", 3, 1000, 16),
    ("normal", 4, 20003, 33), ("ties", 6, 9000, 64), ("equal", 2, 5000, 20),
    ("signed_zero", 3, 4099, 7), ("normal", 2, 8192, 1), ("normal", 3, 77, 77),
])
def test_row_stats(dtype, kind, R, V, K):
    need_gpu()
    x = _rows(kind, R, V, seed=R * 1000 + V + K)
    raw = f32_to_bf16_bits(x) if dtype == "bf16" else x
    ws = dtv.Workspace(DEV)
    maxv, amax, lse, topk = dtv.row_stats(to_device(raw, dtype, DEV), K, ws)
    torch.cuda.synchronize()
    for r in range(R):
        xr = orows.decode(raw[r], dtype)
        m, a = orows.row_max_argmax(xr)
        assert float(maxv[r]) == m and int(amax[r]) == a, (r, float(maxv[r]), m, int(amax[r]), a)
        assert abs(float(lse[r]) - orows.row_lse(xr)) <= 1e-12 * max(1.0, abs(orows.row_lse(xr)))
        np.testing.assert_array_equal(topk[r].cpu().numpy(), orows.topk(xr, K))
    assert ws.status("row_stats") == 0


def _given_tree(parent, token, N, S=1):
    par = torch.tensor(np.asarray(parent, dtype=np.int32).reshape(S, N), device=DEV)
    tok = torch.tensor(np.asarray(token, dtype=np.int32).reshape(S, N), device=DEV)
    tree = dtv.Tree(S, N, DEV, parent=par, token=tok)
    tree.n_nodes.fill_(N)
    return tree


@pytest.mark.parametrize("shape", ["chain65", "star70", "single", "random1024", "chain130"])
def test_given_tree_mask_edges(shape):
    need_gpu()
    rng = np.random.default_rng(7)
    N = {"chain65": 65, "star70": 70, "single": 1, "random1024": 1024, "chain130": 130}[shape]
    if shape.startswith("chain"):
        parent = [-1] + list(range(N - 1))
    elif shape.startswith("star"):
        parent = [-1] + [0] * (N - 1)
    elif shape == "single":
        parent = [-1]
    else:
        parent = [-1] + [int(rng.integers(max(0, i - 40), i)) for i in range(1, N)]
    token = [-1] + [int(rng.integers(0, 50)) for _ in range(1, N)]
    tree = _given_tree(parent, token, N)
    ws = dtv.Workspace(DEV)
    dtv.tree_build_given(tree, ws)
    g = tree_to_numpy(tree)
    assert_tree_equal(g, 0, obuild.given_tree(parent, token), tree.words)
    assert ws.status("given") == 0


@pytest.mark.parametrize("name,seed", [("c1_tiny", 1), ("c5_batched_llama2_70b", 5)])
def test_given_tree_configs(name, seed):
    need_gpu()
    wl = make_workload(name, seed, P=64, V=64) if name.startswith("c5") else make_workload(name, seed)
    step = DraftTreeStep(wl, DEV) if name.startswith("c1") else None
    cfg = wl.cfg
    tree = _given_tree(wl.parent, wl.token, cfg.N, cfg.S) if step is None else step.tree
    ws = dtv.Workspace(DEV)
    dtv.tree_build_given(tree, ws)
    g = tree_to_numpy(tree)
    for s in range(cfg.S):
        assert_tree_equal(g, s, obuild.given_tree(wl.parent[s], wl.token[s]), tree.words)


TALON_CASES = [
    ("c2_talon_llama3_8b", 2, {}),
    ("c2_talon_llama3_8b", 11, {"V": 5000, "P": 64}),
    ("c2_talon_llama3_8b", 12, {"V": 5000, "P": 64, "alpha": 0.0}),
    ("c2_talon_llama3_8b", 13, {"V": 5000, "P": 64, "alpha": 1.0}),
    ("c2_talon_llama3_8b", 14, {"V": 300, "P": 64, "B": 200, "K": 20, "alpha": 0.05}),
    ("c2_talon_llama3_8b", 15, {"V": 12, "P": 64, "B": 30, "K": 12, "alpha": 0.2}),
    ("c2_talon_llama3_8b", 16, {"V": 9000, "P": 64, "S": 3, "B": 40, "K": 7}),
    ("c2_talon_llama3_8b", 17, {"V": 1000, "P": 64, "dtype": "f32", "B": 16, "K": 4}),
    # no gate and a wide second layer (40 frontier rows of 40, 1600 candidates for 60
    # slots): the radix budget selection past the small-pool path
    ("c2_talon_llama3_8b", 18, {"V": 2000, "P": 64, "B": 100, "K": 40, "alpha": 0.0}),
    # rows of four parts whose lists and records exceed one wave's polled words (4 * (15 + 2)
    # > 64): the part merge by ticket in one wave; and of three parts with 3 * 24 > 64 list
    # entries: the merge by the whole workgroup
    ("c2_talon_llama3_8b", 20, {"P": 64, "B": 40, "K": 15}),
    # two sequences of the full shape: 480 part workgroups, more than the device holds at
    # once, so a row's merging part may poll while later rows' parts still wait for a slot
    ("c2_talon_llama3_8b", 22, {"P": 64, "S": 2}),
    ("c2_talon_llama3_8b", 21, {"V": 70001, "P": 64, "B": 40, "K": 24}),
]


@pytest.mark.parametrize("name,seed,ov", TALON_CASES)
def test_talon_build(name, seed, ov):
    need_gpu()
    wl = make_workload(name, seed, **ov)
    cfg = wl.cfg
    d = to_device(wl.draft, cfg.dtype, DEV)
    tree = dtv.Tree(cfg.S, cfg.N, DEV)
    ws = dtv.Workspace(DEV)
    dtv.tree_build_talon(tree, d, cfg.B, cfg.K, cfg.alpha, ws)
    assert ws.status("talon") == 0
    g = tree_to_numpy(tree)
    for s in range(cfg.S):
        ot = ostep.build_tree(wl, s)
        assert_tree_equal(g, s, ot, tree.words)
        assert int(g["layers"][s]) == ot.layers
    # a second call on the same workspace gives the same tree
    dtv.tree_build_talon(tree, d, cfg.B, cfg.K, cfg.alpha, ws)
    g2 = tree_to_numpy(tree)
    for key in ("parent", "token", "anc"):
        np.testing.assert_array_equal(g[key], g2[key])


@pytest.mark.parametrize("B,kept", [(13, [3, 3, 2, 1]), (20, [4, 4, 4, 4]), (9, [2, 1, 1, 1])])
def test_talon_budget_cut_through_a_tie(B, kept):
    """TALON's budget cut through groups of exactly equal path scores of different parents
    (TALON page, 5.2.1: the cap keeps the best remaining-budget candidates; ties go to the
    lower parent slot, then the lower rank). The root row's four best tokens share one logit
    and their four rows are identical (whose second and third values are also equal), so the
    layer-2 pool of 16 holds a group of four equal scores (rank 0) and one of eight (ranks 1
    and 2); with no gate the cut of B - 4 falls inside a group: B = 13 keeps rank 0 and five
    of the eight, B = 9 one of the eight. The tree is compared with the oracle's, whose
    layer-2 children per parent are checked first so that the cut really splits a group."""
    need_gpu()
    wl = make_workload("c2_talon_llama3_8b", 19, V=5000, P=64, B=B, K=4, alpha=0.0)
    d = wl.draft.copy()
    d[0, 0, 10:14] = 0x41F0   # 30.0, above every other logit of the row
    d[0, 2] = d[0, 1]
    d[0, 3] = d[0, 1]
    d[0, 4] = d[0, 1]
    wl.draft = d
    cfg = wl.cfg
    ot = ostep.build_tree(wl, 0)
    assert ot.token[1:5] == [10, 11, 12, 13]
    assert [sum(1 for p in ot.parent if p == v) for v in range(1, 5)] == kept
    dd = to_device(wl.draft, cfg.dtype, DEV)
    tree = dtv.Tree(cfg.S, cfg.N, DEV)
    ws = dtv.Workspace(DEV)
    dtv.tree_build_talon(tree, dd, cfg.B, cfg.K, cfg.alpha, ws)
    assert ws.status("talon") == 0
    assert_tree_equal(tree_to_numpy(tree), 0, ot, tree.words)


def plant_special_values(wl, seed):
    """Rows of the draft table get values that leave the bf16 row kernel's exp table or stress
    its order keys: +0 and -0, magnitudes below 2^-16 (a subnormal and 2^-17), -inf, values
    <= -256, and exact ties at a row's maximum; one row also holds a value above 256, which
    sends its wave to the exponentials shifted by the maximum."""
    rng = np.random.default_rng(seed)
    d = wl.draft.copy()
    S, R, V = d.shape
    special = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x3700, 0xB700, 0xFF80, 0xC3C0, 0xC400],
                       dtype=np.uint16)
    for s in range(S):
        for r in range(min(R, 12)):
            pos = rng.choice(V, size=min(V, 2 * special.size), replace=False)
            d[s, r, pos] = np.resize(special, pos.size)
        # ties at the maximum of rows 1 and 2
        for r in (1, 2):
            if r < R:
                row = orows.decode(d[s, r], "bf16")
                top = int(np.argmax(row))
                tie = rng.choice(V, size=min(V, 3), replace=False)
                d[s, r, tie] = d[s, r, top]
        if R > 3:
            d[s, 3, rng.integers(V)] = 0x4396   # 300.0
    wl.draft = d
    return wl


@pytest.mark.parametrize("V", [128256, 70001, 32000, 5000])
def test_talon_build_special_values(V):
    """The bf16 row reduction of the TALON build (table of exponentials with its fix-ups,
    packed order keys, padding past the row end, single- and multi-part rows) on rows with
    special values: the tree bit-exact and the scores to 1e-12 against the oracle."""
    need_gpu()
    wl = plant_special_values(make_workload("c2_talon_llama3_8b", 31, V=V, P=64), 31)
    cfg = wl.cfg
    d = to_device(wl.draft, cfg.dtype, DEV)
    tree = dtv.Tree(cfg.S, cfg.N, DEV)
    ws = dtv.Workspace(DEV)
    dtv.tree_build_talon(tree, d, cfg.B, cfg.K, cfg.alpha, ws)
    assert ws.status("talon") == 0
    g = tree_to_numpy(tree)
    for s in range(cfg.S):
        assert_tree_equal(g, s, ostep.build_tree(wl, s), tree.words)


def attn_reference(wl, g):
    """The float64 oracle's outputs of every sequence, all rows (one product per KV head)."""
    cfg = wl.cfg
    refs = []
    for s in range(cfg.S):
        N = int(g["n_nodes"][s])
        q = orows.decode(wl.q[s], cfg.dtype).reshape(wl.q.shape[1:])
        k = orows.decode(wl.k[s], cfg.dtype).reshape(wl.k.shape[1:])
        v = orows.decode(wl.v[s], cfg.dtype).reshape(wl.v.shape[1:])
        refs.append(oattn.tree_attention_dense(q[:N], k, v, int(wl.P[s]), list(g["parent"][s, :N])))
    return refs


def attn_compare(o, refs, tol, label):
    """Every (sequence, node, head) row of the GPU output against the oracle; returns the
    worst absolute error and prints it with the number of rows compared."""
    worst, rows = 0.0, 0
    for s, ref in enumerate(refs):
        N = ref.shape[0]
        err = np.abs(o[s, :N].astype(np.float64) - ref)
        assert np.isfinite(err).all(), (label, s)
        e = float(err.max())
        if e > worst:
            worst = e
        rows += N * ref.shape[1]
    print(f"attention parity {label}: worst max-abs error {worst:.3e} over {rows} rows")
    assert worst <= tol, (label, worst)
    return worst


def _attn_check(wl, tol=2e-2, label=None):
    """Build the tree and run tree attention on the GPU, then compare every output row."""
    cfg = wl.cfg
    step = DraftTreeStep(wl, DEV)
    step.build()
    step.attention()
    torch.cuda.synchronize()
    o = step.o.float().cpu().numpy()
    g = tree_to_numpy(step.tree)
    return attn_compare(o, attn_reference(wl, g), tol, label or cfg.name)


def test_attention_c1_fp32():
    need_gpu()
    _attn_check(make_workload("c1_tiny", 1), tol=1e-4)


def test_attention_c2_full():
    need_gpu()
    _attn_check(make_workload("c2_talon_llama3_8b", 2, V=2000))


@pytest.mark.parametrize("P,B", [(0, 16), (1, 63), (127, 64), (300, 200), (64, 1)])
def test_attention_edges(P, B):
    """Prefix lengths 0/ragged, trees across a mask word boundary and a 128-row tile."""
    need_gpu()
    _attn_check(make_workload("c5_batched_llama2_70b", 21, S=2, P=P, B=B, V=64, max_depth=B))


@pytest.mark.parametrize("name,ov", [
    ("c5_batched_llama2_70b", {"V": 64}),
    ("c5_batched_llama2_70b", {"V": 64, "Hq": 8, "Hkv": 8, "D": 64}),
    # 512 packed rows per KV head at head_dim 64
    ("c5_batched_llama2_70b", {"V": 64, "S": 2, "Hq": 32, "Hkv": 4, "D": 64, "B": 63}),
    # 328 rows = 11 row groups over two tiles (5 + 6): a wave with a single group
    ("c5_batched_llama2_70b", {"V": 64, "S": 3, "P": 1000, "B": 40}),
])
def test_attention_large_full(name, ov):
    """Full-size launches (c5: 8 sequences x 8 KV heads, 17 row groups of 32 per KV head,
    three key splits of the 8257-key cache and their merge): every output row."""
    need_gpu()
    _attn_check(make_workload(name, 5, **ov), label=f"{name} {ov}")


@pytest.mark.parametrize("seed,ov", [
    (6, {"V": 64}),
    (62, {"S": 6, "P": 300, "P_min": 0, "B_min": 0, "V": 64}),
])
def test_attention_ragged_serving(seed, ov):
    """Ragged batch: per-request prefix lengths and tree sizes in one launch (every row)."""
    need_gpu()
    _attn_check(make_workload("c6_ragged_serving", seed, **ov), label=f"c6_ragged_serving {ov}")


def test_attention_ragged_prefix_large():
    """A large launch (8 sequences, 8257-key cache, several key splits) with per-sequence
    prefix lengths that leave a split empty or one or two blocks long, or end one key into a
    block (every row)."""
    need_gpu()
    wl = make_workload("c5_batched_llama2_70b", 23, V=64)
    wl.P = np.array([8192, 0, 1, 4160, 4161, 4100, 8000, 63], dtype=np.int32)
    _attn_check(wl, label="c5 ragged prefixes")


def _upload_oracle_tree(otree, S=1):
    tree = _given_tree(otree.parent, otree.token, otree.N, S)
    ws = dtv.Workspace(DEV)
    dtv.tree_build_given(tree, ws)
    return tree


@pytest.mark.parametrize("name,seed,ov,planted", [
    ("c1_tiny", 1, {}, 0.0), ("c1_tiny", 31, {}, 0.6), ("c1_tiny", 32, {"B": 80, "max_depth": 40}, 0.9),
    ("c3_goose_spine", 3, {"P": 16}, 0.0), ("c3_goose_spine", 33, {"P": 16, "spine_p": 0.95}, 0.0),
])
def test_verify_greedy(name, seed, ov, planted):
    need_gpu()
    wl = make_workload(name, seed, planted=planted, **ov)
    cfg = wl.cfg
    otree = ostep.build_tree(wl, 0)
    tree = _upload_oracle_tree(otree)
    target = to_device(wl.target, cfg.dtype, DEV)
    ws = dtv.Workspace(DEV)
    path, plen, bonus, amax = dtv.tree_verify_greedy(tree, target, ws)
    torch.cuda.synchronize()
    ref = overify.greedy(otree.parent, otree.token, otree.row,
                         lambda r: orows.decode(wl.target[0, r], cfg.dtype))
    A = int(plen[0]) - 1
    assert A == ref["A"]
    assert list(path[0, :A + 1].cpu().numpy()) == ref["path"]
    assert int(bonus[0]) == ref["bonus"]
    np.testing.assert_array_equal(amax[0, :otree.N].cpu().numpy(), np.asarray(ref["argmax"]))
    # second call reuses the workspace
    path2, plen2, bonus2, _ = dtv.tree_verify_greedy(tree, target, ws)
    torch.cuda.synchronize()
    assert int(plen2[0]) == A + 1 and int(bonus2[0]) == ref["bonus"]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_kv_compact(dtype, D):
    need_gpu()
    rng = np.random.default_rng(3)
    S, Hkv, P, N = 3, 4, 50, 70
    P_cap = P + N + 5
    x = rng.standard_normal((S, Hkv, P_cap, D), dtype=np.float32)
    y = rng.standard_normal((S, Hkv, P_cap, D), dtype=np.float32)
    kraw = f32_to_bf16_bits(x) if dtype == "bf16" else x
    vraw = f32_to_bf16_bits(y) if dtype == "bf16" else y
    paths = [[0, 3, 9, 40, 69], [0], [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20,
                                      21, 22, 23, 24, 25, 26, 27, 28, 29, 30, 31, 32, 33, 34, 35, 36]]
    path = np.full((S, N), -1, dtype=np.int32)
    for s, p in enumerate(paths):
        path[s, :len(p)] = p
    k = to_device(kraw, dtype, DEV)
    v = to_device(vraw, dtype, DEV)
    Pd = torch.full((S,), P, dtype=torch.int32, device=DEV)
    P_new = dtv.kv_compact(k, v, Pd, torch.tensor(path, device=DEV),
                           torch.tensor([len(p) for p in paths], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    kk = k.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else k.cpu().numpy()
    vv = v.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else v.cpu().numpy()
    for s, p in enumerate(paths):
        k2, v2, Pn = ocompact.kv_compact(kraw[s], vraw[s], P, p)
        np.testing.assert_array_equal(kk[s], k2)
        np.testing.assert_array_equal(vv[s], v2)
        assert int(P_new[s]) == Pn


@pytest.mark.parametrize("name,seed,ov,planted", [
    ("c1_tiny", 1, {}, 0.5),
    ("c2_talon_llama3_8b", 2, {}, 0.0),
])
def test_step_end_to_end(name, seed, ov, planted):
    need_gpu()
    wl = make_workload(name, seed, planted=planted, **ov)
    cfg = wl.cfg
    step = DraftTreeStep(wl, DEV)
    step.run()
    st = step.ws_status()
    assert all(v == 0 for v in st.values()), st
    res = ostep.run_step(wl, with_attention=False)[0]
    g = tree_to_numpy(step.tree)
    assert_tree_equal(g, 0, res["tree"], step.tree.words)
    path, plen, bonus, _ = [t.cpu() for t in step.verify_out]
    A = int(plen[0]) - 1
    assert A == res["verify"]["A"] and list(path[0, :A + 1].numpy()) == res["verify"]["path"]
    assert int(bonus[0]) == res["verify"]["bonus"]
    assert int(step.P_new[0]) == res["P_new"]
    kk = step.k.view(torch.int16).cpu().numpy().view(np.uint16) if cfg.dtype == "bf16" else step.k.cpu().numpy()
    np.testing.assert_array_equal(kk[0], res["k"])


SPINE_CASES = [
    ("c3_goose_spine", 3, {"P": 16}),
    ("c3_goose_spine", 34, {"P": 16, "V": 700, "spine_p": 0.9}),
    ("c3_goose_spine", 35, {"P": 16, "V": 5000, "n_spine": 10, "n_forks": 11, "fork_width": 9, "S": 2}),
    ("c3_goose_spine", 36, {"P": 16, "V": 900, "dtype": "f32", "n_spine": 5, "n_forks": 3, "fork_width": 2}),
    ("c3_goose_spine", 37, {"P": 16, "V": 64, "n_spine": 70, "n_forks": 71, "fork_width": 1}),
    # widths falling linearly with depth, zero at the deepest forks (the adaptive topology)
    ("c3_goose_spine", 38, {"P": 16, "V": 3000, "n_spine": 12, "n_forks": 12,
                            "spine_widths": (5, 4, 3, 2, 1, 1, 0, 0, 0, 0, 0, 0)}),
    # bf16 fork rows longer than one 32768-value part: the chunk kernel with its merge
    ("c3_goose_spine", 39, {"P": 16, "V": 40000, "n_spine": 6, "n_forks": 7, "fork_width": 3}),
]


@pytest.mark.parametrize("name,seed,ov", SPINE_CASES)
def test_spine_build(name, seed, ov):
    need_gpu()
    wl = make_workload(name, seed, **ov)
    cfg = wl.cfg
    tree = dtv.Tree(cfg.S, cfg.N, DEV)
    ws = dtv.Workspace(DEV)
    dtv.tree_build_spine(tree, torch.from_numpy(wl.spine.astype(np.int32)).to(DEV), wl.widths,
                         to_device(wl.draft, cfg.dtype, DEV), ws)
    assert ws.status("spine") == 0
    g = tree_to_numpy(tree)
    for s in range(cfg.S):
        assert_tree_equal(g, s, ostep.build_tree(wl, s), tree.words)


def _upload_tree_with_rows(otrees, n_cap):
    S = len(otrees)
    par = np.full((S, n_cap), -1, dtype=np.int32)
    tok = np.full((S, n_cap), -1, dtype=np.int32)
    rows = np.zeros((S, n_cap), dtype=np.int32)
    for s, t in enumerate(otrees):
        par[s, :t.N] = t.parent
        tok[s, :t.N] = t.token
        rows[s, :t.N] = t.row
    tree = dtv.Tree(S, n_cap, DEV, parent=torch.from_numpy(par).to(DEV), token=torch.from_numpy(tok).to(DEV))
    tree.n_nodes.copy_(torch.tensor([t.N for t in otrees], dtype=torch.int32))
    ws = dtv.Workspace(DEV)
    dtv.tree_build_given(tree, ws)
    tree.row.copy_(torch.from_numpy(rows))
    torch.cuda.synchronize()
    return tree


SAMPLE_CASES = [
    ("c5_batched_llama2_70b", 5, {"P": 16}),
    ("c5_batched_llama2_70b", 51, {"P": 16, "V": 300, "S": 3}),
    ("c5_batched_llama2_70b", 52, {"P": 16, "V": 64, "S": 4, "B": 40, "max_depth": 1}),   # stars: many rejections
    ("c5_batched_llama2_70b", 53, {"P": 16, "V": 5000, "S": 2, "B": 200, "max_depth": 60}),
    ("c5_batched_llama2_70b", 54, {"P": 16, "V": 1000, "S": 2, "dtype": "f32", "noise_sigma": 0.0}),  # p = q
    ("c1_tiny", 55, {"verify": "sample", "B": 30}),
]


@pytest.mark.parametrize("name,seed,ov", SAMPLE_CASES)
def test_verify_sample(name, seed, ov):
    need_gpu()
    wl = make_workload(name, seed, **ov)
    cfg = wl.cfg
    otrees = [ostep.build_tree(wl, s) for s in range(cfg.S)]
    tree = _upload_tree_with_rows(otrees, cfg.N)
    ws = dtv.Workspace(DEV)
    ua = torch.from_numpy(wl.u_acc.view(np.int32)).to(DEV)
    ur = torch.from_numpy(wl.u_res.view(np.int32)).to(DEV)
    tgt = to_device(wl.target, cfg.dtype, DEV)
    drf = to_device(wl.draft, cfg.dtype, DEV)
    for rep in range(2):   # the workspace is reused by the second call
        path, plen, bonus = dtv.tree_verify_sample(tree, tgt, drf, ua, ur, ws)
        assert ws.status("verify_sample") == 0
        for s in range(cfg.S):
            t = otrees[s]
            ref = overify.sample(t.parent, t.token, t.row, lambda r: orows.decode(wl.target[s, r], cfg.dtype),
                                 lambda r: orows.decode(wl.draft[s, r], cfg.dtype), wl.u_acc[s], wl.u_res[s])
            A = int(plen[s]) - 1
            assert A == ref["A"], (s, A, ref["A"])
            assert list(path[s, :A + 1].cpu().numpy()) == ref["path"]
            assert int(bonus[s]) == ref["bonus"], (s, int(bonus[s]), ref["bonus"])


def test_verify_sample_opt_tree():
    """Rejection sampling on an OPT-Tree-shaped tree (rows keyed by build identity)."""
    need_gpu()
    wl = make_workload("c4_opt_llama2_7b", 4, P=16, V=2000, n=64, max_layers=4)
    cfg = wl.cfg
    ot = ostep.build_tree(wl, 0)
    tree = _upload_tree_with_rows([ot], cfg.N)
    ws = dtv.Workspace(DEV)
    path, plen, bonus = dtv.tree_verify_sample(
        tree, to_device(wl.target, cfg.dtype, DEV), to_device(wl.draft, cfg.dtype, DEV),
        torch.from_numpy(wl.u_acc.view(np.int32)).to(DEV), torch.from_numpy(wl.u_res.view(np.int32)).to(DEV), ws)
    ref = overify.sample(ot.parent, ot.token, ot.row, lambda r: orows.decode(wl.target[0, r], cfg.dtype),
                         lambda r: orows.decode(wl.draft[0, r], cfg.dtype), wl.u_acc[0], wl.u_res[0])
    A = int(plen[0]) - 1
    assert A == ref["A"] and list(path[0, :A + 1].cpu().numpy()) == ref["path"] and int(bonus[0]) == ref["bonus"]


@pytest.mark.parametrize("name,seed,ov", [
    ("c3_goose_spine", 3, {}),
    ("c5_batched_llama2_70b", 5, {}),
    # ragged batches: every request has its own prefix length and tree size
    ("c6_ragged_serving", 6, {}),
    ("c6_ragged_serving", 61, {"S": 5, "P": 700, "P_min": 0, "B_min": 0, "V": 3000}),
])
def test_step_end_to_end_all_sequences(name, seed, ov):
    need_gpu()
    wl = make_workload(name, seed, **ov)
    cfg = wl.cfg
    step = DraftTreeStep(wl, DEV)
    step.run()
    st = step.ws_status()
    assert all(v == 0 for v in st.values()), st
    res = ostep.run_step(wl, with_attention=False)
    g = tree_to_numpy(step.tree)
    path, plen, bonus, _ = [t.cpu() for t in step.verify_out]
    kk = step.k.view(torch.int16).cpu().numpy().view(np.uint16)
    vv = step.v.view(torch.int16).cpu().numpy().view(np.uint16)
    for s in range(cfg.S):
        r = res[s]
        assert_tree_equal(g, s, r["tree"], step.tree.words, check_scores=(cfg.build != "given"))
        A = int(plen[s]) - 1
        assert A == r["verify"]["A"] and list(path[s, :A + 1].numpy()) == r["verify"]["path"]
        assert int(bonus[s]) == r["verify"]["bonus"]
        assert int(step.P_new[s]) == r["P_new"]
        np.testing.assert_array_equal(kk[s], r["k"])
        np.testing.assert_array_equal(vv[s], r["v"])


def test_attention_c3_full():
    need_gpu()
    _attn_check(make_workload("c3_goose_spine", 3, V=64))


OPT_CASES = [
    ("c4_opt_llama2_7b", 4, {"P": 16}),
    ("c4_opt_llama2_7b", 41, {"P": 16, "V": 2000, "n": 64, "max_layers": 5}),
    ("c4_opt_llama2_7b", 42, {"P": 16, "V": 50, "n": 100, "max_layers": 4, "delta": 0.0}),
    ("c4_opt_llama2_7b", 43, {"P": 16, "V": 3, "n": 20, "max_layers": 4, "delta": 0.0}),
    ("c4_opt_llama2_7b", 44, {"P": 16, "V": 3000, "n": 40, "max_layers": 3, "dtype": "f32", "S": 2}),
    ("c4_opt_llama2_7b", 45, {"P": 16, "V": 9000, "n": 200, "max_layers": 6, "delta": 0.05, "draft_sigma": 2.0}),
    # root layer in one launch with fp32 rows, and with heavy bf16 ties at the n-th value
    ("c4_opt_llama2_7b", 46, {"P": 16, "V": 20000, "n": 300, "max_layers": 3, "dtype": "f32"}),
    ("c4_opt_llama2_7b", 47, {"P": 16, "V": 32000, "n": 512, "max_layers": 2, "draft_sigma": 0.05, "S": 2}),
    # bf16 rows of odd length (every other row not 16-byte aligned), root in one workgroup
    ("c4_opt_llama2_7b", 48, {"P": 16, "V": 9001, "n": 300, "max_layers": 3, "S": 2}),
    # one-workgroup root at its limit: exactly n lanes hold values (ceil(V / 8) == n); odd
    # frontier width (the last row pair holds one row)
    ("c4_opt_llama2_7b", 49, {"P": 16, "V": 4000, "n": 500, "max_layers": 3}),
    ("c4_opt_llama2_7b", 50, {"P": 16, "V": 5000, "n": 301, "max_layers": 3, "S": 3}),
    # bf16 frontier rows of two parts: the part merge by ticket
    ("c4_opt_llama2_7b", 51, {"P": 16, "V": 40000, "n": 64, "max_layers": 3}),
]


@pytest.mark.parametrize("name,seed,ov", OPT_CASES)
def test_opt_build(name, seed, ov):
    need_gpu()
    wl = make_workload(name, seed, **ov)
    cfg = wl.cfg
    tree = dtv.Tree(cfg.S, cfg.N, DEV)
    ws = dtv.Workspace(DEV)
    d = to_device(wl.draft, cfg.dtype, DEV)
    for rep in range(2):   # the workspace is reused by the second call
        dtv.tree_build_opt(tree, d, cfg.n, cfg.delta, cfg.max_layers, ws)
        assert ws.status("opt") == 0
        g = tree_to_numpy(tree)
        for s in range(cfg.S):
            ot = ostep.build_tree(wl, s)
            assert_tree_equal(g, s, ot, tree.words)
            assert int(g["layers"][s]) == ot.layers


def test_attention_c4_full():
    """The 512-node OPT-Tree tree (9 mask words, 32 KV heads x 17 row groups): every row."""
    need_gpu()
    _attn_check(make_workload("c4_opt_llama2_7b", 4))


def test_step_end_to_end_c4():
    need_gpu()
    wl = make_workload("c4_opt_llama2_7b", 4)
    step = DraftTreeStep(wl, DEV)
    step.run()
    st = step.ws_status()
    assert all(v == 0 for v in st.values()), st
    r = ostep.run_step(wl, with_attention=False)[0]
    g = tree_to_numpy(step.tree)
    assert_tree_equal(g, 0, r["tree"], step.tree.words)
    path, plen, bonus, _ = [t.cpu() for t in step.verify_out]
    A = int(plen[0]) - 1
    assert A == r["verify"]["A"] and list(path[0, :A + 1].numpy()) == r["verify"]["path"]
    assert int(bonus[0]) == r["verify"]["bonus"]
    assert int(step.P_new[0]) == r["P_new"]
    kk = step.k.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(kk[0], r["k"])


@pytest.mark.parametrize("name,seed,ov", [
    ("c1_tiny", 1, {}),
    ("c2_talon_llama3_8b", 2, {}),
    ("c3_goose_spine", 3, {"P": 64}),
    ("c4_opt_llama2_7b", 4, {"P": 64}),
    ("c5_batched_llama2_70b", 5, {"P": 256}),
])
def test_verify_compact_fused_matches_separate(name, seed, ov):
    """Verification that compacts in the same launch gives exactly the separate launches' path,
    bonus, P_new and cache (the separate compaction is itself checked against the oracle)."""
    need_gpu()
    wl = make_workload(name, seed, **ov)
    sep = DraftTreeStep(wl, DEV, fuse_compact=False)
    sep.run()
    fus = DraftTreeStep(wl, DEV, fuse_compact=True)
    fus.run()
    torch.cuda.synchronize()
    for st in (sep, fus):
        assert all(v == 0 for v in st.ws_status().values())
    for a, b in zip(sep.verify_out[:3], fus.verify_out[:3]):
        assert torch.equal(a, b)
    assert torch.equal(sep.P_new, fus.P_new)
    assert torch.equal(sep.k, fus.k) and torch.equal(sep.v, fus.v)


def test_verify_compact_refuses_overfull_cache():
    """P[s] + n_cap beyond P_cap: P_new[s] = -1 and that sequence's cache rows stay as they were."""
    need_gpu()
    wl = make_workload("c5_batched_llama2_70b", 5, P=256)
    step = DraftTreeStep(wl, DEV)
    step.build()
    step.attention()
    k0, v0 = step.k.clone(), step.v.clone()
    P_bad = step.P.clone()
    P_cap = step.k.shape[2]
    P_bad[1] = P_cap - step.tree.n_cap + 1
    dtv.tree_verify_sample(step.tree, step.target, step.draft, step.u_acc, step.u_res, step.ws,
                           out=step.verify_out, kv=(step.k, step.v, P_bad, step.P_new))
    torch.cuda.synchronize()
    assert int(step.P_new[1]) == -1
    assert torch.equal(step.k[1], k0[1]) and torch.equal(step.v[1], v0[1])
    plen = step.verify_out[1]
    for s in (0, 2):
        assert int(step.P_new[s]) == int(step.P[s]) + int(plen[s])


def test_verify_refuses_rows_and_tokens_outside_the_tables():
    """A node whose row lies past the logit tables (R too small for the tree), or, for
    rejection sampling, a drafted token past the vocabulary, is never read: that sequence
    gets path_len 0 and bonus -1, the workspace reports DTV_EDEVICE, and the other
    sequences still match the oracle. After the tree is repaired the same workspaces give
    the oracle's results again."""
    need_gpu()
    wl = make_workload("c5_batched_llama2_70b", 5, P=16, V=300, S=3)
    cfg = wl.cfg
    otrees = [ostep.build_tree(wl, s) for s in range(cfg.S)]
    tgt = to_device(wl.target, cfg.dtype, DEV)
    drf = to_device(wl.draft, cfg.dtype, DEV)
    ua = torch.from_numpy(wl.u_acc.view(np.int32)).to(DEV)
    ur = torch.from_numpy(wl.u_res.view(np.int32)).to(DEV)
    R = wl.target.shape[1]
    ws = dtv.Workspace(DEV)

    def refs(s):
        t = otrees[s]
        dec_t = lambda r: orows.decode(wl.target[s, r], cfg.dtype)
        dec_d = lambda r: orows.decode(wl.draft[s, r], cfg.dtype)
        return (overify.greedy(t.parent, t.token, t.row, dec_t),
                overify.sample(t.parent, t.token, t.row, dec_t, dec_d, wl.u_acc[s], wl.u_res[s]))

    def check_ok(s, out, ref):
        A = int(out[1][s]) - 1
        assert A == ref["A"] and list(out[0][s, :A + 1].cpu().numpy()) == ref["path"]
        assert int(out[2][s]) == ref["bonus"]

    for bad in ("row", "token"):
        tree = _upload_tree_with_rows(otrees, cfg.N)
        if bad == "row":
            tree.row[1, cfg.N - 1] = R
        else:
            tree.token[1, cfg.N - 1] = cfg.V
        torch.cuda.synchronize()
        outs = {}
        if bad == "row":   # greedy never reads a logit at a drafted token
            outs["verify_greedy"] = dtv.tree_verify_greedy(tree, tgt, ws)
        outs["verify_sample"] = dtv.tree_verify_sample(tree, tgt, drf, ua, ur, ws)
        for key, out in outs.items():
            assert ws.status(key) == -6, key
            assert int(out[1][1]) == 0 and int(out[2][1]) == -1, key
            for s in (0, 2):
                check_ok(s, out, refs(s)[0 if key == "verify_greedy" else 1])
    # repaired: the same workspaces give the oracle's results for every sequence
    tree = _upload_tree_with_rows(otrees, cfg.N)
    g = dtv.tree_verify_greedy(tree, tgt, ws)
    smp = dtv.tree_verify_sample(tree, tgt, drf, ua, ur, ws)
    assert ws.status("verify_greedy") == 0 and ws.status("verify_sample") == 0
    for s in range(cfg.S):
        rg, rs = refs(s)
        check_ok(s, g, rg)
        check_ok(s, smp, rs)


def test_kv_compact_aliased_refusal_keeps_its_mark():
    """dtv_kv_compact with P_new aliasing P: a sequence it refuses (too little cache left)
    keeps P = -1 and its rows; the others move their paths and advance P."""
    need_gpu()
    rng = np.random.default_rng(4)
    S, Hkv, D, N = 3, 2, 128, 20
    P_cap = 100
    x = f32_to_bf16_bits(rng.standard_normal((S, Hkv, P_cap, D), dtype=np.float32))
    y = f32_to_bf16_bits(rng.standard_normal((S, Hkv, P_cap, D), dtype=np.float32))
    k = to_device(x, "bf16", DEV)
    v = to_device(y, "bf16", DEV)
    P0 = [30, P_cap - N + 1, 50]
    paths = [[0, 2, 7], [0, 1], [0, 3, 4, 19]]
    path = np.full((S, N), -1, dtype=np.int32)
    for s, p in enumerate(paths):
        path[s, :len(p)] = p
    P = torch.tensor(P0, dtype=torch.int32, device=DEV)
    dtv.kv_compact(k, v, P, torch.tensor(path, device=DEV),
                   torch.tensor([len(p) for p in paths], dtype=torch.int32, device=DEV), P_new=P)
    torch.cuda.synchronize()
    Ph = P.cpu().tolist()
    assert Ph == [P0[0] + 3, -1, P0[2] + 4]
    kk = k.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(kk[1], x[1])
    for s in (0, 2):
        k2, _, Pn = ocompact.kv_compact(x[s], y[s], P0[s], paths[s])
        np.testing.assert_array_equal(kk[s], k2)
        assert Pn == Ph[s]
