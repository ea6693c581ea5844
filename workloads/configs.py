"""The five synthetic workloads of a draft-tree step, and their generator.

Shapes follow the workloads that the pages evaluate on: a Llama-3-8B attention layer
for the TALON tree (32 query heads, 8 KV heads, head dim 128, vocab 128256), a
Llama-2-7B layer for the OPT-Tree tree, a Llama-2-70B layer batched over 8 sequences,
a GOOSE spine tree, and a tiny fp32 case that a CPU checks in milliseconds.

Row tables. Every logit table is ``[S][R][V]``. A tree node carries a row index into
these tables: for trees numbered by slot (given, TALON, spine) the row of slot i is
row i; for OPT-Tree the row is the node's build identity ``1 + (layer-1)*n + position``
(the root is row 0), so a table generated up front serves any tree the build may pick.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Random-stream identifiers (the second entry of every SeedSequence key).
ST_Q, ST_KPRE, ST_VPRE, ST_KTREE, ST_VTREE = 0, 1, 2, 3, 4
ST_DRAFT, ST_TNOISE, ST_PARENT, ST_TOKEN = 5, 6, 7, 8
ST_UACC, ST_URES, ST_SPINE_COIN, ST_SPINE_SUB = 9, 10, 11, 12
ST_TARGET = 13  # independent target rows
ST_PLANT = 14   # coins of the planted-token variant
ST_RAGGED = 15  # per-request prefix lengths and tree sizes of a ragged batch


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, stream: int, *idx: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(stream), *map(int, idx)]))


def _normal(seed, stream, idx, shape, sigma, dtype):
    """sigma * N(0,1) drawn in float32, stored as float32 or as bf16 bits."""
    x = _rng(seed, stream, *idx).standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)


def _as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(a) if dtype == "bf16" else a.astype(np.float32)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    S: int
    Hq: int
    Hkv: int
    D: int
    dtype: str            # "f32" or "bf16": storage and compute type of logits, Q, K, V
    P: int                # KV prefix length per sequence
    V: int                # vocabulary
    build: str            # "given" | "talon" | "spine" | "opt"
    verify: str           # "greedy" | "sample"
    B: int = 0            # draft-node budget (N = B + 1 with the root in slot 0)
    K: int = 0            # TALON root Top-K and per-node expansion width
    alpha: float = 0.0    # TALON gate
    n: int = 0            # OPT-Tree node budget per layer and for the final tree
    delta: float = 0.0    # OPT-Tree stop threshold on the gain of E[A]
    max_layers: int = 0   # OPT-Tree layer cap
    max_depth: int = 0    # random trees: deepest allowed depth
    n_spine: int = 0      # GOOSE spine length
    fork_width: int = 0   # GOOSE branch width at each fork
    n_forks: int = 0      # forks are slots 0..n_forks-1 (root and the first spine nodes)
    spine_p: float = 0.0  # probability a spine token equals the target argmax
    draft_sigma: float = 0.0
    target_sigma: float = 0.0
    noise_sigma: float = 0.0
    target_from: str = ""  # "draft+noise" | "independent" | "target->draft"
    spine_widths: tuple = ()  # GOOSE: per-fork branch widths (forks 0..len-1), instead of n_forks x fork_width
    P_min: int = -1       # ragged batch (given trees): per-request prefix uniform in [P_min, P]
    B_min: int = -1       # ragged batch (given trees): per-request draft nodes uniform in [B_min, B]

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def N(self) -> int:
        """Node capacity per sequence, root included."""
        if self.build == "spine":
            if self.spine_widths:
                return 1 + self.n_spine + int(sum(self.spine_widths))
            return 1 + self.n_spine + self.n_forks * self.fork_width
        if self.build == "opt":
            return 1 + self.n
        return 1 + self.B

    @property
    def rows(self) -> int:
        """Rows of the draft/target tables per sequence."""
        if self.build == "opt":
            return 1 + self.max_layers * self.n
        return self.N


CONFIGS = {
    "c1_tiny": Config(
        name="c1_tiny", S=1, Hq=4, Hkv=4, D=64, dtype="f32", P=128, V=1000,
        build="given", verify="greedy", B=16, max_depth=6,
        draft_sigma=2.0, target_sigma=2.0, target_from="independent"),
    "c2_talon_llama3_8b": Config(
        name="c2_talon_llama3_8b", S=1, Hq=32, Hkv=8, D=128, dtype="bf16", P=2048, V=128256,
        build="talon", verify="greedy", B=60, K=10, alpha=0.1,
        draft_sigma=3.0, noise_sigma=1.0, target_from="draft+noise"),
    "c3_goose_spine": Config(
        name="c3_goose_spine", S=1, Hq=32, Hkv=8, D=128, dtype="bf16", P=4096, V=32000,
        build="spine", verify="greedy", n_spine=24, fork_width=4, n_forks=24, spine_p=0.6,
        draft_sigma=3.0, noise_sigma=1.0, target_from="draft+noise"),
    "c4_opt_llama2_7b": Config(
        name="c4_opt_llama2_7b", S=1, Hq=32, Hkv=32, D=128, dtype="bf16", P=4096, V=32000,
        build="opt", verify="sample", n=512, delta=0.2, max_layers=6,
        draft_sigma=4.0, noise_sigma=1.0, target_from="draft+noise"),
    "c5_batched_llama2_70b": Config(
        name="c5_batched_llama2_70b", S=8, Hq=64, Hkv=8, D=128, dtype="bf16", P=8192, V=32000,
        build="given", verify="sample", B=64, max_depth=10,
        target_sigma=3.0, noise_sigma=1.5, target_from="target->draft"),
    # large-batch ragged serving: every request has its own prefix length and tree size
    "c6_ragged_serving": Config(
        name="c6_ragged_serving", S=16, Hq=32, Hkv=8, D=128, dtype="bf16", P=4096, V=32000,
        build="given", verify="sample", B=64, max_depth=10, P_min=256, B_min=8,
        target_sigma=3.0, noise_sigma=1.5, target_from="target->draft"),
}

CONFIG_ORDER = ["c1_tiny", "c2_talon_llama3_8b", "c3_goose_spine",
                "c4_opt_llama2_7b", "c5_batched_llama2_70b", "c6_ragged_serving"]


def config_by_name(name: str, **overrides) -> Config:
    return dataclasses.replace(CONFIGS[name], **overrides)


@dataclasses.dataclass
class Workload:
    cfg: Config
    seed: int
    P: np.ndarray            # [S] int32 prefix length per sequence
    P_cap: int               # cache capacity per (seq, kv head)
    q: np.ndarray            # [S][N][Hq][D]  f32 or bf16 bits
    k: np.ndarray            # [S][Hkv][P_cap][D]; tree keys at P+slot
    v: np.ndarray            # [S][Hkv][P_cap][D]
    draft: np.ndarray        # [S][R][V]
    target: np.ndarray       # [S][R][V]
    parent: Optional[np.ndarray] = None   # [S][N] int32 (given trees)
    token: Optional[np.ndarray] = None    # [S][N] int32 (given trees; token[.,0] = -1)
    spine: Optional[np.ndarray] = None    # [S][n_spine] int32
    widths: Optional[np.ndarray] = None   # [n_forks] int32
    u_acc: Optional[np.ndarray] = None    # [S][N] uint32
    u_res: Optional[np.ndarray] = None    # [S][N] uint32
    n_nodes: Optional[np.ndarray] = None  # [S] int32 nodes of each request's tree (None: all N)


def _random_parents(seed, s, N, max_depth):
    """parent[i] uniform over earlier slots j whose depth is below max_depth."""
    rng = _rng(seed, ST_PARENT, s)
    parent = np.full(N, -1, dtype=np.int32)
    dep = np.zeros(N, dtype=np.int64)
    for i in range(1, N):
        allowed = np.nonzero(dep[:i] < max_depth)[0]
        j = int(allowed[rng.integers(0, len(allowed))])
        parent[i] = j
        dep[i] = dep[j] + 1
    return parent


def _gumbel_tokens(seed, s, parent, draft_rows_f32):
    """Draw token[i] ~ softmax(draft row of parent[i]) with the Gumbel-max trick."""
    N = parent.shape[0]
    token = np.full(N, -1, dtype=np.int32)
    for i in range(1, N):
        u = _rng(seed, ST_TOKEN, s, i).random(draft_rows_f32.shape[1])
        u = np.clip(u, 1e-300, 1.0 - 1e-16)
        gumb = -np.log(-np.log(u))
        token[i] = int(np.argmax(draft_rows_f32[parent[i]].astype(np.float64) + gumb))
    return token


def make_workload(cfg: Config | str, seed: int, planted: float = 0.0, **overrides) -> Workload:
    """Generate every input of one step for configuration ``cfg`` and ``seed``.

    ``planted`` (random trees only) replaces each token, with that probability, by the
    argmax of the parent's target row, so that greedy acceptance is not trivially zero.
    """
    if isinstance(cfg, str):
        cfg = config_by_name(cfg, **overrides)
    elif overrides:
        cfg = dataclasses.replace(cfg, **overrides)
    S, N, R, V, D = cfg.S, cfg.N, cfg.rows, cfg.V, cfg.D
    dt = cfg.dtype
    ragged = cfg.P_min >= 0 or cfg.B_min >= 0
    if ragged and cfg.build != "given":
        raise ValueError("ragged batches are defined for given trees")
    if ragged:
        rr = _rng(seed, ST_RAGGED, 0)
        P = rr.integers(max(cfg.P_min, 0), cfg.P + 1, size=S).astype(np.int32)
        n_nodes = 1 + rr.integers(max(cfg.B_min, 0), cfg.B + 1, size=S).astype(np.int32)
    else:
        P = np.full(S, cfg.P, dtype=np.int32)
        n_nodes = None
    P_cap = cfg.P + N
    store = np.uint16 if dt == "bf16" else np.float32

    q = np.stack([_normal(seed, ST_Q, (s,), (N, cfg.Hq, D), 1.0, dt) for s in range(S)])
    k = np.zeros((S, cfg.Hkv, P_cap, D), dtype=store)
    v = np.zeros((S, cfg.Hkv, P_cap, D), dtype=store)
    for s in range(S):
        Ps = int(P[s])   # the tree's keys and values sit at Ps + slot
        for h in range(cfg.Hkv):
            k[s, h, :Ps] = _normal(seed, ST_KPRE, (s, h), (Ps, D), 1.0, dt)
            v[s, h, :Ps] = _normal(seed, ST_VPRE, (s, h), (Ps, D), 1.0, dt)
            k[s, h, Ps:Ps + N] = _normal(seed, ST_KTREE, (s, h), (N, D), 1.0, dt)
            v[s, h, Ps:Ps + N] = _normal(seed, ST_VTREE, (s, h), (N, D), 1.0, dt)

    draft = np.zeros((S, R, V), dtype=store)
    target = np.zeros((S, R, V), dtype=store)
    for s in range(S):
        for r in range(R):
            if cfg.target_from == "target->draft":
                t = _normal(seed, ST_TARGET, (s, r), (V,), cfg.target_sigma, dt)
                target[s, r] = t
                noise = _rng(seed, ST_TNOISE, s, r).standard_normal(V, dtype=np.float32)
                d32 = _as_f32(t, dt) + np.float32(cfg.noise_sigma) * noise
                draft[s, r] = f32_to_bf16_bits(d32) if dt == "bf16" else d32
            else:
                d = _normal(seed, ST_DRAFT, (s, r), (V,), cfg.draft_sigma, dt)
                draft[s, r] = d
                if cfg.target_from == "independent":
                    target[s, r] = _normal(seed, ST_TARGET, (s, r), (V,), cfg.target_sigma, dt)
                else:
                    noise = _rng(seed, ST_TNOISE, s, r).standard_normal(V, dtype=np.float32)
                    t32 = _as_f32(d, dt) + np.float32(cfg.noise_sigma) * noise
                    target[s, r] = f32_to_bf16_bits(t32) if dt == "bf16" else t32

    wl = Workload(cfg=cfg, seed=seed, P=P, P_cap=P_cap, q=q, k=k, v=v, draft=draft, target=target,
                  n_nodes=n_nodes)

    if cfg.build == "given":
        parents, tokens = [], []
        for s in range(S):
            Ns = N if n_nodes is None else int(n_nodes[s])
            par = _random_parents(seed, s, Ns, cfg.max_depth)
            tok = _gumbel_tokens(seed, s, par, _as_f32(draft[s], dt))
            if planted > 0.0:
                coin = _rng(seed, ST_PLANT, s).random(Ns)
                for i in range(1, Ns):
                    if coin[i] < planted:
                        tok[i] = int(np.argmax(_as_f32(target[s, par[i]], dt)))
            # slots past a request's tree are unused (parent -1, token -1)
            parents.append(np.concatenate([par, np.full(N - Ns, -1, dtype=par.dtype)]))
            tokens.append(np.concatenate([tok, np.full(N - Ns, -1, dtype=tok.dtype)]))
        wl.parent = np.stack(parents).astype(np.int32)
        wl.token = np.stack(tokens).astype(np.int32)

    if cfg.build == "spine":
        spines = []
        for s in range(S):
            coin = _rng(seed, ST_SPINE_COIN, s).random(cfg.n_spine)
            sub = _rng(seed, ST_SPINE_SUB, s).integers(0, V - 1, size=cfg.n_spine)
            sp = np.zeros(cfg.n_spine, dtype=np.int32)
            for kk in range(cfg.n_spine):
                # the spine token k is the child of slot k (slot 0 = root)
                best = int(np.argmax(_as_f32(target[s, kk], dt)))
                if coin[kk] < cfg.spine_p:
                    sp[kk] = best
                else:
                    sp[kk] = int(sub[kk]) + (1 if sub[kk] >= best else 0)
            spines.append(sp)
        wl.spine = np.stack(spines)
        if cfg.spine_widths:
            wl.widths = np.asarray(cfg.spine_widths, dtype=np.int32)
        else:
            wl.widths = np.full(cfg.n_forks, cfg.fork_width, dtype=np.int32)

    if cfg.verify == "sample":
        wl.u_acc = np.stack([_rng(seed, ST_UACC, s).integers(0, 2**32, size=N, dtype=np.uint64)
                             .astype(np.uint32) for s in range(S)])
        wl.u_res = np.stack([_rng(seed, ST_URES, s).integers(0, 2**32, size=N, dtype=np.uint64)
                             .astype(np.uint32) for s in range(S)])
    return wl


def step_seed(seed: int, t: int) -> int:
    """Seed of step t of a decoding loop started with ``seed`` (step 0 uses ``seed``)."""
    return seed if t == 0 else seed * 100003 + t


def make_step_inputs(cfg: Config | str, seed: int, t: int, planted: float = 0.0, **overrides) -> Workload:
    """Inputs of step t of a synthetic decoding loop.

    Step 0 is ``make_workload(cfg, seed)``: the prefix and the first tree. A later step's
    cache is the loop's state, so its workload carries no prefix: its k and v hold only that
    step's tree keys and values, at slots 0..N-1, which the loop writes after the current
    prefix. Queries, logits, tree and uniforms are the step's own (seed ``step_seed``).
    """
    if t == 0:
        return make_workload(cfg, seed, planted=planted, **overrides)
    ov = dict(overrides)
    ov["P"] = 0
    ov["P_min"] = -1
    return make_workload(cfg, step_seed(seed, t), planted=planted, **ov)
