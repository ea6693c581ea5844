"""The C-ABI library on the CPU: it loads, exports every symbol the header declares,
sizes workspaces, and rejects bad arguments before any launch (no GPU needed)."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import bookkeeping as obook

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dtv.h")


@pytest.fixture(scope="module")
def lib():
    from draft_tree_verification_build_amd import _lib, build_lib
    if not os.path.exists(_lib.LIB_PATH):
        build_lib.build()
    return _lib.load()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dtv_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_symbols()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n


def test_binding_signatures_cover_header(lib):
    from draft_tree_verification_build_amd._lib import SIGNATURES
    assert set(declared_symbols()) == set(SIGNATURES)


def test_status_strings(lib):
    assert lib.dtv_status_str(0) == b"ok"
    assert lib.dtv_status_str(-4) == b"workspace too small"


def test_workspace_queries(lib):
    assert lib.dtv_row_stats_ws_bytes(10, 32000, 512, 1) > 0
    assert lib.dtv_row_stats_ws_bytes(0, 32000, 512, 1) == 0
    assert lib.dtv_tree_build_talon_ws_bytes(1, 60, 10, 128256, 1) > 0
    assert lib.dtv_tree_attn_ws_bytes(1, 61, 32, 8, 128, 2048, 1) > 0
    assert lib.dtv_tree_attn_ws_bytes(1, 61, 32, 7, 128, 2048, 1) == 0   # Hq % Hkv != 0
    assert lib.dtv_tree_verify_greedy_ws_bytes(1, 61, 128256, 1) > 0


def _fake_tree(n_cap=61, words=1):
    from draft_tree_verification_build_amd._lib import DtvTree
    p = 0x1000  # never dereferenced: every call below fails its host-side checks first
    return DtvTree(n_cap, words, p, p, p, p, p, p, p, p)


def test_talon_argument_checks(lib):
    t = _fake_tree()
    ws = ctypes.c_void_p(0x2000)
    call = lambda **kw: lib.dtv_tree_build_talon(
        ctypes.byref(kw.get("tree", t)), kw.get("S", 1), ctypes.c_void_p(0x3000), kw.get("dtype", 1),
        kw.get("R", 61), kw.get("V", 1000), kw.get("B", 60), kw.get("K", 10), kw.get("alpha", 0.1),
        ws, kw.get("ws_bytes", 1 << 30), None)
    assert call(K=65) == -2
    assert call(B=61) == -3                 # B + 1 > n_cap
    assert call(alpha=1.5) == -1
    assert call(R=10) == -1
    assert call(dtype=7) == -2
    assert call(ws_bytes=16) == -4
    assert call(tree=_fake_tree(words=0)) == -3
    assert lib.dtv_tree_build_talon(None, 1, None, 1, 61, 1000, 60, 10, 0.1, None, 0, None) == -1
    assert b"n_cap" in lib.dtv_last_error() or len(lib.dtv_last_error()) > 0


def test_attention_argument_checks(lib):
    t = _fake_tree()
    p = ctypes.c_void_p(0x4000)
    call = lambda **kw: lib.dtv_tree_attn(p, p, p, p, kw.get("P_cap", 2200), kw.get("P_max", 2048),
                                          ctypes.byref(t), 1, kw.get("Hq", 32), kw.get("Hkv", 8),
                                          kw.get("D", 128), kw.get("dtype", 1), kw.get("scale", 0.088),
                                          p, p, kw.get("ws_bytes", 1 << 30), None)
    assert call(Hkv=7) == -1
    assert call(D=96) == -2
    assert call(P_cap=2048) == -3
    assert call(scale=0.0) == -1
    assert call(ws_bytes=64) == -4
    assert call(dtype=0, P_max=20000, P_cap=30000) == -2   # fp32 path limited to 16384 keys


def test_compaction_argument_checks(lib):
    p = ctypes.c_void_p(0x4000)
    assert lib.dtv_kv_compact(p, p, p, p, 100, p, p, 61, 1, 8, 100, 1, None) == -2   # 200-byte rows
    assert lib.dtv_kv_compact(None, p, p, p, 100, p, p, 61, 1, 8, 128, 1, None) == -1


@pytest.mark.parametrize("acc,nd,gamma", [([3, 0, 5], 6, 0.0), ([2, 4], 8, 0.1), ([0] * 5, 0, 0.3),
                                          ([7, 1, 2, 9, 0, 3], 17, 0.02)])
def test_bookkeeping_matches_oracle(lib, acc, nd, gamma):
    from draft_tree_verification_build_amd.api import bookkeeping
    got = bookkeeping(acc, nd, gamma)
    ref = obook.bookkeeping(acc, nd, gamma)
    assert got["E_A"] == ref["E_A"] and got["eta"] == ref["eta"] and got["L"] == ref["L"]
    assert got["speedup"] == pytest.approx(ref["speedup"], rel=1e-15)


def test_bookkeeping_rejects_bad_counts(lib):
    a = np.array([1, -1], dtype=np.int32)
    out = np.zeros(4)
    assert lib.dtv_bookkeeping(a.ctypes.data, 2, 3, 0.1, out.ctypes.data) == -1
    assert lib.dtv_bookkeeping(a.ctypes.data, 0, 3, 0.1, out.ctypes.data) == -1


def test_workspace_refills_when_call_sizes_change():
    """A workspace keeps its per-call state only for calls of the same sizes; the binding
    zero-fills a reused buffer when a call's sizes change (and not otherwise)."""
    import torch
    from draft_tree_verification_build_amd.api import Workspace
    ws = Workspace("cpu")
    b = ws.get("spine", 512, (1, 24, (4, 4)))
    b.fill_(7)
    assert int(ws.get("spine", 512, (1, 24, (4, 4)))[0]) == 7      # same sizes: kept
    assert int(ws.get("spine", 256, (1, 30, (3, 2))).sum()) == 0    # other sizes: zero-filled
    b = ws.get("attn", 512)
    b.fill_(5)
    assert int(ws.get("attn", 512)[0]) == 5                         # no sizes given: kept
    assert isinstance(b, torch.Tensor)


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs the step on one GPU; asked for more it exits with status 2 and says so,
    before touching the GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "4"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _plan(lib, S, n_cap, V, dtype, resident, vec):
    out = np.zeros(7, dtype=np.int64)
    rc = lib.dtv_tree_verify_sample_plan(S, n_cap, V, dtype, resident, vec, out.ctypes.data)
    return rc, out


@pytest.mark.parametrize("S,n_cap,V,dtype,resident,vec", [
    (8, 65, 32000, 1, 256, 1), (1, 513, 32000, 1, 256, 1), (16, 65, 32000, 1, 256, 1),
    (3, 201, 5000, 1, 256, 1), (4, 41, 64, 1, 256, 1), (2, 65, 1000, 0, 256, 1),
    (1, 17, 1000, 0, 256, 1), (8, 65, 32001, 1, 256, 0), (1, 65, 128256, 1, 256, 1),
    (1, 65, 128256, 1, 256, 0), (1, 1024, 4194304, 1, 64, 1), (256, 65, 32000, 1, 256, 1),
    (5, 65, 300, 1, 7, 0), (1, 3, 1, 0, 1, 0),
])
def test_sample_walk_plan_fits_its_buffers(lib, S, n_cap, V, dtype, resident, vec):
    """The walk's division of each vocabulary row over G workgroups stays inside the buffers
    the kernel indexes: G*S workgroups co-resident, slices inside shared memory or inside the
    3*V workspace entries, exchange slots for every rejection plus the bonus draw, and G sums
    plus two values per exchange slot."""
    rc, p = _plan(lib, S, n_cap, V, dtype, resident, vec)
    assert rc == 0, lib.dtv_last_error()
    G, units, su, se, in_lds, xch, pbuf = (int(x) for x in p)
    VEC = 8 if dtype == 1 else 4
    assert 1 <= G <= 32 and G * S <= resident and G + 2 <= 64
    assert units == (V // VEC if vec else V)
    # the kernel's slices [units*gi/G, units*(gi+1)/G): none larger than the plan's
    sizes = [units * (g + 1) // G - units * g // G for g in range(G)]
    assert sum(sizes) == units and max(sizes) <= su
    assert se == su * (VEC if vec else 1)
    assert in_lds == (se <= 4096)
    if not in_lds:
        assert se <= V and pbuf == 3 * V     # entries index the workspace rows, j < V
    # one slot per visited node (at most n_cap), per rejection (at most n_cap - 1) and one
    # for a bonus draw
    assert xch >= 2 * n_cap


@pytest.mark.parametrize("S,n_cap,V,dtype,resident,vec,code", [
    (9, 65, 32000, 1, 8, 1, -2),      # more sequences than co-resident walk workgroups
    (1, 1025, 32000, 1, 256, 1, -2),  # more slots than the walk keeps in shared memory
    (1, 65, 32001, 1, 256, 1, -1),    # 16-byte units need V a multiple of 8 (bf16)
    (1, 65, 1001, 0, 256, 1, -1),     # ... and of 4 (fp32)
    (0, 65, 32000, 1, 256, 1, -1),
    (1, 65, 32000, 5, 256, 1, -1),
])
def test_sample_walk_plan_refusals(lib, S, n_cap, V, dtype, resident, vec, code):
    rc, _ = _plan(lib, S, n_cap, V, dtype, resident, vec)
    assert rc == code, (rc, lib.dtv_last_error())
