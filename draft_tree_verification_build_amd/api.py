"""Python binding of libdtv: argument marshalling only.

Every function takes device tensors (torch is used for device memory and streams) and
forwards raw pointers and sizes to the C entry point of the same name; all computation
happens in the HIP kernels. Errors raise DtvError with the library's message. There is
no CPU fallback: without libdtv.so the first call raises ImportError.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import DtvTree

F32, BF16 = 0, 1


class DtvError(RuntimeError):
    def __init__(self, name: str, code: int):
        lib = _lib.load()
        msg = lib.dtv_last_error().decode() or lib.dtv_status_str(code).decode()
        super().__init__(f"{name} failed ({code}: {lib.dtv_status_str(code).decode()}): {msg}")
        self.code = code


def _call(name: str, *args) -> None:
    lib = _lib.load()
    rc = getattr(lib, name)(*args)
    if rc != 0:
        raise DtvError(name, rc)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libdtv must be contiguous")
    return t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class Workspace:
    """Zero-filled device scratch buffers, one per (purpose, size), kept for reuse."""

    def __init__(self, device):
        self.device = torch.device(device)
        self._bufs: dict = {}
        self._sizes: dict = {}

    def get(self, key, nbytes: int, sizes=None) -> torch.Tensor:
        """The buffer for one kind of call. The library keeps a workspace consistent from
        call to call only while the call's sizes stay the same (the layout of its per-call
        state follows them), so a buffer is zero-filled again when ``sizes`` change."""
        nbytes = max(int(nbytes), 256)
        buf = self._bufs.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
            self._bufs[key] = buf
        elif sizes is not None and self._sizes.get(key) != sizes:
            buf.zero_()
        self._sizes[key] = sizes
        return buf

    def status_words(self) -> dict:
        """Device views of every buffer's status word (the first int32), for a caller that
        reads them together with its own results in one copy instead of one call each."""
        return {k: b[:4].view(torch.int32) for k, b in self._bufs.items()}

    def check(self, stream=None) -> None:
        """Raise DtvError for the first buffer whose device status is an error (the
        buffer is zero-filled again, as its reuse requires)."""
        for k in list(self._bufs):
            rc = self.status(k, stream)
            if rc != 0:
                raise DtvError(f"device status of the {k!r} workspace", rc)

    def status(self, key, stream=None) -> int:
        """Synchronise and return the device status of one workspace; a workspace that
        reports an error is zero-filled again, as the library requires before its reuse."""
        buf = self._bufs[key]
        rc = _lib.load().dtv_ws_status(buf.data_ptr(), _stream(stream))
        if rc != 0:
            buf.zero_()
        return rc


class Tree:
    """Device arrays of S draft trees with n_cap slots each (slot 0 = root)."""

    def __init__(self, S: int, n_cap: int, device, parent: torch.Tensor | None = None,
                 token: torch.Tensor | None = None):
        """``parent``/``token`` ([S][n_cap] int32, device) may be given for trees drafted elsewhere."""
        self.S, self.n_cap = int(S), int(n_cap)
        self.words = (self.n_cap + 63) // 64
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.n_nodes = torch.zeros(S, **i32)
        self.parent = parent if parent is not None else torch.full((S, n_cap), -1, **i32)
        self.token = token if token is not None else torch.full((S, n_cap), -1, **i32)
        for t in (self.parent, self.token):
            if t.shape != (S, n_cap) or t.dtype != torch.int32 or not t.is_contiguous():
                raise ValueError("parent/token must be contiguous int32 [S][n_cap]")
        self.depth = torch.zeros((S, n_cap), **i32)
        self.row = torch.zeros((S, n_cap), **i32)
        self.score = torch.zeros((S, n_cap), dtype=torch.float64, device=dev)
        self.anc = torch.zeros((S, n_cap, self.words), dtype=torch.int64, device=dev)
        self.layers = torch.zeros(S, **i32)
        self._c = DtvTree(self.n_cap, self.words, self.n_nodes.data_ptr(), self.parent.data_ptr(),
                          self.token.data_ptr(), self.depth.data_ptr(), self.row.data_ptr(),
                          self.score.data_ptr(), self.anc.data_ptr(), self.layers.data_ptr())

    @property
    def c(self):
        return ctypes.byref(self._c)


# ----------------------------------------------------------------------------- calls

def row_stats(table: torch.Tensor, K: int, ws: Workspace, row_idx: torch.Tensor | None = None,
              stream=None):
    """Per row of a [R][V] table: (max, argmax, lse, topk[R][K])."""
    V = table.shape[-1]
    R = table.numel() // V if row_idx is None else row_idx.numel()
    dt = _dtype_code(table)
    dev = table.device
    maxv = torch.empty(R, dtype=torch.float32, device=dev)
    amax = torch.empty(R, dtype=torch.int32, device=dev)
    lse = torch.empty(R, dtype=torch.float64, device=dev)
    topk = torch.empty((R, max(K, 1)), dtype=torch.int32, device=dev)
    lib = _lib.load()
    nb = lib.dtv_row_stats_ws_bytes(R, V, K, dt)
    buf = ws.get("row_stats", nb, (R, V, K, dt))
    _call("dtv_row_stats", _ptr(table), dt, R, V, _ptr(row_idx), K, _ptr(maxv), _ptr(amax), _ptr(lse),
          _ptr(topk) if K > 0 else None, buf.data_ptr(), buf.numel(), _stream(stream))
    return maxv, amax, lse, topk[:, :K]


def tree_build_given(tree: Tree, ws: Workspace, stream=None) -> None:
    lib = _lib.load()
    buf = ws.get("given", lib.dtv_tree_build_given_ws_bytes(tree.S), (tree.S, tree.n_cap))
    _call("dtv_tree_build_given", tree.c, tree.S, buf.data_ptr(), buf.numel(), _stream(stream))


def tree_build_talon(tree: Tree, draft: torch.Tensor, B: int, K: int, alpha: float, ws: Workspace,
                     stream=None) -> None:
    """draft: [S][R][V] rows keyed by slot."""
    S, R, V = draft.shape
    dt = _dtype_code(draft)
    lib = _lib.load()
    buf = ws.get("talon", lib.dtv_tree_build_talon_ws_bytes(S, B, K, V, dt), (S, B, K, R, V, dt, tree.n_cap))
    _call("dtv_tree_build_talon", tree.c, S, _ptr(draft), dt, R, V, B, K, float(alpha),
          buf.data_ptr(), buf.numel(), _stream(stream))


def tree_build_spine(tree: Tree, spine: torch.Tensor, widths, draft: torch.Tensor, ws: Workspace,
                     stream=None) -> None:
    """spine [S][n_spine] int32 (device); widths: host ints per fork; draft [S][R][V] keyed by slot."""
    import numpy as np
    S, R, V = draft.shape
    n_spine = spine.shape[1]
    w = np.ascontiguousarray(np.asarray(widths, dtype=np.int32))
    dt = _dtype_code(draft)
    lib = _lib.load()
    buf = ws.get("spine", lib.dtv_tree_build_spine_ws_bytes(S, int(w.size), int(w.max(initial=0)), V, dt),
                 (S, n_spine, tuple(int(x) for x in w), R, V, dt, tree.n_cap))
    _call("dtv_tree_build_spine", tree.c, S, _ptr(spine), n_spine, w.ctypes.data, int(w.size), _ptr(draft), dt,
          R, V, buf.data_ptr(), buf.numel(), _stream(stream))


def tree_build_opt(tree: Tree, draft: torch.Tensor, n: int, delta: float, max_layers: int, ws: Workspace,
                   stream=None) -> None:
    """draft [S][R][V]: row 0 is the root's, row 1+(l-1)*n+p the one of layer l's node p."""
    S, R, V = draft.shape
    dt = _dtype_code(draft)
    lib = _lib.load()
    buf = ws.get("opt", lib.dtv_tree_build_opt_ws_bytes(S, n, V, max_layers, dt), (S, n, R, V, max_layers, dt, tree.n_cap))
    _call("dtv_tree_build_opt", tree.c, S, _ptr(draft), dt, R, V, int(n), float(delta), int(max_layers),
          buf.data_ptr(), buf.numel(), _stream(stream))


BUILD_TALON, BUILD_OPT = 1, 2


def build_params(mode: str, B: int = 0, K: int = 0, alpha: float = 0.0, n: int = 0, delta: float = 0.0,
                 max_layers: int = 0) -> _lib.DtvBuildParams:
    """The parameters of a layered build: mode "talon" (B, K, alpha) or "opt" (n, delta, max_layers)."""
    code = {"talon": BUILD_TALON, "opt": BUILD_OPT}[mode]
    return _lib.DtvBuildParams(code, int(B), int(K), float(alpha), int(n), float(delta), int(max_layers))


def _layered_ws(ws: Workspace, tree: Tree, params, S: int, V: int, dt: int):
    lib = _lib.load()
    nb = lib.dtv_tree_build_layered_ws_bytes(ctypes.byref(params), S, V, dt)
    key = (params.mode, params.B, params.K, params.n, params.max_layers, S, V, dt, tree.n_cap)
    return ws.get("layered", nb, key)


def tree_build_begin(tree: Tree, params, root: torch.Tensor, ws: Workspace, W: torch.Tensor, done: torch.Tensor,
                     stream=None) -> None:
    """Layer 1 of a layered build from each sequence's root row (root [S][V]); writes the next
    frontier's width W [S] and done [S] (int32, device)."""
    S, V = root.shape
    dt = _dtype_code(root)
    buf = _layered_ws(ws, tree, params, S, V, dt)
    _call("dtv_tree_build_begin", tree.c, S, ctypes.byref(params), _ptr(root), dt, V, _ptr(W), _ptr(done),
          buf.data_ptr(), buf.numel(), _stream(stream))


def tree_build_step(tree: Tree, params, layer: int, frontier: torch.Tensor, ws: Workspace, W: torch.Tensor,
                    done: torch.Tensor, stream=None) -> None:
    """Layer `layer` (>= 2) of a layered build from its frontier's rows (frontier [S][W_cap][V])."""
    S, W_cap, V = frontier.shape
    dt = _dtype_code(frontier)
    buf = _layered_ws(ws, tree, params, S, V, dt)
    _call("dtv_tree_build_step", tree.c, S, ctypes.byref(params), int(layer), _ptr(frontier), W_cap, dt, V,
          _ptr(W), _ptr(done), buf.data_ptr(), buf.numel(), _stream(stream))


def tree_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: torch.Tensor, P_max: int,
              tree: Tree, ws: Workspace, scale: float | None = None, o: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """q [S][n_cap][Hq][D]; k, v [S][Hkv][P_cap][D]; P [S] int32 (device)."""
    S, n_cap, Hq, D = q.shape
    Hkv, P_cap = k.shape[1], k.shape[2]
    dt = _dtype_code(q)
    if o is None:
        o = torch.zeros_like(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lib = _lib.load()
    # attention keeps no state between calls (its status word sits first, its partials are
    # rewritten by every call), so its buffer is reused whatever the sizes
    buf = ws.get("attn", lib.dtv_tree_attn_ws_bytes(S, n_cap, Hq, Hkv, D, P_max, dt))
    _call("dtv_tree_attn", _ptr(q), _ptr(k), _ptr(v), _ptr(P), P_cap, int(P_max), tree.c, S, Hq, Hkv,
          D, dt, float(scale), _ptr(o), buf.data_ptr(), buf.numel(), _stream(stream))
    return o


def tree_attn_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: torch.Tensor, P_max: int,
                      tree: Tree, o: torch.Tensor, scale: float | None = None, stream=None) -> torch.Tensor:
    """tree_attn without a workspace (dtv_tree_attn_noalloc): the key-split partials live in
    the library's static per-GPU array; ``o`` must be given (the call allocates nothing)."""
    S, n_cap, Hq, D = q.shape
    Hkv, P_cap = k.shape[1], k.shape[2]
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _call("dtv_tree_attn_noalloc", _ptr(q), _ptr(k), _ptr(v), _ptr(P), P_cap, int(P_max), tree.c, S, Hq, Hkv,
          D, dt, float(scale), _ptr(o), _stream(stream))
    return o


def _kv_cache(kv):
    """(k, v, P, P_new) torch tensors -> the C description of a cache to compact."""
    k, v, P, P_new = kv
    S, Hkv, P_cap, D = k.shape
    if v.shape != k.shape or _dtype_code(v) != _dtype_code(k):
        raise TypeError("k and v must share shape and dtype")
    c = _lib.DtvKvCache(_ptr(k), _ptr(v), _ptr(P), _ptr(P_new), P_cap, Hkv, D)
    return c


def tree_verify_greedy(tree: Tree, target: torch.Tensor, ws: Workspace, out=None, stream=None, kv=None):
    """target [S][R][V]. Returns (path [S][n_cap], path_len [S], bonus [S], argmax [S][n_cap]).

    kv = (k, v, P, P_new): compact that cache along the path in the same launch
    (dtv_tree_verify_greedy_compact); P_new must be its own tensor."""
    S, R, V = target.shape
    dt = _dtype_code(target)
    dev = target.device
    if out is None:
        out = (torch.full((S, tree.n_cap), -1, dtype=torch.int32, device=dev),
               torch.zeros(S, dtype=torch.int32, device=dev),
               torch.zeros(S, dtype=torch.int32, device=dev),
               torch.zeros((S, tree.n_cap), dtype=torch.int32, device=dev))
    path, plen, bonus, amax = out
    lib = _lib.load()
    buf = ws.get("verify_greedy", lib.dtv_tree_verify_greedy_ws_bytes(S, tree.n_cap, V, dt), (S, tree.n_cap, R, V, dt))
    if kv is None:
        _call("dtv_tree_verify_greedy", tree.c, S, _ptr(target), dt, R, V, _ptr(path), _ptr(plen),
              _ptr(bonus), _ptr(amax), buf.data_ptr(), buf.numel(), _stream(stream))
    else:
        c = _kv_cache(kv)
        _call("dtv_tree_verify_greedy_compact", tree.c, S, _ptr(target), dt, R, V, _ptr(path), _ptr(plen),
              _ptr(bonus), _ptr(amax), ctypes.byref(c), buf.data_ptr(), buf.numel(), _stream(stream))
    return out


def tree_verify_sample(tree: Tree, target: torch.Tensor, draft: torch.Tensor, u_acc: torch.Tensor,
                       u_res: torch.Tensor, ws: Workspace, out=None, stream=None, kv=None):
    """target, draft [S][R][V]; u_acc, u_res [S][n_cap] (uint32 bits in an int32 tensor).
    Returns (path [S][n_cap], path_len [S], bonus [S]).

    kv = (k, v, P, P_new): compact that cache along the path in the same launch
    (dtv_tree_verify_sample_compact); P_new must be its own tensor."""
    S, R, V = target.shape
    dt = _dtype_code(target)
    if _dtype_code(draft) != dt:
        raise TypeError("target and draft must share a dtype")
    dev = target.device
    if out is None:
        out = (torch.full((S, tree.n_cap), -1, dtype=torch.int32, device=dev),
               torch.zeros(S, dtype=torch.int32, device=dev),
               torch.zeros(S, dtype=torch.int32, device=dev))
    path, plen, bonus = out[:3]
    lib = _lib.load()
    buf = ws.get("verify_sample", lib.dtv_tree_verify_sample_ws_bytes(S, tree.n_cap, V, dt), (S, tree.n_cap, R, V, dt))
    if kv is None:
        _call("dtv_tree_verify_sample", tree.c, S, _ptr(target), _ptr(draft), dt, R, V, _ptr(u_acc),
              _ptr(u_res), _ptr(path), _ptr(plen), _ptr(bonus), buf.data_ptr(), buf.numel(), _stream(stream))
    else:
        c = _kv_cache(kv)
        _call("dtv_tree_verify_sample_compact", tree.c, S, _ptr(target), _ptr(draft), dt, R, V, _ptr(u_acc),
              _ptr(u_res), _ptr(path), _ptr(plen), _ptr(bonus), ctypes.byref(c), buf.data_ptr(), buf.numel(),
              _stream(stream))
    return out


def kv_compact(k: torch.Tensor, v: torch.Tensor, P: torch.Tensor, path: torch.Tensor,
               path_len: torch.Tensor, P_new: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    S, Hkv, P_cap, D = k.shape
    dt = _dtype_code(k)
    if P_new is None:
        P_new = torch.empty_like(P)
    _call("dtv_kv_compact", _ptr(k), _ptr(v), _ptr(P), _ptr(P_new), P_cap, _ptr(path), _ptr(path_len),
          path.shape[1], S, Hkv, D, dt, _stream(stream))
    return P_new


def kernel_timing(enable: bool, reset: bool = False) -> None:
    """Turn the library's per-launch event timing on or off (optionally dropping the totals)."""
    _call("dtv_kernel_timing", int(bool(enable)), int(bool(reset)))


def kernel_times() -> dict:
    """{kernel name: (total ms, timed launches)} over the launches timed so far."""
    import numpy as np
    lib = _lib.load()
    n = lib.dtv_kernel_times(0, None, 0, None, None)
    if n < 0:
        raise DtvError("dtv_kernel_times", n)
    nb = 96
    names = ctypes.create_string_buffer(max(n, 1) * nb)
    ms = np.zeros(max(n, 1), dtype=np.float64)
    cnt = np.zeros(max(n, 1), dtype=np.int64)
    n = lib.dtv_kernel_times(n, names, nb, ms.ctypes.data, cnt.ctypes.data)
    if n < 0:
        raise DtvError("dtv_kernel_times", n)
    raw = names.raw
    return {raw[i * nb:(i + 1) * nb].split(b"\0", 1)[0].decode(): (float(ms[i]), int(cnt[i])) for i in range(n)}


def bookkeeping(accepted, draft_steps: int, gamma: float) -> dict:
    """Host-side E[A], eta and Speedup from logged counts."""
    import numpy as np
    acc = np.ascontiguousarray(np.asarray(accepted, dtype=np.int32))
    out = np.zeros(4, dtype=np.float64)
    _call("dtv_bookkeeping", acc.ctypes.data, int(acc.size), int(draft_steps), float(gamma), out.ctypes.data)
    return {"E_A": out[0], "eta": out[1], "speedup": out[2], "L": out[3]}
