"""ctypes binding of libtsv.so (include/tsv.h).

Argument marshalling only: every step of a round runs in the library's HIP
kernels.  Tensors are torch tensors on a ROCm device (torch provides device
memory and the stream); outputs that are not passed in are allocated with
torch.  There is no CPU fallback: without the built library every call
raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtsv.so")

TSV_F32, TSV_BF16 = 0, 1
TSV_OK, TSV_EINVAL, TSV_EUNSUPPORTED, TSV_EWORKSPACE, TSV_EHIP = 0, -1, -2, -3, -4
WS_BUILD, WS_ATTN, WS_WALK, WS_COMMIT, WS_EXPAND = 0, 1, 2, 3, 4


class TsvError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {code} ({status_string(code)})")
        self.code = code


class tsv_cost(ctypes.Structure):
    """C_v(n; l) = a + b n + c n^2 + e l n, and c_d (40 bytes)."""
    _fields_ = [("a", ctypes.c_double), ("b", ctypes.c_double), ("c", ctypes.c_double),
                ("e", ctypes.c_double), ("c_d", ctypes.c_double)]


class tsv_cost_fitted(ctypes.Structure):
    """tsv_cost's fields plus the fitted f l term (48 bytes)."""
    _fields_ = [("a", ctypes.c_double), ("b", ctypes.c_double), ("c", ctypes.c_double),
                ("e", ctypes.c_double), ("c_d", ctypes.c_double), ("f", ctypes.c_double)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_long
_S = ctypes.c_size_t
_F = ctypes.c_float

_SIGS = {
    "build_tree": [_P, _I, _I, _I, _I, _I, ctypes.POINTER(tsv_cost), _P, _I,
                   _P, _P, _P, _P, _P, _P, _P, _S, _P],
    "build_tree_topk": [_P, _I, _I, _I, _I, _I, ctypes.POINTER(tsv_cost), _P, _I,
                        _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P],
    "build_tree_noalloc": [_P, _I, _I, _I, _I, _I, ctypes.POINTER(tsv_cost), _P, _I,
                           _P, _P, _P, _P, _P, _P, _P],
    "build_tree_fitted": [_P, _I, _I, _I, _I, _I, ctypes.POINTER(tsv_cost_fitted), _P, _I,
                          _P, _P, _P, _P, _P, _P, _P, _S, _P],
    "build_tree_expand": [_P, _I, _I, _I, _I, _I, ctypes.POINTER(tsv_cost), _P, _I,
                          _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P],
    "tree_verify_attn": [_P, _P, _P, _P, _P, _L, _P, _P, _P, _I, _I, _I, _I, _I,
                         _I, _I, _I, _F, _P, _P, _P, _S, _P],
    "accept_walk": [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _S, _P],
    "commit_path": [_P, _P, _P, _P, _P, _L, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                    _I, _P, _P],
    "tsv_fit_cost": [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                     ctypes.POINTER(ctypes.c_double), _I, ctypes.c_double,
                     ctypes.POINTER(tsv_cost_fitted)],
    "select_global_budget": [_P, _P, _P, _P, _P, _P, _I, _I, _P, _L, _P],
    "unfold_chains": [_P, _P, _I, _I, _I, _P, _P, _P, _P],
    "compress_chains": [_P, _I, _L, _L, _I, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P],
    "refresh_compressed": [_P, _I, _L, _L, _I, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P,
                           _I, _P, _P, _P],
    "tsv_workspace_size": [_I] * 12,
    "tsv_status_string": [_I],
    "tsv_set_tree_method": [_I],
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libtsv.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m tree_structured_verification_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = _I
        h.tsv_workspace_size.restype = _S
        h.tsv_status_string.restype = ctypes.c_char_p
        _lib = h
    return _lib


def status_string(code: int) -> str:
    return lib().tsv_status_string(int(code)).decode()


def set_tree_method(method: int) -> int:
    """Tree selection of the build_tree family: 0 both methods side by side
    (default), 1 serial pops only, 2 level merge only.  Returns the previous
    setting."""
    r = lib().tsv_set_tree_method(int(method))
    if r < 0:
        raise TsvError("tsv_set_tree_method", r)
    return r


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(fn: str, code: int):
    if code != TSV_OK:
        raise TsvError(fn, code)


def _dev(t: torch.Tensor, what: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    return t


def _rows(t: torch.Tensor, what: str, dtype=None) -> int:
    """A device cache or scratch tensor laid out as row_layout() describes;
    returns its pitch."""
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    return row_layout(t, what)


def row_layout(t: torch.Tensor, what: str = "tensor") -> int:
    """Checks that a cache or scratch tensor [B, R, ...] has its per-row
    block (the trailing dims) dense, rows `pitch` elements apart and batches
    R rows apart (the layout the C ABI's row stride describes); returns the
    pitch."""
    if t.dim() < 3:
        raise ValueError(f"{what} must be [B, rows, ...]")
    width = 1
    for d in range(t.dim() - 1, 1, -1):
        if t.shape[d] > 1 and t.stride(d) != width:
            raise ValueError(f"{what}: the row block must be dense")
        width *= t.shape[d]
    pitch = t.stride(1)
    if pitch < width or (t.shape[0] > 1 and t.stride(0) != t.shape[1] * pitch):
        raise ValueError(f"{what}: rows must be {width} or more elements apart and the "
                         "batches one row count apart")
    return pitch


def kv_row_pitch(width: int, element_size: int) -> int:
    """Elements between token rows for a cache whose rows hold `width`
    elements of `element_size` bytes: the row rounded up to whole 128-byte
    lines, plus one line when that gives an even number of lines.  With an
    even number of lines every row puts a given KV head at the same low
    address bits, and on MI355X the heads at some of those offsets stream
    measurably more slowly (the grouped workload's attention takes about
    10 % longer); an odd number of lines rotates every head over them."""
    lines = -(-int(width) * int(element_size) // 128)
    if lines % 2 == 0:
        lines += 1
    return lines * 128 // int(element_size)


def kv_rows(B: int, R: int, row_shape, dtype: torch.dtype, device, pitch: Optional[int] = None,
            zero: bool = True) -> torch.Tensor:
    """A [B, R, *row_shape] view whose rows are `pitch` elements apart
    (kv_row_pitch by default), for caches and scratch rows."""
    row_shape = tuple(int(x) for x in row_shape)
    width = 1
    for x in row_shape:
        width *= x
    es = torch.empty((), dtype=dtype).element_size()
    pitch = kv_row_pitch(width, es) if pitch is None else int(pitch)
    if pitch < width:
        raise ValueError("pitch smaller than the row")
    alloc = torch.zeros if zero else torch.empty
    base = alloc((B, R, pitch), dtype=dtype, device=device)
    return base[:, :, :width].view((B, R) + row_shape)


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return TSV_F32
    if dt == torch.bfloat16:
        return TSV_BF16
    raise ValueError(f"unsupported dtype {dt}")


def workspace_size(which: int, B=1, gamma=1, V=1, top_k=1, N_max=1, L_cap=0, Hq=1,
                   Hkv=1, d_qk=1, d_v=1, dtype=TSV_BF16) -> int:
    return int(lib().tsv_workspace_size(which, B, gamma, V, top_k, N_max, L_cap, Hq,
                                        Hkv, d_qk, d_v, dtype))


def workspace(nbytes: int, device) -> torch.Tensor:
    """Zero-filled device workspace (tree_verify_attn needs zeros on first use
    and leaves them in place; the other entry points accept any contents)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _cost_struct(cost):
    """The plain 5-field cost of build_tree; a model with a non-zero f term
    belongs to build_tree_fitted."""
    if cost is None:
        return None
    if float(getattr(cost, "f", 0.0)) != 0.0:
        raise ValueError("this cost model has an f*l term: use build_tree_fitted")
    return ctypes.byref(tsv_cost(float(cost.a), float(cost.b), float(cost.c),
                                 float(cost.e), float(cost.c_d)))


def _fitted_struct(cost):
    if cost is None:
        return None
    return ctypes.byref(tsv_cost_fitted(float(cost.a), float(cost.b), float(cost.c),
                                        float(cost.e), float(cost.c_d),
                                        float(getattr(cost, "f", 0.0))))


def _tree_outputs(B: int, N_max: int, dev) -> dict:
    W = (N_max + 31) // 32
    return dict(
        n_nodes=torch.empty(B, dtype=torch.int32, device=dev),
        parent=torch.empty(B, N_max, dtype=torch.int32, device=dev),
        token=torch.empty(B, N_max, dtype=torch.int32, device=dev),
        depth=torch.empty(B, N_max, dtype=torch.int32, device=dev),
        score=torch.empty(B, N_max, dtype=torch.float32, device=dev),
        anc_bits=torch.empty(B, N_max, W, dtype=torch.int32, device=dev),
    )


def _build_common(marginals, top_k, N_max, prefix_len, out, ws):
    _dev(marginals, "marginals", torch.float32)
    B, gamma, V = marginals.shape
    dev = marginals.device
    if out is None:
        out = _tree_outputs(B, N_max, dev)
    if prefix_len is not None:
        _dev(prefix_len, "prefix_len", torch.int32)
    if ws is None:
        ws = workspace(workspace_size(WS_BUILD, B, gamma, V, top_k, N_max), dev)
    return B, gamma, V, dev, out, ws


def _tree_ptrs(out):
    return (_ptr(out["n_nodes"]), _ptr(out["parent"]), _ptr(out["token"]), _ptr(out["depth"]),
            _ptr(out["score"]), _ptr(out["anc_bits"]))


def build_tree(marginals: torch.Tensor, top_k: int, n_budget: int, N_max: int,
               cost=None, prefix_len: Optional[torch.Tensor] = None,
               out: Optional[dict] = None, ws: Optional[torch.Tensor] = None) -> dict:
    """marginals fp32 [B, gamma, V]; cost: object with a, b, c, e, c_d (and
    f == 0 if present) or None for the fixed budget."""
    B, gamma, V, dev, out, ws = _build_common(marginals, top_k, N_max, prefix_len, out, ws)
    code = lib().build_tree(
        _ptr(marginals), B, gamma, V, top_k, n_budget, _cost_struct(cost),
        _ptr(prefix_len), N_max, *_tree_ptrs(out), _ptr(ws), ws.numel(), _stream(dev))
    _check("build_tree", code)
    return out


def build_tree_topk(marginals: torch.Tensor, top_k: int, n_budget: int, N_max: int,
                    cost=None, prefix_len: Optional[torch.Tensor] = None,
                    out: Optional[dict] = None, ws: Optional[torch.Tensor] = None) -> dict:
    """build_tree plus the per-position top-k lists (out["topk_idx"] int32,
    out["topk_p"] fp32, both [B, gamma, top_k])."""
    B, gamma, V, dev, out, ws = _build_common(marginals, top_k, N_max, prefix_len, out, ws)
    if "topk_idx" not in out:
        out["topk_idx"] = torch.empty(B, gamma, top_k, dtype=torch.int32, device=dev)
        out["topk_p"] = torch.empty(B, gamma, top_k, dtype=torch.float32, device=dev)
    code = lib().build_tree_topk(
        _ptr(marginals), B, gamma, V, top_k, n_budget, _cost_struct(cost),
        _ptr(prefix_len), N_max, *_tree_ptrs(out), _ptr(out["topk_idx"]), _ptr(out["topk_p"]),
        _ptr(ws), ws.numel(), _stream(dev))
    _check("build_tree_topk", code)
    return out


def build_tree_noalloc(marginals: torch.Tensor, top_k: int, n_budget: int, N_max: int,
                       cost=None, prefix_len: Optional[torch.Tensor] = None,
                       out: Optional[dict] = None) -> dict:
    """build_tree with the library's own per-device scratch instead of a
    workspace (no device allocation by the library; outputs are still the
    caller's)."""
    _dev(marginals, "marginals", torch.float32)
    B, gamma, V = marginals.shape
    dev = marginals.device
    if out is None:
        out = _tree_outputs(B, N_max, dev)
    if prefix_len is not None:
        _dev(prefix_len, "prefix_len", torch.int32)
    code = lib().build_tree_noalloc(
        _ptr(marginals), B, gamma, V, top_k, n_budget, _cost_struct(cost),
        _ptr(prefix_len), N_max, *_tree_ptrs(out), _stream(dev))
    _check("build_tree_noalloc", code)
    return out


def build_tree_fitted(marginals: torch.Tensor, top_k: int, n_budget: int, N_max: int,
                      cost=None, prefix_len: Optional[torch.Tensor] = None,
                      out: Optional[dict] = None, ws: Optional[torch.Tensor] = None) -> dict:
    """build_tree under the fitted cost family (a, b, c, e, c_d, f)."""
    B, gamma, V, dev, out, ws = _build_common(marginals, top_k, N_max, prefix_len, out, ws)
    code = lib().build_tree_fitted(
        _ptr(marginals), B, gamma, V, top_k, n_budget, _fitted_struct(cost),
        _ptr(prefix_len), N_max, *_tree_ptrs(out), _ptr(ws), ws.numel(), _stream(dev))
    _check("build_tree_fitted", code)
    return out


def expanded_rows(steps: int, top_k: int) -> int:
    """Rows of build_tree_expand's input per request: 1 + k + ... + k^(steps-1)."""
    return sum(top_k ** d for d in range(steps))


def build_tree_expand(probs: torch.Tensor, steps: int, top_k: int, n_budget: int, N_max: int,
                      cost=None, prefix_len: Optional[torch.Tensor] = None,
                      with_topk: bool = False, out: Optional[dict] = None,
                      ws: Optional[torch.Tensor] = None) -> dict:
    """probs fp32 [B, P, V]: the expanded nodes' distributions in level order
    (P = expanded_rows(steps, top_k)); outputs as for build_tree."""
    _dev(probs, "probs", torch.float32)
    B, P, V = probs.shape
    if P != expanded_rows(steps, top_k):
        raise ValueError(f"probs has {P} rows per request, {steps} steps of top-{top_k} "
                         f"need {expanded_rows(steps, top_k)}")
    dev = probs.device
    if out is None:
        out = _tree_outputs(B, N_max, dev)
        if with_topk:
            out["topk_idx"] = torch.empty(B, P, top_k, dtype=torch.int32, device=dev)
            out["topk_p"] = torch.empty(B, P, top_k, dtype=torch.float32, device=dev)
    if prefix_len is not None:
        _dev(prefix_len, "prefix_len", torch.int32)
    if ws is None:
        ws = workspace(workspace_size(WS_EXPAND, B, steps, V, top_k, N_max), dev)
    code = lib().build_tree_expand(
        _ptr(probs), B, steps, V, top_k, n_budget, _cost_struct(cost),
        _ptr(prefix_len), N_max, *_tree_ptrs(out),
        _ptr(out.get("topk_idx")), _ptr(out.get("topk_p")), _ptr(ws), ws.numel(),
        _stream(dev))
    _check("build_tree_expand", code)
    return out


def fit_cost(n, l, t, c_d: float = 0.0) -> tsv_cost_fitted:
    """Non-negative least-squares fit of C_v(n; l) = a + b n + c n^2 + e l n + f l to
    measured latencies t at (n, l) (host sequences); returns the
    tsv_cost_fitted struct (with c_d) for build_tree_fitted's adaptive budget."""
    import numpy as np
    n = np.ascontiguousarray(n, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    t = np.ascontiguousarray(t, dtype=np.float64)
    if not (n.shape == l.shape == t.shape) or n.ndim != 1:
        raise ValueError("n, l and t must be 1-D sequences of one length")
    dp = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    out = tsv_cost_fitted()
    code = lib().tsv_fit_cost(dp(n), dp(l), dp(t), int(n.size), float(c_d), ctypes.byref(out))
    _check("tsv_fit_cost", code)
    return out


def select_global_budget(tree: dict, sps: torch.Tensor) -> dict:
    """Batch-global admission over build_tree's outputs (modified in place):
    tree["n_nodes"] becomes each request's admitted count.  sps: float64
    device tensor, engine steps per second at every batch size."""
    for k in ("n_nodes", "parent", "token", "depth", "score", "anc_bits"):
        _dev(tree[k], k)
    _dev(sps, "sps", torch.float64)
    B, N_max = tree["parent"].shape
    code = lib().select_global_budget(
        _ptr(tree["n_nodes"]), _ptr(tree["parent"]), _ptr(tree["token"]), _ptr(tree["depth"]),
        _ptr(tree["score"]), _ptr(tree["anc_bits"]), B, N_max, _ptr(sps), sps.numel(),
        _stream(tree["n_nodes"].device))
    _check("select_global_budget", code)
    return tree


def unfold_chains(tree: dict, gamma: int) -> dict:
    """Root-to-leaf chains of build_tree's trees: n_chains [B], chain_len
    [B, N_max], chain_nodes [B, N_max, gamma] (int32, device)."""
    n_nodes = _dev(tree["n_nodes"], "n_nodes", torch.int32)
    parent = _dev(tree["parent"], "parent", torch.int32)
    B, N_max = parent.shape
    dev = parent.device
    out = dict(n_chains=torch.empty(B, dtype=torch.int32, device=dev),
               chain_len=torch.empty(B, N_max, dtype=torch.int32, device=dev),
               chain_nodes=torch.empty(B, N_max, gamma, dtype=torch.int32, device=dev))
    code = lib().unfold_chains(_ptr(n_nodes), _ptr(parent), B, N_max, gamma,
                               _ptr(out["n_chains"]), _ptr(out["chain_len"]),
                               _ptr(out["chain_nodes"]), _stream(dev))
    _check("unfold_chains", code)
    return out


def _rows2d(rows: torch.Tensor, E: Optional[int]):
    """Scratch rows [B, N_max, ...] viewed as rows of row_stride elements."""
    _dev(rows, "rows")
    if rows.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("rows must be bfloat16 or float32")
    B, N_max = rows.shape[0], rows.shape[1]
    stride = rows[0, 0].numel()
    return B, N_max, stride, (stride if E is None else int(E))


def compress_chains(rows: torch.Tensor, c: int, tail: torch.Tensor, prefix_len: torch.Tensor,
                    chains: dict, gamma: int, E: Optional[int] = None,
                    entries: Optional[torch.Tensor] = None,
                    n_entries: Optional[torch.Tensor] = None):
    """Every chain's compressed entries (block means of c tokens) from the
    scratch rows [B, N_max, ...] (first E columns of a row, default all),
    the prefix's tail sums fp32 [B, E] and unfold_chains' output.
    Returns (entries fp32 [B, N_max, (c-1+gamma)//c, E], n_entries int32
    [B, N_max])."""
    B, N_max, stride, E = _rows2d(rows, E)
    dev = rows.device
    _dev(tail, "tail", torch.float32)
    _dev(prefix_len, "prefix_len", torch.int32)
    nc = _dev(chains["n_chains"], "n_chains", torch.int32)
    cl = _dev(chains["chain_len"], "chain_len", torch.int32)
    cn = _dev(chains["chain_nodes"], "chain_nodes", torch.int32)
    M = (c - 1 + gamma) // c
    if entries is None:
        entries = torch.zeros(B, N_max, M, E, dtype=torch.float32, device=dev)
    if n_entries is None:
        n_entries = torch.empty(B, N_max, dtype=torch.int32, device=dev)
    code = lib().compress_chains(_ptr(rows), dtype_code(rows.dtype), stride, E, int(c), _ptr(tail),
                                 _ptr(prefix_len), _ptr(nc), _ptr(cl), _ptr(cn), B, N_max, gamma,
                                 _ptr(entries), _ptr(n_entries), _stream(dev))
    _check("compress_chains", code)
    return entries, n_entries


def refresh_compressed(rows: torch.Tensor, c: int, prefix_len: torch.Tensor, walk: dict,
                       chains: dict, entries: torch.Tensor, comp: torch.Tensor,
                       tail: torch.Tensor, gamma: int, E: Optional[int] = None,
                       status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Commit the accepted chain's compressed state into comp fp32 [B, Lc_cap,
    E] and tail fp32 [B, E] (both updated in place); walk is accept_walk's
    output.  Call before commit_path.  Returns status int32 [B]."""
    B, N_max, stride, E = _rows2d(rows, E)
    dev = rows.device
    _dev(prefix_len, "prefix_len", torch.int32)
    al = _dev(walk["accept_len"], "accept_len", torch.int32)
    an = _dev(walk["accept_nodes"], "accept_nodes", torch.int32)
    nc = _dev(chains["n_chains"], "n_chains", torch.int32)
    cl = _dev(chains["chain_len"], "chain_len", torch.int32)
    cn = _dev(chains["chain_nodes"], "chain_nodes", torch.int32)
    _dev(entries, "entries", torch.float32)
    _dev(comp, "comp", torch.float32)
    _dev(tail, "tail", torch.float32)
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=dev)
    code = lib().refresh_compressed(_ptr(rows), dtype_code(rows.dtype), stride, E, int(c),
                                    _ptr(prefix_len), _ptr(al), _ptr(an), _ptr(nc), _ptr(cl),
                                    _ptr(cn), _ptr(entries), B, N_max, gamma, _ptr(comp),
                                    comp.shape[1], _ptr(tail), _ptr(status), _stream(dev))
    _check("refresh_compressed", code)
    return status


def tree_verify_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     k_tree: torch.Tensor, v_tree: torch.Tensor, prefix_len: torch.Tensor,
                     n_nodes: torch.Tensor, anc_bits: torch.Tensor, Hkv: int, d_v: int,
                     sm_scale: float, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                     ws: Optional[torch.Tensor] = None):
    """q [B, N_max, Hq, d_qk]; caches [B, L_cap, ...]; scratch [B, N_max, ...].
    A latent cache passes the same tensor as k_cache and v_cache.
    Returns (out [B, N_max, Hq, d_v], lse fp32 [B, N_max, Hq] or None)."""
    _dev(q, "q")
    pitches = {_rows(t, nm, q.dtype) for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache"),
                                                   (k_tree, "k_tree"), (v_tree, "v_tree"))}
    _dev(prefix_len, "prefix_len", torch.int32)
    _dev(n_nodes, "n_nodes", torch.int32)
    _dev(anc_bits, "anc_bits")
    B, N_max, Hq, d_qk = q.shape
    L_cap = k_cache.shape[1]
    if len(pitches) != 1:
        raise ValueError("caches and scratch must share one row pitch")
    stride = pitches.pop()
    dev = q.device
    if out is None:
        out = torch.empty(B, N_max, Hq, d_v, dtype=q.dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(B, N_max, Hq, dtype=torch.float32, device=dev)
    dt = dtype_code(q.dtype)
    if ws is None:
        ws = workspace(workspace_size(WS_ATTN, B, 1, 1, 1, N_max, L_cap, Hq, Hkv, d_qk,
                                      d_v, dt), dev)
    code = lib().tree_verify_attn(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_tree), _ptr(v_tree), stride,
        _ptr(prefix_len), _ptr(n_nodes), _ptr(anc_bits), B, N_max, L_cap, Hq, Hkv, d_qk,
        d_v, dt, float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(dev))
    _check("tree_verify_attn", code)
    return out, lse


def accept_walk(target_logits: torch.Tensor, n_nodes: torch.Tensor, parent: torch.Tensor,
                token: torch.Tensor, gamma: int, out: Optional[dict] = None,
                ws: Optional[torch.Tensor] = None) -> dict:
    """target_logits [B, 1 + N_max, V] (fp32 or bf16)."""
    _dev(target_logits, "target_logits")
    for t, nm in ((n_nodes, "n_nodes"), (parent, "parent"), (token, "token")):
        _dev(t, nm, torch.int32)
    B, rows, V = target_logits.shape
    N_max = rows - 1
    dev = target_logits.device
    dt = dtype_code(target_logits.dtype)
    if out is None:
        out = dict(accept_len=torch.empty(B, dtype=torch.int32, device=dev),
                   accept_nodes=torch.empty(B, gamma, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty(B, gamma + 1, dtype=torch.int32, device=dev))
    if ws is None:
        ws = workspace(workspace_size(WS_WALK, B, gamma, V, 1, N_max, dtype=dt), dev)
    code = lib().accept_walk(
        _ptr(target_logits), dt, B, N_max, V, gamma, _ptr(n_nodes), _ptr(parent),
        _ptr(token), _ptr(out["accept_len"]), _ptr(out["accept_nodes"]),
        _ptr(out["out_tokens"]), _ptr(ws), ws.numel(), _stream(dev))
    _check("accept_walk", code)
    return out


def commit_path(k_cache: torch.Tensor, v_cache: Optional[torch.Tensor],
                prefix_len: torch.Tensor, k_tree: torch.Tensor,
                v_tree: Optional[torch.Tensor], accept_len: torch.Tensor,
                accept_nodes: torch.Tensor, Hkv: int, d_k: int, d_v: int,
                status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Latent caches pass v_cache = v_tree = None.  Updates k_cache, v_cache
    and prefix_len in place; returns status int32 [B]."""
    pitches = {_rows(k_cache, "k_cache"), _rows(k_tree, "k_tree", k_cache.dtype)}
    _dev(prefix_len, "prefix_len", torch.int32)
    _dev(accept_len, "accept_len", torch.int32)
    _dev(accept_nodes, "accept_nodes", torch.int32)
    if v_cache is not None:
        pitches |= {_rows(v_cache, "v_cache", k_cache.dtype), _rows(v_tree, "v_tree", k_cache.dtype)}
    if len(pitches) != 1:
        raise ValueError("caches and scratch must share one row pitch")
    pitch = pitches.pop()
    B, L_cap = k_cache.shape[:2]
    N_max = k_tree.shape[1]
    gamma = accept_nodes.shape[1]
    dev = k_cache.device
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=dev)
    code = lib().commit_path(
        _ptr(k_cache), _ptr(v_cache), _ptr(prefix_len), _ptr(k_tree), _ptr(v_tree),
        pitch, _ptr(accept_len), _ptr(accept_nodes), B, N_max, L_cap, Hkv,
        d_k, d_v, gamma, dtype_code(k_cache.dtype), _ptr(status), _stream(dev))
    _check("commit_path", code)
    return status
