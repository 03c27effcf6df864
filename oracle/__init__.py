"""ctypes front end of the CPU oracle (oracle/gdn_oracle.c).

TEST INFRASTRUCTURE: only the tests, the smoke check and the bench's CPU
baseline use this package.  The HIP library neither imports nor links it.

All arithmetic happens in the C file, in double precision.  This module only
builds the shared object with gcc (no FMA contraction, no fast-math), passes
arrays, and allocates the fp64 state and tail copies the oracle works on.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

OK, ERR_ARG, ERR_TREE = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    """The loaded oracle.  GDN_ORACLE_LIB names another build of the same source
    (the mutation test points it at copies with planted mistakes)."""
    global _lib
    if _lib is None:
        path = os.environ.get("GDN_ORACLE_LIB", _LIB_PATH)
        if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build()
        L = C.CDLL(path)
        P = C.c_void_p
        I = C.c_int
        L.oracle_bf16_to_f64.argtypes = [C.c_uint16]
        L.oracle_bf16_to_f64.restype = C.c_double
        L.oracle_run.argtypes = [I, I, I, I, I, P, P, P, I, I, P, I, P, P, P, P, I, I]
        L.oracle_recur.argtypes = [I, I, I, I, P, P, P, P, P]
        L.oracle_conv.argtypes = [I, I, P, P, I, I, P, I, P]
        L.oracle_tree_tables.argtypes = [I, P, I, P, P]
        L.oracle_tree_verify.argtypes = [I, I, I, I, I, P, P, P, I, I, P, I, P, I, P, P, P, I, I]
        L.oracle_commit_path.argtypes = [I, I, I, I, I, P, P, P, I, I, P, I, P, I, P, P, I, P, P, I, I]
        L.oracle_run_kda.argtypes = [I, I, I, I, I, P, P, P, I, I, P, I, P, P, P]
        L.oracle_recur_kda.argtypes = [I, I, I, I, P, P, P, P, P]
        for f in ("oracle_run", "oracle_recur", "oracle_conv", "oracle_tree_tables",
                  "oracle_tree_verify", "oracle_commit_path", "oracle_run_kda", "oracle_recur_kda"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _act(arr):
    """(contiguous array, is_bf16) for an activation tensor stored as bf16 bits or float32."""
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return arr, 1
    if arr.dtype == np.float32:
        return arr, 0
    raise TypeError(f"activation storage must be uint16 (bf16 bits) or float32, got {arr.dtype}")


def widen(arr) -> np.ndarray:
    """Activation storage to float64 via the oracle's own widening of each element."""
    arr, is_bf16 = _act(arr)
    if not is_bf16:
        return arr.astype(np.float64)
    f = np.vectorize(lib().oracle_bf16_to_f64, otypes=[np.float64])
    if arr.size <= 65536:
        return f(arr)
    table = f(np.arange(65536, dtype=np.uint16))
    return table[arr]


def f64(arr) -> np.ndarray:
    """A fresh C-contiguous float64 copy of a bf16 (uint16 bits), float32 or float64 array."""
    arr = np.asarray(arr)
    if arr.dtype == np.uint16:
        return np.ascontiguousarray(widen(arr))
    return np.array(arr, dtype=np.float64, order="C", copy=True)


def _check(rc, what):
    if rc != OK:
        raise OracleError(rc, what)


class OracleError(RuntimeError):
    def __init__(self, rc, what):
        super().__init__(f"{what}: oracle status {rc}")
        self.rc = rc


def run(shape, state, tail, w, x, a, b, h_range=None, rows=None, want_o=True):
    """T tokens of one sequence.  state [Hv][dv][dk], tail [C][W] (any float or bf16
    storage), x [T][C], a, b [T][Hv].  Returns (o [T][Hv][dv] or None, S, tail) in fp64.
    rows (int32 [T]) picks the token rows of x/a/b in order (default 0..T-1)."""
    Hk, Hv, dk, dv, W = shape.num_k_heads, shape.num_v_heads, shape.head_k_dim, shape.head_v_dim, shape.conv_width
    S = f64(state)
    t = f64(tail)
    w, wb = _act(w)
    x, xb = _act(x)
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        T = len(rows)
    else:
        T = x.shape[0] if x.ndim == 2 else x.size // shape.conv_channels
    lo, hi = (0, Hv) if h_range is None else h_range
    o = np.zeros((T, Hv, dv), dtype=np.float64) if want_o else None
    rc = lib().oracle_run(Hk, Hv, dk, dv, W, _p(S), _p(t), _p(w), wb, T, _p(x), xb, _p(rows),
                          _p(a), _p(b), _p(o), lo, hi)
    _check(rc, "oracle_run")
    return o, S, t


def run_kda(shape, state, tail, w, x, a, b, want_o=True):
    """T tokens of one sequence with the per-channel forget gate (oracle_run_kda).
    state [Hv][dv][dk], tail [C][W], x [T][C], a [T][Hv][dk], b [T][Hv].
    Returns (o [T][Hv][dv] or None, S, tail) in fp64."""
    Hk, Hv, dk, dv, W = shape.num_k_heads, shape.num_v_heads, shape.head_k_dim, shape.head_v_dim, shape.conv_width
    S = f64(state)
    t = f64(tail)
    w, wb = _act(w)
    x, xb = _act(x)
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    T = x.shape[0] if x.ndim == 2 else x.size // shape.conv_channels
    if a.size != T * Hv * dk or b.size != T * Hv:
        raise ValueError("run_kda: a must be [T][Hv][dk] and b [T][Hv]")
    o = np.zeros((T, Hv, dv), dtype=np.float64) if want_o else None
    rc = lib().oracle_run_kda(Hk, Hv, dk, dv, W, _p(S), _p(t), _p(w), wb, T, _p(x), xb, _p(a), _p(b), _p(o))
    _check(rc, "oracle_run_kda")
    return o, S, t


def run_parallel(shape, state, tail, w, x, a, b, want_o=True, threads=None):
    """run() over all value heads, split by q/k head group over host threads.

    The heads are independent (each keeps its own token order), so every
    thread runs the unchanged oracle on its own head range, into disjoint
    slices of one state and output array; each thread shifts a private copy
    of the tail, which all end equal.  Returns what run() returns."""
    import concurrent.futures as fut
    Hk, Hv, dk, dv, W = shape.num_k_heads, shape.num_v_heads, shape.head_k_dim, shape.head_v_dim, shape.conv_width
    G = Hv // Hk
    S = f64(state)
    t0 = f64(tail)
    w, wb = _act(w)
    x, xb = _act(x)
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    T = x.shape[0] if x.ndim == 2 else x.size // shape.conv_channels
    o = np.zeros((T, Hv, dv), dtype=np.float64) if want_o else None
    n = max(1, min(Hk, threads or os.cpu_count() or 1))
    bounds = [(Hk * i // n * G, Hk * (i + 1) // n * G) for i in range(n)]
    tails = [t0.copy() for _ in bounds]

    def one(i):
        lo, hi = bounds[i]
        return lib().oracle_run(Hk, Hv, dk, dv, W, _p(S), _p(tails[i]), _p(w), wb, T, _p(x), xb, None,
                                _p(a), _p(b), _p(o), lo, hi)

    with fut.ThreadPoolExecutor(max_workers=n) as ex:
        for rc in ex.map(one, range(n)):
            _check(rc, "oracle_run")
    for t in tails[1:]:
        assert np.array_equal(t, tails[0])
    return o, S, tails[0]


def recur(shape, state, y, a, b):
    """One token of the recurrence from a conv output y[C]; returns (o [Hv][dv], S)."""
    Hk, Hv, dk, dv = shape.num_k_heads, shape.num_v_heads, shape.head_k_dim, shape.head_v_dim
    S = f64(state)
    y = np.ascontiguousarray(y, dtype=np.float64)
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    o = np.zeros((Hv, dv), dtype=np.float64)
    _check(lib().oracle_recur(Hk, Hv, dk, dv, _p(S), _p(y), _p(a), _p(b), _p(o)), "oracle_recur")
    return o, S


def recur_kda(shape, state, y, a, b):
    """One token of the per-channel-decay recurrence from a conv output y[C], gate
    inputs a [Hv][dk] and b [Hv]; returns (o [Hv][dv], S)."""
    Hk, Hv, dk, dv = shape.num_k_heads, shape.num_v_heads, shape.head_k_dim, shape.head_v_dim
    S = f64(state)
    y = np.ascontiguousarray(y, dtype=np.float64)
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    if a.size != Hv * dk or b.size != Hv:
        raise ValueError("recur_kda: a must be [Hv][dk] and b [Hv]")
    o = np.zeros((Hv, dv), dtype=np.float64)
    _check(lib().oracle_recur_kda(Hk, Hv, dk, dv, _p(S), _p(y), _p(a), _p(b), _p(o)), "oracle_recur_kda")
    return o, S


def conv(tail, w, x):
    """Conv alone: tail [C][W], w [C][W], x [T][C] -> (y [T][C], tail) in fp64."""
    t = f64(tail)
    Cc, W = t.shape
    w, wb = _act(w)
    x, xb = _act(x)
    T = x.shape[0]
    y = np.zeros((T, Cc), dtype=np.float64)
    _check(lib().oracle_conv(Cc, W, _p(t), _p(w), wb, T, _p(x), xb, _p(y)), "oracle_conv")
    return y, t


def tree_tables(parent, max_depth=8):
    """(status, depth[n], order[n]) of a parent array; status OK or ERR_TREE."""
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    n = len(parent)
    depth = np.zeros(n, dtype=np.int32)
    order = np.zeros(n, dtype=np.int32)
    rc = lib().oracle_tree_tables(n, _p(parent), max_depth, _p(depth), _p(order))
    return rc, depth, order


def tree_verify(shape, state, tail, w, parent, x, a, b, max_depth=8, h_range=None):
    """o [n][Hv][dv] (fp64) at every node of the tree, each from its own path replay."""
    Hk, Hv, dk, dv, W = shape.num_k_heads, shape.num_v_heads, shape.head_k_dim, shape.head_v_dim, shape.conv_width
    S = f64(state)
    t = f64(tail)
    w, wb = _act(w)
    x, xb = _act(x)
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    n = len(parent)
    lo, hi = (0, Hv) if h_range is None else h_range
    o = np.zeros((n, Hv, dv), dtype=np.float64)
    rc = lib().oracle_tree_verify(Hk, Hv, dk, dv, W, _p(S), _p(t), _p(w), wb, n, _p(parent), max_depth,
                                  _p(x), xb, _p(a), _p(b), _p(o), lo, hi)
    _check(rc, "oracle_tree_verify")
    return o


def commit_path(shape, state, tail, w, parent, x, a, b, path, max_depth=8, h_range=None):
    """(o [L][Hv][dv], S, tail) after committing `path` from the checkpoint (fp64 copies)."""
    Hk, Hv, dk, dv, W = shape.num_k_heads, shape.num_v_heads, shape.head_k_dim, shape.head_v_dim, shape.conv_width
    S = f64(state)
    t = f64(tail)
    w, wb = _act(w)
    x, xb = _act(x)
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    path = np.ascontiguousarray(path, dtype=np.int32)
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    L = len(path)
    lo, hi = (0, Hv) if h_range is None else h_range
    o = np.zeros((L, Hv, dv), dtype=np.float64)
    rc = lib().oracle_commit_path(Hk, Hv, dk, dv, W, _p(S), _p(t), _p(w), wb, len(parent), _p(parent),
                                  max_depth, _p(x), xb, _p(a), _p(b), L, _p(path), _p(o), lo, hi)
    _check(rc, "oracle_commit_path")
    return o, S, t
