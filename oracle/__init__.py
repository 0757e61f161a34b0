"""Plain FP64 CPU oracle for the Attention Residuals (AttnRes) read, forward and backward.

TEST INFRASTRUCTURE, not product code. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It shares no code with the GPU library
(``attention_residuals_amd``), and the GPU library never imports it.

The arithmetic lives in ``attnres_oracle.c`` (plain C, double precision): the forward follows the
"Equation" section of the "Fast Attention Residuals" PyPI page in its own notation and order, and
the backward is the reverse-mode derivative of those same steps. ``attnres_oracle_multi.c`` does
the same for the page's multi-query read ("Multi-query AttnRes": M queries, each with its own
routing weights and output). This module only marshals arguments (numpy or CPU torch arrays in,
numpy float64 arrays out) and builds the C files with gcc.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attnres_oracle.c")
_SRCS = [_SRC, os.path.join(_HERE, "attnres_oracle_multi.c")]
_LIB = os.path.join(_HERE, "libattnres_oracle.so")

F32, BF16, F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compiles the oracle with gcc (IEEE double arithmetic: no fast-math) and returns the path."""
    if force or _stale():
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off"] + _SRCS + ["-o", tmp, "-lm"],
            check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _stale() -> bool:
    if not os.path.exists(_LIB):
        return True
    t = os.path.getmtime(_LIB)
    return any(os.path.getmtime(f) > t for f in _SRCS + [os.path.join(_HERE, "attnres_oracle.h")])


class _Problem(ctypes.Structure):
    _fields_ = [
        ("S", ctypes.c_int32), ("D", ctypes.c_int32), ("R", ctypes.c_int32),
        ("N", ctypes.c_int64), ("dtype", ctypes.c_int32), ("out_norm", ctypes.c_int32),
        ("eps", ctypes.c_double), ("scale", ctypes.c_double),
        ("values", ctypes.POINTER(ctypes.c_void_p)), ("query", ctypes.c_void_p),
        ("norm_w", ctypes.c_void_p), ("out_w", ctypes.c_void_p), ("dout", ctypes.c_void_p),
    ]


class _Rows(ctypes.Structure):
    _fields_ = [(name, ctypes.POINTER(ctypes.c_double))
                for name in ("y", "lse", "o_rstd", "p", "score", "dvalues")]


class _MultiProblem(ctypes.Structure):
    _fields_ = [
        ("S", ctypes.c_int32), ("D", ctypes.c_int32), ("R", ctypes.c_int32),
        ("M", ctypes.c_int32), ("N", ctypes.c_int64), ("dtype", ctypes.c_int32),
        ("eps", ctypes.c_double), ("scale", ctypes.c_double),
        ("values", ctypes.POINTER(ctypes.c_void_p)), ("queries", ctypes.c_void_p),
        ("dout", ctypes.c_void_p),
    ]


class _MultiRows(ctypes.Structure):
    _fields_ = [(name, ctypes.POINTER(ctypes.c_double)) for name in ("y", "lse", "dvalues")]


class _SelectedProblem(ctypes.Structure):
    _fields_ = [
        ("S", ctypes.c_int32), ("D", ctypes.c_int32), ("R", ctypes.c_int32),
        ("E", ctypes.c_int32), ("K", ctypes.c_int32), ("N", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("eps", ctypes.c_double), ("scale", ctypes.c_double),
        ("values", ctypes.POINTER(ctypes.c_void_p)), ("bank", ctypes.c_void_p),
        ("ids", ctypes.POINTER(ctypes.c_int64)), ("dout", ctypes.c_void_p),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        # ATTNRES_ORACLE_LIB: a copy of the oracle built elsewhere (the mutation tests build copies
        # with one planted mistake each and check that the pins reject them)
        path = os.environ.get("ATTNRES_ORACLE_LIB")
        if not path:
            if _stale():
                build(force=True)
            path = _LIB
        lib = ctypes.CDLL(path)
        lib.attnres_oracle_run.restype = ctypes.c_int
        lib.attnres_oracle_run.argtypes = [
            ctypes.POINTER(_Problem), ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
            ctypes.POINTER(_Rows), ctypes.POINTER(ctypes.c_double),
            ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), ctypes.c_int]
        lib.attnres_oracle_multi_run.restype = ctypes.c_int
        lib.attnres_oracle_multi_run.argtypes = [
            ctypes.POINTER(_MultiProblem), ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
            ctypes.POINTER(_MultiRows), ctypes.POINTER(ctypes.c_double), ctypes.c_int]
        lib.attnres_oracle_selected_run.restype = ctypes.c_int
        lib.attnres_oracle_selected_run.argtypes = [
            ctypes.POINTER(_SelectedProblem), ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
            ctypes.POINTER(_MultiRows), ctypes.POINTER(ctypes.c_double), ctypes.c_int]
        lib.attnres_oracle_threads.restype = ctypes.c_int
        lib.attnres_oracle_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def _storage(a) -> np.ndarray:
    """numpy view of an input in its storage format (bf16 as its uint16 bit pattern)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                return a.view(torch.int16).numpy().view(np.uint16)
            return a.numpy()
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    return np.ascontiguousarray(a)


def _code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle reads float32, float64 or bfloat16 bits (uint16), not {a.dtype}")


def _dptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def threads_used(threads: int = 0) -> int:
    return int(_load().attnres_oracle_threads(int(threads)))


def run(values, query, norm_w=None, out_w=None, dout=None, *, eps: float = 2.0 ** -23,
        scale: float = 1.0, out_norm: bool = False, tokens: Optional[Sequence[int]] = None,
        want: Sequence[str] = ("y", "lse", "o_rstd", "p", "score", "dvalues"),
        reduce: bool = True, threads: int = 0) -> dict:
    """Evaluates the AttnRes read (and its backward when ``dout`` is given) in FP64.

    values: a [S, N, D] array or a sequence of S [N, D] arrays, float32 / float64 / bf16
    (numpy uint16 bit patterns or torch bfloat16). query [R]; norm_w [R] or None; out_w [D] or
    None; dout [N, D] or None. All arrays share one storage format.
    tokens: None for all N tokens, else the token indices whose rows are wanted.
    want: which per-token arrays to return ("y", "lse", "o_rstd", "p", "score", "dvalues").
    reduce: also return dq (and dw, dow when their weights are present), summed over the
    processed tokens. Returns a dict of float64 numpy arrays; dvalues is [S, T, D].
    """
    lib = _load()
    if isinstance(values, (list, tuple)):
        vals = [_storage(v) for v in values]
    else:
        v3 = _storage(values)
        if v3.ndim != 3:
            raise ValueError("packed values must be [S, N, D]")
        vals = [v3[s] for s in range(v3.shape[0])]
    S = len(vals)
    if S < 1:
        raise ValueError("need at least one source")
    N, D = vals[0].shape
    q = _storage(query).reshape(-1)
    R = q.shape[0]
    code = _code(vals[0])
    arrays = list(vals) + [q]
    w = None if norm_w is None else _storage(norm_w).reshape(-1)
    ow = None if out_w is None else _storage(out_w).reshape(-1)
    g = None if dout is None else _storage(dout).reshape(N, D)
    for a in arrays + [x for x in (w, ow, g) if x is not None]:
        if _code(a) != code:
            raise TypeError("all oracle inputs must share one storage format")
    for v in vals:
        if v.shape != (N, D):
            raise ValueError("every source must be [N, D]")
    vals = [np.ascontiguousarray(v) for v in vals]

    ptrs = (ctypes.c_void_p * S)(*[v.ctypes.data for v in vals])
    prob = _Problem(S=S, D=D, R=R, N=N, dtype=code, out_norm=int(bool(out_norm)),
                    eps=float(eps), scale=float(scale),
                    values=ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)),
                    query=q.ctypes.data,
                    norm_w=None if w is None else w.ctypes.data,
                    out_w=None if ow is None else ow.ctypes.data,
                    dout=None if g is None else g.ctypes.data)

    tok = None
    T = N
    if tokens is not None:
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        T = tok.shape[0]

    out = {}
    shapes = {"y": (T, D), "lse": (T,), "o_rstd": (T,), "p": (T, S), "score": (T, S),
              "dvalues": (S, T, D)}
    for name in want:
        if name == "dvalues" and g is None:
            continue
        if name == "o_rstd" and not out_norm:
            continue
        out[name] = np.zeros(shapes[name], dtype=np.float64)
    rows = _Rows(**{k: _dptr(out.get(k)) for k in shapes})

    dq = dw = dow = None
    if reduce and g is not None:
        dq = np.zeros(R, dtype=np.float64)
        if w is not None:
            dw = np.zeros(R, dtype=np.float64)
        if ow is not None and out_norm:
            dow = np.zeros(D, dtype=np.float64)

    rc = lib.attnres_oracle_run(
        ctypes.byref(prob),
        None if tok is None else tok.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        T, ctypes.byref(rows), _dptr(dq), _dptr(dw), _dptr(dow), int(threads))
    if rc != 0:
        raise RuntimeError(f"attnres_oracle_run failed with code {rc}")
    if dq is not None:
        out["dq"] = dq
    if dw is not None:
        out["dw"] = dw
    if dow is not None:
        out["dow"] = dow
    return out


def _sources(values):
    if isinstance(values, (list, tuple)):
        vals = [_storage(v) for v in values]
    else:
        v3 = _storage(values)
        if v3.ndim != 3:
            raise ValueError("packed values must be [S, N, D]")
        vals = [v3[s] for s in range(v3.shape[0])]
    if not vals:
        raise ValueError("need at least one source")
    return [np.ascontiguousarray(v) for v in vals]


def run_multi(values, queries, dout=None, *, eps: float = 2.0 ** -23, scale: float = 1.0,
              tokens: Optional[Sequence[int]] = None, want: Sequence[str] = ("y", "lse", "dvalues"),
              reduce: bool = True, threads: int = 0) -> dict:
    """Evaluates the multi-query AttnRes read (and its backward when ``dout`` is given) in FP64.

    values: [S, N, D] or S arrays [N, D]; queries [M, R]; dout [M, N, D] (query-major) or None;
    one storage format for all. tokens / want / reduce as in ``run``. Returns float64 arrays:
    y [M, T, D], lse [M, T], dvalues [S, T, D] (summed over the queries), dq [M, R].
    """
    lib = _load()
    vals = _sources(values)
    S = len(vals)
    N, D = vals[0].shape
    q = _storage(queries)
    if q.ndim != 2:
        raise ValueError("queries must be [M, R]")
    q = np.ascontiguousarray(q)
    M, R = q.shape
    code = _code(vals[0])
    g = None if dout is None else np.ascontiguousarray(_storage(dout).reshape(M, N, D))
    for a in vals + [q] + ([g] if g is not None else []):
        if _code(a) != code:
            raise TypeError("all oracle inputs must share one storage format")
    for v in vals:
        if v.shape != (N, D):
            raise ValueError("every source must be [N, D]")
    ptrs = (ctypes.c_void_p * S)(*[v.ctypes.data for v in vals])
    prob = _MultiProblem(S=S, D=D, R=R, M=M, N=N, dtype=code, eps=float(eps), scale=float(scale),
                         values=ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)),
                         queries=q.ctypes.data, dout=None if g is None else g.ctypes.data)
    tok = None
    T = N
    if tokens is not None:
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        T = tok.shape[0]
    out = {}
    shapes = {"y": (M, T, D), "lse": (M, T), "dvalues": (S, T, D)}
    for name in want:
        if name == "dvalues" and g is None:
            continue
        out[name] = np.zeros(shapes[name], dtype=np.float64)
    rows = _MultiRows(**{k: _dptr(out.get(k)) for k in shapes})
    dq = np.zeros((M, R), dtype=np.float64) if (reduce and g is not None) else None
    rc = lib.attnres_oracle_multi_run(
        ctypes.byref(prob),
        None if tok is None else tok.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        T, ctypes.byref(rows), _dptr(dq), int(threads))
    if rc != 0:
        raise RuntimeError(f"attnres_oracle_multi_run failed with code {rc}")
    if dq is not None:
        out["dq"] = dq
    return out


def run_selected(values, bank, ids, dout=None, *, eps: float = 2.0 ** -23, scale: float = 1.0,
                 tokens: Optional[Sequence[int]] = None,
                 want: Sequence[str] = ("y", "lse", "dvalues"), reduce: bool = True,
                 threads: int = 0) -> dict:
    """Evaluates the selected-query AttnRes read in FP64: token n reads with the K queries
    bank[ids[n, k]]. values: [S, N, D] or S arrays [N, D]; bank [E, R]; ids [N, K] integers;
    dout [N, K, D] or None. Returns y [T, K, D], lse [T, K], dvalues [S, T, D] and, with
    reduce, dbank [E, R]."""
    lib = _load()
    vals = _sources(values)
    S = len(vals)
    N, D = vals[0].shape
    b = np.ascontiguousarray(_storage(bank))
    if b.ndim != 2:
        raise ValueError("bank must be [E, R]")
    E, R = b.shape
    try:
        import torch
        if isinstance(ids, torch.Tensor):
            ids = ids.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    idx = np.ascontiguousarray(np.asarray(ids, dtype=np.int64).reshape(N, -1))
    K = idx.shape[1]
    code = _code(vals[0])
    g = None if dout is None else np.ascontiguousarray(_storage(dout).reshape(N, K, D))
    for a in vals + [b] + ([g] if g is not None else []):
        if _code(a) != code:
            raise TypeError("all oracle inputs must share one storage format")
    ptrs = (ctypes.c_void_p * S)(*[v.ctypes.data for v in vals])
    prob = _SelectedProblem(S=S, D=D, R=R, E=E, K=K, N=N, dtype=code, eps=float(eps),
                            scale=float(scale),
                            values=ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)),
                            bank=b.ctypes.data,
                            ids=idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                            dout=None if g is None else g.ctypes.data)
    tok = None
    T = N
    if tokens is not None:
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        T = tok.shape[0]
    out = {}
    shapes = {"y": (T, K, D), "lse": (T, K), "dvalues": (S, T, D)}
    for name in want:
        if name == "dvalues" and g is None:
            continue
        out[name] = np.zeros(shapes[name], dtype=np.float64)
    rows = _MultiRows(**{k: _dptr(out.get(k)) for k in shapes})
    dbank = np.zeros((E, R), dtype=np.float64) if (reduce and g is not None) else None
    rc = lib.attnres_oracle_selected_run(
        ctypes.byref(prob),
        None if tok is None else tok.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        T, ctypes.byref(rows), _dptr(dbank), int(threads))
    if rc != 0:
        raise RuntimeError(f"attnres_oracle_selected_run failed with code {rc}")
    if dbank is not None:
        out["dbank"] = dbank
    return out
