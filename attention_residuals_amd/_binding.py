"""ctypes binding of ``libattnres.so`` (the C ABI declared in ``include/attnres.h``).

Argument marshalling only: torch tensors are turned into device pointers, strides and a
descriptor; every step of the computation runs in the library's HIP kernels. There is no
fallback: if the library is missing or a call fails, this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Union

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# ATTNRES_LIB names another build of the same library (the host-side AddressSanitizer build of the
# argument checks, attention_residuals_amd/build_asan.py); by default the in-tree libattnres.so.
LIB_PATH = os.environ.get("ATTNRES_LIB") or os.path.join(_PKG, "libattnres.so")

ATTNRES_F32, ATTNRES_BF16 = 0, 1
EPS_DEFAULT = 2.0 ** -23

# Every function the header declares, with its ctypes signature.
EXPORTS = ("attnres_o32_elems", "attnres_workspace_bytes", "attnres_fwd_workspace_bytes",
           "attnres_fwd", "attnres_bwd", "attnres_bwd_noalloc",
           "attnres_multi_fwd_workspace_bytes",
           "attnres_multi_workspace_bytes", "attnres_multi_fwd", "attnres_multi_bwd",
           "attnres_selected_fwd_workspace_bytes", "attnres_selected_workspace_bytes",
           "attnres_selected_fwd", "attnres_selected_bwd", "attnres_selected_ids_flag",
           "attnres_stream_probe", "attnres_status_str", "attnres_last_error")

QUERY_MAJOR, TOKEN_MAJOR = 0, 1
LAYOUTS = {"query_major": QUERY_MAJOR, "token_major": TOKEN_MAJOR}


class Desc(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int32), ("D", ctypes.c_int32), ("R", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("N", ctypes.c_int64), ("eps", ctypes.c_float),
                ("scale", ctypes.c_float), ("has_norm_weight", ctypes.c_int32),
                ("out_norm", ctypes.c_int32), ("has_out_weight", ctypes.c_int32),
                ("deterministic", ctypes.c_int32), ("accumulate_dvalues", ctypes.c_int32)]


class MultiDesc(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int32), ("D", ctypes.c_int32), ("R", ctypes.c_int32),
                ("M", ctypes.c_int32), ("dtype", ctypes.c_int32), ("N", ctypes.c_int64),
                ("eps", ctypes.c_float), ("scale", ctypes.c_float), ("layout", ctypes.c_int32),
                ("deterministic", ctypes.c_int32), ("accumulate_dvalues", ctypes.c_int32)]


class SelectedDesc(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int32), ("D", ctypes.c_int32), ("R", ctypes.c_int32),
                ("E", ctypes.c_int32), ("K", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("N", ctypes.c_int64), ("eps", ctypes.c_float), ("scale", ctypes.c_float),
                ("deterministic", ctypes.c_int32), ("accumulate_dvalues", ctypes.c_int32)]


class Sources(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("src_stride", ctypes.c_int64),
                ("list", ctypes.POINTER(ctypes.c_void_p)), ("row_stride", ctypes.c_int64)]


class AttnResError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"attnres status {status}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def load() -> ctypes.CDLL:
    """Loads the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m attention_residuals_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64
    pd, ps = ctypes.POINTER(Desc), ctypes.POINTER(Sources)
    lib.attnres_o32_elems.argtypes = [pd, ctypes.POINTER(sz)]
    lib.attnres_workspace_bytes.argtypes = [pd, ctypes.POINTER(sz)]
    lib.attnres_fwd_workspace_bytes.argtypes = [pd, ctypes.POINTER(sz)]
    lib.attnres_fwd.argtypes = [pd, ps, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.attnres_bwd.argtypes = [pd, ps, vp, vp, vp, vp, vp, vp, vp, i64, ps, vp, vp, vp, vp, sz, vp]
    lib.attnres_bwd_noalloc.argtypes = [pd, ps, vp, vp, vp, vp, vp, vp, vp, i64, ps, vp, vp, vp, vp]
    pm = ctypes.POINTER(MultiDesc)
    lib.attnres_multi_fwd_workspace_bytes.argtypes = [pm, ctypes.POINTER(sz)]
    lib.attnres_multi_workspace_bytes.argtypes = [pm, ctypes.POINTER(sz)]
    lib.attnres_multi_fwd.argtypes = [pm, ps, vp, vp, vp, vp, sz, vp]
    lib.attnres_multi_bwd.argtypes = [pm, ps, vp, vp, vp, ps, vp, vp, sz, vp]
    pe = ctypes.POINTER(SelectedDesc)
    lib.attnres_selected_fwd_workspace_bytes.argtypes = [pe, ctypes.POINTER(sz)]
    lib.attnres_selected_workspace_bytes.argtypes = [pe, ctypes.POINTER(sz)]
    lib.attnres_selected_fwd.argtypes = [pe, ps, vp, vp, vp, vp, vp, sz, vp]
    lib.attnres_selected_bwd.argtypes = [pe, ps, vp, vp, vp, vp, ps, vp, vp, sz, vp]
    lib.attnres_selected_ids_flag.argtypes = [vp, sz, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                              vp]
    lib.attnres_stream_probe.argtypes = [ctypes.POINTER(vp), ctypes.c_int32, ctypes.POINTER(vp),
                                         ctypes.c_int32, i64, i64, ctypes.c_int32, ctypes.c_int32,
                                         vp]
    for f in EXPORTS:
        if f not in ("attnres_status_str", "attnres_last_error"):
            getattr(lib, f).restype = ctypes.c_int
    lib.attnres_status_str.argtypes = [ctypes.c_int]
    lib.attnres_status_str.restype = ctypes.c_char_p
    lib.attnres_last_error.argtypes = []
    lib.attnres_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        lib = load()
        detail = lib.attnres_last_error().decode() or lib.attnres_status_str(status).decode()
        raise AttnResError(status, detail)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return ATTNRES_BF16
    if dt == torch.float32:
        return ATTNRES_F32
    raise TypeError(f"AttnRes supports bfloat16 and float32 storage, not {dt}")


def make_desc(S: int, N: int, D: int, R: int, dtype: torch.dtype, *, eps: float = EPS_DEFAULT,
              scale: float = 1.0, has_norm_weight: bool = False, out_norm: bool = False,
              has_out_weight: bool = False, deterministic: bool = False,
              accumulate_dvalues: bool = False) -> Desc:
    return Desc(S=S, D=D, R=R, dtype=_dtype_code(dtype), N=N, eps=eps, scale=scale,
                has_norm_weight=int(has_norm_weight), out_norm=int(out_norm),
                has_out_weight=int(has_out_weight), deterministic=int(deterministic),
                accumulate_dvalues=int(accumulate_dvalues))


class _SourceView:
    """Sources struct for a packed [S, N, D] tensor or a list of [N, D] tensors (kept alive)."""

    def __init__(self, values: Union[torch.Tensor, Sequence[torch.Tensor]]):
        if isinstance(values, torch.Tensor):
            if values.dim() != 3 or values.stride(2) != 1:
                raise ValueError("packed values must be [S, N, D] with unit stride in D")
            self.S, self.N, self.D = values.shape
            self.dtype, self.device = values.dtype, values.device
            self.keep = [values]
            self.ptrs = None
            self.struct = Sources(packed=values.data_ptr(), src_stride=values.stride(0),
                                  list=None, row_stride=values.stride(1))
        else:
            vs = list(values)
            if not vs:
                raise ValueError("need at least one source")
            self.S = len(vs)
            self.N, self.D = vs[0].shape
            self.dtype, self.device = vs[0].dtype, vs[0].device
            rs = vs[0].stride(0)
            for v in vs:
                if v.dim() != 2 or tuple(v.shape) != (self.N, self.D) or v.stride(1) != 1:
                    raise ValueError("every source must be [N, D] with unit stride in D")
                if v.dtype != self.dtype or v.device != self.device:
                    raise ValueError("sources must share dtype and device")
                if v.stride(0) != rs and self.N > 1:
                    raise ValueError("sources must share one row stride")
            self.keep = vs
            self.ptrs = (ctypes.c_void_p * self.S)(*[v.data_ptr() for v in vs])
            self.struct = Sources(packed=None, src_stride=0,
                                  list=ctypes.cast(self.ptrs, ctypes.POINTER(ctypes.c_void_p)),
                                  row_stride=rs if self.N > 1 else self.D)


def o32_elems(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    _check(load().attnres_o32_elems(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def workspace_bytes(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    _check(load().attnres_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def fwd_workspace_bytes(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    _check(load().attnres_fwd_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _scratch(nbytes: int, device, stream, zero: bool = False) -> torch.Tensor:
    """A workspace the binding allocates itself (the caller gave none). It is freed when the
    binding drops it, which torch's caching allocator orders after the work queued so far on the
    CURRENT stream only; when the call runs on another stream, the tensor is recorded on that
    stream too, so its memory is not handed out again before the call's kernels finish. `zero`:
    counters that must be zero at launch (the single-query read's workspaces)."""
    t = (torch.zeros if zero else torch.empty)((nbytes,), dtype=torch.uint8, device=device)
    if stream is not None:
        ts = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(
            stream, device=t.device)
        if ts != torch.cuda.current_stream(t.device):
            t.record_stream(ts)
    return t


def _prep_fwd(values, query: torch.Tensor, norm_w: Optional[torch.Tensor] = None,
                out_w: Optional[torch.Tensor] = None, *, eps: float = EPS_DEFAULT,
                scale: float = 1.0, out_norm: bool = False,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                out_rstd: Optional[torch.Tensor] = None, o32: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, dynamic: bool = True, stream=None):
    """Marshals a forward call: (C function, its arguments, outputs, objects to keep alive)."""
    sv = _SourceView(values)
    desc = make_desc(sv.S, sv.N, sv.D, query.numel(), sv.dtype, eps=eps, scale=scale,
                     has_norm_weight=norm_w is not None, out_norm=out_norm,
                     has_out_weight=out_w is not None)
    dev = sv.device
    if out is None:
        out = torch.empty((sv.N, sv.D), dtype=sv.dtype, device=dev)
    if lse is None:
        lse = torch.empty((sv.N,), dtype=torch.float32, device=dev)
    if out_norm and out_rstd is None:
        out_rstd = torch.empty((sv.N,), dtype=torch.float32, device=dev)
    if o32 is None and o32_elems(desc) > 0:
        o32 = torch.empty((sv.N, sv.D), dtype=torch.float32, device=dev)
    if not dynamic:
        workspace = None
    elif workspace is None:
        workspace = _scratch(fwd_workspace_bytes(desc), dev, stream, zero=True)
    cargs = (ctypes.byref(desc), ctypes.byref(sv.struct), _ptr(query), _ptr(norm_w), _ptr(out_w),
             _ptr(out), _ptr(lse), _ptr(out_rstd), _ptr(o32), _ptr(workspace),
             0 if workspace is None else workspace.numel(), _stream(stream))
    keep = (desc, sv, query, norm_w, out_w, workspace)
    return load().attnres_fwd, cargs, (out, lse, out_rstd, o32), keep


def attnres_fwd(values, query: torch.Tensor, norm_w: Optional[torch.Tensor] = None,
                out_w: Optional[torch.Tensor] = None, **kw):
    """Forward read. values: packed [S, N, D] or a list of [N, D] device tensors.
    Keywords: eps, scale, out_norm, out, lse, out_rstd, o32, workspace, dynamic, stream.
    Returns (out [N, D], lse [N] f32, out_rstd [N] f32 or None, o32 [N, D] f32 or None);
    output buffers are allocated with torch when not given. dynamic: hand tokens out through a
    counter in `workspace` (allocated when not given); False: static token split, no workspace."""
    fn, cargs, outs, _ = _prep_fwd(values, query, norm_w, out_w, **kw)
    _check(fn(*cargs))
    return outs


def _prep_bwd(values, query: torch.Tensor, norm_w: Optional[torch.Tensor],
                out_w: Optional[torch.Tensor], lse: torch.Tensor,
                out_rstd: Optional[torch.Tensor], o32: Optional[torch.Tensor],
                dout: torch.Tensor, *, eps: float = EPS_DEFAULT, scale: float = 1.0,
                out_norm: bool = False, deterministic: bool = False,
                accumulate: bool = False, dvalues=None,
                dq: Optional[torch.Tensor] = None,
                dw: Optional[torch.Tensor] = None, dow: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, noalloc: bool = False, stream=None):
    """Marshals a backward call: (C function, its arguments, outputs, objects to keep alive).
    noalloc: attnres_bwd_noalloc (no workspace; the library's own device array)."""
    sv = _SourceView(values)
    desc = make_desc(sv.S, sv.N, sv.D, query.numel(), sv.dtype, eps=eps, scale=scale,
                     has_norm_weight=norm_w is not None, out_norm=out_norm,
                     has_out_weight=out_w is not None, deterministic=deterministic,
                     accumulate_dvalues=accumulate)
    dev = sv.device
    if dout.dim() != 2 or dout.stride(1) != 1:
        raise ValueError("dout must be [N, D] with unit stride in D")
    if dvalues is None:
        if accumulate:
            raise ValueError("accumulate=True needs the dvalues to add to")
        dvalues = torch.empty((sv.S, sv.N, sv.D), dtype=sv.dtype, device=dev)
    dv = _SourceView(dvalues)
    if dq is None:
        dq = torch.empty((query.numel(),), dtype=sv.dtype, device=dev)
    if norm_w is not None and dw is None:
        dw = torch.empty((query.numel(),), dtype=sv.dtype, device=dev)
    if out_w is not None and dow is None:
        dow = torch.empty((sv.D,), dtype=sv.dtype, device=dev)
    dstride = dout.stride(0) if sv.N > 1 else sv.D
    head = (ctypes.byref(desc), ctypes.byref(sv.struct), _ptr(query), _ptr(norm_w), _ptr(out_w),
            _ptr(lse), _ptr(out_rstd), _ptr(o32), _ptr(dout), dstride, ctypes.byref(dv.struct),
            _ptr(dq), _ptr(dw), _ptr(dow))
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc takes no workspace")
        keep = (desc, sv, dv, query, norm_w, out_w, lse, out_rstd, o32, dout)
        return load().attnres_bwd_noalloc, head + (_stream(stream),), (dvalues, dq, dw, dow), keep
    need = workspace_bytes(desc)
    if workspace is None:
        workspace = _scratch(max(need, 256), dev, stream, zero=True)
    cargs = head + (_ptr(workspace), workspace.numel(), _stream(stream))
    keep = (desc, sv, dv, query, norm_w, out_w, lse, out_rstd, o32, dout, workspace)
    return load().attnres_bwd, cargs, (dvalues, dq, dw, dow), keep


def attnres_bwd_noalloc(values, query: torch.Tensor, norm_w: Optional[torch.Tensor],
                        out_w: Optional[torch.Tensor], lse: torch.Tensor,
                        out_rstd: Optional[torch.Tensor], o32: Optional[torch.Tensor],
                        dout: torch.Tensor, **kw):
    """attnres_bwd through the allocation-free entry point (no workspace: the library's device
    array; calls on one device must not overlap). Keywords as attnres_bwd except workspace; give
    dvalues, dq (and dw, dow) to keep the binding itself from allocating outputs."""
    fn, cargs, outs, _ = _prep_bwd(values, query, norm_w, out_w, lse, out_rstd, o32, dout,
                                   noalloc=True, **kw)
    _check(fn(*cargs))
    return outs


def attnres_bwd(values, query: torch.Tensor, norm_w: Optional[torch.Tensor],
                out_w: Optional[torch.Tensor], lse: torch.Tensor,
                out_rstd: Optional[torch.Tensor], o32: Optional[torch.Tensor],
                dout: torch.Tensor, **kw):
    """Backward read. Keywords: eps, scale, out_norm, deterministic, accumulate, dvalues, dq, dw,
    dow, workspace, stream. dvalues: packed [S, N, D] or list of [N, D] tensors to write
    (allocated packed when None). deterministic: a static token split (both schedules give
    bitwise-reproducible results; the default also hands the last batches out by counter).
    workspace: at least workspace_bytes(desc) bytes whose first 256 are zero before its first use
    (allocated zero-filled when None). accumulate: add this read's gradient to the existing dvalues (which must then be
    given). Returns (dvalues, dq, dw or None, dow or None)."""
    fn, cargs, outs, _ = _prep_bwd(values, query, norm_w, out_w, lse, out_rstd, o32, dout, **kw)
    _check(fn(*cargs))
    return outs


class BoundCall:
    """One library call with every argument marshalled in advance: calling it runs the C entry
    point on the same buffers and stream (a few microseconds of host time, for loops in which the
    per-call marshalling would otherwise leave the GPU waiting). `outputs` are the call's output
    tensors; the inputs and outputs are kept alive by the object and must not be reallocated."""

    def __init__(self, fn, cargs, outputs, keep):
        self._fn, self._cargs, self.outputs, self._keep = fn, cargs, outputs, keep

    def __call__(self):
        status = self._fn(*self._cargs)
        if status != 0:
            _check(status)
        return self.outputs


def bind_fwd(values, query: torch.Tensor, norm_w: Optional[torch.Tensor] = None,
             out_w: Optional[torch.Tensor] = None, **kw) -> BoundCall:
    """attnres_fwd's arguments marshalled once; see BoundCall."""
    return BoundCall(*_prep_fwd(values, query, norm_w, out_w, **kw))


def bind_bwd(values, query: torch.Tensor, norm_w: Optional[torch.Tensor],
             out_w: Optional[torch.Tensor], lse: torch.Tensor, out_rstd: Optional[torch.Tensor],
             o32: Optional[torch.Tensor], dout: torch.Tensor, **kw) -> BoundCall:
    """attnres_bwd's arguments marshalled once; see BoundCall."""
    return BoundCall(*_prep_bwd(values, query, norm_w, out_w, lse, out_rstd, o32, dout, **kw))




# ---------------------------------------------------------------- multi-query read

def make_multi_desc(S: int, N: int, D: int, R: int, M: int, dtype: torch.dtype, *,
                    eps: float = EPS_DEFAULT, scale: float = 1.0, layout: str = "query_major",
                    deterministic: bool = False, accumulate_dvalues: bool = False) -> MultiDesc:
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    return MultiDesc(S=S, D=D, R=R, M=M, dtype=_dtype_code(dtype), N=N, eps=eps, scale=scale,
                     layout=LAYOUTS[layout], deterministic=int(deterministic),
                     accumulate_dvalues=int(accumulate_dvalues))


def multi_workspace_bytes(desc: MultiDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(load().attnres_multi_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def multi_fwd_workspace_bytes(desc: MultiDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(load().attnres_multi_fwd_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def _rows_shape(layout: str, M: int, N: int, D: Optional[int] = None):
    base = (M, N) if layout == "query_major" else (N, M)
    return base if D is None else base + (D,)


def attnres_multi_fwd(values, queries: torch.Tensor, *, eps: float = EPS_DEFAULT,
                      scale: float = 1.0, layout: str = "query_major",
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, dynamic: bool = True,
                      stream=None):
    """Multi-query forward. values: packed [S, N, D] or a list of [N, D]; queries [M, R].
    Returns (y, lse): y [M, N, D] (query_major) or [N, M, D] (token_major), lse [M, N] or [N, M]
    in FP32, allocated with torch when not given."""
    sv = _SourceView(values)
    if queries.dim() != 2 or not queries.is_contiguous():
        raise ValueError("queries must be a contiguous [M, R] tensor")
    M, R = queries.shape
    desc = make_multi_desc(sv.S, sv.N, sv.D, R, M, sv.dtype, eps=eps, scale=scale, layout=layout)
    dev = sv.device
    if out is None:
        out = torch.empty(_rows_shape(layout, M, sv.N, sv.D), dtype=sv.dtype, device=dev)
    if lse is None:
        lse = torch.empty(_rows_shape(layout, M, sv.N), dtype=torch.float32, device=dev)
    if not dynamic:
        workspace = None
    elif workspace is None:
        workspace = _scratch(multi_fwd_workspace_bytes(desc), dev, stream)
    _check(load().attnres_multi_fwd(ctypes.byref(desc), ctypes.byref(sv.struct), _ptr(queries),
                                    _ptr(out), _ptr(lse), _ptr(workspace),
                                    0 if workspace is None else workspace.numel(),
                                    _stream(stream)))
    return out, lse


def attnres_multi_bwd(values, queries: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor, *,
                      eps: float = EPS_DEFAULT, scale: float = 1.0, layout: str = "query_major",
                      deterministic: bool = False, accumulate: bool = False, dvalues=None,
                      dq: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None):
    """Multi-query backward. dout like the forward's y (contiguous, same layout). Returns
    (dvalues, dq [M, R]); dvalues are allocated packed when not given (accumulate needs them)."""
    sv = _SourceView(values)
    M, R = queries.shape
    desc = make_multi_desc(sv.S, sv.N, sv.D, R, M, sv.dtype, eps=eps, scale=scale, layout=layout,
                           deterministic=deterministic, accumulate_dvalues=accumulate)
    dev = sv.device
    if not dout.is_contiguous():
        raise ValueError("dout must be contiguous")
    if dvalues is None:
        if accumulate:
            raise ValueError("accumulate=True needs the dvalues to add to")
        dvalues = torch.empty((sv.S, sv.N, sv.D), dtype=sv.dtype, device=dev)
    dv = _SourceView(dvalues)
    if dq is None:
        dq = torch.empty((M, R), dtype=sv.dtype, device=dev)
    if workspace is None:
        workspace = _scratch(max(multi_workspace_bytes(desc), 256), dev, stream)
    _check(load().attnres_multi_bwd(ctypes.byref(desc), ctypes.byref(sv.struct), _ptr(queries),
                                    _ptr(lse), _ptr(dout), ctypes.byref(dv.struct), _ptr(dq),
                                    _ptr(workspace), workspace.numel(), _stream(stream)))
    return dvalues, dq


# ---------------------------------------------------------------- selected-query read

def make_selected_desc(S: int, N: int, D: int, R: int, E: int, K: int, dtype: torch.dtype, *,
                       eps: float = EPS_DEFAULT, scale: float = 1.0, deterministic: bool = False,
                       accumulate_dvalues: bool = False) -> SelectedDesc:
    return SelectedDesc(S=S, D=D, R=R, E=E, K=K, dtype=_dtype_code(dtype), N=N, eps=eps,
                        scale=scale, deterministic=int(deterministic),
                        accumulate_dvalues=int(accumulate_dvalues))


def selected_workspace_bytes(desc: SelectedDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(load().attnres_selected_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def selected_fwd_workspace_bytes(desc: SelectedDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(load().attnres_selected_fwd_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def _check_ids(ids: torch.Tensor, N: int) -> int:
    if ids.dtype != torch.int64 or ids.dim() != 2 or ids.shape[0] != N or not ids.is_contiguous():
        raise ValueError(f"ids must be a contiguous int64 [N={N}, K] tensor")
    return int(ids.shape[1])


def attnres_selected_fwd(values, bank: torch.Tensor, ids: torch.Tensor, *,
                         eps: float = EPS_DEFAULT, scale: float = 1.0,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, dynamic: bool = True,
                         stream=None):
    """Selected-query forward. values: packed [S, N, D] or a list of [N, D]; bank [E, R]; ids
    [N, K] int64. Returns (y [N, K, D], lse [N, K] FP32)."""
    sv = _SourceView(values)
    if bank.dim() != 2 or not bank.is_contiguous():
        raise ValueError("bank must be a contiguous [E, R] tensor")
    E, R = bank.shape
    K = _check_ids(ids, sv.N)
    desc = make_selected_desc(sv.S, sv.N, sv.D, R, E, K, sv.dtype, eps=eps, scale=scale)
    dev = sv.device
    if out is None:
        out = torch.empty((sv.N, K, sv.D), dtype=sv.dtype, device=dev)
    if lse is None:
        lse = torch.empty((sv.N, K), dtype=torch.float32, device=dev)
    if not dynamic:
        workspace = None
    elif workspace is None:
        workspace = _scratch(selected_fwd_workspace_bytes(desc), dev, stream)
    _check(load().attnres_selected_fwd(ctypes.byref(desc), ctypes.byref(sv.struct), _ptr(bank),
                                       _ptr(ids), _ptr(out), _ptr(lse), _ptr(workspace),
                                       0 if workspace is None else workspace.numel(),
                                       _stream(stream)))
    return out, lse


def attnres_selected_ids_flag(workspace: torch.Tensor, clear: bool = False, stream=None) -> bool:
    """True if a selected-query forward that was given this workspace has read an id outside
    [0, E) since the flag was last cleared (clear=True clears it after reading). Waits for the
    work queued on the stream."""
    flag = ctypes.c_int32(0)
    _check(load().attnres_selected_ids_flag(_ptr(workspace), workspace.numel(), int(bool(clear)),
                                            ctypes.byref(flag), _stream(stream)))
    return bool(flag.value)


def stream_probe(inputs, outputs, chunks_per_thread: int = 1, blocks_per_cu: int = 8,
                 stream=None) -> None:
    """Measurement aid (not the AttnRes computation): streams the rows of every input tensor to
    the outputs (output j = input j for 1 <= j < len(inputs); output 0 and the outputs beyond the
    inputs = XOR of the inputs). At most 128 of each; all tensors contiguous, same shape
    [rows, ...] with rows of a multiple of 16 bytes, on one device."""
    if not inputs or not outputs:
        raise ValueError("stream_probe needs at least one input and one output")
    t0 = inputs[0]
    nbytes = t0.numel() * t0.element_size()
    rows = t0.shape[0] if t0.dim() > 0 else 1
    for t in list(inputs) + list(outputs):
        if not t.is_contiguous() or t.numel() * t.element_size() != nbytes or t.shape[0] != rows:
            raise ValueError("stream_probe tensors must be contiguous and alike")
    ins = (ctypes.c_void_p * len(inputs))(*[_ptr(t) for t in inputs])
    outs = (ctypes.c_void_p * len(outputs))(*[_ptr(t) for t in outputs])
    _check(load().attnres_stream_probe(ins, len(inputs), outs, len(outputs), rows, nbytes // rows,
                                       chunks_per_thread, blocks_per_cu, _stream(stream)))


def attnres_selected_bwd(values, bank: torch.Tensor, ids: torch.Tensor, lse: torch.Tensor,
                         dout: torch.Tensor, *, eps: float = EPS_DEFAULT, scale: float = 1.0,
                         deterministic: bool = False, accumulate: bool = False, dvalues=None,
                         dbank: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None):
    """Selected-query backward. dout [N, K, D] contiguous. Returns (dvalues, dbank [E, R])."""
    sv = _SourceView(values)
    E, R = bank.shape
    K = _check_ids(ids, sv.N)
    desc = make_selected_desc(sv.S, sv.N, sv.D, R, E, K, sv.dtype, eps=eps, scale=scale,
                              deterministic=deterministic, accumulate_dvalues=accumulate)
    dev = sv.device
    if not dout.is_contiguous():
        raise ValueError("dout must be contiguous")
    if dvalues is None:
        if accumulate:
            raise ValueError("accumulate=True needs the dvalues to add to")
        dvalues = torch.empty((sv.S, sv.N, sv.D), dtype=sv.dtype, device=dev)
    dv = _SourceView(dvalues)
    if dbank is None:
        dbank = torch.empty((E, R), dtype=sv.dtype, device=dev)
    if workspace is None:
        workspace = _scratch(max(selected_workspace_bytes(desc), 256), dev, stream)
    _check(load().attnres_selected_bwd(ctypes.byref(desc), ctypes.byref(sv.struct), _ptr(bank),
                                       _ptr(ids), _ptr(lse), _ptr(dout), ctypes.byref(dv.struct),
                                       _ptr(dbank), _ptr(workspace), workspace.numel(),
                                       _stream(stream)))
    return dvalues, dbank
