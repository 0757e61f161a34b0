"""The AttnRes reads as torch custom operators (``torch.library``), so that ``torch.compile`` with
``fullgraph=True`` traces them as single opaque nodes ("Fast Attention Residuals" PyPI page,
Quickstart: the read is used under ``torch.compile(..., fullgraph=True)``).

Each read has a packed-sources form (values [S, N, D]) and a list form (S tensors [N, D]), so a
packed input is never split and restacked. Fake implementations give output shapes and dtypes only
(they ask the library's host-side planner whether the backward needs the FP32 mixture). The real
implementations call the C ABI through ``_binding``; autograd is registered on the forward ops.
Optional outputs that are absent come back as empty tensors.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import torch
from torch import Tensor

from . import _binding as B


def _empty(like: Tensor) -> Tensor:
    return like.new_empty((0,), dtype=torch.float32)


def _opt(t: Tensor) -> Optional[Tensor]:
    return None if t.numel() == 0 else t


def _needs_o32(S: int, N: int, D: int, R: int, dtype, out_norm: bool) -> bool:
    return B.o32_elems(B.make_desc(S, N, D, R, dtype, out_norm=out_norm)) > 0


# ---------------------------------------------------------------- single-query read

def _fwd(values, query, norm_w, out_w, eps, scale, out_norm):
    y, lse, rstd, o32 = B.attnres_fwd(values, query, norm_w, out_w, eps=eps, scale=scale,
                                      out_norm=out_norm)
    return (y, lse, rstd if rstd is not None else _empty(query),
            o32 if o32 is not None else _empty(query))


def _fwd_fake(S, N, D, dtype, like, query, out_norm):
    y = like.new_empty((N, D), dtype=dtype)
    lse = like.new_empty((N,), dtype=torch.float32)
    rstd = like.new_empty((N,) if out_norm else (0,), dtype=torch.float32)
    o32 = like.new_empty((N, D) if _needs_o32(S, N, D, query.shape[0], dtype, out_norm) else (0,),
                         dtype=torch.float32)
    return y, lse, rstd, o32


@torch.library.custom_op("attnres_amd::fwd_packed", mutates_args=(), device_types="cuda")
def fwd_packed(values: Tensor, query: Tensor, norm_w: Optional[Tensor], out_w: Optional[Tensor],
               eps: float, scale: float, out_norm: bool,
               deterministic: bool) -> Tuple[Tensor, Tensor, Tensor, Tensor]:
    return _fwd(values, query, norm_w, out_w, eps, scale, out_norm)


@fwd_packed.register_fake
def _(values, query, norm_w, out_w, eps, scale, out_norm, deterministic):
    S, N, D = values.shape
    return _fwd_fake(S, N, D, values.dtype, values, query, out_norm)


@torch.library.custom_op("attnres_amd::fwd_list", mutates_args=(), device_types="cuda")
def fwd_list(values: List[Tensor], query: Tensor, norm_w: Optional[Tensor],
             out_w: Optional[Tensor], eps: float, scale: float, out_norm: bool,
             deterministic: bool) -> Tuple[Tensor, Tensor, Tensor, Tensor]:
    return _fwd(list(values), query, norm_w, out_w, eps, scale, out_norm)


@fwd_list.register_fake
def _(values, query, norm_w, out_w, eps, scale, out_norm, deterministic):
    N, D = values[0].shape
    return _fwd_fake(len(values), N, D, values[0].dtype, values[0], query, out_norm)


def _bwd(values, dvalues, query, norm_w, out_w, lse, rstd, o32, dy, eps, scale, out_norm,
         deterministic):
    _, dq, dw, dow = B.attnres_bwd(values, query, norm_w, out_w, lse, _opt(rstd), _opt(o32), dy,
                                   eps=eps, scale=scale, out_norm=out_norm,
                                   deterministic=deterministic, dvalues=dvalues)
    return dq, dw if dw is not None else _empty(query), dow if dow is not None else _empty(query)


@torch.library.custom_op("attnres_amd::bwd_packed", mutates_args=(), device_types="cuda")
def bwd_packed(values: Tensor, query: Tensor, norm_w: Optional[Tensor], out_w: Optional[Tensor],
               lse: Tensor, rstd: Tensor, o32: Tensor, dy: Tensor, eps: float, scale: float,
               out_norm: bool, deterministic: bool) -> Tuple[Tensor, Tensor, Tensor, Tensor]:
    dvalues = torch.empty(values.shape, dtype=values.dtype, device=values.device)
    dq, dw, dow = _bwd(values, dvalues, query, norm_w, out_w, lse, rstd, o32, dy.contiguous(),
                       eps, scale, out_norm, deterministic)
    return dvalues, dq, dw, dow


@bwd_packed.register_fake
def _(values, query, norm_w, out_w, lse, rstd, o32, dy, eps, scale, out_norm, deterministic):
    D = values.shape[-1]
    return (values.new_empty(values.shape), query.new_empty(query.shape),
            query.new_empty(query.shape if norm_w is not None else (0,),
                            dtype=query.dtype if norm_w is not None else torch.float32),
            query.new_empty((D,) if out_w is not None else (0,),
                            dtype=query.dtype if out_w is not None else torch.float32))


@torch.library.custom_op("attnres_amd::bwd_list", mutates_args=(), device_types="cuda")
def bwd_list(values: List[Tensor], query: Tensor, norm_w: Optional[Tensor],
             out_w: Optional[Tensor], lse: Tensor, rstd: Tensor, o32: Tensor, dy: Tensor,
             eps: float, scale: float, out_norm: bool,
             deterministic: bool) -> Tuple[List[Tensor], Tensor, Tensor, Tensor]:
    vals = list(values)
    dvalues = [torch.empty(v.shape, dtype=v.dtype, device=v.device) for v in vals]
    dq, dw, dow = _bwd(vals, dvalues, query, norm_w, out_w, lse, rstd, o32, dy.contiguous(), eps,
                       scale, out_norm, deterministic)
    return dvalues, dq, dw, dow


@bwd_list.register_fake
def _(values, query, norm_w, out_w, lse, rstd, o32, dy, eps, scale, out_norm, deterministic):
    D = values[0].shape[-1]
    return ([v.new_empty(v.shape) for v in values], query.new_empty(query.shape),
            query.new_empty(query.shape if norm_w is not None else (0,),
                            dtype=query.dtype if norm_w is not None else torch.float32),
            query.new_empty((D,) if out_w is not None else (0,),
                            dtype=query.dtype if out_w is not None else torch.float32))


def _setup_fwd(ctx, inputs, output):
    values, query, norm_w, out_w, eps, scale, out_norm, deterministic = inputs
    _, lse, rstd, o32 = output
    ctx.packed = isinstance(values, Tensor)
    vals = [values] if ctx.packed else list(values)
    ctx.nsrc = len(vals)
    ctx.has_w, ctx.has_ow = norm_w is not None, out_w is not None
    ctx.args = (eps, scale, out_norm, deterministic)
    ctx.save_for_backward(query, norm_w, out_w, lse, rstd, o32, *vals)


def _backward_fwd(ctx, gy, glse, grstd, go32):
    query, norm_w, out_w, lse, rstd, o32, *vals = ctx.saved_tensors
    eps, scale, out_norm, deterministic = ctx.args
    op = bwd_packed if ctx.packed else bwd_list
    values = vals[0] if ctx.packed else vals
    dvalues, dq, dw, dow = op(values, query, norm_w, out_w, lse, rstd, o32, gy, eps, scale,
                              out_norm, deterministic)
    return (dvalues, dq, dw if ctx.has_w else None, dow if ctx.has_ow else None,
            None, None, None, None)


fwd_packed.register_autograd(_backward_fwd, setup_context=_setup_fwd)
fwd_list.register_autograd(_backward_fwd, setup_context=_setup_fwd)


# ---------------------------------------------------------------- multi-query read

def _rows_shape(layout: str, M: int, N: int, D: Optional[int] = None):
    base = (M, N) if layout == "query_major" else (N, M)
    return base if D is None else base + (D,)


@torch.library.custom_op("attnres_amd::multi_fwd_packed", mutates_args=(), device_types="cuda")
def multi_fwd_packed(values: Tensor, queries: Tensor, eps: float, scale: float, layout: str,
                     deterministic: bool) -> Tuple[Tensor, Tensor]:
    return B.attnres_multi_fwd(values, queries, eps=eps, scale=scale, layout=layout)


@multi_fwd_packed.register_fake
def _(values, queries, eps, scale, layout, deterministic):
    _, N, D = values.shape
    M = queries.shape[0]
    return (values.new_empty(_rows_shape(layout, M, N, D)),
            values.new_empty(_rows_shape(layout, M, N), dtype=torch.float32))


@torch.library.custom_op("attnres_amd::multi_fwd_list", mutates_args=(), device_types="cuda")
def multi_fwd_list(values: List[Tensor], queries: Tensor, eps: float, scale: float, layout: str,
                   deterministic: bool) -> Tuple[Tensor, Tensor]:
    return B.attnres_multi_fwd(list(values), queries, eps=eps, scale=scale, layout=layout)


@multi_fwd_list.register_fake
def _(values, queries, eps, scale, layout, deterministic):
    N, D = values[0].shape
    M = queries.shape[0]
    return (values[0].new_empty(_rows_shape(layout, M, N, D)),
            values[0].new_empty(_rows_shape(layout, M, N), dtype=torch.float32))


@torch.library.custom_op("attnres_amd::multi_bwd_packed", mutates_args=(), device_types="cuda")
def multi_bwd_packed(values: Tensor, queries: Tensor, lse: Tensor, dy: Tensor, eps: float,
                     scale: float, layout: str, deterministic: bool) -> Tuple[Tensor, Tensor]:
    return B.attnres_multi_bwd(values, queries, lse, dy.contiguous(), eps=eps, scale=scale,
                               layout=layout, deterministic=deterministic)


@multi_bwd_packed.register_fake
def _(values, queries, lse, dy, eps, scale, layout, deterministic):
    return values.new_empty(values.shape), queries.new_empty(queries.shape)


@torch.library.custom_op("attnres_amd::multi_bwd_list", mutates_args=(), device_types="cuda")
def multi_bwd_list(values: List[Tensor], queries: Tensor, lse: Tensor, dy: Tensor, eps: float,
                   scale: float, layout: str,
                   deterministic: bool) -> Tuple[List[Tensor], Tensor]:
    vals = list(values)
    dvalues = [torch.empty(v.shape, dtype=v.dtype, device=v.device) for v in vals]
    _, dq = B.attnres_multi_bwd(vals, queries, lse, dy.contiguous(), eps=eps, scale=scale,
                                layout=layout, deterministic=deterministic, dvalues=dvalues)
    return dvalues, dq


@multi_bwd_list.register_fake
def _(values, queries, lse, dy, eps, scale, layout, deterministic):
    return [v.new_empty(v.shape) for v in values], queries.new_empty(queries.shape)


def _setup_multi(ctx, inputs, output):
    values, queries, eps, scale, layout, deterministic = inputs
    _, lse = output
    ctx.packed = isinstance(values, Tensor)
    vals = [values] if ctx.packed else list(values)
    ctx.args = (eps, scale, layout, deterministic)
    ctx.save_for_backward(queries, lse, *vals)


def _backward_multi(ctx, gy, glse):
    queries, lse, *vals = ctx.saved_tensors
    eps, scale, layout, deterministic = ctx.args
    if ctx.packed:
        dvalues, dq = multi_bwd_packed(vals[0], queries, lse, gy, eps, scale, layout,
                                       deterministic)
    else:
        dvalues, dq = multi_bwd_list(vals, queries, lse, gy, eps, scale, layout, deterministic)
    return dvalues, dq, None, None, None, None


multi_fwd_packed.register_autograd(_backward_multi, setup_context=_setup_multi)
multi_fwd_list.register_autograd(_backward_multi, setup_context=_setup_multi)


# ---------------------------------------------------------------- selected-query read

@torch.library.custom_op("attnres_amd::selected_fwd_packed", mutates_args=(), device_types="cuda")
def selected_fwd_packed(values: Tensor, bank: Tensor, ids: Tensor, eps: float, scale: float,
                        deterministic: bool) -> Tuple[Tensor, Tensor]:
    return B.attnres_selected_fwd(values, bank, ids, eps=eps, scale=scale)


@selected_fwd_packed.register_fake
def _(values, bank, ids, eps, scale, deterministic):
    _, N, D = values.shape
    K = ids.shape[1]
    return values.new_empty((N, K, D)), values.new_empty((N, K), dtype=torch.float32)


@torch.library.custom_op("attnres_amd::selected_fwd_list", mutates_args=(), device_types="cuda")
def selected_fwd_list(values: List[Tensor], bank: Tensor, ids: Tensor, eps: float, scale: float,
                      deterministic: bool) -> Tuple[Tensor, Tensor]:
    return B.attnres_selected_fwd(list(values), bank, ids, eps=eps, scale=scale)


@selected_fwd_list.register_fake
def _(values, bank, ids, eps, scale, deterministic):
    N, D = values[0].shape
    K = ids.shape[1]
    return values[0].new_empty((N, K, D)), values[0].new_empty((N, K), dtype=torch.float32)


@torch.library.custom_op("attnres_amd::selected_bwd_packed", mutates_args=(), device_types="cuda")
def selected_bwd_packed(values: Tensor, bank: Tensor, ids: Tensor, lse: Tensor, dy: Tensor,
                        eps: float, scale: float, deterministic: bool) -> Tuple[Tensor, Tensor]:
    return B.attnres_selected_bwd(values, bank, ids, lse, dy.contiguous(), eps=eps, scale=scale,
                                  deterministic=deterministic)


@selected_bwd_packed.register_fake
def _(values, bank, ids, lse, dy, eps, scale, deterministic):
    return values.new_empty(values.shape), bank.new_empty(bank.shape)


@torch.library.custom_op("attnres_amd::selected_bwd_list", mutates_args=(), device_types="cuda")
def selected_bwd_list(values: List[Tensor], bank: Tensor, ids: Tensor, lse: Tensor, dy: Tensor,
                      eps: float, scale: float,
                      deterministic: bool) -> Tuple[List[Tensor], Tensor]:
    vals = list(values)
    dvalues = [torch.empty(v.shape, dtype=v.dtype, device=v.device) for v in vals]
    _, dbank = B.attnres_selected_bwd(vals, bank, ids, lse, dy.contiguous(), eps=eps, scale=scale,
                                      deterministic=deterministic, dvalues=dvalues)
    return dvalues, dbank


@selected_bwd_list.register_fake
def _(values, bank, ids, lse, dy, eps, scale, deterministic):
    return [v.new_empty(v.shape) for v in values], bank.new_empty(bank.shape)


def _setup_selected(ctx, inputs, output):
    values, bank, ids, eps, scale, deterministic = inputs
    _, lse = output
    ctx.packed = isinstance(values, Tensor)
    vals = [values] if ctx.packed else list(values)
    ctx.args = (eps, scale, deterministic)
    ctx.save_for_backward(bank, ids, lse, *vals)


def _backward_selected(ctx, gy, glse):
    bank, ids, lse, *vals = ctx.saved_tensors
    eps, scale, deterministic = ctx.args
    if ctx.packed:
        dvalues, dbank = selected_bwd_packed(vals[0], bank, ids, lse, gy, eps, scale,
                                             deterministic)
    else:
        dvalues, dbank = selected_bwd_list(vals, bank, ids, lse, gy, eps, scale, deterministic)
    return dvalues, dbank, None, None, None, None


selected_fwd_packed.register_autograd(_backward_selected, setup_context=_setup_selected)
selected_fwd_list.register_autograd(_backward_selected, setup_context=_setup_selected)


# ---------------------------------------------------------------- user-facing calls

def _flatten_sources(values, D_last: bool = True):
    if isinstance(values, Tensor):
        S, D = values.shape[0], values.shape[-1]
        lead = values.shape[1:-1]
        flat = values.reshape(S, -1, D)
        if flat.stride(-1) != 1:
            flat = flat.contiguous()
        return True, flat, lead, D
    vs = list(values)
    D = vs[0].shape[-1]
    lead = vs[0].shape[:-1]
    flat = [v.reshape(-1, D) for v in vs]
    flat = [f if f.stride(-1) == 1 else f.contiguous() for f in flat]
    if len({f.stride(0) for f in flat}) > 1:
        flat = [f.contiguous() for f in flat]
    return False, flat, lead, D


def attnres(values, query: Tensor, *, eps: float = B.EPS_DEFAULT, scale: float = 1.0,
            norm_weight: Optional[Tensor] = None, out_norm: bool = False,
            out_weight: Optional[Tensor] = None, deterministic: bool = False) -> Tensor:
    """AttnRes read of S ordered sources with one learned query; returns [..., D].
    values: packed [S, ..., D] or an ordered list/tuple of [..., D]; query [R], 1 <= R <= D.
    Optional key-norm weight [R] and output RMSNorm (with optional weight [D]).
    deterministic=True makes the q/w/ow gradients bitwise reproducible (fixed token split)."""
    if out_weight is not None and not out_norm:
        raise ValueError("out_weight requires out_norm=True")
    packed, flat, lead, D = _flatten_sources(values)
    op = fwd_packed if packed else fwd_list
    y, _, _, _ = op(flat, query.reshape(-1), norm_weight, out_weight, float(eps), float(scale),
                    bool(out_norm), bool(deterministic))
    return y.reshape(*lead, D)


def attnres_multi(values, queries: Tensor, *, eps: float = B.EPS_DEFAULT, scale: float = 1.0,
                  output_layout: str = "query_major", deterministic: bool = False) -> Tensor:
    """Multi-query AttnRes read ("Fast Attention Residuals" page, Multi-query AttnRes): queries
    [M, R], 1 <= M <= 16, each with its own routing weights and full-width output. Returns
    [M, ..., D] (query_major) or [..., M, D] (token_major)."""
    if queries.dim() != 2:
        raise ValueError("queries must be [M, R]")
    if output_layout not in B.LAYOUTS:
        raise ValueError(f"output_layout must be one of {sorted(B.LAYOUTS)}")
    q = queries.contiguous()
    M = q.shape[0]
    packed, flat, lead, D = _flatten_sources(values)
    op = multi_fwd_packed if packed else multi_fwd_list
    y, _ = op(flat, q, float(eps), float(scale), output_layout, bool(deterministic))
    if output_layout == "query_major":
        return y.reshape(M, *lead, D)
    return y.reshape(*lead, M, D)


def attnres_selected(values, query_bank: Tensor, ids: Tensor, *, eps: float = B.EPS_DEFAULT,
                     scale: float = 1.0, deterministic: bool = False) -> Tensor:
    """Selected-query AttnRes read ("Fast Attention Residuals" page, Multi-query AttnRes: per-token
    query selection): token t reads the sources with the K queries query_bank[ids[t, k]] of an
    [E, R] bank. ids: integer [..., K] over the sources' leading shape. Returns [..., K, D]. An id
    outside [0, E) reads a zero query (uniform weights) and adds nothing to the bank's gradient."""
    if query_bank.dim() != 2:
        raise ValueError("query_bank must be [E, R]")
    packed, flat, lead, D = _flatten_sources(values)
    if tuple(ids.shape[:-1]) != tuple(lead):
        raise ValueError(f"ids must be [..., K] over the sources' leading shape {tuple(lead)}")
    K = ids.shape[-1]
    flat_ids = ids.reshape(-1, K).to(torch.int64).contiguous()
    op = selected_fwd_packed if packed else selected_fwd_list
    y, _ = op(flat, query_bank.contiguous(), flat_ids, float(eps), float(scale),
              bool(deterministic))
    return y.reshape(*lead, K, D)
