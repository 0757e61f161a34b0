"""``attnres(values, query, ...)`` as a differentiable torch op backed by the HIP library.

Public signature follows the "Fast Attention Residuals" PyPI page (Quickstart): values are a
packed [S, ..., D] tensor or an ordered list/tuple of [..., D] tensors; query is [R] with
1 <= R <= D; the output keeps width D. Optional key-norm weight ``norm_weight`` [R] and output
RMSNorm (``out_norm``, optional ``out_weight`` [D]) follow the FLA PR page's AttnRes operator.
The forward saves the per-row log-sum-exp (and rho_o, and the FP32 mixture when the backward
streams); the backward recomputes the routing weights from them.
"""
from __future__ import annotations

from typing import Optional, Sequence, Union

import torch

from . import _binding as B


class _AttnResFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, eps, scale, out_norm, deterministic, packed, query, norm_w, out_w, *srcs):
        values = srcs[0] if packed else list(srcs)
        y, lse, rstd, o32 = B.attnres_fwd(values, query, norm_w, out_w, eps=eps, scale=scale,
                                          out_norm=out_norm)
        ctx.eps, ctx.scale, ctx.out_norm, ctx.packed = eps, scale, out_norm, packed
        ctx.deterministic = deterministic
        ctx.save_for_backward(query, norm_w, out_w, lse, rstd, o32, *srcs)
        return y

    @staticmethod
    def backward(ctx, dy):
        query, norm_w, out_w, lse, rstd, o32, *srcs = ctx.saved_tensors
        if dy.stride(-1) != 1:
            dy = dy.contiguous()
        if ctx.packed:
            values = srcs[0]
            dvalues = torch.empty_like(values, memory_format=torch.contiguous_format)
        else:
            values = list(srcs)
            dvalues = [torch.empty(v.shape, dtype=v.dtype, device=v.device) for v in values]
        dvalues, dq, dw, dow = B.attnres_bwd(values, query, norm_w, out_w, lse, rstd, o32, dy,
                                             eps=ctx.eps, scale=ctx.scale,
                                             out_norm=ctx.out_norm,
                                             deterministic=ctx.deterministic, dvalues=dvalues)
        dsrcs = (dvalues,) if ctx.packed else tuple(dvalues)
        return (None, None, None, None, None, dq.view_as(query), dw, dow) + dsrcs


def attnres(values: Union[torch.Tensor, Sequence[torch.Tensor]], query: torch.Tensor, *,
            eps: float = B.EPS_DEFAULT, scale: float = 1.0,
            norm_weight: Optional[torch.Tensor] = None, out_norm: bool = False,
            out_weight: Optional[torch.Tensor] = None,
            deterministic: bool = False) -> torch.Tensor:
    """AttnRes read of S ordered sources with one learned query; returns [..., D].
    deterministic=True makes the q/w/ow gradients bitwise reproducible (fixed token split)."""
    if out_weight is not None and not out_norm:
        raise ValueError("out_weight requires out_norm=True")
    if isinstance(values, torch.Tensor):
        S, D = values.shape[0], values.shape[-1]
        lead = values.shape[1:-1]
        flat = values.reshape(S, -1, D)
        if flat.stride(-1) != 1:
            flat = flat.contiguous()
        y = _AttnResFn.apply(eps, scale, out_norm, deterministic, True, query.reshape(-1),
                             norm_weight, out_weight, flat)
    else:
        vs = list(values)
        D = vs[0].shape[-1]
        lead = vs[0].shape[:-1]
        flat = []
        for v in vs:
            f = v.reshape(-1, D)
            if f.stride(-1) != 1:
                f = f.contiguous()
            flat.append(f)
        if len({f.stride(0) for f in flat}) > 1:
            flat = [f.contiguous() for f in flat]
        y = _AttnResFn.apply(eps, scale, out_norm, deterministic, False, query.reshape(-1),
                             norm_weight, out_weight, *flat)
    return y.reshape(*lead, D)


class _AttnResMultiFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, eps, scale, layout, deterministic, packed, queries, *srcs):
        values = srcs[0] if packed else list(srcs)
        y, lse = B.attnres_multi_fwd(values, queries, eps=eps, scale=scale, layout=layout)
        ctx.eps, ctx.scale, ctx.layout, ctx.packed = eps, scale, layout, packed
        ctx.deterministic = deterministic
        ctx.save_for_backward(queries, lse, *srcs)
        return y

    @staticmethod
    def backward(ctx, dy):
        queries, lse, *srcs = ctx.saved_tensors
        dy = dy.contiguous()
        if ctx.packed:
            values = srcs[0]
            dvalues = torch.empty_like(values, memory_format=torch.contiguous_format)
        else:
            values = list(srcs)
            dvalues = [torch.empty(v.shape, dtype=v.dtype, device=v.device) for v in values]
        dvalues, dq = B.attnres_multi_bwd(values, queries, lse, dy, eps=ctx.eps, scale=ctx.scale,
                                          layout=ctx.layout, deterministic=ctx.deterministic,
                                          dvalues=dvalues)
        dsrcs = (dvalues,) if ctx.packed else tuple(dvalues)
        return (None, None, None, None, None, dq) + dsrcs


def attnres_multi(values: Union[torch.Tensor, Sequence[torch.Tensor]], queries: torch.Tensor, *,
                  eps: float = B.EPS_DEFAULT, scale: float = 1.0,
                  output_layout: str = "query_major", deterministic: bool = False) -> torch.Tensor:
    """Multi-query AttnRes read ("Fast Attention Residuals" page, Multi-query AttnRes): queries
    [M, R], 1 <= M <= 16, each with its own routing weights and full-width output. Returns
    [M, ..., D] (query_major) or [..., M, D] (token_major)."""
    if queries.dim() != 2:
        raise ValueError("queries must be [M, R]")
    q = queries.contiguous()
    M = q.shape[0]
    if isinstance(values, torch.Tensor):
        S, D = values.shape[0], values.shape[-1]
        lead = values.shape[1:-1]
        flat = values.reshape(S, -1, D)
        if flat.stride(-1) != 1:
            flat = flat.contiguous()
        y = _AttnResMultiFn.apply(eps, scale, output_layout, deterministic, True, q, flat)
    else:
        vs = list(values)
        D = vs[0].shape[-1]
        lead = vs[0].shape[:-1]
        flat = [v.reshape(-1, D) for v in vs]
        flat = [f if f.stride(-1) == 1 else f.contiguous() for f in flat]
        if len({f.stride(0) for f in flat}) > 1:
            flat = [f.contiguous() for f in flat]
        y = _AttnResMultiFn.apply(eps, scale, output_layout, deterministic, False, q, *flat)
    if output_layout == "query_major":
        return y.reshape(M, *lead, D)
    return y.reshape(*lead, M, D)
