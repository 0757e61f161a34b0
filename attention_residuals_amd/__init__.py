"""MI355X (gfx950) Attention Residuals (AttnRes) read, forward and backward.

The compute lives in ``libattnres.so`` (hand-written HIP kernels behind the C ABI of
``include/attnres.h``); this package marshals torch tensors into it. Build the library with
``python -m attention_residuals_amd.build``. Nothing here falls back to a CPU implementation.
"""
from ._binding import (ATTNRES_BF16, ATTNRES_F32, EPS_DEFAULT, EXPORTS, AttnResError, BoundCall,
                       Desc, MultiDesc, SelectedDesc, Sources, attnres_bwd, attnres_bwd_noalloc,
                       attnres_fwd,
                       bind_bwd, bind_fwd,
                       attnres_multi_bwd, attnres_multi_fwd, attnres_selected_bwd,
                       attnres_selected_fwd, attnres_selected_ids_flag, fwd_workspace_bytes, load,
                       make_desc,
                       make_multi_desc, make_selected_desc, multi_fwd_workspace_bytes,
                       multi_workspace_bytes, o32_elems, selected_fwd_workspace_bytes,
                       selected_workspace_bytes, workspace_bytes)
from .ops import attnres, attnres_multi, attnres_selected

__all__ = ["attnres", "attnres_multi", "attnres_selected", "attnres_fwd", "attnres_bwd",
           "attnres_bwd_noalloc",
           "bind_fwd", "bind_bwd", "BoundCall",
           "attnres_multi_fwd", "attnres_multi_bwd", "attnres_selected_fwd",
           "attnres_selected_bwd", "attnres_selected_ids_flag", "o32_elems", "workspace_bytes", "fwd_workspace_bytes",
           "multi_workspace_bytes", "multi_fwd_workspace_bytes", "selected_workspace_bytes",
           "selected_fwd_workspace_bytes", "make_desc", "make_multi_desc", "make_selected_desc",
           "MultiDesc", "SelectedDesc",
           "load", "Desc", "Sources", "AttnResError", "EXPORTS", "ATTNRES_BF16", "ATTNRES_F32",
           "EPS_DEFAULT"]
