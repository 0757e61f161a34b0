"""The torch custom operators' fake (shape-only) implementations, on the CPU with fake CUDA
tensors: output shapes and dtypes of every forward and backward op. No kernel runs here (and the
autograd engine needs a device context, so the backward ops are called directly; the GPU tests run
them through autograd and torch.compile)."""
import pytest
import torch
from torch._subclasses.fake_tensor import FakeTensorMode

import attention_residuals_amd as A
from attention_residuals_amd import ops

BF = torch.bfloat16


def _t(*shape, dtype=BF, grad=False):
    t = torch.empty(shape, dtype=dtype, device="cuda")
    return t.requires_grad_(grad) if grad else t


@pytest.mark.parametrize("out_norm,has_w,has_ow", [(False, True, False), (True, False, True),
                                                   (True, False, False)])
def test_single_query_ops_shapes_and_backward(out_norm, has_w, has_ow):
    with FakeTensorMode():
        S, N, D, R = 10 if not out_norm else 64, 37, 4096 if not out_norm else 8192, 512
        v = _t(S, N, D)
        q = _t(R)
        w = _t(R) if has_w else None
        ow = _t(D) if has_ow else None
        y, lse, rstd, o32 = ops.fwd_packed(v, q, w, ow, 2.0 ** -23, 1.0, out_norm, False)
        assert y.shape == (N, D) and y.dtype == BF and lse.shape == (N,)
        assert rstd.shape == ((N,) if out_norm else (0,))
        # the backward streams (and needs the FP32 mixture) exactly when rows do not stay on chip
        assert o32.shape == ((N, D) if out_norm else (0,)) and o32.dtype == torch.float32
        dv, dq, dw, dow = ops.bwd_packed(v, q, w, ow, lse, rstd, o32, y, 2.0 ** -23, 1.0,
                                         out_norm, False)
        assert dv.shape == v.shape and dv.dtype == BF and dq.shape == q.shape
        assert dw.shape == ((R,) if has_w else (0,)) and dow.shape == ((D,) if has_ow else (0,))


def test_list_sources_and_public_wrapper_shapes():
    with FakeTensorMode():
        srcs = [_t(2, 5, 1024) for _ in range(3)]
        q = _t(1024)
        y = A.attnres(srcs, q)
        assert y.shape == (2, 5, 1024)
        flat = [s.reshape(10, 1024) for s in srcs]
        _, lse, rstd, o32 = ops.fwd_list(flat, q, None, None, 1e-6, 1.0, False, False)
        dvs, dq, dw, dow = ops.bwd_list(flat, q, None, None, lse, rstd, o32, y.reshape(10, 1024),
                                        1e-6, 1.0, False, False)
        assert [d.shape for d in dvs] == [f.shape for f in flat] and dq.shape == q.shape


@pytest.mark.parametrize("layout", ["query_major", "token_major"])
def test_multi_query_ops_shapes(layout):
    with FakeTensorMode():
        v = _t(6, 2, 7, 2048)
        qs = _t(3, 256)
        y = A.attnres_multi(v, qs, output_layout=layout)
        assert y.shape == ((3, 2, 7, 2048) if layout == "query_major" else (2, 7, 3, 2048))
        flat = v.reshape(6, 14, 2048)
        yq, lse_q = ops.multi_fwd_packed(flat, qs, 1e-6, 1.0, layout, False)
        dv, dq = ops.multi_bwd_packed(flat, qs, lse_q, yq, 1e-6, 1.0, layout, False)
        assert dv.shape == flat.shape and dq.shape == qs.shape
        y2, lse = ops.multi_fwd_list([_t(14, 2048) for _ in range(6)], qs, 1e-6, 1.0, layout,
                                     False)
        assert lse.shape == ((3, 14) if layout == "query_major" else (14, 3))
        assert lse.dtype == torch.float32


def test_selected_query_ops_shapes():
    with FakeTensorMode():
        v = _t(5, 3, 4, 1024)
        bank = _t(6, 512)
        ids = torch.empty((3, 4, 2), dtype=torch.int64, device="cuda")
        y = A.attnres_selected(v, bank, ids)
        assert y.shape == (3, 4, 2, 1024) and y.dtype == BF
        flat = v.reshape(5, 12, 1024)
        fids = ids.reshape(12, 2)
        yk, lse = ops.selected_fwd_packed(flat, bank, fids, 1e-6, 1.0, False)
        assert yk.shape == (12, 2, 1024) and lse.shape == (12, 2) and lse.dtype == torch.float32
        dv, db = ops.selected_bwd_packed(flat, bank, fids, lse, yk, 1e-6, 1.0, False)
        assert dv.shape == flat.shape and db.shape == bank.shape
        dvs, db2 = ops.selected_bwd_list([flat[s] for s in range(5)], bank, fids, lse, yk, 1e-6,
                                         1.0, False)
        assert [d.shape for d in dvs] == [(12, 1024)] * 5 and db2.shape == bank.shape
        with pytest.raises(ValueError):
            A.attnres_selected(v, bank, torch.empty((3, 2), dtype=torch.int64, device="cuda"))
