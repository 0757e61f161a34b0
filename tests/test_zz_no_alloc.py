"""The allocation-free backward (attnres_bwd_noalloc, include/attnres.h): the library's own device
array instead of a caller workspace. Checked through the C ABI against attnres_bwd on the same
inputs, on two calls in a row (the second smaller, so it reuses the array the first left behind),
and against the FP64 oracle; plus the error return when the partial rows would not fit."""
import pytest
import torch

import attnres_workloads as W
from parity import assert_ok, check_all, gpu_available, inputs_on, run_gpu, run_oracle

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _wl(S, N, D, R, **kw):
    base = W.WORKLOADS["bf16_s10_n32768_d4096"]
    return base.with_(S=S, N=N, D=D, R=R, **kw)


def _noalloc(w, xg):
    import attention_residuals_amd as A
    dev = "cuda"
    y, lse, rstd, o32 = A.attnres_fwd(xg["values"], xg["query"], xg["norm_w"], xg["out_w"],
                                      eps=w.eps, scale=w.scale, out_norm=w.out_norm)
    dv = torch.full_like(xg["values"], float("nan"))
    dq = torch.full((w.R,), float("nan"), dtype=w.torch_dtype, device=dev)
    dw = torch.full_like(dq, float("nan")) if xg["norm_w"] is not None else None
    dow = (torch.full((w.D,), float("nan"), dtype=w.torch_dtype, device=dev)
           if xg["out_w"] is not None else None)
    A.attnres_bwd_noalloc(xg["values"], xg["query"], xg["norm_w"], xg["out_w"], lse, rstd, o32,
                          xg["dout"], eps=w.eps, scale=w.scale, out_norm=w.out_norm, dvalues=dv,
                          dq=dq, dw=dw, dow=dow, deterministic=True)
    torch.cuda.synchronize()
    return {"y": y, "lse": lse, "o_rstd": rstd, "dvalues": dv, "dq": dq, "dw": dw, "dow": dow}


@pytest.mark.parametrize("case", ["twice"])
def test_noalloc_backward_matches_the_workspace_entry_point(case):
    # first call: token-resident backward (exact-bin rows, deterministic: both calls must give the
    # same bits) at the headline width; second, smaller call: streaming backward with the output
    # norm and its weight (dow rows)
    cases = [_wl(10, 4099, 4096, 4096, seed=1901),
             _wl(4, 301, 1024, 1024, out_norm=True, out_weight=True, norm_weight=False,
                 seed=1902)]
    for w in cases:
        print(f"[case] noalloc S={w.S} N={w.N} D={w.D} out_norm={w.out_norm}", flush=True)
        xc = W.generate(w)
        xg = inputs_on(xc, "cuda")
        ref = run_gpu(w, xg, poison=False, deterministic=True)
        got = _noalloc(w, xg)
        for k in ("dvalues", "dq", "dw", "dow"):
            if ref.get(k) is not None:
                assert torch.equal(ref[k], got[k]), k
        assert_ok(check_all(w, got, run_oracle(w, xc)), f"noalloc S={w.S} N={w.N}")


def test_noalloc_rejects_rows_beyond_its_array():
    # D = 16384 keeps one workgroup per CU resident; its exact-bin rows (16384 x 16 bytes each)
    # need more than the 64 MiB array, so the call fails before launching anything
    import attention_residuals_amd as A
    w = _wl(2, 600, 16384, 16384, seed=1903)
    need = A.workspace_bytes(A.make_desc(w.S, w.N, w.D, w.R, w.torch_dtype, has_norm_weight=True,
                                         deterministic=True))
    if need <= 64 << 20:
        pytest.skip(f"this device's backward grid fits the array ({need} bytes)")
    xg = inputs_on(W.generate(w), "cuda")
    y, lse, _, _ = A.attnres_fwd(xg["values"], xg["query"], xg["norm_w"], None)
    dv = torch.full_like(xg["values"], 7.0)
    with pytest.raises(A.AttnResError) as e:
        A.attnres_bwd_noalloc(xg["values"], xg["query"], xg["norm_w"], None, lse, None, None,
                              xg["dout"], dvalues=dv, deterministic=True)
    assert e.value.status == 4  # ATTNRES_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(dv == 7.0)
