"""torch.compile(fullgraph=True) over the AttnRes reads (the "Fast Attention Residuals" page's
Quickstart uses the read this way, and its "Validation scope" checks compiled use against an
independent reference): the custom operators trace as single nodes, compiled forward + backward
equal eager bit for bit, and the compiled outputs and gradients match the FP64 oracle on the same
inputs. torch.library.opcheck validates the registrations (schema, fake implementations, autograd)
on small inputs."""
import numpy as np
import pytest
import torch

import attnres_workloads as W
import oracle
from parity import (assert_ok, compare_rows, compare_stat, compare_vec, gpu_available,
                    multi_bwd_passes, to_f64)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _step(read, values, query, weight, dy):
    y = read(values, query, weight)
    return (y.float() * dy.float()).sum()


def _inputs(seed, S=6, N=2 * 129, D=1024, R=512):
    w = W.Workload("compile", S=S, N=N, D=D, R=R, dtype="bf16", norm_weight=True, out_norm=False,
                   out_weight=False, seed=seed)
    return W.generate(w, device="cuda")


def _grads(fn, x, as_list):
    v = x["values"].clone().requires_grad_(True)
    q = x["query"].clone().requires_grad_(True)
    wt = x["norm_w"].clone().requires_grad_(True)
    vals = list(v.unbind(0)) if as_list else v
    loss = fn(vals, q, wt, x["dout"])
    loss.backward()
    return loss.detach(), v.grad, q.grad, wt.grad


@pytest.mark.parametrize("backend", ["aot_eager", "inductor"])
@pytest.mark.parametrize("as_list", [False, True])
def test_compiled_read_matches_eager(backend, as_list):
    import attention_residuals_amd as A
    if backend == "inductor":
        pytest.importorskip("triton")
    torch._dynamo.reset()
    x = _inputs(3100)

    def read(values, query, weight):
        return A.attnres(values, query, norm_weight=weight, deterministic=True)

    def step(values, query, weight, dy):
        return _step(read, values, query, weight, dy)

    eager = _grads(step, x, as_list)
    compiled = _grads(torch.compile(step, fullgraph=True, dynamic=False, backend=backend), x,
                      as_list)
    # the loss is a float sum the compiler may reorder; the gradients pass through the read's
    # kernels unchanged and must match bit for bit
    torch.testing.assert_close(eager[0], compiled[0], rtol=1e-5, atol=0)
    for a, b in zip(eager[1:], compiled[1:]):
        assert torch.equal(a, b)
    # and against the oracle: the compiled forward's output, and the compiled gradients of
    # sum(y * dy) (dL/dy = dy)
    y = torch.compile(read, fullgraph=True, dynamic=False, backend=backend)(
        list(x["values"].unbind(0)) if as_list else x["values"], x["query"], x["norm_w"])
    xc = {k: v.cpu() for k, v in x.items() if v is not None}
    ref = oracle.run(xc["values"], xc["query"], xc["norm_w"], None, xc["dout"])
    D = x["values"].shape[2]
    res = {"y": compare_rows(to_f64(y), ref["y"], "bf16"),
           "dvalues": compare_rows(to_f64(compiled[1]), ref["dvalues"], "bf16"),
           "dq": compare_vec(to_f64(compiled[2]), ref["dq"], "bf16"),
           "dw": compare_vec(to_f64(compiled[3]), ref["dw"], "bf16")}
    assert_ok(res, f"compiled read {backend} list={as_list} D={D}")


def test_compiled_multi_query_read_matches_eager():
    import attention_residuals_amd as A
    torch._dynamo.reset()
    x = _inputs(3200, S=5, D=2048, R=2048)
    qs = torch.randn((2, 2048), device="cuda").to(torch.bfloat16)
    dy = torch.randn((2, x["values"].shape[1], 2048), device="cuda").to(torch.bfloat16)

    def step(values, queries):
        return (A.attnres_multi(values, queries, deterministic=True).float() * dy.float()).sum()

    def grads(fn):
        v = x["values"].clone().requires_grad_(True)
        q = qs.clone().requires_grad_(True)
        loss = fn(v, q)
        loss.backward()
        return loss.detach(), v.grad, q.grad

    eager = grads(step)
    compiled = grads(torch.compile(step, fullgraph=True, dynamic=False, backend="aot_eager"))
    torch.testing.assert_close(eager[0], compiled[0], rtol=1e-5, atol=0)
    for a, b in zip(eager[1:], compiled[1:]):
        assert torch.equal(a, b)
    y = torch.compile(lambda v, q: A.attnres_multi(v, q, deterministic=True), fullgraph=True,
                      dynamic=False, backend="aot_eager")(x["values"], qs)
    V = x["values"].cpu()
    ref = oracle.run_multi(V, qs.cpu(), dy.cpu())
    S, D = V.shape[0], V.shape[2]
    res = {"y": compare_rows(to_f64(y).reshape(-1, D), ref["y"].reshape(-1, D), "bf16"),
           "dvalues": compare_rows(to_f64(compiled[1]), ref["dvalues"], "bf16",
                                   roundings=multi_bwd_passes(S, D, qs.shape[0], "bf16"))}
    for m in range(qs.shape[0]):
        res[f"dq{m}"] = compare_vec(to_f64(compiled[2][m]), ref["dq"][m], "bf16")
    assert_ok(res, "compiled multi-query read")


@pytest.mark.parametrize("as_list", [False, True])
def test_compiled_selected_query_read_matches_eager(as_list):
    import attention_residuals_amd as A
    torch._dynamo.reset()
    x = _inputs(3250, S=5, D=2048, R=2048)
    N = x["values"].shape[1]
    g = torch.Generator(device="cuda").manual_seed(3251)
    bank = torch.randn((7, 2048), generator=g, device="cuda").to(torch.bfloat16)
    ids = torch.randint(0, 7, (2, N // 2, 3), generator=g, device="cuda", dtype=torch.int64)
    dy = torch.randn((2, N // 2, 3, 2048), generator=g, device="cuda").to(torch.bfloat16)

    def step(values, b):
        y = A.attnres_selected(values, b, ids, deterministic=True)
        return (y.float() * dy.float()).sum()

    def grads(fn):
        v = x["values"].view(5, 2, N // 2, 2048).clone().requires_grad_(True)
        b = bank.clone().requires_grad_(True)
        loss = fn(list(v.unbind(0)) if as_list else v, b)
        loss.backward()
        return loss.detach(), v.grad, b.grad

    eager = grads(step)
    compiled = grads(torch.compile(step, fullgraph=True, dynamic=False, backend="aot_eager"))
    torch.testing.assert_close(eager[0], compiled[0], rtol=1e-5, atol=0)
    for a, b in zip(eager[1:], compiled[1:]):
        assert torch.equal(a, b)
    vals = x["values"].view(5, 2, N // 2, 2048)
    y = torch.compile(lambda v, b: A.attnres_selected(v, b, ids, deterministic=True),
                      fullgraph=True, dynamic=False, backend="aot_eager")(
        list(vals.unbind(0)) if as_list else vals, bank)
    K = ids.shape[-1]
    ref = oracle.run_selected(x["values"].cpu(), bank.cpu(), ids.reshape(N, K).cpu(),
                              dy.reshape(N, K, 2048).cpu())
    res = {"y": compare_rows(to_f64(y).reshape(-1, 2048), ref["y"].reshape(-1, 2048), "bf16"),
           "dvalues": compare_rows(to_f64(compiled[1]).reshape(5, N, 2048), ref["dvalues"],
                                   "bf16",
                                   roundings=multi_bwd_passes(5, 2048, K, "bf16", selected=True,
                                                              E=7)),
           "dbank": compare_vec(to_f64(compiled[2]), ref["dbank"], "bf16")}
    assert_ok(res, f"compiled selected-query read list={as_list}")


def test_opcheck_registrations():
    from attention_residuals_amd import ops
    x = _inputs(3300, S=4, N=67, D=256, R=256)
    v = x["values"].requires_grad_(True)
    q = x["query"].requires_grad_(True)
    w = x["norm_w"].requires_grad_(True)
    torch.library.opcheck(ops.fwd_packed, (v, q, w, None, 2.0 ** -23, 1.0, False, True))
    srcs = [t.detach().clone().requires_grad_(True) for t in x["values"].unbind(0)]
    torch.library.opcheck(ops.fwd_list, (srcs, q, None, None, 2.0 ** -23, 1.0, False, True))
    qs = torch.randn((3, 256), device="cuda").to(torch.bfloat16).requires_grad_(True)
    torch.library.opcheck(ops.multi_fwd_packed, (v, qs, 2.0 ** -23, 1.0, "token_major", True))
    bank = torch.randn((5, 256), device="cuda").to(torch.bfloat16).requires_grad_(True)
    ids = torch.randint(0, 5, (67, 3), device="cuda", dtype=torch.int64)
    torch.library.opcheck(ops.selected_fwd_packed, (v, bank, ids, 2.0 ** -23, 1.0, True))
    torch.library.opcheck(ops.selected_fwd_list, (srcs, bank, ids, 2.0 ** -23, 1.0, True))
