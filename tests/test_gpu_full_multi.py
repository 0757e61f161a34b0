"""Full-size GPU parity of the multi-query and selected-query reads ("Fast Attention Residuals"
PyPI page, Multi-query AttnRes) against the FP64 oracles, through the C ABI, in the launch
configuration the benchmark times (`bench.py --queries M`, `--bank E --slots K`): the sources of the
S=10, N=32768, D=4096 bf16 workload, dynamic token schedules, inputs drawn by the same generators.

Sampled tokens' output rows, lse and dvalues rows are compared one by one with the oracle; dq (per
query) and dbank (per bank row) against the oracle's reduction over all N tokens. Tolerances as in
tests/parity.py; dvalues carry one bf16 rounding per backward launch group.
"""
import numpy as np
import pytest
import torch

import attnres_workloads as W
import oracle
from parity import (assert_ok, compare_rows, compare_stat, compare_vec, gpu_available,
                    multi_bwd_passes, sample_tokens, to_f64)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

HEADLINE = W.ALL[W.HEADLINE]


def _groups(w, M, selected, E=None):
    return multi_bwd_passes(w.S, w.D, M, w.dtype, selected, R=w.R, E=E)


# M = 2: the query-group kernels; M = 4: the separate-tile matrix-core backward with dq summed in
# LDS; M = 6: the compact one (sources and dY rows in one tile, dq summed in LDS); M = 8: the
# separate-tile backward and its dq pass
@pytest.mark.parametrize("M,layout", [(2, "query_major"), (4, "token_major"), (6, "query_major"),
                                      (8, "token_major")])
def test_multi_query_full_size(M, layout):
    import attention_residuals_amd as A
    w = HEADLINE
    print(f"[case] full multi M={M} {layout}", flush=True)
    values = W.generate(w, device="cuda", with_dout=False)["values"]
    mi = W.multi_inputs(w, M, layout, device="cuda")
    q, g = mi["queries"], mi["dout"]
    y, lse = A.attnres_multi_fwd(values, q, eps=w.eps, scale=w.scale, layout=layout)
    dv, dq = A.attnres_multi_bwd(values, q, lse, g, eps=w.eps, scale=w.scale, layout=layout)
    torch.cuda.synchronize()
    toks = sample_tokens(w.N, 24, seed=w.seed + M)
    sel = torch.tensor(toks, device="cuda")
    gq = g if layout == "query_major" else g.transpose(0, 1)
    yq = y if layout == "query_major" else y.transpose(0, 1)
    lq = lse if layout == "query_major" else lse.transpose(0, 1)
    vc, qc, gc = values.cpu(), q.cpu(), gq.contiguous().cpu()
    ref = oracle.run_multi(vc, qc, gc, eps=w.eps, scale=w.scale, tokens=toks, reduce=False)
    red = oracle.run_multi(vc, qc, gc, eps=w.eps, scale=w.scale, want=(), reduce=True)
    res = {"y": compare_rows(to_f64(yq.index_select(1, sel)).reshape(-1, w.D),
                             ref["y"].reshape(-1, w.D), w.dtype),
           "lse": compare_stat(to_f64(lq.index_select(1, sel)), ref["lse"]),
           "dvalues": compare_rows(to_f64(dv.index_select(1, sel)), ref["dvalues"], w.dtype,
                                   roundings=_groups(w, M, False))}
    for m in range(M):
        res[f"dq{m}"] = compare_vec(to_f64(dq[m]), red["dq"][m], w.dtype)
    assert_ok(res, f"full multi M={M} {layout}")
    del values, mi, y, lse, dv
    torch.cuda.empty_cache()


def test_multi_query_full_size_forward_sixteen_slots():
    # the sixteen-query tile forward (sixteen staged rows, static stride), as
    # `bench.py --queries 16` runs it (outputs and lse of sampled tokens)
    import attention_residuals_amd as A
    w, M, layout = HEADLINE, 16, "query_major"
    print(f"[case] full multi forward M={M} {layout}", flush=True)
    values = W.generate(w, device="cuda", with_dout=False)["values"]
    q = W.multi_inputs(w, M, layout, device="cuda")["queries"]
    y, lse = A.attnres_multi_fwd(values, q, eps=w.eps, scale=w.scale, layout=layout)
    torch.cuda.synchronize()
    toks = sample_tokens(w.N, 24, seed=w.seed + M)
    sel = torch.tensor(toks, device="cuda")
    ref = oracle.run_multi(values.cpu(), q.cpu(), eps=w.eps, scale=w.scale, tokens=toks,
                           want=("y", "lse"), reduce=False)
    res = {"y": compare_rows(to_f64(y.index_select(1, sel)).reshape(-1, w.D),
                             ref["y"].reshape(-1, w.D), w.dtype),
           "lse": compare_stat(to_f64(lse.index_select(1, sel)), ref["lse"])}
    assert_ok(res, f"full multi forward M={M} {layout}")
    del values, y, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("E,K", [(8, 2), (8, 4), (8, 8)])  # slot groups, compact tile, separate tiles
def test_selected_query_full_size(E, K):
    import attention_residuals_amd as A
    w = HEADLINE
    print(f"[case] full selected E={E} K={K}", flush=True)
    values = W.generate(w, device="cuda", with_dout=False)["values"]
    si = W.selected_inputs(w, E, K, device="cuda")
    bank, ids, g = si["bank"], si["ids"], si["dout"]
    y, lse = A.attnres_selected_fwd(values, bank, ids, eps=w.eps, scale=w.scale)
    dv, db = A.attnres_selected_bwd(values, bank, ids, lse, g, eps=w.eps, scale=w.scale)
    torch.cuda.synchronize()
    toks = sample_tokens(w.N, 24, seed=w.seed + K)
    sel = torch.tensor(toks, device="cuda")
    vc, bc, ic, gc = values.cpu(), bank.cpu(), ids.cpu(), g.cpu()
    ref = oracle.run_selected(vc, bc, ic, gc, eps=w.eps, scale=w.scale, tokens=toks, reduce=False)
    red = oracle.run_selected(vc, bc, ic, gc, eps=w.eps, scale=w.scale, want=(), reduce=True)
    res = {"y": compare_rows(to_f64(y.index_select(0, sel)).reshape(-1, w.D),
                             ref["y"].reshape(-1, w.D), w.dtype),
           "lse": compare_stat(to_f64(lse.index_select(0, sel)), ref["lse"]),
           "dvalues": compare_rows(to_f64(dv.index_select(1, sel)), ref["dvalues"], w.dtype,
                                   roundings=_groups(w, K, True, E))}
    got_b = to_f64(db)
    for e in range(E):
        if not np.any(red["dbank"][e]):
            assert np.all(got_b[e] == 0), f"bank row {e} was selected by no token but is nonzero"
            continue
        res[f"dbank{e}"] = compare_vec(got_b[e], red["dbank"][e], w.dtype)
    assert_ok(res, f"full selected E={E} K={K}")
    del values, si, y, lse, dv
    torch.cuda.empty_cache()
