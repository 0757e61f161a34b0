"""GPU parity of the multi-query read ("Fast Attention Residuals" PyPI page, Multi-query AttnRes)
against the FP64 multi-query oracle, through the C ABI.

Tolerances are the single-query read's (tests/parity.py), applied to every query's output rows,
to dvalues (summed over the queries), and per query to dq_m (relative L2 for bf16).
Covered: M = 1 (served by the single-query kernels), 2, 3 (a padded group of four), 4, 5 and 16
(several groups: later groups accumulate into dvalues), both output layouts, sliced keys, bf16 and
FP32, accumulation into existing dvalues, the widest rows (two query groups per launch), list
sources, ragged token counts, several tokens per workgroup in both schedules, determinism and the
static schedule, the autograd wrapper, N = 0, and the unsupported (non-resident) shapes.
"""
import math

import numpy as np
import pytest
import torch

import attnres_workloads as W
import oracle
from parity import (TOL_F32, assert_ok, compare_rows, compare_stat, compare_vec, gpu_available,
                    half_ulp_bf16, multi_bwd_groups, tile_fwd, to_f64)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _inputs(S, N, D, R, M, dtype, seed, device="cpu"):
    return W.multi_case(S, N, D, R, M, dtype, seed, device)   # dY query-major


def _to_layout(x, layout):
    """[M, N, ...] query-major -> the layout's order."""
    return x.contiguous() if layout == "query_major" else x.transpose(0, 1).contiguous()


def _from_layout(x, layout):
    return x if layout == "query_major" else x.transpose(0, 1)


def _run(V, Q, G, layout="query_major", dvalues=None, accumulate=False, deterministic=False,
         dynamic=True, packed=True):
    import attention_residuals_amd as A
    vals = V if packed else [V[s] for s in range(V.shape[0])]
    y, lse = A.attnres_multi_fwd(vals, Q, layout=layout, dynamic=dynamic)
    dv, dq = A.attnres_multi_bwd(vals, Q, lse, _to_layout(G, layout), layout=layout,
                                 deterministic=deterministic, accumulate=accumulate,
                                 dvalues=dvalues)
    torch.cuda.synchronize()
    dv = torch.stack(dv) if isinstance(dv, list) else dv
    return _from_layout(y, layout), _from_layout(lse, layout), dv, dq


def _bwd_groups(S, D, M, dtype, R=None):
    """The backward's launch groups (first query, count), as the library plans them."""
    return multi_bwd_groups(S, D, M, dtype, R=R)


def _dvalues_slack(V, Q, G, init, groups):
    """Rounding allowance of dvalues built group by group, each launch rounding the running sum to
    bf16: half an ulp of every running sum (from the oracle's per-group contributions)."""
    partial = np.zeros((V.shape[0], V.shape[1], V.shape[2])) if init is None else \
        init.double().numpy().copy()
    slack = np.zeros_like(partial)
    for m0, cnt in groups:
        partial += oracle.run_multi(V, Q[m0:m0 + cnt], G[m0:m0 + cnt], want=("dvalues",),
                                    reduce=False)["dvalues"]
        slack += half_ulp_bf16(partial)
    return slack


def _check(V, Q, G, label, dtype, init=None, f32_tol=None, **kw):
    Vg, Qg, Gg = V.cuda(), Q.cuda(), G.cuda()
    dvalues = None
    if init is not None:
        dvalues = init.cuda()
        if not kw.get("packed", True):
            dvalues = [dvalues[s].clone() for s in range(V.shape[0])]
    y, lse, dv, dq = _run(Vg, Qg, Gg, dvalues=dvalues, **kw)
    ref = oracle.run_multi(V, Q, G)
    if init is not None:
        ref["dvalues"] = ref["dvalues"] + init.double().numpy()
    M = Q.shape[0]
    res = {}
    res["y"] = compare_rows(to_f64(y).reshape(-1, V.shape[2]), ref["y"].reshape(-1, V.shape[2]),
                            dtype)
    res["lse"] = compare_stat(to_f64(lse), ref["lse"])
    S, D = V.shape[0], V.shape[2]
    groups = _bwd_groups(S, D, M, dtype, Q.shape[1])
    slack = (_dvalues_slack(V, Q, G, init, groups)
             if dtype == "bf16" and (len(groups) > 1 or init is not None) else None)
    res["dvalues"] = compare_rows(to_f64(dv), ref["dvalues"], dtype, slack=slack,
                                  f32_tol=f32_tol)
    for m in range(M):
        res[f"dq{m}"] = compare_vec(to_f64(dq[m]), ref["dq"][m], dtype)
    assert_ok(res, label)
    return y, lse, dv, dq


@pytest.mark.parametrize("S,N,D,R,M,dtype,layout", [
    (10, 701, 4096, 4096, 2, "bf16", "query_major"),
    (8, 513, 2048, 512, 3, "bf16", "token_major"),
    (6, 257, 1024, 1024, 4, "bf16", "query_major"),
    (5, 300, 2048, 2048, 5, "bf16", "token_major"),
    (4, 129, 256, 256, 16, "f32", "query_major"),
    (5, 333, 1024, 1024, 1, "bf16", "token_major"),
    (4, 211, 8192, 8192, 4, "bf16", "query_major"),
    (24, 199, 2048, 640, 2, "bf16", "query_major"),
    # FP32 with a 3-wide key over 1024 columns: held to the FP32 floor of these inputs (a plain
    # FP32 evaluation's error, tests/test_fp32_floor.py), which exceeds the literal 1e-5 bound
    (3, 97, 1024, 3, 3, "f32", "token_major"),
    # bf16 with three or more queries, S <= 16 and D <= 4096: the matrix-core forward (one pass)
    (10, 333, 4096, 4096, 8, "bf16", "token_major"),
    (16, 129, 1024, 1024, 16, "bf16", "query_major"),
    (6, 211, 1032, 1032, 3, "bf16", "query_major"),    # ragged last column group
    (12, 157, 3072, 768, 5, "bf16", "token_major"),    # sliced key, three column groups
    (2, 300, 2048, 7, 4, "bf16", "query_major"),        # slice start inside a chunk
    (10, 257, 4096, 4096, 16, "bf16", "token_major"),  # the largest staged-query LDS (~145 KiB)
    # more than twelve sources with up to four queries: the matrix-core backward that sums dq in
    # its own LDS (no second pass over the sources)
    (14, 300, 2048, 2048, 4, "bf16", "token_major"),
    (16, 201, 1024, 512, 3, "bf16", "query_major"),
    (13, 150, 3072, 3072, 3, "bf16", "query_major"),   # separate tiles, S + M = 16, dq in LDS
    # sources and dY rows in one tile (S + M <= 16), five to eight queries with dq summed in LDS
    (10, 257, 4096, 4096, 6, "bf16", "query_major"),   # the largest that fits (~155 KiB)
    (8, 300, 2048, 2048, 8, "bf16", "token_major"),
    (11, 211, 3072, 1024, 5, "bf16", "token_major"),   # sliced key
    (9, 211, 2048, 2048, 7, "bf16", "query_major"),    # second group of four cut after three
    # sources and dY rows in one tile (S + M <= 16) with dq formed by the dq kernel
    (9, 257, 4096, 1024, 7, "bf16", "query_major"),    # sliced key, sixteen rows
    (4, 300, 1024, 1024, 12, "bf16", "token_major"),
    (2, 199, 3072, 3072, 14, "bf16", "query_major"),
])
def test_multi_query_parity(S, N, D, R, M, dtype, layout):
    V, Q, G = _inputs(S, N, D, R, M, dtype, seed=2000 + S * M + D)
    print(f"[case] S={S} N={N} D={D} R={R} M={M} {dtype} {layout}", flush=True)
    f32_tol = None
    if dtype == "f32" and R < 8:
        from fp32_floor import fp32_floor
        floor = fp32_floor(V.numpy(), Q.numpy(), G.numpy(), oracle.run_multi(V, Q, G)["dvalues"])
        f32_tol = max(TOL_F32, floor)
    _check(V, Q, G, f"multi S={S} N={N} D={D} R={R} M={M} {dtype} {layout}", dtype,
           layout=layout, f32_tol=f32_tol)


@pytest.mark.parametrize("M,dynamic", [(2, False), (2, True), (4, False), (4, True), (6, False),
                                       (6, True)])
def test_multi_query_several_tokens_per_workgroup(M, dynamic):
    # enough tokens that every workgroup of the forward's grid (static: 8x the resident count;
    # dynamic: one resident pass taking tickets) and of the backward's reads several, so the
    # one-token-ahead prefetch and the token loop are checked against the oracle, not only the
    # first token of each workgroup
    S, N, D, R = 6, 9001, 2048, 2048
    V, Q, G = _inputs(S, N, D, R, M, "bf16", seed=2050 + M)
    print(f"[case] multi several tokens per workgroup M={M} dynamic={dynamic}", flush=True)
    _check(V, Q, G, f"multi N={N} M={M} dynamic={dynamic}", "bf16", dynamic=dynamic,
           deterministic=not dynamic)


# (6, 6) and (10, 6) at D = 4096: the compact tile summing dq in LDS beside the accumulated rows;
# (14, 3) as a list: the separate tiles' whole-line dv stores into separate allocations
@pytest.mark.parametrize("S,M,packed,D", [(6, 2, True, 2048), (6, 6, False, 2048),
                                          (14, 3, True, 2048), (10, 6, True, 4096),
                                          (14, 3, False, 2048)])
def test_multi_query_accumulate_into_dvalues(S, M, packed, D):
    N, R = 301, D
    V, Q, G = _inputs(S, N, D, R, M, "bf16", seed=2100 + M)
    init = (2.0 * torch.randn((S, N, D), generator=torch.Generator().manual_seed(5))).to(V.dtype)
    _check(V, Q, G, f"multi accumulate M={M}", "bf16", init=init, accumulate=True, packed=packed)


@pytest.mark.parametrize("S,M", [(6, 4), (10, 12), (16, 9)])
def test_separate_tiles_with_list_sources(S, M):
    # the separate-tile backward (M <= 4, or S + M > 16) with sources as a list: each lane's two
    # whole-line dv stores pick their rows' allocations from the pointer table
    N, D, R = 301, 2048, 2048
    V, Q, G = _inputs(S, N, D, R, M, "bf16", seed=2150 + S * M)
    print(f"[case] separate tiles, list sources S={S} M={M}", flush=True)
    _check(V, Q, G, f"multi list S={S} M={M}", "bf16", packed=False)


@pytest.mark.parametrize("S,N,D,R,M", [(10, 3001, 4096, 4096, 4), (5, 999, 2048, 640, 11)])
def test_matrix_core_forward_matches_the_vector_kernels(S, N, D, R, M, monkeypatch):
    # the one-pass matrix-core forward and the query-group vector kernels (ATTNRES_MULTI_MFMA=0)
    # agree to one bf16 ulp plus the matrix-core path's weight rounding (p as two bf16 terms:
    # relative error <= 2^-18 of sum_s p_s |v_s|); both are compared with the oracle elsewhere
    import attention_residuals_amd as A
    V, Q, _ = (t.cuda() for t in _inputs(S, N, D, R, M, "bf16", seed=2250 + M))
    y1, l1 = A.attnres_multi_fwd(V, Q)
    monkeypatch.setenv("ATTNRES_MULTI_MFMA", "0")
    y0, l0 = A.attnres_multi_fwd(V, Q)
    torch.cuda.synchronize()
    a, b = to_f64(y0), to_f64(y1)
    ulp = 2.0 * half_ulp_bf16(np.maximum(np.abs(a), np.abs(b)))
    assert np.all(np.abs(a - b) <= ulp + 2e-5 * np.sqrt(np.mean(a * a)))
    assert np.max(np.abs(to_f64(l0) - to_f64(l1))) <= 1e-5 * (1 + np.max(np.abs(to_f64(l0))))


@pytest.mark.parametrize("D", [1544, 2048])
@pytest.mark.parametrize("case", ["one_token", "three_tokens", "list_sources", "strided_rows"])
def test_matrix_core_forward_edges(case, D):
    # the matrix-core forward (bf16, 3 <= M <= 16) with fewer tokens than workgroups, sources as a
    # list of separate allocations, and rows further apart than D (a view into wider rows); at
    # D = 2048 the backward runs on matrix cores too
    import attention_residuals_amd as A
    S, R, M = 7, D, 6
    N = {"one_token": 1, "three_tokens": 3}.get(case, 301)
    V, Q, G = _inputs(S, N, D, R, M, "bf16", seed=2400 + N)
    print(f"[case] matrix-core forward {case} D={D}", flush=True)
    if case == "list_sources":
        vals = [V[s].clone().cuda() for s in range(S)]
    elif case == "strided_rows":
        wide = torch.zeros((S, N, D + 72), dtype=V.dtype, device="cuda")
        wide[:, :, :D] = V.cuda()
        vals = wide[:, :, :D]
        assert vals.stride(1) == D + 72
    else:
        vals = V.cuda()
    y, lse = A.attnres_multi_fwd(vals, Q.cuda())
    dv, dq = A.attnres_multi_bwd(vals, Q.cuda(), lse, G.cuda())
    torch.cuda.synchronize()
    dv = torch.stack(dv) if isinstance(dv, list) else dv
    ref = oracle.run_multi(V, Q, G)
    res = {"y": compare_rows(to_f64(y).reshape(-1, D), ref["y"].reshape(-1, D), "bf16"),
           "lse": compare_stat(to_f64(lse), ref["lse"]),
           "dvalues": compare_rows(to_f64(dv), ref["dvalues"], "bf16",
                                   slack=_dvalues_slack(V, Q, G, None,
                                                        _bwd_groups(S, D, M, "bf16", Q.shape[1])))}
    for m in range(M):
        res[f"dq{m}"] = compare_vec(to_f64(dq[m]), ref["dq"][m], "bf16")
    assert_ok(res, f"matrix-core forward {case}")


def test_multi_query_schedules_and_determinism():
    S, N, D, R, M = 10, 3001, 4096, 4096, 2
    V, Q, G = (t.cuda() for t in _inputs(S, N, D, R, M, "bf16", seed=2200))
    det1 = _run(V, Q, G, deterministic=True, dynamic=False)
    det2 = _run(V, Q, G, deterministic=True, dynamic=False)
    dyn = _run(V, Q, G)
    for a, b in zip(det1, det2):
        assert torch.equal(a, b)
    for k in range(3):  # y, lse, dvalues: per token, independent of the schedule
        assert torch.equal(det1[k], dyn[k])
    a, b = to_f64(det1[3]), to_f64(dyn[3])
    assert np.linalg.norm(a - b) <= 4e-3 * np.linalg.norm(a)


def test_multi_query_autograd_wrapper():
    import attention_residuals_amd as A
    S, N, D, R, M = 4, 2 * 37, 1024, 256, 3
    V, Q, G = _inputs(S, N, D, R, M, "bf16", seed=2300)
    v = V.cuda().view(S, 2, 37, D).clone().requires_grad_(True)
    q = Q.cuda().clone().requires_grad_(True)
    y = A.attnres_multi(v, q, output_layout="token_major")
    assert y.shape == (2, 37, M, D)
    y.backward(G.cuda().permute(1, 0, 2).reshape(2, 37, M, D))
    ref = oracle.run_multi(V, Q, G)
    got_y = to_f64(y.detach().reshape(N, M, D)).transpose(1, 0, 2)
    assert compare_rows(got_y.reshape(-1, D), ref["y"].reshape(-1, D), "bf16")["ok"]
    assert compare_rows(to_f64(v.grad.reshape(S, N, D)), ref["dvalues"], "bf16")["ok"]
    for m in range(M):
        assert compare_vec(to_f64(q.grad[m]), ref["dq"][m], "bf16")["ok"]


def test_multi_query_zero_tokens_and_unsupported_shape():
    import attention_residuals_amd as A
    V = torch.empty((3, 0, 256), dtype=torch.bfloat16, device="cuda")
    Q = torch.randn((2, 256), device="cuda").to(torch.bfloat16)
    y, lse = A.attnres_multi_fwd(V, Q)
    dv, dq = A.attnres_multi_bwd(V, Q, lse, torch.empty((2, 0, 256), dtype=torch.bfloat16,
                                                         device="cuda"))
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.all(dq == 0)
    big = torch.empty((64, 4, 8192), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(A.AttnResError) as e:
        A.attnres_multi_fwd(big, torch.zeros((2, 8192), dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == 2



def _fwd_counter_case(fwd, ref, N, label, uses_counter):
    """Runs the forward `fwd(dynamic, workspace)` with a workspace (poisoned) and without one
    (static stride): outputs must agree bit for bit (per-token results do not depend on which
    workgroup ran the token) and match the oracle. Sixteen-slot kernels take their tokens from the
    workspace's counter (reset, then one ticket per batch: at most N); the others leave it alone."""
    ws = torch.full((256,), 0xFF, dtype=torch.uint8, device="cuda")
    y_d, lse_d = fwd(True, ws)
    y_s, lse_s = fwd(False, None)
    torch.cuda.synchronize()
    tickets = int(ws[:4].cpu().view(torch.int32).item())
    if uses_counter:
        assert 0 < tickets <= N, f"{label}: token counter not used ({tickets})"
    else:
        assert tickets == -1, f"{label}: token counter touched ({tickets})"
    assert torch.equal(y_d, y_s) and torch.equal(lse_d, lse_s), label
    D = y_d.shape[-1]
    res = {"y": compare_rows(to_f64(y_d).reshape(-1, D), ref["y"].reshape(-1, D), "bf16"),
           "lse": compare_stat(to_f64(lse_d).reshape(-1), ref["lse"].reshape(-1))}
    assert_ok(res, label)


@pytest.mark.parametrize("M,S,D,R,layout", [
    (16, 10, 1280, 1280, "query_major"),  # older forward, sixteen slots: rows loaded in place
    (12, 7, 2560, 768, "token_major"),    # older forward, padded to sixteen slots, sliced key
    (4, 10, 1280, 1280, "token_major"),   # older forward, four slots: static stride
    (16, 10, 1024, 1024, "query_major"),  # tile forward: static stride, workspace untouched
    (12, 7, 3072, 768, "token_major"),    # tile forward, sliced key
])
def test_matrix_core_forward_token_counter(M, S, D, R, layout):
    # enough tokens for at least two per resident workgroup, so the counter schedule runs
    import attention_residuals_amd as A
    N = 2 * 4 * 256 + 37
    print(f"[case] matrix-core forward counter M={M} S={S} D={D} R={R} {layout} N={N}", flush=True)
    V, Q, _ = _inputs(S, N, D, R, M, "bf16", seed=4100 + M)
    Vg, Qg = V.cuda(), Q.cuda()

    def fwd(dynamic, ws):
        y, lse = A.attnres_multi_fwd(Vg, Qg, layout=layout, dynamic=dynamic, workspace=ws)
        return _from_layout(y, layout), _from_layout(lse, layout)

    ref = oracle.run_multi(V, Q, want=("y", "lse"))
    _fwd_counter_case(fwd, ref, N, f"matrix-core forward counter M={M} {layout}",
                      M > 8 and not tile_fwd(S, D, M, "bf16", R=R))


@pytest.mark.parametrize("D", [1280, 1024])  # older forward (counter), tile forward (none)
def test_matrix_core_selected_forward_token_counter(D):
    import attention_residuals_amd as A
    S, N, E, K = 10, 2 * 4 * 256 + 37, 8, 12
    print(f"[case] matrix-core selected forward counter E={E} K={K} N={N}", flush=True)
    g = torch.Generator().manual_seed(4200)
    V = torch.randn((S, N, D), generator=g).to(torch.bfloat16)
    bank = (torch.randn((E, D), generator=g) / math.sqrt(D)).to(torch.bfloat16)
    ids = torch.randint(0, E, (N, K), generator=g, dtype=torch.int64)
    Vg, bg, ig = V.cuda(), bank.cuda(), ids.cuda()

    def fwd(dynamic, ws):
        return A.attnres_selected_fwd(Vg, bg, ig, dynamic=dynamic, workspace=ws)

    ref = oracle.run_selected(V, bank, ids, want=("y", "lse"))
    _fwd_counter_case(fwd, ref, N, f"matrix-core selected forward counter D={D}",
                      not tile_fwd(S, D, K, "bf16", E=E))
