"""HIP graph capture and replay of the multi-query and selected-query reads (several launch groups:
ticket resets, accumulating later groups, the finaliser). Each read is captured once into a
torch.cuda.CUDAGraph with preallocated outputs and workspaces, then replayed four times on inputs
copied into the captured buffers (alternating two input sets), with eager work and synchronisation
between replays; every replay is compared with an eager call on the same inputs: bitwise for y,
lse and dvalues (per-token results), and bitwise for dq / dbank in deterministic mode (else to the
reduction-order tolerance of the schedules test). Every replay is also compared with the FP64
oracle on the inputs copied in for it (the "Fast Attention Residuals" page, "Validation scope":
replayed use checked against an independent reference)."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import (assert_ok, compare_rows, compare_stat, compare_vec, gpu_available,
                    multi_bwd_passes, to_f64)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _sources(S, N, D, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    V = torch.empty((S, N, D), dtype=torch.bfloat16, device="cuda")
    for s in range(S):
        V[s].copy_(torch.randn((N, D), generator=g, device="cuda") * math.sqrt(1.0 + s))
    return V, g


def _close(a, b, deterministic):
    if deterministic:
        assert torch.equal(a, b)
    else:
        x, y = to_f64(a), to_f64(b)
        assert np.linalg.norm(x - y) <= 4e-3 * np.linalg.norm(y)


def _replay_and_compare(capture_step, eager_step, bufs, inputs, outs, reduced, deterministic,
                        check_oracle):
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        capture_step(s)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        capture_step(s)
    torch.cuda.synchronize()
    for xin in inputs + inputs:
        for k in bufs:
            bufs[k].copy_(xin[k])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = eager_step(xin)
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k], ref[k]), k
        for k in reduced:
            _close(reduced[k], ref[k], deterministic)
        check_oracle(xin)


# D = 2048: the tile forward, and the compact (M = 5, dq summed in LDS) or separate-tile (M = 12,
# with the dq pass) matrix-core backward; D = 1280: the older matrix-core forward, whose sixteen-slot kernel takes tokens from the
# forward workspace's counter unless deterministic, and the query-group backward
@pytest.mark.parametrize("M,D,deterministic", [(5, 2048, True), (5, 2048, False), (12, 2048, True),
                                               (12, 2048, False), (12, 1280, True),
                                               (12, 1280, False)])
def test_multi_query_graph_replay(M, D, deterministic):
    import attention_residuals_amd as A
    S, N = 6, 1531
    inputs = []
    for seed in (21, 22):
        V, g = _sources(S, N, D, seed)
        Q = (torch.randn((M, D), generator=g, device="cuda") / math.sqrt(D)).to(torch.bfloat16)
        G = torch.randn((N, M, D), generator=g, device="cuda").to(torch.bfloat16)
        inputs.append({"V": V, "Q": Q, "G": G})
    bufs = {k: v.clone() for k, v in inputs[0].items()}
    desc = A.make_multi_desc(S, N, D, D, M, torch.bfloat16, layout="token_major",
                             deterministic=deterministic)
    y = torch.empty((N, M, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((N, M), dtype=torch.float32, device="cuda")
    dv = torch.empty((S, N, D), dtype=torch.bfloat16, device="cuda")
    dq = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((A.multi_workspace_bytes(desc),), dtype=torch.uint8, device="cuda")
    fws = torch.empty((A.multi_fwd_workspace_bytes(desc),), dtype=torch.uint8, device="cuda")

    def step(s):
        A.attnres_multi_fwd(bufs["V"], bufs["Q"], layout="token_major", out=y, lse=lse,
                            workspace=None if deterministic else fws,
                            dynamic=not deterministic, stream=s)
        A.attnres_multi_bwd(bufs["V"], bufs["Q"], lse, bufs["G"], layout="token_major",
                            deterministic=deterministic, dvalues=dv, dq=dq, workspace=ws,
                            stream=s)

    def eager(x):
        ye, le = A.attnres_multi_fwd(x["V"], x["Q"], layout="token_major",
                                     dynamic=not deterministic)
        dve, dqe = A.attnres_multi_bwd(x["V"], x["Q"], le, x["G"], layout="token_major",
                                       deterministic=deterministic)
        return {"y": ye, "lse": le, "dv": dve, "dq": dqe}

    refs = {}

    def check(x):
        key = id(x)
        if key not in refs:  # the oracle of each input set, computed once
            refs[key] = oracle.run_multi(x["V"].cpu(), x["Q"].cpu(),
                                         x["G"].transpose(0, 1).contiguous().cpu())
        ref = refs[key]
        res = {"y": compare_rows(to_f64(y.transpose(0, 1)).reshape(-1, D),
                                 ref["y"].reshape(-1, D), "bf16"),
               "lse": compare_stat(to_f64(lse.transpose(0, 1)), ref["lse"]),
               "dvalues": compare_rows(to_f64(dv), ref["dvalues"], "bf16",
                                       roundings=multi_bwd_passes(S, D, M, "bf16"))}
        for m in range(M):
            res[f"dq{m}"] = compare_vec(to_f64(dq[m]), ref["dq"][m], "bf16")
        assert_ok(res, f"multi graph replay M={M} deterministic={deterministic}")

    print(f"[case] multi graph M={M} D={D} deterministic={deterministic}", flush=True)
    _replay_and_compare(step, eager, bufs, inputs, {"y": y, "lse": lse, "dv": dv}, {"dq": dq},
                        deterministic, check)


# K = 3: the slot-group backward; K = 6: the compact matrix-core backward; K = 12: the
# separate-tile one
@pytest.mark.parametrize("E,K,deterministic", [(6, 3, True), (6, 3, False), (48, 3, False),
                                               (6, 6, False), (6, 12, False)])
def test_selected_query_graph_replay(E, K, deterministic):
    import attention_residuals_amd as A
    S, N, D = 6, 1531, 2048
    inputs = []
    for seed in (31, 32):
        V, g = _sources(S, N, D, seed)
        bank = (torch.randn((E, D), generator=g, device="cuda") / math.sqrt(D)).to(torch.bfloat16)
        ids = torch.randint(0, E, (N, K), generator=g, device="cuda", dtype=torch.int64)
        G = torch.randn((N, K, D), generator=g, device="cuda").to(torch.bfloat16)
        inputs.append({"V": V, "bank": bank, "ids": ids, "G": G})
    bufs = {k: v.clone() for k, v in inputs[0].items()}
    desc = A.make_selected_desc(S, N, D, D, E, K, torch.bfloat16, deterministic=deterministic)
    y = torch.empty((N, K, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((N, K), dtype=torch.float32, device="cuda")
    dv = torch.empty((S, N, D), dtype=torch.bfloat16, device="cuda")
    db = torch.empty((E, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((A.selected_workspace_bytes(desc),), dtype=torch.uint8, device="cuda")
    fws = torch.empty((A.selected_fwd_workspace_bytes(desc),), dtype=torch.uint8, device="cuda")

    def step(s):
        A.attnres_selected_fwd(bufs["V"], bufs["bank"], bufs["ids"], out=y, lse=lse,
                               workspace=None if deterministic else fws,
                               dynamic=not deterministic, stream=s)
        A.attnres_selected_bwd(bufs["V"], bufs["bank"], bufs["ids"], lse, bufs["G"],
                               deterministic=deterministic, dvalues=dv, dbank=db, workspace=ws,
                               stream=s)

    def eager(x):
        ye, le = A.attnres_selected_fwd(x["V"], x["bank"], x["ids"], dynamic=not deterministic)
        dve, dbe = A.attnres_selected_bwd(x["V"], x["bank"], x["ids"], le, x["G"],
                                          deterministic=deterministic)
        return {"y": ye, "lse": le, "dv": dve, "db": dbe}

    refs = {}

    def check(x):
        key = id(x)
        if key not in refs:
            refs[key] = oracle.run_selected(x["V"].cpu(), x["bank"].cpu(), x["ids"].cpu(),
                                            x["G"].cpu())
        ref = refs[key]
        res = {"y": compare_rows(to_f64(y).reshape(-1, D), ref["y"].reshape(-1, D), "bf16"),
               "lse": compare_stat(to_f64(lse), ref["lse"]),
               "dvalues": compare_rows(to_f64(dv), ref["dvalues"], "bf16",
                                       roundings=multi_bwd_passes(S, D, K, "bf16", selected=True,
                                                                  E=E)),
               "dbank": compare_vec(to_f64(db), ref["dbank"], "bf16")}
        assert_ok(res, f"selected graph replay E={E} K={K} deterministic={deterministic}")

    print(f"[case] selected graph E={E} K={K} deterministic={deterministic}", flush=True)
    _replay_and_compare(step, eager, bufs, inputs, {"y": y, "lse": lse, "dv": dv}, {"db": db},
                        deterministic, check)
