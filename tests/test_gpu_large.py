"""GPU parity at sizes where one source exceeds 4 GiB (S = 2, N = 2^19 + 3, D = 4096 bf16: 4.3 GB per
source), so the row offsets of the last tokens pass 2^32 bytes. Sampled tokens (the first, the last
and random ones) are compared row by row with the FP64 oracle, and dq / dw against the oracle's
reduction over all N tokens; the two-query read likewise (sampled rows, dq over all tokens)."""
import math

import numpy as np
import pytest
import torch

import attnres_workloads as W
import oracle
from parity import (assert_ok, check_all, compare_rows, compare_stat, compare_vec, gpu_available,
                    inputs_on, run_gpu, run_oracle, sample_tokens, to_f64)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

N_LARGE = (1 << 19) + 3


def _workload():
    return W.Workload("bf16_s2_n524291_d4096", S=2, N=N_LARGE, D=4096, R=4096, dtype="bf16",
                      norm_weight=True, out_norm=False, out_weight=False, seed=911)


def test_single_query_sources_beyond_4gib():
    w = _workload()
    assert N_LARGE * w.D * 2 > (1 << 32)
    print(f"[case] large single-query S={w.S} N={w.N} D={w.D}", flush=True)
    xg = W.generate(w, device="cuda")
    got = run_gpu(w, xg, poison=False)
    xc = inputs_on(xg, "cpu")
    del xg
    toks = sample_tokens(w.N, 24, seed=5) + [w.N - 2]
    toks = sorted(set(toks))
    ref = dict(run_oracle(w, xc, tokens=toks, reduce=False))
    ref.update({k: v for k, v in run_oracle(w, xc, reduce=True, want=()).items()
                if k in ("dq", "dw")})
    assert_ok(check_all(w, got, ref, tokens=toks), "large single-query")
    del got
    torch.cuda.empty_cache()


def test_two_query_read_sources_beyond_4gib():
    import attention_residuals_amd as A
    w = _workload()
    print(f"[case] large two-query S={w.S} N={w.N} D={w.D}", flush=True)
    xg = W.generate(w, device="cuda", with_dout=False)
    V = xg["values"]
    del xg
    g = torch.Generator(device="cuda").manual_seed(12)
    Q = (torch.randn((2, w.D), generator=g, device="cuda") / math.sqrt(w.D)).to(torch.bfloat16)
    G = torch.randn((2, w.N, w.D), generator=g, device="cuda").to(torch.bfloat16)
    y, lse = A.attnres_multi_fwd(V, Q)
    dv, dq = A.attnres_multi_bwd(V, Q, lse, G)
    torch.cuda.synchronize()
    toks = sorted(set(sample_tokens(w.N, 12, seed=6) + [w.N - 2]))
    idx = torch.tensor(toks, device="cuda")
    ref = oracle.run_multi(V.index_select(1, idx).cpu(), Q.cpu(), G.index_select(1, idx).cpu(),
                           reduce=False)
    res = {"y": compare_rows(to_f64(y.index_select(1, idx)).reshape(-1, w.D),
                             ref["y"].reshape(-1, w.D), "bf16"),
           "lse": compare_stat(to_f64(lse.index_select(1, idx)), ref["lse"]),
           "dvalues": compare_rows(to_f64(dv.index_select(1, idx)), ref["dvalues"], "bf16")}
    del y, dv
    red = oracle.run_multi(V.cpu(), Q.cpu(), G.cpu(), want=(), reduce=True)
    for m in range(2):
        res[f"dq{m}"] = compare_vec(to_f64(dq[m]), red["dq"][m], "bf16")
    assert_ok(res, "large two-query")
    del V, G
    torch.cuda.empty_cache()
