"""GPU parity of the five workloads (and, at full size, the benchmark table's two other rows)
against the FP64 oracle, through the C ABI.

Reduced token counts: every output of every token is compared element by element (token counts
are not multiples of the persistent grid, so workgroups end on a ragged tail). Full sizes, in
the launch configuration the benchmark times: sampled tokens' rows are compared one by one with
the oracle, and dq/dw/dow against the oracle's reduction over all N tokens.
"""
import pytest
import torch

import attnres_workloads as W
from parity import (assert_ok, check_all, gpu_available, inputs_on, run_gpu, run_oracle,
                    sample_tokens)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

REDUCED_N = {
    "tiny_f32_s4_n256_d256": 256,
    "bf16_s8_n8192_d2048": 3001,
    "bf16_s10_n32768_d4096": 1531,
    "bf16_s64_n8192_d8192_outnorm": 61,
    "bf16_s24_n16384_d2048_r512": 2003,
}


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_reduced_n(name):
    w = W.small(W.WORKLOADS[name], REDUCED_N[name])
    print(f"[case] {name} N={w.N}", flush=True)
    xc = W.generate(w)
    got = run_gpu(w, inputs_on(xc, "cuda"))
    ref = run_oracle(w, xc)
    assert_ok(check_all(w, got, ref), f"{name} N={w.N}")


@pytest.mark.parametrize("name", list(W.ALL))
def test_workload_full_size(name):
    w = W.ALL[name]
    print(f"[case] full {name}", flush=True)
    xg = W.generate(w, device="cuda")
    got = run_gpu(w, xg, poison=False)
    xc = inputs_on(xg, "cpu")
    del xg
    toks = sample_tokens(w.N, 48, seed=w.seed)
    ref_rows = run_oracle(w, xc, tokens=toks, reduce=False)
    ref_red = run_oracle(w, xc, reduce=True, want=())
    ref = dict(ref_rows)
    ref.update({k: v for k, v in ref_red.items() if k in ("dq", "dw", "dow")})
    assert_ok(check_all(w, got, ref, tokens=toks), f"full {name}")
    torch.cuda.empty_cache()
