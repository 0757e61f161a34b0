"""Pins for the FP64 multi-query oracle ("Fast Attention Residuals" PyPI page, "Multi-query
AttnRes": M queries read the same sources, each with its own routing weights and output).

Checks against things other than the multi-query oracle itself, chosen so that plausible mistakes
(mixing the softmax or delta of different queries, dq_m taking another query's scores, source
gradients kept from the last query instead of summed, the key-norm derivative taken per query
with the wrong key) fail at least one:
  * reverse-mode gradients from torch.autograd over the plain float64 formula;
  * central finite differences of the oracle's own forward;
  * decomposition: the read with M queries equals M single-query reads (already pinned by
    tests/test_oracle_pins.py): outputs and dq_m per query, source gradients summed;
  * special cases: M = 1 is the single-query read; equal queries give equal outputs; a zero query
    gives the mean of the sources.
The selected-query read (per-token queries bank[ids[n, k]]) is pinned by torch.autograd over a
gather of the bank, finite differences on the bank, and equality with the multi-query read when
every token selects the same rows (a repeated row collects both query gradients).
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _problem(seed, S, N, D, R, M):
    rng = np.random.default_rng(seed)
    V = rng.standard_normal((S, N, D)) * np.sqrt(1.0 + np.arange(S))[:, None, None]
    Q = rng.standard_normal((M, R)) / math.sqrt(R)
    G = rng.standard_normal((M, N, D))
    return V, Q, G


CASES = [  # S, N, D, R, M, eps, scale
    (3, 2, 8, 8, 2, 2.0 ** -23, 1.0),
    (4, 3, 16, 5, 3, 1e-3, 0.7),
    (1, 2, 8, 3, 4, 2.0 ** -23, 1.0),
    (5, 2, 12, 12, 16, 0.25, 1.3),
]


def _torch_multi(V, Q, eps, scale):
    D = V.shape[-1]
    R = Q.shape[1]
    t = V[:, :, D - R:]                                   # [S, N, R]
    k = t / torch.sqrt((t * t).mean(-1, keepdim=True) + eps)
    score = scale * torch.einsum("snr,mr->msn", k, Q)     # [M, S, N]
    p = torch.softmax(score, dim=1)
    y = torch.einsum("msn,snd->mnd", p, V)
    return y, torch.logsumexp(score, dim=1)


@pytest.mark.parametrize("case", CASES)
def test_torch_autograd_f64(case):
    S, N, D, R, M, eps, scale = case
    V, Q, G = _problem(11 + S + M, S, N, D, R, M)
    out = oracle.run_multi(V, Q, G, eps=eps, scale=scale)
    tV = torch.tensor(V, requires_grad=True)
    tQ = torch.tensor(Q, requires_grad=True)
    y, lse = _torch_multi(tV, tQ, eps, scale)
    (y * torch.tensor(G)).sum().backward()
    np.testing.assert_allclose(out["y"], y.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out["lse"], lse.detach().numpy(), rtol=1e-12, atol=1e-13)
    gV, gQ = tV.grad.numpy(), tQ.grad.numpy()
    np.testing.assert_allclose(out["dvalues"], gV, rtol=1e-10, atol=1e-12 * np.abs(gV).max())
    np.testing.assert_allclose(out["dq"], gQ, rtol=1e-10, atol=1e-12 * np.abs(gQ).max())


@pytest.mark.parametrize("case", CASES[:3])
def test_finite_differences(case):
    S, N, D, R, M, eps, scale = case
    V, Q, G = _problem(23 + S + M, S, N, D, R, M)
    out = oracle.run_multi(V, Q, G, eps=eps, scale=scale)
    h = 1e-6

    def loss():
        y = oracle.run_multi(V, Q, eps=eps, scale=scale, want=("y",), reduce=False)["y"]
        return float(np.sum(y * G))

    def check(name, analytic, arr):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = loss()
            arr[idx] = old - h
            lm = loss()
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.abs(analytic - num).max() / max(np.abs(num).max(), 1e-30)
        assert err <= 1e-6, f"{name}: relative FD error {err:.3e} for {case}"

    check("dvalues", out["dvalues"], V)
    check("dq", out["dq"], Q)


@pytest.mark.parametrize("case", CASES)
def test_equals_one_single_query_read_per_query(case):
    S, N, D, R, M, eps, scale = case
    V, Q, G = _problem(37 + S + M, S, N, D, R, M)
    out = oracle.run_multi(V, Q, G, eps=eps, scale=scale)
    dv = np.zeros_like(V)
    for m in range(M):
        one = oracle.run(V, Q[m], None, None, G[m], eps=eps, scale=scale)
        np.testing.assert_allclose(out["y"][m], one["y"], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(out["lse"][m], one["lse"], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(out["dq"][m], one["dq"], rtol=1e-11,
                                   atol=1e-13 * np.abs(one["dq"]).max())
        dv += one["dvalues"]
    np.testing.assert_allclose(out["dvalues"], dv, rtol=1e-11, atol=1e-13 * np.abs(dv).max())


def test_equal_queries_give_equal_outputs_and_zero_query_the_mean():
    S, N, D, R = 4, 3, 16, 16
    V, Q, G = _problem(5, S, N, D, R, 3)
    Q[1] = Q[0]
    Q[2] = 0.0
    out = oracle.run_multi(V, Q, G)
    np.testing.assert_array_equal(out["y"][0], out["y"][1])
    np.testing.assert_allclose(out["y"][2], V.mean(axis=0), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(out["lse"][2], np.log(S), rtol=1e-14)


def test_token_subset_and_bf16_storage():
    S, N, D, R, M = 3, 9, 16, 8, 2
    V, Q, G = _problem(41, S, N, D, R, M)
    full = oracle.run_multi(V, Q, G)
    sub = oracle.run_multi(V, Q, G, tokens=[7, 2, 2], reduce=False)
    np.testing.assert_array_equal(sub["y"], full["y"][:, [7, 2, 2]])
    np.testing.assert_array_equal(sub["dvalues"], full["dvalues"][:, [7, 2, 2]])
    # bf16 storage decodes exactly: the same values stored as float64 give the same results
    tV, tQ, tG = (torch.tensor(a).to(torch.bfloat16) for a in (V, Q, G))
    b = oracle.run_multi(tV, tQ, tG)
    f = oracle.run_multi(tV.double().numpy(), tQ.double().numpy(), tG.double().numpy())
    for k in ("y", "lse", "dvalues", "dq"):
        np.testing.assert_array_equal(b[k], f[k])


# ---------------------------------------------------------------- selected-query read

def _selected_problem(seed, S, N, D, R, E, K):
    rng = np.random.default_rng(seed)
    V = rng.standard_normal((S, N, D)) * np.sqrt(1.0 + np.arange(S))[:, None, None]
    bank = rng.standard_normal((E, R)) / math.sqrt(R)
    ids = rng.integers(0, E, size=(N, K))
    G = rng.standard_normal((N, K, D))
    return V, bank, ids, G


SEL_CASES = [  # S, N, D, R, E, K, eps, scale
    (3, 4, 8, 8, 3, 2, 2.0 ** -23, 1.0),
    (4, 5, 16, 5, 6, 3, 1e-3, 0.7),
    (2, 3, 8, 3, 1, 4, 0.25, 1.3),
]


@pytest.mark.parametrize("case", SEL_CASES)
def test_selected_torch_autograd_f64(case):
    S, N, D, R, E, K, eps, scale = case
    V, bank, ids, G = _selected_problem(51 + S + K, S, N, D, R, E, K)
    out = oracle.run_selected(V, bank, ids, G, eps=eps, scale=scale)
    tV = torch.tensor(V, requires_grad=True)
    tB = torch.tensor(bank, requires_grad=True)
    t = tV[:, :, D - R:]
    k = t / torch.sqrt((t * t).mean(-1, keepdim=True) + eps)       # [S, N, R]
    q = tB[torch.tensor(ids)]                                        # [N, K, R]
    score = scale * torch.einsum("snr,nkr->nks", k, q)               # [N, K, S]
    p = torch.softmax(score, dim=-1)
    y = torch.einsum("nks,snd->nkd", p, tV)
    (y * torch.tensor(G)).sum().backward()
    np.testing.assert_allclose(out["y"], y.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out["lse"], torch.logsumexp(score, -1).detach().numpy(),
                               rtol=1e-12, atol=1e-13)
    gV, gB = tV.grad.numpy(), tB.grad.numpy()
    np.testing.assert_allclose(out["dvalues"], gV, rtol=1e-10, atol=1e-12 * np.abs(gV).max())
    np.testing.assert_allclose(out["dbank"], gB, rtol=1e-10, atol=1e-12 * np.abs(gB).max())


def test_selected_finite_differences_on_the_bank():
    S, N, D, R, E, K = 3, 4, 8, 4, 3, 2
    V, bank, ids, G = _selected_problem(61, S, N, D, R, E, K)
    out = oracle.run_selected(V, bank, ids, G)
    h = 1e-6
    num = np.zeros_like(bank)
    for idx in np.ndindex(bank.shape):
        old = bank[idx]
        bank[idx] = old + h
        lp = float(np.sum(oracle.run_selected(V, bank, ids, want=("y",), reduce=False)["y"] * G))
        bank[idx] = old - h
        lm = float(np.sum(oracle.run_selected(V, bank, ids, want=("y",), reduce=False)["y"] * G))
        bank[idx] = old
        num[idx] = (lp - lm) / (2 * h)
    err = np.abs(out["dbank"] - num).max() / np.abs(num).max()
    assert err <= 1e-6, err


def test_selected_with_fixed_ids_is_the_multi_query_read():
    # every token selecting rows (2, 0, 2) of the bank is the multi-query read with those queries;
    # the repeated row's gradient is the sum of its two query gradients
    S, N, D, R, E = 4, 6, 16, 8, 3
    V, bank, _, _ = _selected_problem(71, S, N, D, R, E, 3)
    ids = np.tile(np.array([2, 0, 2]), (N, 1))
    G = np.random.default_rng(72).standard_normal((N, 3, D))
    sel = oracle.run_selected(V, bank, ids, G)
    mq = oracle.run_multi(V, bank[[2, 0, 2]], G.transpose(1, 0, 2))
    np.testing.assert_array_equal(sel["y"], mq["y"].transpose(1, 0, 2))
    np.testing.assert_array_equal(sel["lse"], mq["lse"].T)
    np.testing.assert_allclose(sel["dvalues"], mq["dvalues"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sel["dbank"][2], mq["dq"][0] + mq["dq"][2], rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(sel["dbank"][0], mq["dq"][1], rtol=1e-11, atol=1e-14)
    np.testing.assert_array_equal(sel["dbank"][1], 0.0)
