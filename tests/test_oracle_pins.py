"""Pins for the FP64 oracle: checks against things other than the oracle itself.

Each test is chosen so that a plausible mistake in the oracle (a dropped eps, a sum instead of a
mean, the slice taken from the wrong end, a wrong sign in the key-norm derivative, dq and dw
swapped, a missing output-norm term) fails at least one of them:
  * hand-worked examples from the definition (tests/golden/hand_example_s2_d2.json);
  * central finite differences of the oracle's own forward, in FP64 (brute force);
  * reverse-mode gradients from torch.autograd over the plain float64 formula (a library routine
    deriving the backward on its own);
  * special cases with closed forms (S=1, q=0, scale=0, equal sources, outside-the-slice rows);
  * invariants (softmax normalisation, source permutation, key-scale invariance at eps=0,
    Euler homogeneity q.dq = w.dw, unit RMS after the output norm at eps=0, linearity in dY);
  * exact decoding of the bfloat16 storage format.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example_s2_d2.json")


def _rand_problem(seed, S, N, D, R, norm_w, out_norm, out_w, scale=1.0):
    rng = np.random.default_rng(seed)
    V = rng.standard_normal((S, N, D)) * np.sqrt(1.0 + np.arange(S))[:, None, None]
    q = rng.standard_normal(R) / math.sqrt(R)
    w = 1.0 + 0.1 * rng.standard_normal(R) if norm_w else None
    ow = 1.0 + 0.1 * rng.standard_normal(D) if (out_norm and out_w) else None
    g = rng.standard_normal((N, D))
    return V, q, w, ow, g


# ---------------------------------------------------------------- hand-worked examples

def test_hand_examples():
    with open(GOLDEN) as f:
        fixture = json.load(f)
    for case in fixture["cases"]:
        V = np.array(case["values"], dtype=np.float64)
        q = np.array(case["query"], dtype=np.float64)
        w = None if case["norm_w"] is None else np.array(case["norm_w"], dtype=np.float64)
        out = oracle.run(V, q, w, eps=case["eps"], scale=case["scale"])
        s0, s1 = (eval(e, {"sqrt": math.sqrt}) for e in case["expected"]["score"])
        p0 = 1.0 / (1.0 + math.exp(s1 - s0))
        p1 = 1.0 - p0
        env = {"p0": p0, "p1": p1}
        y = [eval(e, env) for e in case["expected"]["y"]]
        np.testing.assert_allclose(out["score"][0], [s0, s1], rtol=1e-14, err_msg=case["name"])
        np.testing.assert_allclose(out["p"][0], [p0, p1], rtol=1e-14, err_msg=case["name"])
        np.testing.assert_allclose(out["y"][0], y, rtol=1e-14, err_msg=case["name"])
        np.testing.assert_allclose(out["lse"][0], math.log(math.exp(s0) + math.exp(s1)),
                                   rtol=1e-14, err_msg=case["name"])


# ---------------------------------------------------------------- finite differences

FD_CASES = [
    # S, N, D, R, norm_w, out_norm, out_w, eps, scale
    (1, 1, 8, 8, True, False, False, 1e-3, 1.0),
    (2, 3, 8, 3, True, False, False, 0.25, 0.7),
    (3, 1, 16, 1, False, False, False, 2.0 ** -23, 1.0),
    (3, 3, 16, 16, True, True, True, 0.1, 1.3),
    (5, 3, 8, 8, False, True, False, 2.0 ** -23, 1.0),
    (5, 1, 16, 3, True, True, False, 0.05, 2.0),
    (2, 3, 16, 16, False, True, True, 1.0, 0.5),
]


def _loss(V, q, w, ow, g, out_norm, eps, scale):
    y = oracle.run(V, q, w, ow, eps=eps, scale=scale, out_norm=out_norm, want=("y",),
                   reduce=False)["y"]
    return float(np.sum(y * g))


@pytest.mark.parametrize("case", FD_CASES)
def test_finite_differences(case):
    S, N, D, R, has_w, out_norm, has_ow, eps, scale = case
    V, q, w, ow, g = _rand_problem(7 + S * 13 + D, S, N, D, R, has_w, out_norm, has_ow)
    out = oracle.run(V, q, w, ow, g, eps=eps, scale=scale, out_norm=out_norm)
    h = 1e-6

    def fd(arr, idx):
        old = arr[idx]
        arr[idx] = old + h
        lp = _loss(V, q, w, ow, g, out_norm, eps, scale)
        arr[idx] = old - h
        lm = _loss(V, q, w, ow, g, out_norm, eps, scale)
        arr[idx] = old
        return (lp - lm) / (2 * h)

    def check(name, analytic, arr):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            num[idx] = fd(arr, idx)
        ref = max(np.abs(num).max(), 1e-30)
        err = np.abs(analytic.reshape(arr.shape) - num).max() / ref
        assert err <= 1e-6, f"{name}: relative FD error {err:.3e} for case {case}"

    check("dvalues", out["dvalues"], V)
    check("dq", out["dq"], q)
    if w is not None:
        check("dw", out["dw"], w)
    if ow is not None:
        check("dow", out["dow"], ow)


# ---------------------------------------------------------------- torch.autograd (float64)

def _torch_read(V, q, w, ow, out_norm, eps, scale):
    D = V.shape[-1]
    R = q.shape[0]
    t = V[:, :, D - R:]
    r = torch.sqrt((t * t).mean(-1, keepdim=True) + eps)
    k = t / r
    if w is not None:
        k = k * w
    score = scale * (k * q).sum(-1)
    p = torch.softmax(score, dim=0)
    o = (p.unsqueeze(-1) * V).sum(0)
    if out_norm:
        o = o * torch.rsqrt((o * o).mean(-1, keepdim=True) + eps)
        if ow is not None:
            o = o * ow
    return o, torch.logsumexp(score, dim=0)


@pytest.mark.parametrize("case", FD_CASES + [(4, 17, 64, 16, True, False, False, 2.0 ** -23, 1.0),
                                             (6, 9, 32, 32, True, True, True, 1e-4, 1.0)])
def test_torch_autograd_f64(case):
    S, N, D, R, has_w, out_norm, has_ow, eps, scale = case
    V, q, w, ow, g = _rand_problem(99 + S + N, S, N, D, R, has_w, out_norm, has_ow)
    out = oracle.run(V, q, w, ow, g, eps=eps, scale=scale, out_norm=out_norm)
    tV = torch.tensor(V, requires_grad=True)
    tq = torch.tensor(q, requires_grad=True)
    tw = None if w is None else torch.tensor(w, requires_grad=True)
    tow = None if ow is None else torch.tensor(ow, requires_grad=True)
    y, lse = _torch_read(tV, tq, tw, tow, out_norm, eps, scale)
    (y * torch.tensor(g)).sum().backward()
    np.testing.assert_allclose(out["y"], y.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out["lse"], lse.detach().numpy(), rtol=1e-12, atol=1e-13)
    gV = tV.grad.numpy()
    np.testing.assert_allclose(out["dvalues"], gV, rtol=1e-10, atol=1e-12 * np.abs(gV).max())
    np.testing.assert_allclose(out["dq"], tq.grad.numpy(), rtol=1e-10,
                               atol=1e-12 * np.abs(tq.grad.numpy()).max())
    if w is not None:
        np.testing.assert_allclose(out["dw"], tw.grad.numpy(), rtol=1e-10,
                                   atol=1e-12 * np.abs(tw.grad.numpy()).max())
    if ow is not None:
        np.testing.assert_allclose(out["dow"], tow.grad.numpy(), rtol=1e-10,
                                   atol=1e-12 * np.abs(tow.grad.numpy()).max())


# ---------------------------------------------------------------- special cases

def test_single_source_returns_it():
    V, q, w, _, g = _rand_problem(3, 1, 5, 16, 16, True, False, False)
    out = oracle.run(V, q, w, None, g)
    assert np.array_equal(out["y"], V[0])
    assert np.array_equal(out["dvalues"][0], g)
    assert np.all(out["dq"] == 0.0) and np.all(out["dw"] == 0.0)
    assert np.all(out["p"] == 1.0)


@pytest.mark.parametrize("zero", ["query", "scale"])
def test_zero_query_or_scale_gives_uniform_mean(zero):
    S, N, D = 5, 4, 24
    V, q, w, _, g = _rand_problem(4, S, N, D, 8, True, False, False)
    if zero == "query":
        q = np.zeros_like(q)
    out = oracle.run(V, q, w, None, g, scale=0.0 if zero == "scale" else 1.0)
    np.testing.assert_allclose(out["y"], V.mean(axis=0), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(out["lse"], np.full(N, math.log(S)), rtol=1e-15)
    np.testing.assert_allclose(out["p"], np.full((N, S), 1.0 / S), rtol=1e-15)


def test_equal_sources():
    S, N, D = 4, 3, 16
    _, q, w, _, g = _rand_problem(5, S, N, D, D, True, False, False)
    v = np.random.default_rng(1).standard_normal((N, D))
    V = np.stack([v] * S)
    out = oracle.run(V, q, w, None, g)
    np.testing.assert_allclose(out["y"], v, rtol=1e-14, atol=1e-15)
    for s in range(S):
        np.testing.assert_allclose(out["dvalues"][s], g / S, rtol=1e-12, atol=1e-14)
    assert np.abs(out["dq"]).max() < 1e-13 and np.abs(out["dw"]).max() < 1e-13


def test_outside_slice_gradient_is_routing_weight_times_dy():
    S, N, D, R = 3, 6, 16, 5
    V, q, w, _, g = _rand_problem(6, S, N, D, R, True, False, False)
    out = oracle.run(V, q, w, None, g)
    for s in range(S):
        np.testing.assert_allclose(out["dvalues"][s][:, :D - R],
                                   out["p"][:, s:s + 1] * g[:, :D - R], rtol=1e-14, atol=1e-15)
    # and the slice columns do depend on the routing derivative
    assert not np.allclose(out["dvalues"][0][:, D - R:], out["p"][:, :1] * g[:, D - R:])


def test_slice_is_the_final_coordinates():
    # Changing coordinates outside the slice changes neither scores nor routing weights.
    S, N, D, R = 3, 4, 12, 4
    V, q, w, _, _ = _rand_problem(8, S, N, D, R, True, False, False)
    a = oracle.run(V, q, w)
    V2 = V.copy()
    V2[:, :, :D - R] *= -3.0
    b = oracle.run(V2, q, w)
    np.testing.assert_array_equal(a["score"], b["score"])
    V3 = V.copy()
    V3[:, :, D - 1] += 1.0
    c = oracle.run(V3, q, w)
    assert not np.allclose(a["score"], c["score"])


# ---------------------------------------------------------------- invariants

def test_softmax_normalisation_and_lse():
    V, q, w, _, _ = _rand_problem(9, 7, 11, 32, 32, True, False, False)
    out = oracle.run(V, q, w)
    np.testing.assert_allclose(out["p"].sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(np.exp(out["score"] - out["lse"][:, None]), out["p"], rtol=1e-13)


def test_source_permutation():
    V, q, w, _, g = _rand_problem(10, 6, 5, 16, 8, True, False, False)
    perm = np.array([3, 0, 5, 1, 4, 2])
    a = oracle.run(V, q, w, None, g)
    b = oracle.run(V[perm], q, w, None, g)
    np.testing.assert_allclose(a["y"], b["y"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(a["dq"], b["dq"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(a["dw"], b["dw"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(a["dvalues"][perm], b["dvalues"], rtol=1e-12, atol=1e-14)


def test_key_scale_invariance_at_zero_eps():
    # With eps = 0 the score does not see the scale of t_s, so the slice gradient has no
    # component along t_s beyond the mixture term: <t_s, dV_s - p_s dY>_slice = 0.
    S, N, D, R = 4, 5, 16, 16
    V, q, w, _, g = _rand_problem(11, S, N, D, R, True, False, False)
    out = oracle.run(V, q, w, None, g, eps=0.0)
    for s in range(S):
        t = V[s][:, D - R:]
        resid = out["dvalues"][s][:, D - R:] - out["p"][:, s:s + 1] * g[:, D - R:]
        proj = np.sum(t * resid, axis=1)
        assert np.abs(proj).max() < 1e-12 * max(1.0, np.abs(resid).max() * np.abs(t).max() * R)
    # scaling a whole source by c > 0 leaves the routing weights unchanged at eps = 0
    V2 = V.copy()
    V2[2] *= 7.5
    np.testing.assert_allclose(oracle.run(V2, q, w, eps=0.0)["score"][:, 2], out["score"][:, 2],
                               rtol=1e-13)


def test_euler_homogeneity_q_dot_dq_equals_w_dot_dw():
    # score is linear in q and in w, so q.dq = w.dw = sum over tokens and sources of dscore*score
    V, q, w, _, g = _rand_problem(12, 5, 9, 32, 32, True, False, False)
    out = oracle.run(V, q, w, None, g)
    a = float(q @ out["dq"])
    b = float(w @ out["dw"])
    assert abs(a - b) <= 1e-12 * max(abs(a), 1.0)
    assert abs(a) > 1e-6  # not trivially zero


def test_output_norm_unit_rms_at_zero_eps():
    V, q, w, _, _ = _rand_problem(13, 4, 6, 32, 32, False, True, False)
    out = oracle.run(V, q, w, None, out_norm=True, eps=0.0)
    np.testing.assert_allclose(np.mean(out["y"] ** 2, axis=1), 1.0, rtol=1e-14)
    o = np.einsum("ns,snd->nd", out["p"], V)
    np.testing.assert_allclose(out["o_rstd"], 1.0 / np.sqrt(np.mean(o * o, axis=1)), rtol=1e-13)


def test_backward_linear_in_dy():
    V, q, w, ow, g = _rand_problem(14, 3, 4, 16, 8, True, True, True)
    a = oracle.run(V, q, w, ow, g, out_norm=True, eps=0.01)
    b = oracle.run(V, q, w, ow, -2.5 * g, out_norm=True, eps=0.01)
    for k in ("dvalues", "dq", "dw", "dow"):
        np.testing.assert_allclose(b[k], -2.5 * a[k], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- storage formats

def test_bf16_decode_is_exact():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F, 0x0001], dtype=np.uint16)
    expect = [1.0, -2.0, 1.0078125, 0.0, -0.0, 3.3895313892515355e38, 2.0 ** -133]
    V = np.stack([bits.reshape(1, -1)])  # S=1 returns the source exactly
    q = np.array([0x3F80], dtype=np.uint16)
    out = oracle.run(V, q)
    assert list(out["y"][0]) == expect


def test_storage_formats_agree():
    rng = np.random.default_rng(15)
    S, N, D, R = 3, 8, 32, 16
    V32 = rng.standard_normal((S, N, D)).astype(np.float32)
    q32 = (rng.standard_normal(R) / 4).astype(np.float32)
    g32 = rng.standard_normal((N, D)).astype(np.float32)
    a = oracle.run(V32, q32, None, None, g32)
    b = oracle.run(V32.astype(np.float64), q32.astype(np.float64), None, None,
                   g32.astype(np.float64))
    for k in ("y", "lse", "dvalues", "dq"):
        assert np.array_equal(a[k], b[k]), k
    tv = torch.from_numpy(V32).to(torch.bfloat16)
    tq = torch.from_numpy(q32).to(torch.bfloat16)
    tg = torch.from_numpy(g32).to(torch.bfloat16)
    c = oracle.run(tv, tq, None, None, tg)
    d = oracle.run(tv.double().numpy(), tq.double().numpy(), None, None, tg.double().numpy())
    for k in ("y", "lse", "dvalues", "dq"):
        assert np.array_equal(c[k], d[k]), k


def test_token_subset_matches_full_run():
    V, q, w, ow, g = _rand_problem(16, 4, 20, 16, 16, True, True, True)
    full = oracle.run(V, q, w, ow, g, out_norm=True)
    toks = [19, 0, 7, 7, 3]
    sub = oracle.run(V, q, w, ow, g, out_norm=True, tokens=toks, reduce=False)
    np.testing.assert_array_equal(sub["y"], full["y"][toks])
    np.testing.assert_array_equal(sub["dvalues"], full["dvalues"][:, toks])
    np.testing.assert_array_equal(sub["o_rstd"], full["o_rstd"][toks])


def test_thread_count_does_not_change_results_beyond_rounding():
    V, q, w, _, g = _rand_problem(17, 3, 64, 16, 16, True, False, False)
    a = oracle.run(V, q, w, None, g, threads=1)
    b = oracle.run(V, q, w, None, g, threads=4)
    np.testing.assert_array_equal(a["y"], b["y"])
    np.testing.assert_array_equal(a["dvalues"], b["dvalues"])
    np.testing.assert_allclose(a["dq"], b["dq"], rtol=1e-13)


# ---------------------------------------------------------------- tolerance reading

def test_bf16_tolerance_reading_is_well_posed():
    # The stated bf16 bound (2e-2 * rms) taken literally rejects the correctly rounded answer;
    # the reading used by the GPU parity tests (error beyond half a bf16 ulp) accepts it and still
    # rejects an error of the size the bound is meant to catch.
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    from parity import compare_rows
    import attnres_workloads as W
    w = W.small(W.WORKLOADS["bf16_s10_n32768_d4096"], 96)
    x = W.generate(w)
    r = oracle.run(x["values"], x["query"], x["norm_w"], None, x["dout"])
    for key in ("y", "dvalues"):
        exact = r[key]
        rounded = torch.from_numpy(exact).to(torch.bfloat16).double().numpy()
        res = compare_rows(rounded, exact, "bf16")
        assert res["ok"] and res["metric"] < 1e-6, (key, res)
        if key == "dvalues":
            assert res["literal"] > 2e-2, res  # the literal reading would fail here
        bad = rounded.copy()
        bad.flat[7] += 0.05 * np.sqrt(np.mean(exact ** 2))
        assert not compare_rows(bad, exact, "bf16")["ok"], key
