"""GPU parity of the selected-query read ("Fast Attention Residuals" PyPI page, Multi-query AttnRes:
per-token query selection from an [E, R] bank) against the FP64 oracle, through the C ABI.

Tolerances are the single-query read's (tests/parity.py), applied to every (token, slot) output row,
to dvalues (summed over the K slots; one bf16 rounding per backward launch group), and per bank
row to dbank (relative L2; rows no token selected must be exactly zero).
Covered: banks whose FP32 partial rows fit in LDS and banks that take the global partial blocks,
K = 1 (a padded slot), 2, 3, 4, 5 and 7 (several groups), repeated ids within a token (E = 1), key slices
whose start is not a multiple of four, the two-chunk rows of D = 8192, bf16 and FP32, ids outside
the bank, accumulation into existing dvalues, list sources, several tokens per workgroup in both
schedules, determinism and the static schedule, the autograd wrapper and N = 0.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import (assert_ok, compare_rows, compare_stat, compare_vec, gpu_available,
                    multi_bwd_passes, to_f64)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _inputs(S, N, D, R, E, K, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    V = torch.empty((S, N, D), dtype=dt)
    for s in range(S):
        V[s].copy_(torch.randn((N, D), generator=g) * math.sqrt(1.0 + s))
    bank = (torch.randn((E, R), generator=g) / math.sqrt(R)).to(dt)
    ids = torch.randint(0, E, (N, K), generator=g, dtype=torch.int64)
    G = torch.randn((N, K, D), generator=g).to(dt)
    return V, bank, ids, G


def _run(V, bank, ids, G, dvalues=None, accumulate=False, deterministic=False, dynamic=True,
         packed=True):
    import attention_residuals_amd as A
    vals = V if packed else [V[s] for s in range(V.shape[0])]
    y, lse = A.attnres_selected_fwd(vals, bank, ids, dynamic=dynamic)
    dv, db = A.attnres_selected_bwd(vals, bank, ids, lse, G, deterministic=deterministic,
                                    accumulate=accumulate, dvalues=dvalues)
    torch.cuda.synchronize()
    dv = torch.stack(dv) if isinstance(dv, list) else dv
    return y, lse, dv, db


def _bwd_groups(S, D, K, dtype, E=None, R=None):
    """Backward launch groups of the selected-query read (each rounds dvalues to storage)."""
    return multi_bwd_passes(S, D, K, dtype, selected=True, R=R, E=E)


def _compare_bank(got, ref, dtype, res):
    for e in range(ref.shape[0]):
        if not np.any(ref[e]):
            assert np.all(got[e] == 0), f"bank row {e} was selected by no token but is nonzero"
            continue
        res[f"dbank{e}"] = compare_vec(got[e], ref[e], dtype)


def _check(V, bank, ids, G, label, dtype, init=None, ref_bank=None, ref_ids=None, **kw):
    dvalues = None
    if init is not None:
        dvalues = init.cuda()
        if not kw.get("packed", True):
            dvalues = [dvalues[s].clone() for s in range(V.shape[0])]
    y, lse, dv, db = _run(V.cuda(), bank.cuda(), ids.cuda(), G.cuda(), dvalues=dvalues, **kw)
    ref = oracle.run_selected(V, bank if ref_bank is None else ref_bank,
                              ids if ref_ids is None else ref_ids, G)
    if init is not None:
        ref["dvalues"] = ref["dvalues"] + init.double().numpy()
    S, N, D = V.shape
    K = ids.shape[1]
    res = {"y": compare_rows(to_f64(y).reshape(-1, D), ref["y"].reshape(-1, D), dtype),
           "lse": compare_stat(to_f64(lse), ref["lse"]),
           "dvalues": compare_rows(to_f64(dv), ref["dvalues"], dtype,
                                     roundings=_bwd_groups(S, D, K, dtype, bank.shape[0],
                                                           bank.shape[1]))}
    _compare_bank(to_f64(db), ref["dbank"][:bank.shape[0]], dtype, res)
    assert_ok(res, label)
    return y, lse, dv, db


@pytest.mark.parametrize("S,N,D,R,E,K,dtype", [
    (10, 701, 4096, 4096, 8, 2, "bf16"),    # partial bank in LDS where a workgroup may hold 160 KiB
    (10, 301, 4096, 4096, 16, 2, "bf16"),   # partial bank in global blocks
    (8, 513, 2048, 512, 16, 3, "bf16"),     # LDS bank, three slots in one slot-group launch
    (6, 257, 1024, 1024, 4, 1, "f32"),      # LDS bank, a padded slot
    (4, 300, 8192, 8192, 3, 2, "bf16"),     # two chunks per thread
    (5, 129, 256, 5, 3, 5, "f32"),          # slice start not a multiple of four, three groups
    (3, 97, 2048, 6, 3, 2, "bf16"),
    (24, 199, 2048, 640, 5, 2, "bf16"),
    (4, 200, 512, 512, 1, 3, "bf16"),       # every slot names the same row
    (12, 333, 1024, 1024, 40, 2, "bf16"),   # many rows (global blocks)
    (10, 301, 4096, 4096, 8, 4, "bf16"),    # four slots: the separate-tile matrix-core backward
    (8, 257, 1024, 1024, 4, 4, "f32"),      # four slots, FP32
    (10, 211, 2048, 2048, 24, 7, "bf16"),   # seven slots: groups of four and three, global blocks
    (6, 149, 2048, 2048, 40, 4, "bf16"),    # a bank too large to stage: the slot-group forward
    # the one-pass matrix-core backward (bf16 slots beyond one slot-group launch: K > 4, or K > 2
    # with S > 10; or 4 <= K with S + K <= 16, the compact tile; E <= 16, D = 256 nt)
    (16, 257, 4096, 4096, 6, 16, "bf16"),   # sixteen slots and sources
    (12, 211, 2048, 2048, 8, 3, "bf16"),    # three slots, twelve sources (separate tiles)
    (4, 200, 1024, 256, 8, 6, "bf16"),      # compact tile, sliced key
    (10, 201, 4096, 4096, 16, 4, "bf16"),   # four slots, a bank only the compact tile fits
    (9, 129, 4096, 4096, 7, 7, "bf16"),     # compact tile, sixteen rows
    (5, 300, 3072, 1024, 3, 9, "bf16"),     # twelve column tiles per wave, sliced key
    (12, 150, 1024, 1024, 16, 5, "bf16"),   # sixteen bank rows
])
def test_selected_parity(S, N, D, R, E, K, dtype):
    print(f"[case] selected S={S} N={N} D={D} R={R} E={E} K={K} {dtype}", flush=True)
    V, bank, ids, G = _inputs(S, N, D, R, E, K, dtype, seed=3000 + S * K + D + E)
    _check(V, bank, ids, G, f"selected S={S} N={N} D={D} R={R} E={E} K={K} {dtype}", dtype)


@pytest.mark.parametrize("K,dynamic", [(2, False), (2, True), (3, True), (4, False), (4, True),
                                       (6, True)])  # six slots: the compact matrix-core backward
def test_selected_several_tokens_per_workgroup(K, dynamic):
    # every workgroup reads several tokens (static grid of 8x the resident count, or tickets), so
    # the next token's ids, bank rows and source rows loaded one token ahead are checked
    S, N, D, R, E = 6, 9001, 2048, 2048, 8
    print(f"[case] selected several tokens per workgroup K={K} dynamic={dynamic}", flush=True)
    V, bank, ids, G = _inputs(S, N, D, R, E, K, "bf16", seed=3050 + K)
    _check(V, bank, ids, G, f"selected N={N} K={K} dynamic={dynamic}", "bf16", dynamic=dynamic,
           deterministic=not dynamic)


def test_selected_ids_outside_the_bank_read_a_zero_query():
    # the kernels' reading of an id outside [0, E): a zero query (uniform weights over the sources)
    # and no bank gradient, i.e. the read with a zero row appended to the bank at index E
    S, N, D, R, E, K = 6, 211, 1024, 1024, 5, 3
    print("[case] selected invalid ids", flush=True)
    V, bank, ids, G = _inputs(S, N, D, R, E, K, "bf16", seed=3100)
    ids[::7, 0] = -1
    ids[3::11, 2] = E
    ids[5::13, 1] = 1 << 40
    ext = torch.cat([bank, torch.zeros((1, R), dtype=bank.dtype)])
    ref_ids = torch.where((ids < 0) | (ids >= E), torch.full_like(ids, E), ids)
    _check(V, bank, ids, G, "selected invalid ids", "bf16", ref_bank=ext, ref_ids=ref_ids)


@pytest.mark.parametrize("K", [2, 3])  # the query-group forward and the matrix-core forward
def test_selected_ids_outside_the_bank_set_the_workspace_flag(K):
    # a forward given its workspace flags an id outside [0, E) in the workspace's flag word; the
    # flag stays set over a later clean call and is cleared on request
    import attention_residuals_amd as A
    S, N, D, R, E = 6, 211, 1024, 1024, 5
    print(f"[case] selected id flag K={K}", flush=True)
    V, bank, ids, _ = (t.cuda() for t in _inputs(S, N, D, R, E, K, "bf16", seed=3150 + K))
    desc = A.make_selected_desc(S, N, D, R, E, K, torch.bfloat16)
    ws = torch.zeros((A.selected_fwd_workspace_bytes(desc),), dtype=torch.uint8, device="cuda")
    A.attnres_selected_fwd(V, bank, ids, workspace=ws)
    assert not A.attnres_selected_ids_flag(ws)
    bad = ids.clone()
    bad[N // 2, K - 1] = E
    A.attnres_selected_fwd(V, bank, bad, workspace=ws)
    assert A.attnres_selected_ids_flag(ws)
    A.attnres_selected_fwd(V, bank, ids, workspace=ws)      # sticky over a clean call
    assert A.attnres_selected_ids_flag(ws, clear=True)
    assert not A.attnres_selected_ids_flag(ws)
    bad[N // 2, K - 1] = -3
    A.attnres_selected_fwd(V, bank, bad, workspace=ws)
    assert A.attnres_selected_ids_flag(ws)


@pytest.mark.parametrize("K,packed", [(2, True), (3, False), (4, True), (6, False)])
def test_selected_accumulate_into_dvalues(K, packed):
    S, N, D, R, E = 6, 301, 2048, 2048, 6
    print(f"[case] selected accumulate K={K} packed={packed}", flush=True)
    V, bank, ids, G = _inputs(S, N, D, R, E, K, "bf16", seed=3200 + K)
    init = (2.0 * torch.randn((S, N, D), generator=torch.Generator().manual_seed(7))).to(V.dtype)
    _check(V, bank, ids, G, f"selected accumulate K={K}", "bf16", init=init, accumulate=True,
           packed=packed)


def test_selected_schedules_and_determinism():
    S, N, D, R, E, K = 10, 3001, 4096, 1024, 12, 2
    print("[case] selected schedules", flush=True)
    V, bank, ids, G = (t.cuda() for t in _inputs(S, N, D, R, E, K, "bf16", seed=3300))
    det1 = _run(V, bank, ids, G, deterministic=True, dynamic=False)
    det2 = _run(V, bank, ids, G, deterministic=True, dynamic=False)
    dyn = _run(V, bank, ids, G)
    for a, b in zip(det1, det2):
        assert torch.equal(a, b)
    for k in range(3):
        assert torch.equal(det1[k], dyn[k])
    a, b = to_f64(det1[3]), to_f64(dyn[3])
    assert np.linalg.norm(a - b) <= 4e-3 * np.linalg.norm(a)


def test_selected_autograd_wrapper():
    import attention_residuals_amd as A
    S, N, D, R, E, K = 4, 2 * 37, 1024, 256, 7, 2
    print("[case] selected autograd", flush=True)
    V, bank, ids, G = _inputs(S, N, D, R, E, K, "bf16", seed=3400)
    v = V.cuda().view(S, 2, 37, D).clone().requires_grad_(True)
    b = bank.cuda().clone().requires_grad_(True)
    y = A.attnres_selected(v, b, ids.cuda().view(2, 37, K))
    assert y.shape == (2, 37, K, D)
    y.backward(G.cuda().view(2, 37, K, D))
    ref = oracle.run_selected(V, bank, ids, G)
    assert compare_rows(to_f64(y.detach().reshape(-1, D)), ref["y"].reshape(-1, D), "bf16")["ok"]
    assert compare_rows(to_f64(v.grad.reshape(S, N, D)), ref["dvalues"], "bf16")["ok"]
    res = {}
    _compare_bank(to_f64(b.grad), ref["dbank"], "bf16", res)
    assert_ok(res, "selected autograd dbank")


def test_selected_zero_tokens():
    import attention_residuals_amd as A
    V = torch.empty((3, 0, 256), dtype=torch.bfloat16, device="cuda")
    bank = torch.randn((4, 256), device="cuda").to(torch.bfloat16)
    ids = torch.empty((0, 2), dtype=torch.int64, device="cuda")
    y, lse = A.attnres_selected_fwd(V, bank, ids)
    dv, db = A.attnres_selected_bwd(V, bank, ids, lse,
                                    torch.empty((0, 2, 256), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert y.shape == (0, 2, 256) and torch.all(db == 0)
