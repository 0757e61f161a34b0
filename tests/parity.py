"""Parity helpers: run the HIP path and the FP64 oracle on the same seeded inputs and compare.

Tolerances (written here, applied in every GPU parity test):
  * FP32 storage: max |gpu - ref| <= 1e-5 * rms(ref) for every output (y, dvalues, dq, dw, dow).
  * BF16 storage, y and dvalues (and dow): the literal bound 2e-2 * rms(ref) applied to the error
    beyond the rounding that any bf16 result must carry:
        max_i (|gpu_i - ref_i| - half_ulp_bf16(max(|gpu_i|, |ref_i|))) <= 2e-2 * rms(ref).
    Storing the exactly rounded oracle in bf16 alone already gives max |err| / rms of several
    1e-2 on large-magnitude elements, so the literal bound without the half ulp rejects even the
    correctly rounded answer. The literal ratio is reported alongside.
  * A bf16 result built by k passes that each round it to storage (the multi-query backward with
    more than four queries adds every group of queries into dvalues, so dvalues carry one rounding
    per group) may differ from the reference by k half ulps beyond the bound above: the same
    reading with half_ulp replaced by k * half_ulp.
  * BF16 dq and dw: relative L2 error ||gpu - ref|| / ||ref|| <= 1e-2.
  * FP32 per-row statistics lse and o_rstd: |gpu - ref| <= 2e-5 * (1 + |ref|).
rms(x) = sqrt(mean(x^2)) over the whole compared tensor.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np
import torch

import attnres_workloads as W
import oracle

TOL_F32 = 1e-5
TOL_BF16_ROWS = 2e-2
TOL_BF16_VEC = 1e-2
TOL_STAT = 2e-5


def gpu_available() -> bool:
    return torch.cuda.is_available()


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half a bfloat16 ulp at |x| (8 significant bits): 2^(exponent - 8)."""
    ax = np.abs(x)
    _, k = np.frexp(np.where(ax > 0, ax, 1.0))  # ax = m 2^k, 0.5 <= m < 1
    h = np.ldexp(1.0, k - 9)
    return np.where(ax > 0, h, 0.0)


def rms(x: np.ndarray) -> float:
    return float(np.sqrt(np.mean(np.square(x, dtype=np.float64)))) if x.size else 0.0


def compare_rows(g: np.ndarray, r: np.ndarray, dtype: str, roundings: int = 1,
                 slack: Optional[np.ndarray] = None, f32_tol: Optional[float] = None) -> dict:
    """Element-by-element comparison of a row tensor (y, dvalues, dow); `roundings` = how many
    times the result was rounded to bf16 storage on its way (1 for every single pass). `slack`,
    when given, replaces the rounding allowance element by element: a result built in several
    passes, each rounding its running sum to bf16, may be off by half an ulp of every running sum
    (which can exceed the final value's), so callers pass the sum of those half ulps. `f32_tol`
    replaces the FP32 bound where a measured FP32 floor exceeds it (tests/test_fp32_floor.py)."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    scale = rms(r)
    err = np.abs(g - r)
    literal = float(err.max() / scale) if scale > 0 else float(err.max())
    if dtype == "f32":
        tol = TOL_F32 if f32_tol is None else f32_tol
        return {"literal": literal, "metric": literal, "tol": tol, "ok": literal <= tol,
                "finite": bool(np.isfinite(g).all())}
    if slack is None:
        slack = roundings * half_ulp_bf16(np.maximum(np.abs(g), np.abs(r)))
    excess = err - slack
    metric = float(max(excess.max(), 0.0) / scale) if scale > 0 else float(max(excess.max(), 0))
    return {"literal": literal, "metric": metric, "tol": TOL_BF16_ROWS,
            "ok": metric <= TOL_BF16_ROWS and bool(np.isfinite(g).all()),
            "finite": bool(np.isfinite(g).all())}


def compare_vec(g: np.ndarray, r: np.ndarray, dtype: str) -> dict:
    """Comparison of a reduced gradient (dq, dw)."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert g.shape == r.shape
    nr = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(g - r) / nr) if nr > 0 else float(np.linalg.norm(g))
    if dtype == "f32":
        scale = rms(r)
        lit = float(np.abs(g - r).max() / scale) if scale > 0 else float(np.abs(g - r).max())
        return {"literal": lit, "metric": lit, "rel_l2": rel, "tol": TOL_F32,
                "ok": lit <= TOL_F32 or (scale == 0 and lit <= 1e-30)}
    return {"rel_l2": rel, "metric": rel, "tol": TOL_BF16_VEC,
            "ok": (rel <= TOL_BF16_VEC) if nr > 0 else (np.abs(g).max() <= 1e-30)}


def compare_stat(g: np.ndarray, r: np.ndarray) -> dict:
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    err = np.abs(g - r) / (1.0 + np.abs(r))
    m = float(err.max()) if err.size else 0.0
    return {"metric": m, "tol": TOL_STAT, "ok": m <= TOL_STAT}


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def inputs_on(x: dict, device: str) -> dict:
    return {k: (None if v is None else v.to(device)) for k, v in x.items()}


def poison_(t: Optional[torch.Tensor]) -> None:
    """Fills a freshly allocated output with NaN so unwritten elements cannot pass."""
    if t is None:
        return
    if t.dtype in (torch.float32, torch.bfloat16, torch.float16):
        t.fill_(float("nan"))
    else:
        t.fill_(0xFF)


def run_gpu(w: W.Workload, xg: dict, *, packed: bool = True, poison: bool = True,
            values=None, dvalues=None, dout=None, stream=None, deterministic: bool = False,
            accumulate: bool = False) -> dict:
    """Forward + backward through the C ABI on the device tensors xg; returns device tensors.
    accumulate: the backward adds into the given dvalues (never poisoned)."""
    import attention_residuals_amd as A
    v = xg["values"] if values is None else values
    if values is None and not packed:
        v = [xg["values"][s] for s in range(w.S)]
    dev = xg["query"].device
    N, D = w.N, w.D
    desc = A.make_desc(w.S, N, D, w.R, w.torch_dtype, eps=w.eps, scale=w.scale,
                       has_norm_weight=xg["norm_w"] is not None, out_norm=w.out_norm,
                       has_out_weight=xg["out_w"] is not None, deterministic=deterministic,
                       accumulate_dvalues=accumulate)
    y = torch.empty((N, D), dtype=w.torch_dtype, device=dev)
    lse = torch.empty((N,), dtype=torch.float32, device=dev)
    rstd = torch.empty((N,), dtype=torch.float32, device=dev) if w.out_norm else None
    n32 = A.o32_elems(desc)
    o32 = torch.empty((N, D), dtype=torch.float32, device=dev) if n32 else None
    if dvalues is None:
        dvalues = torch.empty((w.S, N, D), dtype=w.torch_dtype, device=dev)
        if not packed:
            dvalues = [dvalues[s] for s in range(w.S)]
    dq = torch.empty((w.R,), dtype=w.torch_dtype, device=dev)
    dw = torch.empty((w.R,), dtype=w.torch_dtype, device=dev) if xg["norm_w"] is not None else None
    dow = torch.empty((D,), dtype=w.torch_dtype, device=dev) if xg["out_w"] is not None else None
    ws = torch.zeros((max(A.workspace_bytes(desc), 256),), dtype=torch.uint8, device=dev)
    if poison:
        for t in (y, lse, rstd, o32, dq, dw, dow):
            poison_(t)
        if not accumulate:
            for t in (dvalues if isinstance(dvalues, list) else [dvalues]):
                poison_(t)
        ws[256:].fill_(0xFF)  # partial rows; the counter words must start at zero
    A.attnres_fwd(v, xg["query"], xg["norm_w"], xg["out_w"], eps=w.eps, scale=w.scale,
                  out_norm=w.out_norm, out=y, lse=lse, out_rstd=rstd, o32=o32, stream=stream)
    g = xg["dout"] if dout is None else dout
    A.attnres_bwd(v, xg["query"], xg["norm_w"], xg["out_w"], lse, rstd, o32, g, eps=w.eps,
                  scale=w.scale, out_norm=w.out_norm, deterministic=deterministic,
                  accumulate=accumulate, dvalues=dvalues, dq=dq, dw=dw, dow=dow, workspace=ws,
                  stream=stream)
    torch.cuda.synchronize()
    dv = torch.stack(dvalues) if isinstance(dvalues, list) else dvalues
    return {"y": y, "lse": lse, "o_rstd": rstd, "o32": o32, "dvalues": dv, "dq": dq, "dw": dw,
            "dow": dow}


def run_oracle(w: W.Workload, xc: dict, tokens: Optional[Sequence[int]] = None,
               reduce: bool = True, want=("y", "lse", "o_rstd", "dvalues")) -> dict:
    return oracle.run(xc["values"], xc["query"], xc["norm_w"], xc["out_w"], xc["dout"],
                      eps=w.eps, scale=w.scale, out_norm=w.out_norm, tokens=tokens,
                      want=want, reduce=reduce)


def check_all(w: W.Workload, got: dict, ref: dict, tokens: Optional[Sequence[int]] = None,
              check_reduced: bool = True) -> dict:
    """Compares GPU outputs (device tensors, all tokens) with oracle outputs (for `tokens`)."""
    res = {}
    idx = None if tokens is None else torch.as_tensor(np.asarray(tokens), dtype=torch.long,
                                                      device=got["y"].device)

    def rows(t, dim=0):
        return t if idx is None else t.index_select(dim, idx)

    res["y"] = compare_rows(to_f64(rows(got["y"])), ref["y"], w.dtype)
    res["lse"] = compare_stat(to_f64(rows(got["lse"])), ref["lse"])
    if w.out_norm:
        res["o_rstd"] = compare_stat(to_f64(rows(got["o_rstd"])), ref["o_rstd"])
    res["dvalues"] = compare_rows(to_f64(rows(got["dvalues"], 1)), ref["dvalues"], w.dtype)
    if check_reduced:
        res["dq"] = compare_vec(to_f64(got["dq"]), ref["dq"], w.dtype)
        if got["dw"] is not None:
            res["dw"] = compare_vec(to_f64(got["dw"]), ref["dw"], w.dtype)
        if got["dow"] is not None:
            res["dow"] = compare_rows(to_f64(got["dow"]), ref["dow"], w.dtype)
    return res


def assert_ok(res: dict, label: str) -> None:
    bad = {k: v for k, v in res.items() if not v["ok"]}
    summary = ", ".join(f"{k}={v['metric']:.3g}" for k, v in res.items())
    print(f"[parity] {label}: {summary}", flush=True)
    assert not bad, f"{label}: out of tolerance: {bad}"


def multi_mfma_bwd(S: int, D: int, M: int, dtype: str, R=None, row_stride=None) -> bool:
    """True when the multi-query backward runs in one pass on matrix cores: bf16, 3 <= M <= 16,
    2 <= S <= 16, D in (1024, 2048, 3072, 4096), R and the row stride multiples of 8 elements
    (accumulating into dvalues, M = 3 with S <= 12 runs the query-group kernel instead: one launch,
    one pass as well, so the launch groups are the same)."""
    R = D if R is None else R
    row_stride = D if row_stride is None else row_stride
    return (dtype == "bf16" and 3 <= M <= 16 and 2 <= S <= 16 and D in (1024, 2048, 3072, 4096)
            and R % 8 == 0 and row_stride % 8 == 0)


LDS_PER_BLOCK = 160 * 1024  # gfx950


def tile_fwd(S: int, D: int, M: int, dtype: str, R=None, row_stride=None, E=None) -> bool:
    """True when the multi-query (or, with E, selected-query) forward runs in the tile kernel with
    a static token stride: bf16, 5 <= M <= 16 (3 <= M for the selected read), 2 <= S <= 16, D in (1024, 2048, 3072, 4096), R and
    the row stride multiples of 8 elements, and the staged rows (M; or E plus a zero row) within the
    workgroup's LDS beside the exchange (with more than eight queries also the output staging
    blocks, where they fit). Other shapes take the older forward, whose sixteen-slot kernels draw
    tokens from a counter in the workspace."""
    R = D if R is None else R
    row_stride = D if row_stride is None else row_stride
    rows = M if E is None else E + 1
    lds = rows * (D + 8) * 2 + (8 * (256 + 16) + 256) * 4
    if E is None and M > 8 and lds + 8 * 2048 <= LDS_PER_BLOCK:
        lds += 8 * 2048
    return (dtype == "bf16" and (5 if E is None else 3) <= M <= 16 and 2 <= S <= 16
            and D in (1024, 2048, 3072, 4096) and R % 8 == 0 and row_stride % 8 == 0
            and lds <= LDS_PER_BLOCK)


def sel_slots_per_launch(S: int, D: int, dtype: str) -> int:
    """Slots per launch of the selected read's slot-group backward: four with one 16-byte chunk
    per thread (D <= 512 chunks at eight waves) and S <= 10, else two."""
    return 4 if (D // (8 if dtype == "bf16" else 4) <= 512 and S <= 10) else 2


def sel_mfma_bwd(S: int, D: int, K: int, E: int, dtype: str, R=None, row_stride=None) -> bool:
    """True when the selected-query backward runs in one pass on matrix cores: bf16, 3 <= K <= 16
    and more slots than the slot-group kernel takes in one launch (sel_slots_per_launch), or
    K >= 4 with S + K <= 16 (the compact tile); 2 <= S <= 16, D in (1024, 2048, 3072, 4096), R and
    the row stride multiples of 8 elements, E <= 16 and the staged bank within the workgroup's LDS
    beside the exchange (the compact tile: E rows; the separate tiles: E + 1 and the transposed
    four-row groups)."""
    R = D if R is None else R
    row_stride = D if row_stride is None else row_stride
    if not (dtype == "bf16" and 3 <= K <= 16 and 2 <= S <= 16 and D in (1024, 2048, 3072, 4096)
            and R % 8 == 0 and row_stride % 8 == 0 and 1 <= E <= 16):
        return False
    compact = S + K <= 16
    if K <= sel_slots_per_launch(S, D, dtype) and not (K >= 4 and compact):
        return False
    # the compact tile (the bank as E rows) or the separate tiles (E + 1 rows and the transposed
    # four-row groups), whichever fits (up to four slots the separate tiles are preferred)
    compact_lds = E * (D + 8) * 2 + (8 * (2 * 256 + 16) + 512 + 64 + 16) * 4
    separate_lds = ((E + 1) * (D + 8) * 2 + 16 * 4 + -(-E // 4) * D * 8
                    + (8 * (2 * 256 + 16) + 512 + 64) * 4)
    return (compact and compact_lds <= LDS_PER_BLOCK) or separate_lds <= LDS_PER_BLOCK


def multi_bwd_groups(S: int, D: int, M: int, dtype: str, selected: bool = False, R=None,
                     row_stride=None, E=None) -> list:
    """Backward launch groups (first query, count) of the multi- and selected-query reads as the
    library plans them: one pass on matrix cores where multi_mfma_bwd (multi-query read) or
    sel_mfma_bwd (selected read, E bank rows) holds, else up to four queries per launch with one
    16-byte chunk per thread (D <= 512 chunks at eight waves) and S <= 12 (selected read: S <= 10),
    else two, sized as evenly
    as possible (larger groups first). Each launch after the first adds into dvalues, rounding the
    running sum to storage again."""
    if not selected and multi_mfma_bwd(S, D, M, dtype, R, row_stride):
        return [(0, M)]
    if selected and E is not None and sel_mfma_bwd(S, D, M, E, dtype, R, row_stride):
        return [(0, M)]
    if selected:
        per = sel_slots_per_launch(S, D, dtype)
    else:
        per = 4 if (D // (8 if dtype == "bf16" else 4) <= 512 and S <= 12) else 2
    n = -(-M // per)
    out, m0 = [], 0
    for i in range(n):
        cnt = M // n + (1 if i < M % n else 0)
        out.append((m0, cnt))
        m0 += cnt
    return out


def multi_bwd_passes(S: int, D: int, M: int, dtype: str, selected: bool = False, R=None,
                     row_stride=None, E=None) -> int:
    return len(multi_bwd_groups(S, D, M, dtype, selected, R, row_stride, E))


def sample_tokens(N: int, k: int, seed: int) -> list:
    rng = np.random.default_rng(seed)
    picks = set([0, N - 1, N // 2]) | set(rng.integers(0, N, size=k).tolist())
    return sorted(t for t in picks if 0 <= t < N)
