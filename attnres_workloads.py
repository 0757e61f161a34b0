"""Seeded synthetic workloads for the AttnRes read (inputs only; none of the method's arithmetic).

This is the one module both sides of every parity check use: the GPU library's tests and bench
feed these tensors to the HIP path, and the FP64 oracle reads host copies of the very same
tensors. It draws, scales and rounds inputs; it computes nothing the method computes.

Recipe (every workload):
  * ``torch.Generator`` seeded with the workload's seed, standard normals drawn in FP32;
  * draw order: values (source 0 .. S-1, each [N, D]), query [R], key-norm weight [R] (when the
    workload has one), output-norm weight [D] (when it has one), upstream gradient dY [N, D];
  * values of source s are N(0,1) * sqrt(1+s); the query is N(0,1) / sqrt(D) (or / sqrt(R) for the
    sliced low-rank read); weights are 1 + 0.1 N(0,1); dY is N(0,1);
  * each tensor is rounded once to the workload's storage dtype.

The shapes are those of the FLA PR page's benchmark rows ("[Perf] Parallelize AttnRes
long-sequence reduction", benchmark table: L sources, T tokens, width D, B=H=1) and of the
24-source, quarter-rank read of the "Fast Attention Residuals" page (Training performance,
Quarter-rank routing). No public dataset is involved: synthetic draws stand in for activations.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import torch

EPS_DEFAULT = 2.0 ** -23


@dataclass(frozen=True)
class Workload:
    name: str
    S: int
    N: int
    D: int
    R: int
    dtype: str                 # "f32" or "bf16"
    norm_weight: bool          # key-norm weight w[R]
    out_norm: bool             # output RMSNorm after the mixture
    out_weight: bool           # output-norm weight ow[D] (only with out_norm)
    seed: int
    query_over_rank: bool = False  # query N(0,1)/sqrt(R) instead of /sqrt(D)
    eps: float = EPS_DEFAULT
    scale: float = 1.0

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def algorithmic_bytes(self) -> int:
        """Bytes one forward + backward must move: fwd reads V and writes y, bwd reads V and dY
        and writes dV; plus the FP32 per-row statistics (lse, and o_rstd with the output norm),
        each written once and read once."""
        b = self.elem_bytes
        rows = (3 * self.S + 2) * self.N * self.D * b
        stats = 2 * 4 * self.N * (2 if self.out_norm else 1)
        return rows + stats


# The five workloads. Names say what each is; sizes follow the module docstring's sources.
WORKLOADS = {
    "tiny_f32_s4_n256_d256": Workload(
        "tiny_f32_s4_n256_d256", S=4, N=256, D=256, R=256, dtype="f32",
        norm_weight=True, out_norm=False, out_weight=False, seed=1001),
    "bf16_s8_n8192_d2048": Workload(
        "bf16_s8_n8192_d2048", S=8, N=8192, D=2048, R=2048, dtype="bf16",
        norm_weight=True, out_norm=False, out_weight=False, seed=1002),
    "bf16_s10_n32768_d4096": Workload(
        "bf16_s10_n32768_d4096", S=10, N=32768, D=4096, R=4096, dtype="bf16",
        norm_weight=True, out_norm=False, out_weight=False, seed=1003),
    "bf16_s64_n8192_d8192_outnorm": Workload(
        "bf16_s64_n8192_d8192_outnorm", S=64, N=8192, D=8192, R=8192, dtype="bf16",
        norm_weight=False, out_norm=True, out_weight=False, seed=1004),
    "bf16_s24_n16384_d2048_r512": Workload(
        "bf16_s24_n16384_d2048_r512", S=24, N=16384, D=2048, R=512, dtype="bf16",
        norm_weight=False, out_norm=False, out_weight=False, seed=1005, query_over_rank=True),
}

# The FLA PR page's two other benchmark rows at D = 2048 / 4096 (same recipe): measured by the
# benchmark for context and covered by the full-size parity tests.
BENCH_ROWS = {
    "bf16_s10_n8192_d4096": Workload(
        "bf16_s10_n8192_d4096", S=10, N=8192, D=4096, R=4096, dtype="bf16",
        norm_weight=True, out_norm=False, out_weight=False, seed=1006),
    "bf16_s8_n32768_d2048": Workload(
        "bf16_s8_n32768_d2048", S=8, N=32768, D=2048, R=2048, dtype="bf16",
        norm_weight=True, out_norm=False, out_weight=False, seed=1007),
}

ALL = {**WORKLOADS, **BENCH_ROWS}

HEADLINE = "bf16_s10_n32768_d4096"
TINY = "tiny_f32_s4_n256_d256"


def generate(w: Workload, device: str = "cpu", with_dout: bool = True) -> dict:
    """Draws the workload's inputs (see module docstring). Returns a dict with ``values``
    [S, N, D], ``query`` [R], ``norm_w`` [R] or None, ``out_w`` [D] or None, ``dout`` [N, D] or
    None, all in the workload's storage dtype on ``device``."""
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    dt = w.torch_dtype
    values = torch.empty((w.S, w.N, w.D), dtype=dt, device=device)
    for s in range(w.S):
        x = torch.randn((w.N, w.D), generator=gen, dtype=torch.float32, device=device)
        x.mul_(math.sqrt(1.0 + s))
        values[s].copy_(x)
        del x
    qd = w.R if w.query_over_rank else w.D
    query = (torch.randn((w.R,), generator=gen, dtype=torch.float32, device=device)
             / math.sqrt(qd)).to(dt)
    norm_w = None
    if w.norm_weight:
        norm_w = (1.0 + 0.1 * torch.randn((w.R,), generator=gen, dtype=torch.float32,
                                          device=device)).to(dt)
    out_w = None
    if w.out_norm and w.out_weight:
        out_w = (1.0 + 0.1 * torch.randn((w.D,), generator=gen, dtype=torch.float32,
                                         device=device)).to(dt)
    dout = None
    if with_dout:
        dout = torch.randn((w.N, w.D), generator=gen, dtype=torch.float32,
                           device=device).to(dt)
    return {"values": values, "query": query, "norm_w": norm_w, "out_w": out_w, "dout": dout}


def multi_inputs(w: Workload, M: int, layout: str = "query_major", device: str = "cpu") -> dict:
    """Inputs of the multi-query read over the workload's sources: ``queries`` [M, R] (standard
    normals over sqrt(R) or sqrt(D), like the single query) and ``dout`` ([M, N, D] query-major or
    [N, M, D] token-major standard normals), from their own generator seeded seed + 100 * M."""
    g = torch.Generator(device=device).manual_seed(w.seed + 100 * M)
    qd = w.R if w.query_over_rank else w.D
    queries = torch.randn((M, w.R), generator=g, device=device) / math.sqrt(qd)
    shape = (M, w.N, w.D) if layout == "query_major" else (w.N, M, w.D)
    dout = torch.randn(shape, generator=g, device=device)
    return {"queries": queries.to(w.torch_dtype), "dout": dout.to(w.torch_dtype)}


def multi_case(S: int, N: int, D: int, R: int, M: int, dtype: str, seed: int,
               device: str = "cpu"):
    """A small multi-query case (parity tests): values [S, N, D] with source s ~ N(0,1) sqrt(1+s),
    queries [M, R] ~ N(0,1) / sqrt(R), query-major dY [M, N, D] ~ N(0,1), drawn in that order from
    one generator and rounded once to the storage dtype."""
    g = torch.Generator(device=device).manual_seed(seed)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    V = torch.empty((S, N, D), dtype=dt, device=device)
    for s in range(S):
        V[s].copy_(torch.randn((N, D), generator=g, device=device) * math.sqrt(1.0 + s))
    Q = (torch.randn((M, R), generator=g, device=device) / math.sqrt(R)).to(dt)
    G = torch.randn((M, N, D), generator=g, device=device).to(dt)
    return V, Q, G


def selected_inputs(w: Workload, E: int, K: int, device: str = "cpu") -> dict:
    """Inputs of the selected-query read over the workload's sources: ``bank`` [E, R] (scaled like
    the single query), ``ids`` [N, K] int64 uniform over the bank, ``dout`` [N, K, D] standard
    normals, from their own generator seeded seed + 1000 * E + K."""
    g = torch.Generator(device=device).manual_seed(w.seed + 1000 * E + K)
    qd = w.R if w.query_over_rank else w.D
    bank = (torch.randn((E, w.R), generator=g, device=device) / math.sqrt(qd)).to(w.torch_dtype)
    ids = torch.randint(0, E, (w.N, K), generator=g, device=device, dtype=torch.int64)
    dout = torch.randn((w.N, K, w.D), generator=g, device=device).to(w.torch_dtype)
    return {"bank": bank, "ids": ids, "dout": dout}


def small(w: Workload, N: int, seed: Optional[int] = None, **kw) -> Workload:
    """The same workload at a reduced token count (and optionally another seed)."""
    return w.with_(N=N, seed=w.seed if seed is None else seed, **kw)
