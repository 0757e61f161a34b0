"""Benchmark of the AttnRes read, forward + backward, on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input resident in HBM:
attnres_fwd (forward kernel) then attnres_bwd (backward kernel + finaliser), through the C ABI,
on torch's current stream. Default workload: S=10 sources, N=32768 tokens, D=4096, R=D, bf16,
key-norm weight, no output norm (the FLA PR page's L=10, T=32768, D=4096 benchmark row).

Prints ONE JSON line. `value` is algorithmic HBM bytes per step / time per step (GB/s);
algorithmic bytes = fwd reads V and writes y, bwd reads V and dY and writes dV, plus the FP32
per-row statistics written once and read once. The `roofline` object is for the backward call
(backward kernel + its finaliser, the dominant launch), timed with HIP events on the launch
stream over the timed region. `cpu_baseline` times the FP64 CPU oracle (test infrastructure) on
the same inputs.

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 50] [--workload NAME] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
# B200 Triton fwdbwd median for this exact workload (FLA PR page, benchmark table, L=10,
# T=32768, D=4096 bf16, candidate column): another machine's number, quoted as context.
B200_MS = {"bf16_s10_n32768_d4096": 3.268607974052429,
           "bf16_s8_n8192_d2048": 0.4638400077819824,
           "bf16_s64_n8192_d8192_outnorm": 11.95311975479126,
           "bf16_s10_n8192_d4096": 0.9022,
           "bf16_s8_n32768_d2048": 1.2953}
METRIC = "AttnRes fwd+bwd ms and HBM GB/s (% peak), S=10,N=32768,D=4096 bf16, 1 GPU"


def kernel_source_hash(scope: str = "single") -> str:
    """Hash of the library sources. scope "single": the single-query read's (its kernels, their
    instantiations, the shared argument structs and the host planner; the multi- and
    selected-query kernels' own files are left out, since the default workload never runs them);
    scope "all": every source file."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_residuals_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if scope == "single" and name.startswith(("attnres_multi_", "attnres_sel_")):
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


# VALU issue peak of MI355X: 256 CUs x 4 SIMDs, each issuing one wave64 VALU instruction every
# 4 cycles (16 lanes; packed FP32 is not used), at 2.4 GHz: 614.4 G wave-instructions per second
# (39.3 T lane operations per second, 78.6 TFLOP/s of FP32 FMA).
PEAK_VALU_GINSTR = 256 * 4 * 2.4e9 / 4 / 1e9


def cpu_info() -> dict:
    """The host CPU as /proc/cpuinfo names it: model, physical cores (distinct (package, core)
    pairs) and logical CPUs, plus the CPUs this process may run on."""
    model, pairs, logical = None, set(), 0
    try:
        with open("/proc/cpuinfo") as f:
            phys = core = None
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "processor":
                    logical += 1
                elif k == "model name" and model is None:
                    model = v
                elif k == "physical id":
                    phys = v
                elif k == "core id":
                    core = v
                elif not k and phys is not None:
                    pairs.add((phys, core))
                    phys = core = None
            if phys is not None:
                pairs.add((phys, core))
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = os.cpu_count()
    return {"cpu_model": model, "physical_cores": len(pairs) or None, "logical_cpus": logical or None,
            "cpus_available": allowed}


def stream_ceiling(streams_fwd, streams_bwd, fwd_bytes, bwd_bytes, reps=10):
    """The practical ceiling of the step's traffic: attnres_stream_probe moving the forward's and
    the backward's streams (lists of (inputs, outputs) tensors, rows as the kernels read them)
    with no arithmetic, timed with HIP events on the current stream (median of `reps` runs of
    each launch shape; the fastest shape counts). Returns GB/s of the forward, the backward and
    the whole step at the algorithmic bytes."""
    import numpy as np
    import torch
    from attention_residuals_amd._binding import stream_probe
    stream = torch.cuda.current_stream()
    res, shape = {}, {}
    for name, (ins, outs) in (("fwd", streams_fwd), ("bwd", streams_bwd)):
        best = None
        for cpt in (1, 2):
            for bpc in (1, 2, 4, 8, 16):
                for _ in range(2):
                    stream_probe(ins, outs, cpt, bpc)
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(reps)]
                for a, b in ev:
                    a.record(stream)
                    stream_probe(ins, outs, cpt, bpc)
                    b.record(stream)
                torch.cuda.synchronize()
                t = float(np.median([a.elapsed_time(b) for a, b in ev]))
                if best is None or t < best[0]:
                    best = (t, cpt, bpc)
        res[name] = best[0]
        shape[name] = {"chunks_per_thread": best[1], "blocks_per_cu": best[2]}
    return {"kind": "attnres_stream_probe: the step's row streams, no arithmetic (fastest of 10 "
                    "launch shapes)", "shapes": shape,
            "fwd_ms": round(res["fwd"], 4), "bwd_ms": round(res["bwd"], 4),
            "fwd_GBps": round(fwd_bytes / (res["fwd"] * 1e-3) / 1e9, 1),
            "bwd_GBps": round(bwd_bytes / (res["bwd"] * 1e-3) / 1e9, 1),
            "step_GBps": round((fwd_bytes + bwd_bytes) / ((res["fwd"] + res["bwd"]) * 1e-3) / 1e9, 1)}


def load_valu(run_key: str):
    """Committed SQ_INSTS_VALU counts (wave instructions per call of each entry point) of the
    configuration `run_key`, if they were taken on the current sources (all files); else None."""
    path = os.path.join(ROOT, "profiles", "valu_counts.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash_all") != kernel_source_hash("all"):
        return None
    return rec.get("runs", {}).get(run_key)


def roofline_for(kernel: str, bwd_bytes: int, fwd_bytes: int, bwd_ms: float, fwd_ms: float,
                 run_key: str, traffic=None, ceiling_gbps=None) -> dict:
    """Roofline object of the backward call (the dominant one). With committed VALU counts for
    this configuration the kernels' VALU busy fraction is known: when it exceeds the HBM fraction
    the call is bound by VALU issue and reported against PEAK_VALU_GINSTR, else against HBM."""
    hbm = bwd_bytes / (bwd_ms * 1e-3) / 1e9
    out = {"bound": "hbm", "kernel": kernel, "achieved": round(hbm, 1), "peak": PEAK_HBM_GBPS,
           "unit": "GB/s", "frac": round(hbm / PEAK_HBM_GBPS, 4), "traffic": traffic,
           "fwd_achieved": round(fwd_bytes / (fwd_ms * 1e-3) / 1e9, 1)}
    if ceiling_gbps:
        # the same backward traffic moved by the stream probe: the practical ceiling
        out["ceiling"] = ceiling_gbps
        out["frac_of_ceiling"] = round(hbm / ceiling_gbps, 4)
    v = load_valu(run_key)
    if v is not None:
        valu = v["bwd_call_valu_instr"] / (bwd_ms * 1e-3) / 1e9
        out["valu_achieved_ginstr"] = round(valu, 1)
        out["valu_frac"] = round(valu / PEAK_VALU_GINSTR, 4)
        out["fwd_valu_frac"] = round(v["fwd_call_valu_instr"] / (fwd_ms * 1e-3) / 1e9
                                     / PEAK_VALU_GINSTR, 4)
        if valu / PEAK_VALU_GINSTR > hbm / PEAK_HBM_GBPS:
            out.update({"bound": "alu", "achieved": round(valu, 1), "peak": PEAK_VALU_GINSTR,
                        "unit": "G VALU instr/s", "frac": round(valu / PEAK_VALU_GINSTR, 4),
                        "hbm_achieved": round(hbm, 1), "hbm_frac": round(hbm / PEAK_HBM_GBPS, 4)})
    return out


def input_checksums(x: dict) -> dict:
    """FP64 sum of every input tensor (taken after the timed steps): identifies the synthetic
    inputs a line was measured on."""
    import torch
    return {k: float(torch.sum(v, dtype=torch.float64).item()) for k, v in x.items()
            if v is not None}


def load_traffic(workload: str, scope: str = "single"):
    """HBM traffic of the backward call from committed rocprofv3 counter summaries, if they were
    taken on the current kernel sources (same source hash over `scope`, as kernel_source_hash);
    else None."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(scope):
        return None
    return rec.get("bwd_call_hbm_bytes")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 50 warm-up steps: on a fresh box the first ~10 ms of launches run host-bound (a short-token
    # step measured 0.43 ms per step there and 0.19 ms once warm)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="bf16_s10_n32768_d4096")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--accumulate", action="store_true",
                    help="the backward adds into existing dvalues (reads them: +S*N*D elements)")
    ap.add_argument("--queries", type=int, default=0, metavar="M",
                    help="time the multi-query read with M queries on the workload's sources "
                         "(no key-norm weight, no output norm)")
    ap.add_argument("--layout", default="query_major", choices=["query_major", "token_major"],
                    help="output layout of the multi-query read")
    ap.add_argument("--bank", type=int, default=0, metavar="E",
                    help="time the selected-query read: per-token queries from an [E, R] bank "
                         "(with --slots K ids per token, uniform over the bank)")
    ap.add_argument("--slots", type=int, default=2, metavar="K",
                    help="queries per token of the selected-query read")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time the oracle baseline repeats its pass for")
    ap.add_argument("--check", type=int, default=1, help="sampled-token parity check (0 = off)")
    # every event record costs the GPU ~3 us (three per step slowed the headline step by 0.7% and
    # the short-token step by 5.5%), so the per-call events bracket every E-th timed step only
    ap.add_argument("--event-every", type=int, default=5, metavar="E",
                    help="record the per-call HIP events on every E-th timed step")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the read "
              "shards over tokens, so N GPUs run N independent copies of this step plus one "
              "small all-reduce of the q/w gradients.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}), flush=True)
        return 0

    import attention_residuals_amd as A
    import attnres_workloads as W

    w = W.ALL[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.bank:
        return run_selected(args, w)
    if args.queries:
        return run_multi(args, w)
    x = W.generate(w, device=dev)
    N, D, S, R = w.N, w.D, w.S, w.R
    desc = A.make_desc(S, N, D, R, w.torch_dtype, eps=w.eps, scale=w.scale,
                       has_norm_weight=x["norm_w"] is not None, out_norm=w.out_norm,
                       has_out_weight=x["out_w"] is not None, accumulate_dvalues=args.accumulate)
    y = torch.empty((N, D), dtype=w.torch_dtype, device=dev)
    lse = torch.empty((N,), dtype=torch.float32, device=dev)
    rstd = torch.empty((N,), dtype=torch.float32, device=dev) if w.out_norm else None
    o32 = torch.empty((N, D), dtype=torch.float32, device=dev) if A.o32_elems(desc) else None
    dv = (torch.zeros if args.accumulate else torch.empty)((S, N, D), dtype=w.torch_dtype, device=dev)
    dq = torch.empty((R,), dtype=w.torch_dtype, device=dev)
    dw = torch.empty((R,), dtype=w.torch_dtype, device=dev) if x["norm_w"] is not None else None
    dow = torch.empty((D,), dtype=w.torch_dtype, device=dev) if x["out_w"] is not None else None
    # counters zero before first use (the library leaves them zero after every call)
    ws = torch.zeros((max(A.workspace_bytes(desc), 256),), dtype=torch.uint8, device=dev)
    fws = torch.zeros((A.fwd_workspace_bytes(desc),), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    # both calls marshalled once (the C entry points then run with a few microseconds of host
    # time per call, so short steps do not leave the GPU waiting for the Python loop)
    fwd = A.bind_fwd(x["values"], x["query"], x["norm_w"], x["out_w"], eps=w.eps,
                     scale=w.scale, out_norm=w.out_norm, out=y, lse=lse, out_rstd=rstd,
                     o32=o32, workspace=fws, stream=stream)
    bwd = A.bind_bwd(x["values"], x["query"], x["norm_w"], x["out_w"], lse, rstd, o32,
                     x["dout"], eps=w.eps, scale=w.scale, out_norm=w.out_norm,
                     accumulate=args.accumulate, dvalues=dv, dq=dq, dw=dw, dow=dow,
                     workspace=ws, stream=stream)

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()

    # timed region: K steps, events around the two calls of every E-th step
    every = max(1, args.event_every)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
          for _ in range((args.steps + every - 1) // every)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        e = ev[k // every] if k % every == 0 else None
        if e:
            e[0].record(stream)
        fwd()
        if e:
            e[1].record(stream)
        bwd()
        if e:
            e[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [e[0].elapsed_time(e[1]) for e in ev]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in ev]
    ms_per_step = wall * 1e3 / args.steps
    ev_step = [a + b for a, b in zip(fwd_ms, bwd_ms)]

    algo = w.algorithmic_bytes() + (S * N * D * w.elem_bytes if args.accumulate else 0)
    b = w.elem_bytes
    bwd_bytes = ((3 if args.accumulate else 2) * S + 1) * N * D * b + 4 * N * (2 if w.out_norm else 1)
    fwd_bytes = (S + 1) * N * D * b + 4 * N * (2 if w.out_norm else 1)
    bwd_avg = float(np.mean(bwd_ms))
    fwd_avg = float(np.mean(fwd_ms))
    achieved = bwd_bytes / (bwd_avg * 1e-3) / 1e9
    value = algo / (ms_per_step * 1e-3) / 1e9

    check = None
    if args.check and args.accumulate:
        # the timed steps summed their gradients into dv: start from zero for the check
        dv.zero_()
        fwd()
        bwd()
        torch.cuda.synchronize()
    if args.check:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from parity import check_all, run_oracle, sample_tokens
        toks = sample_tokens(N, 6, seed=7)
        sel = torch.tensor(toks, device=dev)
        xc = {"values": x["values"].index_select(1, sel).cpu(), "dout": x["dout"].index_select(0, sel).cpu()}
        xc.update({k: (None if x[k] is None else x[k].cpu()) for k in ("query", "norm_w", "out_w")})
        wt = w.with_(N=len(toks))
        ref = run_oracle(wt, xc, reduce=False)
        got = {"y": y, "lse": lse, "o_rstd": rstd, "dvalues": dv, "dq": dq, "dw": dw, "dow": dow}
        res = check_all(w, got, ref, tokens=toks, check_reduced=False)
        check = {k: {"metric": v["metric"], "ok": bool(v["ok"])} for k, v in res.items()}

    cpu = None
    if not args.no_cpu:
        import oracle
        xc = {k: (None if v is None else v.cpu()) for k, v in x.items()}
        # whole passes over the full workload, repeated until about 10 s of CPU time
        reps, tc = 0, 0.0
        while reps == 0 or (tc < args.cpu_seconds and reps < 100):
            t1 = time.perf_counter()
            oracle.run(xc["values"], xc["query"], xc["norm_w"], xc["out_w"], xc["dout"],
                       eps=w.eps, scale=w.scale, out_norm=w.out_norm, want=(), reduce=True)
            tc += time.perf_counter() - t1
            reps += 1
        cpu = {"value": round(algo * reps / tc / 1e9, 3), "unit": "GB/s",
               "cores": oracle.threads_used(), "kind": "oracle", **cpu_info(),
               "ms_per_step": round(tc * 1e3 / reps, 1),
               "sample": f"{reps} passes over the full workload ({S} sources x {N} tokens x "
                         f"{D}), forward and backward with the dq/dw reduction, FP64, OpenMP "
                         f"over tokens, {tc:.1f} s in total"}

    # the practical ceiling: the same row streams moved with no arithmetic (after the check: the
    # probe overwrites y and dvalues)
    # probe overwrites y and dvalues). Not with accumulation: its backward reads and writes the
    # same dvalues rows, which the probe's disjoint streams cannot express.
    ceiling = None
    if not args.accumulate:
        vs = [x["values"][s] for s in range(S)]
        ceiling = stream_ceiling((vs, [y]), (vs + [x["dout"]], [dv[s] for s in range(S)]),
                                 fwd_bytes, bwd_bytes)
        ceiling["value_frac"] = round(value / ceiling["step_GBps"], 4)
    traffic = None if args.accumulate else load_traffic(w.name)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(B200_MS[w.name] / ms_per_step, 3) if w.name in B200_MS else None),
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "S": S, "N": N, "D": D, "R": R,
                   "norm_weight": w.norm_weight, "out_norm": w.out_norm,
                   "accumulate_dvalues": args.accumulate,
                   "algorithmic_bytes": algo, "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBPS, 1),
                   "fwd_ms": round(fwd_avg, 4), "bwd_ms": round(bwd_avg, 4),
                   "event_ms_per_step": round(float(np.mean(ev_step)), 4),
                   # per-step HIP-event times of fwd + bwd: median and 10th / 90th percentiles
                   "event_ms_step_median": round(float(np.median(ev_step)), 4),
                   "event_ms_step_p10": round(float(np.percentile(ev_step, 10)), 4),
                   "event_ms_step_p90": round(float(np.percentile(ev_step, 90)), 4),
                   "b200_ms_context": B200_MS.get(w.name),
                   "input_checksums_f64": input_checksums(x)},
        "roofline": roofline_for("attnres_bwd (backward kernel + finaliser)", bwd_bytes, fwd_bytes,
                                 bwd_avg, fwd_avg,
                                 w.name + ("_accumulate" if args.accumulate else ""), traffic,
                                 ceiling["bwd_GBps"] if ceiling else None),
        "practical_ceiling": ceiling,
        "cpu_baseline": cpu,
        "parity_check": check,
        "source_hash": kernel_source_hash(),
    }
    print(json.dumps(out), flush=True)
    return 0


def _timed(args, fwd, bwd, stream):
    """Warm-up, then K timed steps with HIP events around the calls of every E-th step (on the
    launch stream)."""
    import numpy as np
    import torch
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    every = max(1, args.event_every)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
          for _ in range((args.steps + every - 1) // every)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        e = ev[k // every] if k % every == 0 else None
        if e:
            e[0].record(stream)
        fwd()
        if e:
            e[1].record(stream)
        bwd()
        if e:
            e[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    return wall * 1e3 / args.steps, fwd_ms, bwd_ms


def run_multi(args, w) -> int:
    """The multi-query read ("Fast Attention Residuals" page, Multi-query AttnRes) with M queries
    over the workload's sources; one JSON line like the default mode."""
    import numpy as np
    import torch
    import attention_residuals_amd as A
    import attnres_workloads as W

    dev = "cuda:0"
    M, S, N, D, R = args.queries, w.S, w.N, w.D, w.R
    x = W.generate(w, device=dev, with_dout=False)
    values = x["values"]
    del x
    mi = W.multi_inputs(w, M, args.layout, device=dev)
    queries, dout = mi["queries"], mi["dout"]
    shape = tuple(dout.shape)
    desc = A.make_multi_desc(S, N, D, R, M, w.torch_dtype, eps=w.eps, scale=w.scale,
                             layout=args.layout, accumulate_dvalues=args.accumulate)
    y = torch.empty(shape, dtype=w.torch_dtype, device=dev)
    lse = torch.empty(shape[:2], dtype=torch.float32, device=dev)
    dv = (torch.zeros if args.accumulate else torch.empty)((S, N, D), dtype=w.torch_dtype,
                                                           device=dev)
    dq = torch.empty((M, R), dtype=w.torch_dtype, device=dev)
    ws = torch.empty((max(A.multi_workspace_bytes(desc), 256),), dtype=torch.uint8, device=dev)
    fws = torch.empty((A.multi_fwd_workspace_bytes(desc),), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def fwd():
        A.attnres_multi_fwd(values, queries, eps=w.eps, scale=w.scale, layout=args.layout,
                            out=y, lse=lse, workspace=fws, stream=stream)

    def bwd():
        A.attnres_multi_bwd(values, queries, lse, dout, eps=w.eps, scale=w.scale,
                            layout=args.layout, accumulate=args.accumulate, dvalues=dv, dq=dq,
                            workspace=ws, stream=stream)

    ms, fwd_ms, bwd_ms = _timed(args, fwd, bwd, stream)
    b = w.elem_bytes
    acc = S * N * D * b if args.accumulate else 0
    fwd_bytes = (S + M) * N * D * b + 4 * M * N
    bwd_bytes = (2 * S + M) * N * D * b + 4 * M * N + acc
    algo = fwd_bytes + bwd_bytes
    value = algo / (ms * 1e-3) / 1e9

    check = None
    if args.check:
        if args.accumulate:
            dv.zero_()
        fwd()
        bwd()
        torch.cuda.synchronize()
        import oracle
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from parity import compare_rows, compare_stat, multi_bwd_passes, sample_tokens
        toks = sample_tokens(N, 6, seed=7)
        sel = torch.tensor(toks, device=dev)
        gq = dout if args.layout == "query_major" else dout.transpose(0, 1)
        yq = y if args.layout == "query_major" else y.transpose(0, 1)
        lq = lse if args.layout == "query_major" else lse.transpose(0, 1)
        ref = oracle.run_multi(values.index_select(1, sel).cpu(), queries.cpu(),
                               gq.index_select(1, sel).cpu(), eps=w.eps, scale=w.scale,
                               reduce=False)
        f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()
        groups = multi_bwd_passes(S, D, M, w.dtype)
        res = {"y": compare_rows(f64(yq.index_select(1, sel)).reshape(-1, D),
                                 ref["y"].reshape(-1, D), w.dtype),
               "lse": compare_stat(f64(lq.index_select(1, sel)), ref["lse"]),
               "dvalues": compare_rows(f64(dv.index_select(1, sel)), ref["dvalues"], w.dtype,
                                       roundings=groups)}
        check = {k: {"metric": v["metric"], "ok": bool(v["ok"])} for k, v in res.items()}

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}_multi_m{M}_{args.layout}", "S": S, "N": N, "D": D,
                   "R": R, "M": M, "layout": args.layout, "accumulate_dvalues": args.accumulate,
                   "algorithmic_bytes": algo,
                   "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBPS, 1),
                   "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4)},
        "roofline": roofline_for("attnres_multi_bwd (backward kernels + finaliser)", bwd_bytes,
                                 fwd_bytes, bwd_ms, fwd_ms, f"{w.name}_multi_m{M}_{args.layout}",
                                 None if args.accumulate else
                                 load_traffic(f"{w.name}_multi_m{M}_{args.layout}", "all")),
        "cpu_baseline": None,
        "parity_check": check,
        "source_hash": kernel_source_hash("all"),
    }
    print(json.dumps(out), flush=True)
    return 0


def run_selected(args, w) -> int:
    """The selected-query read ("Fast Attention Residuals" page, Multi-query AttnRes: per-token
    query selection) with K ids per token, uniform over an [E, R] bank; one JSON line."""
    import torch
    import attention_residuals_amd as A
    import attnres_workloads as W

    dev = "cuda:0"
    E, K, S, N, D, R = args.bank, args.slots, w.S, w.N, w.D, w.R
    x = W.generate(w, device=dev, with_dout=False)
    values = x["values"]
    del x
    si = W.selected_inputs(w, E, K, device=dev)
    bank, ids, dout = si["bank"], si["ids"], si["dout"]
    desc = A.make_selected_desc(S, N, D, R, E, K, w.torch_dtype, eps=w.eps, scale=w.scale,
                                accumulate_dvalues=args.accumulate)
    y = torch.empty((N, K, D), dtype=w.torch_dtype, device=dev)
    lse = torch.empty((N, K), dtype=torch.float32, device=dev)
    dv = (torch.zeros if args.accumulate else torch.empty)((S, N, D), dtype=w.torch_dtype,
                                                           device=dev)
    dbank = torch.empty((E, R), dtype=w.torch_dtype, device=dev)
    ws = torch.empty((max(A.selected_workspace_bytes(desc), 256),), dtype=torch.uint8, device=dev)
    fws = torch.empty((A.selected_fwd_workspace_bytes(desc),), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def fwd():
        A.attnres_selected_fwd(values, bank, ids, eps=w.eps, scale=w.scale, out=y, lse=lse,
                               workspace=fws, stream=stream)

    def bwd():
        A.attnres_selected_bwd(values, bank, ids, lse, dout, eps=w.eps, scale=w.scale,
                               accumulate=args.accumulate, dvalues=dv, dbank=dbank, workspace=ws,
                               stream=stream)

    ms, fwd_ms, bwd_ms = _timed(args, fwd, bwd, stream)
    b = w.elem_bytes
    acc = S * N * D * b if args.accumulate else 0
    # sources, outputs / output gradients, lse and ids per token; the bank (and its gradient) once
    fwd_bytes = (S + K) * N * D * b + 12 * K * N + E * R * b
    bwd_bytes = (2 * S + K) * N * D * b + 12 * K * N + 2 * E * R * b + acc
    algo = fwd_bytes + bwd_bytes
    value = algo / (ms * 1e-3) / 1e9

    check = None
    if args.check:
        if args.accumulate:
            dv.zero_()
        fwd()
        bwd()
        torch.cuda.synchronize()
        import oracle
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from parity import compare_rows, compare_stat, multi_bwd_passes, sample_tokens
        toks = sample_tokens(N, 6, seed=7)
        sel = torch.tensor(toks, device=dev)
        ref = oracle.run_selected(values.index_select(1, sel).cpu(), bank.cpu(),
                                  ids.index_select(0, sel).cpu(),
                                  dout.index_select(0, sel).cpu(), eps=w.eps, scale=w.scale,
                                  reduce=False)
        f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()
        res = {"y": compare_rows(f64(y.index_select(0, sel)).reshape(-1, D),
                                 ref["y"].reshape(-1, D), w.dtype),
               "lse": compare_stat(f64(lse.index_select(0, sel)), ref["lse"]),
               "dvalues": compare_rows(f64(dv.index_select(1, sel)), ref["dvalues"], w.dtype,
                                       roundings=multi_bwd_passes(S, D, K, w.dtype,
                                                                  selected=True, R=R, E=E))}
        check = {k: {"metric": v["metric"], "ok": bool(v["ok"])} for k, v in res.items()}

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}_selected_e{E}_k{K}", "S": S, "N": N, "D": D, "R": R,
                   "E": E, "K": K, "accumulate_dvalues": args.accumulate,
                   "algorithmic_bytes": algo,
                   "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBPS, 1),
                   "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4)},
        "roofline": roofline_for("attnres_selected_bwd (backward kernels + finaliser)", bwd_bytes,
                                 fwd_bytes, bwd_ms, fwd_ms, f"{w.name}_selected_e{E}_k{K}",
                                 None if args.accumulate else
                                 load_traffic(f"{w.name}_selected_e{E}_k{K}", "all")),
        "cpu_baseline": None,
        "parity_check": check,
        "source_hash": kernel_source_hash("all"),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
