#!/usr/bin/env python3
"""Relation-KL forward+backward benchmark on one MI355X.

One step = the whole linear-memory relation-KL path over every relation map
of the workload (Q/Q, K/K, V/V), each map being: phase 1 (per-row LSE),
phase 2 row sweep (row KL + row term of dX_s), phase 2 column sweep (column
term of dX_s) and the fp64 loss reduction, launched exactly as `larard_loss`
launches them.  Inputs are resident in HBM before timing starts.

Prints ONE JSON line.  `value` is the step's algorithmic TFLOP/s: causal
relation KL does 6 contractions of depth d over the n(n+1)/2 unmasked pairs
per head-map (2 in phase 1, 4 in phase 2), i.e. 6*d*n*(n+1) flops; split
mode's extra recompute is not counted.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="llama2_16k")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-n", type=int, default=0,
                   help="sequence length of the oracle sample (default: the workload's n)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="before warm-up, run one fp32 elementwise copy (y = x * 1) of this many MiB; "
                        "its FETCH_SIZE/WRITE_SIZE counters calibrate the HBM traffic figures")
    p.add_argument("--summarize", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "COPY_MIB"),
                   help="write the markdown summary of rocprofv3 kernel-trace/stats and FETCH_SIZE/WRITE_SIZE "
                        "runs of this script to stdout and exit")
    p.add_argument("--trace-cmd", default="", help="(with --summarize) command lines to record in the summary")
    p.add_argument("--core-only", action="store_true",
                   help="time only the step (and its one-call check): skip the forward-only, fused-map, "
                        "projection and cross-relation sections, whose launches share kernel symbols with "
                        "the step and would mix into a profiler's per-kernel averages")
    return p.parse_args()


def causal_pairs(n: int) -> int:
    return n * (n + 1) // 2


def cpu_baseline(w, maps, sample_n: int):
    """Time the fp64 oracle on two head-maps (Q/Q and K/K of b=0, h=0) on the host cores."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    n = sample_n or w.n
    names = [k for k in ("Q", "K") if k in maps] or list(maps)[:1]
    dt = 0.0
    for name in names:
        xt, xs = maps[name].head64(0, 0)
        xt, xs = xt[:n], xs[:n]
        t0 = time.perf_counter()
        r = oracle.relation_kl_head(xt, xs, w.scale, True)
        dt += time.perf_counter() - t0
        assert np.isfinite(r["loss"])
        del r
    flops = len(names) * 12.0 * w.d * causal_pairs(n)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"{len(names)} head-maps ({', '.join(k + '/' + k for k in names)} of b=0, h=0) of {w.name} "
                      f"at n={n}, d={w.d}: dense fp64 numpy oracle (loss, LSE, row KL, dX_s); "
                      f"algorithmic flops 12*d*n(n+1)/2 per head-map"}


# ---------------------------------------------------------------------------
# rocprofv3 summaries (kernel trace + HBM traffic), kept as text under profiles/
# ---------------------------------------------------------------------------
def library_source_id() -> str:
    """Stamp of the built library (hash of its sources); loading it needs no GPU."""
    import linear_memory_relation_amd as lmr
    from linear_memory_relation_amd.build import source_id
    got = lmr.source_id()
    if got != source_id():
        raise SystemExit(f"liblarard.so (src {got}) was not built from the current sources "
                         f"(src {source_id()}); rebuild before profiling or summarising")
    return got


def kernel_kind(name: str) -> str:
    if "lse_fwd_kernel" in name:
        return "lse_fwd"
    if "kl_sweep_kernel" in name:
        return "kl_rows" if ", 0, " in name else "kl_cols"
    if "reduce_rows_kernel" in name or "reduce_final_kernel" in name:
        return "reduce"
    if "MulFunctor" in name:
        return "copy_calibration"
    return "other"


def _csv_rows(d: str, suffix: str):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no *{suffix} under {d}")
    return rows


def _pmc_per_dispatch(d: str, counter: str):
    """Mean of `counter` (KiB) per dispatch, by kernel name."""
    per = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        key = (r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id")))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return {k: (float(np.mean(v)), len(v)) for k, v in out.items()}


def summarize(trace_dir: str, fetch_dir: str, write_dir: str, copy_mib: str, cmds: str) -> str:
    copy_bytes = int(copy_mib) * 2 ** 20
    stats = _csv_rows(trace_dir, "kernel_stats.csv")
    fetch = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_dir, "WRITE_SIZE")
    lines = ["# Kernel time and HBM traffic of one relation-KL step (llama2_16k workload)", ""]
    lines += ["Workload: B=1, H=32, n=16384, d=128, bf16, maps Q/Q, K/K, V/V, causal, split dX mode.", ""]
    lines += [f"Library: {__import__('linear_memory_relation_amd').version()}", ""]
    lines += ["Commands (run from the repository root; rocprofv3 wrote CSV under the -d directory):", "", "```"]
    lines += [c for c in cmds.split(";;") if c] + ["```", ""]
    lines += ["## Kernel trace (rocprofv3 --kernel-trace --stats)", ""]
    lines += ["| kernel | kind | calls | avg ms | min ms | max ms | share of GPU time |", "|---|---|---|---|---|---|---|"]
    def col(r, *names):
        for k in names:
            for kk in r:
                if kk.lower().replace("_", "") == k.lower().replace("_", ""):
                    return r[kk]
        raise SystemExit(f"column {names} not in {list(r)}")
    for r in sorted(stats, key=lambda r: -float(col(r, "TotalDurationNs"))):
        name = col(r, "Name", "KernelName", "Kernel_Name")
        lines.append(f"| `{name[:90]}` | {kernel_kind(name)} | {col(r, 'Calls')} | "
                     f"{float(col(r, 'AverageNs')) / 1e6:.4f} | {float(col(r, 'MinNs')) / 1e6:.4f} | "
                     f"{float(col(r, 'MaxNs')) / 1e6:.4f} | {float(col(r, 'Percentage')):.2f}% |")
    cal = [k for k in fetch if kernel_kind(k) == "copy_calibration"]
    if not cal or not [k for k in write if kernel_kind(k) == "copy_calibration"]:
        raise SystemExit("calibration copy kernel not found in the counter runs")
    f_cal = fetch[cal[0]][0] * 1024 / copy_bytes
    w_cal = write[[k for k in write if kernel_kind(k) == "copy_calibration"][0]][0] * 1024 / copy_bytes
    lines += ["", "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)", ""]
    lines += [f"Calibration: an fp32 copy of {copy_mib} MiB reads and writes {copy_bytes} bytes; its counters read "
              f"FETCH_SIZE x {f_cal:.4f} and WRITE_SIZE x {w_cal:.4f} of that, and every figure below is divided "
              f"by these factors.", ""]
    lines += ["| kernel | kind | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (calibrated) |",
              "|---|---|---|---|---|---|"]
    traffic = {}
    for name, (fk, cnt) in sorted(fetch.items(), key=lambda kv: -kv[1][0]):
        wk = write.get(name, (0.0, 0))[0]
        tb = fk * 1024 / f_cal + wk * 1024 / w_cal
        kind = kernel_kind(name)
        if kind in ("lse_fwd", "kl_rows", "kl_cols"):
            traffic[kind] = tb
        lines.append(f"| `{name[:90]}` | {kind} | {cnt} | {fk:.1f} | {wk:.1f} | {tb:.4e} |")
    lines += ["", "Machine-readable (read by bench.py while the kernel sources are unchanged):", ""]
    lines.append(f"library_source_id: {library_source_id()}")
    for k, v in sorted(traffic.items()):
        lines.append(f"traffic_bytes_per_launch {k}: {v:.6e}")
    return "\n".join(lines) + "\n"


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "kernel_trace_and_traffic_llama2_16k.md")


def recorded_traffic(kind: str, workload: str):
    """Calibrated HBM bytes per launch of `kind` from the committed summary, or None when the
    summary is missing, covers another workload or was taken on a library built from other sources."""
    import linear_memory_relation_amd as lmr
    if workload != "llama2_16k" or not os.path.exists(TRAFFIC_SUMMARY):
        return None
    src, val = None, None
    with open(TRAFFIC_SUMMARY) as f:
        for line in f:
            if line.startswith("library_source_id:"):
                src = line.split(":", 1)[1].strip()
            if line.startswith(f"traffic_bytes_per_launch {kind}:"):
                val = float(line.split(":", 1)[1])
    if src != lmr.source_id():
        return None
    return val


def extra_sections(args, bufs, w, scale, dev, units, step_flops):
    """Timings beside the step: forward-only loss, all maps fused in one launch
    per phase, the projection backward and the query/key cross relation."""
    import torch
    import linear_memory_relation_amd as lmr
    # Forward-only loss (one phase-1 sweep with the KL accumulator + reduce),
    # timed the same way: 2 GEMM-units per head-map.
    def fwd_step():
        for b in bufs:
            lmr.kl_fwd(b["xt"], b["xs"], scale, True, b["lse_t"], b["lse_s"], b["row_kl"])
            lmr.reduce_loss(b["row_kl"], b["partials"], b["loss"], 1.0)
    for _ in range(args.warmup):
        fwd_step()
    torch.cuda.synchronize()
    s3, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s3.record()
    for _ in range(args.steps):
        fwd_step()
    e3.record()
    torch.cuda.synchronize()
    ms_fwd = s3.elapsed_time(e3) / args.steps
    losses_fwd = {b["name"]: float(b["loss"].cpu()) for b in bufs}
    fwd_info = {"ms_per_step": round(ms_fwd, 4),
                "tflops": round(sum(2 * units(b) for b in bufs) / (ms_fwd * 1e-3) / 1e12, 3),
                "pct_bf16_peak": round(100 * sum(2 * units(b) for b in bufs) / (ms_fwd * 1e-3) / 1e12
                                       / PEAK_BF16_TFLOPS, 2),
                "losses": losses_fwd,
                "what": "larard_kl_fwd + reduce per map; algorithmic flops 2 GEMM-units per head-map"}

    # The same step with every map in one launch per phase (larard_multi_loss).
    wsm = torch.empty(lmr.multi_workspace_bytes([(b["xt"], b["xs"], 1.0, b["dx"]) for b in bufs]),
                      dtype=torch.uint8, device=dev)
    mlist = [(b["xt"], b["xs"], 1.0, b["dx"]) for b in bufs]
    mloss = torch.empty((), dtype=torch.float32, device=dev)

    def fused_step():
        lmr.multi_loss(mlist, scale, True, 1.0, workspace=wsm, out=mloss)
    for _ in range(args.warmup):
        fused_step()
    torch.cuda.synchronize()
    s5, e5 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s5.record()
    for _ in range(args.steps):
        fused_step()
    e5.record()
    torch.cuda.synchronize()
    ms_fused = s5.elapsed_time(e5) / args.steps
    fused_info = {"ms_per_step": round(ms_fused, 4),
                  "tflops": round(step_flops / (ms_fused * 1e-3) / 1e12, 3),
                  "loss_sum": float(mloss.cpu()),
                  "what": "all maps in one launch per phase (larard_multi_loss, weights 1)"}
    del wsm

    # Projection backward of the first map: dW = h^T R^T(dX_s) with synthetic
    # bf16 hidden states of model width H*d and the student rotation (PI).
    proj = None
    bq0 = bufs[0]
    dm = bq0["H"] * bq0["d"]
    if dm % 128 == 0:
        g = torch.Generator(device=dev)
        g.manual_seed(1234)
        hst = torch.randn((bq0["B"], bq0["n"], dm), generator=g, device=dev).to(torch.bfloat16)
        pos = torch.arange(bq0["n"], dtype=torch.float64) / (w.factor if w.kind == "pi" else 1.0)
        inv = (w.base * (w.factor ** (bq0["d"] / (bq0["d"] - 2)) if w.kind == "ntk" else w.base)) ** (
            -2.0 * torch.arange(bq0["d"] // 2, dtype=torch.float64) / bq0["d"])
        ang = torch.outer(pos, inv)
        rc, rs = torch.cos(ang).float().to(dev), torch.sin(ang).float().to(dev)
        wsp = torch.empty(int(lmr.load().larard_proj_bwd_workspace_bytes(bq0["B"], bq0["n"], dm, bq0["H"], bq0["d"])),
                          dtype=torch.uint8, device=dev)
        dW = torch.empty((dm, dm), dtype=torch.float32, device=dev)
        for _ in range(args.warmup):
            lmr.proj_bwd(hst, bq0["dx"], rc, rs, workspace=wsp, out=dW)
        torch.cuda.synchronize()
        s6, e6 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s6.record()
        for _ in range(args.steps):
            lmr.proj_bwd(hst, bq0["dx"], rc, rs, workspace=wsp, out=dW)
        e6.record()
        torch.cuda.synchronize()
        ms_p = s6.elapsed_time(e6) / args.steps
        pflops = 2.0 * dm * dm * bq0["B"] * bq0["n"]
        proj = {"ms": round(ms_p, 4), "tflops": round(pflops / (ms_p * 1e-3) / 1e12, 3),
                "pct_bf16_peak": round(100 * pflops / (ms_p * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                "what": f"larard_proj_bwd for map {bq0['name']}: dW [{dm}x{dm}] = h^T R^T(dX_s), "
                        f"K = B*n = {bq0['B'] * bq0['n']}; synthetic bf16 h; flops 2*dm*H*d*B*n"}
        del hst, wsp, dW

    # General relation X != Y on the same data: the query/key map (X = Q,
    # Y = K), fwd+bwd through one larard_xy_loss call (dX_s and dY_s).
    cross = None
    names = [b["name"] for b in bufs]
    if "Q" in names and "K" in names:
        bq, bk = bufs[names.index("Q")], bufs[names.index("K")]
        if bq["xt"].shape == bk["xt"].shape:
            wsx = torch.empty(lmr.workspace_bytes(bq["B"], bq["H"], bq["n"]), dtype=torch.uint8, device=dev)
            dyq = torch.empty_like(bq["dx"])

            def cross_step():
                lmr.xy_loss(bq["xt"], bq["xs"], bk["xt"], bk["xs"], scale, True, 1.0, workspace=wsx,
                            out=bq["loss"], dx=bq["dx"], dy=dyq)
            for _ in range(args.warmup):
                cross_step()
            torch.cuda.synchronize()
            s4, e4 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s4.record()
            for _ in range(args.steps):
                cross_step()
            e4.record()
            torch.cuda.synchronize()
            ms_x = s4.elapsed_time(e4) / args.steps
            cross = {"ms_per_map": round(ms_x, 4),
                     "tflops": round(6 * units(bq) / (ms_x * 1e-3) / 1e12, 3),
                     "pct_bf16_peak": round(100 * 6 * units(bq) / (ms_x * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                     "loss": float(bq["loss"].cpu()),
                     "what": "query/key relation (X=Q, Y=K) via larard_xy_loss: LSE, row KL, dX_s and dY_s; "
                             "6 GEMM-units per head"}
            del wsx, dyq
    return fwd_info, proj, cross, fused_info


def main():
    args = parse()
    if args.summarize:
        sys.stdout.write(summarize(*args.summarize, args.trace_cmd))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this kernel shards by heads "
              f"with no exchange but a scalar loss sum; this benchmark measures a single GPU.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_memory_relation_amd as lmr
    import synth_inputs as si

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lmr.load()
    dev = torch.device("cuda:0")
    w = si.WORKLOADS[args.workload]
    maps = si.make_inputs(w)
    scale = w.scale

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    torch.cuda.synchronize()
    base_alloc = torch.cuda.memory_allocated()
    bufs = []
    for name, m in maps.items():
        B, H, n, d = m.xt.shape
        bufs.append(dict(
            name=name, B=B, H=H, n=n, d=d, xt=to_dev(m.xt), xs=to_dev(m.xs),
            lse_t=torch.empty((B, H, n), dtype=torch.float64, device=dev),
            lse_s=torch.empty((B, H, n), dtype=torch.float64, device=dev),
            row_kl=torch.empty((B, H, n), dtype=torch.float32, device=dev),
            partials=torch.empty((B * H,), dtype=torch.float64, device=dev),
            dx=torch.empty((B, H, n, d), dtype=torch.float32, device=dev),
            loss=torch.empty((), dtype=torch.float32, device=dev)))
    input_bytes = sum(b["xt"].numel() * 2 * 2 for b in bufs)
    dx_bytes = sum(b["dx"].numel() * 4 for b in bufs)
    stat_bytes = sum(b["lse_t"].numel() * (8 + 8 + 4) + b["partials"].numel() * 8 for b in bufs)
    torch.cuda.synchronize()
    if args.calib_copy_mib > 0:
        src = torch.ones(args.calib_copy_mib * 2 ** 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.reset_peak_memory_stats()

    kinds = ["lse_fwd", "kl_rows", "kl_cols", "reduce"]

    def step(events=None):
        for b in bufs:
            a = (b["xt"], b["xs"])
            if events is not None:
                events[b["name"]][0].record()
            lmr.lse_fwd(*a, scale, True, b["lse_t"], b["lse_s"])
            if events is not None:
                events[b["name"]][1].record()
            lmr.kl_bwd_rows(*a, b["lse_t"], b["lse_s"], b["row_kl"], b["dx"], scale, True, 1.0)
            if events is not None:
                events[b["name"]][2].record()
            lmr.kl_bwd_cols(*a, b["lse_t"], b["lse_s"], b["dx"], scale, True, 1.0)
            if events is not None:
                events[b["name"]][3].record()
            lmr.reduce_loss(b["row_kl"], b["partials"], b["loss"], 1.0)
            if events is not None:
                events[b["name"]][4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps with HIP events around every kernel, on the stream
    # the kernels are launched on (torch's current stream).
    ev = [{b["name"]: [torch.cuda.Event(enable_timing=True) for _ in range(5)] for b in bufs}
          for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for k in range(args.steps):
        step(ev[k])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    per_kernel = {k: [] for k in kinds}
    for k in range(args.steps):
        for b in bufs:
            e = ev[k][b["name"]]
            for j, kind in enumerate(kinds):
                per_kernel[kind].append(e[j].elapsed_time(e[j + 1]))
    peak_alloc = torch.cuda.max_memory_allocated() - base_alloc

    # Independent check of the one-call path: same kernels, no events.
    torch.cuda.synchronize()
    s2, e2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ws = [torch.empty(lmr.workspace_bytes(b["B"], b["H"], b["n"]), dtype=torch.uint8, device=dev) for b in bufs]
    s2.record()
    for _ in range(args.steps):
        for b, wsb in zip(bufs, ws):
            lmr.loss(b["xt"], b["xs"], scale, True, 1.0, workspace=wsb, out=b["loss"], dx=b["dx"])
    e2.record()
    torch.cuda.synchronize()
    ms_step_oneshot = s2.elapsed_time(e2) / args.steps
    losses = {b["name"]: float(b["loss"].cpu()) for b in bufs}

    def units(b):
        return b["B"] * b["H"] * 2 * b["d"] * causal_pairs(b["n"])
    step_flops = sum(6 * units(b) for b in bufs)

    fwd_info, proj, cross, fused_info = None, None, None, None
    if not args.core_only:
        fwd_info, proj, cross, fused_info = extra_sections(args, bufs, w, scale, dev, units, step_flops)

    # Algorithmic work.  Per head-map P = n(n+1)/2 unmasked pairs, one
    # contraction = 2*d*P flops.  Phase 1: 2 contractions; the row sweep
    # carries phase 2's recompute (2) and the row term (1); the column sweep's
    # algorithmic share is the column term (1) -- its recompute is split-mode
    # overhead and is not counted.
    alg = {"lse_fwd": 2, "kl_rows": 3, "kl_cols": 1, "reduce": 0}
    exe = {"lse_fwd": 2, "kl_rows": 3, "kl_cols": 3, "reduce": 0}
    kern = {}
    for kind in kinds:
        t = float(np.mean(per_kernel[kind]))
        fl = np.mean([alg[kind] * units(b) for b in bufs])
        fe = np.mean([exe[kind] * units(b) for b in bufs])
        kern[kind] = {"avg_ms": t, "share": float(np.sum(per_kernel[kind]) / total_ms),
                      "alg_tflops": fl / (t * 1e-3) / 1e12 if fl else 0.0,
                      "executed_tflops": fe / (t * 1e-3) / 1e12 if fe else 0.0}
    # Roofline of every sweep kernel; `roofline` is the one with the largest
    # share of the step's time (the row and column sweeps are close, so the
    # choice can differ between runs).
    def roof(kind):
        fl = float(np.mean([alg[kind] * units(b) for b in bufs]))
        ach = fl / (kern[kind]["avg_ms"] * 1e-3) / 1e12
        return {"kernel": kind, "bound": "mfma", "achieved": round(ach, 3), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": recorded_traffic(kind, w.name),
                "alg_flops_per_launch": fl,
                "executed_frac": round(kern[kind]["executed_tflops"] / PEAK_BF16_TFLOPS, 4),
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)"}
    sweeps = [k for k in kinds if alg[k] > 0]
    dom = max(kinds, key=lambda k: kern[k]["share"])
    value = step_flops / (ms_step * 1e-3) / 1e12

    out = {
        "metric": "relation-KL fwd+bwd ms/step & TFLOP/s (% bf16 MFMA peak) at H=32,d=128,n=16K",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "n": w.n, "d": w.d, "heads": w.heads,
                   "maps": list(maps), "causal": True, "scale": scale, "dx_mode": "split"},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roof(dom),
        "rooflines": {k: roof(k) for k in sweeps},
        "kernels": kern,
        "ms_per_step_one_call": round(ms_step_oneshot, 4),
        "wall_s_timed": round(wall, 3),
        "memory": {"peak_alloc_bytes_during_steps": int(peak_alloc), "inputs_bytes": input_bytes,
                   "dx_bytes": dx_bytes, "statistics_bytes": stat_bytes,
                   "bhn_bound_bytes": int(sum(20 * b["B"] * b["H"] * b["n"] for b in bufs)),
                   "dense_fp32_map_bytes_one_matrix": int(sum(4 * b["B"] * b["H"] * b["n"] ** 2 for b in bufs))},
        "losses": losses,
        "forward_only": fwd_info,
        "cross_relation": cross,
        "proj_bwd": proj,
        "fused_maps": fused_info,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, maps, args.cpu_sample_n)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
