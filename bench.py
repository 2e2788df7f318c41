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
    p.add_argument("--summarize", nargs=2, metavar=("TRACE_DIR", "COPY_MIB"),
                   help="write the markdown summary of a rocprofv3 kernel-trace/stats run of this script and of "
                        "its --pmc runs (--pmc-dir, one per counter group) to stdout and exit")
    p.add_argument("--pmc-dir", action="append", default=[],
                   help="(with --summarize) rocprofv3 -d directory of one --pmc run; repeat per counter group")
    p.add_argument("--trace-cmd", default="", help="(with --summarize) command lines to record in the summary")
    p.add_argument("--extra-workloads", default="llama2_4k,llama3_gqa_8k,llama2_32k",
                   help="comma-separated workloads timed after the headline one (same step, fewer steps); "
                        "empty to skip")
    p.add_argument("--extra-steps", type=int, default=5)
    p.add_argument("--proj-only", action="store_true",
                   help="time only the projection backward of every map of --workload (model width = the "
                        "first map's H*d) after one step has produced dX_s, and print one JSON line")
    p.add_argument("--trace-table", metavar="TRACE_DIR",
                   help="print a markdown table of every kernel of a rocprofv3 --kernel-trace run and exit")
    p.add_argument("--core-only", action="store_true",
                   help="time only the step (and its one-call check): skip the forward-only, fused-map, "
                        "projection and cross-relation sections, whose launches share kernel symbols with "
                        "the step and would mix into a profiler's per-kernel averages")
    return p.parse_args()


def causal_pairs(n: int) -> int:
    return n * (n + 1) // 2


def cpu_baseline(w, maps, sample_n: int):
    """Time the fp64 oracle on two head-maps (Q/Q and K/K of b=0, h=0) on the host cores, and
    extrapolate it (labelled as such) to the workload's whole step; the tiny fp32 workload is
    small enough to time in full."""
    import oracle
    import synth_inputs as si
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
    step_flops = w.head_maps() * 12.0 * w.d * causal_pairs(w.n)
    tiny = si.WORKLOADS["tiny_f32"]
    tq = si.make_inputs(tiny)["Q"]
    t0 = time.perf_counter()
    oracle.relation_kl(tq.xt64, tq.xs64, tiny.scale, True)
    dt_tiny = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"{len(names)} head-maps ({', '.join(k + '/' + k for k in names)} of b=0, h=0) of {w.name} "
                      f"at n={n}, d={w.d}: dense fp64 numpy oracle (loss, LSE, row KL, dX_s); "
                      f"algorithmic flops 12*d*n(n+1)/2 per head-map",
            "step_seconds_extrapolated": round(dt * step_flops / flops, 1),
            "extrapolation": f"EXTRAPOLATED: the sample's time scaled by flops to all {w.head_maps()} head-maps "
                             f"of {w.name} (every head-map of one workload costs the oracle the same)",
            "tiny_f32_full_step_seconds": round(dt_tiny, 4),
            "tiny_f32": "the whole tiny_f32 workload (1 head, n=256, d=64), timed, not extrapolated"}


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
    if "kl_fused_kernel" in name:
        return "kl_bwd"
    if "kl_sweep_kernel" in name:
        return "kl_rows" if ", 0, " in name else "kl_cols"
    if "reduce_rows_kernel" in name or "reduce_final_kernel" in name:
        return "reduce"
    if "MulFunctor" in name:
        return "copy_calibration"
    return "other"


def _find(d: str, suffix: str):
    import glob
    return sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))


def _csv_rows(d: str, suffix: str):
    import csv
    rows = []
    for path in _find(d, suffix):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no *{suffix} under {d}")
    return rows


def _db_query(d: str, sql: str):
    """Rows of `sql` over every rocprofv3 SQLite output (*_results.db) under d."""
    import sqlite3
    out = []
    for path in _find(d, "_results.db"):
        con = sqlite3.connect(path)
        try:
            out.extend(con.execute(sql).fetchall())
        finally:
            con.close()
    return out


def _trace_stats(d: str):
    """[(kernel name, calls, avg ns, min ns, max ns, total ns)] of a --kernel-trace run (SQLite or CSV output)."""
    if _find(d, "_results.db"):
        rows = _db_query(d, "select name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
                            "from kernels group by name")
    else:
        def col(r, *names):
            for k in names:
                for kk in r:
                    if kk.lower().replace("_", "") == k.lower().replace("_", ""):
                        return r[kk]
            raise SystemExit(f"column {names} not in {list(r)}")
        rows = [(col(r, "Name", "KernelName", "Kernel_Name"), int(col(r, "Calls")), float(col(r, "AverageNs")),
                 float(col(r, "MinNs")), float(col(r, "MaxNs")), float(col(r, "TotalDurationNs")))
                for r in _csv_rows(d, "kernel_stats.csv")]
    if not rows:
        raise SystemExit(f"no kernel trace under {d}")
    return sorted(rows, key=lambda r: -r[5])


def _pmc_all(dirs):
    """Per-dispatch counter values from rocprofv3 --pmc runs: {counter: {kernel: [value per dispatch]}}.
    Rows of one (dispatch, counter) are summed (covers per-dimension rows as well as aggregated ones)."""
    per = {}
    for d in dirs:
        if _find(d, "_results.db"):
            rows = _db_query(d, "select counter_name, kernel_name, dispatch_id, value from counters_collection")
        else:
            rows = [(r["Counter_Name"], r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id")),
                     r["Counter_Value"]) for r in _csv_rows(d, "counter_collection.csv")]
        for ctr, name, disp, val in rows:
            key = (ctr, name, d, disp)
            per[key] = per.get(key, 0.0) + float(val)
    out = {}
    for (ctr, name, _, _), v in per.items():
        out.setdefault(ctr, {}).setdefault(name, []).append(v)
    return out


# Chip constants for AMD's derived utilisation expressions (MfmaUtil, VALUBusy):
# 256 CUs, 4 SIMDs each, 8 XCDs (GRBM_GUI_ACTIVE is counted once per XCD).
CU_NUM, SIMD_NUM, XCD_NUM = 256, 1024, 8
FLOPS_PER_MFMA = 2 * 32 * 32 * 16        # v_mfma_f32_32x32x16_bf16
ALG_UNITS = {"lse_fwd": 2, "kl_bwd": 4, "kl_rows": 2, "kl_cols": 2}


def summarize(trace_dir: str, copy_mib: str, pmc_dirs, cmds: str) -> str:
    import linear_memory_relation_amd as lmr
    copy_bytes = int(copy_mib) * 2 ** 20
    stats = _trace_stats(trace_dir)
    pmc = _pmc_all(pmc_dirs)
    lines = ["# Kernel time, hardware counters and HBM traffic of one relation-KL step (llama2_16k workload)", ""]
    lines += ["Workload: B=1, H=32, n=16384, d=128, bf16, maps Q/Q, K/K, V/V, causal.", ""]
    lines += [f"Library: {lmr.version()}", ""]
    lines += ["Commands (run from the repository root; rocprofv3 wrote its output under the -d directory):", "",
              "```"]
    lines += [c for c in cmds.split(";;") if c] + ["```", ""]
    lines += ["## Kernel trace (rocprofv3 --kernel-trace --stats)", ""]
    lines += ["| kernel | kind | calls | avg ms | min ms | max ms | share of GPU time |", "|---|---|---|---|---|---|---|"]
    total = sum(r[5] for r in stats)
    avg_ns = {}
    for name, calls, avg, mn, mx, tot in stats:
        kind = kernel_kind(name)
        if kind in ALG_UNITS:
            avg_ns[kind] = float(avg)
        lines.append(f"| `{name[:90]}` | {kind} | {calls} | {avg / 1e6:.4f} | {mn / 1e6:.4f} | {mx / 1e6:.4f} | "
                     f"{100 * tot / total:.2f}% |")

    def by_kind(ctr):
        """Mean per dispatch of a counter, by kernel kind (sweep kernels only)."""
        res = {}
        for name, vals in pmc.get(ctr, {}).items():
            kind = kernel_kind(name)
            if kind in ALG_UNITS or kind == "copy_calibration":
                res.setdefault(kind, []).extend(vals)
        return {k: float(np.mean(v)) for k, v in res.items()}

    machine = {}
    # ---- MFMA / VALU utilisation --------------------------------------------
    gui = by_kind("GRBM_GUI_ACTIVE")
    busy = by_kind("SQ_VALU_MFMA_BUSY_CYCLES")
    mops = by_kind("SQ_INSTS_VALU_MFMA_MOPS_BF16")
    nmfma = by_kind("SQ_INSTS_MFMA")
    valu = by_kind("SQ_ACTIVE_INST_VALU")
    coex = by_kind("SQ_VALU_MFMA_COEXEC_CYCLES")
    if gui and busy:
        import linear_memory_relation_amd as lmr
        from synth_inputs import WORKLOADS
        w = WORKLOADS["llama2_16k"]
        hp1 = lmr.loss_head_group(w.B, 32, w.n, w.d)    # heads per phase-1 launch (a head group of a map)
        hp2 = lmr.loss_sweep_group(w.B, 32, w.n, w.d)   # heads per phase-2 launch (a sub-group)
        unit = {k: (hp1 if k == "lse_fwd" else hp2) * 2 * w.d * causal_pairs(w.n) for k in ALG_UNITS}
        lines += ["", "## MFMA and VALU utilisation (rocprofv3 --pmc, one dispatch at a time)", ""]
        lines += [f"Per sweep kernel, mean over its dispatches (phase 1: one per head group of {hp1} heads of a "
                  f"map; phase 2: one per sub-group of {hp2} heads):",
                  "- `clock` = GRBM_GUI_ACTIVE per XCD / kernel-trace average duration;",
                  "- `MFMA busy` = sum of SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs) "
                  "(AMD's MfmaUtil expression);",
                  "- `VALU busy` = sum of SQ_ACTIVE_INST_VALU / 256 CUs / GRBM_GUI_ACTIVE per XCD "
                  "(AMD's VALUBusy expression);",
                  "- `executed flop` = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 and, as a cross-check, SQ_INSTS_MFMA x "
                  f"{FLOPS_PER_MFMA} (one v_mfma_f32_32x32x16_bf16);",
                  "- `co-issue` = sum of SQ_VALU_MFMA_COEXEC_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs): "
                  "cycles in which a SIMD issued a VALU instruction while its MFMA unit was busy;",
                  "- `algorithmic flop` = the kernel's share of the method's 6 GEMM-units (phase 1: 2; phase 2: 4, "
                  "credited 2 to each split sweep, which executes 3), one unit = 2*d*n(n+1)/2 flop per head.", ""]
        lines += ["| kind | clock GHz | MFMA busy | VALU busy | co-issue | executed flop (MOPS) | "
                  "executed flop (insts) | algorithmic flop | executed / algorithmic |",
                  "|---|---|---|---|---|---|---|---|---|"]
        for kind in ALG_UNITS:
            if kind not in gui:
                continue
            g = gui[kind] / XCD_NUM
            clk = g / avg_ns[kind] if kind in avg_ns else float("nan")
            mb = busy.get(kind, float("nan")) / (g * SIMD_NUM)
            vb = valu.get(kind, float("nan")) / CU_NUM / g
            ef = mops.get(kind, float("nan")) * 512
            ei = nmfma.get(kind, float("nan")) * FLOPS_PER_MFMA
            af = ALG_UNITS[kind] * unit[kind]
            co = coex.get(kind, float("nan")) / (g * SIMD_NUM)
            lines.append(f"| {kind} | {clk:.3f} | {mb:.3f} | {vb:.3f} | {co:.3f} | {ef:.4e} | {ei:.4e} | {af:.4e} | "
                         f"{ef / af:.3f} |")
            machine[kind] = {"clock_ghz": clk, "mfma_busy": mb, "valu_busy": vb, "executed_flops": ef,
                             "executed_over_algorithmic": ef / af}
            if kind in coex:
                machine[kind]["mfma_valu_coissue"] = co
    # ---- other SQ counters, raw ---------------------------------------------
    other = [c for c in sorted(pmc) if c.startswith("SQ_") and c not in (
        "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_MFMA", "SQ_ACTIVE_INST_VALU")]
    if other:
        lines += ["", "## Further SQ counters (mean per dispatch, summed over the chip)", ""]
        lines += ["| counter | " + " | ".join(ALG_UNITS) + " |", "|---|" + "---|" * len(ALG_UNITS)]
        for c in other:
            v = by_kind(c)
            lines.append(f"| {c} | " + " | ".join(f"{v[k]:.4e}" if k in v else "-" for k in ALG_UNITS) + " |")
    # ---- HBM traffic -------------------------------------------------------
    fetch, write = by_kind("FETCH_SIZE"), by_kind("WRITE_SIZE")
    if fetch and write:
        if "copy_calibration" not in fetch or "copy_calibration" not in write:
            raise SystemExit("calibration copy kernel not found in the FETCH_SIZE / WRITE_SIZE runs")
        f_cal = fetch["copy_calibration"] * 1024 / copy_bytes
        w_cal = write["copy_calibration"] * 1024 / copy_bytes
        lines += ["", "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)", ""]
        lines += [f"Calibration: an fp32 copy of {copy_mib} MiB reads and writes {copy_bytes} bytes; its counters "
                  f"read FETCH_SIZE x {f_cal:.4f} and WRITE_SIZE x {w_cal:.4f} of that, and every figure below is "
                  f"divided by these factors.", ""]
        lines += ["| kind | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (calibrated) |", "|---|---|---|---|"]
        for kind in ALG_UNITS:
            if kind not in fetch:
                continue
            tb = fetch[kind] * 1024 / f_cal + write.get(kind, 0.0) * 1024 / w_cal
            machine.setdefault(kind, {})["traffic_bytes_per_launch"] = tb
            lines.append(f"| {kind} | {fetch[kind]:.1f} | {write.get(kind, 0.0):.1f} | {tb:.4e} |")
    lines += ["", "Machine-readable (read by bench.py while the library sources are unchanged):", ""]
    lines.append(f"library_source_id: {library_source_id()}")
    for kind, vals in sorted(machine.items()):
        for k, v in sorted(vals.items()):
            lines.append(f"counter {kind} {k}: {v:.6e}")
    return "\n".join(lines) + "\n"


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "sweep_kernels_llama2_16k.md")


def recorded_counters(kind: str, workload: str):
    """Counter-derived figures of `kind` (traffic, MFMA/VALU busy, executed flops) from the committed
    summary, or {} when the summary is missing, covers another workload or was taken on a library
    built from other sources."""
    import linear_memory_relation_amd as lmr
    if workload != "llama2_16k" or not os.path.exists(TRAFFIC_SUMMARY):
        return {}
    src, vals = None, {}
    with open(TRAFFIC_SUMMARY) as f:
        for line in f:
            if line.startswith("library_source_id:"):
                src = line.split(":", 1)[1].strip()
            if line.startswith(f"counter {kind} "):
                key, val = line[len(f"counter {kind} "):].split(":", 1)
                vals[key.strip()] = float(val)
    if src != lmr.source_id():
        return {}
    return vals


def time_proj(b, w, dev, dm, steps, warmup):
    """ms and TFLOP/s of larard_proj_bwd for map b: dW [dm, H*d] = h^T R^T(dX_s) with synthetic bf16
    hidden states h [B, n, dm], the map's dX_s as the last step left it, and the student rotation of
    the workload (none for V)."""
    import torch
    import linear_memory_relation_amd as lmr
    hd = b["H"] * b["d"]
    if dm % 128 or hd % 128:
        return None
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    hst = torch.randn((b["B"], b["n"], dm), generator=g, device=dev).to(torch.bfloat16)
    rc = rs = None
    if b["name"] != "V":
        pos = torch.arange(b["n"], dtype=torch.float64) / (w.factor if w.kind == "pi" else 1.0)
        inv = (w.base * (w.factor ** (b["d"] / (b["d"] - 2)) if w.kind == "ntk" else w.base)) ** (
            -2.0 * torch.arange(b["d"] // 2, dtype=torch.float64) / b["d"])
        ang = torch.outer(pos, inv)
        rc, rs = torch.cos(ang).float().to(dev), torch.sin(ang).float().to(dev)
    wsp = torch.empty(max(256, int(lmr.load().larard_proj_bwd_workspace_bytes(b["B"], b["n"], dm, b["H"], b["d"]))),
                      dtype=torch.uint8, device=dev)
    dW = torch.empty((dm, hd), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        lmr.proj_bwd(hst, b["dx"], rc, rs, workspace=wsp, out=dW)
    torch.cuda.synchronize()
    s6, e6 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s6.record()
    for _ in range(steps):
        lmr.proj_bwd(hst, b["dx"], rc, rs, workspace=wsp, out=dW)
    e6.record()
    torch.cuda.synchronize()
    ms_p = s6.elapsed_time(e6) / steps
    pflops = 2.0 * dm * hd * b["B"] * b["n"]
    del hst, wsp, dW
    return {"ms": round(ms_p, 4), "tflops": round(pflops / (ms_p * 1e-3) / 1e12, 3),
            "pct_bf16_peak": round(100 * pflops / (ms_p * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "what": f"larard_proj_bwd for map {b['name']}: dW [{dm}x{hd}] = h^T R^T(dX_s), "
                    f"K = B*n = {b['B'] * b['n']}; synthetic bf16 h; flops 2*dm*H*d*B*n"}


def trace_table(trace_dir: str) -> str:
    """Markdown table of every kernel of a rocprofv3 --kernel-trace run."""
    rows = _trace_stats(trace_dir)
    total = sum(r[5] for r in rows)
    out = ["| kernel | calls | avg ms | min ms | max ms | share of GPU time |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, tot in rows:
        out.append(f"| `{name[:100]}` | {calls} | {avg / 1e6:.4f} | {mn / 1e6:.4f} | {mx / 1e6:.4f} | "
                   f"{100 * tot / total:.2f}% |")
    return "\n".join(out) + "\n"


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
    proj = time_proj(bufs[0], w, dev, bufs[0]["H"] * bufs[0]["d"], args.steps, args.warmup)

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


def make_buffers(w, dev):
    """Device inputs and outputs of every map of workload `w` (inputs resident in HBM)."""
    import torch
    import synth_inputs as si
    maps = si.make_inputs(w)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
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
    for b in bufs:
        b["groups"] = head_groups(b)
    return maps, bufs


def head_groups(b):
    """Views of one map's tensors as larard_loss schedules its heads: phase 1 and phase 2 run for
    heads [h0, h0+g) of the flattened B*H heads before the next group (larard_loss_head_group),
    and within a group phase 2 runs per sub-group (larard_loss_sweep_group), so that the heads'
    projections stay in the last-level cache between the sweeps that read them."""
    import linear_memory_relation_amd as lmr
    bh, n, d = b["B"] * b["H"], b["n"], b["d"]
    g1 = lmr.loss_head_group(b["B"], b["H"], n, d)
    g2 = lmr.loss_sweep_group(b["B"], b["H"], n, d)

    def views(h0, c):
        def sl(t, tail):
            return t.reshape(1, bh, *tail)[:, h0:h0 + c]
        return dict(heads=c, xt=sl(b["xt"], (n, d)), xs=sl(b["xs"], (n, d)), lse_t=sl(b["lse_t"], (n,)),
                    lse_s=sl(b["lse_s"], (n,)), row_kl=sl(b["row_kl"], (n,)), dx=sl(b["dx"], (n, d)))
    out = []
    for h0 in range(0, bh, g1):
        c = min(g1, bh - h0)
        grp = views(h0, c)
        grp["sub"] = [views(k0, min(g2, h0 + c - k0)) for k0 in range(h0, h0 + c, g2)]
        out.append(grp)
    return out


# Kernels of one map's step in each phase-2 mode (the events bracket each).
KINDS = {"fused": ["lse_fwd", "kl_bwd", "reduce"], "split": ["lse_fwd", "kl_rows", "kl_cols", "reduce"]}
# GEMM-units per head-map: algorithmic (the method's 6: phase 1 does 2, phase 2 does 4) and executed
# (phase 2 computes its logit tiles twice, once for the row term and once for the column term).  In
# split mode each of phase 2's two sweeps executes 3 (both logit tiles and one contraction) and is
# credited with half of phase 2's 4.
ALG = {"lse_fwd": 2, "kl_bwd": 4, "kl_rows": 2, "kl_cols": 2, "reduce": 0}
EXE = {"lse_fwd": 2, "kl_bwd": 6, "kl_rows": 3, "kl_cols": 3, "reduce": 0}


def run_steps(bufs, scale, steps, warmup, events=True, mode="split"):
    """Warm up, then time `steps` steps: each map, head group by head group (head_groups), runs
    phase 1 and phase 2 -- one fused sweep, or the row and column sweeps in split mode -- and then
    the map's loss reduction, as larard_loss launches them, with HIP events on the launch stream
    around every launch.  Returns (ms per step, per-kernel launch times in ms, total ms, wall
    seconds of the timed region); per-kernel entries are (ms, heads of the launch)."""
    import torch
    import linear_memory_relation_amd as lmr
    sweeps = KINDS[mode][1:-1]
    plan = []                      # kinds of one step's launches, in order, with their head counts
    for b in bufs:
        for grp in b["groups"]:
            plan.append(("lse_fwd", grp["heads"]))
            for sg in grp["sub"]:
                plan += [(k, sg["heads"]) for k in sweeps]
        plan.append(("reduce", b["B"] * b["H"]))

    def step(ev=None):
        marks = iter(ev) if ev is not None else None

        def mark():
            if marks is not None:
                next(marks).record()
        mark()
        for b in bufs:
            for grp in b["groups"]:
                lmr.lse_fwd(grp["xt"], grp["xs"], scale, True, grp["lse_t"], grp["lse_s"])
                mark()
                for sg in grp["sub"]:
                    a = (sg["xt"], sg["xs"], sg["lse_t"], sg["lse_s"])
                    if mode == "fused":
                        lmr.kl_bwd(*a, scale, True, 1.0, dx_mode=lmr.DX_FUSED, row_kl=sg["row_kl"], dx=sg["dx"])
                    else:
                        lmr.kl_bwd_rows(*a, sg["row_kl"], sg["dx"], scale, True, 1.0)
                        mark()
                        lmr.kl_bwd_cols(*a, sg["dx"], scale, True, 1.0)
                    mark()
            lmr.reduce_loss(b["row_kl"], b["partials"], b["loss"], 1.0)
            mark()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(plan) + 1)] for _ in range(steps)] \
        if events else [None] * steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for k in range(steps):
        step(ev[k])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(stop)
    per_kernel = {k: [] for k in KINDS[mode]}
    if events:
        for k in range(steps):
            e = ev[k]
            for j, (kind, heads) in enumerate(plan):
                per_kernel[kind].append((e[j].elapsed_time(e[j + 1]), heads))
    return total_ms / steps, per_kernel, total_ms, wall


def kernel_ms(per_kernel):
    """Mean launch time (ms) per kernel kind."""
    return {k: float(np.mean([t for t, _ in v])) for k, v in per_kernel.items() if v}


def units(b):
    """One GEMM-unit of a map: 2*d flop per kept pair, over all its heads."""
    return b["B"] * b["H"] * units_per_head(b)


def units_per_head(b):
    """One GEMM-unit of one head: 2*d flop per kept pair."""
    return 2 * b["d"] * causal_pairs(b["n"])


def memory_report(bufs, base_alloc, peak_alloc, free_before, free_after_alloc, free_after_steps):
    inputs = sum(b["xt"].numel() * 2 * 2 for b in bufs)
    dx = sum(b["dx"].numel() * 4 for b in bufs)
    stats = sum(b["lse_t"].numel() * (8 + 8 + 4) + b["partials"].numel() * 8 for b in bufs)
    return {"peak_alloc_bytes_during_steps": int(peak_alloc),
            "hip_mem_used_by_buffers_bytes": int(free_before - free_after_alloc),
            "hip_mem_growth_during_steps_bytes": int(free_after_alloc - free_after_steps),
            "inputs_bytes": inputs, "dx_bytes": dx, "statistics_bytes": stats,
            "extra_beyond_inputs_and_dx_bytes": int(peak_alloc - inputs - dx),
            "bhn_bound_bytes": int(sum(20 * b["B"] * b["H"] * b["n"] + 8 * b["B"] * b["H"] for b in bufs)),
            "dense_fp32_map_bytes_one_matrix": int(sum(4 * b["B"] * b["H"] * b["n"] ** 2 for b in bufs))}


def time_fused_maps(bufs, scale, steps, warmup):
    """ms per step of the same step with every map in one launch per phase (larard_multi_loss)."""
    import torch
    import linear_memory_relation_amd as lmr
    mlist = [(b["xt"], b["xs"], 1.0, b["dx"]) for b in bufs]
    wsm = torch.empty(lmr.multi_workspace_bytes(mlist), dtype=torch.uint8, device=bufs[0]["xt"].device)
    out = torch.empty((), dtype=torch.float32, device=bufs[0]["xt"].device)
    for _ in range(warmup):
        lmr.multi_loss(mlist, scale, True, 1.0, workspace=wsm, out=out)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        lmr.multi_loss(mlist, scale, True, 1.0, workspace=wsm, out=out)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def reference_gemm(dev, reps: int = 200, size: int = 8192):
    """The vendor library's dense bf16 GEMM (torch.matmul, hipBLASLt underneath) on random normal
    operands, timed over enough repetitions to reach the clock the GPU sustains under MFMA load.
    It is a measured reference for what a plain MFMA contraction reaches on this GPU, beside the
    nominal peak; the relation-KL step's figures stay priced against the nominal peak."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    a = torch.randn(size, size, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(size, size, device=dev, dtype=torch.bfloat16, generator=g)
    c = torch.empty(size, size, device=dev, dtype=torch.bfloat16)
    for _ in range(5):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    tflops = 2.0 * size ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"what": "torch.matmul bf16 x bf16 -> bf16 (fp32 accumulate), random normal operands",
            "shape_mnk": [size, size, size], "reps": reps, "ms": round(ms, 4), "tflops": round(tflops, 1),
            "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4)}


def extra_workload(name, args, dev):
    """ms/step, TFLOP/s and memory of one more workload, timed like the headline one."""
    import gc
    import torch
    import synth_inputs as si
    w = si.WORKLOADS[name]
    torch.cuda.synchronize()
    free_before = torch.cuda.mem_get_info()[0]
    base_alloc = torch.cuda.memory_allocated()
    maps, bufs = make_buffers(w, dev)
    del maps
    torch.cuda.synchronize()
    free_after_alloc = torch.cuda.mem_get_info()[0]
    torch.cuda.reset_peak_memory_stats()
    # AUTO's phase-2 mode for this length (fused up to n = 8192, as larard_kl_bwd
    # decides), and the other mode beside it.
    mode = "fused" if w.n <= 8192 else "split"
    other = "split" if mode == "fused" else "fused"
    # Per-kernel times from one evented run; the two modes' step times from
    # event-free runs in alternation (A B A B), so that neither mode pays the
    # events or the first-run warm-up alone.
    _, per_kernel, _, _ = run_steps(bufs, w.scale, args.extra_steps, 2, mode=mode)
    free_after_steps = torch.cuda.mem_get_info()[0]
    t = {mode: [], other: []}
    for _ in range(2):
        for m in (mode, other):
            t[m].append(run_steps(bufs, w.scale, args.extra_steps, 1, events=False, mode=m)[0])
    ms, ms_other = float(np.mean(t[mode])), float(np.mean(t[other]))
    peak = torch.cuda.max_memory_allocated() - base_alloc
    memory = memory_report(bufs, base_alloc, peak, free_before, free_after_alloc, free_after_steps)
    flops = sum(6 * units(b) for b in bufs)
    ms_maps = time_fused_maps(bufs, w.scale, args.extra_steps, 2)
    out = {"workload": name, "B": w.B, "n": w.n, "d": w.d, "heads": w.heads, "steps": args.extra_steps,
           "ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 3),
           "pct_bf16_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
           "kernels_avg_ms": {k: round(v, 4) for k, v in kernel_ms(per_kernel).items()},
           "heads_per_group": {b["name"]: [b["groups"][0]["heads"], b["groups"][0]["sub"][0]["heads"]]
                               for b in bufs},
           "phase2_mode": mode, f"ms_per_step_{other}_phase2": round(ms_other, 4),
           "fused_maps_ms_per_step": round(ms_maps, 4),
           "losses": {b["name"]: float(b["loss"].cpu()) for b in bufs},
           "memory": memory}
    del bufs
    gc.collect()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.summarize:
        sys.stdout.write(summarize(args.summarize[0], args.summarize[1], args.pmc_dir, args.trace_cmd))
        return
    if args.trace_table:
        sys.stdout.write(trace_table(args.trace_table))
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
    scale = w.scale
    if args.proj_only:
        maps, bufs = make_buffers(w, dev)
        run_steps(bufs, scale, 1, 1, events=False)          # dX_s of every map
        dm = bufs[0]["H"] * bufs[0]["d"]
        print(json.dumps({"workload": w.name, "proj_bwd": {b["name"]: time_proj(b, w, dev, dm, args.steps,
                                                                                 args.warmup) for b in bufs}}),
              flush=True)
        return

    torch.cuda.synchronize()
    free_before = torch.cuda.mem_get_info()[0]
    base_alloc = torch.cuda.memory_allocated()
    maps, bufs = make_buffers(w, dev)
    torch.cuda.synchronize()
    free_after_alloc = torch.cuda.mem_get_info()[0]
    if args.calib_copy_mib > 0:
        src = torch.ones(args.calib_copy_mib * 2 ** 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
        free_after_alloc = torch.cuda.mem_get_info()[0]
    torch.cuda.reset_peak_memory_stats()

    # Timed region: K steps with HIP events around every kernel, on the stream
    # the kernels are launched on (torch's current stream).
    ms_step, per_kernel, total_ms, wall = run_steps(bufs, scale, args.steps, args.warmup, mode="split")
    free_after_steps = torch.cuda.mem_get_info()[0]
    # The same step with phase 2 as the fused single sweep, timed alike (the
    # other mode larard_kl_bwd offers; AUTO takes the split one).
    ms_fused, per_fused, _, _ = run_steps(bufs, scale, args.steps, 1, mode="fused")
    phase2_fused = {"ms_per_step": round(ms_fused, 4),
                    "kernels_avg_ms": {k: round(v, 4) for k, v in kernel_ms(per_fused).items()},
                    "what": "phase 2 as one launch per map (LARARD_DX_FUSED): each row block's row and column "
                            "terms in one sweep, dX_s stored once"}
    peak_alloc = torch.cuda.max_memory_allocated() - base_alloc
    memory = memory_report(bufs, base_alloc, peak_alloc, free_before, free_after_alloc, free_after_steps)

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
    del ws

    step_flops = sum(6 * units(b) for b in bufs)

    fwd_info, proj, cross, fused_info = None, None, None, None
    if not args.core_only:
        fwd_info, proj, cross, fused_info = extra_sections(args, bufs, w, scale, dev, units, step_flops)

    # Algorithmic work.  Per head-map P = n(n+1)/2 unmasked pairs, one
    # contraction (GEMM-unit) = 2*d*P flops.  Phase 1: 2 units; phase 2: 4
    # (the logit recompute of both maps, the row term and the column term),
    # executed as 6 because phase 2 forms every logit tile twice.
    # Every launch's algorithmic and executed flops follow from its head count
    # (a head group of one map; the maps of one workload share n and d).
    uph = units_per_head(bufs[0])
    kern = {}
    for kind in KINDS["split"]:
        ms_l = np.array([t for t, _ in per_kernel[kind]])
        heads_l = np.array([hh for _, hh in per_kernel[kind]], dtype=np.float64)
        fl, fe = ALG[kind] * uph * heads_l, EXE[kind] * uph * heads_l
        kern[kind] = {"avg_ms": float(ms_l.mean()), "launches_per_step": len(ms_l) // args.steps,
                      "heads_per_launch": float(heads_l.mean()),
                      "share": float(ms_l.sum() / total_ms),
                      "alg_flops_per_launch": float(fl.mean()),
                      "alg_tflops": float(fl.sum() / (ms_l.sum() * 1e-3) / 1e12),
                      "executed_tflops": float(fe.sum() / (ms_l.sum() * 1e-3) / 1e12)}

    # Roofline of every sweep kernel; `roofline` is the one with the largest
    # share of the step's time.  Counter-derived figures (HBM traffic, MFMA and
    # VALU busy fractions, executed flops) come from the committed rocprofv3
    # summary when it was taken on a library built from the same sources.
    def roof(kind):
        fl = kern[kind]["alg_flops_per_launch"]
        ach = kern[kind]["alg_tflops"]
        ctr = recorded_counters(kind, w.name)
        return {"kernel": kind, "bound": "mfma", "achieved": round(ach, 3), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": ctr.get("traffic_bytes_per_launch"),
                "alg_flops_per_launch": fl,
                "executed_frac": round(kern[kind]["executed_tflops"] / PEAK_BF16_TFLOPS, 4),
                "counters": {k: ctr[k] for k in ("mfma_busy", "valu_busy", "mfma_valu_coissue", "clock_ghz",
                                                 "executed_flops", "executed_over_algorithmic") if k in ctr} or None,
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)"}
    sweeps = [k for k in KINDS["split"] if ALG[k] > 0]
    dom = max(KINDS["split"], key=lambda k: kern[k]["share"])
    value = step_flops / (ms_step * 1e-3) / 1e12
    roof_dom, roof_all = roof(dom), {k: roof(k) for k in sweeps}

    extra = {}
    del bufs
    torch.cuda.empty_cache()
    for name in [x for x in args.extra_workloads.split(",") if x and x != w.name]:
        extra[name] = extra_workload(name, args, dev)
    gemm_ref = None
    if not args.core_only:
        gemm_ref = reference_gemm(dev)
        gemm_ref["step_value_over_gemm"] = round(value / gemm_ref["tflops"], 4)

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
        "roofline": roof_dom,
        "rooflines": roof_all,
        "kernels": kern,
        "ms_per_step_one_call": round(ms_step_oneshot, 4),
        "fused_phase2": phase2_fused,
        "wall_s_timed": round(wall, 3),
        "memory": memory,
        "losses": losses,
        "other_workloads": extra,
        "forward_only": fwd_info,
        "cross_relation": cross,
        "proj_bwd": proj,
        "fused_maps": fused_info,
        "reference_gemm": gemm_ref,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, maps, args.cpu_sample_n)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
