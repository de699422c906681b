#!/usr/bin/env python3
"""MoE-layer benchmark on one MI355X.

A step is one pass of the whole hot path over one batch: router GEMM + top-k
(ft_moe_route), alignment (ft_moe_align), grouped expert FFN (ft_moe_ffn) and
combine (ft_moe_combine), on inputs already resident in HBM.  Layer weight
banks rotate between steps so that the bytes touched between two uses of the
same weights exceed four times the 256 MB Infinity Cache.

With no --workload the headline is the largest single-GPU workload, the
753B-A40B-shaped layer (H 6144, 256 experts, top-8, I 2048, bf16 weights) at
prefill T = 16384 with the per-expert N(0, 1) router bias that skews the load.
The line carries the roofline of its dominant kernel (the gate/up grouped GEMM:
HBM- or MFMA-bound by its arithmetic intensity against the ridge point), its
decode points (T = 1, 32; HBM-bound weight streaming, rated as active-expert
bytes over the gate/up + down kernel time), the CPU oracle's rate on a bounded
sample of the same workload, and under "other_workloads" the same
measurements for the 35B-A3B bf16, 284B-A13B MXFP4 and 753B-A40B MXFP4 layers
and the 8-layer slot-cache stack.  A decode point's tokens/s comes from replays
of the step captured as a HIP graph (ft_moe_graph_*); the same step enqueued
call by call is reported beside it (eager_*).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA
MALL_BYTES = 256 << 20
CAL_BYTES = 1 << 30            # calibration copy
GEMM_SRC = os.path.join(ROOT, "expert_ffn_execution_amd", "csrc", "gemm_mfma.hip")
DEFAULT_WORKLOAD = "753b_a40b_bf16"
EXTRA_WORKLOADS = ("35b_a3b_bf16", "284b_a13b_mxfp4", "753b_a40b_mxfp4")
# gate/up GEMM kernel (MODE_GATED) by weight format, as rocprofv3 names it
GEMM1_KERNEL = {"bf16": "gemm_pipe_kernelILi0ELi0E", "mxfp4": "gemm_pipe_kernelILi0ELi1E",
                "fp8": "gemm_pipe_kernelILi0ELi2E", "nvfp4": "gemm_pipe_kernelILi0ELi3E"}


def traffic_json(workload, T):
    return os.path.join(ROOT, "profiles", f"gemm1_traffic_{workload}_T{T}.json")


def _sha(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def stored_traffic(workload, T):
    """HBM bytes per gate/up GEMM launch from the committed counter summary of
    this workload and token count, or None when there is none or the kernel
    source changed since the counters were taken."""
    try:
        with open(traffic_json(workload, T)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != _sha(GEMM_SRC):
        return None
    return t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]


def summarize_pmc(fetch_dir, write_dir, workload, T):
    """rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of this benchmark (one
    workload) -> the committed traffic summary of its gate/up GEMM.  Counters
    are KiB per dispatch; each is scaled by its reading for the 1 GiB
    calibration copy."""
    from expert_ffn_execution_amd import synth
    kname = GEMM1_KERNEL[synth.SHAPES[workload].wdtype]
    T = int(T)
    import csv
    import glob

    def read(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows += [r for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]
        for f in glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True):
            rows += [{"Kernel_Name": n, "Counter_Value": v} for n, v in rocpd_rows(
                f, "select kernel_name, value from counters_collection where counter_name = ?",
                (counter,))]
        cal = [float(r["Counter_Value"]) for r in rows
               if "copyBuffer" in r["Kernel_Name"] or "copy" in r["Kernel_Name"].lower()]
        cal = max(cal) if cal else float("nan")
        g1 = [float(r["Counter_Value"]) for r in rows if kname in r["Kernel_Name"]]
        return cal, (sum(g1) / len(g1) if g1 else float("nan")), len(g1)

    fc, fg, nf = read(fetch_dir, "FETCH_SIZE")
    wc, wg, nw = read(write_dir, "WRITE_SIZE")
    f_scale, w_scale = CAL_BYTES / (fc * 1024.0), CAL_BYTES / (wc * 1024.0)
    out = {"source_sha256": _sha(GEMM_SRC), "kernel": kname, "workload": workload, "T": T,
           "calibration_copy_bytes": CAL_BYTES,
           "fetch_kib_calibration": fc, "write_kib_calibration": wc,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "fetch_kib_per_launch": fg, "write_kib_per_launch": wg, "launches": [nf, nw],
           "fetch_bytes_per_launch": fg * 1024.0 * f_scale,
           "write_bytes_per_launch": wg * 1024.0 * w_scale}
    with open(traffic_json(workload, T), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def summarize_counters(pmc_dir, workload):
    """rocprofv3 --pmc run (rocpd database) of this benchmark -> the mean per
    dispatch of every collected counter, for the workload's two expert GEMMs.
    A counter's value is summed over its hardware instances first."""
    import glob
    from expert_ffn_execution_amd import synth
    k1 = GEMM1_KERNEL[synth.SHAPES[workload].wdtype]
    kernels = {"gemm1": k1, "gemm2": k1.replace("ILi0E", "ILi1E", 1)}
    per = {}
    for db in glob.glob(os.path.join(pmc_dir, "**", "*_results.db"), recursive=True):
        for name, counter, value, disp in rocpd_rows(
                db, "select kernel_name, counter_name, value, dispatch_id from counters_collection"):
            for tag, key in kernels.items():
                if key in name:
                    d = per.setdefault(tag, {}).setdefault(counter, {})
                    d[disp] = d.get(disp, 0.0) + value
        # with --kernel-trace in the same run: the mean duration of the same dispatches
        try:
            for tag, key in kernels.items():
                r = rocpd_rows(db, "select avg(duration), count(*) from kernels where name like ?",
                               (f"%{key}%",))
                if r and r[0][1]:
                    per.setdefault("duration_ns", {})[tag] = {"mean": r[0][0], "n": r[0][1]}
        except Exception:  # counters-only run: no kernels view
            pass
    dur = per.pop("duration_ns", {})
    out = {tag: {c: sum(v.values()) / len(v) for c, v in cs.items()} for tag, cs in per.items()}
    out["dispatches"] = {tag: len(next(iter(cs.values()))) for tag, cs in per.items()}
    out["kernels"] = kernels
    if dur:
        out["duration_ns"] = dur
    print(json.dumps(out))
    return out


def run_mfma_rate():
    """The stand-alone issue-rate probe (built next to the library), run as a
    child process; its JSON lines pass through."""
    import subprocess
    exe = os.path.join(ROOT, "expert_ffn_execution_amd", "mfma_rate")
    if not os.path.exists(exe):
        raise SystemExit(f"{exe} is not built: run python -m expert_ffn_execution_amd.build")
    r = subprocess.run([exe], timeout=300)
    return r.returncode


# A helper process started before this one touches the GPU runs amd-smi when
# asked and answers with the GFX (per-XCD) clocks in MHz: a process that has
# initialised the GPU starts no other program itself.
_CLOCK_HELPER = r"""
import json, re, subprocess, sys
for line in sys.stdin:
    if line.strip() != "go":
        break
    try:
        r = subprocess.run(["amd-smi", "metric", "--clock"], capture_output=True, text=True, timeout=30)
        mhz = [int(v) for v in re.findall(r"GFX_\d+:\s*CLK:\s*(\d+)\s*MHz", r.stdout)]
    except Exception:
        mhz = []
    print(json.dumps(mhz), flush=True)
"""


class ClockSampler:
    """GPU clocks read by amd-smi on request (see _CLOCK_HELPER)."""

    def __init__(self):
        import subprocess
        self.p = subprocess.Popen([sys.executable, "-c", _CLOCK_HELPER], stdin=subprocess.PIPE,
                                  stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)

    def sample(self):
        try:
            self.p.stdin.write("go\n")
            self.p.stdin.flush()
            return json.loads(self.p.stdout.readline() or "[]")
        except (OSError, ValueError):
            return []

    def close(self):
        try:
            self.p.stdin.write("quit\n")
            self.p.stdin.flush()
            self.p.wait(timeout=10)
        except Exception:
            self.p.kill()


def rocpd_rows(db, query, params=()):
    """Rows of a query on a rocprofv3 rocpd database (its SQLite output)."""
    import sqlite3
    con = sqlite3.connect(db)
    try:
        return list(con.execute(query, params))
    finally:
        con.close()


def summarize_stats(stats, command, out_md, top=16):
    """rocprofv3 --kernel-trace --stats output (kernel_stats.csv, or the rocpd
    database *_results.db) -> a short markdown table of kernel durations."""
    import csv
    if stats.endswith(".db"):
        rows = []
        q = ("select name, count(*), sum(duration), avg(duration), min(duration), max(duration) "
             "from kernels group by name order by sum(duration) desc")
        res = rocpd_rows(stats, q)
        tot = sum(r[2] for r in res)
        for name, n, sm, av, mn, mx in res:
            rows.append({"Name": name, "Calls": n, "AverageNs": av, "MinNs": mn, "MaxNs": mx,
                         "Percentage": 100.0 * sm / tot})
    else:
        rows = list(csv.DictReader(open(stats)))
    lines = [f"# {os.path.basename(out_md)[:-3]}", "", "Command (from the repository root):", "",
             "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        name = r["Name"].replace("|", "/")
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--summarize-stats", nargs=3, metavar=("STATS_CSV", "COMMAND", "OUT_MD"),
                    help="format a rocprofv3 kernel_stats.csv as a markdown summary")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-extras", action="store_true",
                    help="only the chosen workload (no other_workloads section)")
    ap.add_argument("--tokens", type=int, default=0, help="prefill tokens (default: workload's)")
    ap.add_argument("--decode", default="", help="decode token counts, e.g. 1,16,64 "
                                                 "(default: workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "WORKLOAD", "T"),
                    help="write the traffic summary from two rocprofv3 --pmc runs of one workload")
    ap.add_argument("--mfma-rate", action="store_true",
                    help="run the matrix-core issue-rate probe (bf16 vs block-scaled fp8 x fp4 and "
                         "fp4 x fp4; burst and sustained) and print its JSON lines")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("PMC_DIR", "WORKLOAD"),
                    help="mean per dispatch of each counter of a rocprofv3 --pmc run, for the "
                         "workload's two expert GEMMs")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Bank:
    """One layer's weights in device slots plus its router and bias."""

    def __init__(self, sh, layer, dev):
        import torch
        from expert_ffn_execution_amd import ftmoe as ft
        from expert_ffn_execution_amd import synth
        n = synth.n_experts_total(sh)
        self.stride = ft.slot_stride(sh.wdtype, sh.H, sh.I)
        self.pool = torch.empty((n, self.stride), dtype=torch.uint8, device=dev)
        for e in range(n):
            ex = synth.gen_expert(sh, e, layer, device=dev)
            ft.pack_expert(ex, sh.wdtype, sh.H, sh.I, self.pool[e])
        self.wts = ft.make_weights(sh.wdtype, sh.E, sh.H, sh.I, self.pool, n_shared=sh.n_shared,
                                   shared_slot=sh.E if sh.n_shared else 0)
        self.wr = synth.gen_router(sh, layer, device=dev)
        self.bias = synth.gen_bias(sh, layer, device=dev)
        self.expert_bytes = ft.expert_layout(sh.wdtype, sh.H, sh.I)[0]


def run_point(sh, banks, T, steps, warmup, dev, prefill, clock=None):
    """Time `steps` full steps at T tokens; returns a dict of measurements.
    With a ClockSampler, the GPU clocks are then sampled while about three
    seconds of the same steps run (untimed)."""
    import torch
    from expert_ffn_execution_amd import ftmoe as ft
    from expert_ffn_execution_amd import synth

    nx = 16 if T <= 64 else 2
    xs = [synth.gen_x(sh, T, step=i, device=dev) for i in range(nx)]
    E, k = sh.E, sh.k
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    al = (torch.empty(E, dtype=torch.int32, device=dev),
          torch.empty(E + 1, dtype=torch.int32, device=dev),
          torch.empty(T * k, dtype=torch.int32, device=dev),
          torch.empty(T * k, dtype=torch.int32, device=dev))
    aws = torch.empty(max(1, ft.align_workspace(T, k, E)), dtype=torch.uint8, device=dev)
    fws = torch.empty(ft.ffn_workspace(banks[0].wts, T, k), dtype=torch.uint8, device=dev)
    y = torch.empty((T * k + sh.n_shared * T, sh.H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, sh.H), dtype=torch.bfloat16, device=dev)

    def step(i):
        b = banks[i % len(banks)]
        x = xs[i % nx]
        ft.route(T, E, k, x=x, w_router=b.wr, bias=b.bias, logits_out=logits, ids=ids, w=w)
        ft.align(ids, E, ws=aws, out=al)
        ft.ffn(b.wts, x, k, al[2], al[1], y=y, ws=fws)
        ft.combine(y, al[3], w, n_shared=sh.n_shared, out=out)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    hev = ft.HipEvents()
    prof = {which: [(hev.create(), hev.create()) for _ in range(steps)]
            for which in (ft.PROF_GEMM1, ft.PROF_GEMM2)}
    active = []
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        for which, lst in prof.items():
            ft.set_profile_events(which, *lst[i])
        step(warmup + i)
    t1.record()
    torch.cuda.synchronize()
    for which in prof:
        ft.set_profile_events(which, None, None)
    ms = t0.elapsed_time(t1) / steps
    clock_mhz = None
    if clock is not None:
        # enqueue ~3 s of steps, then ask for the clocks while they run
        import threading
        got = []
        for i in range(max(1, int(3000 / ms))):
            step(warmup + steps + i)
        th = threading.Thread(target=lambda: got.append(clock.sample()))
        th.start()
        th.join(timeout=60)
        torch.cuda.synchronize()
        clock_mhz = got[0] if got else []
    # the two expert kernels carry their events on their own dispatch: these are
    # kernel durations; the FFN's time is their sum (its tile-list kernel aside)
    dur = {which: sum(hev.elapsed_ms(a, b) for a, b in lst) / steps
           for which, lst in prof.items()}
    dur[ft.PROF_FFN] = dur[ft.PROF_GEMM1] + dur[ft.PROF_GEMM2]
    hev.close()
    # distinct active experts of each timed step (recomputed outside the timed region)
    for i in range(steps):
        b = banks[(warmup + i) % len(banks)]
        x = xs[(warmup + i) % nx]
        ids_i, _, _ = ft.route(T, E, k, x=x, w_router=b.wr, bias=b.bias)
        cnt = torch.bincount(ids_i.reshape(-1).long(), minlength=E)
        active.append(int((cnt > 0).sum().item()))
    torch.cuda.synchronize()
    n_act = sum(active) / steps
    eb = banks[0].expert_bytes
    ffn_bytes = (n_act + sh.n_shared) * eb
    # bytes of the gate/up matrices (codes + block scales for MXFP4 and NVFP4) of the experts read
    _, offs = ft.expert_layout(sh.wdtype, sh.H, sh.I)
    w13 = (offs[2] - offs[0]) + ((offs[5] - offs[3]) if sh.wdtype in ("mxfp4", "nvfp4") else 0)
    w13_bytes = (n_act + sh.n_shared) * w13
    rows = T * k + sh.n_shared * T
    # gate/up kernel's algorithmic bytes: its weights, each token's input row once
    # (bf16) and h written once (bf16)
    g1_bytes = w13_bytes + T * sh.H * 2 + rows * sh.I * 2
    fl1 = 2.0 * rows * 2 * sh.I * sh.H
    fl2 = 2.0 * rows * sh.I * sh.H
    res = {
        "T": T, "ms_per_step": ms, "tokens_per_s": T / (ms / 1e3), "gpu_clock_mhz": clock_mhz,
        "ffn_ms": dur[ft.PROF_FFN], "gemm1_ms": dur[ft.PROF_GEMM1], "gemm2_ms": dur[ft.PROF_GEMM2],
        "active_experts": n_act, "weight_bytes": ffn_bytes,
        "ffn_gbs": ffn_bytes / (dur[ft.PROF_FFN] * 1e-3) / 1e9,
        "gemm1_gbs": w13_bytes / (dur[ft.PROF_GEMM1] * 1e-3) / 1e9,
        "gemm2_gbs": (ffn_bytes - w13_bytes) / (dur[ft.PROF_GEMM2] * 1e-3) / 1e9,
        "w13_bytes": w13_bytes,
        "gemm1_bytes": g1_bytes,
        "gemm1_alg_gbs": g1_bytes / (dur[ft.PROF_GEMM1] * 1e-3) / 1e9,
        "gemm1_tflops": fl1 / (dur[ft.PROF_GEMM1] * 1e-3) / 1e12,
        "gemm2_tflops": fl2 / (dur[ft.PROF_GEMM2] * 1e-3) / 1e12,
        "ffn_tflops": (fl1 + fl2) / (dur[ft.PROF_FFN] * 1e-3) / 1e12,
        "gemm1_flops": fl1,
    }
    return res


def gemm1_roofline(r):
    """The gate/up GEMM against its roofline: HBM when its arithmetic
    intensity (flops per algorithmic byte) is below the ridge point (bf16 MFMA
    peak / HBM peak = 312 flop/B), else MFMA; the other fraction rides along."""
    ai = r["gemm1_flops"] / r["gemm1_bytes"]
    ridge = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
    hbm = {"achieved": r["gemm1_alg_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": r["gemm1_alg_gbs"] / HBM_PEAK_GBS}
    mfma = {"achieved": r["gemm1_tflops"], "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
            "frac": r["gemm1_tflops"] / MFMA_BF16_PEAK_TFS}
    (bound, first), (oname, other) = (("hbm", hbm), ("mfma", mfma)) if ai < ridge else \
        (("mfma", mfma), ("hbm", hbm))
    return {"bound": bound, **first, "flop_per_byte": ai, "ridge_flop_per_byte": ridge,
            "bytes_per_launch": r["gemm1_bytes"], "flops_per_launch": r["gemm1_flops"],
            "other_bound": {"bound": oname, **other}}


def cpu_baseline(sh, bank, T, dev, seconds):
    """The CPU oracle timed on a bounded token sample of the same workload."""
    import numpy as np
    import torch
    from expert_ffn_execution_amd import ftmoe as ft
    from expert_ffn_execution_amd import synth
    from oracle import oracle as orc

    x = synth.gen_x(sh, T, step=0, device=dev).cpu()
    wr = bank.wr.cpu()
    bias = None if bank.bias is None else bank.bias.cpu().numpy()
    _, offs = ft.expert_layout(sh.wdtype, sh.H, sh.I)
    H, I = sh.H, sh.I
    raw = bank.pool.cpu()
    experts = []
    for e in range(synth.n_experts_total(sh)):
        r = raw[e]
        shapes = {"gate": (I, H), "up": (I, H), "down": (H, I)}
        ex = {}
        for m, name in enumerate(("gate", "up", "down")):
            rows, K = shapes[name]
            if sh.wdtype in ("mxfp4", "nvfp4"):
                nb = 32 if sh.wdtype == "mxfp4" else 16
                ex[name] = r[offs[m]:offs[m] + rows * K // 2].view(rows, K // 2)
                ex[name + "_sc"] = r[offs[3 + m]:offs[3 + m] + rows * K // nb].view(rows, K // nb)
                if sh.wdtype == "nvfp4":
                    t0 = offs[5] + H * I // 16 + 4 * m
                    ex[name + "_ts"] = r[t0:t0 + 4].view(torch.float32)
            elif sh.wdtype == "fp8":
                ex[name] = r[offs[m]:offs[m] + rows * K].view(rows, K)
                ex[name + "_sc"] = r[offs[3 + m]:offs[3 + m] + 4].view(torch.float32)
            else:
                dt = torch.bfloat16 if sh.wdtype == "bf16" else torch.float32
                es = 2 if sh.wdtype == "bf16" else 4
                ex[name] = r[offs[m]:offs[m] + rows * K * es].view(dt).view(rows, K)
        experts.append(ex)
    routed, shared = experts[:sh.E], (experts[sh.E] if sh.n_shared else None)

    def run(n):
        xs = x[:n]
        t = time.perf_counter()
        lg = orc.router_logits(xs, wr)
        ids, w = orc.route(lg, sh.k, bias)
        orc.align(ids, sh.E)
        orc.moe_layer(xs, ids, w, routed, sh.wdtype, I, shared=shared)
        return time.perf_counter() - t

    n = 16
    t = run(n)
    n2 = int(min(T, max(n, n * seconds / max(t, 1e-3))))
    if n2 > n:
        n, t = n2, run(n2)
    return {"value": n / t, "unit": "tokens/s", "cores": orc.max_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"first {n} tokens of the T={T} batch, layer 0 weights "
                      f"(router GEMM, top-k, align, per-token expert loops, combine), "
                      f"{t:.1f} s"}


def cpu_model():
    """The host CPU's model name, with its family / model numbers (from
    /proc/cpuinfo; a virtual machine may report only the brand)."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break  # the first processor's block is enough
                k, _, v = line.partition(":")
                info.setdefault(k.strip(), v.strip())
    except OSError:
        pass
    name = info.get("model name")
    if not name:
        import platform
        return platform.processor() or "unknown"
    if "cpu family" in info and "model" in info:
        name += f" (family {info['cpu family']}, model {info['model']})"
    return name


def h2d_peak_gbs(dev, nbytes=1 << 30):
    """Measured pinned host -> device copy rate (the slot cache's copy path)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    s = torch.cuda.Stream(device=dev)
    best = 0.0
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            a.record()
            dst.copy_(src, non_blocking=True)
            b.record()
        b.synchronize()
        best = max(best, nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    return best


def run_slot_stack(args):
    """8 layers of the 35B-A3B layer shape behind a 512-slot global LRU over a
    pinned host pool: decode T=1 steps, then one prefill, each timed against
    the same layers fully resident in HBM.  Returns the JSON line's dict."""
    import torch
    from expert_ffn_execution_amd import ftmoe as ft
    from expert_ffn_execution_amd import synth
    from expert_ffn_execution_amd.stack import SlotStack

    dev = "cuda:0"
    sh = synth.SLOT_STACK
    L = synth.SLOT_STACK_LAYERS
    steps = synth.SLOT_STACK_DECODE_STEPS
    T_pre = max(synth.POINTS[sh.name])
    peak = h2d_peak_gbs(dev)
    log(f"pinned H2D peak {peak:.1f} GB/s")
    st = SlotStack(sh, L, n_slots=L * synth.SLOT_STACK_SLOTS_PER_LAYER)
    resident = [st.host[l].to(dev) for l in range(L)]
    rwts = [ft.make_weights(sh.wdtype, sh.E, sh.H, sh.I, p) for p in resident]

    rbufs = {}

    def resident_bufs(l, T):
        # per-layer buffers reused from step to step, as the stack does
        if (l, T) not in rbufs:
            i32, f32 = torch.int32, torch.float32
            rbufs[(l, T)] = dict(
                logits=torch.empty((T, sh.E), dtype=f32, device=dev),
                ids=torch.empty((T, sh.k), dtype=i32, device=dev),
                w=torch.empty((T, sh.k), dtype=f32, device=dev),
                al=(torch.empty(sh.E, dtype=i32, device=dev), torch.empty(sh.E + 1, dtype=i32, device=dev),
                    torch.empty(T * sh.k, dtype=i32, device=dev), torch.empty(T * sh.k, dtype=i32, device=dev)),
                aws=torch.empty(max(1, ft.align_workspace(T, sh.k, sh.E)), dtype=torch.uint8, device=dev),
                fws=torch.empty(max(256, ft.ffn_workspace(rwts[l], T, sh.k)), dtype=torch.uint8, device=dev),
                y=torch.empty((T * sh.k, sh.H), dtype=torch.bfloat16, device=dev),
                out=torch.empty((T, sh.H), dtype=torch.bfloat16, device=dev))
        return rbufs[(l, T)]

    def resident_pass(xs):
        cs = torch.cuda.current_stream()
        outs = []
        for l in range(L):
            T = xs[l].shape[0]
            b = resident_bufs(l, T)
            ids, w, _ = ft.route(T, sh.E, sh.k, x=xs[l], w_router=st.routers[l], bias=st.biases[l],
                                 logits_out=b["logits"], ids=b["ids"], w=b["w"], stream=cs)
            c, off, perm, inv = ft.align(ids, sh.E, ws=b["aws"], out=b["al"], stream=cs)
            y = ft.ffn(rwts[l], xs[l], sh.k, perm, off, y=b["y"], ws=b["fws"], stream=cs)
            outs.append(ft.combine(y, inv, w, out=b["out"], stream=cs))
        return outs

    def timed(fn, batches):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for xs in batches:
            fn(xs)
        torch.cuda.synchronize()
        return time.perf_counter() - t

    dec = [[synth.gen_x(sh, 1, step=s, device=dev, layer=l) for l in range(L)]
           for s in range(steps)]
    warm = [[synth.gen_x(sh, 1, step=10_000 + s, device=dev, layer=l) for l in range(L)]
            for s in range(args.warmup)]
    timed(resident_pass, warm)
    t_res = timed(resident_pass, dec)
    timed(st.forward, warm)
    s0 = dataclasses_replace(st.stats)
    t_dec = timed(st.forward, dec)
    d = {k: getattr(st.stats, k) - getattr(s0, k) for k in
         ("demand", "hits", "prefetch_hits", "misses", "bytes_h2d")}
    # the same decode without host waits (device-table passes): experts not in
    # a slot are read from the pinned pool over the host link, and the LRU
    # takes each pass's routing afterwards; the final flush is timed too
    dtx = [[synth.gen_x(sh, 1, step=60_000 + s, device=dev, layer=l) for l in range(L)]
           for s in range(steps)]

    def dt_run(batches):
        for xs in batches:
            st.forward(xs, device_table=True)
        st.flush()

    timed(dt_run, [warm])
    s4 = dataclasses_replace(st.stats)
    t_dt = timed(dt_run, [dtx])
    dt = {k: getattr(st.stats, k) - getattr(s4, k) for k in
          ("demand", "hits", "prefetch_hits", "misses", "bytes_h2d")}
    # the same decode steps with each layer's misses split between PCIe copies
    # and host cores (split_misses with the calibrated Bp, Bh)
    bp, bh = st.calibrate()
    log(f"calibration: Bp {bp:.1f} GB/s (pinned H2D of one expert), Bh {bh:.1f} GB/s (host FFN)")
    hyb = [[synth.gen_x(sh, 1, step=30_000 + s, device=dev, layer=l) for l in range(L)]
           for s in range(steps)]
    timed(lambda xs: st.forward(xs, hybrid=True), warm)
    s2 = dataclasses_replace(st.stats)
    t_hyb = timed(lambda xs: st.forward(xs, hybrid=True), hyb)
    t_off = timed(st.forward, [[synth.gen_x(sh, 1, step=40_000 + s, device=dev, layer=l)
                                for l in range(L)] for s in range(steps)])
    h = {k: getattr(st.stats, k) - getattr(s2, k) for k in
         ("demand", "misses", "cpu_experts", "bytes_h2d")}
    # a tight budget (128 slots for 8 layers of 128 experts): misses are the rule
    st.resize(128)
    tight = {}
    for mode in ("offload", "hybrid"):
        xs_t = [[synth.gen_x(sh, 1, step=50_000 + s, device=dev, layer=l) for l in range(L)]
                for s in range(steps)]
        fwd = (lambda xs: st.forward(xs, hybrid=True)) if mode == "hybrid" else st.forward
        timed(fwd, warm)
        s3 = dataclasses_replace(st.stats)
        tt = timed(fwd, xs_t)
        tight[mode] = {"ms_per_step": tt / steps * 1e3,
                       "misses_per_step": (st.stats.misses - s3.misses) / steps,
                       "host_experts_per_step": (st.stats.cpu_experts - s3.cpu_experts) / steps,
                       "h2d_bytes_per_step": (st.stats.bytes_h2d - s3.bytes_h2d) / steps}
    st.resize(L * synth.SLOT_STACK_SLOTS_PER_LAYER)
    pre = [synth.gen_x(sh, T_pre, step=20_000, device=dev, layer=l) for l in range(L)]
    t_res_pre = timed(resident_pass, [pre])
    s1 = dataclasses_replace(st.stats)
    t_pre = timed(lambda xs: st.forward(xs, prefill=True), [pre])
    pre_bytes = st.stats.bytes_h2d - s1.bytes_h2d
    st.close()
    h2d_gbs = d["bytes_h2d"] / t_dec / 1e9
    line = {
        "metric": "MoE-layer tokens/s through a slot-cached layer stack (decode T=1)",
        "value": steps * L / t_dec, "unit": "layer-tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": t_dec / steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32" if sh.wdtype == "f32" else "bf16", "data": "synthetic",
        "config": {"workload": f"{sh.name}: {L} layers H{sh.H} E{sh.E} k{sh.k} I{sh.I}, "
                               f"{L * synth.SLOT_STACK_SLOTS_PER_LAYER} slots global LRU, "
                               f"Zipf({sh.bias_param}) router bias, pinned host pool",
                   "decode_tokens": 1, "decode_steps": steps, "prefill_tokens": T_pre},
        "roofline": {"bound": "h2d", "achieved": h2d_gbs, "peak": peak, "unit": "GB/s",
                     "frac": h2d_gbs / peak, "traffic": None,
                     "kernel": "expert copies host->device (hipMemcpyAsync, copy stream)"},
        "slot_cache": {
            "demand": d["demand"], "hit_rate": d["hits"] / max(1, d["demand"]),
            "prefetch_hit_rate": d["prefetch_hits"] / max(1, d["demand"]),
            "misses": d["misses"], "h2d_bytes_decode": d["bytes_h2d"],
            "decode_ms_per_step": t_dec / steps * 1e3,
            "resident_decode_ms_per_step": t_res / steps * 1e3,
            "exposed_stall_ms_per_step": (t_dec - t_res) / steps * 1e3,
            "prefill_ms": t_pre * 1e3, "resident_prefill_ms": t_res_pre * 1e3,
            "prefill_h2d_bytes": pre_bytes,
            "prefill_h2d_gbs": pre_bytes / t_pre / 1e9,
            "prefill_tokens_per_s": T_pre / t_pre,
            "prefetch_warnings": st.stats.prefetch_warnings,
            "device_table_decode": {
                "ms_per_step": t_dt / steps * 1e3,
                "vs_resident": t_dt / t_res,
                "hit_rate": dt["hits"] / max(1, dt["demand"]),
                "misses": dt["misses"], "h2d_bytes": dt["bytes_h2d"],
            },
        },
        "hybrid_decode": {
            "bp_gbs": bp, "bh_gbs": bh,
            "ms_per_step": t_hyb / steps * 1e3,
            "offload_ms_per_step_same_state": t_off / steps * 1e3,
            "host_experts_per_step": h["cpu_experts"] / steps,
            "misses_per_step": h["misses"] / steps,
            "h2d_bytes_per_step": h["bytes_h2d"] / steps,
            "tight_budget_128_slots": tight,
        },
    }
    del resident, rwts, rbufs
    torch.cuda.empty_cache()
    return line


def dataclasses_replace(obj):
    import dataclasses
    return dataclasses.replace(obj)


def run_graph_point(sh, banks, T, steps, warmup, dev):
    """Decode step replayed as captured HIP graphs (ft_moe_graph_*), one per
    weight bank, rotating like the eager loop; returns ms per step."""
    import torch
    from expert_ffn_execution_amd import ftmoe as ft
    from expert_ffn_execution_amd import synth

    graphs = []
    for i, b in enumerate(banks):
        x = synth.gen_x(sh, T, step=i, device=dev).contiguous()
        st = ft.LayerStep(b.wts, x, sh.k, b.wr, bias=b.bias)
        graphs.append(st.capture())
    for i in range(warmup):
        graphs[i % len(graphs)].launch()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        graphs[(warmup + i) % len(graphs)].launch()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    for g in graphs:
        g.close()
    return ms


def run_fused_point(sh, banks, T, steps, warmup, dev):
    """The same decode step as one fused kernel (ft_moe_step_fused), called
    eagerly and replayed as one-node graphs, rotating over the weight banks
    like the other decode timings; None where the fused step does not take the
    shape (it returns FT_ERR_UNSUPPORTED)."""
    import torch
    from expert_ffn_execution_amd import ftmoe as ft
    from expert_ffn_execution_amd import synth

    steps_ = []
    for i, b in enumerate(banks):
        x = synth.gen_x(sh, T, step=i, device=dev).contiguous()
        steps_.append(ft.LayerStep(b.wts, x, sh.k, b.wr, bias=b.bias))
    try:
        steps_[0].run_fused()
    except ft.FtError as e:
        if e.status == ft.ERR_UNSUPPORTED:
            return None
        raise
    out = {}
    graphs = [st.capture_fused() for st in steps_]
    try:
        for label, calls in (("fused_ms_per_step", [st.run_fused for st in steps_]),
                             ("fused_graph_ms_per_step", [g.launch for g in graphs])):
            for i in range(warmup):
                calls[i % len(calls)]()
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for i in range(steps):
                calls[(warmup + i) % len(calls)]()
            t1.record()
            torch.cuda.synchronize()
            out[label] = t0.elapsed_time(t1) / steps
    finally:
        for g in graphs:
            g.close()
    out["fused_timeouts"] = ft.fused_timeouts()
    return out


def decode_entry(sh, r, g_ms, T, fused=None):
    """One decode point: graph-replayed step rate, and the FFN's weight
    streaming rated as active-expert bytes (gate/up + down of every distinct
    routed expert, plus the shared one) over the sum of the gate/up and down
    kernel durations (and, second, over the whole replayed step)."""
    ffn_s = r["ffn_ms"] * 1e-3
    narrow = sh.wdtype in ("mxfp4", "fp8", "nvfp4") and T >= 2
    # bf16: down rows on matrix cores from 2 tokens, gate/up rows too at 2-4
    # tokens on rows of at most 2048 (the library's dispatch rule)
    if sh.wdtype == "bf16" and T >= 2:
        kern = ("gate/up + down weight streaming on matrix cores (stream_mx_kernel)"
                if T <= 4 and sh.H <= 2048 else
                "gate/up weight streaming (stream_kernel) + down on matrix cores (stream_mx_kernel)")
    elif narrow:
        kern = "gate/up + down weight streaming on matrix cores (stream_mx_kernel)"
    else:
        kern = "gate/up + down weight streaming (stream_kernel)"
    return {
        "T": T, "tokens_per_s": T / (g_ms / 1e3), "ms_per_step": g_ms,
        "eager_tokens_per_s": r["tokens_per_s"], "eager_ms_per_step": r["ms_per_step"],
        "ffn_us": r["ffn_ms"] * 1e3, "gate_up_us": r["gemm1_ms"] * 1e3,
        "down_us": r["gemm2_ms"] * 1e3, "active_experts": r["active_experts"],
        "gate_up_gbs": r["gemm1_gbs"], "down_gbs": r["gemm2_gbs"],
        "step_gbs": r["weight_bytes"] / (g_ms * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": r["weight_bytes"] / ffn_s / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": r["weight_bytes"] / ffn_s / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "kernel": kern,
                     "bytes_per_step": r["weight_bytes"]},
        **({"fused": fused} if fused else {})}


def run_workload(name, args, dev, with_cpu, clock=None):
    """Prefill point, decode points and (optionally) the CPU oracle of one
    workload; its weight banks are freed before returning."""
    import torch
    from expert_ffn_execution_amd import ftmoe as ft
    from expert_ffn_execution_amd import synth

    sh = synth.SHAPES[name]
    pts = synth.POINTS[sh.name]
    T_pre = args.tokens or max(pts)
    dec = [int(v) for v in args.decode.split(",")] if args.decode else [p for p in pts if p <= 64]
    n_exp = synth.n_experts_total(sh)
    bank_bytes = n_exp * ft.slot_stride(sh.wdtype, sh.H, sh.I)
    n_banks = max(2, min(8, math.ceil(4 * MALL_BYTES * 4 / bank_bytes)))
    log(f"workload {sh.name}: {n_banks} weight banks of {bank_bytes / 1e9:.2f} GB")
    banks = [Bank(sh, l, dev) for l in range(n_banks)]
    torch.cuda.synchronize()

    head = run_point(sh, banks, T_pre, args.steps, args.warmup, dev, prefill=True, clock=clock)
    log("prefill", sh.name, json.dumps(head))
    decode = []
    for T in dec:
        r = run_point(sh, banks, T, max(args.steps, 50), args.warmup, dev, prefill=False)
        g_ms = run_graph_point(sh, banks, T, max(args.steps, 50), args.warmup, dev)
        fused = run_fused_point(sh, banks, T, max(args.steps, 50), args.warmup, dev)
        decode.append(decode_entry(sh, r, g_ms, T, fused))
        log("decode", sh.name, json.dumps(decode[-1]))
    cpu = None
    if with_cpu:
        cpu = cpu_baseline(sh, banks[0], T_pre, dev, args.cpu_seconds)
        log("cpu", json.dumps(cpu))
    del banks
    torch.cuda.empty_cache()
    return {"sh": sh, "T": T_pre, "n_banks": n_banks, "head": head, "decode": decode, "cpu": cpu,
            "roofline": dict(**gemm1_roofline(head), traffic=stored_traffic(sh.name, T_pre),
                             kernel="gate/up grouped GEMM + SwiGLU (gemm1)")}


def summary_of(w):
    """The other_workloads entry of one workload."""
    h = w["head"]
    return {"prefill": {"T": w["T"], "tokens_per_s": h["tokens_per_s"], "ms_per_step": h["ms_per_step"],
                        "gemm1_us": h["gemm1_ms"] * 1e3, "gemm2_us": h["gemm2_ms"] * 1e3,
                        "gemm1_tflops": h["gemm1_tflops"], "gemm2_tflops": h["gemm2_tflops"],
                        "ffn_tflops": h["ffn_tflops"], "roofline": w["roofline"]},
            "decode": w["decode"], "weights": w["sh"].wdtype}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1"}))
        log("the MoE-layer path here is single-GPU; multi-GPU runs are not supported")
        sys.exit(2)
    if args.mfma_rate:
        sys.exit(run_mfma_rate())
    import torch
    from expert_ffn_execution_amd import ftmoe as ft
    from expert_ffn_execution_amd import synth

    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    # started before anything here touches the GPU; not under a profiler (its
    # preloaded library initialises the GPU in every process it starts) and
    # not in the single-workload runs the profiles use
    under_profiler = any(k.startswith("ROCPROF") for k in os.environ)
    clock = (ClockSampler() if args.workload == DEFAULT_WORKLOAD and not args.no_extras
             and not under_profiler else None)
    ft.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    # a plain device copy of known size (1 GiB), outside every timed region: under
    # rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE calibrate the counters
    cal = torch.empty(CAL_BYTES, dtype=torch.uint8, device=dev)
    torch.empty_like(cal).copy_(cal)
    del cal
    if args.workload == synth.SLOT_STACK.name:
        print(json.dumps(run_slot_stack(args)), flush=True)
        return
    w = run_workload(args.workload, args, dev, with_cpu=not args.no_cpu_baseline, clock=clock)
    if clock is not None:
        clock.close()
    sh, head = w["sh"], w["head"]
    others = {}
    if not args.no_extras and args.workload == DEFAULT_WORKLOAD and not args.tokens and not args.decode:
        for name in EXTRA_WORKLOADS:
            others[name] = summary_of(run_workload(name, args, dev, with_cpu=False))
        st = run_slot_stack(args)
        others[synth.SLOT_STACK.name] = {k: st[k] for k in ("value", "unit", "ms_per_step", "config",
                                                             "roofline", "slot_cache", "hybrid_decode")}
    line = {
        "metric": "MoE-layer tokens/s (prefill); decode HBM GB/s and prefill MFMA TFLOP/s vs peak",
        "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32" if sh.wdtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{sh.name} prefill T={w['T']}", "H": sh.H, "E": sh.E, "k": sh.k,
                   "I": sh.I, "n_shared": sh.n_shared, "tokens": w["T"], "weights": sh.wdtype,
                   "activations": "bf16", "router_bias": sh.bias if sh.bias == "none" else
                   f"{sh.bias}({sh.bias_param})", "weight_banks": w["n_banks"]},
        "roofline": w["roofline"],
        # per-XCD GFX clocks that amd-smi read while the same prefill steps ran
        # right after the timed ones (the peaks above assume 2.4 GHz)
        "gpu_clock_mhz": head["gpu_clock_mhz"],
        "prefill_detail": {"gemm1_us": head["gemm1_ms"] * 1e3, "gemm2_us": head["gemm2_ms"] * 1e3,
                           "gemm1_tflops": head["gemm1_tflops"], "gemm2_tflops": head["gemm2_tflops"],
                           "ffn_tflops": head["ffn_tflops"],
                           "ffn_mfma_frac": head["ffn_tflops"] / MFMA_BF16_PEAK_TFS},
        "decode": w["decode"],
        "cpu_baseline": w["cpu"],
    }
    if others:
        line["other_workloads"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
