#!/usr/bin/env python3
"""Benchmark of one Muon optimizer step on one MI355X.

A step is one muon_step call over a whole packed buffer of Muon-target
matrices: momentum, Frobenius normalisation, five Newton-Schulz iterations per
matrix, weight decay and the lr-scaled update, all in libmuonstep's kernels.
The headline workload is an owner's packed buffer at 1/8 share of a 7B-class
model (16 x 4096x4096, 8 x 11008x4096, 4 x 4096x11008; bf16 gradients, fp32
params and momentum) with the standard quintic in bf16.

Prints one JSON line: Muon-target elements per second (whole job) of the
headline workload, the per-step time, the roofline of the dominant kernel (the
Newton-Schulz update GEMM, timed per launch with HIP events on its stream over
the timed region), NS TFLOP/s against the bf16 dense MFMA peak, the CPU oracle
timed on a bounded sample of the same workload, and under "configs" every
workload (tiny fp32, one layer, owner share, MoE experts, per-head split) with
both methods, plus Gram-vs-standard step times per shape group.

    python bench.py [--gpus 1] [--steps 10] [--warmup 2] [--no-cpu-baseline]
    python bench.py --workload 3 --method standard|gram [...]   # one workload only
    python bench.py --copy-calibration   # plain copy of known size (counter scale)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16/fp16 MFMA
FP32_PEAK_TFLOPS = 157.3        # MI355X fp32 (vector / MFMA)
HBM_PEAK_GBS = 8000.0
METRIC = "Muon-target elements/s per step; NS TFLOP/s as % of bf16 MFMA peak"


def ns_flops(m: int, n: int, method: str) -> float:
    """Nominal Newton-Schulz FLOPs of one m x n problem (m <= n), five steps:
    standard 5 x (2 m^2 n + 2 m^3 + 2 m^2 n); gram 2 m^2 n (R0) + 5 x (2 m^3 for Q)
    + 4 x (2 m^3 for P) + 4 x (4 m^3 for R) + 2 m^2 n (P X0)."""
    if method == "standard":
        return 20.0 * m * m * n + 10.0 * m ** 3
    return 4.0 * m * m * n + 34.0 * m ** 3


def ns_flops_min(m: int, n: int, method: str) -> float:
    """Newton-Schulz FLOPs of one problem with every symmetric product counted once
    per lower-triangle entry (the least MFMA work the method needs): standard
    5 x (m^2 n + m^3 + 2 m^2 n); gram m^2 n (R0) + 5 x m^3 (Q) + 4 x 2 m^3 (P)
    + 4 x (m^3 + m^3) (T = R Q and R <- Q T) + 2 m^2 n (P X0)."""
    if method == "standard":
        return 15.0 * m * m * n + 5.0 * m ** 3
    return 3.0 * m * m * n + 21.0 * m ** 3


def problems(wl):
    out = []
    for e in wl.entries:
        pr = e.split_rows or e.rows
        for _ in range(e.rows // pr):
            out.append((min(pr, e.cols), max(pr, e.cols)))
    return out


def device_inputs(wl, dev, seed=0):
    """Synthetic inputs on the device, the workload's recipe: params N(0,1) fp32;
    grads (1e-3/4) U V^T + 1e-5 E (rank 16) stored bf16 (N(0,1) for fp32 grads);
    momentum zero."""
    import torch
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    n = wl.numel
    params = torch.randn(n, device=dev, generator=gen)
    gdt = torch.float32 if wl.grad_dtype == "f32" else torch.bfloat16
    grads = torch.zeros(n, device=dev, dtype=gdt)
    for off, e in zip(wl.offsets, wl.entries):
        if wl.kind == "gaussian":
            g = torch.randn(e.rows, e.cols, device=dev, generator=gen)
        else:
            u = torch.randn(e.rows, 16, device=dev, generator=gen)
            v = torch.randn(e.cols, 16, device=dev, generator=gen)
            g = (1e-3 / 4.0) * (u @ v.t()) + 1e-5 * torch.randn(e.rows, e.cols, device=dev,
                                                                 generator=gen)
        grads[off:off + e.rows * e.cols] = g.reshape(-1).to(gdt)
        del g
    mom = torch.zeros(n, device=dev)
    return params, grads, mom


def gemm_source_hash() -> str:
    """SHA-256 prefix of what decides the GEMM kernels' code: gemm.hip and the
    flags it is compiled with (include paths, which differ between machines,
    left out)."""
    from newton_schulz_step_amd import build as B
    src = os.path.join(ROOT, "newton_schulz_step_amd", "csrc", "gemm.hip")
    h = hashlib.sha256(open(src, "rb").read())
    flags = [f for f in B.FLAGS + B.EXTRA.get("gemm.hip", []) if not f.startswith("-I")]
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


WORKLOAD_SLUG = {1: "tiny_fp32", 2: "one_layer", 3: "owner_share_7b", 4: "moe_experts",
                 5: "per_head_split"}


def traffic_path(workload: int, method: str) -> str:
    return os.path.join(ROOT, "profiles",
                        f"traffic_ns_gemm_update_{WORKLOAD_SLUG[workload]}_{method}.json")


def measured_traffic(kernel: str, workload: int, method: str):
    """HBM bytes per launch of `kernel` from committed rocprofv3 counter runs, or
    None when there are none or the kernel source changed since they were taken."""
    path = traffic_path(workload, method)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_symbol") is None or rec.get("gemm_sha256_16") != gemm_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def summarize_counters(fetch_csv, write_csv, fetch_copy_csv, write_copy_csv, copy_bytes,
                       symbol, workload, method):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of `symbol`, each scaled
    by what the same counter reads for the plain copy of `copy_bytes` bytes."""
    import csv

    def per_dispatch(path, name_part):
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
                if name_part in r["Kernel_Name"]]
        return sum(vals) / len(vals), len(vals)

    fetch_kib, nf = per_dispatch(fetch_csv, symbol)
    write_kib, nw = per_dispatch(write_csv, symbol)
    cf, _ = per_dispatch(fetch_copy_csv, "copy_batch_kernel")
    cw, _ = per_dispatch(write_copy_csv, "copy_batch_kernel")
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    rec = {"kernel_symbol": symbol, "workload": WORKLOAD_SLUG[workload], "method": method,
           "dispatches": [nf, nw], "fetch_kib_per_dispatch": fetch_kib,
           "write_kib_per_dispatch": write_kib, "copy_bytes": copy_bytes,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_read_bytes_per_launch": fetch_kib * 1024.0 * f_scale,
           "hbm_write_bytes_per_launch": write_kib * 1024.0 * w_scale,
           "gemm_sha256_16": gemm_source_hash()}
    rec["hbm_bytes_per_launch"] = rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]

    # cross-check of the streaming passes: scaled counter bytes over all their
    # dispatches against the algorithmic bytes of the same dispatches (the run
    # does 1 warm-up + 2 timed steps of the workload, then the AdamW measurement)
    import workloads as W
    wl = W.workload(workload)
    steps = 3
    mom_bytes = wl.muon_elements * (10 if wl.grad_dtype != "f32" else 12) * steps

    def total(path, name_part):
        return sum(float(r["Counter_Value"]) for r in csv.DictReader(open(path))
                   if name_part in r["Kernel_Name"])

    def streaming(name_part, algorithmic):
        rd = total(fetch_csv, name_part) * 1024.0 * f_scale
        wr = total(write_csv, name_part) * 1024.0 * w_scale
        return {"counter_read_bytes": rd, "counter_write_bytes": wr,
                "algorithmic_bytes": algorithmic,
                "counter_over_algorithmic": (rd + wr) / algorithmic if algorithmic else None}

    rec["streaming"] = {"momentum_sumsq_kernel": streaming("momentum_sumsq_kernel", mom_bytes)}
    run = f"python3 $REPO/bench.py --workload {workload} --method {method} --steps 2 --warmup 1 --no-cpu-baseline"
    cal = "python3 $REPO/bench.py --copy-calibration"
    rec["commands"] = [
        "cd /tmp && export TMPDIR=/tmp",
        f"rocprofv3 --pmc FETCH_SIZE -d <fetch> -o run --output-format csv -- {run}",
        f"rocprofv3 --pmc WRITE_SIZE -d <write> -o run --output-format csv -- {run}",
        f"rocprofv3 --pmc FETCH_SIZE -d <fetch_copy> -o run --output-format csv -- {cal}",
        f"rocprofv3 --pmc WRITE_SIZE -d <write_copy> -o run --output-format csv -- {cal}",
        "python3 bench.py --summarize-counters <fetch>/run_counter_collection.csv "
        "<write>/run_counter_collection.csv <fetch_copy>/run_counter_collection.csv "
        "<write_copy>/run_counter_collection.csv",
    ]
    return rec


def summarize_mfma(csv_path, symbol):
    """MFMA utilisation of `symbol` from a rocprofv3 run with SQ_VALU_MFMA_BUSY_CYCLES
    and GRBM_GUI_ACTIVE: MFMA-busy SIMD cycles over the SIMD cycles the kernel was
    active (GRBM_GUI_ACTIVE is summed over the 8 XCDs; 256 CUs x 4 SIMDs)."""
    import csv
    busy, gui, n = 0.0, 0.0, 0
    for r in csv.DictReader(open(csv_path)):
        if symbol not in r["Kernel_Name"]:
            continue
        if r["Counter_Name"] == "SQ_VALU_MFMA_BUSY_CYCLES":
            busy += float(r["Counter_Value"])
            n += 1
        elif r["Counter_Name"] == "GRBM_GUI_ACTIVE":
            gui += float(r["Counter_Value"])
    frac = busy / (gui / 8.0 * 1024.0) if gui > 0 else None
    return {"kernel_symbol": symbol, "dispatches": n, "mfma_busy_cycles": busy,
            "gui_active_cycles": gui, "mfma_busy_fraction": frac}


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(wl, method, budget_s=25.0):
    """The float64 oracle (as it stands) on one matrix per shape group, in table
    order, while the budget lasts; the untimed groups and the other matrices of
    each group are extrapolated by nominal NS FLOPs."""
    import numpy as np
    import oracle
    import workloads as W
    cores, blas = os.cpu_count(), "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if pools:
            cores = max(d.get("num_threads", 0) for d in pools)
            blas = "; ".join(f"{d.get('internal_api')} {d.get('version')} "
                             f"({d.get('threading_layer', '?')} threads, {d.get('architecture', '?')})"
                             for d in pools)
    except Exception:  # pragma: no cover
        pass
    groups = {}
    for i, e in enumerate(wl.entries):
        pr = e.split_rows or e.rows
        key = (min(pr, e.cols), max(pr, e.cols))
        groups.setdefault(key, []).append(i)
    timed_flops, timed_s, names = 0.0, 0.0, []
    for key, idx in groups.items():
        if timed_s > budget_s * 0.4 and names:
            break
        i = idx[0]
        e = wl.entries[i]
        g, p = W.entry_values(wl, i)
        g64 = W.grad_as_f64(wl, g.ravel())
        t0 = time.perf_counter()
        oracle.muon_step(p.ravel(), g64, np.zeros(g64.size), [(0, e.rows, e.cols, e.split_rows)],
                         lr=wl.lr, mu=wl.momentum, weight_decay=wl.weight_decay, method=method)
        dt = time.perf_counter() - t0
        blocks = e.rows // (e.split_rows or e.rows)
        timed_flops += blocks * ns_flops(key[0], key[1], method)
        timed_s += dt
        names.append(f"{e.rows}x{e.cols}" + (f"/split{e.split_rows}" if e.split_rows else ""))
    total_flops = sum(ns_flops(m, n, method) for m, n in problems(wl))
    est_step_s = timed_s * total_flops / timed_flops
    return {"value": wl.muon_elements / est_step_s, "unit": "elements/s", "cores": int(cores),
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "blas": blas,
            "sample": (f"float64 exact-mode oracle, {method} NS, one matrix per shape group "
                       f"({', '.join(names)}) timed {timed_s:.1f} s; whole step extrapolated "
                       f"by nominal NS FLOPs to {est_step_s:.1f} s")}


def copy_calibration(nbytes: int = 1 << 32) -> dict:
    """One plain device copy of `nbytes` through the library's copy kernel
    (muon_pack with a single entry): the known-size reference that scales the
    FETCH_SIZE / WRITE_SIZE counters, and the copy bandwidth of this GPU."""
    import torch
    import newton_schulz_step_amd as nss
    nss.load()
    dev = torch.device("cuda:0")
    n = nbytes // 4
    src = torch.ones(n, device=dev)
    dst = torch.zeros(n, device=dev)
    cols = 65536
    tab = [(0, n // cols, cols, 0)]          # one entry covering the whole buffer
    for _ in range(2):
        nss.pack(dst, [src], tab)
    torch.cuda.synchronize()
    reps = 5
    nss.profile_begin()
    for _ in range(reps):
        nss.pack(dst, [src], tab)
    torch.cuda.synchronize()
    launches, ms = nss.profile_end()["copy_batch"]
    return {"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": launches,
            "avg_launch_ms": ms / launches, "copy_gbs": 2 * nbytes * launches / (ms * 1e-3) / 1e9}


def adamw_pass(wl, steps: int = 10) -> dict:
    """AdamW over the workload's non-2D tensors (one flat buffer), bf16 grads:
    26 algorithmic bytes per element (p, m, v read and written, g read)."""
    import torch
    import newton_schulz_step_amd as nss
    n = sum(wl.adamw_sizes)
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    p = torch.randn(n, device=dev, generator=gen)
    g = torch.randn(n, device=dev, generator=gen).to(torch.bfloat16)
    m = torch.zeros(n, device=dev)
    v = torch.zeros(n, device=dev)
    kw = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    nss.adamw(p, g, m, v, step=1, **kw)
    torch.cuda.synchronize()
    nss.profile_begin()
    for t in range(steps):
        nss.adamw(p, g, m, v, step=t + 2, **kw)
    torch.cuda.synchronize()
    launches, ms = nss.profile_end()["adamw"]
    gbs = 26.0 * n * launches / (ms * 1e-3) / 1e9
    return {"elements": n, "launches": launches, "avg_launch_ms": ms / launches, "gbs": gbs,
            "frac_of_hbm": gbs / HBM_PEAK_GBS}


def workload_hyper(nss, wl, method):
    ns_dtype = "f32" if wl.ns_dtype == "f32" else ("bf16" if method == "standard" else "f16")
    h = nss.hyper(ns_method=method, ns_dtype=ns_dtype, grad_dtype=wl.grad_dtype, lr=wl.lr,
                  momentum=wl.momentum, weight_decay=wl.weight_decay)
    return h, ns_dtype


def timed_steps(nss, bufs, tab, h, ws, steps, warmup):
    """`warmup` untimed steps, then `steps` timed ones between device
    synchronisations, with the library's per-launch events on. Returns (elapsed
    seconds, {kernel kind: (launches, summed ms)})."""
    import torch
    params, grads, mom = bufs
    for _ in range(warmup):
        nss.step(params, grads, mom, tab, h, ws=ws)
    torch.cuda.synchronize()
    nss.profile_begin()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        nss.step(params, grads, mom, tab, h, ws=ws)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    return elapsed, nss.profile_end()


def dominant_roofline(wl, method, ns_dtype, h, kstats, steps):
    """Roofline of the step's dominant kernel, from its summed launch time.

    Standard: the update GEMM B X (+ a X), algorithmic 2 m^2 n per problem per
    launch; on 128-row problems in 16-bit the update and the next X X^T are one
    pass (ns_update_gram), bound by memory: algorithmic bytes per problem per
    launch are X read and X' written (2 m n elements) plus B read and A' written
    (2 m^2 elements). Gram: its symmetric GEMM family (R0, five Q, four T = R Q,
    four R <- Q T), counting the lower tiles these launches compute: m^2 n + 13 m^3
    per problem; on 128-row problems in fp16, where the chain runs in LDS, the
    apply X = P X0, bound by memory: X0 read (2 m n bytes), params read and
    written (8 m n)."""
    probs = problems(wl)
    peak = FP32_PEAK_TFLOPS if ns_dtype == "f32" else BF16_PEAK_TFLOPS
    bound, unit, roof_peak = "mfma", "TFLOP/s", peak
    if method == "standard" and kstats.get("ns_update_gram", (0, 0.0))[1] > \
            kstats.get("ns_gemm_update", (0, 0.0))[1]:
        dom_kind = "ns_update_gram"
        dt_name = {"bf16": "__bf16", "f16": "_Float16"}[ns_dtype]
        dom_kernel = f"muon::ns_update_gram<{dt_name}>"
        launches, dom_ms = kstats[dom_kind]
        dom_work = sum(2 * (2.0 * m * n + 2.0 * m * m) for m, n in probs if m <= 128) * \
            (h.ns_steps - 1) * steps
        bound, unit, roof_peak = "hbm", "GB/s", HBM_PEAK_GBS
        achieved = dom_work / (dom_ms * 1e-3) / 1e9 if dom_ms > 0 else None
    elif method == "standard":
        dom_kind = "ns_gemm_update"
        tile = 256 if probs and probs[0][0] >= 512 else 128
        dt_name = {"bf16": "__bf16", "f16": "_Float16", "f32": "float"}[ns_dtype]
        dom_kernel = f"muon::ns_gemm<{dt_name}, {tile}, false, 0, true, false>"
        launches, dom_ms = kstats.get(dom_kind, (0, 0.0))
        dom_flops = sum(2.0 * m * m * n for m, n in probs) * (h.ns_steps - 1) * steps
        achieved = dom_flops / (dom_ms * 1e-3) / 1e12 if dom_ms > 0 else None
    elif kstats.get("gram_gemm_apply", (0, 0.0))[1] > kstats.get("gram_gemm_sym", (0, 0.0))[1]:
        # 128-row problems in fp16 (the chain runs in LDS): the apply X = P X0,
        # bound by memory: X0 read, fp32 params read and written
        dom_kind = "gram_gemm_apply"
        dom_kernel = "muon::ns_gemm<_Float16, 128, false, 1, true, false>"
        launches, dom_ms = kstats[dom_kind]
        dom_work = sum(2.0 * m * n + 8.0 * m * n for m, n in probs if m <= 128) * steps
        bound, unit, roof_peak = "hbm", "GB/s", HBM_PEAK_GBS
        achieved = dom_work / (dom_ms * 1e-3) / 1e9 if dom_ms > 0 else None
    else:
        dom_kind = "gram_gemm_sym"
        tile = 256 if probs and probs[0][0] >= 512 else 128
        dom_kernel = f"muon::ns_gemm<{'_Float16' if ns_dtype == 'f16' else 'float'}, {tile}, true, 0, false, HAS_D>"
        launches, dom_ms = kstats.get(dom_kind, (0, 0.0))
        dom_flops = sum(1.0 * m * m * n + 13.0 * m ** 3 for m, n in probs) * steps
        achieved = dom_flops / (dom_ms * 1e-3) / 1e12 if dom_ms > 0 else None
    return {"bound": bound, "kernel": dom_kernel, "kind": dom_kind, "launches": launches,
            "avg_launch_ms": dom_ms / launches if launches else None,
            "achieved": achieved, "peak": roof_peak, "unit": unit,
            "frac": achieved / roof_peak if achieved else None}


def step_summary(wl, method, ns_dtype, elapsed, kstats, steps):
    """Per-step figures of one timed run over a whole workload (or a sub-table):
    Muon elements/s; NS TFLOP/s over the summed NS kernel time, both with the
    nominal FLOPs and with symmetric products counted once; the step's
    algorithmic bandwidth (18 B per element for 16-bit gradients, 20 B for fp32:
    gradient read, momentum and params read and written); and the step's
    fraction of its roofline: the larger of the ideal MFMA time (least FLOPs at
    the dense peak) and the ideal HBM time (algorithmic bytes at 8 TB/s), over
    the measured step time."""
    probs = problems(wl)
    elems = sum(m * n for m, n in probs)
    step_s = elapsed / steps
    ns_kinds = [k for k in kstats if k.startswith(("ns_gemm", "gram_gemm", "ns_update_gram"))]
    ns_ms = sum(kstats[k][1] for k in ns_kinds) / steps
    nominal = sum(ns_flops(m, n, method) for m, n in probs)
    least = sum(ns_flops_min(m, n, method) for m, n in probs)
    peak = FP32_PEAK_TFLOPS if ns_dtype == "f32" else BF16_PEAK_TFLOPS
    bpe = 20.0 if wl.grad_dtype == "f32" else 18.0
    t_mfma = least / (peak * 1e12)
    t_hbm = elems * bpe / (HBM_PEAK_GBS * 1e9)
    return {
        "ms_per_step": step_s * 1e3, "elements_per_s": elems / step_s, "muon_elements": elems,
        "ns_ms_per_step": ns_ms,
        "ns_tflops_nominal": nominal / (ns_ms * 1e-3) / 1e12 if ns_ms > 0 else None,
        "ns_tflops_least": least / (ns_ms * 1e-3) / 1e12 if ns_ms > 0 else None,
        "ns_least_frac_of_peak": least / (ns_ms * 1e-3) / 1e12 / peak if ns_ms > 0 else None,
        "step_algorithmic_gbs": elems * bpe / step_s / 1e9,
        "step_bound": "mfma" if t_mfma >= t_hbm else "hbm",
        "step_roofline_frac": max(t_mfma, t_hbm) / step_s,
        "kernels_ms_per_step": {k: round(v[1] / steps, 4) for k, v in kstats.items()},
    }


def group_key(e):
    pr = e.split_rows or e.rows
    return (min(pr, e.cols), max(pr, e.cols))


def measure_workload(nss, wid, steps, warmup, groups=True):
    """Both methods over the whole workload, then each shape group alone with both
    methods (the pages say Gram NS is about twice as fast on rectangular
    matrices). Inputs are drawn on the device once and shared by all runs (the
    cost does not depend on the values)."""
    import torch
    import workloads as W
    dev = torch.device("cuda:0")
    wl = W.workload(wid)
    bufs = device_inputs(wl, dev)
    tab = wl.table()
    hs = {m: workload_hyper(nss, wl, m) for m in ("standard", "gram")}
    ws = nss.workspace(max(nss.workspace_size(tab, h) for h, _ in hs.values()), dev)
    out = {"workload": wl.title, "muon_elements": wl.muon_elements}
    for method, (h, ns_dtype) in hs.items():
        elapsed, kstats = timed_steps(nss, bufs, tab, h, ws, steps, warmup)
        row = step_summary(wl, method, ns_dtype, elapsed, kstats, steps)
        row["ns_dtype"] = ns_dtype
        row["dominant_kernel"] = dominant_roofline(wl, method, ns_dtype, h, kstats, steps)
        out[method] = row
    if groups:
        keys = []
        for e in wl.entries:
            if group_key(e) not in keys:
                keys.append(group_key(e))
        rows = []
        for key in keys:
            idx = [i for i, e in enumerate(wl.entries) if group_key(e) == key]
            sub = [tab[i] for i in idx]
            sub_wl = W.Workload(wl.wid, wl.title, tuple(wl.entries[i] for i in idx), wl.grad_dtype,
                                wl.ns_dtype, wl.lr, wl.momentum, wl.weight_decay)
            r = {"m": key[0], "n": key[1], "problems": len(problems(sub_wl))}
            for method, (h, ns_dtype) in hs.items():
                elapsed, kstats = timed_steps(nss, bufs, sub, h, ws, steps, 1)
                r[method + "_ms"] = elapsed * 1e3 / steps
                r[method + "_ns_ms"] = step_summary(sub_wl, method, ns_dtype, elapsed, kstats,
                                                    steps)["ns_ms_per_step"]
            r["standard_over_gram"] = r["standard_ms"] / r["gram_ms"]
            r["flops_standard_over_gram"] = ns_flops(key[0], key[1], "standard") / ns_flops(key[0], key[1], "gram")
            rows.append(r)
        out["shape_groups"] = rows
    del bufs, ws
    torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=None,
                    help="time this workload only (default: the owner share, then every workload)")
    ap.add_argument("--method", default="standard", choices=["standard", "gram"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload table")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV",
                                                              "FETCH_COPY_CSV", "WRITE_COPY_CSV"))
    ap.add_argument("--summarize-mfma", metavar="MFMA_CSV")
    args = ap.parse_args()
    workload = args.workload if args.workload is not None else 3
    if args.summarize_mfma:
        symbol = ("_ZN4muon7ns_gemmIDF16bLi256ELb0ELi0ELb1ELb0EEEvNS_9GemmBatchE" if args.method == "standard"
                  else "_ZN4muon7ns_gemmIDF16_Li256ELb1ELi0ELb0ELb0EEEvNS_9GemmBatchE")
        rec = summarize_mfma(args.summarize_mfma, symbol)
        run = (f"python3 $REPO/bench.py --workload {workload} --method {args.method} "
               "--steps 2 --warmup 1 --no-cpu-baseline")
        rec["commands"] = [
            "cd /tmp && export TMPDIR=/tmp",
            f"rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE -d <mfma> -o run --output-format csv -- {run}",
            f"python3 bench.py --workload {workload} --method {args.method} "
            "--summarize-mfma <mfma>/run_counter_collection.csv",
        ]
        path = os.path.join(ROOT, "profiles", f"mfma_ns_gemm_update_{WORKLOAD_SLUG[workload]}_{args.method}.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return 0
    if args.summarize_counters:
        ns_dtype = "bf16" if args.method == "standard" else "f16"
        symbol = ("_ZN4muon7ns_gemmIDF16bLi256ELb0ELi0ELb1ELb0EEEvNS_9GemmBatchE" if ns_dtype == "bf16"
                  else "_ZN4muon7ns_gemmIDF16_Li256ELb1ELi0ELb0ELb0EEEvNS_9GemmBatchE")
        rec = summarize_counters(*args.summarize_counters, copy_bytes=1 << 32, symbol=symbol,
                                 workload=workload, method=args.method)
        with open(traffic_path(workload, args.method), "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "owner exchange is not part of this library", file=sys.stderr)
        return 2

    import torch
    import newton_schulz_step_amd as nss
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    nss.load()
    if args.copy_calibration:
        print(json.dumps(copy_calibration()), flush=True)
        return 0
    dev = torch.device("cuda:0")
    wl = W.workload(workload)
    h, ns_dtype = workload_hyper(nss, wl, args.method)
    tab = wl.table()
    bufs = device_inputs(wl, dev)
    ws = nss.workspace(nss.workspace_size(tab, h), dev)
    torch.cuda.synchronize()
    elapsed, kstats = timed_steps(nss, bufs, tab, h, ws, args.steps, args.warmup)

    probs = problems(wl)
    elems = wl.muon_elements
    value = elems * args.steps / elapsed
    ns_total = sum(ns_flops(m, n, args.method) for m, n in probs) * args.steps
    ns_kinds = [k for k in kstats if k.startswith(("ns_gemm", "gram_gemm"))]
    ns_ms = sum(kstats[k][1] for k in ns_kinds)
    peak = FP32_PEAK_TFLOPS if ns_dtype == "f32" else BF16_PEAK_TFLOPS
    roof = dominant_roofline(wl, args.method, ns_dtype, h, kstats, args.steps)
    roof["traffic"] = measured_traffic(roof["kernel"], workload, args.method)
    mom_launches, mom_ms = kstats.get("momentum_sumsq", (0, 0.0))
    gbytes = elems * (10 if wl.grad_dtype != "f32" else 12) * args.steps / 1e9
    summary = step_summary(wl, args.method, ns_dtype, elapsed, kstats, args.steps)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ns_dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.title + ": " + ", ".join(
                sorted({f"{sum(1 for x in wl.entries if (x.rows, x.cols) == (e.rows, e.cols))}x"
                        f"{e.rows}x{e.cols}" for e in wl.entries})),
            "ns_method": args.method, "ns_dtype": ns_dtype, "grad_dtype": wl.grad_dtype,
            "param_dtype": "f32", "muon_elements": elems, "problems": len(probs),
            "lr": wl.lr, "momentum": wl.momentum, "weight_decay": wl.weight_decay,
            "ns_steps": h.ns_steps, "parallelism": "single GPU",
        },
        "ns_tflops": ns_total / (ns_ms * 1e-3) / 1e12 if ns_ms > 0 else None,
        "ns_frac_of_peak": (ns_total / (ns_ms * 1e-3) / 1e12 / peak) if ns_ms > 0 else None,
        "ns_tflops_least": summary["ns_tflops_least"],
        "ns_least_frac_of_peak": summary["ns_least_frac_of_peak"],
        "step_roofline_frac": summary["step_roofline_frac"],
        "roofline": {k: roof[k] for k in ("bound", "kernel", "launches", "avg_launch_ms", "achieved",
                                           "peak", "unit", "frac", "traffic")},
        "momentum_pass": {
            "launches": mom_launches,
            "gbs": gbytes / (mom_ms * 1e-3) if mom_ms > 0 else None,
            "frac_of_hbm": gbytes / (mom_ms * 1e-3) / HBM_PEAK_GBS if mom_ms > 0 else None,
        },
        "kernels_ms_per_step": summary["kernels_ms_per_step"],
    }
    del bufs, ws
    torch.cuda.empty_cache()
    out["adamw_pass"] = adamw_pass(W.workload(5))
    out["adamw_pass"]["workload"] = "32000x4096 embedding + 65 vectors of 4096 (per-head workload's AdamW part)"
    if args.workload is None and not args.no_configs:
        csteps = max(3, min(args.steps, 10))
        out["configs"] = {}
        for wid in (1, 2, 3, 4, 5):
            t0 = time.perf_counter()
            out["configs"][WORKLOAD_SLUG[wid]] = measure_workload(nss, wid, csteps, 1)
            print(f"[bench] workload {wid} measured in {time.perf_counter() - t0:.1f} s",
                  file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.method)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
