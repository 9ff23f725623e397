#!/usr/bin/env python3
"""Benchmark: 2-D convolution backward-data on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--problem NAME]

Workload (default): the bf16 NHWC stride-(1,2) problem of fusilli issue #101
-- dY 16x1x256x2048, W 2048x1x2x2048 (KYXC), dX 16x1x512x2048, fp32
accumulation, bf16 result -- seeded synthetic N(0,1) / N(0,0.02) operands
already resident in HBM.  One step = one cbd_run (every launch of the hot
path: the residue-class GEMM kernel, plus the zero-fill kernel when the
problem has unreached phases).

Prints ONE JSON line:
  value        useful TFLOP/s (2*N*C*(K/G)*Ho*Wo*Y*X per step, zero-insertion
               work excluded) over the K timed steps, wall clock between two
               device synchronisations; the K calls are captured once in a HIP
               graph and replayed (cbd_run launches kernels only), or with
               --no-graph issued one by one.  Before them: the W warmup calls,
               then untimed calls for about --settle-ms of GPU time (the clock
               of the part rises over the first tens of milliseconds of
               sustained load; `settle` in the line gives the count);
  roofline     dominant kernel: algorithmic flops (or bytes) per launch divided
               by its mean launch duration from HIP events recorded on the
               launch stream (around the replay / K, or around each call),
               against the bf16 dense MFMA peak (or HBM);
               `traffic` = HBM bytes per launch from rocprofv3 FETCH_SIZE +
               WRITE_SIZE (profiles/, scaled by a plain copy of known size),
               null when the kernel source changed after the counters were taken;
  cpu_baseline the CPU oracle's loop nest on the host cores over the whole
               problem (one call, nothing scaled), with the parity of the
               GPU's whole dX against it (relative L2, max error, bf16 ulps,
               exact zeros; `pass` applies the fp32 or bf16 tolerance);
  machine      GPU name and architecture, HIP version, maximum shader clock,
               host CPU model.

    python bench.py --all      one line per workload problem: warm, graph and
                               cold (caches flushed) us/call, roofline fractions,
                               and the same sampled oracle check (about 1 s each).
    python bench.py --problem P --cold-calls 50
                               only calls each after a cache sweep (run under
                               rocprofv3 --kernel-trace for cold kernel durations).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "conv bwd-data useful TFLOP/s + µs/call on 1 MI355X, % of MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU * 2.4 GHz * 4096 dense bf16 flop/clk/CU
PEAK_F32_TFLOPS = 157.3     # 256 CU * 2.4 GHz * 256 f32 MFMA flop/clk/CU
PEAK_HBM_GBS = 8000.0
# (kernel family, row variant) -> source file and kernel symbol
KERNEL_SRC = {(0, 0): "kern_igemm_generic.hip", (1, 0): "kern_igemm_nhwc_bf16.hip",
              (2, 0): "kern_grouped_direct.hip", (2, 1): "kern_grouped_rows.hip",
              (2, 2): "kern_grouped_pipe.hip", (2, 3): "kern_grouped_mfma.hip",
              (2, 4): "kern_grouped_wide.hip", (3, 0): "kern_nchw_rows.hip"}
KERNEL_SYMBOL = {(0, 0): "igemm_generic_kernel", (1, 0): "igemm_nhwc_bf16_kernel",
                 (2, 0): "grouped_direct_kernel", (2, 1): "grouped_rows_kernel",
                 (2, 2): "grouped_pipe_kernel", (2, 3): "grouped_mfma_kernel",
                 (2, 4): "grouped_wide_kernel", (3, 0): "nchw_rows_kernel"}
# Bound of each workload problem (dense-contraction rows on MFMA, the rest on
# HBM; the small fp32 rows are launch-latency bound in practice).
LATENCY_BOUND = ("c1", "c2-14-1", "c2-14-3", "c2-15-1", "c2-15-3", "c2-16-1", "c2-16-3")
HBM_BOUND = ("c3b", "c5-s2", "c5-s1")


def describe(p):
    lay = "NCHW/KCYX" if p.layout == 0 else "NHWC/KYXC"
    return (f"conv2d_bwd_data {p.dtype} {lay} N={p.n} G={p.g} C={p.c} K={p.k} "
            f"Hi={p.hi} Wi={p.wi} {p.y}x{p.x} stride=({p.sh},{p.sw}) pad=({p.ph},{p.pw}) "
            f"dil=({p.dh},{p.dw})")


def algorithmic_bytes(p, info):
    """dY elements some valid tap reads + all of W + all of dX (zeros included)."""
    es = 4 if p.dtype == "f32" else 2
    ho, wo = info.ho, info.wo

    def used(extent_out, extent_in, pad, dil, taps, stride):
        return sum(1 for o in range(extent_out)
                   if any(0 <= o * stride + t * dil - pad < extent_in for t in range(taps)))
    dy_used = p.n * p.k * used(ho, p.hi, p.ph, p.dh, p.y, p.sh) * used(wo, p.wi, p.pw, p.dw, p.x, p.sw)
    return es * (dy_used + p.k * (p.c // p.g) * p.y * p.x + p.n * p.c * p.hi * p.wi)


def kernel_key(info):
    return (info.kernel, info.variant)


# Headers every kernel source includes: a change in them changes the kernels.
KERNEL_HEADERS = ("cbd_device.h", "cbd_kernarg.h", "cbd_internal.h", "cbd_geo.h", "generic_shapes.h")


def kernel_digest(key):
    """sha256 over the kernel's source file followed by the shared headers."""
    h = hashlib.sha256()
    for f in (KERNEL_SRC[key],) + KERNEL_HEADERS:
        h.update(open(os.path.join(ROOT, "dnn_conv2d_bwd_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def read_traffic(key, problem):
    """HBM bytes per launch recorded under profiles/ for this kernel on this
    problem, if the kernel source and shared headers still match the ones the
    counters were taken on."""
    name = KERNEL_SYMBOL[key][:-len("_kernel")]
    path = os.path.join(ROOT, "profiles", f"{name}_{problem}_traffic.txt")
    if not os.path.exists(path):
        return None
    digest = kernel_digest(key)
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != digest:
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(p, dy, w, info, dx_gpu=None):
    """The oracle's loop nest (bwd_data: fp64, OpenMP over the host threads)
    on the whole problem, one call, wall-clocked; nothing is scaled.  Given
    the GPU's dX (host array in the layout's memory order), also the parity
    of the whole GPU result against that oracle result (parity_of)."""
    import oracle

    total = p.n * p.c * p.hi * p.wi
    t0 = time.perf_counter()
    ref = oracle.bwd_data(p, dy, w)
    dt = time.perf_counter() - t0
    threads = oracle.num_threads()
    out = {"value": round(info.useful_flops / dt / 1e12, 6), "unit": "TFLOP/s",
           "cores": threads, "oracle_threads": threads, "kind": "oracle", "oracle_s": round(dt, 3),
           "sample": f"the whole problem: one call of the oracle's fp64 loop nest (bwd_data) "
                     f"over all {total} dX elements on {threads} OpenMP threads, {dt:.2f} s; "
                     f"nothing scaled"}
    if dx_gpu is not None:
        out["parity"] = parity_of(p, dx_gpu.ravel(), ref.ravel())
    return out


def parity_of(p, got, ref64):
    """The GPU's dX (flat, any float dtype) against the oracle (flat fp64).
    fp32: relative L2 <= 1e-5 and max |err| <= 1e-4 max |ref|.  bf16: relative
    L2 <= 8e-3 and every element within 2 bf16 ulps of the oracle rounded to
    f32 then bf16, ulps counted at magnitude max(|ref|, 2^-10 rms(ref))
    (floored) and at |ref| itself (strict, reported only).  Elements whose
    oracle value is exactly 0 (unreached or edge positions) must be exactly 0."""
    import numpy as np

    import oracle

    got = got.astype(np.float64)
    ref32 = oracle.round_f32(ref64).astype(np.float64)
    norm = float(np.linalg.norm(ref64))
    rel_l2 = float(np.linalg.norm(got - ref64) / norm) if norm > 0 else float(np.abs(got).max())
    max_ref = float(np.abs(ref64).max())
    max_abs = float(np.abs(got - ref64).max())
    zeros_ok = bool(np.all(got[ref64 == 0.0] == 0.0))
    res = {"elements": int(len(ref64)), "rel_l2": rel_l2, "max_abs": max_abs, "max_ref": max_ref,
           "zeros_ok": zeros_ok}
    if p.dtype == "f32":
        ok = rel_l2 <= 1e-5 and max_abs <= 1e-4 * max_ref
    else:
        rb = oracle.bf16_bits_to_f32(oracle.round_bf16_bits(ref32.astype(np.float32))).astype(np.float64)
        rms = float(np.sqrt(np.mean(ref32 ** 2)))

        def ulps(mag):
            e = np.floor(np.log2(np.maximum(mag, np.finfo(np.float32).tiny)))
            return np.abs(got - rb) / np.exp2(e - 7)
        floored = ulps(np.maximum(np.abs(ref32), 2.0 ** -10 * rms))
        strict = ulps(np.abs(ref32))
        res.update({"ulp_max": float(floored.max()), "ulp_viol_floored": int((floored > 2).sum()),
                    "ulp_viol_strict": int((strict > 2).sum())})
        ok = rel_l2 <= 8e-3 and res["ulp_viol_floored"] == 0
    res["pass"] = bool(ok and zeros_ok)
    return res


def graph_us(cbd, torch, pl, dy_d, w_d, dx_d, ws=None, calls=200, reps=3):
    """GPU µs per call: `calls` calls captured in a HIP graph, replayed once
    untimed and then `reps` times under one event pair (no host launch cost;
    a replay's own fixed launch cost, ≈ 12 µs, is spread over `calls`)."""
    stream = torch.cuda.current_stream()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        cbd.run(pl, dy_d, w_d, dx_d, stream=cap, workspace=ws)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            for _ in range(calls):
                cbd.run(pl, dy_d, w_d, dx_d, stream=cap, workspace=ws)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(reps):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    return g0.elapsed_time(g1) * 1e3 / (calls * reps)


def roof_of(p, info, us):
    """(bound, achieved, peak, unit) of a problem's own roofline at `us` per call."""
    if p.name in HBM_BOUND:
        return "hbm", algorithmic_bytes(p, info) / us / 1e3, PEAK_HBM_GBS, "GB/s"
    peak = PEAK_BF16_TFLOPS if p.dtype == "bf16" else PEAK_F32_TFLOPS
    return "mfma", info.useful_flops / us / 1e6, peak, "TFLOP/s"


SECONDARY = ("c3a", "c3b", "c5-s2", "c5-s1")


def secondary_rows():
    """Graph-mode µs per call and roofline fraction of the other rows whose
    kernels carry a roofline claim (no oracle)."""
    import torch

    import dnn_conv2d_bwd_amd as cbd
    from cbd_inputs import draw, problem_by_name, seed_for

    rows = {}
    for name in SECONDARY:
        p = problem_by_name(name)
        dt = cbd.F32 if p.dtype == "f32" else cbd.BF16
        pl = cbd.plan(p.n, p.g, p.c, p.k, p.hi, p.wi, p.y, p.x, (p.sh, p.sw), (p.ph, p.pw),
                      (p.dh, p.dw), p.layout, dt)
        info = pl.info()
        sh = pl.shapes()
        tdt = torch.float32 if p.dtype == "f32" else torch.bfloat16
        dy_d = torch.from_numpy(draw(p.dist_dy, seed_for(p, "dy"), sh["dy"], p.dtype)).to(tdt).cuda()
        w_d = torch.from_numpy(draw(p.dist_w, seed_for(p, "w"), sh["w"], p.dtype)).to(tdt).cuda()
        dx_d = torch.empty(sh["dx"], dtype=tdt, device="cuda")
        ws = (torch.empty(pl.workspace_size(), dtype=torch.uint8, device="cuda")
              if pl.workspace_size() else None)
        for _ in range(10):
            cbd.run(pl, dy_d, w_d, dx_d, workspace=ws)
        us = graph_us(cbd, torch, pl, dy_d, w_d, dx_d, ws)
        bound, ach, peak, unit = roof_of(p, info, us)
        rows[name] = {"workload": describe(p), "kernel": KERNEL_SYMBOL[kernel_key(info)],
                      "us_graph": round(us, 3), "bound": bound, "achieved": round(ach, 2),
                      "peak": peak, "unit": unit, "frac": round(ach / peak, 4)}
        del dy_d, w_d, dx_d, ws
    return rows


def machine():
    """GPU name, HIP version, shader clock and host CPU model."""
    import torch

    props = torch.cuda.get_device_properties(0)
    cpu = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    # Highest shader-clock level the amdgpu kernel module lists (sysfs), if readable.
    sclk = None
    import glob
    for f in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"):
        try:
            for line in open(f):
                tok = line.split(":", 1)[-1].strip().split()[0].lower()
                if tok.endswith("mhz"):
                    sclk = max(sclk or 0, int(float(tok[:-3])))
        except (OSError, ValueError, IndexError):
            pass
    return {"gpu_name": torch.cuda.get_device_name(0), "gcn_arch": getattr(props, "gcnArchName", ""),
            "hip_version": torch.version.hip, "sclk_max_mhz": sclk,
            "cpu_model": cpu, "host_cpus": os.cpu_count()}


def copy_calibration(nbytes, reps):
    """A plain device copy of known size (for scaling rocprofv3 byte counters)."""
    import torch

    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- profiles ---
# Summaries under profiles/ of rocprofv3 passes over this script, one pass per
# directory under RAW named <pass>_<problem>:
#   kt    rocprofv3 --kernel-trace --stats ... -- bench.py PROF --problem P --steps 50 --warmup 5
#           (with the clock-settle calls; the summary also gives the 50 timed calls alone)
#   ktng  the same with --no-graph (calls issued one by one)
#   ktcold rocprofv3 --kernel-trace --stats ... -- bench.py PROF --problem P --cold-calls 50
#           (each call after a cache sweep: the kernel's cold duration)
#   fetch rocprofv3 --pmc FETCH_SIZE ... -- bench.py PROF --problem P --steps 10 --warmup 2
#           --no-graph --settle-ms 0 --copy-calibration-mib 1024      (write: WRITE_SIZE)
#   mfma  rocprofv3 --pmc <MFMA_COUNTERS> ... --no-graph --settle-ms 0; stall: <STALL_COUNTERS>
PROF = "--cpu-seconds 0 --no-secondary"
MFMA_COUNTERS = "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE"
STALL_COUNTERS = ("SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY "
                  "SQ_VALU_MFMA_BUSY_CYCLES SQ_WAIT_INST_LDS SQ_WAVES")
ROCPROF = "cd /tmp && rocprofv3"


def pass_command(kind, prob):
    out = f"--output-format csv -d <out>/{kind}_{prob} -o prof -- python3 bench.py {PROF} --problem {prob}"
    if kind in ("kt", "ktng"):
        return f"{ROCPROF} --kernel-trace --stats {out} --steps 50 --warmup 5" + (" --no-graph" if kind == "ktng" else "")
    if kind == "ktcold":
        return f"{ROCPROF} --kernel-trace --stats {out} --cold-calls 50"
    pmc = {"fetch": "FETCH_SIZE", "write": "WRITE_SIZE", "mfma": MFMA_COUNTERS, "stall": STALL_COUNTERS}[kind]
    cal = " --copy-calibration-mib 1024" if kind in ("fetch", "write") else ""
    return f"{ROCPROF} --pmc {pmc} {out} --steps 10 --warmup 2 --no-graph --settle-ms 0{cal}"


def summarize_profiles(raw):
    """Write the profiles/ summaries of the rocprofv3 passes found under raw."""
    import collections
    import csv
    import statistics

    import dnn_conv2d_bwd_amd as cbd
    from cbd_inputs import problem_by_name

    def kernel_of(prob):
        p = problem_by_name(prob)
        dt = cbd.F32 if p.dtype == "f32" else cbd.BF16
        info = cbd.plan(p.n, p.g, p.c, p.k, p.hi, p.wi, p.y, p.x, (p.sh, p.sw), (p.ph, p.pw),
                        (p.dh, p.dw), p.layout, dt).info()
        return kernel_key(info), describe(p)

    def trace(d, sym):
        """Kernel name and its dispatch durations (us) in start order."""
        rows = [r for r in csv.DictReader(open(os.path.join(d, "prof_kernel_trace.csv"))) if sym in r["Kernel_Name"]]
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0 for r in rows]
        return rows[0]["Kernel_Name"], durs

    def bench_line(d):
        f = d.rstrip("/") + ".out"
        try:
            return json.loads(open(f).read().strip().splitlines()[-1])
        except (OSError, ValueError, IndexError):
            return None

    def counters(d, sym):
        agg = collections.defaultdict(float)
        grid = {}
        for r in csv.DictReader(open(os.path.join(d, "prof_counter_collection.csv"))):
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"], r["Counter_Name"])
            agg[key] += float(r["Counter_Value"])
            grid[int(r["Dispatch_Id"])] = int(r.get("Grid_Size") or 0)
        mine = collections.defaultdict(list)
        copies = collections.defaultdict(list)
        for (disp, k, c), v in agg.items():
            if sym in k:
                mine[c].append(v)
            elif "copyBuffer" in k:
                copies[c].append((grid[disp], v))
        # calibration copies: the largest copy dispatches (smaller ones are
        # the operands' staging copies)
        cal = {}
        for c, lst in copies.items():
            g = max(x for x, _ in lst)
            cal[c] = [v for x, v in lst if x == g]
        return mine, cal

    written = []
    passes = collections.defaultdict(dict)
    for d in sorted(os.listdir(raw)):
        if os.path.isdir(os.path.join(raw, d)) and "_" in d:
            kind, prob = d.split("_", 1)
            passes[prob][kind] = os.path.join(raw, d)
    for prob, ks in passes.items():
        key, desc = kernel_of(prob)
        sym = KERNEL_SYMBOL[key][:-len("_kernel")]
        base = os.path.join(ROOT, "profiles", f"{sym}_{prob}")
        summary_cmd = f"python3 bench.py --summarize-profiles <out>"
        if "kt" in ks:
            out = ["# rocprofv3 kernel-trace summary: " + desc, ""]
            for kind, title in (("kt", "calls replayed from a HIP graph (the benchmark's timing)"),
                                ("ktng", "calls issued one by one")):
                if kind not in ks:
                    continue
                name, d_ = trace(ks[kind], sym)
                b = bench_line(ks[kind])
                steps = b["steps"] if b else 50
                row = lambda lbl, x: (f"| {lbl} | {len(x)} | {statistics.mean(x):.3f} | {statistics.median(x):.3f} | "
                                      f"{min(x):.3f} | {max(x):.3f} |")
                out += [f"## {prob}, {title}", f"command: {pass_command(kind, prob)}", f"summary: {summary_cmd}",
                        f"kernel: {name}", "",
                        "| dispatches | calls | avg us | median us | min us | max us |", "|---|---|---|---|---|---|",
                        row("all (warmup, capture, clock settle, timed)", d_),
                        row(f"the {steps} timed calls (the last {steps})", d_[-steps:]), ""]
                if b:
                    out += [f"The same run's own HIP-event time per call ({b['config']['timing']}, after "
                            f"{b.get('settle', {}).get('calls', 0)} clock-settle calls): "
                            f"{b['roofline']['launch_us_mean']} us.", ""]
            open(base + "_kernel_trace.md", "w").write("\n".join(out))
            written.append(base + "_kernel_trace.md")
        if "ktcold" in ks:
            name, d_ = trace(ks["ktcold"], sym)
            b = bench_line(ks["ktcold"])
            row = (f"| {len(d_)} | {statistics.mean(d_):.3f} | {statistics.median(d_):.3f} | "
                   f"{min(d_):.3f} | {max(d_):.3f} |")
            out = [f"# rocprofv3 kernel-trace summary, cold caches: {desc}", "",
                   f"## {prob}, calls each after a 512 MiB read sweep (L2 and MALL evicted), one at a time",
                   f"command: {pass_command('ktcold', prob)}", f"summary: {summary_cmd}",
                   f"kernel: {name}", "",
                   "| dispatches | avg us | median us | min us | max us |", "|---|---|---|---|---|", row, ""]
            if b:
                med = statistics.median(d_)
                if prob in HBM_BOUND:
                    mb = b["alg_mbytes"]
                    roof = (f"Algorithmic bytes {mb} MB per call: {mb / med:.3f} TB/s at the median "
                            f"dispatch, {mb / med / (PEAK_HBM_GBS / 1e3):.3f} of 8 TB/s.")
                else:
                    gf = b["useful_gflop"]
                    peak = PEAK_BF16_TFLOPS if "bf16" in desc else PEAK_F32_TFLOPS
                    roof = (f"Useful {gf} GFLOP per call: {gf / med * 1e3:.1f} TFLOP/s at the median "
                            f"dispatch, {gf / med * 1e3 / peak:.3f} of the dense MFMA peak ({peak} TFLOP/s; "
                            f"no clock-settle calls before these dispatches).")
                out += [roof + " The same run's HIP-event pair around each call (which adds the launch "
                        f"latency of a lone call): median {b['us_cold_event_median']} us, mean "
                        f"{b['us_cold_event_mean']} us ({b['launches']} launch(es) per call).", ""]
            open(base + "_cold_kernel_trace.md", "w").write("\n".join(out))
            written.append(base + "_cold_kernel_trace.md")
        if "fetch" in ks and "write" in ks:
            f, cf = counters(ks["fetch"], sym)
            w, cw = counters(ks["write"], sym)
            cfm, cwm = statistics.mean(cf["FETCH_SIZE"]), statistics.mean(cw["WRITE_SIZE"])
            kib = 1024.0 * 1024  # the calibration copy moves 1024 MiB each way
            sf, sw = kib / cfm, kib / cwm
            fk, wk = statistics.mean(f["FETCH_SIZE"]), statistics.mean(w["WRITE_SIZE"])
            rd, wr = fk * 1024 * sf, wk * 1024 * sw
            lines = [f"# HBM traffic of {KERNEL_SYMBOL[key]} per launch: {desc} (rocprofv3 derived counters)",
                     f"command_fetch: {pass_command('fetch', prob)}", f"command_write: {pass_command('write', prob)}",
                     f"summary: {summary_cmd}",
                     f"kernel_source: dnn_conv2d_bwd_amd/csrc/{KERNEL_SRC[key]} + {' + '.join(KERNEL_HEADERS)}",
                     f"source_sha256: {kernel_digest(key)}",
                     f"fetch_size_kib_per_dispatch: {fk:.1f} (dispatches {len(f['FETCH_SIZE'])})",
                     f"write_size_kib_per_dispatch: {wk:.1f} (dispatches {len(w['WRITE_SIZE'])})",
                     f"copy_calibration: plain device copy of 1024 MiB (__amd_rocclr_copyBuffer, the largest-grid "
                     f"copy dispatches only: {len(cf['FETCH_SIZE'])} and {len(cw['WRITE_SIZE'])}); FETCH_SIZE "
                     f"{cfm:.1f} KiB, WRITE_SIZE {cwm:.1f} KiB per dispatch",
                     f"scale_fetch: {sf:.4f}", f"scale_write: {sw:.4f}",
                     f"hbm_read_bytes_per_launch: {rd:.0f}", f"hbm_write_bytes_per_launch: {wr:.0f}",
                     f"hbm_bytes_per_launch: {rd + wr:.0f}", ""]
            open(base + "_traffic.txt", "w").write("\n".join(lines))
            written.append(base + "_traffic.txt")
        for kind, title in (("mfma", "MFMA counters"), ("stall", "wave stall counters")):
            if kind not in ks:
                continue
            c, _ = counters(ks[kind], sym)
            n = len(next(iter(c.values())))
            lines = [f"# {title} of {KERNEL_SYMBOL[key]}: {desc} (rocprofv3 --pmc, mean per dispatch)",
                     f"command: {pass_command(kind, prob)}", f"summary: {summary_cmd}",
                     f"kernel_source: dnn_conv2d_bwd_amd/csrc/{KERNEL_SRC[key]} + {' + '.join(KERNEL_HEADERS)}",
                     f"source_sha256: {kernel_digest(key)}", f"dispatches: {n}"]
            lines += [f"{k}: {statistics.mean(v):.0f}" for k, v in sorted(c.items())]
            m = {k: statistics.mean(v) for k, v in c.items()}
            if kind == "mfma":
                lines += ["", f"executed_bf16_flop: {m['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / 1e9:.4f} G (512 x MOPS)",
                          f"mfma_busy_cycles_per_simd: {m['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024:.0f} (1024 SIMDs)",
                          f"gui_active_cycles_per_xcd: {m['GRBM_GUI_ACTIVE'] / 8:.0f} (8 XCDs)",
                          f"mfma_busy_fraction: {m['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024 / (m['GRBM_GUI_ACTIVE'] / 8):.3f}"]
            else:
                wv = m.get("SQ_WAVES", 1.0)
                q = lambda k: m[k] * 4 / wv  # noqa: E731  (quad-cycle counters -> cycles per wave)
                lines += ["", f"per wave ({wv:.0f} waves; SQ_WAVE_CYCLES, SQ_WAIT_* and SQ_ACTIVE_INST_ANY count "
                              f"4-cycle units):",
                          f"  wave_cycles: {q('SQ_WAVE_CYCLES'):.0f}",
                          f"  wait_any (waitcnt and barrier): {q('SQ_WAIT_ANY'):.0f}",
                          f"  wait_inst_any (instruction ready, not issued): {q('SQ_WAIT_INST_ANY'):.0f}",
                          f"  wait_inst_lds: {q('SQ_WAIT_INST_LDS'):.0f}",
                          f"  active_inst_any: {q('SQ_ACTIVE_INST_ANY'):.0f}",
                          f"  mfma_busy_cycles per SIMD: {m['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024:.0f}"]
            open(base + f"_{kind}_counters.txt", "w").write("\n".join(lines + [""]))
            written.append(base + f"_{kind}_counters.txt")
    for f in written:
        print(os.path.relpath(f, ROOT))


def settle(args, torch, graph, call, stream):
    """Untimed calls for about args.settle_ms of GPU time, issued back to back
    (whole replays of the captured graph, or single calls), ending with a
    synchronisation; returns the number of calls.  The part raises its clock
    over the first few tens of milliseconds of sustained load after an idle
    period (MI355X, headline problem: 60 us per call over the first 200 calls,
    52 us from about 30 ms on), so timed steps taken right after a short
    warmup measure the ramp rather than the sustained rate."""
    if args.settle_ms <= 0:
        return 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    if graph is not None:
        graph.replay()
        per, unit = args.steps, "replay"
    else:
        call()
        per, unit = 1, "call"
    e1.record(stream)
    torch.cuda.synchronize()
    ms = max(e0.elapsed_time(e1), 1e-3)
    n = max(1, min(100000, int(math.ceil(args.settle_ms / ms))))
    for _ in range(n):
        graph.replay() if graph is not None else call()
    torch.cuda.synchronize()
    return (n + 1) * per


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="after the warmup steps, untimed calls for about this much GPU time so "
                         "that the clock reaches its sustained level before the timed steps "
                         "(0 disables; reported in the JSON line)")
    ap.add_argument("--problem", default="c4")
    ap.add_argument("--cpu-seconds", type=float, default=1.0,
                    help="0 skips the CPU baseline; any other value runs the oracle once on the "
                         "whole problem (a few seconds for the headline problem)")
    ap.add_argument("--no-secondary", dest="secondary", action="store_false",
                    help="leave out the graph-mode µs and roofline fractions of the other "
                         "roofline rows (c3a, c3b, c5-s2, c5-s1)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain copy of this size (rocprofv3 counter scaling)")
    ap.add_argument("--force-kernel", type=int, default=-1)
    ap.add_argument("--batch", type=int, default=0,
                    help="override the problem's batch N (e.g. one GPU's share of a "
                         "batch-sharded job)")
    ap.add_argument("--rows-per-wg", type=int, default=0,
                    help="grouped problems: output rows per workgroup of the pipelined row "
                         "kernel (0 automatic, -1 the one-row kernel)")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="time the calls issued one by one on the stream instead of replayed "
                         "from a captured HIP graph")
    ap.add_argument("--ksplit", type=int, default=0,
                    help="large-tile or generic kernel: split each tile's K loop over this many "
                         "workgroups (f32 workspace + finalising kernel); 0 the planner's choice "
                         "(a workspace is passed whenever the plan asks for one), 1 never")
    ap.add_argument("--static-shape", type=int, default=0, choices=(-1, 0, 1),
                    help="large-tile kernel: shape-specialised instance when one matches (0), "
                         "required (1) or never, i.e. the descriptor-driven kernel (-1)")
    ap.add_argument("--per-class", action="store_true",
                    help="one main launch per residue class (ablation of the single launch)")
    ap.add_argument("--cols-per-wg", type=int, default=0,
                    help="grouped MFMA kernel: positions of a row per workgroup (0 automatic)")
    ap.add_argument("--grouped-dot", action="store_true",
                    help="grouped problems: dot-product instructions instead of 4x4x4 MFMA")
    ap.add_argument("--no-split", action="store_true",
                    help="time the zero-insertion form (comparison baseline) instead of the "
                         "residue split")
    ap.add_argument("--grouped-sweep", action="store_true",
                    help="time the ResNeXt-style grouped sweep (32 shapes), one JSON line each")
    ap.add_argument("--all", action="store_true",
                    help="one JSON line per workload problem: warm and cold (caches "
                         "flushed) µs/call and the roofline fraction; not the bench line")
    ap.add_argument("--cold-flush", choices=("read", "write"), default="read",
                    help="--all, --cold-calls: how the 512 MiB sweep before each cold call "
                         "evicts the caches")
    ap.add_argument("--cold-calls", type=int, default=0,
                    help="run only this many calls of --problem, each after a cache sweep "
                         "and alone on the GPU (for a kernel trace of cold dispatches); "
                         "prints their event-pair times, not the bench line")
    ap.add_argument("--summarize-profiles", metavar="RAW", default=None,
                    help="write the profiles/ summaries of the rocprofv3 passes under RAW "
                         "(<pass>_<problem> directories; no GPU needed)")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(backward-data shards by batch with no collective: each GPU would run this "
              f"same launch on its own slice of the batch)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dnn_conv2d_bwd_amd as cbd
    from cbd_inputs import draw, problem_by_name, seed_for

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.all:
        all_problems(args)
        return
    if args.grouped_sweep:
        grouped_sweep(args)
        return
    p = problem_by_name(args.problem)
    if args.batch:
        p = p.with_(n=args.batch)
    dt = cbd.F32 if p.dtype == "f32" else cbd.BF16
    pl = cbd.plan(p.n, p.g, p.c, p.k, p.hi, p.wi, p.y, p.x, (p.sh, p.sw), (p.ph, p.pw),
                  (p.dh, p.dw), p.layout, dt, force_kernel=args.force_kernel,
                  no_split=args.no_split, rows_per_wg=args.rows_per_wg,
                  grouped_dot=args.grouped_dot, cols_per_wg=args.cols_per_wg,
                  ksplit=args.ksplit, per_class=args.per_class,
                  static_shape=args.static_shape)
    info = pl.info()
    sh = pl.shapes()
    dy = draw(p.dist_dy, seed_for(p, "dy"), sh["dy"], p.dtype)
    w = draw(p.dist_w, seed_for(p, "w"), sh["w"], p.dtype)
    tdt = torch.float32 if p.dtype == "f32" else torch.bfloat16
    dy_d = torch.from_numpy(dy).to(tdt).cuda()
    w_d = torch.from_numpy(w).to(tdt).cuda()
    dx_d = torch.empty(sh["dx"], dtype=tdt, device="cuda")
    ws = (torch.empty(pl.workspace_size(), dtype=torch.uint8, device="cuda")
          if pl.workspace_size() else None)
    # with a workspace the plan runs its split configuration, if it has one
    eff_ksplit = info.ksplit if info.ksplit > 1 else (info.auto_ksplit if ws is not None else 1)
    stream = torch.cuda.current_stream()
    if args.cold_calls:
        cold_calls(args, torch, np, cbd, p, info, pl, dy_d, w_d, dx_d, ws, stream)
        return

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib << 20, 5)

    for _ in range(args.warmup):
        cbd.run(pl, dy_d, w_d, dx_d, stream=stream, workspace=ws)
    torch.cuda.synchronize()

    # Timed region: the K calls captured once in a HIP graph and replayed
    # (the calls launch kernels only, so they capture; no host launch cost
    # between steps), or with --no-graph issued one by one on the stream,
    # each between its own event pair.
    graph = None
    timing = "stream"
    if args.graph:
        try:
            graph = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream()
            cap.wait_stream(stream)
            with torch.cuda.stream(cap):
                cbd.run(pl, dy_d, w_d, dx_d, stream=cap, workspace=ws)
                torch.cuda.synchronize()
                with torch.cuda.graph(graph, stream=cap):
                    for _ in range(args.steps):
                        cbd.run(pl, dy_d, w_d, dx_d, stream=cap, workspace=ws)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            timing = f"hip graph of {args.steps} calls"
        except Exception as e:  # capture unsupported here: time on the stream
            graph = None
            timing = f"stream (graph capture failed: {type(e).__name__})"
    torch.cuda.synchronize()
    settle_calls = settle(args, torch, graph, lambda: cbd.run(pl, dy_d, w_d, dx_d, stream=stream, workspace=ws),
                          stream)
    if graph is not None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        launch_s = e0.elapsed_time(e1) / 1e3 / args.steps
    else:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            cbd.run(pl, dy_d, w_d, dx_d, stream=stream, workspace=ws)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        launch_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    step_s = wall / args.steps

    flops = info.useful_flops
    alg_bytes = algorithmic_bytes(p, info)
    if p.name in HBM_BOUND:
        roof = {"bound": "hbm", "achieved": round(alg_bytes / launch_s / 1e9, 2),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        peak = PEAK_BF16_TFLOPS if p.dtype == "bf16" else PEAK_F32_TFLOPS
        roof = {"bound": "mfma", "achieved": round(flops / launch_s / 1e12, 2), "peak": peak,
                "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = read_traffic(kernel_key(info), p.name) if not (args.batch or args.no_split) else None
    roof["kernel"] = KERNEL_SYMBOL[kernel_key(info)]
    roof["launch_us_mean"] = round(launch_s * 1e6, 3)
    roof["launches_per_step"] = info.launches + (eff_ksplit > info.ksplit)

    out = {
        "metric": METRIC,
        "value": round(flops / step_s / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"calls": settle_calls, "target_ms": args.settle_ms},
        "ms_per_step": round(step_s * 1e3, 6),
        "us_per_call": round(step_s * 1e6, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic (seeded SplitMix64 / Box-Muller operands, no dataset)",
        "config": {"workload": describe(p), "problem": p.name,
                   "form": "zero-insertion (no residue split)" if args.no_split else "residue split",
                   "timing": timing,
                   "kernel": cbd.KERNEL_NAMES[info.kernel], "subgemms": info.num_subgemms,
                   "zero_regions": info.num_zero_regions, "grid": info.grid_main,
                   "rows_per_wg": info.rows_per_wg, "cols_per_wg": info.cols_per_wg,
                   "ksplit": eff_ksplit, "launches": info.launches + (eff_ksplit > info.ksplit),
                   "static_shape": info.static_shape,
                   "useful_gflop": round(flops / 1e9, 4),
                   "executed_gmac": round(info.executed_macs / 1e9, 4),
                   "alg_mbytes": round(alg_bytes / 1e6, 3)},
        "roofline": roof,
        "gpu": torch.cuda.get_device_name(0) or "gfx950",
        "machine": machine(),
    }
    if args.secondary:
        out["secondary"] = secondary_rows()
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(p, dy, w, info, dx_gpu=dx_d.float().cpu().numpy())
    print(json.dumps(out), flush=True)


def grouped_sweep(args):
    """Each grouped-sweep shape: 10 warm-up calls, then args.steps calls
    under one event pair (warm: the host's launch rate bounds the small
    shapes) and the same calls replayed from a HIP graph (GPU time only);
    algorithmic bytes per µs against the HBM roofline (every shape has
    arithmetic intensity far below the bf16 ridge)."""
    import torch

    import dnn_conv2d_bwd_amd as cbd
    from cbd_inputs import GROUPED_SWEEP, draw, seed_for

    stream = torch.cuda.current_stream()
    for p in GROUPED_SWEEP:
        pl = cbd.plan(p.n, p.g, p.c, p.k, p.hi, p.wi, p.y, p.x, (p.sh, p.sw), (p.ph, p.pw),
                      (p.dh, p.dw), p.layout, cbd.BF16)
        info = pl.info()
        sh = pl.shapes()
        dy_d = torch.from_numpy(draw(p.dist_dy, seed_for(p, "dy"), sh["dy"], p.dtype)).to(torch.bfloat16).cuda()
        w_d = torch.from_numpy(draw(p.dist_w, seed_for(p, "w"), sh["w"], p.dtype)).to(torch.bfloat16).cuda()
        dx_d = torch.empty(sh["dx"], dtype=torch.bfloat16, device="cuda")
        for _ in range(10):
            cbd.run(pl, dy_d, w_d, dx_d, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            cbd.run(pl, dy_d, w_d, dx_d, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        us_g = graph_us(cbd, torch, pl, dy_d, w_d, dx_d)
        nbytes = algorithmic_bytes(p, info)
        gbs, gbs_g = nbytes / us / 1e3, nbytes / us_g / 1e3
        print(json.dumps({
            "problem": p.name, "workload": describe(p), "kernel": cbd.KERNEL_NAMES[info.kernel],
            "variant": info.variant, "grid": info.grid_main, "us_warm": round(us, 3),
            "us_graph": round(us_g, 3),
            "useful_tflops": round(info.useful_flops / us / 1e6, 3),
            "useful_tflops_graph": round(info.useful_flops / us_g / 1e6, 3),
            "alg_mbytes": round(nbytes / 1e6, 3), "gbs": round(gbs, 1), "gbs_graph": round(gbs_g, 1),
            "roofline": "hbm", "frac": round(gbs / PEAK_HBM_GBS, 4),
            "frac_graph": round(gbs_g / PEAK_HBM_GBS, 4)}), flush=True)
        del dy_d, w_d, dx_d


def cache_sweep(torch, how):
    """A callable that evicts L2 and the MALL with a sweep over a 512 MiB
    buffer: a read sweep (a row-wise max, one output per 8 KiB row, no
    cross-block reduction) leaves the caches clean; a write sweep (a fill
    kernel) leaves dirty lines whose write-back falls into whatever runs next."""
    flush = torch.ones(64 << 20, dtype=torch.float64, device="cuda")  # 512 MiB
    rows = flush.view(65536, 1024)
    rowmax = torch.empty(65536, dtype=torch.float64, device="cuda")

    def evict():
        if how == "write":
            flush.fill_(1.0)
        else:
            torch.amax(rows, dim=1, out=rowmax)
    return evict


def cold_calls(args, torch, np, cbd, p, info, pl, dy_d, w_d, dx_d, ws, stream):
    """Calls each preceded by a cache sweep and followed by a synchronisation:
    every dispatch of the problem's kernels in this run starts with cold
    caches, so a kernel trace of the run gives the kernel's own cold duration
    (without the launch latency that the event pair around a single call
    includes).  Prints one JSON line with the event-pair times."""
    evict = cache_sweep(torch, args.cold_flush)
    us = []
    for _ in range(args.cold_calls):
        evict()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        cbd.run(pl, dy_d, w_d, dx_d, stream=stream, workspace=ws)
        b.record(stream)
        torch.cuda.synchronize()
        us.append(a.elapsed_time(b) * 1e3)
    us = np.array(us)
    print(json.dumps({"problem": p.name, "workload": describe(p), "kernel": KERNEL_SYMBOL[kernel_key(info)],
                      "launches": info.launches, "cold_calls": args.cold_calls,
                      "cold_flush": args.cold_flush + " sweep of 512 MiB",
                      "us_cold_event_median": round(float(np.median(us)), 3),
                      "us_cold_event_mean": round(float(np.mean(us)), 3),
                      "alg_mbytes": round(algorithmic_bytes(p, info) / 1e6, 3),
                      "useful_gflop": round(info.useful_flops / 1e9, 5)}), flush=True)


def all_problems(args):
    """Every workload problem: warm = back-to-back calls under one event pair
    (host launch cost included: small problems are bounded by it); graph = the
    same calls replayed from a captured HIP graph (GPU time only); cold = calls
    each preceded (outside its event pair) by a sweep over a 512 MiB buffer
    that evicts L2 and the MALL: a read sweep by default, which leaves the
    caches clean (a write sweep, --cold-flush write, leaves dirty lines whose
    write-back then falls inside the timed call).  Fractions are of the
    problem's own roofline."""
    import numpy as np
    import torch

    import dnn_conv2d_bwd_amd as cbd
    from cbd_inputs import PROBLEMS, draw, seed_for

    stream = torch.cuda.current_stream()
    evict = cache_sweep(torch, args.cold_flush)
    torch.cuda.synchronize()
    mach = machine()
    for p in PROBLEMS:
        dt = cbd.F32 if p.dtype == "f32" else cbd.BF16
        pl = cbd.plan(p.n, p.g, p.c, p.k, p.hi, p.wi, p.y, p.x, (p.sh, p.sw), (p.ph, p.pw),
                      (p.dh, p.dw), p.layout, dt)
        info = pl.info()
        sh = pl.shapes()
        tdt = torch.float32 if p.dtype == "f32" else torch.bfloat16
        dy_h = draw(p.dist_dy, seed_for(p, "dy"), sh["dy"], p.dtype)
        w_h = draw(p.dist_w, seed_for(p, "w"), sh["w"], p.dtype)
        dy_d = torch.from_numpy(dy_h).to(tdt).cuda()
        w_d = torch.from_numpy(w_h).to(tdt).cuda()
        dx_d = torch.empty(sh["dx"], dtype=tdt, device="cuda")
        for _ in range(10):
            cbd.run(pl, dy_d, w_d, dx_d, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            cbd.run(pl, dy_d, w_d, dx_d, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        warm = e0.elapsed_time(e1) * 1e3 / args.steps
        cold = []
        for _ in range(50):
            evict()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            cbd.run(pl, dy_d, w_d, dx_d, stream=stream)
            b.record(stream)
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b) * 1e3)
        cold = np.array(cold)
        # GPU time without host launch cost: calls captured in a HIP graph
        # (the calls launch kernels only: no allocation, copy or memset).
        us_graph = graph_us(cbd, torch, pl, dy_d, w_d, dx_d)
        # the descriptor-driven kernel of the same plan (static_shape=-1), for
        # the shape-specialised instances' comparison
        us_dyn = None
        if info.static_shape:
            pd = cbd.plan(p.n, p.g, p.c, p.k, p.hi, p.wi, p.y, p.x, (p.sh, p.sw), (p.ph, p.pw),
                          (p.dh, p.dw), p.layout, dt, static_shape=-1)
            for _ in range(10):
                cbd.run(pd, dy_d, w_d, dx_d, stream=stream)
            us_dyn = graph_us(cbd, torch, pd, dy_d, w_d, dx_d)
        flops, nbytes = info.useful_flops, algorithmic_bytes(p, info)
        if p.name in HBM_BOUND:
            bound, peak, unit = "hbm", PEAK_HBM_GBS, "GB/s"
            ach = lambda us: nbytes / us / 1e3
        else:
            bound = "mfma"
            peak = PEAK_BF16_TFLOPS if p.dtype == "bf16" else PEAK_F32_TFLOPS
            unit = "TFLOP/s"
            ach = lambda us: flops / us / 1e6
        med = float(np.median(cold))
        line = {
            "problem": p.name, "workload": describe(p), "dtype": p.dtype,
            "layout": "NCHW/KCYX" if p.layout == 0 else "NHWC/KYXC",
            "shape": {"dx": list(sh["dx"]), "dy": list(sh["dy"]), "w": list(sh["w"])},
            "seed": {"dy": seed_for(p, "dy"), "w": seed_for(p, "w")},
            "kernel": KERNEL_SYMBOL[kernel_key(info)],
            "launches": info.launches, "grid": info.grid_main,
            "useful_gflop": round(flops / 1e9, 5), "executed_gmac": round(info.executed_macs / 1e9, 5),
            "alg_mbytes": round(nbytes / 1e6, 3),
            "static_shape": info.static_shape,
            "us_graph_descriptor_driven": round(us_dyn, 2) if us_dyn is not None else None,
            "us_warm": round(warm, 2), "us_graph": round(us_graph, 2),
            "us_cold_median": round(med, 2), "cold_flush": args.cold_flush + " sweep of 512 MiB",
            "us_cold_p10": round(float(np.percentile(cold, 10)), 2),
            "us_cold_p90": round(float(np.percentile(cold, 90)), 2),
            "bound": bound + (" (launch latency in practice)" if p.name in LATENCY_BOUND else ""),
            "achieved_warm": round(ach(warm), 2), "achieved_graph": round(ach(us_graph), 2),
            "achieved_cold": round(ach(med), 2), "unit": unit, "peak": peak,
            "frac_warm": round(ach(warm) / peak, 4), "frac_graph": round(ach(us_graph) / peak, 4),
            "frac_cold": round(ach(med) / peak, 4)}
        if args.cpu_seconds > 0:
            # The oracle on the whole problem, and the GPU result's parity.
            cb = cpu_baseline(p, dy_h, w_h, info, dx_gpu=dx_d.float().cpu().numpy())
            line.update({"oracle_s": cb["oracle_s"], "oracle_threads": cb["cores"],
                         "oracle_tflops": cb["value"], "oracle_sample": cb["sample"],
                         "parity": cb["parity"]})
        line.update(mach)
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
