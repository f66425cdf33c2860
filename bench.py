"""Benchmark: causal attention forward + backward TFLOP/s (fp16 inputs, fp32
accumulation, head width 64) on one MI355X, and the fraction of the fp16
dense MFMA peak.

One step is one pass of the whole path over one batch of synthetic input:
forward (sa_forward_ex), then the backward's row terms, key pass and dQ pass
(the three launches of sa_backward_ex, issued one by one so each can be timed).
Inputs are resident in HBM before the timed region starts.

FLOPs are algorithmic: per admitted (query, key) pair and query head, the
forward's two products cost 4 * 64 and the backward's five cost 10 * 64; a
causal square counts T^2 / 2 pairs.

Prints ONE JSON line.  With --gpus above 1 it exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal attn fwd+bwd TFLOP/s (fp16, d=64) and % of MFMA fp16 peak"
# MI355X dense fp16 MFMA: 256 CUs x 2.4 GHz x 4096 FLOP/clock/CU (the published 2.5 PFLOP/s).
PEAK_TFLOPS = 256 * 2.4e9 * 4096 / 1e12
HBM_PEAK_GBS = 8000.0
HEAD_DIM = 64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
HEADLINE_WORKLOAD = "causal_gqa_t4096"
KERNEL_SOURCES = [os.path.join(ROOT, "causal_streaming_attention_amd", "csrc", f)
                  for f in ("sa_device.h", "sa_forward.hip", "sa_backward.hip", "sa_query.hip")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def pairs_per_head(w, seqlens):
    """Admitted (query, key) pairs per query head, summed over the batch."""
    if seqlens is not None:
        sq = float(np.sum(np.asarray(seqlens, dtype=np.float64) ** 2))
        return sq * (0.5 if w.causal else 1.0)
    return w.batch * float(w.T) * w.T * (0.5 if w.causal else 1.0)


def kernel_flops(w, seqlens):
    p = pairs_per_head(w, seqlens) * w.heads
    return {"forward": 4 * HEAD_DIM * p, "key_pass": 8 * HEAD_DIM * p, "dq_pass": 2 * HEAD_DIM * p,
            "row_terms": 0.0, "total": 14 * HEAD_DIM * p}


def row_terms_bytes(w):
    rows = w.batch * w.heads * w.T
    return rows * (HEAD_DIM * 2 * 2 + 4)   # dO and O fp16 rows in, D fp32 out


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters for this kernel source, else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash() or t.get("workload") != workload:
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def device_info():
    """The denominator's inputs as the device reports them: CU count and name from the runtime, the
    maximum shader clock from rocminfo (a child process), or None where unavailable."""
    import subprocess
    import torch
    info = {"peak_denominator": "256 CUs x 2.4 GHz x 4096 fp16 FLOP/clk/CU = %.1f TFLOP/s" % PEAK_TFLOPS}
    try:
        p = torch.cuda.get_device_properties(0)
        info.update({"name": p.name, "arch": getattr(p, "gcnArchName", None), "cu_count": p.multi_processor_count})
    except (RuntimeError, AssertionError):
        pass
    try:
        r = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30)
        gpu = r.stdout.split("gfx950", 1)
        if len(gpu) == 2:
            for line in gpu[1].splitlines():
                if "Max Clock Freq" in line:
                    info["max_clock_mhz"] = int("".join(ch for ch in line.split(":", 1)[1] if ch.isdigit()))
                    break
    except (OSError, ValueError, subprocess.SubprocessError):
        pass
    return info


def gpu_state():
    """Shader/memory clocks and package power from rocm-smi (a child process), or None."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"], capture_output=True, text=True,
                           timeout=20)
        d = json.loads(r.stdout)
    except (OSError, ValueError, subprocess.SubprocessError):
        return None
    out = {}
    for card, fields in d.items():
        if isinstance(fields, dict):
            out[card] = {k: v for k, v in fields.items()
                         if any(t in k.lower() for t in ("sclk", "mclk", "power"))}
    return out or None


def cpu_baseline(w, x, budget_s: float = 10.0):
    """Time the binary64 oracle on the same inputs, one K/V head group (its G query
    heads of one sequence, the whole forward and backward) at a time, until about
    `budget_s` seconds of CPU work are done or every group has run; reported in the
    workload's FLOP convention."""
    import oracle
    from causal_streaming_attention_amd.workloads import SCALE
    G = w.heads // w.kv_heads
    groups = [(b, kv) for b in range(w.batch) for kv in range(w.kv_heads)]
    flops, dt, done = 0.0, 0.0, 0
    for b, kv in groups:
        sl = None if x["seqlens"] is None else x["seqlens"][b:b + 1]
        t0 = time.perf_counter()
        oracle.backward(x["Q"][b:b + 1, kv * G:(kv + 1) * G], x["K"][b:b + 1, kv:kv + 1],
                        x["Vt"][b:b + 1, kv:kv + 1], x["dO"][b:b + 1, kv * G:(kv + 1) * G],
                        s=SCALE, causal=w.causal, seqlens=sl)
        dt += time.perf_counter() - t0
        n = w.T if sl is None else int(sl[0])
        flops += 14 * HEAD_DIM * (n * float(n) * (0.5 if w.causal else 1.0)) * G
        done += 1
        if dt >= budget_s:
            break
    what = "the whole job" if done == len(groups) else f"{done} of {len(groups)} groups"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{what} of {w.name} (K/V head groups of {G} query heads, batch row by batch row): "
                      f"full forward and backward, {flops / 1e9:.2f} GFLOP in {dt:.1f} s",
            "cpu": _cpu_model() if _cpu_model() != "unknown" else platform.processor(), "nproc": os.cpu_count()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


KERNEL_NAMES = {"forward": "sa_forward_kernel", "row_terms": "sa_row_terms_kernel", "key_pass": "sa_key_kernel",
                "dq_pass": "sa_dq_kernel"}


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(dirpath, suffix):
    for root, _, files in os.walk(dirpath):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {dirpath}")


def summarize_profile(dirs, workload, command):
    """Write profiles/kernel_trace_<workload>.txt from a --kernel-trace --stats run and, given the
    FETCH_SIZE and WRITE_SIZE pass directories of a --calibrate-copy-mb run, profiles/traffic.json
    and profiles/hbm_traffic_<workload>.txt.  Counter bytes are scaled by what the same counter
    reads for the closing device copy, whose bytes are known."""
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    import re
    trace_dir = dirs[0]
    stats = _read_csv(_find(trace_dir, "kernel_stats.csv"))
    # The bench's per-kernel figures average the last K launches (its second timed pass); the
    # stats' average also holds the warm-up launches, which start on a low clock.
    m = re.search(r"bench\.py --steps (\d+)", command)
    last_k = int(m.group(1)) if m else 0
    per_dispatch = {}
    if last_k:
        try:
            rows = _read_csv(_find(trace_dir, "kernel_trace.csv"))
        except FileNotFoundError:
            rows = []
        for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
            for short, key in KERNEL_NAMES.items():
                if key in r["Kernel_Name"]:
                    per_dispatch.setdefault(short, []).append(
                        (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"# rocprofv3 kernel trace, workload {workload}", f"# command: {command}"]
    if per_dispatch:
        lines.append(f"# last{last_k}_us: average over each kernel's last {last_k} launches (the timed steps the "
                     "bench's per-kernel figures average); avg_us includes the warm-up launches")
    lines += ["", f"{'kernel':<12} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10}"
              + (f" {'last' + str(last_k) + '_us':>10}" if per_dispatch else "")]
    for short, key in KERNEL_NAMES.items():
        for r in stats:
            if key in r["Name"]:
                line = (f"{short:<12} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
                        f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f}")
                if per_dispatch.get(short):
                    tail = per_dispatch[short][-last_k:]
                    line += f" {sum(tail) / len(tail):>10.2f}"
                lines.append(line)
    with open(os.path.join(ROOT, "profiles", f"kernel_trace_{workload}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    if len(dirs) < 3:
        return
    per = {}
    for label, d in (("FETCH_SIZE", dirs[1]), ("WRITE_SIZE", dirs[2])):
        rows = [r for r in _read_csv(_find(d, "counter_collection.csv")) if r["Counter_Name"] == label]
        last = max(rows, key=lambda r: int(r["Dispatch_Id"]))          # the calibration copy
        copy_kib = float(last["Counter_Value"])
        per[label] = {"copy_kib": copy_kib, "kernels": {}}
        for short, key in KERNEL_NAMES.items():
            vals = [float(r["Counter_Value"]) for r in rows if key in r["Kernel_Name"]]
            if vals:
                per[label]["kernels"][short] = sum(vals) / len(vals)
    m = re.search(r"--calibrate-copy-mb[= ](\d+)", command)
    copy_bytes = int(m.group(1)) << 20 if m else None
    if copy_bytes is None:
        raise ValueError("--profile-command must name --calibrate-copy-mb=N")
    fr = copy_bytes / (per["FETCH_SIZE"]["copy_kib"] * 1024)
    fw = copy_bytes / (per["WRITE_SIZE"]["copy_kib"] * 1024)
    traffic = {"workload": workload, "source_hash": kernel_source_hash(), "command": command,
               "copy_bytes": copy_bytes, "fetch_scale": fr, "write_scale": fw, "kernels": {}}
    lines = [f"# rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE (KiB per dispatch), workload {workload}",
             f"# command: {command}",
             f"# scale: a {copy_bytes >> 20} MiB device copy reads FETCH_SIZE {per['FETCH_SIZE']['copy_kib']:.0f} KiB "
             f"and WRITE_SIZE {per['WRITE_SIZE']['copy_kib']:.0f} KiB: read x{fr:.3f}, write x{fw:.3f}", "",
             f"{'kernel':<12} {'FETCH_KiB':>12} {'WRITE_KiB':>12} {'read_MB':>10} {'write_MB':>10}"]
    for short in KERNEL_NAMES:
        fk = per["FETCH_SIZE"]["kernels"].get(short)
        wk = per["WRITE_SIZE"]["kernels"].get(short)
        if fk is None or wk is None:
            continue
        rb, wb = fk * 1024 * fr, wk * 1024 * fw
        traffic["kernels"][short] = {"read_bytes": rb, "write_bytes": wb, "hbm_bytes_per_launch": rb + wb}
        lines.append(f"{short:<12} {fk:>12.0f} {wk:>12.0f} {rb / 1e6:>10.1f} {wb / 1e6:>10.1f}")
    with open(os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if workload == HEADLINE_WORKLOAD:   # the bench line's roofline reads the headline workload's bytes
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(traffic, f, indent=1)
    print("\n".join(lines))


def summarize_all_kernels(d, workload, command):
    """Write profiles/kernel_trace_all_paths_<workload>.txt: every kernel instantiation of a full bench run
    (the headline and the variants timed beside it), by name with its template arguments."""
    import re
    stats = [r for r in _read_csv(_find(d, "kernel_stats.csv")) if "sa_" in r["Name"]]
    lines = [f"# rocprofv3 kernel trace of the full bench (every path), workload {workload}", f"# command: {command}",
             "# template arguments: forward / query <causal, varlen, V as rows>; key <causal, varlen, waves pairs "
             "per group>; dq <causal, varlen, epilogue: 0 plain, 1 rotated, 2 projection>; the key pass's dS store, "
             "V rows and projection stores are run-time choices within one instantiation", "",
             f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10}  kernel"]
    def readable(mangled):
        # sa::<anon>::<name><literal template arguments>: a length-prefixed name, then L<b|i><value>E items
        m = re.match(r"_ZN2sa12_GLOBAL__N_1(\d+)", mangled)
        if not m:
            return mangled
        n = int(m.group(1))
        name = mangled[m.end():m.end() + n]
        args = re.findall(r"L([bi])(\d+)E", mangled[m.end() + n:].split("EEv")[0] + "E")
        vals = [("true" if v == "1" else "false") if t == "b" else v for t, v in args]
        return f"{name}<{', '.join(vals)}>"

    for r, name in sorted(((r, readable(r["Name"])) for r in stats), key=lambda t: t[1]):
        lines.append(f"{int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} {float(r['MinNs']) / 1e3:>10.2f} "
                     f"{float(r['MaxNs']) / 1e3:>10.2f}  {name}")
    with open(os.path.join(ROOT, "profiles", f"kernel_trace_all_paths_{workload}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


SQ_COUNTERS = ["SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
               "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"]


def summarize_counters(d, workload, command):
    """Write profiles/sq_counters_<workload>.txt from one rocprofv3 --pmc run of SQ_COUNTERS:
    per-dispatch averages for each kernel, and the derived per-wave instruction mix and
    the share of LDS-active cycles lost to bank conflicts."""
    rows = _read_csv(_find(d, "counter_collection.csv"))
    lines = [f"# rocprofv3 --pmc {' '.join(SQ_COUNTERS)} (per-dispatch averages), workload {workload}",
             f"# command: {command}", ""]
    for short, key in KERNEL_NAMES.items():
        vals = {}
        for r in rows:
            if key in r["Kernel_Name"]:
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        if not vals:
            continue
        avg = {k: sum(v) / len(v) for k, v in vals.items()}
        lines.append(f"{short}:")
        for k in SQ_COUNTERS:
            if k in avg:
                lines.append(f"  {k:28s} {avg[k]:16.6g}")
        waves = avg.get("SQ_WAVES", 0.0)
        if waves > 0:
            lines.append(f"  per wave: MFMA {avg.get('SQ_INSTS_MFMA', 0) / waves:.1f}, "
                         f"VALU {avg.get('SQ_INSTS_VALU', 0) / waves:.1f}, LDS {avg.get('SQ_INSTS_LDS', 0) / waves:.1f}")
        if avg.get("SQ_LDS_IDX_ACTIVE", 0) > 0:
            lines.append(f"  LDS bank-conflict cycles / LDS-active cycles: "
                         f"{avg.get('SQ_LDS_BANK_CONFLICT', 0) / avg['SQ_LDS_IDX_ACTIVE']:.3f}")
        lines.append("")
    with open(os.path.join(ROOT, "profiles", f"sq_counters_{workload}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def clock_settle(seconds: float):
    """Keep the GPU busy with plain fp16 matrix products for about `seconds` before the warm-up.

    An idle MI355X sits at a low shader clock and ramps up over tens of milliseconds of load, so a short
    warm-up leaves the timed steps on a rising clock (a cold step then runs faster than the headline).
    This load is not the attention step and is not timed."""
    import torch
    a = torch.randn(4096, 4096, dtype=torch.float16, device="cuda")
    b = torch.randn(4096, 4096, dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            a = torch.matmul(a, b) * 1e-3
        torch.cuda.synchronize()
        n += 8
    return {"seconds": round(time.perf_counter() - t0, 3), "fp16_gemms_4096": n,
            "note": "GPU held busy before the warm-up so the timed steps start at the loaded clock; not timed"}


def time_workload(name: str, steps: int, warmup: int, block_order: int = 0):
    """One workload's fwd+bwd step (the headline's four launches), timed like the headline: `warmup` steps,
    then `steps` steps between one pair of events, then the same with events between the launches."""
    import torch
    import causal_streaming_attention_amd as sa
    from causal_streaming_attention_amd.workloads import SCALE, WORKLOADS, generate
    w = WORKLOADS[name]
    x = generate(w)
    buf = sa.Buffers(x, w.causal, block_order=block_order)
    c = sa.base2_scale(SCALE)
    sh = buf.shape
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev: ev[0].record(stream)
        sa.sa_forward_ex(sh, buf.Q, buf.K, buf.Vt, buf.O, buf.L, c, stream)
        if ev: ev[1].record(stream)
        sa.sa_row_terms(sh, buf.dO, buf.O, buf.D, stream)
        if ev: ev[2].record(stream)
        sa.sa_key_pass(sh, buf.Q, buf.K, buf.Vt, buf.dO, buf.L, buf.D, buf.dS, buf.ws_bytes, c, SCALE, buf.dK,
                       buf.dVt, stream)
        if ev: ev[3].record(stream)
        sa.sa_dq_pass(sh, buf.K, buf.dS, buf.ws_bytes, SCALE, buf.dQ, stream)
        if ev: ev[4].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    ms = max(a.elapsed_time(b) / steps, (time.perf_counter() - t0) * 1e3 / steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    names = ["forward", "row_terms", "key_pass", "dq_pass"]
    per = {n: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(steps)]))
           for i, n in enumerate(names)}
    fl = kernel_flops(w, x["seqlens"])
    tf = fl["total"] / (ms * 1e-3) / 1e12
    out = {"ms_per_step": round(ms, 4), "tflops": round(tf, 2), "pct_mfma_peak": round(100 * tf / PEAK_TFLOPS, 2),
           "flops_per_step": fl["total"], "steps": steps, "warmup": warmup,
           "shape": {"batch": w.batch, "T": w.T, "heads": w.heads, "kv_heads": w.kv_heads, "causal": w.causal,
                     "varlen": w.varlen},
           "kernels_ms": {n: round(per[n], 4) for n in names},
           "kernels_tflops": {n: round(fl[n] / (per[n] * 1e-3) / 1e12, 1) for n in names if fl[n] > 0}}
    del buf
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=150,
                    help="untimed steps first; the shader clock ramps up over the first ~60 steps (~30 ms)")
    ap.add_argument("--workload", default=HEADLINE_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--block-order", type=int, default=0)
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the two-launch backward and the V-as-rows run timed beside the headline path "
                         "(profiles then see only the headline's kernels)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="after the timed steps, run one device copy of this many MiB (the reference dispatch "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize-profile", nargs="+", metavar="DIR",
                    help="summarize rocprofv3 output directories (kernel trace, then FETCH_SIZE and WRITE_SIZE "
                         "passes of a --calibrate-copy-mb run) into profiles/ and exit")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="summarize one rocprofv3 --pmc run of the SQ counters into profiles/ and exit")
    ap.add_argument("--summarize-all-kernels", metavar="DIR",
                    help="summarize a rocprofv3 --kernel-trace --stats run of the full bench (every path) into "
                         "profiles/ and exit")
    ap.add_argument("--profile-command", default="", help="command line recorded in the summaries")
    ap.add_argument("--clock-settle-s", type=float, default=0.5,
                    help="seconds of plain fp16 GEMM load before the warm-up so the timed steps start at the "
                         "loaded clock (0: none)")
    ap.add_argument("--chunk-mib", type=int, nargs="*", default=[128, 256],
                    help="workspace sizes (MiB) at which the chunked split backward is timed beside the headline")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip timing the other four workloads beside the headline")
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile, args.workload, args.profile_command)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload, args.profile_command)
        return
    if args.summarize_all_kernels:
        summarize_all_kernels(args.summarize_all_kernels, args.workload, args.profile_command)
        return
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(the sharding plan is design only)", file=sys.stderr)
        sys.exit(2)

    import torch
    import causal_streaming_attention_amd as sa
    from causal_streaming_attention_amd.workloads import SCALE, WORKLOADS, generate

    w = WORKLOADS[args.workload]
    x = generate(w)
    buf = sa.Buffers(x, w.causal, block_order=args.block_order)
    c = sa.base2_scale(SCALE)
    sh = buf.shape
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev: ev[0].record(stream)
        sa.sa_forward_ex(sh, buf.Q, buf.K, buf.Vt, buf.O, buf.L, c, stream)
        if ev: ev[1].record(stream)
        sa.sa_row_terms(sh, buf.dO, buf.O, buf.D, stream)
        if ev: ev[2].record(stream)
        sa.sa_key_pass(sh, buf.Q, buf.K, buf.Vt, buf.dO, buf.L, buf.D, buf.dS, buf.ws_bytes, c, SCALE, buf.dK,
                       buf.dVt, stream)
        if ev: ev[3].record(stream)
        sa.sa_dq_pass(sh, buf.K, buf.dS, buf.ws_bytes, SCALE, buf.dQ, stream)
        if ev: ev[4].record(stream)

    def timed(step_fn, n_kernels):
        """K steps between one pair of events (the step time: max of the events' and the host's clock), then
        K more steps with an event between launches for the per-kernel averages.  Events between the
        launches cost the step about 10 us, so the step time is taken without them."""
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        for _ in range(args.steps):
            step_fn()
        b.record(stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        step_ms = max(a.elapsed_time(b) / args.steps, wall_ms)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_kernels + 1)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for k in range(args.steps):
            step_fn(evs[k])
        torch.cuda.synchronize()
        per_k = [float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)]))
                 for i in range(n_kernels)]
        with_events = float(np.mean([evs[k][0].elapsed_time(evs[k][n_kernels]) for k in range(args.steps)]))
        return step_ms, per_k, with_events

    # The clock snapshot (a child process, during which the GPU idles and its clock drops) is taken before
    # the warm-up, so that the timed steps follow the warm-up directly.
    state_before = None if args.headline_only else gpu_state()
    settle = clock_settle(args.clock_settle_s) if args.clock_settle_s > 0 else None
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    names = ["forward", "row_terms", "key_pass", "dq_pass"]
    ms_per_step, per_list, step_with_events = timed(step, len(names))
    per = dict(zip(names, per_list))
    fl = kernel_flops(w, x["seqlens"])
    value = fl["total"] / (ms_per_step * 1e-3) / 1e12
    state_after = None if args.headline_only else gpu_state()
    bwd_ms = per["row_terms"] + per["key_pass"] + per["dq_pass"]
    phases = {"step_ms_with_kernel_events": round(step_with_events, 4),
              "forward_ms": round(per["forward"], 4), "backward_ms": round(bwd_ms, 4),
              "forward_tflops": round(fl["forward"] / (per["forward"] * 1e-3) / 1e12, 1),
              "backward_tflops": round((fl["key_pass"] + fl["dq_pass"]) / (bwd_ms * 1e-3) / 1e12, 1)}

    # Cold steps: a 512 MiB scratch write between steps (outside the timed
    # region) evicts the caches before each one.
    cold = None
    if not args.headline_only:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        cold_ms = []
        for _ in range(min(args.steps, 5)):
            scratch.fill_(1)
            torch.cuda.synchronize()
            ev[0].record(stream)
            step()
            ev[1].record(stream)
            torch.cuda.synchronize()
            cold_ms.append(ev[0].elapsed_time(ev[1]))
        del scratch
        cms = float(np.median(cold_ms))
        cold = {"ms_per_step": round(cms, 4), "tflops": round(fl["total"] / (cms * 1e-3) / 1e12, 2),
                "steps": len(cold_ms), "note": "median; 512 MiB scratch write before each step, host-synchronised"}

    dominant = max(("forward", "key_pass", "dq_pass"), key=lambda n: per[n])
    achieved = fl[dominant] / (per[dominant] * 1e-3) / 1e12
    traffic = load_traffic(dominant, w.name)
    roofline = {"bound": "mfma", "kernel": dominant, "achieved": round(achieved, 2), "peak": round(PEAK_TFLOPS, 1),
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": traffic,
                "algorithmic_flops_per_launch": fl[dominant], "avg_launch_ms": round(per[dominant], 4)}

    kernels = {}
    for n in names:
        e = {"ms": round(per[n], 4)}
        if fl[n] > 0:
            e["tflops"] = round(fl[n] / (per[n] * 1e-3) / 1e12, 1)
            e["frac_mfma_peak"] = round(fl[n] / (per[n] * 1e-3) / 1e12 / PEAK_TFLOPS, 4)
        else:
            gbs = row_terms_bytes(w) / (per[n] * 1e-3) / 1e9
            e["gb_per_s"] = round(gbs, 1)
            e["frac_hbm_peak"] = round(gbs / HBM_PEAK_GBS, 4)
        kernels[n] = e

    # The two-launch backward (query pass for D and dQ, key pass storing no
    # dS), timed the same way beside the three-launch path.
    def step2(ev=None):
        if ev: ev[0].record(stream)
        sa.sa_forward_ex(sh, buf.Q, buf.K, buf.Vt, buf.O, buf.L, c, stream)
        if ev: ev[1].record(stream)
        sa.sa_query_pass(sh, buf.dO, buf.O, buf.L, buf.Q, buf.K, buf.Vt, c, SCALE, buf.D, buf.dQ, stream)
        if ev: ev[2].record(stream)
        sa.sa_key_pass(sh, buf.Q, buf.K, buf.Vt, buf.dO, buf.L, buf.D, None, 0, c, SCALE, buf.dK, buf.dVt,
                       stream)
        if ev: ev[3].record(stream)

    two_pass = v_rows = None
    if not args.headline_only:
        for _ in range(args.warmup):
            step2()
        names2 = ["forward", "query_pass", "key_pass_no_ds"]
        step2_ms, per2_list, _ = timed(step2, len(names2))
        per2 = dict(zip(names2, per2_list))
        two_pass = {"ms_per_step": round(step2_ms, 4),
                    "tflops": round(fl["total"] / (step2_ms * 1e-3) / 1e12, 2),
                    "kernels_ms": {n: round(per2[n], 4) for n in names2},
                    "note": "same workload and FLOP convention; the backward recomputes S, P, dP in both passes "
                            "and stores no dS"}

        # The headline path with V passed as rows [KV][T][64] (and dV returned so).
        bufr = sa.Buffers(x, w.causal, block_order=args.block_order, v_rows=True)
        shr = bufr.shape

        def step3(ev=None):
            if ev: ev[0].record(stream)
            sa.sa_forward_ex(shr, bufr.Q, bufr.K, bufr.Vt, bufr.O, bufr.L, c, stream)
            if ev: ev[1].record(stream)
            sa.sa_row_terms(shr, bufr.dO, bufr.O, bufr.D, stream)
            if ev: ev[2].record(stream)
            sa.sa_key_pass(shr, bufr.Q, bufr.K, bufr.Vt, bufr.dO, bufr.L, bufr.D, bufr.dS, bufr.ws_bytes, c, SCALE,
                           bufr.dK, bufr.dVt, stream)
            if ev: ev[3].record(stream)
            sa.sa_dq_pass(shr, bufr.K, bufr.dS, bufr.ws_bytes, SCALE, bufr.dQ, stream)
            if ev: ev[4].record(stream)

        for _ in range(args.warmup):
            step3()
        step3_ms, per3_list, _ = timed(step3, len(names))
        per3 = dict(zip(names, per3_list))
        v_rows = {"ms_per_step": round(step3_ms, 4),
                  "tflops": round(fl["total"] / (step3_ms * 1e-3) / 1e12, 2),
                  "kernels_ms": {n: round(per3[n], 4) for n in names},
                  "note": "the same step with V as rows [KV][T][64] (no transposed copy of V) and dV returned "
                          "as rows; bitwise-identical outputs"}

    # The dQ pass with the rotated epilogue (dQ turned back by the inverse
    # half-split rotation into a bfloat16 [T][width] projection gradient), on
    # the headline's stored dS, timed alone beside the plain dQ pass.
    dq_rotated = None
    if not args.headline_only:
        width = (w.heads + 2 * w.kv_heads) * HEAD_DIM
        theta = torch.rand(w.T, 32, device="cuda", dtype=torch.float32) * 6.2831855
        cos_t, sin_t = torch.cos(theta).contiguous(), torch.sin(theta).contiguous()
        dqkv = torch.zeros(w.batch, w.T, width, dtype=torch.int16, device="cuda")
        rot_args = (sh, buf.K, buf.dS, buf.ws_bytes, SCALE, cos_t, sin_t, dqkv, width, stream)
        for _ in range(args.warmup):
            sa.sa_dq_pass_rotated(*rot_args)
        ra, rb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ra.record(stream)
        for _ in range(args.steps):
            sa.sa_dq_pass_rotated(*rot_args)
        rb.record(stream)
        torch.cuda.synchronize()
        rot_ms = ra.elapsed_time(rb) / args.steps
        dq_rotated = {"ms": round(rot_ms, 4), "tflops": round(fl["dq_pass"] / (rot_ms * 1e-3) / 1e12, 1),
                      "projection_width": width,
                      "note": "sa_dq_pass_rotated alone, back to back: dQ turned back by the inverse half-split "
                              "rotation and stored as the bfloat16 Q slice of a token-major [T][width] gradient"}

    # The backward storing dQ, dK, dV straight into a fused QKV projection's
    # token-major gradient (binary32 and bfloat16), timed like the headline's
    # backward on the same inputs.
    projection = None
    if not args.headline_only:
        pw = (w.heads + 2 * w.kv_heads) * HEAD_DIM
        g32 = torch.zeros(w.batch, w.T, pw, dtype=torch.float32, device="cuda")
        g16 = torch.zeros(w.batch, w.T, pw, dtype=torch.int16, device="cuda")
        qc, kc, vc = 0, HEAD_DIM * w.heads, HEAD_DIM * (w.heads + w.kv_heads)
        p32, p16 = g32.data_ptr(), g16.data_ptr()

        def step_proj(ev=None):
            if ev: ev[0].record(stream)
            sa.sa_forward_ex(sh, buf.Q, buf.K, buf.Vt, buf.O, buf.L, c, stream)
            if ev: ev[1].record(stream)
            sa.sa_backward_projection(sh, buf.dO, buf.O, buf.L, buf.D, buf.dS, buf.ws_bytes, buf.Q, buf.K, buf.Vt,
                                      c, SCALE, p32 + 4 * qc, p16 + 2 * qc, p32 + 4 * kc, p16 + 2 * kc,
                                      p32 + 4 * vc, p16 + 2 * vc, pw, stream)
            if ev: ev[2].record(stream)

        for _ in range(args.warmup):
            step_proj()
        proj_ms, proj_per, _ = timed(step_proj, 2)
        projection = {"ms_per_step": round(proj_ms, 4), "tflops": round(fl["total"] / (proj_ms * 1e-3) / 1e12, 2),
                      "backward_ms": round(proj_per[1], 4), "projection_width": pw,
                      "note": "the headline step with sa_backward_projection: dQ, dK, dV written token-major into "
                              "a fused QKV projection's gradient, binary32 and bfloat16"}

        def step_proj2(ev=None):
            if ev: ev[0].record(stream)
            sa.sa_forward_ex(sh, buf.Q, buf.K, buf.Vt, buf.O, buf.L, c, stream)
            if ev: ev[1].record(stream)
            sa.sa_backward_two_pass_projection(sh, buf.dO, buf.O, buf.L, buf.D, buf.Q, buf.K, buf.Vt, c, SCALE,
                                               p32 + 4 * qc, p16 + 2 * qc, p32 + 4 * kc, p16 + 2 * kc,
                                               p32 + 4 * vc, p16 + 2 * vc, pw, stream)
            if ev: ev[2].record(stream)

        for _ in range(args.warmup):
            step_proj2()
        p2_ms, p2_per, _ = timed(step_proj2, 2)
        projection["two_pass"] = {"ms_per_step": round(p2_ms, 4),
                                  "tflops": round(fl["total"] / (p2_ms * 1e-3) / 1e12, 2),
                                  "backward_ms": round(p2_per[1], 4)}

    # The chunked split backward (sa_backward_chunked): the key and dQ passes
    # in query-row chunks over a workspace of a few sizes, so that one chunk's
    # dS at a time is written and read back, timed like the headline.
    chunked = None
    if not args.headline_only:
        chunked = {}
        for mib in args.chunk_mib:
            ws_bytes = mib << 20
            if ws_bytes < sa.sa_backward_chunked_min_bytes(sh):
                continue
            ws_bytes = min(ws_bytes, buf.ws_bytes)

            def step_chunked(ev=None, ws_bytes=ws_bytes):
                if ev: ev[0].record(stream)
                sa.sa_forward_ex(sh, buf.Q, buf.K, buf.Vt, buf.O, buf.L, c, stream)
                if ev: ev[1].record(stream)
                sa.sa_backward_chunked(sh, buf.dO, buf.O, buf.L, buf.D, buf.dS, ws_bytes, buf.Q, buf.K, buf.Vt, c,
                                       SCALE, buf.dQ, buf.dK, buf.dVt, stream)
                if ev: ev[2].record(stream)

            for _ in range(args.warmup):
                step_chunked()
            ch_ms, ch_per, _ = timed(step_chunked, 2)
            chunked[f"{mib}MiB"] = {"ms_per_step": round(ch_ms, 4),
                                    "tflops": round(fl["total"] / (ch_ms * 1e-3) / 1e12, 2),
                                    "backward_ms": round(ch_per[1], 4), "workspace_bytes": ws_bytes}

    # Every other workload of the path, timed the same way (the headline's
    # launches, its step count, and at least as many warm-up steps as the
    # headline's), each on its own buffers, freed afterwards.
    others = None
    if not args.headline_only and not args.no_other_workloads:
        others = {}
        for name in ("tiny_causal_t128", "causal_mha_t1024", "varlen_b16_t2048", "long_causal_gqa_t16384"):
            others[name] = time_workload(name, args.steps, max(args.warmup, 3), args.block_order)

    if args.calibrate_copy_mb > 0:
        n = args.calibrate_copy_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)      # the last dispatch of the run: n bytes read, n bytes written
        torch.cuda.synchronize()

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.T, "heads": w.heads, "kv_heads": w.kv_heads,
                   "head_dim": HEAD_DIM, "causal": w.causal, "varlen": w.varlen, "parallelism": "single GPU"},
        "pct_mfma_peak": round(100 * value / PEAK_TFLOPS, 2),
        "flops_per_step": fl["total"],
        "kernels": kernels,
        "phases": phases,
        "roofline": roofline,
    }
    if settle is not None:
        out["clock_settle"] = settle
    if cold is not None:
        out["cold"] = cold
    if state_before is not None or state_after is not None:
        out["gpu_state"] = {"before": state_before, "after": state_after}
    if not args.headline_only:
        out["device"] = device_info()
    if two_pass is not None:
        out["two_pass_backward"] = two_pass
    if v_rows is not None:
        out["v_rows"] = v_rows
    if dq_rotated is not None:
        out["dq_pass_rotated"] = dq_rotated
    if projection is not None:
        out["projection_backward"] = projection
    if chunked is not None:
        out["chunked_backward"] = chunked
    if others is not None:
        out["other_workloads"] = others
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
