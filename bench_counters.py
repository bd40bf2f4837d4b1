#!/usr/bin/env python3
"""Profiles one bench.py workload with rocprofv3 and writes the summaries
that bench.py and the documentation use.

Runs, each as its own rocprofv3 process with the program directly after
``--`` (this script itself never touches the GPU):
  1. ``--kernel-trace --stats`` over a short bench run (per-kernel durations);
  2. ``--pmc FETCH_SIZE`` and 3. ``--pmc WRITE_SIZE`` over a 3-step bench run;
  4./5. the same two counters over a plain device copy of known size
     (``bench.py --copy-calib-mb``), which calibrates the counters to bytes;
  6. ``--pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES
     GRBM_GUI_ACTIVE`` over a 3-step bench run and 7. over a bf16 matrix
     product of known flop count (``bench.py --mfma-calib``): MFMA flops per
     call and the fraction of SIMD cycles the matrix units were busy.

Writes profiles/kernel_stats_<workload>.txt, profiles/hbm_traffic_<workload>.txt,
profiles/mfma_<workload>.txt and, for bench.py's default workload,
profiles/hbm_traffic.txt and profiles/mfma.txt (JSON read by bench.py: HBM
bytes and MFMA counters per call, tagged with a hash of the kernel sources).

    python bench_counters.py [--config N] [--cache dtype|e4m3] [--form merged|factored]
                             [--out <dir for the raw profiler output>]
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.abspath(__file__))
CALLS = ("mla_compress_append", "mla_q_proj", "mla_attention", "mla_out_proj")
COPY_MB = 512
MFMA_N = 4096
MFMA_CTRS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
N_SIMD = 1024  # 256 CUs x 4 SIMDs
N_XCD = 8      # GRBM_GUI_ACTIVE comes summed over the XCDs' graphics blocks


def run(cmd, out_dir, name, timeout):
    log = os.path.join(out_dir, name + ".log")
    print("[counters] " + " ".join(cmd), flush=True)
    with open(log, "w") as f:
        r = subprocess.run(cmd, stdout=f, stderr=subprocess.STDOUT, timeout=timeout, cwd="/tmp",
                           env=dict(os.environ, TMPDIR="/tmp"))
    print(f"[counters] {name}: exit {r.returncode}", flush=True)
    if r.returncode != 0:
        with open(log) as f:
            sys.stdout.write(f.read()[-3000:])
        raise SystemExit(r.returncode)


def find(out_dir, name, suffix):
    hits = glob.glob(os.path.join(out_dir, name, "**", "*" + suffix), recursive=True)
    if not hits:
        raise SystemExit(f"no {suffix} under {out_dir}/{name}")
    return hits[0]


def mla_kernel(name: str) -> bool:
    return name.startswith("_ZN3mla") or "mla::" in name


def counter_per_dispatch(path):
    """{dispatch id: (kernel name, summed counter value)}"""
    out = {}
    with open(path) as f:
        rd = csv.DictReader(f)
        need = {"Dispatch_Id", "Kernel_Name", "Counter_Value"}
        if not need <= set(rd.fieldnames or []):
            raise SystemExit(f"{path}: columns {rd.fieldnames}")
        for r in rd:
            d = int(r["Dispatch_Id"])
            name, val = r["Kernel_Name"], float(r["Counter_Value"])
            prev = out.get(d, (name, 0.0))
            out[d] = (name, prev[1] + val)
    return out


def counters_per_dispatch(path):
    """{dispatch id: (kernel name, {counter name: summed value})}"""
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            name, vals = out.setdefault(d, (r["Kernel_Name"], {}))
            vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


# weight form of the profiled run (set by main): it fixes the launches per call
FORM = "merged"


def steps(per_dispatch):
    """The bench steps in the dispatch list, each a list of (call, dispatch id).

    A step is: the append GEMM (followed by the quantising store kernel for
    an E4M3 cache), the q-projection (merged: the c_Q and q GEMMs; factored:
    the c_Q GEMM and the fused per-head kernel, or four GEMMs above 16
    rows), the attention plan / split / merge kernels, then the output
    projection (merged: its GEMM, preceded by the fp32 -> bf16 staging of
    o_lat when the large tiling takes it; factored: two GEMMs); a GEMM whose
    K range is split is followed by its epilogue kernel.  Steps are anchored
    at their attention plan kernels."""
    ids = [d for d in sorted(per_dispatch) if mla_kernel(per_dispatch[d][0])]
    names = [per_dispatch[d][0] for d in ids]
    plans = [i for i, n in enumerate(names) if "attn_plan" in n]
    q_groups, out_groups = 2, 1
    if FORM == "factored":
        out_groups = 2
        q_groups = 2 if any("q_fused" in n for n in names) else 4

    def gemm_groups_before(end, count):
        groups, i = [], end - 1
        while len(groups) < count:
            g = [i]
            if "cache_store" in names[i]:  # E4M3 append: its GEMM (+ epilogue), then the quantising store
                i -= 1
                g.insert(0, i)
            if "splitk_epilogue" in names[i]:
                i -= 1
                g.insert(0, i)
            groups.insert(0, g)
            i -= 1
        return groups

    out = []
    for plan in plans:
        if plan < 3:
            continue
        pre = gemm_groups_before(plan, 1 + q_groups)
        calls = [("mla_compress_append", i) for i in pre[0]] + [("mla_q_proj", i) for g in pre[1:] for i in g]
        calls += [("mla_attention", plan), ("mla_attention", plan + 1), ("mla_attention", plan + 2)]
        i = plan + 3
        if i < len(names) and "f32_to_bf16" in names[i]:
            calls.append(("mla_out_proj", i))
            i += 1
        for _ in range(out_groups):
            if i < len(names):
                calls.append(("mla_out_proj", i))
                i += 1
            if i < len(names) and "splitk_epilogue" in names[i]:
                calls.append(("mla_out_proj", i))
                i += 1
        out.append([(c, ids[k]) for c, k in calls])
    return out


def last_step(per_dispatch):
    """(call, kernel name, value) for the dispatches of the last bench step."""
    return [(c, per_dispatch[d][0], per_dispatch[d][1]) for c, d in steps(per_dispatch)[-1]]


def trace_durations(path, skip=5):
    """Per position of a step: mean duration (us) over the traced steps after
    the first `skip` (warm-up), from a kernel-trace CSV."""
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            per[d] = (r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    st = steps(per)[skip:]
    n = len(st[-1])
    st = [s for s in st if len(s) == n]
    return [sum(per[s[k][1]][1] for s in st) / len(st) for k in range(n)]


def trace_passes(path, warmup, k):
    """Mean traced duration (us) of each call per bench pass: warm-up, the
    timed region, the back-to-back steps that time the roofline call, and the
    pass with a marker between the calls."""
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            per[d] = (r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    st = steps(per)
    bounds = {"warm-up": (0, warmup), "timed": (warmup, warmup + k), "roofline": (warmup + k, warmup + 2 * k),
              "marked": (warmup + 2 * k, warmup + 3 * k)}
    out = {}
    for name, (a, b) in bounds.items():
        sel = st[a:b]
        if not sel:
            continue
        tot = {c: 0.0 for c in CALLS}
        for s_ in sel:
            for c, d in s_:
                tot[c] += per[d][1]
        out[name] = {c: v / len(sel) for c, v in tot.items()}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=None, help="workload index (default: bench.py's)")
    ap.add_argument("--cache", choices=("dtype", "e4m3"), default="dtype", help="bench.py --cache")
    ap.add_argument("--form", choices=("merged", "factored"), default="merged", help="bench.py --form")
    ap.add_argument("--out", default=os.path.join(tempfile.gettempdir(), "mla_counters"))
    ap.add_argument("--profiles-dir", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--summarize-only", action="store_true",
                    help="rebuild the summaries from the profiler output already under --out")
    args = ap.parse_args()
    global FORM
    FORM = args.form
    sys.path.insert(0, ROOT)
    import bench as bench_mod
    if args.config is None:
        args.config = bench_mod.DEFAULT_CONFIG
    # the profiler runs from /tmp: every path handed to it is absolute
    args.out = os.path.abspath(args.out)
    args.profiles_dir = os.path.abspath(args.profiles_dir)
    os.makedirs(args.out, exist_ok=True)
    py = sys.executable
    bench = [py, os.path.join(ROOT, "bench.py"), "--config", str(args.config), "--no-cpu-baseline",
             "--cache", args.cache] + (["--form", args.form] if args.form != "merged" else [])
    trace_steps, trace_warmup = 20, 5
    stats_cmd = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d",
                 os.path.join(args.out, "trace"), "-o", "run", "--"] + bench + ["--steps", str(trace_steps),
                                                                              "--warmup", str(trace_warmup)]
    if not args.summarize_only:
        run(stats_cmd, args.out, "trace", 600)
    pmc = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        cmd = ["timeout", "-s", "KILL", "120", "rocprofv3", "--pmc", ctr, "--output-format", "csv", "-d",
               os.path.join(args.out, "pmc_" + ctr), "-o", "run", "--"] + bench + ["--steps", "3", "--warmup", "1"]
        if not args.summarize_only:
            run(cmd, args.out, "pmc_" + ctr, 180)
        pmc[ctr] = counter_per_dispatch(find(args.out, "pmc_" + ctr, "counter_collection.csv"))
        cmd = ["timeout", "-s", "KILL", "60", "rocprofv3", "--pmc", ctr, "--output-format", "csv", "-d",
               os.path.join(args.out, "copy_" + ctr), "-o", "run", "--", py, os.path.join(ROOT, "bench.py"),
               "--copy-calib-mb", str(COPY_MB), "--steps", "3"]
        if not args.summarize_only:
            run(cmd, args.out, "copy_" + ctr, 120)
        pmc["copy_" + ctr] = counter_per_dispatch(find(args.out, "copy_" + ctr, "counter_collection.csv"))

    # MFMA counters over the bench and over a matrix product of known size
    mf_cmd = ["timeout", "-s", "KILL", "120", "rocprofv3", "--pmc", *MFMA_CTRS, "--output-format", "csv", "-d",
              os.path.join(args.out, "pmc_mfma"), "-o", "run", "--"] + bench + ["--steps", "3", "--warmup", "1"]
    cal_cmd = ["timeout", "-s", "KILL", "60", "rocprofv3", "--pmc", *MFMA_CTRS, "--output-format", "csv", "-d",
               os.path.join(args.out, "cal_mfma"), "-o", "run", "--", py, os.path.join(ROOT, "bench.py"),
               "--mfma-calib", str(MFMA_N), "--steps", "3"]
    if not args.summarize_only:
        run(mf_cmd, args.out, "pmc_mfma", 180)
        run(cal_cmd, args.out, "cal_mfma", 120)
    mf = counters_per_dispatch(find(args.out, "pmc_mfma", "counter_collection.csv"))
    cal = counters_per_dispatch(find(args.out, "cal_mfma", "counter_collection.csv"))
    cal_mops = sorted(v["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for n, v in cal.values()
                      if v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) > 0)
    flops_per_mop = 2.0 * MFMA_N ** 3 / cal_mops[len(cal_mops) // 2]

    # calibration: the copy reads and writes COPY_MB MiB per launch
    true_bytes = COPY_MB * (1 << 20)
    factors = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        vals = [v for (n, v) in pmc["copy_" + ctr].values() if "add" in n.lower()]
        kib = sorted(vals)[len(vals) // 2]
        factors[ctr] = true_bytes / (kib * 1024.0)

    fetch, write = last_step(pmc["FETCH_SIZE"]), last_step(pmc["WRITE_SIZE"])
    calls = {c: 0.0 for c in CALLS}
    rows = []
    for (call, name, f), (_, _, w) in zip(fetch, write):
        fb = f * 1024.0 * factors["FETCH_SIZE"]
        wb = w * 1024.0 * factors["WRITE_SIZE"]
        calls[call] += fb + wb
        rows.append((call, name, f, w, fb, wb))

    stats = find(args.out, "trace", "kernel_stats.csv")
    with open(stats) as f:
        krows = sorted(csv.DictReader(f), key=lambda r: -float(r["TotalDurationNs"]))
    # mean duration of each position of a step over the traced steps (one
    # kernel can serve several calls, so durations go by position, not name)
    pos_us = trace_durations(find(args.out, "trace", "kernel_trace.csv"))

    # MFMA per dispatch of the last step: counted flops, busy fraction, and
    # the rate over that position's mean duration in the trace pass
    mrows, mcalls = [], {c: {"flops": 0.0, "us": 0.0, "busy": 0.0, "active": 0.0} for c in CALLS}
    mf_step = last_step({d: (n, d) for d, (n, _) in mf.items()})
    if len(mf_step) != len(pos_us):
        raise SystemExit(f"step shapes differ: {len(mf_step)} counted dispatches, {len(pos_us)} traced")
    for k, (call, name, d) in enumerate(mf_step):
        v = mf[int(d)][1]
        flops = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * flops_per_mop
        busy, active = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), v.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
        us = pos_us[k]
        mrows.append((call, name, flops, busy / (active * N_SIMD) if active else 0.0, us))
        m = mcalls[call]
        m["flops"] += flops
        m["us"] += us
        m["busy"] += busy
        m["active"] += active * N_SIMD
    sys.path.insert(0, ROOT)
    from synthetic import config
    workload = (config(args.config).name + ("_e4m3" if args.cache == "e4m3" else "") +
                ("_factored" if args.form == "factored" else ""))
    form_arg = f" --form {args.form}" if args.form != "merged" else ""

    prof = args.profiles_dir
    os.makedirs(prof, exist_ok=True)
    with open(os.path.join(prof, f"kernel_stats_{workload}.txt"), "w") as f:
        f.write(f"# rocprofv3 kernel-trace statistics, workload {workload}\n")
        f.write("# command (run from /tmp): " + " ".join(stats_cmd).replace(ROOT, ".") + "\n")
        f.write(f"{'kernel':90s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'total_%':>8s}\n")
        for r in krows:
            f.write(f"{r['Name'][:90]:90s} {r['Calls']:>6s} {float(r['AverageNs']) / 1e3:10.2f} "
                    f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):8.2f}\n")
        f.write("# per bench pass: mean traced duration (us) of each call's kernels per step (warm-up; timed\n"
                "# region; back-to-back steps with an event pair around the roofline call; pass with a marker\n"
                "# between the calls)\n")
        passes = trace_passes(find(args.out, "trace", "kernel_trace.csv"), trace_warmup, trace_steps)
        f.write(f"# {'call':22s}" + "".join(f" {p:>10s}" for p in passes) + "\n")
        for c in CALLS:
            f.write(f"# {c:22s}" + "".join(f" {passes[p][c]:10.2f}" for p in passes) + "\n")
    with open(os.path.join(prof, f"hbm_traffic_{workload}.txt"), "w") as f:
        f.write(f"# HBM traffic per dispatch, workload {workload}, last step of a 3-step bench run\n")
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            f.write(f"# command: timeout -s KILL 120 rocprofv3 --pmc {ctr} --output-format csv -d <dir> -o run -- "
                    f"python ./bench.py --config {args.config} --no-cpu-baseline --cache {args.cache}{form_arg} "
                    f"--steps 3 --warmup 1\n")
            f.write(f"# calibration: timeout -s KILL 60 rocprofv3 --pmc {ctr} ... -- python ./bench.py "
                    f"--copy-calib-mb {COPY_MB} --steps 3 ; factor {factors[ctr]:.4f} bytes per counted byte\n")
        f.write(f"{'call':22s} {'kernel':70s} {'FETCH_KiB':>12s} {'WRITE_KiB':>12s} {'read_MB':>10s} {'write_MB':>10s}\n")
        for call, name, fk, wk, fb, wb in rows:
            f.write(f"{call:22s} {name[:70]:70s} {fk:12.0f} {wk:12.0f} {fb / 1e6:10.2f} {wb / 1e6:10.2f}\n")
        for c in CALLS:
            f.write(f"# {c}: {calls[c] / 1e6:.2f} MB per call (read + write)\n")
    with open(os.path.join(prof, f"mfma_{workload}.txt"), "w") as f:
        f.write(f"# MFMA counters per dispatch, workload {workload}, last step of a 3-step bench run\n")
        f.write("# command: " + " ".join(mf_cmd).replace(ROOT, ".").replace(args.out, "<dir>") + "\n")
        f.write("# calibration: " + " ".join(cal_cmd).replace(ROOT, ".").replace(args.out, "<dir>") +
                f" ; {flops_per_mop:.1f} flops per counted operation (2 n^3 over the product's counter)\n")
        f.write(f"# busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {N_XCD} XCDs x {N_SIMD} SIMDs); "
                f"rate = counted flops / "
                f"that dispatch's mean duration over the steps of the kernel-trace run; peak 2500 TFLOP/s (dense bf16)\n")
        f.write(f"{'call':22s} {'kernel':70s} {'GFLOP':>10s} {'avg_us':>9s} {'TFLOP/s':>9s} {'%peak':>7s} {'busy%':>7s}\n")
        for call, name, fl, bz, us in mrows:
            f.write(f"{call:22s} {name[:70]:70s} {fl / 1e9:10.3f} {us:9.2f} {fl / (us * 1e-6) / 1e12:9.1f} "
                    f"{100 * fl / (us * 1e-6) / 2.5e15:7.2f} {100 * bz:7.2f}\n")
        for c in CALLS:
            m = mcalls[c]
            f.write(f"# {c}: {m['flops'] / 1e9:.3f} GFLOP counted, {m['flops'] / (m['us'] * 1e-6) / 1e12:.1f} TFLOP/s "
                    f"({100 * m['flops'] / (m['us'] * 1e-6) / 2.5e15:.2f}% of peak), MFMA busy "
                    f"{100 * m['busy'] / max(m['active'], 1):.2f}% of SIMD cycles\n")
    if args.config == bench_mod.DEFAULT_CONFIG and args.cache == "dtype" and args.form == "merged":
        mout = {"workload": workload, "source_hash": bench_mod.kernel_source_hash(), "flops_per_mop": flops_per_mop,
                "calls": {c: {"gflop": round(m["flops"] / 1e9, 4),
                              "busy_pct": round(100 * m["busy"] / max(m["active"], 1), 2)} for c, m in mcalls.items()}}
        with open(os.path.join(prof, "mfma.txt"), "w") as f:
            json.dump(mout, f, indent=1)
            f.write("\n")
        out = {"workload": workload, "source_hash": bench_mod.kernel_source_hash(), "factors": factors,
               "calls": {c: round(v) for c, v in calls.items()}}
        with open(os.path.join(prof, "hbm_traffic.txt"), "w") as f:
            json.dump(out, f, indent=1)
            f.write("\n")
    print(json.dumps({"factors": factors, "calls_MB": {c: round(v / 1e6, 2) for c, v in calls.items()}}))


if __name__ == "__main__":
    main()
