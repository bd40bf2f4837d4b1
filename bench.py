#!/usr/bin/env python3
"""MLA decode benchmark on one MI355X.

A step is one pass of the layer's hot path over one batch, through the C
ABI: mla_compress_append (latent down-projection + RoPE + append),
mla_q_proj (merged query projection), mla_attention (split-KV attention over
the latent cache + log-sum-exp merge) and mla_out_proj (merged output
projection).  The default workload is the largest single-GPU DeepSeek-V2-shaped
decode layer: batch 64, context lengths uniform in [512, 16384], a paged bf16
latent cache of 64-token pages, fp32 accumulation.  Inputs are seeded and
synthetic and sit in HBM before the timed region starts.

The roofline object describes the latent-cache attention (mla_attention:
plan, split and merge kernels), the kernel the method's decode cost is
about; its duration is the mean of an event pair around that call in K
more steps queued back to back behind the timed region (the median is
reported beside it).

Prints ONE JSON line (see the "roofline" and "cpu_baseline" objects).
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

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
F32_PEAK_TFLOPS = 157.3      # MI355X dense fp32 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma.txt")
KERNEL_SOURCES = ("mla_gemm.hip", "mla_attn.hip", "mla_cache.hip", "mla_common.h")
DEFAULT_CONFIG = 2
ROOFLINE_CALL = "mla_attention"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", type=int, default=DEFAULT_CONFIG,
                   help="workload index (2: V2 decode, B=64, paged, 512..16384 cached tokens)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--form", choices=("merged", "factored"), default="merged",
                   help="absorbed weights: merged products (default) or the factors applied at run time")
    p.add_argument("--prefill", choices=("absorbed", "expanded"), default="absorbed",
                   help="expanded: the step is append + mla_prefill_expanded (factored weights, contiguous cache; "
                        "the V3 chunked-prefill workload)")
    p.add_argument("--cache", choices=("dtype", "e4m3"), default="dtype",
                   help="latent cache rows: the layer dtype, or E4M3 codes with one scale per row (bf16 layers)")
    p.add_argument("--graph", action="store_true",
                   help="replay each step from a HIP graph captured once per input copy")
    p.add_argument("--copies", type=int, default=4,
                   help="input sets (absorbed weights, cache, activations) rotated over the steps, so that no "
                        "step finds its inputs in the 256 MB last-level cache")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget for the oracle sample")
    p.add_argument("--copy-calib-mb", type=int, default=0,
                   help="only run a plain device copy of this many MB (counter calibration)")
    p.add_argument("--mfma-calib", type=int, default=0,
                   help="only run a bf16 n x n x n matrix product (MFMA counter calibration)")
    return p.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for s in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "head_latent_attention_13_amd", "csrc", s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(call: str, workload: str):
    """HBM bytes per launch from the committed counter runs, if they were
    taken on this workload with the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return t.get("calls", {}).get(call)


def measured_mfma(workload: str):
    """MFMA counters per call (counted GFLOP, busy % of SIMD cycles) from the
    committed counter run, if it was taken on this workload with the current
    kernel sources; else None."""
    try:
        with open(MFMA_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return t.get("calls")


def copy_calibration(mb: int, steps: int):
    """A plain streaming kernel of known traffic (reads and writes mb MiB per
    launch) for scaling the HBM byte counters."""
    import torch
    n = mb * (1 << 20) // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(steps):
        torch.add(a, 1.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": steps}))


def mfma_calibration(n: int, steps: int):
    """A bf16 matrix product of known flop count (2 n^3 per launch) for
    scaling the MFMA operation counter."""
    import torch
    a = torch.ones(n, n, dtype=torch.bfloat16, device="cuda")
    b = torch.ones(n, n, dtype=torch.bfloat16, device="cuda")
    for _ in range(steps):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    print(json.dumps({"mfma_calibration_flops": 2 * n ** 3, "launches": steps}))


def cpu_baseline(case, n_budget_s: float):
    """The expanded fp64 oracle timed on a bounded sample of the workload.

    Work units are (sequence, block of its new tokens, block of heads); a
    unit runs the oracle's row and query projections for those tokens and
    its expanded attention for those heads over the sequence's whole visible
    history.  Units run in order until the time budget is spent; the rate is
    tokens x (heads done / all heads) per second, i.e. whole-layer tokens/s.
    """
    import numpy as np
    import threadpoolctl
    from oracle import expanded as OE
    cfg = case.cfg
    W = {k: np.asarray(v, np.float64) for k, v in case.weights.items()}
    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    H, n_q = cfg.n_heads, cfg.n_q
    kq = min(n_q, 16)
    work = 0.0                       # tokens x fraction of heads
    units, t0 = 0, time.perf_counter()
    first_desc = None
    for b in range(cfg.batch):
        rows = case.rows[b]
        m = int(case.cached[b]) + n_q
        hsz = int(max(8, min(H, (H * 4200) // max(m, 1))))
        for q0 in range(0, n_q, kq):
            xq = case.x_new[b][q0:q0 + kq]
            pos = int(case.cached[b]) + q0 + np.arange(len(xq))
            # rows of all new tokens up to this block (causal: later ones unseen)
            c_new, k_new = OE.latent_rows(W, case.x_new[b][:q0 + len(xq)], int(case.cached[b]) + np.arange(q0 + len(xq)),
                                          cfg.rope_base)
            c = np.concatenate([np.asarray(rows[:, :cfg.d_latent], np.float64), c_new])
            kp = np.concatenate([np.asarray(rows[:, cfg.d_latent:], np.float64), k_new])
            _, q_nope, q_pe = OE.query(W, xq, pos, cfg.rope_base)
            for h0 in range(0, H, hsz):
                hs = list(range(h0, min(H, h0 + hsz)))
                OE.attention(W, q_nope, q_pe, c, kp, pos, cfg.softmax_scale, heads=hs)
                work += len(xq) * len(hs) / H
                units += 1
                if first_desc is None:
                    first_desc = f"{len(xq)} new token(s) x {len(hs)} heads over {m} visible rows"
                if time.perf_counter() - t0 > n_budget_s:
                    break
            if time.perf_counter() - t0 > n_budget_s:
                break
        if time.perf_counter() - t0 > n_budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": work / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"expanded fp64 oracle (row and query projections + per-head expanded attention), {units} work "
                      f"units of {first_desc} each, {work:.3g} whole-layer tokens in {dt:.1f} s"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (batch sharding would need no "
              "exchange between GPUs). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calib_mb:
        copy_calibration(args.copy_calib_mb, args.steps)
        return
    if args.mfma_calib:
        mfma_calibration(args.mfma_calib, args.steps)
        return

    import head_latent_attention_13_amd as mla
    from synthetic import config, make_case

    torch.cuda.set_device(0)
    cfg = config(args.config)
    if args.prefill == "expanded":
        if cfg.paged:
            print("--prefill expanded needs a contiguous cache", file=sys.stderr)
            sys.exit(2)
        args.form = "factored"
    e4 = args.cache == "e4m3"
    if e4 and (cfg.dtype != "bf16" or args.prefill == "expanded"):
        print("--cache e4m3 needs a bf16 layer and the absorbed path", file=sys.stderr)
        sys.exit(2)
    case = make_case(cfg, args.config, history="rows")
    B, n_q, H, R = cfg.batch, cfg.n_q, cfg.n_heads, cfg.row
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    devt = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(tdt)
    dims = mla.make_dims(cfg.d_model, H, cfg.d_latent, cfg.d_q_latent, cfg.d_nope, cfg.d_rope, cfg.d_v,
                         cfg.dtype, cfg.rope_base, form=args.form)
    raw = {k: devt(v) for k, v in case.weights.items()}

    # one-time absorption, timed on its own: a second call into the layer's
    # buffer (allocated by then; the call rewrites the same values)
    layer = mla.MLALayer(dims, raw, max_batch=B, max_nq=n_q)
    torch.cuda.synchronize()
    t_abs0 = torch.cuda.Event(enable_timing=True)
    t_abs1 = torch.cuda.Event(enable_timing=True)
    t_abs0.record()
    mla.mla_absorb_weights(dims, raw, layer.absorbed)
    t_abs1.record()
    torch.cuda.synchronize()
    absorb_ms = t_abs0.elapsed_time(t_abs1)
    NC = max(1, args.copies)
    layers = [layer] + [mla.MLALayer(dims, raw, max_batch=B, max_nq=n_q) for _ in range(NC - 1)]
    del raw

    kv_len = case.cached + n_q
    if cfg.paged:
        P = cfg.page_size
        table = torch.from_numpy(case.page_table).cuda()
        pool = torch.zeros(case.n_pages, P, R, dtype=tdt, device="cuda")
        for b in range(B):
            npg = (int(kv_len[b]) + P - 1) // P
            tmp = torch.zeros(npg * P, R, dtype=tdt, device="cuda")
            tmp[:len(case.rows[b])] = devt(case.rows[b])
            pool[table[b, :npg].long()] = tmp.view(npg, P, R)
        cache = mla.Cache(pool=pool, page_table=table, page_size=P, n_pages=case.n_pages,
                          max_pages_per_seq=case.page_table.shape[1])
    else:
        s_max = int(kv_len.max())
        pool = torch.zeros(B, s_max, R, dtype=tdt, device="cuda")
        for b in range(B):
            pool[b, :len(case.rows[b])] = devt(case.rows[b])
        cache = mla.Cache(pool=pool, s_max=s_max)
    scales = None
    if e4:
        # the same history rows, quantised by the library into an E4M3 cache
        # of the same layout (one sequence at a time, through its row of the
        # page table)
        e4pool = torch.zeros(pool.shape, dtype=torch.uint8, device="cuda")
        scales = torch.zeros(pool.shape[:2], dtype=torch.float32, device="cuda")
        for b in range(B):
            S = len(case.rows[b])
            if S == 0:
                continue
            rows32 = torch.from_numpy(np.ascontiguousarray(case.rows[b], np.float32)).cuda()
            if cfg.paged:
                one = mla.Cache(pool=e4pool, page_table=table[b:b + 1].contiguous(), page_size=P, n_pages=case.n_pages,
                                max_pages_per_seq=case.page_table.shape[1], scales=scales)
            else:
                one = mla.Cache(pool=e4pool[b:b + 1], s_max=s_max, scales=scales[b:b + 1])
            layer.store_rows(rows32, torch.zeros(1, dtype=torch.int32, device="cuda"), 1, S, one)
        torch.cuda.synchronize()
        assert layer.device_error() == 0
        pool = e4pool
        cache = (mla.Cache(pool=pool, page_table=table, page_size=P, n_pages=case.n_pages,
                           max_pages_per_seq=case.page_table.shape[1], scales=scales) if cfg.paged
                 else mla.Cache(pool=pool, s_max=s_max, scales=scales))
    x = devt(case.x_new.reshape(B * n_q, cfg.d_model))
    pos = torch.from_numpy(case.cached.astype(np.int32)).cuda()
    kv = torch.from_numpy(kv_len.astype(np.int32)).cuda()
    # copy j of every input: step k runs on copy k % NC
    if cfg.paged:
        caches = [cache] + [mla.Cache(pool=pool.clone(), page_table=table.clone(), page_size=cache.page_size,
                                      n_pages=cache.n_pages, max_pages_per_seq=cache.max_pages_per_seq,
                                      scales=None if scales is None else scales.clone())
                            for _ in range(NC - 1)]
    else:
        caches = [cache] + [mla.Cache(pool=pool.clone(), s_max=cache.s_max,
                                      scales=None if scales is None else scales.clone()) for _ in range(NC - 1)]
    xs = [x] + [x.clone() for _ in range(NC - 1)]
    poss = [pos] + [pos.clone() for _ in range(NC - 1)]
    kvs = [kv] + [kv.clone() for _ in range(NC - 1)]
    qs = [torch.empty(B * n_q, H, R, dtype=tdt, device="cuda") for _ in range(NC)]
    o_lats = [torch.empty(B * n_q, H, cfg.d_latent, dtype=torch.float32, device="cuda") for _ in range(NC)]
    ys = [torch.empty(B * n_q, cfg.d_model, dtype=torch.float32, device="cuda") for _ in range(NC)]

    expanded = args.prefill == "expanded"
    calls = (("mla_compress_append", "mla_prefill_expanded") if expanded else
             ("mla_compress_append", "mla_q_proj", "mla_attention", "mla_out_proj"))

    def step(k, evs=None):
        # evs: {marker position: event}; position i sits before call i
        def mark(i):
            if evs is not None and i in evs:
                evs[i].record()
        j = k % NC
        ly, cc, xx, qq, ol = layers[j], caches[j], xs[j], qs[j], o_lats[j]
        mark(0)
        ly.append(xx, poss[j], B, n_q, cc)
        mark(1)
        if expanded:
            ly.prefill_expanded(xx, kvs[j], B, n_q, cc, ys[j])
            mark(2)
            return
        ly.q_proj(xx, kvs[j], B, n_q, qq)
        mark(2)
        ly.attention(qq, kvs[j], B, n_q, cc, ol)
        mark(3)
        ly.out_proj(ol, B * n_q, ys[j])
        mark(4)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    run = step
    if args.graph:
        # one graph per input copy, captured after the warm-up (the library
        # allocates nothing and issues no memset, so a step captures whole)
        graphs = []
        for j in range(NC):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(j)
            graphs.append(g)
        torch.cuda.synchronize()

        def run(k):
            graphs[k % NC].replay()

        for k in range(args.warmup):
            run(k)
        torch.cuda.synchronize()
    # timed region: K whole steps back to back, events only at its ends
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for k in range(args.steps):
        run(k)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    # The roofline call is timed inside back-to-back steps: K more steps are
    # queued behind the timed region before the host waits, with an event
    # pair around that call only (the per-call markers below leave idle
    # gaps of about 10 us before every call; the mean time in that pass is
    # reported beside it as ms_marked_pass).
    roof_call = "mla_prefill_expanded" if expanded else ROOFLINE_CALL
    ri = calls.index(roof_call)
    rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for k in range(args.steps):
        step(k, {ri: rev[k][0], ri + 1: rev[k][1]})
    torch.cuda.synchronize()
    roof_samples = [a.elapsed_time(b) for a, b in rev]
    # per-call breakdown: a second pass with an event between the calls (the
    # markers themselves cost a few microseconds per call, so this pass is
    # not used for the step time)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    for k in range(args.steps):
        step(k, dict(enumerate(ev[k])))
    torch.cuda.synchronize()
    call_samples = {c: [ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(args.steps)] for i, c in enumerate(calls)}
    marked_roof_ms = float(np.mean(call_samples[roof_call]))
    call_samples[roof_call] = roof_samples
    per_call_ms = {c: float(np.mean(v)) for c, v in call_samples.items()}
    per_call_median_ms = {c: float(np.median(v)) for c, v in call_samples.items()}
    step_median_ms = float(np.median([ev[k][0].elapsed_time(ev[k][-1]) for k in range(args.steps)]))
    assert all(ly.device_error() == 0 and ly.prefill_error() == 0 for ly in layers)

    # ---- algorithmic bytes / flops per call (one step) ------------------
    eb = 2 if cfg.dtype == "bf16" else 4
    M = B * n_q
    rows_visible = int(kv_len.sum())
    pairs = int(sum(int(c) * n_q + n_q * (n_q + 1) // 2 for c in case.cached))  # unmasked (query, key) pairs
    _, wbytes, _ = mla.mla_absorbed_layout(dims)
    row_bytes = R + 4 if e4 else R * eb  # E4M3: one byte per element plus the row's fp32 scale
    cache_bytes = (rows_visible if n_q == 1 else int(B * (int(case.cached.max()) + n_q))) * row_bytes
    algo = {
        "mla_compress_append": {"bytes": wbytes[0] + M * cfg.d_model * eb + M * row_bytes,
                                "flops": 2 * M * cfg.d_model * R},
        "mla_q_proj": {"bytes": wbytes[1] + wbytes[2] + M * cfg.d_model * eb + M * H * R * eb,
                       "flops": 2 * M * cfg.d_model * cfg.d_q_latent + 2 * M * cfg.d_q_latent * H * R},
        "mla_attention": {"bytes": cache_bytes + M * H * R * eb + M * H * cfg.d_latent * 4,
                          "flops": 2 * H * pairs * (R + cfg.d_latent)},
        "mla_out_proj": {"bytes": wbytes[3] + M * H * cfg.d_latent * 4 + M * cfg.d_model * 4,
                         "flops": 2 * M * H * cfg.d_latent * cfg.d_model},
    }
    if expanded:
        # queries, per-head keys/values of every cache slot (written, read back), causal attention per
        # head with 192-wide keys and 128-wide values, the W_O product
        s_slots = B * cache.s_max
        kv_bytes = 2 * s_slots * H * (cfg.d_nope + cfg.d_v) * eb
        algo["mla_prefill_expanded"] = {
            "bytes": wbytes[1] + wbytes[2] + wbytes[3] + M * cfg.d_model * eb + s_slots * R * eb + kv_bytes
                     + M * cfg.d_model * 4,
            "flops": 2 * M * (cfg.d_model * cfg.d_q_latent + cfg.d_q_latent * H * (cfg.d_nope + cfg.d_rope))
                     + 2 * s_slots * cfg.d_latent * H * (cfg.d_nope + cfg.d_v)
                     + 2 * H * pairs * (cfg.d_nope + cfg.d_rope + cfg.d_v)
                     + 2 * M * H * cfg.d_v * cfg.d_model}
    if args.form == "factored" and not expanded:
        # the factors plus the intermediates c_Q W_UQ and o_lat W_UV (written, read back)
        algo["mla_q_proj"] = {
            "bytes": wbytes[1] + wbytes[2] + M * cfg.d_model * eb + M * H * R * eb + 2 * M * H * cfg.d_nope * eb,
            "flops": 2 * M * (cfg.d_model * cfg.d_q_latent + cfg.d_q_latent * H * (cfg.d_nope + cfg.d_rope)
                              + H * cfg.d_nope * cfg.d_latent)}
        algo["mla_out_proj"] = {
            "bytes": wbytes[3] + M * H * cfg.d_latent * 4 + M * cfg.d_model * 4 + 2 * M * H * cfg.d_v * eb,
            "flops": 2 * M * H * cfg.d_v * (cfg.d_latent + cfg.d_model)}
    mfma_peak = BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else F32_PEAK_TFLOPS
    kernels = {}
    for c in calls:
        t = per_call_ms[c] * 1e-3
        gbs = algo[c]["bytes"] / t / 1e9
        tfl = algo[c]["flops"] / t / 1e12
        t_hbm = algo[c]["bytes"] / (HBM_PEAK_GBS * 1e9)
        t_mfma = algo[c]["flops"] / (mfma_peak * 1e12)
        bound = "hbm" if t_hbm >= t_mfma else "mfma"
        kernels[c] = {"ms": round(per_call_ms[c], 4), "ms_median": round(per_call_median_ms[c], 4), "bound": bound,
                      "GB_s": round(gbs, 1),
                      "TFLOP_s": round(tfl, 2), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                      "mfma_frac": round(tfl / mfma_peak, 4),
                      "roofline_frac": round((t_hbm if bound == "hbm" else t_mfma) / t, 4)}
    dom = roof_call
    kernels[dom]["timed"] = "inside back-to-back steps"
    kernels[dom]["ms_marked_pass"] = round(marked_roof_ms, 4)
    d = kernels[dom]
    workload = cfg.name + ("_e4m3" if e4 else "")
    traffic = measured_traffic(dom, workload)
    if d["bound"] == "hbm":
        roofline = {"bound": "hbm", "achieved": d["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(d["GB_s"] / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom,
                    "algorithmic_bytes": algo[dom]["bytes"], "ms": d["ms"]}
    else:
        roofline = {"bound": "mfma", "achieved": d["TFLOP_s"], "peak": mfma_peak, "unit": "TFLOP/s",
                    "frac": round(d["TFLOP_s"] / mfma_peak, 4), "traffic": traffic, "kernel": dom,
                    "algorithmic_flops": algo[dom]["flops"], "ms": d["ms"]}
    att = kernels["mla_prefill_expanded" if expanded else "mla_attention"]

    out = {
        "metric": "MLA decode tokens/s + latent-cache HBM GB/s & MFMA % of peak, 1 MI355X",
        "value": round(M / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median_marked": round(step_median_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; random-init weights of the DeepSeek-V2 layer shape)",
        "config": {"workload": workload, "batch": B, "cached_tokens": (list(cfg.cached) if isinstance(cfg.cached, tuple)
                                                                      else int(cfg.cached)),
                   "new_tokens": n_q, "heads": H, "d_latent": cfg.d_latent, "d_rope": cfg.d_rope,
                   "d_model": cfg.d_model, "cache": "paged" if cfg.paged else "contiguous",
                   "cache_rows": "e4m3 + fp32 scale per row" if e4 else cfg.dtype,
                   "weights": args.form, "prefill": args.prefill,
                   "launch": "HIP graph per step" if args.graph else "stream"},
        "roofline": roofline,
        "latent_cache_GB_s": round(cache_bytes / (per_call_ms["mla_prefill_expanded" if expanded else "mla_attention"]
                                                   * 1e-3) / 1e9, 1),
        "attention_mfma_pct": round(100 * att["mfma_frac"], 2),
        "attention_roofline_frac": att["roofline_frac"],
        # measured from the allocation (paged pools round up to whole pages)
        "kv_bytes_per_token_per_layer": round((pool.numel() * pool.element_size()
                                               + (0 if scales is None else scales.numel() * 4)) / int(kv_len.sum()), 1),
        "kernels": kernels,
        # rocprofv3 counters (SQ_INSTS_VALU_MFMA_MOPS_BF16 calibrated on a product of known size,
        # SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE), when taken on these kernel sources
        "mfma_counters": (measured_mfma(workload) if args.form == "merged" and not expanded else None),
        "absorb_ms_once": round(absorb_ms, 3),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
