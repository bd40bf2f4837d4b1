"""Host test of the profile summaries' bookkeeping: bench_counters.py splits
a rocprofv3 kernel trace into bench steps and attributes each dispatch to one
of the four calls, then averages every call per bench pass.  A synthetic
trace with known durations checks that attribution (no GPU involved)."""
import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench_counters as bc  # noqa: E402

# one merged-form decode step at 16 rows: append GEMM + split-K epilogue,
# c_Q GEMM + epilogue, q GEMM, attention plan / split / merge, output GEMM +
# epilogue (call, kernel name)
STEP = [
    ("mla_compress_append", "void mla::gemm_kernel<1, 2, 4>(mla::GemmArgs)"),
    ("mla_compress_append", "_ZN3mla22splitk_epilogue_kernelIDF16bEEvNS_8GemmArgsE"),
    ("mla_q_proj", "void mla::gemm_kernel<1, 2, 4>(mla::GemmArgs)"),
    ("mla_q_proj", "_ZN3mla22splitk_epilogue_kernelIDF16bEEvNS_8GemmArgsE"),
    ("mla_q_proj", "void mla::gemm_kernel<1, 9, 4>(mla::GemmArgs)"),
    ("mla_attention", "mla::attn_plan_kernel(mla::AttnArgs, int)"),
    ("mla_attention", "_ZN3mla17attn_split_kernelINS_7AttnCfgIDF16bLi128E"),
    ("mla_attention", "void mla::attn_merge_kernel<128, 512>(mla::AttnArgs)"),
    ("mla_out_proj", "void mla::gemm_kernel<1, 10, 4>(mla::GemmArgs)"),
    ("mla_out_proj", "_ZN3mla22splitk_epilogue_kernelIDF16bEEvNS_8GemmArgsE"),
]


def _write_trace(path, warmup, k, dur):
    """Absorption kernels first, then warmup + 3k steps; dispatch d of step s
    lasts dur(s, position) ns."""
    rows = []
    t, d = 0, 1
    for name in ("void mla::absorb_tile_kernel<true>(mla::ProdArgs)", "_ZN3mla11pack_kernelIDF16bEEvNS_10AbsorbArgs"):
        rows.append({"Dispatch_Id": d, "Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + 1000})
        t += 2000
        d += 1
    for s in range(warmup + 3 * k):
        for p, (_, name) in enumerate(STEP):
            n = dur(s, p)
            rows.append({"Dispatch_Id": d, "Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + n})
            t += n + 100
            d += 1
        # a torch copy between steps is not an mla kernel and is ignored
        rows.append({"Dispatch_Id": d, "Kernel_Name": "__amd_rocclr_copyBuffer", "Start_Timestamp": t,
                     "End_Timestamp": t + 50})
        t += 150
        d += 1
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)


@pytest.mark.parametrize("warmup,k", [(5, 20), (1, 3)])
def test_trace_passes_attribute_every_call_per_pass(tmp_path, warmup, k):
    bc.FORM = "merged"
    bounds = [warmup, warmup + k, warmup + 2 * k, warmup + 3 * k]

    def pass_of(s):
        return sum(s >= b for b in bounds[:3])

    # durations encode the pass and the position: 1000 * (pass + 1) + 10 * position
    def dur(s, p):
        return 1000 * (pass_of(s) + 1) + 10 * p

    path = str(tmp_path / "run_kernel_trace.csv")
    _write_trace(path, warmup, k, dur)
    got = bc.trace_passes(path, warmup, k)
    assert list(got) == ["warm-up", "timed", "roofline", "marked"]
    for i, name in enumerate(got):
        for call in bc.CALLS:
            want = sum(1000 * (i + 1) + 10 * p for p, (c, _) in enumerate(STEP) if c == call) / 1e3
            assert got[name][call] == pytest.approx(want), (name, call)


def test_trace_durations_average_positions_after_warmup(tmp_path):
    bc.FORM = "merged"
    warmup, k = 5, 20

    def dur(s, p):
        return 3000 if s < warmup else 2000 + 10 * p  # warm-up steps are slower and skipped

    path = str(tmp_path / "run_kernel_trace.csv")
    _write_trace(path, warmup, k, dur)
    got = bc.trace_durations(path, skip=warmup)
    assert got == pytest.approx([(2000 + 10 * p) / 1e3 for p in range(len(STEP))])
