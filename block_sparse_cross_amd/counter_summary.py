"""Matrix-core and LDS counter summary of the attention kernels at the
strong-scaling share, from three `rocprofv3 --pmc` runs of `bench.py` (two
passes of matrix-core and instruction counters, one of LDS counters) and the
bench line one of them printed (for the plan's live pairs).

    python -m block_sparse_cross_amd.counter_summary PASS_A_DIR PASS_B_DIR LDS_DIR BENCH_LOG [--out FILE]
    python -m block_sparse_cross_amd.counter_summary --trace TRACE_DIR

The second form prints the per-kernel table of a `rocprofv3 --kernel-trace --stats`
run (its kernel_stats.csv: calls, total, average, min and max time in
microseconds, share of GPU time), as the kernel-trace profiles show it.

Per kernel, means over its dispatches: the clock (GRBM_GUI_ACTIVE per XCD over
the dispatch time), matrix-core busy (SQ_VALU_MFMA_BUSY_CYCLES over clock cycles
x 1024 SIMDs), executed FLOPs (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) against the
FLOPs the kernel is credited with (4, 8 and 2 d-contractions of 2 d hq FLOPs per
live pair for the forward, dK/dV and dq-from-dS kernels), the instruction mix,
and the LDS conflict and wait shares.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import json
import os
import re
import sys

# d-contractions per live pair credited to (and executed by) each kernel
CREDIT = {"attn_fwd_bf16_kernel": 4, "attn_bwd_dkdv_kernel": 8, "attn_bwd_dq_ds_kernel": 2}
N_XCD, N_SIMD = 8, 1024
PEAK_TFLOPS = 2500.0
PASS_A = ("SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS "
          "SQ_WAIT_INST_ANY SQ_BUSY_CU_CYCLES")
PASS_B = ("SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_WAVE_CYCLES SQ_ACTIVE_INST_LDS "
          "SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VALU SQ_INSTS_SALU GRBM_GUI_ACTIVE")
PASS_LDS = ("SQ_LDS_BANK_CONFLICT SQ_LDS_ADDR_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS "
            "SQ_LDS_DATA_FIFO_FULL SQ_WAIT_ANY SQ_WAVE_CYCLES GRBM_GUI_ACTIVE")
SELECT = '--kernel-include-regex "attn_fwd_bf16|attn_bwd_dkdv|attn_bwd_dq|lse_merge"'
SELECT_LDS = '--kernel-include-regex "attn_fwd_bf16|attn_bwd_dkdv|attn_bwd_dq|gemm_bf16"'
RUN = "-o run -- python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline"


def load(d: str):
    """Per kernel: counter -> values over dispatches, and dispatch times (us)."""
    counters = collections.defaultdict(lambda: collections.defaultdict(list))
    times = collections.defaultdict(list)
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            m = re.search(r"::(\w+_kernel)", r["Kernel_Name"])
            if not m:
                continue
            k = m.group(1)
            counters[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                times[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return counters, times


def mean(x):
    return sum(x) / len(x)


def summarize(dir_a: str, dir_b: str, dir_lds: str, bench_log: str) -> str:
    a, ta = load(dir_a)
    b, _ = load(dir_b)
    lds, _ = load(dir_lds)
    line = [x for x in open(bench_log) if x.startswith('{"metric"')][-1]
    bench = json.loads(line)
    P = int(re.search(r"P=(\d+) ranks", bench["config"]["workload"]).group(1))
    pairs = bench["config"]["live_pairs_per_head"] / P  # mean live pairs per head per rank
    unit = 2 * 128 * 32 * pairs                          # one d-contraction, FLOPs
    out = ["# Matrix-core counters: attention kernels at the strong-scaling share (strong8)", "",
           "Commands (run from the repository root on one MI355X; two passes of seven SQ "
           "counters and GRBM_GUI_ACTIVE, one LDS pass; one warmup and one timed step, so "
           "every kernel has 2 dispatches per emulated rank; then the summary):", "", "```"]
    for name, ctrs, sel in (("mA", PASS_A, SELECT), ("mB", PASS_B, SELECT), ("lds", PASS_LDS, SELECT_LDS)):
        out.append("timeout -s KILL 240 rocprofv3 --pmc %s %s --output-format csv -d gpurun_out/prof/%s %s "
                   "> gpurun_out/prof/%s.log" % (ctrs, sel, name, RUN, name))
    out += ["python3 -m block_sparse_cross_amd.counter_summary gpurun_out/prof/mA gpurun_out/prof/mB "
            "gpurun_out/prof/lds gpurun_out/prof/mA.log", "```", "",
            "Per dispatch (means over the dispatches). The clock is GRBM_GUI_ACTIVE per XCD over the "
            "dispatch time (8 XCDs); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (clock cycles x 1024 SIMDs); "
            "executed FLOPs = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; credited FLOPs = the mask-live work "
            "each kernel is credited with (4, 8 and 2 d-contractions of 2 d hq FLOPs per live pair for "
            "the forward, dK/dV and dq; dq comes from the dS the dK/dV kernel stores, so the backward "
            "executes exactly its 10 credited contractions), from the plan's mean %.4g live pairs per "
            "head per rank. attn_bwd_dq_kernel, the recomputing dQ kernel, is launched too but exits "
            "at once (every query group is stored)." % pairs, "",
            "| kernel | dispatches | mean time (us) | clock (GHz) | MFMA busy | executed TFLOP (counter) "
            "| credited TFLOP | executed TFLOP/s | credited TFLOP/s | credited % of 2.5 PF | VALU instr "
            "per MFMA | LDS instr per MFMA | VALU co-issued with MFMA | waves waiting on issue |",
            "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    bwd_flops = bwd_us = 0.0
    clocks = {}
    busy_of = {}
    for k, c in CREDIT.items():
        m = {n: mean(x) for n, x in list(a[k].items()) + list(b[k].items())}
        us = mean(ta[k])
        cyc = m["GRBM_GUI_ACTIVE"] / N_XCD
        clk = cyc / (us * 1e-6) / 1e9
        busy = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_SIMD)
        executed = m["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        credited = c / 2 * unit
        clocks[k], busy_of[k] = clk, busy
        if k != "attn_fwd_bf16_kernel":
            bwd_flops += credited
            bwd_us += us
        out.append("| %s | %d | %.0f | %.2f | %.1f%% | %.3f | %.3f | %.0f | %.0f | %.1f%% | %.2f | %.2f | "
                   "%.1f%% | %.1f%% |" % (
                       k, len(ta[k]), us, clk, 100 * busy, executed / 1e12, credited / 1e12,
                       executed / (us * 1e-6) / 1e12, credited / (us * 1e-6) / 1e12,
                       100 * credited / (us * 1e-6) / 1e12 / PEAK_TFLOPS,
                       m["SQ_INSTS_VALU"] / m["SQ_INSTS_MFMA"], m["SQ_INSTS_LDS"] / m["SQ_INSTS_MFMA"],
                       100 * m["SQ_VALU_MFMA_COEXEC_CYCLES"] / m["SQ_VALU_MFMA_BUSY_CYCLES"],
                       100 * m["SQ_WAIT_INST_ANY"] / m["SQ_WAVE_CYCLES"]))
    bw = bwd_flops / (bwd_us * 1e-6) / 1e12
    out += ["", "Backward (dK/dV + dq kernels of one call): %.0f credited TFLOP/s = %.1f%% of the bf16 "
            "peak." % (bw, 100 * bw / PEAK_TFLOPS), "",
            "Reading: the dK/dV kernel runs at a lower clock than without the dS stores (%.2f GHz here; "
            "2.16-2.19 GHz when it stores nothing): writing 2 bytes per pair to HBM adds to the board's "
            "power draw. The dq kernel is bound by streaming the dS (its matrix cores are busy %.0f%% of "
            "the cycles)." % (clocks["attn_bwd_dkdv_kernel"], 100 * busy_of["attn_bwd_dq_ds_kernel"]),
            "", "## LDS pass", "",
            "Per dispatch (means over the dispatches): LDS bank-conflict and address-conflict cycles as a "
            "share of the cycles the LDS was active, waves waiting to issue an LDS instruction and waves "
            "waiting for anything (a dependency, a count or a barrier) as shares of wave cycles, LDS "
            "data-FIFO-full cycles.", "",
            "| kernel | bank conflicts / LDS active | address conflicts / LDS active | waiting on LDS issue "
            "| waiting on anything | LDS FIFO full (cycles) |", "|---|---:|---:|---:|---:|---:|"]
    for k in CREDIT:
        m = {n: mean(x) for n, x in lds[k].items()}
        act = m["SQ_LDS_IDX_ACTIVE"]
        out.append("| %s | %.4f | %.4f | %.1f%% | %.1f%% | %.0f |" % (
            k, m["SQ_LDS_BANK_CONFLICT"] / act, m["SQ_LDS_ADDR_CONFLICT"] / act,
            100 * m["SQ_WAIT_INST_LDS"] / m["SQ_WAVE_CYCLES"],
            100 * m["SQ_WAIT_ANY"] / m["SQ_WAVE_CYCLES"], m["SQ_LDS_DATA_FIFO_FULL"]))
    return "\n".join(out) + "\n"


def strip_params(name: str) -> str:
    """A kernel's name without its trailing parameter list."""
    depth = 0
    for i in range(len(name) - 1, -1, -1):
        if name[i] == ")":
            depth += 1
        elif name[i] == "(":
            depth -= 1
            if depth == 0:
                return name[:i]
    return name


def trace_table(d: str) -> str:
    """The kernel_stats.csv of a kernel-trace run as a markdown table, by total time."""
    f = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)[0]
    rows = sorted(csv.DictReader(open(f)), key=lambda r: -float(r["TotalDurationNs"]))
    out = ["| kernel | calls | total (us) | average (us) | min (us) | max (us) | % of GPU time |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = strip_params(re.sub(r"^void ", "", r["Name"].replace("(anonymous namespace)::", "")))
        name = name[len("splitkv::"):] if name.startswith("splitkv::") else name
        out.append("| %s | %s | %.1f | %.1f | %.1f | %.1f | %.2f |" % (
            name, r["Calls"], float(r["TotalDurationNs"]) / 1e3, float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return "\n".join(out) + "\n"


def main(argv=None) -> int:
    argv = sys.argv[1:] if argv is None else argv
    if argv and argv[0] == "--trace":
        sys.stdout.write(trace_table(argv[1]))
        return 0
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("pass_a")
    ap.add_argument("pass_b")
    ap.add_argument("lds")
    ap.add_argument("bench_log")
    ap.add_argument("--out", default="")
    args = ap.parse_args(argv)
    text = summarize(args.pass_a, args.pass_b, args.lds, args.bench_log)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    else:
        sys.stdout.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
