"""Benchmark of the Split-KV per-device hot path on one MI355X.

One step = one pass of the whole hot path over one synthetic micro-batch:
  plan (chunk costs + LPT) -> partial attention forward of every emulated rank
  -> LSE merge of the P partials -> backward of every emulated rank (Delta
  computed once from the merged output, dq accumulated over ranks).
  With --merge-form per-rank the merge is done as each rank would do it with
  the partials on different devices: an LSE reduction, each rank rescaling its
  own partial, and Delta accumulated from the rescaled partials.
The rank-local K/V buffers are materialised once before timing (in the real
system that is the per-step all-to-all, outside this path).

Prints one JSON line. `value` = mask-live attention FLOPs (forward 4*d*Hq per
live query-key pair, backward 10*d*Hq) of all ranks per second of step time.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# What decides the machine code and launch shapes of the kernels whose traffic
# is recorded (plan, forward, merge, backward): their sources, the shared
# device header, the compile-time constants of the internal header and the
# build flags. Entry points, declarations and the C header only route calls
# to them. Measured HBM traffic is reported only while this hash matches the
# one recorded with it.
KERNEL_SOURCES = ["block_sparse_cross_amd/csrc/" + f for f in
                  ("attn_bwd.hip", "attn_fwd.hip", "merge.hip", "plan.hip", "common.hpp")] + \
    ["block_sparse_cross_amd/build.py"]
CONSTANT_SOURCES = ["block_sparse_cross_amd/csrc/internal.hpp"]   # only its constexpr lines

# The kernels one call of each entry point launches (names as in a trace).
ENTRY_KERNELS = {
    "splitkv_plan": ["chunk_cost_kernel", "lpt_kernel"],
    "splitkv_attn_fwd": ["block_range_kernel", "attn_fwd_bf16_kernel"],
    "splitkv_lse_merge": ["lse_merge_kernel"],
    "splitkv_lse_reduce": ["lse_reduce_kernel"],
    "splitkv_lse_rescale": ["lse_rescale_kernel"],
    "splitkv_delta": ["delta_rows_kernel"],
    "splitkv_attn_bwd": ["block_range_kernel", "bwd_prep", "chunk_range_kernel",
                         "ds_offsets_kernel", "attn_bwd_dkdv_kernel", "attn_bwd_dq_kernel",
                         "attn_bwd_dq_ds_kernel"],
}
COPY_CALIBRATION_BYTES = 1 << 30   # the --copy-calibration device copy


def sources_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(f.encode())
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    for f in CONSTANT_SOURCES:
        h.update(f.encode())
        with open(os.path.join(ROOT, f)) as fh:
            for line in fh:
                if "constexpr" in line:
                    h.update(line.encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """Per-launch HBM traffic recorded under profiles/ for this workload, if it
    was taken with the current kernel sources; else None."""
    want = sources_hash()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*traffic*.md"))):
        with open(path) as fh:
            for line in fh:
                if line.startswith("traffic-json: "):
                    rec = json.loads(line[len("traffic-json: "):])
                    if rec.get("workload") == workload and rec.get("sources_sha256") == want:
                        return rec
    return None


def summarize_counters(fetch_dir: str, write_dir: str, workload: str, command: str) -> str:
    """Markdown summary of two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE,
    KiB per dispatch) of `bench.py --copy-calibration`: each counter is scaled by
    what it reads for the 1 GiB device copy, then summed over the kernels of one
    call of each entry point."""
    import csv

    def per_kernel(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r["Counter_Name"] == counter:
                        vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    out = {}
    factors = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = per_kernel(d, counter)
        copies = [v for name, vs in vals.items() if "copyBuffer" in name for v in vs]
        big = max(copies) if copies else 0.0
        if big <= 0:
            raise SystemExit("no copy dispatch found for %s calibration" % counter)
        factors[counter] = COPY_CALIBRATION_BYTES / (big * 1024.0)
        for key, kernels in ENTRY_KERNELS.items():
            tot, seen = 0.0, False
            for k in kernels:
                ks = [v for name, vs in vals.items() if k in name for v in vs]
                if ks:
                    tot += sum(ks) / len(ks)
                    seen = True
            if seen:  # entry points the profiled run did not call are left out
                out.setdefault(key, {})[counter] = tot * 1024.0 * factors[counter]
    rec = {"workload": workload, "sources_sha256": sources_hash(),
           "calibration": {"fetch_factor": round(factors["FETCH_SIZE"], 4),
                           "write_factor": round(factors["WRITE_SIZE"], 4)},
           "per_launch_bytes": {k: {"fetch": round(v.get("FETCH_SIZE", 0.0)),
                                    "write": round(v.get("WRITE_SIZE", 0.0))}
                                for k, v in out.items()}}
    lines = ["# HBM traffic per call: %s" % workload, "",
             "Commands (run from the repository root on one MI355X, one counter per pass):", "",
             "```", command, "```", "",
             "Each counter is scaled by the factor that makes the 1 GiB device copy of "
             "`--copy-calibration` read (FETCH_SIZE) and write (WRITE_SIZE) 1 GiB: "
             "fetch x%.4f, write x%.4f. Figures are per call of the entry point (the mean "
             "per dispatch of each of its kernels, summed)." % (factors["FETCH_SIZE"],
                                                                factors["WRITE_SIZE"]), "",
             "| entry point | fetch (GB) | write (GB) |", "|---|---:|---:|"]
    for k, v in rec["per_launch_bytes"].items():
        lines.append("| %s | %.3f | %.3f |" % (k, v["fetch"] / 1e9, v["write"] / 1e9))
    lines += ["", "Kernel sources hash (bench.py reports `roofline.traffic` only while it "
              "matches): `%s`" % rec["sources_sha256"], "", "traffic-json: " + json.dumps(rec)]
    return "\n".join(lines) + "\n"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="strong8 (the default: the largest fwd+bwd share on one GPU), weak8, "
                         "qs4/qs8/qs16/qs32, weak64 or tiny; --layer defaults to weak8")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-blocks", type=int, default=24,
                    help="blocks (of B query rows) in the oracle's timed forward + backward "
                         "sample")
    ap.add_argument("--own-blocks", action="store_true",
                    help="whole mask: also the own-block partial of every block (its B "
                         "block keys), merged with the P context partials and in the backward")
    ap.add_argument("--recompute-dq", action="store_true",
                    help="take dq by recomputing S and dP (the minimum backward workspace) "
                         "instead of from the dS the dK/dV pass stores")
    ap.add_argument("--merge-form", choices=("merged", "per-rank"), default="merged",
                    help="merged: one LSE-merge kernel over the P partials and Delta from the "
                         "merged output; per-rank: the form each rank applies when the partials "
                         "sit on different devices (LSE reduction, each rank rescales its own "
                         "partial, Delta accumulated from the rescaled partials)")
    ap.add_argument("--layer", action="store_true",
                    help="time one whole draft layer instead: QProj, every rank's KeyValueProj, "
                         "attention, the per-rank merge and output projection (Eq. 5), and the "
                         "backward of all of it")
    ap.add_argument("--d-model", type=int, default=5120,
                    help="hidden size H for --layer (Table 2: 5120 for the 32/8/128 drafter)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the traffic summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--command", default="",
                    help="with --summarize-counters: the profiling commands, for the record")
    args = ap.parse_args()
    if args.workload is None:
        args.workload = "weak8" if args.layer else "strong8"
    return args


def main():
    args = parse()
    if args.summarize_counters:
        sys.stdout.write(summarize_counters(args.summarize_counters[0], args.summarize_counters[1],
                                            args.workload, args.command))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)
    if args.layer:
        layer_bench(args)
        return

    import torch
    from block_sparse_cross_amd import binding, inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    w = inputs.WORKLOADS[args.workload]
    seed = args.seed

    def to_dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(
                torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    # ---------------------------------------------------------------- setup
    t_setup = time.time()
    s, a = inputs.workload_anchors(w, seed)
    sd, ad = to_dev(s), to_dev(a)
    q = to_dev(inputs.gen_q(w, seed))
    do = to_dev(inputs.gen_do(w, seed))
    plan_out = binding.splitkv_plan(sd, ad, w.B, w.S, w.m, w.P, w.J)
    torch.cuda.synchronize()
    cost = plan_out[0].cpu().numpy()
    bundles = plan_out[2].cpu().numpy()
    load = plan_out[3].cpu().numpy()
    locs = []
    for p in range(w.P):
        ids = bundles[p]
        k = to_dev(inputs.gen_local_kv(w, seed, ids, "k"))
        v = to_dev(inputs.gen_local_kv(w, seed, ids, "v"))
        locs.append((to_dev(ids.astype(np.int64) * w.m), k, v))
    Q, hq, d = w.Q, w.hq, w.d
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    n_parts = w.P + (1 if args.own_blocks else 0)
    o_parts = torch.empty((n_parts, Q, hq, d), dtype=tdt, device=dev)
    l_parts = torch.empty((n_parts, Q, hq), dtype=torch.float32, device=dev)
    if args.own_blocks:   # block keys/values and the own-block windows
        kb = to_dev(inputs.gen_block_kv(w, seed, "k"))
        vb = to_dev(inputs.gen_block_kv(w, seed, "v"))
        bs, ba, bcs, blen = binding.own_block_local(sd, w.B)
        dkb, dvb = torch.empty_like(kb), torch.empty_like(vb)
    o = torch.empty((Q, hq, d), dtype=tdt, device=dev)
    lse = torch.empty((Q, hq), dtype=torch.float32, device=dev)
    dq = torch.empty((Q, hq, d), dtype=torch.float32, device=dev)
    delta = torch.empty((Q, hq), dtype=torch.float32, device=dev)
    dks = [torch.empty_like(k) for _, k, _ in locs]
    dvs = [torch.empty_like(v) for _, _, v in locs]
    an = binding.make_anchors(sd, ad, w.B)
    hd = binding.make_heads(hq, w.hkv, d, tdt)
    # the backward's workspace holds every rank's dS unless dq is recomputed
    # (one rank at a time: the largest rank's room serves all)
    ds_bytes = 0
    if not args.recompute_dq:
        calls = [(sd, ad, cs, w.m) for cs, _, _ in locs]
        if args.own_blocks:
            calls.append((bs, ba, bcs, blen))
        ds_bytes = max(binding.splitkv_attn_bwd_ds_bytes(s_, a_, w.B, cs_, m_, hq, w.hkv, d, tdt)
                       for s_, a_, cs_, m_ in calls)
    ws_bytes = max(binding.splitkv_workspace_bytes(binding.SPLITKV_OP_FWD, an, hd, None),
                   binding.splitkv_workspace_bytes(binding.SPLITKV_OP_BWD, an, hd, None) +
                   ds_bytes)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    per_rank = args.merge_form == "per-rank"
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    n_ev = 5

    def step(events=None):
        def mark(i):
            if events is not None:
                events[i].record()
        mark(0)
        binding.splitkv_plan(sd, ad, w.B, w.S, w.m, w.P, w.J, out=plan_out)
        mark(1)
        for p, (cs, k, v) in enumerate(locs):
            binding.splitkv_attn_fwd(sd, ad, w.B, cs, w.m, q, k, v,
                                     out=(o_parts[p], l_parts[p]), workspace=ws)
        if args.own_blocks:
            binding.splitkv_attn_fwd(bs, ba, w.B, bcs, blen, q, kb, vb,
                                     out=(o_parts[w.P], l_parts[w.P]), workspace=ws)
        mark(2)
        if per_rank:
            binding.splitkv_lse_reduce(l_parts, out=lse)
            for p in range(n_parts):
                binding.splitkv_lse_rescale(o_parts[p], l_parts[p], lse, out=o_parts[p])
        else:
            binding.splitkv_lse_merge(o_parts, l_parts, out=(o, lse))
        mark(3)
        dq.zero_()
        if per_rank:
            for p in range(n_parts):
                binding.splitkv_delta(o_parts[p], do, delta=delta, accumulate=p > 0)
        for p, (cs, k, v) in enumerate(locs):
            binding.splitkv_attn_bwd(sd, ad, w.B, cs, w.m, q, k, v,
                                     o if p == 0 and not per_rank else None, do,
                                     lse, dq, delta=delta, out=(dks[p], dvs[p]), workspace=ws)
        if args.own_blocks:
            binding.splitkv_attn_bwd(bs, ba, w.B, bcs, blen, q, kb, vb, None, do, lse, dq,
                                     delta=delta, out=(dkb, dvb), workspace=ws)
        mark(4)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[ev() for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    phase = np.zeros(4)
    for e in events:
        for j in range(4):
            phase[j] += e[j].elapsed_time(e[j + 1])
    phase /= args.steps                      # ms per step: plan, fwd (P calls), merge, bwd (P calls)
    ms_step = wall * 1e3 / args.steps
    step_gpu = sorted(e[0].elapsed_time(e[4]) for e in events)   # GPU time of each timed step

    pairs = int(cost.sum())                  # sum over ranks of live (row, key) pairs per head
    D = (w.N // w.P) * w.B * w.B             # own-block pairs per rank (Section 4.2's D)
    if args.own_blocks:
        pairs += w.N * w.B * w.B             # every row also sees its block's B keys
    fwd_flops = 4.0 * d * hq * pairs
    bwd_flops = 10.0 * d * hq * pairs
    value = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12
    fwd_tflops = fwd_flops / (phase[1] * 1e-3) / 1e12
    bwd_tflops = bwd_flops / (phase[3] * 1e-3) / 1e12
    e_in = 2 if tdt == torch.bfloat16 else 4
    rows = Q * hq
    if per_rank:   # LSE reduction, then each partial read and written once (in place)
        merge_bytes = n_parts * rows * 4 + rows * 4 + n_parts * rows * (2 * d * e_in + 8)
    else:
        merge_bytes = n_parts * rows * (d * e_in + 4) + rows * (d * e_in + 4)
    merge_gbs = merge_bytes / (phase[2] * 1e-3) / 1e9
    dominant = "bwd" if phase[3] >= phase[1] else "fwd"
    ach = bwd_tflops if dominant == "bwd" else fwd_tflops
    entry = "splitkv_attn_bwd" if dominant == "bwd" else "splitkv_attn_fwd"
    rec = load_traffic(args.workload + ("+own" if args.own_blocks else ""))
    traffic = None
    if rec is not None and entry in rec["per_launch_bytes"]:
        t = rec["per_launch_bytes"][entry]
        traffic = t["fetch"] + t["write"]

    result = {
        "metric": "mask-live attn fwd+bwd TFLOP/s (% MFMA peak) + LSE-merge GB/s, 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "step_gpu_ms": {"median": round(float(np.median(step_gpu)), 3),
                        "min": round(step_gpu[0], 3)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if tdt == torch.bfloat16 else "fp32",
        "data": "synthetic",
        "config": {
            "workload": "%s: b=%d x L=%d context (S=%d), %d anchors/sample x B=%d (Q=%d), "
                        "Hq/Hkv/d=%d/%d/%d, m=%d, P=%d ranks x J=%d chunks, all ranks "
                        "emulated on one GPU%s" % (w.name, w.b, w.L, w.S, w.A, w.B, Q, hq,
                                                   w.hkv, d, w.m, w.P, w.J,
                                                   ", plus every block's own B keys"
                                                   if args.own_blocks else ""),
            "step": ("plan + fwd(all ranks + own blocks) + merge of P+1 + bwd(all ranks + own "
                     "blocks)" if args.own_blocks else
                     "plan + fwd(all ranks) + merge + bwd(all ranks)"),
            "live_pairs_per_head": pairs,
            "merge_form": args.merge_form,
            "dq": "recomputed (S, dP again)" if args.recompute_dq else
                  "from the dS the dK/dV pass stored (%.2f GB of workspace)" % (ds_bytes / 1e9),
        },
        "fwd_tflops": round(fwd_tflops, 2),
        "bwd_tflops": round(bwd_tflops, 2),
        "fwd_frac_peak": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
        "bwd_frac_peak": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
        "merge_gbs": round(merge_gbs, 1),
        "merge_frac_hbm": round(merge_gbs / PEAK_HBM_GBS, 4),
        "plan_us": round(phase[0] * 1e3, 1),
        "phase_ms": {"plan": round(phase[0], 4), "fwd_all_ranks": round(phase[1], 4),
                     "merge": round(phase[2], 4), "bwd_all_ranks": round(phase[3], 4)},
        "rank_load_max_over_mean": round(float(load.max() / load.mean()), 5),
        # rho with every rank's own blocks added (W_p = C_p + D, Section 4.2)
        "rank_load_max_over_mean_with_D": round(float((load.max() + D) / (load.mean() + D)), 5),
        "roofline": {
            "bound": "mfma",
            "kernel": (("splitkv_attn_bwd (attn_bwd_dkdv_kernel + %s)" %
                        ("attn_bwd_dq_kernel" if args.recompute_dq else "attn_bwd_dq_ds_kernel"))
                       if dominant == "bwd" else "splitkv_attn_fwd (attn_fwd_bf16_kernel)"),
            "per_launch": "one emulated rank's call; achieved = the phase's mask-live FLOPs "
                          "over its measured time (= per-launch FLOPs / mean launch time)",
            "achieved": round(ach, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            # HBM bytes (read + write) per call, from the calibrated counters
            # under profiles/ while they match the current kernel sources
            "traffic": traffic,
        },
        "setup_s": round(setup_s, 1),
    }

    # Context measured on the same box after the timed steps: a dense bf16
    # product through the vendor library and a plain 1 GiB device copy (the
    # ceilings the attention and merge rates can be read against).
    # host side of one plan call (argument checks and two launches, enqueued
    # without waiting), apart from its GPU time above
    torch.cuda.synchronize()
    n_calls = 200
    t0 = time.perf_counter()
    for _ in range(n_calls):
        binding.splitkv_plan(sd, ad, w.B, w.S, w.m, w.P, w.J, out=plan_out)
    result["plan_host_us"] = round((time.perf_counter() - t0) * 1e6 / n_calls, 1)
    torch.cuda.synchronize()

    result["context"] = box_ceilings(torch, dev)
    result["merge_frac_copy"] = round(merge_gbs / result["context"]["device_copy_gbs"], 4)
    # the attention rates against the product loop's rate on random operands
    # (the backward executes the 10 credited d-contractions per pair, or 14
    # when dq recomputes S and dP)
    ceil = result["context"]["mfma_loop_random_bf16_tflops"]
    executed = 1.4 if args.recompute_dq else 1.0
    result["frac_of_mfma_loop"] = {"fwd": round(fwd_tflops / ceil, 4),
                                   "bwd_credited": round(bwd_tflops / ceil, 4),
                                   "bwd_executed": round(bwd_tflops * executed / ceil, 4)}

    if args.copy_calibration:
        x = torch.empty(1 << 29, dtype=torch.float16, device=dev)  # 1 GiB
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        del x, y

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, seed, s, a, bundles, load, q, locs, args)
    print(json.dumps(result), flush=True)


def box_ceilings(torch, dev) -> dict:
    """Dense bf16 8192^3 product (torch.matmul, the vendor library), a 1 GiB
    device-to-device copy and a pure matrix-core loop (libsplitkv_ceiling.so)
    on random and on constant bf16 operands, each the median of 5 timed runs
    after 2 warmups."""
    def med_ms(fn):
        for _ in range(2):
            fn()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]
    n = 8192
    a = torch.randn((n, n), device=dev).to(torch.bfloat16)
    b = torch.randn((n, n), device=dev).to(torch.bfloat16)
    gemm_ms = med_ms(lambda: torch.matmul(a, b))
    del a, b
    x = torch.empty(1 << 29, dtype=torch.float16, device=dev)   # 1 GiB
    y = torch.empty_like(x)
    copy_ms = med_ms(lambda: y.copy_(x))
    del x, y
    mfma = mfma_ceiling_tflops(torch, dev, med_ms)
    return {"dense_bf16_gemm_tflops": round(2.0 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
            "device_copy_gbs": round(2.0 * (1 << 30) / (copy_ms * 1e-3) / 1e9, 1),
            "mfma_loop_random_bf16_tflops": mfma["random"],
            "mfma_loop_constant_bf16_tflops": mfma["constant"],
            "what": "torch.matmul bf16 8192^3; a 1 GiB device copy (read + write bytes); a loop "
                    "of v_mfma_f32_32x32x16_bf16 products alone (2048 workgroups, 8 "
                    "accumulators per wave) on random N(0, 0.05^2) and on constant operands; "
                    "medians of 5 after the timed steps"}


def mfma_ceiling_tflops(torch, dev, med_ms) -> dict:
    """Rate of the matrix-core loop of libsplitkv_ceiling.so (the practical
    product ceiling the attention kernels run against: the board's power limit
    lowers the clock when the products toggle real data)."""
    import ctypes
    from block_sparse_cross_amd import build as B
    if not os.path.exists(B.CEILING_LIB):
        raise RuntimeError("%s is missing: build first (__graft_entry__.build())" % B.CEILING_LIB)
    lib = ctypes.CDLL(B.CEILING_LIB)
    fn = lib.splitkv_ceiling_mfma
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                   ctypes.c_void_p]
    n_wg, iters = 2048, 2000
    flop = float(n_wg) * 4 * iters * 32 * 32768
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    operands = {"random": (torch.randn(8 * 64 * 8, generator=g, device=dev) * 0.05).to(
                    torch.bfloat16),
                "constant": torch.full((8 * 64 * 8,), 0.0078125, device=dev,
                                       dtype=torch.bfloat16)}
    out = torch.empty(n_wg * 256, device=dev)
    res = {}
    for name, fr in operands.items():
        def run():
            rc = fn(ctypes.c_void_p(fr.data_ptr()), iters, n_wg, ctypes.c_void_p(out.data_ptr()),
                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise RuntimeError("splitkv_ceiling_mfma failed: %d" % rc)
        res[name] = round(flop / (med_ms(run) * 1e-3) / 1e12, 1)
    return res


def layer_bench(args):
    """One whole draft layer (forward + backward) per step on one GPU, all ranks emulated."""
    import torch
    from block_sparse_cross_amd import binding, inputs
    from block_sparse_cross_amd.layer import DraftLayer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = inputs.WORKLOADS[args.workload]
    assert w.dtype == "bf16", "--layer runs the bf16 workloads"
    H, seed = args.d_model, args.seed
    nq, nkv = w.hq * w.d, w.hkv * w.d

    def dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(
                torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    t_setup = time.time()
    s, a = inputs.workload_anchors(w, seed)
    sd, ad = dev(s), dev(a)
    plan_out = binding.splitkv_plan(sd, ad, w.B, w.S, w.m, w.P, w.J)
    torch.cuda.synchronize()
    cost = plan_out[0].cpu().numpy()
    bundles = plan_out[2].cpu().numpy()
    X = dev(inputs.gen_matrix(w.Q, H, seed, inputs.T_X, 1.0))
    dY = dev(inputs.gen_matrix(w.Q, H, seed, inputs.T_DY, 1.0))
    Wq = dev(inputs.gen_matrix(nq, H, seed, inputs.T_WQ, H ** -0.5))
    Wk = dev(inputs.gen_matrix(nkv, H, seed, inputs.T_WK, H ** -0.5))
    Wv = dev(inputs.gen_matrix(nkv, H, seed, inputs.T_WV, H ** -0.5))
    Wo = dev(inputs.gen_matrix(H, nq, seed, inputs.T_WO, nq ** -0.5))
    bo = dev(inputs.gen_matrix(1, H, seed, inputs.T_BO, 1.0, dtype="fp32")[0])
    U = [dev(np.concatenate([inputs.gen_matrix(w.m, H, seed, inputs.T_CTX, 1.0,
                                               first_row=int(j) * w.m) for j in b]))
         for b in bundles]
    cs = [dev(b.astype(np.int64) * w.m) for b in bundles]
    layer = DraftLayer(sd, ad, w.B, w.hq, w.hkv, w.d, cs, w.m, Wq, Wk, Wv, Wo, bo,
                       own_blocks=args.own_blocks)
    grads = None
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    def step(events=None):
        nonlocal grads
        if events is not None:
            events[0].record()
        binding.splitkv_plan(sd, ad, w.B, w.S, w.m, w.P, w.J, out=plan_out)
        if events is not None:
            events[1].record()
        layer.forward(X, U)
        if events is not None:
            events[2].record()
        grads = layer.backward(dY, grads)
        if events is not None:
            events[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    phase = np.zeros(3)
    for e in events:
        for j in range(3):
            phase[j] += e[j].elapsed_time(e[j + 1])
    phase /= args.steps
    pairs = int(cost.sum())
    if args.own_blocks:
        pairs += w.N * w.B * w.B                  # every row also sees its block's B keys
    attn_flops = 14.0 * w.d * w.hq * pairs        # credited: 4 forward + 10 backward per pair
    gemm_flops = layer.gemm_flops()
    value = (attn_flops + gemm_flops) / (ms_step * 1e-3) / 1e12
    result = {
        "metric": "draft-layer fwd+bwd TFLOP/s (mask-live attention + projections), 1 MI355X",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": "%s with d_model=%d: Q=%d query rows, S=%d context rows, P=%d ranks x "
                        "J=%d chunks of m=%d, Hq/Hkv/d=%d/%d/%d, all ranks emulated on one GPU%s"
                        % (w.name, H, w.Q, w.S, w.P, w.J, w.m, w.hq, w.hkv, w.d,
                           ", whole mask (plus every block's own B keys)" if args.own_blocks
                           else ""),
            "step": "plan + layer forward (QProj, per-rank KeyValueProj, attention, LSE "
                    "reduction, per-rank rescale and OProj summed with the bias once) + layer "
                    "backward (OProjBwd, Delta, attention backward, QProj/KeyValueProj backward)",
            "live_pairs_per_head": pairs},
        "attn_flops_credited": attn_flops, "gemm_flops": gemm_flops,
        "phase_ms": {"plan": round(phase[0], 4), "layer_fwd": round(phase[1], 4),
                     "layer_bwd": round(phase[2], 4)},
        "roofline": {"bound": "mfma", "kernel": "whole draft layer (attention + projections)",
                     "achieved": round(value, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(result), flush=True)


def cpu_baseline(w, seed, s, a, bundles, load, q, locs, args):
    """The oracle (fp64 C, OpenMP) timed on this host on a bounded sample of the
    same workload: the forward (Eq. 3) and the backward (Algorithm 1: Delta,
    then dq, dk, dv) of a seeded subset of the blocks against the max-loaded
    rank's local keys, FLOPs counted like the GPU's (14 d Hq per live pair)."""
    import oracle
    from block_sparse_cross_amd import inputs

    oracle.lib()
    r = int(np.argmax(load))
    ids = bundles[r]
    pos = oracle.local_key_positions(ids, w.m)
    k = inputs.as_f32(inputs.gen_local_kv(w, seed, ids, "k")).astype(np.float64)
    v = inputs.as_f32(inputs.gen_local_kv(w, seed, ids, "v")).astype(np.float64)
    g = np.random.default_rng(seed + 12345)
    blocks = np.sort(g.choice(w.N, size=min(args.cpu_blocks, w.N), replace=False))
    qs = inputs.as_f32(inputs.gen_q(w, seed, blocks=blocks)).astype(np.float64)
    dos = inputs.as_f32(inputs.gen_do(w, seed, blocks=blocks)).astype(np.float64)
    qs = qs.reshape(len(blocks) * w.B, w.hq, w.d)
    dos = dos.reshape(len(blocks) * w.B, w.hq, w.d)
    sb, ab = s[blocks], a[blocks]                  # the sample as its own set of blocks
    rows = np.arange(len(blocks) * w.B)
    live = int(sum(((pos >= sb[i]) & (pos < ab[i])).sum() for i in range(len(blocks)))) * w.B
    scale = w.d ** -0.5
    t0 = time.perf_counter()
    o, lse = oracle.partial_attn(rows, w.B, sb, ab, qs, pos, k, v, scale)
    dlt = oracle.delta(o, dos)
    oracle.attn_bwd(w.B, sb, ab, qs, dos, lse, dlt, pos, k, v, scale, rows, np.arange(len(pos)))
    dt = time.perf_counter() - t0
    flops = 14.0 * w.d * w.hq * live
    cores = oracle.omp_threads()
    # the oracle's work is proportional to the live pairs it visits, so its time
    # for the max-loaded rank's whole share (every block) and for the whole
    # step (every rank) follows from the sample by that ratio
    rank_pairs = int(load[r])
    all_pairs = int(load.sum())
    # the plan (Eq. 6 + LPT) of the whole workload, and the Eq. 4 merge of the
    # P partials over a sample of rows, bytes counted as for the GPU's merge
    t0 = time.perf_counter()
    oracle.plan(s, a, w.B, w.S, w.m, w.P, w.J)
    plan_ms = (time.perf_counter() - t0) * 1e3
    mrows = 32768
    o_parts = g.standard_normal((w.P, mrows, w.d))
    l_parts = g.standard_normal((w.P, mrows))
    t0 = time.perf_counter()
    oracle.merge(o_parts, l_parts)
    merge_s = time.perf_counter() - t0
    merge_bytes = w.P * mrows * (w.d * 2 + 4) + mrows * (w.d * 2 + 4)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "cpu_model": cpu_model(),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample_live_pairs_per_head": live,
            "extrapolated": {
                "rank_share_s": round(dt * rank_pairs / live, 1),
                "step_s": round(dt * all_pairs / live, 1),
                "how": "measured seconds x (live pairs of rank %d's whole share, or of all %d "
                       "ranks) / live pairs of the sample; labelled as an extrapolation, not "
                       "measured" % (r, w.P)},
            "plan_ms": round(plan_ms, 3),
            "merge_gbs": round(merge_bytes / merge_s / 1e9, 3),
            "merge_sample": "%d partials x %d rows of d=%d (bytes as the GPU's bf16 merge)"
                            % (w.P, mrows, w.d),
            "sample": "fp64 forward (Eq. 3) + backward (Algorithm 1: Delta, dq, dk, dv) of %d "
                      "seeded blocks (%d query rows) x %d heads against rank %d's %d local keys "
                      "(%d live pairs per head); FLOPs counted as 14 d Hq per live pair"
                      % (len(blocks), len(rows), w.hq, r, len(pos), live)}

def cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


if __name__ == "__main__":
    main()
