"""Planner study: load balance and planning latency of No balance, Zigzag and the
cost-aware LPT plan, on the GPU, over the load-balancing workloads of the
Split-KV paper's §5.5 (Figures 9 and 10) and a sweep of the chunks per rank J.

Every assignment is computed by the library (`splitkv_plan` for LPT,
`splitkv_plan_baseline` for the two position-based rules), and the LPT bundles
are placed on physical ranks by `splitkv_locality_match` (the step's
all-to-all volume is reported with and without that placement). This module builds
the seeded anchors, times each call with HIP events on the stream it runs on,
and turns the rank loads C_p into the imbalance 100(rho - 1) of §4.2, with
W_p = C_p + D and D = (N/P) B^2.

Workloads (§5.5): b = 4 packed samples, 8k queries per sample (512 anchors of
B = 16), anchors uniform without replacement over each sample's response (the
last three quarters). Context-length study: P = 8, 16k..256k per sample.
CP-size study: 256k per sample, P = 8..64. LPT uses J chunks per rank of
m = S / (P J) positions.

    python -m block_sparse_cross_amd.planner_study [--seeds 3] [--reps 30] [--out FILE]
"""
from __future__ import annotations

import argparse
import json
import statistics
import sys
import time
from typing import Dict, List

import numpy as np
import torch

from . import binding
from . import inputs as I

CONTEXT_LENGTHS = (16384, 32768, 65536, 131072, 262144)
CP_SIZES = (8, 16, 32, 64)
J_SWEEP = (1, 2, 4, 8, 16, 32)


def workload(L: int, P: int, J: int) -> I.Workload:
    return I.Workload("planner", b=4, L=L, A=512, B=16, hq=32, hkv=8, d=128, dtype="bf16",
                      scale=1.0, P=P, m=(4 * L) // (P * J))


def imbalance_pct(load: np.ndarray, n_blocks: int, B: int) -> float:
    P = len(load)
    w = load.astype(np.float64) + n_blocks / P * B * B
    return 100.0 * (w.max() / w.mean() - 1.0)


def _time_call(fn, reps: int) -> float:
    """Median GPU microseconds of one fn() call over reps calls. Each call is
    bracketed by events behind a short spin kernel, so the host has enqueued the
    events and the call before the GPU reaches them: the interval is the
    planner's own kernels, not the host's launch overhead."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000000)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    return statistics.median(times)


def run_case(L: int, P: int, J: int, seed: int, reps: int) -> Dict:
    """Imbalance of the three rules on one seeded draw, and their latencies."""
    w = workload(L, P, J)
    s_np, a_np = I.workload_anchors(w, seed)
    st, ln = I.sample_bounds(w)
    dev = torch.device("cuda")
    s = torch.from_numpy(s_np).to(dev)
    a = torch.from_numpy(a_np).to(dev)
    out = {"L": L, "P": P, "J": J, "m": w.m, "seed": seed}
    i64 = dict(dtype=torch.int64, device=dev)
    nb_out = (torch.empty(P, **i64), torch.empty(P, **i64))
    zz_out = (torch.empty(2 * P * len(st), **i64), torch.empty(P, **i64))
    lpt_out = (torch.empty(P * J, **i64), torch.empty(P * J, dtype=torch.int32, device=dev),
               torch.empty((P, J), dtype=torch.int32, device=dev), torch.empty(P, **i64))
    plans = {
        "no_balance": lambda: binding.splitkv_plan_baseline(
            binding.SPLITKV_BASELINE_NO_BALANCE, s, a, w.B, st, ln, P, out=nb_out),
        "zigzag": lambda: binding.splitkv_plan_baseline(
            binding.SPLITKV_BASELINE_ZIGZAG, s, a, w.B, st, ln, P, out=zz_out),
        "lpt": lambda: binding.splitkv_plan(s, a, w.B, w.S, w.m, P, J, out=lpt_out),
    }
    for name, fn in plans.items():
        res = fn()
        torch.cuda.synchronize()
        load = res[-1].cpu().numpy()
        out[name] = imbalance_pct(load, w.N, w.B)
        out[name + "_us"] = _time_call(fn, reps) if reps > 0 else None
    # the step's all-to-all: context rows that leave their first holder, with
    # LPT bundle p on rank p and with the locality matching of §4.2
    bundles = lpt_out[2]
    match_out = (torch.empty(P, dtype=torch.int32, device=dev),
                 torch.empty((P, P), **i64), torch.empty(2, **i64))
    match = lambda: binding.splitkv_locality_match(bundles, w.m, out=match_out)
    match()
    torch.cuda.synchronize()
    b = bundles.cpu().numpy()
    in_place = int((b // J == np.arange(P)[:, None]).sum()) * w.m
    out["moved_plan_order"] = 100.0 * (w.S - in_place) / w.S
    out["moved_matched"] = 100.0 * int(match_out[2][1].item()) / w.S
    out["match_us"] = _time_call(match, reps) if reps > 0 else None
    return out


def _mean_std(xs: List[float]):
    return float(np.mean(xs)), float(np.std(xs))


def study(seeds: int, reps: int, log=sys.stderr) -> Dict:
    rows = {"context": [], "cp": [], "j_sweep": []}
    cases = ([("context", L, 8, 8) for L in CONTEXT_LENGTHS]
             + [("cp", 262144, P, 8) for P in CP_SIZES]
             + [("j_sweep", 262144, P, J) for P in (8, 64) for J in J_SWEEP])
    for group, L, P, J in cases:
        t0 = time.time()
        per_seed = [run_case(L, P, J, sd, reps if sd == 0 else 0) for sd in range(seeds)]
        row = {"L": L, "P": P, "J": J, "m": per_seed[0]["m"]}
        for k in ("no_balance", "zigzag", "lpt"):
            row[k] = float(np.mean([r[k] for r in per_seed]))
            row[k + "_us"] = per_seed[0][k + "_us"]
        for k in ("moved_plan_order", "moved_matched"):
            row[k] = float(np.mean([r[k] for r in per_seed]))
        row["match_us"] = per_seed[0]["match_us"]
        rows[group].append(row)
        print("planner study: %s L=%d P=%d J=%d done in %.1f s" % (group, L, P, J, time.time() - t0),
              file=log, flush=True)
    summary = {}
    for group in ("context", "cp"):
        for k in ("no_balance", "zigzag", "lpt"):
            summary["%s_%s" % (group, k)] = _mean_std([r[k] for r in rows[group]])
    return {"rows": rows, "summary": summary, "seeds": seeds, "reps": reps,
            "device": torch.cuda.get_device_name(0)}


def to_markdown(res: Dict) -> str:
    out = []
    s = res["summary"]
    out.append("Imbalance 100(rho - 1), mean (std) over the study's configurations; each "
               "configuration is the mean over %d seeded draws.\n" % res["seeds"])
    out.append("| study | No balance | Zigzag | LPT (J = 8) |")
    out.append("|---|---:|---:|---:|")
    for group, label in (("context", "context length 16k-256k, P = 8"),
                         ("cp", "CP size 8-64, 256k")):
        out.append("| %s | %s |" % (label, " | ".join(
            "%.2f (%.2f)" % s["%s_%s" % (group, k)] for k in ("no_balance", "zigzag", "lpt"))))
    out.append("")
    out.append("Per configuration (imbalance %%; median planning latency in us, one call, "
               "HIP events, %d repeats):\n" % res["reps"])
    out.append("| study | per-sample L | P | J | m | No balance | Zigzag | LPT | "
               "No balance us | Zigzag us | LPT us |")
    out.append("|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|")
    for group in ("context", "cp", "j_sweep"):
        for r in res["rows"][group]:
            out.append("| %s | %d | %d | %d | %d | %.2f | %.2f | %.2f | %s | %s | %s |" % (
                group, r["L"], r["P"], r["J"], r["m"], r["no_balance"], r["zigzag"], r["lpt"],
                *["%.1f" % r[k + "_us"] if r[k + "_us"] is not None else "-"
                  for k in ("no_balance", "zigzag", "lpt")]))
    out.append("")
    out.append("LPT's all-to-all (§4.2): context rows that leave the rank first holding them "
               "(rank r holds the r-th contiguous part of the packed context), % of S, with "
               "bundle p on rank p and after the locality matching; GPU time of one "
               "`splitkv_locality_match` call:\n")
    out.append("| study | per-sample L | P | J | moved, plan order | moved, matched | match us |")
    out.append("|---|---:|---:|---:|---:|---:|---:|")
    for group in ("context", "cp", "j_sweep"):
        for r in res["rows"][group]:
            out.append("| %s | %d | %d | %d | %.1f | %.1f | %s |" % (
                group, r["L"], r["P"], r["J"], r["moved_plan_order"], r["moved_matched"],
                "%.1f" % r["match_us"] if r["match_us"] is not None else "-"))
    return "\n".join(out) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--seeds", type=int, default=3)
    ap.add_argument("--reps", type=int, default=30)
    ap.add_argument("--out", default=None, help="write the markdown tables here")
    ap.add_argument("--json", default=None, help="write the raw results here")
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("planner study: needs a GPU", file=sys.stderr)
        return 2
    res = study(args.seeds, args.reps)
    md = to_markdown(res)
    print(md)
    if args.out:
        with open(args.out, "w") as f:
            f.write(md)
    if args.json:
        with open(args.json, "w") as f:
            json.dump(res, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
