"""Board power and clocks while the attention calls of the strong-scaling share's
critical rank run back to back: the forward (Eq. 3), the backward with dq from
the stored dS, and the backward recomputing S and dP for dq (Algorithm 1,
AttnBwd_p). Each kind of call loops for a few seconds while the system
management tool (`amd-smi metric -p -c`) is polled from a thread; the median
socket power and the median graphics clock (mean over the chip's graphics
clock domains) over the samples inside the loop are reported with the time per
call and the credited TFLOP/s. It measures why the kernels run below the
matrix cores' spec rate: under this load the board sits at its power limit and
the clock drops accordingly.

    python -m block_sparse_cross_amd.power_study [--seconds 6] [--out FILE]
"""
from __future__ import annotations

import argparse
import re
import statistics
import subprocess
import sys
import threading
import time

import numpy as np
import torch

from . import binding
from . import inputs as I

SMI = "amd-smi"


def sample_once() -> tuple:
    """(socket power W, mean graphics clock MHz) from one amd-smi query, or None."""
    try:
        out = subprocess.run([SMI, "metric", "-p", "-c", "-g", "0"], capture_output=True,
                             text=True, timeout=5).stdout
    except (OSError, subprocess.TimeoutExpired):
        return None
    p = re.search(r"SOCKET_POWER: (\d+) W", out)
    clocks = [int(x) for x in re.findall(r"GFX_\d+:\s+CLK: (\d+) MHz", out)]
    if not p or not clocks:
        return None
    return int(p.group(1)), sum(clocks) / len(clocks)


class Sampler(threading.Thread):
    """Polls sample_once every `period` seconds until stopped."""

    def __init__(self, period: float = 0.25):
        super().__init__(daemon=True)
        self.period, self.samples, self.stop = period, [], threading.Event()

    def run(self):
        while not self.stop.is_set():
            t = time.time()
            s = sample_once()
            if s is not None:
                self.samples.append((t, *s))
            self.stop.wait(self.period)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--seconds", type=float, default=6.0)
    ap.add_argument("--out", default="")
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("power_study needs a GPU", file=sys.stderr)
        return 2
    w = I.WORKLOADS["strong8"]
    dev = "cuda"

    def to_dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(
                torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    s, a = I.workload_anchors(w, 0)
    sd, ad = to_dev(s), to_dev(a)
    q, do = to_dev(I.gen_q(w, 0)), to_dev(I.gen_do(w, 0))
    _, _, bundles, load = [t.cpu().numpy() for t in
                           binding.splitkv_plan(sd, ad, w.B, w.S, w.m, w.P, w.J)]
    r = int(np.argmax(load))
    ids = bundles[r]
    k, v = to_dev(I.gen_local_kv(w, 0, ids, "k")), to_dev(I.gen_local_kv(w, 0, ids, "v"))
    cs = to_dev(ids.astype(np.int64) * w.m)
    ws = binding.bwd_workspace(sd, ad, w.B, cs, w.m, w.hq, w.hkv, w.d, torch.bfloat16)
    ws_min = binding.bwd_workspace(sd, ad, w.B, cs, w.m, w.hq, w.hkv, w.d, torch.bfloat16,
                                   ds_bytes=0)
    o, lse = binding.splitkv_attn_fwd(sd, ad, w.B, cs, w.m, q, k, v, workspace=ws)
    dq = torch.zeros((w.Q, w.hq, w.d), dtype=torch.float32, device=dev)
    pairs = float(load[r])
    calls = {
        "forward": (lambda: binding.splitkv_attn_fwd(sd, ad, w.B, cs, w.m, q, k, v,
                                                     workspace=ws), 4),
        "backward, dq from the stored dS": (lambda: binding.splitkv_attn_bwd(
            sd, ad, w.B, cs, w.m, q, k, v, o, do, lse, dq, workspace=ws), 10),
        "backward, dq recomputed": (lambda: binding.splitkv_attn_bwd(
            sd, ad, w.B, cs, w.m, q, k, v, o, do, lse, dq, workspace=ws_min), 10),
    }
    idle = sample_once()
    rows = []
    for name, (fn, units) in calls.items():
        fn()
        torch.cuda.synchronize()
        smp = Sampler()
        smp.start()
        t0 = time.time()
        n = 0
        while time.time() - t0 < args.seconds:
            for _ in range(4):
                fn()
            n += 4
            torch.cuda.synchronize()
        t1 = time.time()
        smp.stop.set()
        smp.join()
        inside = [x for x in smp.samples if t0 + 0.5 < x[0] < t1 - 0.1]
        ms = 1e3 * (t1 - t0) / n
        rows.append((name, ms, units * w.d * w.hq * pairs / ms / 1e9,
                     statistics.median([x[1] for x in inside]) if inside else float("nan"),
                     statistics.median([x[2] for x in inside]) if inside else float("nan"),
                     len(inside)))
        print("done:", name, flush=True)
    lines = ["Board power and clocks, strong8 critical rank (rank %d), calls back to back for %.0f s "
             "each; medians over the amd-smi samples inside each loop." % (r, args.seconds), "",
             "Idle before the loops: %s W, graphics clock %s MHz." %
             (idle[0] if idle else "n/a", "%.0f" % idle[1] if idle else "n/a"), "",
             "| call | ms per call | credited TFLOP/s | socket power (W) | graphics clock (MHz) | samples |",
             "|---|---:|---:|---:|---:|---:|"]
    for name, ms, tf, pw, clk, ns in rows:
        lines.append("| %s | %.2f | %.0f | %.0f | %.0f | %d |" % (name, ms, tf, pw, clk, ns))
    text = "\n".join(lines) + "\n"
    print(text)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
