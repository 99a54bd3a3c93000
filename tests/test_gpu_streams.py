"""Stream order at the C ABI: every entry point enqueues all its kernels on the
stream it is given (and on no other). The inputs of a whole small step (plan,
every rank's forward, the merge, every rank's backward) are produced on a
side stream behind a long spin, and the step is called on that stream; a
kernel launched anywhere else would read the inputs before they exist and
change the result, which must equal the same step run on the default stream
bit for bit (every kernel here is deterministic)."""
import contextlib

import numpy as np
import pytest
import torch

from block_sparse_cross_amd import binding, inputs
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


def run_step(w, sd, ad, q, do, locs, stream=None):
    # torch's own work (stack, zeros) goes to the same stream as the calls
    ctx = torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()
    with ctx:
        plan = binding.splitkv_plan(sd, ad, w.B, w.S, w.m, w.P, w.J, stream=stream)
        parts = [binding.splitkv_attn_fwd(sd, ad, w.B, cs, w.m, q, k, v, stream=stream)
                 for cs, k, v in locs]
        o, lse = binding.splitkv_lse_merge(torch.stack([p[0] for p in parts]),
                                           torch.stack([p[1] for p in parts]), stream=stream)
        dq = torch.zeros((w.Q, w.hq, w.d), dtype=torch.float32, device="cuda")
        grads = [binding.splitkv_attn_bwd(sd, ad, w.B, cs, w.m, q, k, v, o, do, lse, dq,
                                          stream=stream)
                 for cs, k, v in locs]
    return plan, parts, (o, lse), dq, grads


def flat(res):
    plan, parts, merged, dq, grads = res
    out = list(plan) + [x for p in parts for x in p] + list(merged) + [dq]
    out += [x for g in grads for x in g[:2]]
    return out


def test_whole_step_runs_on_the_given_stream():
    w = inputs.Workload("streams", b=2, L=2048, A=8, B=16, hq=32, hkv=8, d=128, dtype="bf16",
                        scale=128 ** -0.5, P=4, m=128)
    s, a = inputs.workload_anchors(w, 3)
    sd, ad = to_dev(s), to_dev(a)
    _, _, bundles, _ = [t.cpu().numpy() for t in
                        binding.splitkv_plan(sd, ad, w.B, w.S, w.m, w.P, w.J)]
    q, do = to_dev(inputs.gen_q(w, 3)), to_dev(inputs.gen_do(w, 3))
    locs = [(to_dev(ids.astype(np.int64) * w.m), to_dev(inputs.gen_local_kv(w, 3, ids, "k")),
             to_dev(inputs.gen_local_kv(w, 3, ids, "v"))) for ids in bundles]
    ref = [x.clone() for x in flat(run_step(w, sd, ad, q, do, locs))]
    torch.cuda.synchronize()

    # the same inputs, written on a side stream only after a long spin
    side = torch.cuda.Stream()
    srcs = [sd, ad, q, do] + [x for loc in locs for x in loc]
    dsts = [torch.zeros_like(x) for x in srcs]
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        torch.cuda._sleep(100_000_000)
        for dst, src in zip(dsts, srcs):
            dst.copy_(src)
    sd2, ad2, q2, do2 = dsts[:4]
    locs2 = [tuple(dsts[4 + 3 * i: 7 + 3 * i]) for i in range(len(locs))]
    got = flat(run_step(w, sd2, ad2, q2, do2, locs2, stream=side))
    side.synchronize()
    torch.cuda.synchronize()
    assert len(got) == len(ref)
    for i, (x, y) in enumerate(zip(got, ref)):
        assert torch.equal(x, y), "output %d differs from the default-stream step" % i
