"""A whole small step (plan, every rank's forward, the merge, a fill of dq and
every rank's no-allocation backward) captured once in a HIP graph and
replayed: the entry points launch kernels only (no allocation, memset or
synchronisation), so the graph must reproduce the eager step bit for bit on
every replay. Between replays the program runs eager work of its own (another
whole step, which also uses the backward's fixed scratch, and a library
matmul) and synchronises; the static inputs are rewritten between replays so
that each replay must read them anew."""
import numpy as np
import pytest
import torch

from block_sparse_cross_amd import binding, inputs
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


def test_captured_step_replays_match_eager():
    w = inputs.Workload("graph", b=2, L=2048, A=8, B=16, hq=32, hkv=8, d=128, dtype="bf16",
                        scale=128 ** -0.5, P=4, m=128)
    s, a = inputs.workload_anchors(w, 3)
    sd, ad = to_dev(s), to_dev(a)
    _, _, bundles, _ = [t.cpu().numpy() for t in
                        binding.splitkv_plan(sd, ad, w.B, w.S, w.m, w.P, w.J)]
    starts = [to_dev(ids.astype(np.int64) * w.m) for ids in bundles]

    def values(seed):
        q, do = to_dev(inputs.gen_q(w, seed)), to_dev(inputs.gen_do(w, seed))
        kv = [(to_dev(inputs.gen_local_kv(w, seed, ids, "k")),
               to_dev(inputs.gen_local_kv(w, seed, ids, "v"))) for ids in bundles]
        return [q, do] + [x for pair in kv for x in pair]

    # every buffer one step touches, allocated up front
    def buffers():
        dev = sd.device
        keys = bundles.shape[1] * w.m
        return dict(
            plan=(torch.empty(w.P * w.J, dtype=torch.int64, device=dev),
                  torch.empty(w.P * w.J, dtype=torch.int32, device=dev),
                  torch.empty((w.P, w.J), dtype=torch.int32, device=dev),
                  torch.empty(w.P, dtype=torch.int64, device=dev)),
            o_parts=torch.empty((w.P, w.Q, w.hq, w.d), dtype=torch.bfloat16, device=dev),
            lse_parts=torch.empty((w.P, w.Q, w.hq), dtype=torch.float32, device=dev),
            o=torch.empty((w.Q, w.hq, w.d), dtype=torch.bfloat16, device=dev),
            lse=torch.empty((w.Q, w.hq), dtype=torch.float32, device=dev),
            dq=torch.empty((w.Q, w.hq, w.d), dtype=torch.float32, device=dev),
            delta=torch.empty((w.Q, w.hq), dtype=torch.float32, device=dev),
            dkv=[(torch.empty((keys, w.hkv, w.d), dtype=torch.bfloat16, device=dev),
                  torch.empty((keys, w.hkv, w.d), dtype=torch.bfloat16, device=dev))
                 for _ in range(w.P)],
            ws=[torch.empty(max(1, binding.splitkv_workspace_bytes(
                binding.SPLITKV_OP_FWD, binding.make_anchors(sd, ad, w.B),
                binding.make_heads(w.hq, w.hkv, w.d, torch.bfloat16),
                binding.make_local(cs, w.m))), dtype=torch.uint8, device=dev)
                for cs in starts])

    def step(vals, buf, stream):
        q, do = vals[0], vals[1]
        binding.splitkv_plan(sd, ad, w.B, w.S, w.m, w.P, w.J, out=buf["plan"], stream=stream)
        for p, cs in enumerate(starts):
            k, v = vals[2 + 2 * p], vals[3 + 2 * p]
            binding.splitkv_attn_fwd(sd, ad, w.B, cs, w.m, q, k, v,
                                     out=(buf["o_parts"][p], buf["lse_parts"][p]),
                                     workspace=buf["ws"][p], stream=stream)
        binding.splitkv_lse_merge(buf["o_parts"], buf["lse_parts"], out=(buf["o"], buf["lse"]),
                                  stream=stream)
        buf["dq"].zero_()                     # a fill kernel, on the current stream
        for p, cs in enumerate(starts):
            k, v = vals[2 + 2 * p], vals[3 + 2 * p]
            binding.splitkv_attn_bwd_noalloc(sd, ad, w.B, cs, w.m, q, k, v, buf["o"], do,
                                             buf["lse"], buf["dq"],
                                             delta=buf["delta"], out=buf["dkv"][p],
                                             stream=stream)

    def outputs(buf):
        out = list(buf["plan"]) + [buf["o_parts"], buf["lse_parts"], buf["o"], buf["lse"],
                                   buf["dq"], buf["delta"]]
        return [x.clone() for x in out + [x for pair in buf["dkv"] for x in pair]]

    def eager(vals):
        buf = buffers()
        step(vals, buf, torch.cuda.current_stream())
        torch.cuda.synchronize()
        return outputs(buf)

    va, vb = values(3), values(4)
    want_a, want_b = eager(va), eager(vb)
    assert not torch.equal(want_a[-1], want_b[-1])

    static = [x.clone() for x in va]
    sbuf = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):             # warm-up off the default stream
        step(static, sbuf, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(static, sbuf, torch.cuda.current_stream())
    torch.cuda.synchronize()

    x = torch.randn(512, 512, device=sd.device)
    for i, (vals, want) in enumerate(((va, want_a), (vb, want_b), (va, want_a), (vb, want_b))):
        for dst, src in zip(static, vals):
            dst.copy_(src)
        for t in list(sbuf["plan"]) + [sbuf[n] for n in ("o_parts", "lse_parts", "o", "lse",
                                                         "dq", "delta")] + \
                [y for pair in sbuf["dkv"] for y in pair]:
            t.fill_(7)                        # stale results must be overwritten
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outputs(sbuf)
        assert len(got) == len(want)
        for j, (g, r) in enumerate(zip(got, want)):
            assert torch.equal(g, r), "replay %d: output %d differs from the eager step" % (i, j)
        # eager work between replays, including another step on the fixed scratch
        other = eager(vb if vals is va else va)
        assert torch.equal(other[-1], (want_b if vals is va else want_a)[-1])
        x = torch.tanh(x @ x) * 0.5
        torch.cuda.synchronize()
