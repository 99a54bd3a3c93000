"""GPU parity of Eq. 4 in its per-rank halves (LSE reduction, then each rank's
rescaled partial) and of Delta accumulated over ranks, against the oracle; and
the whole per-rank protocol at the weak-scaling share: its outputs agree with
the one-kernel merge and the o-given backward."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_amd import binding, inputs
from tests.helpers import (assert_close_bf16, assert_close_f32, assert_lse, to_dev, to_f64,
                           vals64)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("P,rows", [(1, 1000), (3, 4097), (8, 8192), (64, 333)])
def test_lse_reduce(P, rows):
    _, lp = inputs.gen_partials(P, rows, 8, seed=P, dtype="fp32")
    got = to_f64(binding.splitkv_lse_reduce(to_dev(lp)))
    assert_lse(got, oracle.lse_reduce(lp.astype(np.float64)), tol=1e-5)


@pytest.mark.parametrize("din,dout", [("bf16", torch.bfloat16), ("bf16", torch.float32),
                                      ("fp32", torch.float32), ("fp32", torch.bfloat16)])
@pytest.mark.parametrize("d", [64, 128, 8])
def test_rescale(din, dout, d):
    P, rows = 4, 3001
    o, lp = inputs.gen_partials(P, rows, d, seed=d + P, dtype=din)
    lse = oracle.lse_reduce(lp.astype(np.float64))
    lse_d = to_dev(lse.astype(np.float32))
    for p in range(P):
        got = to_f64(binding.splitkv_lse_rescale(to_dev(o[p]), to_dev(lp[p]), lse_d,
                                                 out_dtype=dout))
        ref = oracle.lse_rescale(vals64(o[p]), lp[p].astype(np.float64),
                                 lse.astype(np.float32).astype(np.float64))
        empty = np.isneginf(lp[p])
        assert (got[empty] == 0).all()
        if dout == torch.float32 and din == "fp32":
            assert_close_f32(got, ref, "rescale")
        else:
            assert_close_bf16(got, ref, "rescale")


def test_rescale_in_place_and_sum_equals_merge():
    P, rows, d = 6, 5000, 128
    o, lp = inputs.gen_partials(P, rows, d, seed=5, dtype="fp32")
    od, ld = to_dev(o), to_dev(lp)
    om, lm = binding.splitkv_lse_merge(od, ld)
    lse = binding.splitkv_lse_reduce(ld)
    for p in range(P):
        binding.splitkv_lse_rescale(od[p], ld[p], lse, out=od[p])  # in place
    torch.cuda.synchronize()
    assert_lse(to_f64(lse), to_f64(lm), tol=1e-6)
    assert_close_f32(to_f64(od.sum(0)), to_f64(om), "sum of rescaled partials")


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128, 16])
def test_delta_and_accumulate(dt, d):
    rows = 4099
    o, _ = inputs.gen_partials(2, rows, d, seed=31, dtype=dt)
    do, _ = inputs.gen_partials(2, rows, d, seed=32, dtype=dt)
    od, dod = to_dev(o), to_dev(do)
    delta = binding.splitkv_delta(od[0], dod[0])
    binding.splitkv_delta(od[1], dod[1], delta=delta, accumulate=True)
    ref = (oracle.delta(vals64(o[0])[:, None], vals64(do[0])[:, None])
           + oracle.delta(vals64(o[1])[:, None], vals64(do[1])[:, None]))[:, 0]
    got = to_f64(delta)
    scale = np.abs(ref).max()
    assert np.abs(got - ref).max() <= 1e-5 * scale


def test_invalid_arguments_enqueue_nothing():
    dev = "cuda"
    l = torch.zeros(4, dtype=torch.float32, device=dev)
    x24 = torch.zeros((4, 24), dtype=torch.float32, device=dev)
    out = torch.full((4, 24), 7.0, dtype=torch.float32, device=dev)
    with pytest.raises(binding.SplitKVError):
        binding.splitkv_delta(x24, x24, delta=out[:, 0].contiguous())  # d/8 = 3
    # in place with different element types
    st = binding.lib().splitkv_lse_rescale(4, 24, out.data_ptr(), binding.SPLITKV_BF16,
                                           l.data_ptr(), l.data_ptr(), out.data_ptr(),
                                           binding.SPLITKV_FP32, None)
    assert st == binding.SPLITKV_ERR_INVALID_ARG
    # d % 8 != 0
    st = binding.lib().splitkv_lse_rescale(4, 20, x24.data_ptr(), binding.SPLITKV_FP32,
                                           l.data_ptr(), l.data_ptr(), out.data_ptr(),
                                           binding.SPLITKV_FP32, None)
    assert st == binding.SPLITKV_ERR_INVALID_ARG
    st = binding.lib().splitkv_lse_reduce(0, 4, l.data_ptr(), out.data_ptr(), None)
    assert st == binding.SPLITKV_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert (out == 7.0).all()


def test_weak8_per_rank_protocol():
    """All 8 emulated ranks of the weak-scaling share in the per-rank form:
    LSE reduction, each rank's rescaled partial, Delta accumulated from the
    rescaled partials, and each rank's backward with that Delta. Compared with
    the one-kernel merge and the o-given backward (same kernels otherwise),
    and with the oracle on sampled rows of the merged output."""
    w = inputs.WORKLOADS["weak8"]
    s, a = inputs.workload_anchors(w, 0)
    sd, ad = to_dev(s), to_dev(a)
    _, _, bundles, _ = [t.cpu().numpy() for t in binding.splitkv_plan(sd, ad, w.B, w.S, w.m,
                                                                      w.P, w.J)]
    q = to_dev(inputs.gen_q(w, 0))
    do = to_dev(inputs.gen_do(w, 0))
    kv = []
    parts_o, parts_l = [], []
    for p in range(w.P):
        ids = bundles[p]
        k = to_dev(inputs.gen_local_kv(w, 0, ids, "k"))
        v = to_dev(inputs.gen_local_kv(w, 0, ids, "v"))
        cs = to_dev(ids.astype(np.int64) * w.m)
        kv.append((cs, k, v))
        o, l = binding.splitkv_attn_fwd(sd, ad, w.B, cs, w.m, q, k, v, o_dtype=torch.float32)
        parts_o.append(o)
        parts_l.append(l)
    lse = binding.splitkv_lse_reduce(torch.stack(parts_l))
    bars = [binding.splitkv_lse_rescale(parts_o[p], parts_l[p], lse) for p in range(w.P)]
    delta = torch.zeros(lse.shape, dtype=torch.float32, device="cuda")
    for p in range(w.P):
        binding.splitkv_delta(bars[p], do, delta=delta, accumulate=True)
    om, lm = binding.splitkv_lse_merge(torch.stack(parts_o), torch.stack(parts_l))
    osum = torch.stack(bars).sum(0)
    torch.cuda.synchronize()
    assert_lse(to_f64(lse), to_f64(lm), tol=1e-5)
    assert_close_f32(to_f64(osum), to_f64(om), "per-rank sum vs merge")
    d_ref = binding.splitkv_delta(om, do)
    torch.cuda.synchronize()
    dr, dg = to_f64(d_ref), to_f64(delta)
    assert np.abs(dg - dr).max() <= 1e-5 * np.abs(dr).max()
    # backward of one rank: Delta given (o = None) vs o given
    cs, k, v = kv[3]
    dq1 = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    dq2 = torch.zeros_like(dq1)
    r1 = binding.splitkv_attn_bwd(sd, ad, w.B, cs, w.m, q, k, v, None, do, lse, dq1, delta=delta)
    r2 = binding.splitkv_attn_bwd(sd, ad, w.B, cs, w.m, q, k, v, om.to(torch.bfloat16), do, lm,
                                  dq2)
    torch.cuda.synchronize()
    assert_close_bf16(to_f64(dq1), to_f64(dq2), "dq")
    assert_close_bf16(to_f64(r1[0]), to_f64(r2[0]), "dk")
    assert_close_bf16(to_f64(r1[1]), to_f64(r2[1]), "dv")
    # merged output on sampled rows against the unsplit oracle
    rows = np.array([0, 1, 17, 40])
    kg = inputs.gen_kv_rows(w, 0, "k", 0, w.S)
    vg = inputs.gen_kv_rows(w, 0, "v", 0, w.S)
    qn = inputs.gen_q(w, 0)
    o_ref, l_ref = oracle.partial_attn(rows, w.B, s, a, vals64(qn[rows]), np.arange(w.S),
                                       vals64(kg), vals64(vg), w.d ** -0.5)
    assert_lse(to_f64(lse)[rows], l_ref)
    assert_close_bf16(to_f64(osum)[rows], o_ref, "per-rank merged o")
