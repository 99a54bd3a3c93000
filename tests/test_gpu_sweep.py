"""A seeded sweep of random shapes through the partial attention (Eq. 3) and
its backward (Algorithm 1, AttnBwd_p, with dq taken from the stored dS), each
checked on every row and key against the oracle, at the tolerances of the
fixed cases. Each case draws its own mix of block size B, head grouping
(including groups that are not powers of two), head dimension, chunk size
and count, local chunk subset, samples per batch, anchors per sample and
logit scale, so that combinations the fixed cases do not pair up are covered
too (for instance B = 1 with a group of 3, or one sample whose chunks are all
local). A second sweep runs the whole method on random shapes: the GPU's plan
over P ranks, every rank's forward, the merge and every rank's backward, against
the oracle's unsplit attention over the whole context; a third adds the own-block
keys (the whole mask) and the per-rank form of the merge."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_amd import binding, inputs
from tests.helpers import assert_close_bf16, assert_lse, to_dev, to_f64, vals64
from tests.test_gpu_attn import gpu_fwd, make_case, oracle_fwd

pytestmark = pytest.mark.gpu

N_CASES = 24


def draw(i):
    """Parameters of sweep case i (seeded by i alone)."""
    g = np.random.default_rng(9000 + i)
    hq, hkv = [(2, 1), (4, 1), (4, 4), (6, 2), (8, 2), (12, 4), (16, 2), (32, 8)][g.integers(8)]
    m = int(g.choice([8, 16, 33, 64, 96, 200]))
    n_chunks = int(g.integers(1, 17))
    n_samples = int(g.choice([s for s in (1, 2, 3, 4) if (m * n_chunks) % s == 0]))
    L = m * n_chunks // n_samples
    A = int(min(g.choice([1, 6, 16, 40]), (L - L // 4)))
    return dict(B=int(g.choice([1, 3, 7, 16, 24])), hq=hq, hkv=hkv, d=int(g.choice([64, 128])),
                m=m, n_chunks=n_chunks, J=int(g.integers(1, n_chunks + 1)), n_samples=n_samples,
                A=max(A, 1), scale_vals=None if g.random() < 0.75 else 1.0,
                empty_block=bool(g.random() < 0.5))


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_fwd_and_bwd(i):
    p = draw(i)
    print("sweep case", i, p, flush=True)
    c = make_case(9100 + i, **p)
    Q = c["q"].shape[0]
    # forward of the local partial
    o, lse = gpu_fwd(c)
    o_ref, l_ref = oracle_fwd(c)
    assert_lse(lse, l_ref)
    assert_close_bf16(o, o_ref, "o_p")
    # backward with the global lse and o of the whole context
    o_full, l_full = oracle.partial_attn(np.arange(Q), c["B"], c["s"], c["a"], vals64(c["q"]),
                                         np.arange(c["S"]), vals64(c["kg"]), vals64(c["vg"]),
                                         c["d"] ** -0.5)
    o_bf = inputs.f32_to_bf16_bits(o_full.astype(np.float32))
    lse32 = l_full.astype(np.float32)
    dl = oracle.delta(vals64(o_bf), vals64(c["do"]))
    sd, ad = to_dev(c["s"]), to_dev(c["a"])
    cs = to_dev(c["chunk_ids"].astype(np.int64) * c["m"])
    ws = binding.bwd_workspace(sd, ad, c["B"], cs, c["m"], c["hq"], c["hkv"], c["d"],
                               torch.bfloat16)
    dq = torch.zeros(c["q"].shape, dtype=torch.float32, device="cuda")
    dk, dv, delta = binding.splitkv_attn_bwd(sd, ad, c["B"], cs, c["m"], to_dev(c["q"]),
                                             to_dev(c["k"]), to_dev(c["v"]), to_dev(o_bf),
                                             to_dev(c["do"]), to_dev(lse32), dq, workspace=ws)
    torch.cuda.synchronize()
    dq_ref, dk_ref, dv_ref = oracle.attn_bwd(c["B"], c["s"], c["a"], vals64(c["q"]),
                                             vals64(c["do"]), lse32.astype(np.float64), dl,
                                             c["pos"], vals64(c["k"]), vals64(c["v"]),
                                             c["d"] ** -0.5, np.arange(Q),
                                             np.arange(len(c["pos"])))
    np.testing.assert_allclose(to_f64(delta), dl, rtol=1e-4, atol=1e-6)
    assert_close_bf16(to_f64(dq), dq_ref, "dq")
    assert_close_bf16(to_f64(dk), dk_ref, "dk")
    assert_close_bf16(to_f64(dv), dv_ref, "dv")


N_PROTOCOL = 12


def draw_protocol(i):
    """Parameters of whole-protocol case i: P ranks of J chunks of m positions."""
    g = np.random.default_rng(9500 + i)
    P, J = int(g.choice([2, 3, 4, 8])), int(g.integers(1, 5))
    m = int(g.choice([16, 33, 64, 128]))
    hq, hkv = [(4, 1), (6, 2), (8, 2), (32, 8)][g.integers(4)]
    n_chunks = P * J
    n_samples = int(g.choice([s for s in (1, 2, 3, 4) if (m * n_chunks) % s == 0]))
    L = m * n_chunks // n_samples
    A = int(min(g.choice([2, 6, 16]), L - L // 4))
    return P, J, dict(B=int(g.choice([1, 5, 16])), hq=hq, hkv=hkv, d=int(g.choice([64, 128])),
                      m=m, n_chunks=n_chunks, J=n_chunks, n_samples=n_samples, A=A,
                      empty_block=bool(g.random() < 0.5))


@pytest.mark.parametrize("i", range(N_PROTOCOL))
def test_sweep_whole_protocol(i):
    """The method end to end on one GPU: the GPU's plan (Eq. 6, LPT) splits the
    context into P bundles of J chunks; every rank's partial forward (Eq. 3),
    merged (Eq. 4), equals the unsplit attention over the whole context, and
    every rank's backward (Algorithm 1, given the global o and lse) sums to the
    unsplit dq and, put back at each key's place, gives the unsplit dk and dv."""
    P, J, p = draw_protocol(i)
    print("protocol case", i, "P", P, "J", J, p, flush=True)
    c = make_case(9600 + i, **p)
    Q, S, m = c["q"].shape[0], c["S"], c["m"]
    sd, ad = to_dev(c["s"]), to_dev(c["a"])
    _, _, bundles, _ = [t.cpu().numpy() for t in binding.splitkv_plan(sd, ad, c["B"], S, m, P, J)]
    assert sorted(bundles.ravel().tolist()) == list(range(P * J))
    qd, dod = to_dev(c["q"]), to_dev(c["do"])
    ranks = []
    for ids in bundles:
        pos = oracle.local_key_positions(ids.astype(np.int64), m)
        ranks.append((pos, to_dev(ids.astype(np.int64) * m), to_dev(c["kg"][pos]),
                      to_dev(c["vg"][pos])))
    # forward: every rank's partial, then the merge
    parts = [binding.splitkv_attn_fwd(sd, ad, c["B"], cs, m, qd, k, v) for _, cs, k, v in ranks]
    om, lm = binding.splitkv_lse_merge(torch.stack([x[0] for x in parts]),
                                       torch.stack([x[1] for x in parts]))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.partial_attn(np.arange(Q), c["B"], c["s"], c["a"], vals64(c["q"]),
                                       np.arange(S), vals64(c["kg"]), vals64(c["vg"]),
                                       c["d"] ** -0.5)
    assert_lse(to_f64(lm), l_ref, "merged lse")
    assert_close_bf16(to_f64(om), o_ref, "merged o")
    # backward of every rank from the global o and lse; dq summed, dk and dv placed
    o_bf = inputs.f32_to_bf16_bits(o_ref.astype(np.float32))
    lse32 = l_ref.astype(np.float32)
    od, ld = to_dev(o_bf), to_dev(lse32)
    dq = torch.zeros(c["q"].shape, dtype=torch.float32, device="cuda")
    dk = np.zeros(c["kg"].shape, dtype=np.float64)
    dv = np.zeros(c["vg"].shape, dtype=np.float64)
    for pos, cs, k, v in ranks:
        ws = binding.bwd_workspace(sd, ad, c["B"], cs, m, c["hq"], c["hkv"], c["d"],
                                   torch.bfloat16)
        dk_p, dv_p, _ = binding.splitkv_attn_bwd(sd, ad, c["B"], cs, m, qd, k, v, od, dod, ld,
                                                 dq, workspace=ws)
        torch.cuda.synchronize()
        dk[pos], dv[pos] = to_f64(dk_p), to_f64(dv_p)
    dl = oracle.delta(vals64(o_bf), vals64(c["do"]))
    dq_ref, dk_ref, dv_ref = oracle.attn_bwd(c["B"], c["s"], c["a"], vals64(c["q"]),
                                             vals64(c["do"]), lse32.astype(np.float64), dl,
                                             np.arange(S), vals64(c["kg"]), vals64(c["vg"]),
                                             c["d"] ** -0.5, np.arange(Q), np.arange(S))
    assert_close_bf16(to_f64(dq), dq_ref, "dq summed over ranks")
    assert_close_bf16(dk, dk_ref, "dk")
    assert_close_bf16(dv, dv_ref, "dv")


N_FULL_MASK = 8


@pytest.mark.parametrize("i", range(N_FULL_MASK))
def test_sweep_full_mask(i):
    """The whole mask (Figure 1: each block's rows also attend the B tokens of
    their own block) on random shapes: every rank's context partial plus the
    own-block partial, merged over P + 1 partials by the one-kernel merge and
    by the per-rank form (LSE reduction, then each partial rescaled and summed),
    against the oracle's whole-mask attention; the backward of every rank and
    of the own blocks, from the GPU's forward, against the oracle's whole-mask
    backward."""
    P, J, p = draw_protocol(100 + i)
    p.pop("empty_block")
    print("full-mask case", i, "P", P, "J", J, p, flush=True)
    c = make_case(9700 + i, empty_block=False, **p)
    g = np.random.default_rng(9800 + i)
    Q, S, m, B = c["q"].shape[0], c["S"], c["m"], c["B"]
    kb = inputs.normal_values(g, (Q, c["hkv"], c["d"]), c["d"] ** -0.5, "bf16")
    vb = inputs.normal_values(g, (Q, c["hkv"], c["d"]), c["d"] ** -0.5, "bf16")
    sd, ad = to_dev(c["s"]), to_dev(c["a"])
    _, _, bundles, _ = [t.cpu().numpy() for t in binding.splitkv_plan(sd, ad, B, S, m, P, J)]
    qd, dod, kbd, vbd = to_dev(c["q"]), to_dev(c["do"]), to_dev(kb), to_dev(vb)
    bs, ba, bcs, blen = binding.own_block_local(sd, B)
    ranks = []
    for ids in bundles:
        pos = oracle.local_key_positions(ids.astype(np.int64), m)
        ranks.append((pos, to_dev(ids.astype(np.int64) * m), to_dev(c["kg"][pos]),
                      to_dev(c["vg"][pos])))
    parts = [binding.splitkv_attn_fwd(sd, ad, B, cs, m, qd, k, v) for _, cs, k, v in ranks]
    parts.append(binding.splitkv_attn_fwd(bs, ba, B, bcs, blen, qd, kbd, vbd))
    o_parts = torch.stack([x[0] for x in parts])
    l_parts = torch.stack([x[1] for x in parts])
    om, lm = binding.splitkv_lse_merge(o_parts, l_parts)
    # per-rank form: the reduced lse, each partial rescaled to it, summed in fp32
    lr = binding.splitkv_lse_reduce(l_parts)
    o_sum = torch.zeros(c["q"].shape, dtype=torch.float32, device="cuda")
    for x in parts:
        o_sum += binding.splitkv_lse_rescale(x[0], x[1], lr, out_dtype=torch.float32)
    torch.cuda.synchronize()
    scale = c["d"] ** -0.5
    o_ref, l_ref = oracle.full_mask_attn(B, c["s"], c["a"], vals64(c["q"]), np.arange(S),
                                         vals64(c["kg"]), vals64(c["vg"]), vals64(kb),
                                         vals64(vb), scale)
    assert_lse(to_f64(lm), l_ref, "merged lse")
    assert_close_bf16(to_f64(om), o_ref, "merged o")
    assert_lse(to_f64(lr), l_ref, "reduced lse")
    assert_close_bf16(to_f64(o_sum), o_ref, "sum of rescaled partials")
    # backward from the GPU's own forward
    dq = torch.zeros(c["q"].shape, dtype=torch.float32, device="cuda")
    delta = torch.empty((Q, c["hq"]), dtype=torch.float32, device="cuda")
    grads = []
    for r, (_, cs, k, v) in enumerate(ranks):
        ws = binding.bwd_workspace(sd, ad, B, cs, m, c["hq"], c["hkv"], c["d"], torch.bfloat16)
        grads.append(binding.splitkv_attn_bwd(sd, ad, B, cs, m, qd, k, v, om if r == 0 else None,
                                              dod, lm, dq, delta=delta, workspace=ws)[:2])
    ws = binding.bwd_workspace(bs, ba, B, bcs, blen, c["hq"], c["hkv"], c["d"], torch.bfloat16)
    dkb, dvb, _ = binding.splitkv_attn_bwd(bs, ba, B, bcs, blen, qd, kbd, vbd, None, dod, lm, dq,
                                           delta=delta, workspace=ws)
    torch.cuda.synchronize()
    dq_ref, dk_ref, dv_ref, dkb_ref, dvb_ref = oracle.full_mask_bwd(
        B, c["s"], c["a"], vals64(c["q"]), vals64(c["do"]), to_f64(om), to_f64(lm),
        np.arange(S), vals64(c["kg"]), vals64(c["vg"]), vals64(kb), vals64(vb), scale)
    assert_close_bf16(to_f64(dq), dq_ref, "dq")
    for r, (pos, _, _, _) in enumerate(ranks):
        assert_close_bf16(to_f64(grads[r][0]), dk_ref[pos], "dk rank %d" % r)
        assert_close_bf16(to_f64(grads[r][1]), dv_ref[pos], "dv rank %d" % r)
    assert_close_bf16(to_f64(dkb), dkb_ref, "dk (own blocks)")
    assert_close_bf16(to_f64(dvb), dvb_ref, "dv (own blocks)")
