"""The whole block-sparse mask on the GPU (Figure 1 and §3.1 of the Split-KV
paper): every emulated rank's context partial plus the own-block partial (a
block's rows also attend all B tokens of their own block), merged by Eq. 4 over
P + 1 partials; the backward as every rank's call plus the own-block call, dq
accumulated. Compared with the oracle's whole-mask composition, itself pinned
to dense masked attention (tests/test_oracle_fullmask.py)."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_amd import binding, inputs
from helpers import assert_close_bf16, assert_lse, to_dev, to_f64, vals64

pytestmark = pytest.mark.gpu

CASES = [
    dict(),
    dict(d=64),
    dict(hq=6, hkv=2),                    # GQA group of 3
    dict(B=8, A=5, m=64, P=2, J=4),
]


def _case(seed, B=16, hq=8, hkv=2, d=128, m=128, P=4, J=2, n_samples=2, A=6):
    g = np.random.default_rng(seed)
    S = m * P * J
    L = S // n_samples
    s, a = inputs.random_tiny_anchors(g, n_samples, L, A, L // 4)
    a[1] = s[1]                           # one block with no context keys
    N = len(s)
    sv = d ** -0.5
    return dict(s=s, a=a, B=B, m=m, P=P, J=J, S=S, N=N, Q=N * B, hq=hq, hkv=hkv, d=d,
                q=inputs.normal_values(g, (N * B, hq, d), sv, "bf16"),
                do=inputs.normal_values(g, (N * B, hq, d), sv, "bf16"),
                kg=inputs.normal_values(g, (S, hkv, d), sv, "bf16"),
                vg=inputs.normal_values(g, (S, hkv, d), sv, "bf16"),
                kb=inputs.normal_values(g, (N * B, hkv, d), sv, "bf16"),
                vb=inputs.normal_values(g, (N * B, hkv, d), sv, "bf16"))


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_full_mask_forward_merge_backward(idx):
    c = _case(500 + idx, **CASES[idx])
    B, Q, P = c["B"], c["Q"], c["P"]
    sd, ad = to_dev(c["s"]), to_dev(c["a"])
    _, _, bundles, _ = binding.splitkv_plan(sd, ad, B, c["S"], c["m"], P, c["J"])
    bundles = bundles.cpu().numpy()
    q, do = to_dev(c["q"]), to_dev(c["do"])
    kb, vb = to_dev(c["kb"]), to_dev(c["vb"])
    bs, ba, bcs, blen = binding.own_block_local(sd, B)
    ranks = []
    for p in range(P):
        pos = oracle.local_key_positions(bundles[p], c["m"])
        ranks.append((pos, to_dev(bundles[p].astype(np.int64) * c["m"]),
                      to_dev(c["kg"][pos]), to_dev(c["vg"][pos])))
    parts = [binding.splitkv_attn_fwd(sd, ad, B, cs, c["m"], q, k, v) for _, cs, k, v in ranks]
    parts.append(binding.splitkv_attn_fwd(bs, ba, B, bcs, blen, q, kb, vb))
    o, lse = binding.splitkv_lse_merge(torch.stack([x[0] for x in parts]),
                                       torch.stack([x[1] for x in parts]))
    torch.cuda.synchronize()

    scale = c["d"] ** -0.5
    o_ref, lse_ref = oracle.full_mask_attn(B, c["s"], c["a"], vals64(c["q"]), np.arange(c["S"]),
                                           vals64(c["kg"]), vals64(c["vg"]), vals64(c["kb"]),
                                           vals64(c["vb"]), scale)
    assert_close_bf16(to_f64(o), o_ref, "o")
    assert_lse(to_f64(lse), lse_ref)

    # backward with the GPU's own forward outputs (so only the backward is compared)
    dq = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    delta = torch.empty((Q, c["hq"]), dtype=torch.float32, device="cuda")
    grads = []
    for p, (_, cs, k, v) in enumerate(ranks):
        dk, dv, _ = binding.splitkv_attn_bwd(sd, ad, B, cs, c["m"], q, k, v, o if p == 0 else None,
                                             do, lse, dq, delta=delta)
        grads.append((dk, dv))
    dkb, dvb, _ = binding.splitkv_attn_bwd(bs, ba, B, bcs, blen, q, kb, vb, None, do, lse, dq,
                                           delta=delta)
    torch.cuda.synchronize()
    dq_ref, dk_ref, dv_ref, dkb_ref, dvb_ref = oracle.full_mask_bwd(
        B, c["s"], c["a"], vals64(c["q"]), vals64(c["do"]), to_f64(o), to_f64(lse),
        np.arange(c["S"]), vals64(c["kg"]), vals64(c["vg"]), vals64(c["kb"]), vals64(c["vb"]), scale)
    assert_close_bf16(to_f64(dq), dq_ref, "dq")
    for p, (pos, _, _, _) in enumerate(ranks):
        assert_close_bf16(to_f64(grads[p][0]), dk_ref[pos], "dk rank %d" % p)
        assert_close_bf16(to_f64(grads[p][1]), dv_ref[pos], "dv rank %d" % p)
    assert_close_bf16(to_f64(dkb), dkb_ref, "dk (own blocks)")
    assert_close_bf16(to_f64(dvb), dvb_ref, "dv (own blocks)")


def test_own_block_partial_at_full_size_sampled_blocks():
    """The own-block call at the weak-scaling share's shape (Q = 8192 rows, 32/8
    heads, d = 128): forward on every row, checked on sampled blocks; backward
    with synthetic global lse and o, dq and the block keys' gradients checked on
    the same blocks (a block's rows and keys interact only with each other)."""
    w = inputs.WORKLOADS["weak8"]
    s, a = inputs.workload_anchors(w, 0)
    sd = to_dev(s)
    q, do = inputs.gen_q(w, 0), inputs.gen_do(w, 0)
    kb, vb = inputs.gen_block_kv(w, 0, "k"), inputs.gen_block_kv(w, 0, "v")
    bs, ba, bcs, blen = binding.own_block_local(sd, w.B)
    qd, kbd, vbd, dod = to_dev(q), to_dev(kb), to_dev(vb), to_dev(do)
    o_b, l_b = binding.splitkv_attn_fwd(bs, ba, w.B, bcs, blen, qd, kbd, vbd)
    lse = to_dev(inputs.gen_lse_like(w.Q, w.hq, 0, center=3.0))
    o_syn = to_dev(inputs.gen_o_like(w, 0, w.Q))
    dq = torch.zeros(qd.shape, dtype=torch.float32, device="cuda")
    dkb, dvb, delta = binding.splitkv_attn_bwd(bs, ba, w.B, bcs, blen, qd, kbd, vbd, o_syn, dod,
                                               lse, dq)
    torch.cuda.synchronize()
    g = np.random.default_rng(3)
    blocks = np.sort(g.choice(w.N, size=24, replace=False))
    rows = (blocks[:, None] * w.B + np.arange(w.B)[None, :]).reshape(-1)
    scale = w.d ** -0.5
    sb, ab, pb = oracle.own_block_windows(w.N, w.B)
    o_ref, l_ref = oracle.partial_attn(rows, w.B, sb, ab, vals64(q[rows]), pb[rows],
                                       vals64(kb[rows]), vals64(vb[rows]), scale)
    assert_close_bf16(to_f64(o_b)[rows], o_ref, "o (own blocks)")
    assert_lse(to_f64(l_b)[rows], l_ref)
    # backward restricted to the sampled blocks, renumbered 0 .. 23
    nb = len(blocks)
    rs, ra, rp = oracle.own_block_windows(nb, w.B)
    dl = to_f64(delta)[rows]
    dq_ref, dk_ref, dv_ref = oracle.attn_bwd(w.B, rs, ra, vals64(q[rows]), vals64(do[rows]),
                                             to_f64(lse)[rows], dl, rp, vals64(kb[rows]),
                                             vals64(vb[rows]), scale, np.arange(nb * w.B),
                                             np.arange(nb * w.B))
    np.testing.assert_allclose(dl, oracle.delta(vals64(inputs.gen_o_like(w, 0, w.Q)[rows]),
                                                vals64(do[rows])), rtol=1e-4, atol=1e-6)
    assert_close_bf16(to_f64(dq)[rows], dq_ref, "dq (own blocks)")
    assert_close_bf16(to_f64(dkb)[rows], dk_ref, "dk (own blocks)")
    assert_close_bf16(to_f64(dvb)[rows], dv_ref, "dv (own blocks)")


@pytest.mark.parametrize("n,B", [(0, 16), (1, 16), (7, 4), (512, 16), (4096, 16)])
def test_own_block_layout_matches_oracle(n, B):
    """splitkv_own_block_local writes the windows [iB, (i+1)B), chunk start 0
    and segment length n B that the oracle's own-block windows define."""
    s = torch.zeros(n, dtype=torch.int64, device="cuda")
    bs, ba, bcs, blen = binding.own_block_local(s, B)
    torch.cuda.synchronize()
    rs, ra, rp = oracle.own_block_windows(n, B)
    np.testing.assert_array_equal(bs.cpu().numpy(), rs)
    np.testing.assert_array_equal(ba.cpu().numpy(), ra)
    assert bcs.cpu().numpy().tolist() == [0] and blen == n * B == len(rp)
