"""A seeded sweep of random shapes through the partial attention (Eq. 3) and
its backward (Algorithm 1, AttnBwd_p, with dq taken from the stored dS), each
checked on every row and key against the oracle, at the tolerances of the
fixed cases. Each case draws its own mix of block size B, head grouping
(including groups that are not powers of two), head dimension, chunk size
and count, local chunk subset, samples per batch, anchors per sample and
logit scale, so that combinations the fixed cases do not pair up are covered
too (for instance B = 1 with a group of 3, or one sample whose chunks are all
local)."""
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
