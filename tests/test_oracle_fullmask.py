"""Pins for the oracle's whole-mask composition (Figure 1 and §3.1 of the
Split-KV paper): a block's rows attend the context window [s_i, a_i) and all B
tokens of their own block (bidirectional within the block).

The composition (two partials merged by Eq. 4; backward as the sum of the two
key sets' local backwards with the global lse and Delta) is checked against the
definition written out with library routines: dense masked attention in fp64
torch over the concatenated key sequence (context keys, then the Q block
keys) with the boolean mask of Figure 1, and torch autograd through it.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_amd import inputs


def _case(seed, n_samples=2, L=96, A=3, B=4, hq=4, hkv=2, d=16, empty_window=True):
    g = np.random.default_rng(seed)
    s, a = inputs.random_tiny_anchors(g, n_samples, L, A, prompt=L // 4)
    if empty_window:
        a[0] = s[0]          # a row block with no context keys at all
    N = len(s)
    Q, S = N * B, n_samples * L
    return dict(B=B, s=s, a=a, N=N, Q=Q, S=S, hq=hq, hkv=hkv, d=d,
                q=g.standard_normal((Q, hq, d)), do=g.standard_normal((Q, hq, d)),
                k=g.standard_normal((S, hkv, d)), v=g.standard_normal((S, hkv, d)),
                kb=g.standard_normal((Q, hkv, d)), vb=g.standard_normal((Q, hkv, d)))


def _figure1_mask(c):
    """[Q, S + Q] boolean: context x visible iff s_i <= x < a_i, block key y
    visible iff it lies in the row's own block (i = row // B)."""
    B, Q, S = c["B"], c["Q"], c["S"]
    blk = np.arange(Q) // B
    x = np.arange(S)
    ctx = (x[None, :] >= c["s"][blk][:, None]) & (x[None, :] < c["a"][blk][:, None])
    own = (np.arange(Q)[None, :] // B) == blk[:, None]
    return np.concatenate([ctx, own], axis=1)


def _dense(c, req_grad=False):
    """Masked attention over [context; block] keys in fp64 torch; returns the
    tensors (with grad if asked), the output [Q, hq, d] and lse [Q, hq]."""
    G = c["hq"] // c["hkv"]
    t = {n: torch.tensor(c[n], dtype=torch.float64, requires_grad=req_grad)
         for n in ("q", "k", "v", "kb", "vb")}
    keys = torch.cat([t["k"], t["kb"]], 0).repeat_interleave(G, 1)      # [S+Q, hq, d]
    vals = torch.cat([t["v"], t["vb"]], 0).repeat_interleave(G, 1)
    scale = c["d"] ** -0.5
    z = torch.einsum("qhd,khd->hqk", t["q"], keys) * scale
    mask = torch.from_numpy(_figure1_mask(c))[None]
    z = z.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(z, dim=-1)                                    # [hq, Q]
    p = torch.exp(z - lse[..., None])
    o = torch.einsum("hqk,khd->qhd", p, vals)
    return t, o, lse.transpose(0, 1)


@pytest.mark.parametrize("seed", range(4))
def test_full_mask_forward_matches_dense_masked_attention(seed):
    c = _case(seed)
    o, lse = oracle.full_mask_attn(c["B"], c["s"], c["a"], c["q"], np.arange(c["S"]), c["k"],
                                   c["v"], c["kb"], c["vb"], c["d"] ** -0.5)
    _, o_ref, lse_ref = _dense(c)
    np.testing.assert_allclose(o, o_ref.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref.numpy(), rtol=1e-12, atol=1e-12)
    assert np.all(np.isfinite(lse))   # every row sees its own block


def test_own_block_only_is_block_diagonal_attention():
    """With every context window empty the mask is block diagonal: each block is
    plain (unmasked) attention among its own B tokens."""
    c = _case(7)
    c["a"] = c["s"].copy()
    o, _ = oracle.full_mask_attn(c["B"], c["s"], c["a"], c["q"], np.arange(c["S"]), c["k"],
                                 c["v"], c["kb"], c["vb"], c["d"] ** -0.5)
    B, G = c["B"], c["hq"] // c["hkv"]
    for i in range(c["N"]):
        r = slice(i * B, (i + 1) * B)
        qt = torch.tensor(c["q"][r]).transpose(0, 1)
        kt = torch.tensor(c["kb"][r]).transpose(0, 1).repeat_interleave(G, 0).contiguous()
        vt = torch.tensor(c["vb"][r]).transpose(0, 1).repeat_interleave(G, 0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=c["d"] ** -0.5)
        np.testing.assert_allclose(o[r], ref.transpose(0, 1).numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_full_mask_backward_matches_autograd(seed):
    c = _case(10 + seed)
    t, o_ref, _ = _dense(c, req_grad=True)
    (o_ref * torch.tensor(c["do"])).sum().backward()
    o, lse = oracle.full_mask_attn(c["B"], c["s"], c["a"], c["q"], np.arange(c["S"]), c["k"],
                                   c["v"], c["kb"], c["vb"], c["d"] ** -0.5)
    dq, dk, dv, dkb, dvb = oracle.full_mask_bwd(c["B"], c["s"], c["a"], c["q"], c["do"], o, lse,
                                                np.arange(c["S"]), c["k"], c["v"], c["kb"],
                                                c["vb"], c["d"] ** -0.5)
    for name, got in (("q", dq), ("k", dk), ("v", dv), ("kb", dkb), ("vb", dvb)):
        np.testing.assert_allclose(got, t[name].grad.numpy(), rtol=1e-9, atol=1e-11,
                                   err_msg="d" + name)


def test_own_block_windows():
    s, a, pos = oracle.own_block_windows(3, 16)
    assert s.tolist() == [0, 16, 32] and a.tolist() == [16, 32, 48]
    assert pos.tolist() == list(range(48))
