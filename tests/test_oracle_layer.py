"""Pin of the oracle's draft-layer composition (Algorithm 1 with Eq. 3-5 in
Split-KV form, forward and backward) against torch fp64 autograd of the same
layer on ONE device: dense masked attention over the whole context, one
output projection of the merged output. Nothing of the split, the LSE merge or
the per-rank output projection (Eq. 5) appears in the reference, so the pin
checks all of them and the gradient flow through every projection."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_amd import inputs


def dense_layer(X, U, Wq, Wk, Wv, Wo, bo, s, a, B, hq, hkv, d, scale, own_blocks=False):
    """Keys are the context rows U (and, for the whole mask, the query rows X
    after them); row r of block i sees context positions [s_i, a_i) and, with
    own_blocks, the B rows of its own block (Figure 1)."""
    Q, S = X.shape[0], U.shape[0]
    G = hq // hkv
    KV = torch.cat([U, X], 0) if own_blocks else U
    n = KV.shape[0]
    q = (X @ Wq.T).view(Q, hq, d).transpose(0, 1)                 # [hq, Q, d]
    k = (KV @ Wk.T).view(n, hkv, d).transpose(0, 1).repeat_interleave(G, 0)
    v = (KV @ Wv.T).view(n, hkv, d).transpose(0, 1).repeat_interleave(G, 0)
    blk = torch.arange(Q) // B
    x = torch.arange(n)
    mask = (x[None, :] >= s[blk][:, None]) & (x[None, :] < a[blk][:, None])   # [Q, n]
    if own_blocks:
        mask |= (x[None, :] >= S + blk[:, None] * B) & (x[None, :] < S + (blk[:, None] + 1) * B)
    z = (q @ k.transpose(1, 2)) * scale
    z = z.masked_fill(~mask[None], float("-inf"))
    p = torch.softmax(z, dim=-1)
    o = (p @ v).transpose(0, 1).reshape(Q, hq * d)
    return o @ Wo.T + bo


def make_case(seed, P=4, J=2, m=16, B=4, hq=4, hkv=2, d=16, H=24):
    g = np.random.default_rng(seed)
    S = P * J * m
    s, a = inputs.random_tiny_anchors(g, n_samples=2, L=S // 2, A=3, prompt=6)
    Q = len(s) * B
    mats = {"X": (Q, H), "U": (S, H), "Wq": (hq * d, H), "Wk": (hkv * d, H),
            "Wv": (hkv * d, H), "Wo": (H, hq * d), "dY": (Q, H)}
    vals = {k: g.standard_normal(size=sh) * (1.0 if k in ("X", "U", "dY") else sh[1] ** -0.5)
            for k, sh in mats.items()}
    vals["bo"] = g.standard_normal(size=H)
    bundles = g.permutation(P * J).reshape(P, J)
    bundles.sort(axis=1)
    return s, a, B, hq, hkv, d, m, bundles, vals


@pytest.mark.parametrize("own", [False, True])
@pytest.mark.parametrize("seed", range(4))
def test_split_kv_layer_equals_dense_layer_and_autograd(seed, own):
    s, a, B, hq, hkv, d, m, bundles, v = make_case(seed)
    scale = d ** -0.5
    fwd = oracle.draft_layer_forward(v["X"], v["U"], v["Wq"], v["Wk"], v["Wv"], v["Wo"],
                                     v["bo"], s, a, B, hq, hkv, d, scale, bundles, m,
                                     own_blocks=own)
    bwd = oracle.draft_layer_backward(fwd, v["dY"], v["X"], v["U"], v["Wq"], v["Wk"], v["Wv"],
                                      v["Wo"], s, a, B, hq, hkv, d, scale)
    T = {k: torch.tensor(x, dtype=torch.float64, requires_grad=k != "dY") for k, x in v.items()}
    Y = dense_layer(T["X"], T["U"], T["Wq"], T["Wk"], T["Wv"], T["Wo"], T["bo"],
                    torch.tensor(s), torch.tensor(a), B, hq, hkv, d, scale, own_blocks=own)
    (Y * T["dY"]).sum().backward()
    np.testing.assert_allclose(fwd["Y"], Y.detach().numpy(), rtol=0, atol=1e-11)
    for ours, name in (("dX", "X"), ("dU", "U"), ("dWq", "Wq"), ("dWk", "Wk"), ("dWv", "Wv"),
                       ("dWo", "Wo"), ("dbo", "bo")):
        np.testing.assert_allclose(bwd[ours], T[name].grad.numpy(), rtol=0, atol=1e-10,
                                   err_msg=ours)


def test_eq5_bias_added_once():
    # with zero weights everywhere but the bias, Y is the bias (not P times it)
    s, a, B, hq, hkv, d, m, bundles, v = make_case(11)
    fwd = oracle.draft_layer_forward(v["X"], v["U"], v["Wq"], v["Wk"], v["Wv"],
                                     np.zeros_like(v["Wo"]), v["bo"], s, a, B, hq, hkv, d,
                                     d ** -0.5, bundles, m)
    np.testing.assert_array_equal(fwd["Y"], np.broadcast_to(v["bo"], fwd["Y"].shape))
