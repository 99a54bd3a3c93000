"""Pins for the oracle's attention half (Eq. 3 partials, Eq. 4 merge, backward).

The oracle is checked against things other than itself:
  * special cases that reduce to a library routine (dense and causal attention
    = torch's scaled_dot_product_attention in fp64 on the CPU; a general
    anchor mask = SDPA with a boolean mask);
  * closed forms (q = 0 gives lse = log #live and o = mean of the live values;
    two equal partials merge to lse + log 2);
  * the exact identity of Eq. 4 (merging partials over a disjoint split of the
    keys equals the unsplit result);
  * central finite differences and fp64 torch autograd through a split-and-merge
    formulation (the per-partial backward of Algorithm 1) for the gradients.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_amd import inputs


def _sdpa(q, k, v, scale, mask=None, causal=False):
    """q [n, hq, d], k/v [nk, hkv, d] -> [n, hq, d] via torch SDPA (fp64, CPU)."""
    hq, hkv = q.shape[1], k.shape[1]
    G = hq // hkv
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2))).repeat_interleave(G, 0)
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2))).repeat_interleave(G, 0)
    am = None if mask is None else torch.from_numpy(mask)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(),
                                                         attn_mask=am, is_causal=causal,
                                                         scale=scale)
    return o.numpy().transpose(1, 0, 2)


def _rand(g, *shape):
    return g.standard_normal(size=shape)


def test_dense_special_case_matches_sdpa():
    # one chunk covering everything, every window the whole context
    g = np.random.default_rng(1)
    B, N, S, hq, hkv, d = 4, 3, 37, 4, 2, 16
    q, k, v = _rand(g, N * B, hq, d), _rand(g, S, hkv, d), _rand(g, S, hkv, d)
    s, a = np.zeros(N, np.int64), np.full(N, S, np.int64)
    o, lse = oracle.partial_attn(np.arange(N * B), B, s, a, q, np.arange(S), k, v, d ** -0.5)
    ref = _sdpa(q, k, v, d ** -0.5)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    assert np.isfinite(lse).all()


def test_causal_special_case_matches_sdpa():
    # B = 1 and a_r = r + 1: row r attends keys [0, r] -> causal attention
    g = np.random.default_rng(2)
    S, hq, hkv, d = 29, 2, 1, 8
    q, k, v = _rand(g, S, hq, d), _rand(g, S, hkv, d), _rand(g, S, hkv, d)
    s, a = np.zeros(S, np.int64), np.arange(1, S + 1)
    o, _ = oracle.partial_attn(np.arange(S), 1, s, a, q, np.arange(S), k, v, 0.3)
    ref = _sdpa(q, k, v, 0.3, causal=True)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_anchor_mask_matches_sdpa_with_boolean_mask():
    g = np.random.default_rng(3)
    s, a = inputs.random_tiny_anchors(g, n_samples=3, L=40, A=3, prompt=10)
    # plus one block whose window [80, 82) misses every local chunk
    s, a = np.append(s, 80), np.append(a, 82)
    B, hq, hkv, d = 5, 6, 2, 8
    S = 120
    Q = len(s) * B
    q, k, v = _rand(g, Q, hq, d), _rand(g, S, hkv, d), _rand(g, S, hkv, d)
    # a local buffer of 3 non-adjacent chunks of 8 keys, in ascending position
    chunks = [1, 6, 11]
    pos = oracle.local_key_positions(chunks, 8)
    kl, vl = k[pos], v[pos]
    o, lse = oracle.partial_attn(np.arange(Q), B, s, a, q, pos, kl, vl, 0.5)
    blk = np.arange(Q) // B
    mask = (pos[None, :] >= s[blk][:, None]) & (pos[None, :] < a[blk][:, None])
    live = mask.any(axis=1)
    assert live.any() and (~live).any()          # both kinds of rows occur
    ref = _sdpa(q[live], kl, vl, 0.5, mask=mask[live])
    np.testing.assert_allclose(o[live], ref, rtol=1e-12, atol=1e-12)
    assert (o[~live] == 0).all() and np.isneginf(lse[~live]).all()


def test_zero_query_closed_form():
    # q = 0 -> all scores 0: lse = log(#live keys), o = mean of live values
    g = np.random.default_rng(4)
    B, S, hq, hkv, d = 2, 30, 2, 2, 4
    s, a = np.array([0, 0, 10]), np.array([7, 19, 10])     # last window empty
    q = np.zeros((3 * B, hq, d))
    k, v = _rand(g, S, hkv, d), _rand(g, S, hkv, d)
    o, lse = oracle.partial_attn(np.arange(3 * B), B, s, a, q, np.arange(S), k, v, 1.0)
    for r in range(3 * B):
        i = r // B
        n = a[i] - s[i]
        if n == 0:
            assert np.isneginf(lse[r]).all() and (o[r] == 0).all()
            continue
        np.testing.assert_allclose(lse[r], np.log(n), rtol=0, atol=1e-14)
        for h in range(hq):
            np.testing.assert_allclose(o[r, h], v[s[i]:a[i], h].mean(axis=0), atol=1e-14)


def _split_case(seed, B=4, hq=4, hkv=2, d=8, m=8, n_chunks=8):
    g = np.random.default_rng(seed)
    S = m * n_chunks
    s, a = inputs.random_tiny_anchors(g, n_samples=2, L=S // 2, A=4, prompt=4)
    Q = len(s) * B
    q, k, v, do = (_rand(g, Q, hq, d), _rand(g, S, hkv, d), _rand(g, S, hkv, d),
                   _rand(g, Q, hq, d))
    return g, s, a, B, S, m, q, k, v, do


@pytest.mark.parametrize("seed", range(5))
def test_merge_of_disjoint_partials_equals_unsplit(seed):
    g, s, a, B, S, m, q, k, v, _ = _split_case(seed)
    Q = q.shape[0]
    rows = np.arange(Q)
    o_full, l_full = oracle.partial_attn(rows, B, s, a, q, np.arange(S), k, v, 0.35)
    # an arbitrary disjoint split of the chunks over 3 "ranks"
    perm = g.permutation(S // m)
    groups = [sorted(perm[0:2]), sorted(perm[2:5]), sorted(perm[5:])]
    parts_o, parts_l = [], []
    for ch in groups:
        pos = oracle.local_key_positions(ch, m)
        o_p, l_p = oracle.partial_attn(rows, B, s, a, q, pos, k[pos], v[pos], 0.35)
        parts_o.append(o_p.reshape(-1, q.shape[2]))
        parts_l.append(l_p.reshape(-1))
    o_m, l_m = oracle.merge(np.stack(parts_o), np.stack(parts_l))
    live = np.isfinite(l_full.reshape(-1))
    np.testing.assert_allclose(o_m, o_full.reshape(-1, q.shape[2]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_m[live], l_full.reshape(-1)[live], rtol=0, atol=1e-12)
    assert np.isneginf(l_m[~live]).all()


def test_merge_special_cases():
    g = np.random.default_rng(7)
    P, R, d = 5, 33, 8
    o = _rand(g, P, R, d)
    lse = _rand(g, P, R) * 3
    lse[:, 4] = -np.inf
    o[:, 4] = 0
    lse[2, 7] = -np.inf
    o[2, 7] = 0
    # P = 1 is the identity
    o1, l1 = oracle.merge(o[:1], lse[:1])
    np.testing.assert_array_equal(o1, o[0])
    np.testing.assert_array_equal(l1, lse[0])
    # permutation invariance
    om, lm = oracle.merge(o, lse)
    perm = g.permutation(P)
    op, lp = oracle.merge(o[perm], lse[perm])
    np.testing.assert_allclose(op, om, atol=1e-13)
    np.testing.assert_allclose(lp, lm, atol=1e-13)
    # all-empty row -> (0, -inf), no NaN anywhere
    assert np.isneginf(lm[4]) and (om[4] == 0).all()
    assert np.isfinite(om).all()
    # two identical partials: lse + log 2 and the same o
    o2, l2 = oracle.merge(np.stack([o[0], o[0]]), np.stack([lse[0], lse[0]]))
    fin = np.isfinite(lse[0])
    np.testing.assert_allclose(l2[fin], lse[0][fin] + np.log(2.0), atol=1e-14)
    np.testing.assert_allclose(o2, o[0], atol=1e-14)


def _loss_and_grads_fd(s, a, B, S, q, k, v, do, scale, eps=1e-6):
    """Central finite differences of L = <do, o_unsplit> w.r.t. a few entries."""
    Q = q.shape[0]

    def loss(qq, kk, vv):
        o, _ = oracle.partial_attn(np.arange(Q), B, s, a, qq, np.arange(S), kk, vv, scale)
        return float((o * do).sum())

    g = np.random.default_rng(11)
    out = {}
    for name, arr in (("q", q), ("k", k), ("v", v)):
        idx = [tuple(g.integers(0, n) for n in arr.shape) for _ in range(6)]
        vals = []
        for ix in idx:
            ap, am = arr.copy(), arr.copy()
            ap[ix] += eps
            am[ix] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = ap, am
            vals.append((loss(**{"qq": args_p["q"], "kk": args_p["k"], "vv": args_p["v"]}) -
                         loss(**{"qq": args_m["q"], "kk": args_m["k"], "vv": args_m["v"]}))
                        / (2 * eps))
        out[name] = (idx, np.array(vals))
    return out


def _oracle_full_bwd(s, a, B, S, q, k, v, do, scale, key_sel=None, pos=None, kl=None, vl=None):
    Q = q.shape[0]
    o, lse = oracle.partial_attn(np.arange(Q), B, s, a, q, np.arange(S), k, v, scale)
    dl = oracle.delta(o, do)
    if pos is None:
        pos, kl, vl = np.arange(S), k, v
    keys = np.arange(len(pos)) if key_sel is None else key_sel
    return oracle.attn_bwd(B, s, a, q, do, lse, dl, pos, kl, vl, scale, np.arange(Q), keys)


def test_backward_matches_finite_differences():
    g, s, a, B, S, m, q, k, v, do = _split_case(21, d=4, hq=2, hkv=1, m=4, n_chunks=6)
    scale = 0.7
    dq, dk, dv = _oracle_full_bwd(s, a, B, S, q, k, v, do, scale)
    fd = _loss_and_grads_fd(s, a, B, S, q, k, v, do, scale)
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        idx, vals = fd[name]
        got = np.array([grad[ix] for ix in idx])
        np.testing.assert_allclose(got, vals, rtol=1e-6, atol=1e-8), name


def _torch_split_merge(s, a, B, q, k, v, scale, groups, m):
    """Split attention over key groups + Eq. 4 merge, in fp64 torch (autograd)."""
    Q, hq, d = q.shape
    G = hq // k.shape[1]
    blk = torch.arange(Q) // B
    st, en = torch.from_numpy(s)[blk], torch.from_numpy(a)[blk]
    outs, lses = [], []
    for ch in groups:
        pos = torch.from_numpy(oracle.local_key_positions(ch, m))
        kk = k[pos].repeat_interleave(G, 1)           # [n, hq, d]
        vv = v[pos].repeat_interleave(G, 1)
        z = torch.einsum("rhd,nhd->rhn", q, kk) * scale
        live = (pos[None, :] >= st[:, None]) & (pos[None, :] < en[:, None])
        z = z.masked_fill(~live[:, None, :], float("-inf"))
        l = torch.logsumexp(z, dim=-1)                # -inf for empty rows
        p = torch.where(live[:, None, :], torch.exp(z - l[..., None].clamp_min(-1e300)),
                        torch.zeros_like(z))
        outs.append(torch.einsum("rhn,nhd->rhd", p, vv))
        lses.append(l)
    L = torch.stack(lses)                             # [P, Q, hq]
    lmax = L.max(dim=0).values
    safe = torch.where(torch.isfinite(lmax), lmax, torch.zeros_like(lmax))
    w = torch.exp(L - safe)                           # exp(-inf) = 0 for empty partials
    tot = w.sum(dim=0)
    lg = torch.where(tot > 0, safe + torch.log(tot.clamp_min(1e-300)),
                     torch.full_like(tot, float("-inf")))
    o = sum(torch.where(torch.isfinite(lses[p])[..., None],
                        torch.exp(lses[p] - lg.clamp_min(-1e300))[..., None] * outs[p],
                        torch.zeros_like(outs[p])) for p in range(len(groups)))
    return o, lg


@pytest.mark.parametrize("seed", range(3))
def test_backward_matches_torch_autograd_of_split_and_merge(seed):
    """Algorithm 1's backward through MERGE_BWD (per-partial form), computed by
    torch autograd, equals the oracle's global form for every rank's keys."""
    g, s, a, B, S, m, q, k, v, do = _split_case(100 + seed)
    scale = 0.4
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    perm = g.permutation(S // m)
    groups = [sorted(perm[:3]), sorted(perm[3:])]
    o, _ = _torch_split_merge(s, a, B, qt, kt, vt, scale, groups, m)
    (o * torch.from_numpy(do)).sum().backward()
    # oracle: per rank p, the local backward with global lse / Delta; dq summed
    Q = q.shape[0]
    o_full, lse = oracle.partial_attn(np.arange(Q), B, s, a, q, np.arange(S), k, v, scale)
    np.testing.assert_allclose(o_full, o.detach().numpy(), atol=1e-12)
    dl = oracle.delta(o_full, do)
    dq_sum = np.zeros_like(q)
    for ch in groups:
        pos = oracle.local_key_positions(ch, m)
        dq_p, dk_p, dv_p = oracle.attn_bwd(B, s, a, q, do, lse, dl, pos, k[pos], v[pos], scale,
                                           np.arange(Q), np.arange(len(pos)))
        dq_sum += dq_p
        np.testing.assert_allclose(dk_p, kt.grad.numpy()[pos], atol=1e-12)
        np.testing.assert_allclose(dv_p, vt.grad.numpy()[pos], atol=1e-12)
    np.testing.assert_allclose(dq_sum, qt.grad.numpy(), atol=1e-12)


def test_backward_empty_rows_contribute_nothing():
    g, s, a, B, S, m, q, k, v, do = _split_case(5)
    a = a.copy()
    a[0] = s[0]                                   # first block: empty window
    Q = q.shape[0]
    dq, dk, dv = _oracle_full_bwd(s, a, B, S, q, k, v, do, 0.5)
    assert (dq[:B] == 0).all()
    # removing those rows entirely leaves dk, dv unchanged
    keep = np.arange(B, Q)
    o, lse = oracle.partial_attn(np.arange(Q), B, s, a, q, np.arange(S), k, v, 0.5)
    dl = oracle.delta(o, do)
    lse2 = lse.copy()
    lse2[:B] = -np.inf
    _, dk2, dv2 = oracle.attn_bwd(B, s, a, q, do, lse2, dl, np.arange(S), k, v, 0.5,
                                  keep, np.arange(S))
    np.testing.assert_array_equal(dk, dk2)
    np.testing.assert_array_equal(dv, dv2)
