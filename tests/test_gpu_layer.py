"""One draft layer in Split-KV form on the GPU (block_sparse_cross_amd.layer)
against the oracle's composition (fp64 on the exact bf16 inputs): forward Y and
every gradient, at a small size spanning several tiles of every kernel, and Y
and dX through the oracle's whole chain on sampled rows at the weak-scaling
share with the 27B drafter's width.

Tolerance: the bf16 bounds the attention outputs and gradients are held to
(relative Frobenius error <= 1e-2, max abs error <= 2e-2), the absolute bound
scaled by the reference's largest magnitude where that exceeds 1 (the weight
gradients are sums over thousands of rows and reach ~10). The GPU keeps q, k,
v, the partials, the rescaled partials, do and the rank-summed dq as bf16
between steps; measured errors are <= 5e-3 relative Frobenius."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_amd import inputs
from block_sparse_cross_amd.layer import DraftLayer
from tests.helpers import rel_fro, to_dev, to_f64, vals64

pytestmark = pytest.mark.gpu


def assert_layer_close(got, ref, what):
    assert np.isfinite(got).all(), what
    rf = rel_fro(got, ref)
    err = float(np.abs(got - ref).max())
    bound = 2e-2 * max(1.0, float(np.abs(ref).max()))
    assert rf <= 1e-2 and err <= bound, "%s: rel fro %.3e, max err %.3e (bound %.3e)" % (
        what, rf, err, bound)


def build_case(seed, P=4, J=2, m=128, B=16, hq=4, hkv=2, d=64, H=192, L=512, A=6):
    g = np.random.default_rng(seed)
    S = P * J * m
    s, a = inputs.random_tiny_anchors(g, n_samples=S // L, L=L, A=A, prompt=L // 4)
    Q = len(s) * B
    mk = lambda r, c, tid, sc: inputs.gen_matrix(r, c, seed, tid, sc)  # noqa: E731
    t = {"X": mk(Q, H, inputs.T_X, 1.0), "U": mk(S, H, inputs.T_CTX, 1.0),
         "Wq": mk(hq * d, H, inputs.T_WQ, H ** -0.5), "Wk": mk(hkv * d, H, inputs.T_WK, H ** -0.5),
         "Wv": mk(hkv * d, H, inputs.T_WV, H ** -0.5), "Wo": mk(H, hq * d, inputs.T_WO, (hq * d) ** -0.5),
         "dY": mk(Q, H, inputs.T_DY, 1.0)}
    bo = inputs.gen_matrix(1, H, seed, inputs.T_BO, 1.0, dtype="fp32")[0]
    bundles = g.permutation(P * J).reshape(P, J)
    bundles.sort(axis=1)
    return s, a, B, hq, hkv, d, m, bundles, t, bo


@pytest.mark.parametrize("own", [False, True])
@pytest.mark.parametrize("seed", [0, 1])
def test_layer_matches_oracle(seed, own):
    s, a, B, hq, hkv, d, m, bundles, t, bo = build_case(seed)
    dev = {k: to_dev(v) for k, v in t.items()}
    sd, ad = to_dev(s), to_dev(a)
    cs = [to_dev(b.astype(np.int64) * m) for b in bundles]
    U_parts = [dev["U"][torch.from_numpy(oracle.local_key_positions(b, m)).cuda()].contiguous()
               for b in bundles]
    layer = DraftLayer(sd, ad, B, hq, hkv, d, cs, m, dev["Wq"], dev["Wk"], dev["Wv"], dev["Wo"],
                       to_dev(bo), own_blocks=own)
    Y = layer.forward(dev["X"], U_parts)
    g = layer.backward(dev["dY"])
    torch.cuda.synchronize()
    f64 = {k: vals64(v) for k, v in t.items()}
    fwd = oracle.draft_layer_forward(f64["X"], f64["U"], f64["Wq"], f64["Wk"], f64["Wv"],
                                     f64["Wo"], bo, s, a, B, hq, hkv, d, d ** -0.5, bundles, m,
                                     own_blocks=own)
    bwd = oracle.draft_layer_backward(fwd, f64["dY"], f64["X"], f64["U"], f64["Wq"], f64["Wk"],
                                      f64["Wv"], f64["Wo"], s, a, B, hq, hkv, d, d ** -0.5)
    assert_layer_close(to_f64(Y), fwd["Y"], "Y")
    for k in ("dX", "dWq", "dWk", "dWv", "dWo", "dbo"):
        assert_layer_close(to_f64(g[k]), bwd[k], k)
    dU = np.zeros_like(bwd["dU"])
    for p, b in enumerate(bundles):
        dU[oracle.local_key_positions(b, m)] = to_f64(g["dU"][p])
    assert_layer_close(dU, bwd["dU"], "dU")


def test_layer_full_size_weak8_sampled():
    """The weak-scaling share at P = 8 with the 27B drafter's width (Table 2:
    d_model 5120, 32/8 heads of 128) through the same calls bench.py --layer
    times. Each product is checked on sampled rows against the fp64 product of
    the bf16 operands the GPU used (its own q, rescaled partials, do, dq, dk,
    dv), i.e. the definition of that step; then Y and dX on the same rows
    against the oracle's whole chain from the layer inputs."""
    w = inputs.WORKLOADS["weak8"]
    H, seed = 5120, 0
    s, a = inputs.workload_anchors(w, seed)
    sd, ad = to_dev(s), to_dev(a)
    from block_sparse_cross_amd import binding
    _, _, bundles, _ = [x.cpu().numpy() for x in binding.splitkv_plan(sd, ad, w.B, w.S, w.m,
                                                                      w.P, w.J)]
    nq, nkv = w.hq * w.d, w.hkv * w.d
    X = inputs.gen_matrix(w.Q, H, seed, inputs.T_X, 1.0)
    Wq = inputs.gen_matrix(nq, H, seed, inputs.T_WQ, H ** -0.5)
    Wk = inputs.gen_matrix(nkv, H, seed, inputs.T_WK, H ** -0.5)
    Wv = inputs.gen_matrix(nkv, H, seed, inputs.T_WV, H ** -0.5)
    Wo = inputs.gen_matrix(H, nq, seed, inputs.T_WO, nq ** -0.5)
    dY = inputs.gen_matrix(w.Q, H, seed, inputs.T_DY, 1.0)
    bo = inputs.gen_matrix(1, H, seed, inputs.T_BO, 1.0, dtype="fp32")[0]
    # rank p's context rows: its chunks of the seeded [S, H] context features
    U = [np.concatenate([inputs.gen_matrix(w.m, H, seed, inputs.T_CTX, 1.0,
                                           first_row=int(j) * w.m) for j in b])
         for b in bundles]
    cs = [to_dev(b.astype(np.int64) * w.m) for b in bundles]
    layer = DraftLayer(sd, ad, w.B, w.hq, w.hkv, w.d, cs, w.m, to_dev(Wq), to_dev(Wk),
                       to_dev(Wv), to_dev(Wo), to_dev(bo))
    Y = layer.forward(to_dev(X), [to_dev(u) for u in U])
    Yh = to_f64(Y)                                # before backward reuses nothing of Y
    g = layer.backward(to_dev(dY))
    torch.cuda.synchronize()
    rg = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, w.Q - 1], rg.choice(w.Q, 6, replace=False)]))
    x64, wq, wk, wv, wo, dy = (vals64(z) for z in (X, Wq, Wk, Wv, Wo, dY))
    obar = [to_f64(layer.o_parts[p]).reshape(w.Q, nq) for p in range(w.P)]
    q = to_f64(layer.q)
    assert_layer_close(q[rows], x64[rows] @ wq.T, "q = X Wq^T")
    assert_layer_close(Yh[rows], sum(ob[rows] for ob in obar) @ wo.T + bo[None, :],
                       "Y = sum_p obar_p Wo^T + bo")
    assert_layer_close(to_f64(layer.do)[rows], dy[rows] @ wo, "do = dY Wo")
    dlt_ref = sum((ob[rows].reshape(-1, w.hq, w.d) * to_f64(layer.do)[rows].reshape(-1, w.hq, w.d)
                   ).sum(-1) for ob in obar)
    assert_layer_close(to_f64(layer.delta)[rows], dlt_ref, "Delta = sum_p <do, obar_p>")
    dq16 = to_f64(layer.dq16)
    assert_layer_close(to_f64(g["dX"])[rows], dq16[rows] @ wq, "dX = dq Wq")
    cols = rg.choice(nq, 4, replace=False)
    assert_layer_close(to_f64(g["dWq"])[cols], dq16[:, cols].T @ x64, "dWq = dq^T X")
    hcols = rg.choice(H, 4, replace=False)
    assert_layer_close(to_f64(g["dWo"])[hcols], sum(dy[:, hcols].T @ ob for ob in obar),
                       "dWo = sum_p dY^T obar_p")
    assert_layer_close(to_f64(g["dbo"]), dy.sum(axis=0), "dbo")
    p = 3
    keys = np.unique(np.concatenate([[0, w.J * w.m - 1], rg.choice(w.J * w.m, 6, replace=False)]))
    u64 = vals64(U[p])
    k_ref = u64[keys] @ wk.T
    assert_layer_close(to_f64(layer.k[p])[keys], k_ref, "k_p = U_p Wk^T")
    dk = to_f64(layer.dk[p]).reshape(-1, nkv)
    dv = to_f64(layer.dv[p]).reshape(-1, nkv)
    assert_layer_close(to_f64(g["dU"][p])[keys], dk[keys] @ wk + dv[keys] @ wv,
                       "dU_p = dk_p Wk + dv_p Wv")
    kc = rg.choice(nkv, 3, replace=False)
    dwk_ref = np.zeros((3, H))
    for pp in range(w.P):
        dkp = to_f64(layer.dk[pp]).reshape(-1, nkv)
        dwk_ref += dkp[:, kc].T @ vals64(U[pp])
    assert_layer_close(to_f64(g["dWk"])[kc], dwk_ref, "dWk = sum_p dk_p^T U_p")

    # The sampled rows through the oracle's own chain from the layer inputs
    # (fp64 on the bf16 values), no GPU intermediate: q = X Wq^T; every rank's
    # k_p = U_p Wk^T, v_p = U_p Wv^T and its Eq. 3 partial; the Eq. 4 merge as
    # each rank applies it (LSE reduction, rescaled partials); Y = the summed
    # OProj of the rescaled partials + bo. Backward: do = dY Wo, Delta =
    # sum_p <do, obar_p>, each rank's dq (Algorithm 1, global lse and Delta),
    # summed; dX = dq Wq.
    n, scale = len(rows), w.d ** -0.5
    q_r = (x64[rows] @ wq.T).reshape(n, w.hq, w.d)
    parts = []
    for pp in range(w.P):
        pos = oracle.local_key_positions(bundles[pp], w.m)
        u64p = vals64(U[pp])
        kp = (u64p @ wk.T).reshape(-1, w.hkv, w.d)
        vp = (u64p @ wv.T).reshape(-1, w.hkv, w.d)
        o_p, l_p = oracle.partial_attn(rows, w.B, s, a, q_r, pos, kp, vp, scale)
        parts.append((pos, kp, vp, o_p, l_p))
    lse_r = oracle.lse_reduce(np.stack([pt[4].reshape(-1) for pt in parts]))
    obar_r = [oracle.lse_rescale(pt[3].reshape(-1, w.d), pt[4].reshape(-1), lse_r).reshape(n, nq)
              for pt in parts]
    assert_layer_close(Yh[rows], sum(ob @ wo.T for ob in obar_r) + bo[None, :],
                       "Y, oracle chain from X, U and the weights")
    do_r = (dy[rows] @ wo).reshape(n, w.hq, w.d)
    dlt_r = sum(oracle.delta(ob.reshape(n, w.hq, w.d), do_r) for ob in obar_r)
    # the oracle's backward indexes q, do, lse and Delta by row: full-height
    # arrays holding the sampled rows (the others are not read for them)
    full = lambda x: np.zeros((w.Q,) + x.shape[1:])  # noqa: E731
    qf, dof, lf, df = full(q_r), full(do_r), full(dlt_r), full(dlt_r)
    qf[rows], dof[rows], lf[rows], df[rows] = q_r, do_r, lse_r.reshape(n, w.hq), dlt_r
    dq_r = sum(oracle.attn_bwd(w.B, s, a, qf, dof, lf, df, pt[0], pt[1], pt[2], scale, rows,
                               np.zeros(0, dtype=np.int64))[0] for pt in parts)
    assert_layer_close(to_f64(g["dX"])[rows], dq_r.reshape(n, nq) @ wq,
                       "dX, oracle chain from X, U, dY and the weights")
