"""Stored dS in the backward (Algorithm 1, AttnBwd_p): with room past the
minimum workspace, the dK/dV pass writes each pair's dS and dq is taken from
it instead of recomputing S and dP. The room asked for must equal the layout's
definition (every 32-key group that a 64-vector chunk's key union touches, one
4 KB tile per group and kv head); dk and dv must not change at all, and dq
only by the rounding of the two orders of summation."""
import numpy as np
import pytest
import torch

from block_sparse_cross_amd import binding, inputs
from tests.test_gpu_attn import make_case
from tests.helpers import rel_fro, to_dev, to_f64

pytestmark = pytest.mark.gpu


def host_need(c):
    """Stored-dS bytes from the definition, on the host."""
    G = c["hq"] // c["hkv"]
    lo = np.searchsorted(c["pos"], c["s"], side="left")
    hi = np.searchsorted(c["pos"], c["a"], side="left")
    n_vec = len(c["s"]) * c["B"] * G
    blk = np.arange(n_vec) // G // c["B"]
    vlo, vhi = lo[blk], hi[blk]
    live = vlo < vhi
    total = 0
    for c0 in range(0, n_vec, 64):
        sl = slice(c0, min(c0 + 64, n_vec))
        if not live[sl].any():
            continue
        ulo, uhi = vlo[sl][live[sl]].min(), vhi[sl][live[sl]].max()
        total += -(-uhi // 32) - ulo // 32
    return total * c["hkv"] * 4096


CASES = [dict(), dict(d=64), dict(hq=4, hkv=4), dict(hq=16, hkv=2, B=5, m=50),
         dict(hq=6, hkv=2, B=5, m=50), dict(B=1, A=40, hq=2, hkv=1),
         dict(J=12, n_chunks=12, m=16), dict(J=1, n_chunks=1, m=700)]


def dev_args(c):
    cs = to_dev(c["chunk_ids"].astype(np.int64) * c["m"])
    return to_dev(c["s"]), to_dev(c["a"]), c["B"], cs, c["m"]


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_ds_bytes_match_the_layout(idx):
    c = make_case(500 + idx, **CASES[idx])
    need = binding.splitkv_attn_bwd_ds_bytes(*dev_args(c), c["hq"], c["hkv"], c["d"],
                                             torch.bfloat16)
    assert need == host_need(c)
    assert need > 0
    assert binding.splitkv_attn_bwd_ds_bytes(*dev_args(c), c["hq"], c["hkv"], c["d"],
                                             torch.float32) == 0


def run(c, ws, dq0, lse):
    dq = dq0.clone()
    s, a, B, cs, m = dev_args(c)
    dk, dv, delta = binding.splitkv_attn_bwd(s, a, B, cs, m, to_dev(c["q"]), to_dev(c["k"]),
                                             to_dev(c["v"]), to_dev(c["o"]), to_dev(c["do"]),
                                             lse, dq, workspace=ws)
    torch.cuda.synchronize()
    return dq, dk, dv, delta


def with_o(c, seed):
    g = np.random.default_rng(seed)
    Q = c["q"].shape[0]
    c["o"] = inputs.normal_values(g, c["q"].shape, c["d"] ** -0.5, "bf16")
    lse = (g.standard_normal((Q, c["hq"])) * 0.5 + 3.0).astype(np.float32)
    lse[0, :] = -np.inf                       # a row with no live key anywhere
    return to_dev(lse)


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_stored_and_recomputed_dq_agree(idx):
    c = make_case(600 + idx, **CASES[idx])
    lse = with_o(c, idx)
    args = (*dev_args(c), c["hq"], c["hkv"], c["d"], torch.bfloat16)
    need = binding.splitkv_attn_bwd_ds_bytes(*args)
    dq0 = torch.randn(c["q"].shape, dtype=torch.float32, device="cuda")  # dq accumulates
    ref = run(c, None, dq0, lse)
    for room in (need, need // 2, 4096 * c["hkv"], need + 12345):
        got = run(c, binding.bwd_workspace(*args, ds_bytes=room), dq0, lse)
        for name, x, y in zip(("dk", "dv", "delta"), got[1:], ref[1:]):
            assert torch.equal(x, y), "%s changed with %d bytes of stored dS" % (name, room)
        d_got, d_ref = to_f64(got[0]) - to_f64(dq0), to_f64(ref[0]) - to_f64(dq0)
        assert rel_fro(d_got, d_ref) <= 2e-3, room
        assert np.abs(d_got - d_ref).max() <= 1e-2 * max(1.0, np.abs(d_ref).max()), room
        # rows without a live key keep dq exactly
        assert torch.equal(got[0][0], dq0[0])


def test_workspace_reused_by_a_smaller_call():
    """The same workspace for a larger, then a smaller input: nothing the first
    call stored may leak into the second (equal to a fresh workspace)."""
    big, small = make_case(700, n_chunks=16, J=9, A=6), make_case(701, m=50, hq=4, hkv=2)
    for c in (big, small):
        c["lse"] = with_o(c, 3)
    ws_big = binding.bwd_workspace(*dev_args(big), big["hq"], big["hkv"], big["d"],
                                   torch.bfloat16)
    dq_b = torch.zeros(big["q"].shape, dtype=torch.float32, device="cuda")
    run(big, ws_big, dq_b, big["lse"])
    dq_s = torch.zeros(small["q"].shape, dtype=torch.float32, device="cuda")
    got = run(small, ws_big, dq_s, small["lse"])
    fresh = run(small, binding.bwd_workspace(*dev_args(small), small["hq"], small["hkv"],
                                             small["d"], torch.bfloat16), dq_s, small["lse"])
    for x, y in zip(got, fresh):
        assert torch.equal(x, y)
