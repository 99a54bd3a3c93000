"""splitkv_attn_bwd_noalloc (the backward on the library's fixed per-device
scratch, for callers that cannot allocate) against splitkv_attn_bwd on the
same inputs: both run the same kernels in the same order, so every output
(dq accumulated, dk, dv, Delta) must be bit-identical. Two calls in a row, the
second with a smaller input, so nothing the first left in the scratch may
leak into the second; inputs beyond the scratch are rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_amd import binding, inputs
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


def case(seed, n_samples, L, A, m, J, hq=8, hkv=2, d=128, B=16):
    g = np.random.default_rng(seed)
    S = n_samples * L
    s, a = inputs.random_tiny_anchors(g, n_samples, L, A, L // 4)
    N = len(s)
    ids = np.sort(g.choice(S // m, size=J, replace=False))
    pos = oracle.local_key_positions(ids, m)
    sv = d ** -0.5
    q = inputs.normal_values(g, (N * B, hq, d), sv, "bf16")
    do = inputs.normal_values(g, (N * B, hq, d), sv, "bf16")
    o = inputs.normal_values(g, (N * B, hq, d), sv, "bf16")
    kg = inputs.normal_values(g, (S, hkv, d), sv, "bf16")
    vg = inputs.normal_values(g, (S, hkv, d), sv, "bf16")
    lse = (g.standard_normal((N * B, hq)) * 0.5 + 3.0).astype(np.float32)
    lse[0, :] = -np.inf                       # a row with no live key anywhere
    return dict(s=to_dev(s), a=to_dev(a), B=B, m=m, cs=to_dev(ids.astype(np.int64) * m),
                q=to_dev(q), do=to_dev(do), o=to_dev(o), k=to_dev(kg[pos]), v=to_dev(vg[pos]),
                lse=to_dev(lse))


def run(c, noalloc, dq0):
    dq = dq0.clone()
    delta = torch.empty(c["lse"].shape, dtype=torch.float32, device="cuda")
    dk, dv = torch.empty_like(c["k"]), torch.empty_like(c["v"])
    args = (c["s"], c["a"], c["B"], c["cs"], c["m"], c["q"], c["k"], c["v"], c["o"], c["do"],
            c["lse"], dq)
    if noalloc:
        binding.splitkv_attn_bwd_noalloc(*args, delta=delta, out=(dk, dv))
    else:
        binding.splitkv_attn_bwd(*args, delta=delta, out=(dk, dv))
    torch.cuda.synchronize()
    return dq, dk, dv, delta


def test_two_calls_in_a_row_match_the_workspace_backward():
    # first a larger input, then a smaller one (fewer blocks, chunks and keys)
    for c in (case(1, n_samples=3, L=4096, A=24, m=128, J=20),
              case(2, n_samples=1, L=2048, A=5, m=64, J=3)):
        dq0 = torch.randn(c["q"].shape, dtype=torch.float32, device="cuda")  # dq accumulates
        want = run(c, False, dq0)
        got = run(c, True, dq0)
        for name, x, y in zip(("dq", "dk", "dv", "delta"), got, want):
            assert torch.equal(x, y), name + " differs from splitkv_attn_bwd"


def test_inputs_beyond_the_scratch_are_rejected():
    # a shape whose backward scratch exceeds the fixed array: refused on the
    # host before anything is enqueued (the kernels never see these pointers)
    t = torch.zeros(16, dtype=torch.int64, device="cuda")
    buf = torch.zeros(1024, dtype=torch.float32, device="cuda")
    n_blocks, B, hq, hkv, d = 300000, 16, 8, 8, 64
    an = binding.Anchors(t.data_ptr(), t.data_ptr(), n_blocks, B)
    hd = binding.make_heads(hq, hkv, d, torch.bfloat16)
    loc = binding.Local(t.data_ptr(), 1, 64)
    need = binding.splitkv_workspace_bytes(binding.SPLITKV_OP_BWD, an, hd, loc)
    assert need > (48 << 20)
    p = buf.data_ptr()
    st = binding.lib().splitkv_attn_bwd_noalloc(
        ctypes.byref(an), ctypes.byref(hd), ctypes.byref(loc), p, p, p, p, p, p, p, p, p, p,
        torch.cuda.current_stream().cuda_stream)
    assert st == binding.SPLITKV_ERR_WORKSPACE
