"""Tensors whose device addresses straddle a multiple of 2^32.

The attention kernels address their global -> LDS tile copies as a 64-bit
base in scalar registers (stepped per pass with carry) plus a 32-bit per-lane
offset, and the dK/dV kernel adds 32-bit chunk offsets to a 64-bit chunk base.
A tensor placed so that a multiple of 2^32 falls inside it has addresses
whose low word has bit 31 set and rows that cross into the next 4 GiB; every
output must be bit-identical to the same call on the same values elsewhere.
"""
import numpy as np
import pytest
import torch

from block_sparse_cross_amd import binding
from tests.helpers import to_dev
from tests.test_gpu_attn import make_case

pytestmark = pytest.mark.gpu

GIB4 = 1 << 32


def straddle(t: torch.Tensor, keep: list) -> torch.Tensor:
    """A copy of t in a fresh buffer, placed so that the next multiple of 2^32
    above the buffer's start lies in the middle of the copy (256-byte aligned)."""
    nbytes = t.numel() * t.element_size()
    buf = torch.empty(GIB4 + nbytes + 4096, dtype=torch.uint8, device="cuda")
    keep.append(buf)
    base = buf.data_ptr()
    boundary = ((base >> 32) + 1) << 32
    start = (boundary - base - nbytes // 2) & ~255
    assert 0 <= start and start + nbytes <= buf.numel()
    view = buf[start:start + nbytes].view(t.dtype).view(t.shape)
    view.copy_(t)
    lo, hi = view.data_ptr(), view.data_ptr() + nbytes
    assert lo >> 32 != (hi - 1) >> 32, "the copy must cross a 4 GiB boundary"
    return view


def run(c, q, k, v, do):
    cs = to_dev(c["chunk_ids"].astype(np.int64) * c["m"])
    s, a = to_dev(c["s"]), to_dev(c["a"])
    o, lse = binding.splitkv_attn_fwd(s, a, c["B"], cs, c["m"], q, k, v)
    dq = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    dk, dv, delta = binding.splitkv_attn_bwd(s, a, c["B"], cs, c["m"], q, k, v, o, do, lse, dq)
    torch.cuda.synchronize()
    return [o, lse, dq, dk, dv, delta]


@pytest.mark.parametrize("kw", [dict(), dict(d=64, hq=4, hkv=4, m=200)])
def test_outputs_do_not_depend_on_where_tensors_sit(kw):
    c = make_case(500, **kw)
    q, k, v, do = (to_dev(c[n]) for n in ("q", "k", "v", "do"))
    ref = run(c, q, k, v, do)
    keep = []
    try:
        got = run(c, *(straddle(t, keep) for t in (q, k, v, do)))
        for name, g, r in zip(("o", "lse", "dq", "dk", "dv", "delta"), got, ref):
            assert torch.equal(g, r), name + " differs when the inputs straddle 2^32"
    finally:
        keep.clear()
        torch.cuda.empty_cache()
