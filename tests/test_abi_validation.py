"""Host-side validation of every C-ABI entry point (CPU only, no GPU): each
call below breaks one documented rule of include/splitkv.h and must return
the documented status before anything is enqueued, so no device memory is
touched (the pointers are never dereferenced). The same file runs under
AddressSanitizer + UndefinedBehaviorSanitizer in test_sanitizers.py."""
import ctypes
import math

import pytest

from block_sparse_cross_amd import binding as b

OK, INV, UNS, WS = b.SPLITKV_OK, b.SPLITKV_ERR_INVALID_ARG, b.SPLITKV_ERR_UNSUPPORTED, \
    b.SPLITKV_ERR_WORKSPACE
P16 = 0x100000      # a 16-byte aligned address (never dereferenced)
MIS = 0x100008      # 8 bytes off
ref = ctypes.byref


@pytest.fixture(scope="module")
def L():
    return b.lib()


def an(n=4, B=16, s=P16, a=P16):
    return b.Anchors(s, a, n, B)


def hd(hq=8, hkv=2, d=128, dtype=b.SPLITKV_BF16, scale=128 ** -0.5):
    return b.Heads(hq, hkv, d, dtype, scale)


def loc(n=2, m=64, cs=P16):
    return b.Local(cs, n, m)


def test_plan(L):
    x = an()
    assert L.splitkv_plan(None, 256, 64, 2, 2, P16, P16, P16, P16, None) == INV
    assert L.splitkv_plan(ref(x), 255, 64, 2, 2, P16, P16, P16, P16, None) == INV  # P J m != S
    assert L.splitkv_plan(ref(x), 256, 64, 2, 2, None, P16, P16, P16, None) == INV
    assert L.splitkv_plan(ref(x), 2048 * 64, 64, 2048, 1, P16, P16, P16, P16, None) == UNS
    assert L.splitkv_plan(ref(x), 8192 * 64, 64, 2, 4096, P16, P16, P16, P16, None) == UNS
    big = an(n=1 << 30)
    assert L.splitkv_plan(ref(big), 1 << 24, 1 << 20, 4, 4, P16, P16, P16, P16, None) == UNS
    assert L.splitkv_plan(ref(an(n=2, s=None)), 256, 64, 2, 2, P16, P16, P16, P16, None) == INV


def test_locality_and_baseline(L):
    assert L.splitkv_locality_match(P16, 0, 2, 64, P16, P16, P16, None) == INV
    assert L.splitkv_locality_match(P16, 4, 2, 64, None, P16, P16, None) == INV
    assert L.splitkv_locality_match(P16, 257, 1, 64, P16, P16, P16, None) == UNS
    i64 = ctypes.c_int64 * 2
    st, ln = i64(0, 100), i64(100, 100)
    x = an()
    assert L.splitkv_plan_baseline(5, ref(x), 2, st, ln, 2, P16, P16, None) == INV
    assert L.splitkv_plan_baseline(1, ref(x), 2, st, ln, 3, P16, P16, None) == INV  # 100 % 6
    assert L.splitkv_plan_baseline(0, ref(x), 2, i64(1, 100), ln, 2, P16, P16, None) == INV
    assert L.splitkv_plan_baseline(0, ref(x), 2, st, i64(100, 0), 2, P16, P16, None) == INV
    assert L.splitkv_plan_baseline(0, ref(x), 129, st, ln, 2, P16, P16, None) == UNS
    assert L.splitkv_plan_baseline(0, ref(x), 2, st, ln, 3, P16, P16, None) == INV  # 200 % 3


def test_validate_anchors(L):
    out = ctypes.c_void_p(P16)
    assert L.splitkv_validate_anchors(None, 10, out, None) == INV
    assert L.splitkv_validate_anchors(ref(an()), -1, out, None) == INV
    assert L.splitkv_validate_anchors(ref(an()), 10, None, None) == INV
    assert L.splitkv_validate_anchors(ref(an(B=0)), 10, out, None) == INV


def test_attention_forward(L):
    x, l = an(), loc()
    ws = b.splitkv_workspace_bytes(b.SPLITKV_OP_FWD, x, hd(), l)
    assert ws > 0 and ws % 256 == 0
    def call(a=x, h=hd(), lc=l, q=P16, k=P16, v=P16, o=P16, od=b.SPLITKV_BF16, lse=P16,
             w=P16, wb=ws):
        return L.splitkv_attn_fwd(ref(a), ref(h), ref(lc), q, k, v, o, od, lse, w, wb, None)
    assert call(h=hd(hq=6, hkv=4)) == INV
    assert call(h=hd(d=96)) == UNS
    assert call(h=hd(dtype=7)) == UNS
    assert call(h=hd(scale=-1.0)) == INV
    assert call(h=hd(scale=float("nan"))) == INV
    assert call(h=hd(scale=math.inf)) == INV
    assert call(od=5) == UNS
    assert call(q=None) == INV
    assert call(lse=None) == INV
    assert call(lc=loc(cs=None)) == INV
    assert call(lc=loc(n=-1)) == INV
    assert call(lc=loc(n=1 << 20, m=1 << 12)) == UNS           # J m >= 2^31
    assert call(a=an(n=1 << 26)) == UNS                        # N B hq >= 2^31
    assert call(h=hd(hq=1 << 18, hkv=1 << 18)) == UNS          # hq d >= 2^25
    assert call(wb=ws - 1) == WS
    assert call(w=None) == WS
    for k in ("q", "k", "v", "o"):
        assert call(**{k: MIS}) == INV, k


def test_attention_backward(L):
    x, h, l = an(), hd(), loc()
    ws = b.splitkv_workspace_bytes(b.SPLITKV_OP_BWD, x, h, l)
    assert ws > b.splitkv_workspace_bytes(b.SPLITKV_OP_FWD, x, h, l)
    def args(**kw):
        d = dict(q=P16, k=P16, v=P16, o=P16, do=P16, lse=P16, delta=P16, dq=P16, dk=P16, dv=P16)
        d.update(kw)
        return [d[n] for n in ("q", "k", "v", "o", "do", "lse", "delta", "dq", "dk", "dv")]
    def call(w=P16, wb=ws, a=x, **kw):
        return L.splitkv_attn_bwd(ref(a), ref(h), ref(l), *args(**kw), w, wb, None)
    def call_na(a=x, **kw):
        return L.splitkv_attn_bwd_noalloc(ref(a), ref(h), ref(l), *args(**kw), None)
    for c in (call, call_na):
        assert c(dq=None) == INV
        assert c(delta=None) == INV
        assert c(dk=None) == INV
        for k in ("q", "k", "v", "o", "do", "dq", "dk", "dv"):
            assert c(**{k: MIS}) == INV, k
    assert call(wb=ws - 1) == WS
    # the no-allocation form: shapes whose scratch exceeds the fixed array
    big = an(n=300000)
    need = b.splitkv_workspace_bytes(b.SPLITKV_OP_BWD, big, h, l)
    assert need > (48 << 20)
    assert call_na(a=big) == WS


def test_merge_family(L):
    bf, f32 = b.SPLITKV_BF16, b.SPLITKV_FP32
    assert L.splitkv_lse_merge(0, 8, 128, P16, bf, P16, P16, bf, P16, None) == INV
    assert L.splitkv_lse_merge(2, 8, 100, P16, bf, P16, P16, bf, P16, None) == INV
    assert L.splitkv_lse_merge(2, 8, 128, P16, 9, P16, P16, bf, P16, None) == UNS
    assert L.splitkv_lse_merge(2, 8, 128, None, bf, P16, P16, bf, P16, None) == INV
    assert L.splitkv_lse_merge(2, 8, 128, MIS, bf, P16, P16, bf, P16, None) == INV
    assert L.splitkv_lse_merge(2, 8, 128, P16, bf, P16, MIS, bf, P16, None) == INV
    assert L.splitkv_lse_merge(2, 0, 128, None, bf, None, None, bf, None, None) == OK  # nothing to do
    assert L.splitkv_lse_reduce(0, 8, P16, P16, None) == INV
    assert L.splitkv_lse_reduce(2, 8, None, P16, None) == INV
    assert L.splitkv_lse_rescale(8, 128, P16, bf, P16, P16, MIS, bf, None) == INV
    assert L.splitkv_lse_rescale(8, 100, P16, bf, P16, P16, P16, bf, None) == INV
    assert L.splitkv_delta(8, 100, P16, bf, P16, bf, P16, 0, None) == INV
    assert L.splitkv_delta(8, 1024, P16, bf, P16, bf, P16, 0, None) == INV     # d / 8 > 64
    assert L.splitkv_delta(8, 128, MIS, bf, P16, bf, P16, 0, None) == INV
    assert L.splitkv_cast_bf16(12, P16, P16, None) == INV
    assert L.splitkv_cast_bf16(16, MIS, P16, None) == INV


def test_rescale_in_place_needs_one_dtype(L):
    bf, f32 = b.SPLITKV_BF16, b.SPLITKV_FP32
    assert L.splitkv_lse_rescale(8, 128, P16, bf, P16, P16, P16, f32, None) == INV


def test_products(L):
    NT = b.SPLITKV_GEMM_NT
    f32 = b.SPLITKV_FP32
    assert L.splitkv_gemm(9, 16, 16, 16, P16, P16, P16, f32, None, 0, None) == INV
    assert L.splitkv_gemm(NT, 16, 16, 12, P16, P16, P16, f32, None, 0, None) == INV
    assert L.splitkv_gemm(NT, 16, 16, 16, P16, P16, P16, 9, None, 0, None) == UNS
    assert L.splitkv_gemm(NT, 16, 16, 16, None, P16, P16, f32, None, 0, None) == INV
    assert L.splitkv_gemm(NT, 1 << 28, 16, 16, P16, P16, P16, f32, None, 0, None) == UNS
    for i in range(3):
        p = [P16, P16, P16]
        p[i] = MIS
        assert L.splitkv_gemm(NT, 16, 16, 16, *p, f32, None, 0, None) == INV
    assert L.splitkv_gemm_pair(NT, 16, 16, 32, P16, P16, P16, P16, P16, f32, None, 0, None) == INV
    assert L.splitkv_gemm_pair(NT, 16, 16, 64, P16, P16, MIS, P16, P16, f32, None, 0, None) == INV


def test_workspace_queries_with_missing_structs(L):
    assert b.splitkv_workspace_bytes(b.SPLITKV_OP_FWD) == 0
    assert b.splitkv_workspace_bytes(b.SPLITKV_OP_BWD, an()) == 0
    assert b.splitkv_workspace_bytes(99, an(), hd(), loc()) == 0


def test_own_block_layout(L):
    n = ctypes.c_int64(0)
    assert L.splitkv_own_block_local(-1, 16, P16, P16, P16, ctypes.byref(n), None) == INV
    assert L.splitkv_own_block_local(4, 0, P16, P16, P16, ctypes.byref(n), None) == INV
    assert L.splitkv_own_block_local(4, 16, None, P16, P16, ctypes.byref(n), None) == INV
    assert L.splitkv_own_block_local(4, 16, P16, P16, P16, None, None) == INV
    assert L.splitkv_own_block_local(1 << 27, 16, P16, P16, P16, ctypes.byref(n), None) == UNS
