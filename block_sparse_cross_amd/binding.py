"""Thin Python binding of libsplitkv.so (the C ABI in include/splitkv.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, and their device pointers are handed to the library together with
torch's current HIP stream. Every step of the hot path runs in the library's
kernels; there is no fallback. If the library is missing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SPLITKV_LIB may name another build of the same library (e.g. one with host
# sanitizers); there is no other implementation behind these calls.
LIB_PATH = os.environ.get("SPLITKV_LIB") or os.path.join(_HERE, "libsplitkv.so")

SPLITKV_OK = 0
SPLITKV_ERR_INVALID_ARG = -1
SPLITKV_ERR_UNSUPPORTED = -2
SPLITKV_ERR_WORKSPACE = -3
SPLITKV_ERR_HIP = -4

SPLITKV_BF16 = 0
SPLITKV_FP32 = 1

SPLITKV_OP_PLAN, SPLITKV_OP_FWD, SPLITKV_OP_BWD, SPLITKV_OP_MERGE = 0, 1, 2, 3

SPLITKV_BASELINE_NO_BALANCE, SPLITKV_BASELINE_ZIGZAG = 0, 1

EXPORTED = ("splitkv_workspace_bytes", "splitkv_validate_anchors", "splitkv_plan",
            "splitkv_locality_match", "splitkv_plan_baseline",
            "splitkv_attn_fwd", "splitkv_lse_merge", "splitkv_lse_reduce", "splitkv_lse_rescale",
            "splitkv_delta", "splitkv_gemm", "splitkv_gemm_pair", "splitkv_cast_bf16",
            "splitkv_attn_bwd", "splitkv_attn_bwd_ds_bytes", "splitkv_attn_bwd_noalloc",
            "splitkv_own_block_local", "splitkv_status_str")

SPLITKV_GEMM_NT, SPLITKV_GEMM_NN, SPLITKV_GEMM_TN = 0, 1, 2


class SplitKVError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (%d)" % (fn, status_str(status), status))
        self.status = status


class Anchors(ctypes.Structure):
    _fields_ = [("s", ctypes.c_void_p), ("a", ctypes.c_void_p), ("n_blocks", ctypes.c_int64),
                ("block_size", ctypes.c_int32)]


class Heads(ctypes.Structure):
    _fields_ = [("hq", ctypes.c_int32), ("hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class Local(ctypes.Structure):
    _fields_ = [("chunk_start", ctypes.c_void_p), ("n_chunks", ctypes.c_int32),
                ("chunk_len", ctypes.c_int64)]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libsplitkv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libsplitkv.so is not built; run `python -m "
                               "block_sparse_cross_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        A, H, Lc = ctypes.POINTER(Anchors), ctypes.POINTER(Heads), ctypes.POINTER(Local)
        L.splitkv_workspace_bytes.argtypes = [ctypes.c_int, A, H, Lc]
        L.splitkv_workspace_bytes.restype = sz
        L.splitkv_validate_anchors.argtypes = [A, ctypes.c_int64, vp, vp]
        L.splitkv_validate_anchors.restype = ctypes.c_int
        L.splitkv_locality_match.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                             vp, vp, vp, vp]
        L.splitkv_locality_match.restype = ctypes.c_int
        L.splitkv_own_block_local.argtypes = [ctypes.c_int64, ctypes.c_int32, vp, vp, vp,
                                              ctypes.POINTER(ctypes.c_int64), vp]
        L.splitkv_own_block_local.restype = ctypes.c_int
        L.splitkv_plan.argtypes = [A, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_int32, vp, vp, vp, vp, vp]
        L.splitkv_plan.restype = ctypes.c_int
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.splitkv_plan_baseline.argtypes = [ctypes.c_int, A, ctypes.c_int32, i64p, i64p,
                                            ctypes.c_int32, vp, vp, vp]
        L.splitkv_plan_baseline.restype = ctypes.c_int
        L.splitkv_attn_fwd.argtypes = [A, H, Lc, vp, vp, vp, vp, ctypes.c_int, vp, vp, sz, vp]
        L.splitkv_attn_fwd.restype = ctypes.c_int
        L.splitkv_lse_merge.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, vp,
                                        ctypes.c_int, vp, vp, ctypes.c_int, vp, vp]
        L.splitkv_lse_merge.restype = ctypes.c_int
        L.splitkv_lse_reduce.argtypes = [ctypes.c_int32, ctypes.c_int64, vp, vp, vp]
        L.splitkv_lse_reduce.restype = ctypes.c_int
        L.splitkv_lse_rescale.argtypes = [ctypes.c_int64, ctypes.c_int32, vp, ctypes.c_int, vp, vp,
                                          vp, ctypes.c_int, vp]
        L.splitkv_lse_rescale.restype = ctypes.c_int
        L.splitkv_delta.argtypes = [ctypes.c_int64, ctypes.c_int32, vp, ctypes.c_int, vp,
                                    ctypes.c_int, vp, ctypes.c_int, vp]
        L.splitkv_delta.restype = ctypes.c_int
        L.splitkv_gemm.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, vp]
        L.splitkv_gemm.restype = ctypes.c_int
        L.splitkv_gemm_pair.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, vp, vp, vp, vp, vp, ctypes.c_int, vp,
                                        ctypes.c_int, vp]
        L.splitkv_gemm_pair.restype = ctypes.c_int
        L.splitkv_cast_bf16.argtypes = [ctypes.c_int64, vp, vp, vp]
        L.splitkv_cast_bf16.restype = ctypes.c_int
        L.splitkv_attn_bwd.argtypes = [A, H, Lc, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.splitkv_attn_bwd.restype = ctypes.c_int
        L.splitkv_attn_bwd_ds_bytes.argtypes = [A, H, Lc, vp, sz, vp, vp]
        L.splitkv_attn_bwd_ds_bytes.restype = ctypes.c_int
        L.splitkv_attn_bwd_noalloc.argtypes = [A, H, Lc, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                               vp]
        L.splitkv_attn_bwd_noalloc.restype = ctypes.c_int
        L.splitkv_status_str.argtypes = [ctypes.c_int]
        L.splitkv_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().splitkv_status_str(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != SPLITKV_OK:
        raise SplitKVError(fn, status)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return SPLITKV_BF16
    if t == torch.float32:
        return SPLITKV_FP32
    raise TypeError("unsupported dtype %s (bf16 or fp32)" % t)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr() if t.numel() > 0 else None


def _stream(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def make_anchors(s: torch.Tensor, a: torch.Tensor, block_size: int) -> Anchors:
    if s.dtype != torch.int64 or a.dtype != torch.int64 or s.shape != a.shape or s.dim() != 1:
        raise ValueError("anchors: s and a must be int64 vectors of equal length")
    return Anchors(_ptr(s), _ptr(a), s.numel(), int(block_size))


def make_heads(hq: int, hkv: int, d: int, dtype: torch.dtype, scale: Optional[float] = None) -> Heads:
    return Heads(int(hq), int(hkv), int(d), _dtype_code(dtype),
                 float(d ** -0.5 if scale is None else scale))


def make_local(chunk_start: torch.Tensor, chunk_len: int) -> Local:
    if chunk_start.dtype != torch.int64 or chunk_start.dim() != 1:
        raise ValueError("chunk_start must be an int64 vector")
    return Local(_ptr(chunk_start), chunk_start.numel(), int(chunk_len))


def splitkv_workspace_bytes(op: int, an: Optional[Anchors] = None, hd: Optional[Heads] = None,
                            loc: Optional[Local] = None) -> int:
    return int(lib().splitkv_workspace_bytes(
        int(op), ctypes.byref(an) if an is not None else None,
        ctypes.byref(hd) if hd is not None else None,
        ctypes.byref(loc) if loc is not None else None))


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    """(pointer, size) of the caller's workspace, or of a fresh one of nbytes.
    A caller-supplied workspace is passed as is; the library checks its size."""
    if ws is None:
        if nbytes == 0:
            return None, 0
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _keepalive.append(ws)
        if len(_keepalive) > 4:
            del _keepalive[0]
    return _ptr(ws), ws.numel() * ws.element_size()


# Recently allocated workspaces stay referenced until later calls so that the
# caching allocator cannot hand their memory out while a kernel still uses it.
_keepalive = []


def splitkv_plan(s: torch.Tensor, a: torch.Tensor, block_size: int, S: int, m: int, P: int,
                 J: int, out: Optional[Tuple[torch.Tensor, ...]] = None,
                 stream: Optional[torch.cuda.Stream] = None):
    """Eq. 6 chunk costs + cost-aware LPT on the GPU.

    Returns (chunk_cost int64 [P*J], chunk_owner int32 [P*J],
    rank_chunks int32 [P, J], rank_load int64 [P]) as device tensors."""
    dev = s.device
    if out is None:
        out = (torch.empty(P * J, dtype=torch.int64, device=dev),
               torch.empty(P * J, dtype=torch.int32, device=dev),
               torch.empty((P, J), dtype=torch.int32, device=dev),
               torch.empty(P, dtype=torch.int64, device=dev))
    cost, owner, chunks, load = out
    an = make_anchors(s, a, block_size)
    _check("splitkv_plan", lib().splitkv_plan(ctypes.byref(an), int(S), int(m), int(P), int(J),
                                              _ptr(cost), _ptr(owner), _ptr(chunks), _ptr(load),
                                              _stream(stream)))
    return out


def baseline_range_count(strategy: int, n_samples: int, P: int) -> int:
    """Number of ranges splitkv_plan_baseline prices (P, or 2P per sample)."""
    return P if strategy == SPLITKV_BASELINE_NO_BALANCE else 2 * P * n_samples


def splitkv_validate_anchors(s: torch.Tensor, a: torch.Tensor, block_size: int, S: int,
                             out: Optional[torch.Tensor] = None,
                             stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Device-side check that every window [s_i, a_i) lies in [0, S) (empty
    windows allowed). Returns a device int64 tensor [2]: the number of invalid
    blocks and the index of the first one (-1 if none)."""
    if out is None:
        out = torch.empty(2, dtype=torch.int64, device=s.device)
    an = make_anchors(s, a, block_size)
    _check("splitkv_validate_anchors",
           lib().splitkv_validate_anchors(ctypes.byref(an), int(S), _ptr(out), _stream(stream)))
    return out


def splitkv_locality_match(rank_chunks: torch.Tensor, m: int,
                           out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                           stream: Optional[torch.cuda.Stream] = None):
    """Place a plan's bundles (device int32 [P][J], as splitkv_plan returns them)
    on physical ranks keeping the most context rows in place (§4.2). Returns
    device tensors (phys_rank int32 [P], send_rows int64 [P][P], kept_moved
    int64 [2])."""
    if rank_chunks.dim() != 2 or rank_chunks.dtype != torch.int32 or not rank_chunks.is_contiguous():
        raise ValueError("rank_chunks must be a contiguous int32 [P][J] tensor")
    P, J = rank_chunks.shape
    dev = rank_chunks.device
    if out is None:
        out = (torch.empty(P, dtype=torch.int32, device=dev),
               torch.empty((P, P), dtype=torch.int64, device=dev),
               torch.empty(2, dtype=torch.int64, device=dev))
    perm, send, km = out
    _check("splitkv_locality_match",
           lib().splitkv_locality_match(_ptr(rank_chunks), int(P), int(J), int(m), _ptr(perm),
                                        _ptr(send), _ptr(km), _stream(stream)))
    return out


def splitkv_plan_baseline(strategy: int, s: torch.Tensor, a: torch.Tensor, block_size: int,
                          sample_start, sample_len, P: int,
                          out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                          stream: Optional[torch.cuda.Stream] = None):
    """Context work of a position-based assignment (No balance or Zigzag) on the GPU.

    sample_start, sample_len: the packed samples (host integer sequences).
    Returns (range_cost int64 [R], rank_load int64 [P]) as device tensors."""
    n = len(sample_start)
    st = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in sample_start])
    ln = (ctypes.c_int64 * max(len(sample_len), 1))(*[int(x) for x in sample_len])
    if len(sample_len) != n:
        raise ValueError("sample_start and sample_len differ in length")
    dev = s.device
    if out is None:
        R = baseline_range_count(strategy, n, P)
        out = (torch.empty(max(R, 1), dtype=torch.int64, device=dev),
               torch.empty(max(P, 1), dtype=torch.int64, device=dev))
    cost, load = out
    an = make_anchors(s, a, block_size)
    _check("splitkv_plan_baseline",
           lib().splitkv_plan_baseline(int(strategy), ctypes.byref(an), n, st, ln, int(P),
                                       _ptr(cost), _ptr(load), _stream(stream)))
    return out


def own_block_local(s: torch.Tensor, block_size: int, stream: Optional[torch.cuda.Stream] = None):
    """Windows and key table for the own-block part of the mask (Figure 1 of the
    Split-KV paper: a block's rows also attend all B tokens of their own block),
    from splitkv_own_block_local. Returns (s', a', chunk_start, chunk_len) to
    pass to splitkv_attn_fwd / splitkv_attn_bwd with the block keys and
    values (block i's window over them is [iB, (i+1)B))."""
    n = s.numel()
    s2 = torch.empty(n, dtype=torch.int64, device=s.device)
    a2 = torch.empty(n, dtype=torch.int64, device=s.device)
    cs = torch.empty(1, dtype=torch.int64, device=s.device)
    clen = ctypes.c_int64(0)
    _check("splitkv_own_block_local", lib().splitkv_own_block_local(
        int(n), int(block_size), _ptr(s2), _ptr(a2), _ptr(cs), ctypes.byref(clen),
        _stream(stream)))
    return s2, a2, cs, int(clen.value)


def splitkv_attn_fwd(s, a, block_size: int, chunk_start, chunk_len: int, q, k, v,
                     scale: Optional[float] = None, o_dtype: Optional[torch.dtype] = None,
                     out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                     workspace: Optional[torch.Tensor] = None,
                     stream: Optional[torch.cuda.Stream] = None):
    """Eq. 3 partial attention of all query rows against the local chunks.

    q [Q, hq, d]; k, v [J*m, hkv, d]. Returns (o_part [Q, hq, d], lse_part fp32 [Q, hq])."""
    Q, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != v.shape or k.shape[2] != d or q.dtype != k.dtype or k.dtype != v.dtype:
        raise ValueError("q/k/v shapes or dtypes disagree")
    if k.shape[0] != chunk_start.numel() * chunk_len:
        raise ValueError("k/v rows must equal n_chunks * chunk_len")
    if Q != s.numel() * block_size:
        raise ValueError("q rows must equal n_blocks * block_size")
    o_dtype = q.dtype if o_dtype is None else o_dtype
    if out is None:
        out = (torch.empty((Q, hq, d), dtype=o_dtype, device=q.device),
               torch.empty((Q, hq), dtype=torch.float32, device=q.device))
    o, lse = out
    if o.shape != (Q, hq, d) or lse.shape != (Q, hq) or lse.dtype != torch.float32:
        raise ValueError("output shapes disagree")
    an, hd, loc = make_anchors(s, a, block_size), make_heads(hq, hkv, d, q.dtype, scale), \
        make_local(chunk_start, chunk_len)
    nbytes = splitkv_workspace_bytes(SPLITKV_OP_FWD, an, hd, loc)
    ws_ptr, ws_bytes = _workspace(nbytes, q.device, workspace)
    _check("splitkv_attn_fwd", lib().splitkv_attn_fwd(
        ctypes.byref(an), ctypes.byref(hd), ctypes.byref(loc), _ptr(q), _ptr(k), _ptr(v),
        _ptr(o), _dtype_code(o.dtype), _ptr(lse), ws_ptr, ws_bytes, _stream(stream)))
    return o, lse


def splitkv_lse_merge(o_parts: torch.Tensor, lse_parts: torch.Tensor,
                      out_dtype: Optional[torch.dtype] = None,
                      out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                      stream: Optional[torch.cuda.Stream] = None):
    """Eq. 4 merge. o_parts [P, rows..., d], lse_parts fp32 [P, rows...]."""
    P = o_parts.shape[0]
    d = o_parts.shape[-1]
    rows = lse_parts[0].numel()
    if lse_parts.shape[0] != P or o_parts[0].numel() != rows * d or lse_parts.dtype != torch.float32:
        raise ValueError("partials disagree")
    out_dtype = o_parts.dtype if out_dtype is None else out_dtype
    if out is None:
        out = (torch.empty(o_parts.shape[1:], dtype=out_dtype, device=o_parts.device),
               torch.empty(lse_parts.shape[1:], dtype=torch.float32, device=o_parts.device))
    o, lse = out
    if o.numel() != rows * d or lse.numel() != rows:
        raise ValueError("output shapes disagree")
    _check("splitkv_lse_merge", lib().splitkv_lse_merge(
        int(P), int(rows), int(d), _ptr(o_parts), _dtype_code(o_parts.dtype), _ptr(lse_parts),
        _ptr(o), _dtype_code(o.dtype), _ptr(lse), _stream(stream)))
    return o, lse


def splitkv_lse_reduce(lse_parts: torch.Tensor, out: Optional[torch.Tensor] = None,
                       stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """LSE half of Eq. 4: lse_parts fp32 [P, rows...] -> lse fp32 [rows...]."""
    if lse_parts.dtype != torch.float32 or lse_parts.dim() < 2:
        raise ValueError("lse_parts must be fp32 [P, rows...]")
    P, rows = lse_parts.shape[0], lse_parts[0].numel()
    if out is None:
        out = torch.empty(lse_parts.shape[1:], dtype=torch.float32, device=lse_parts.device)
    if out.numel() != rows or out.dtype != torch.float32:
        raise ValueError("output shape disagrees")
    _check("splitkv_lse_reduce", lib().splitkv_lse_reduce(int(P), int(rows), _ptr(lse_parts),
                                                          _ptr(out), _stream(stream)))
    return out


def splitkv_lse_rescale(o_part: torch.Tensor, lse_part: torch.Tensor, lse: torch.Tensor,
                        out_dtype: Optional[torch.dtype] = None,
                        out: Optional[torch.Tensor] = None,
                        stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """One rank's rescaled partial exp(lse_part - lse) * o_part (rows..., d)."""
    d = o_part.shape[-1]
    rows = lse_part.numel()
    if o_part.numel() != rows * d or lse.numel() != rows or \
            lse_part.dtype != torch.float32 or lse.dtype != torch.float32:
        raise ValueError("partial, its lse and the reduced lse disagree")
    if out is None:
        out_dtype = o_part.dtype if out_dtype is None else out_dtype
        out = torch.empty(o_part.shape, dtype=out_dtype, device=o_part.device)
    if out.numel() != rows * d:
        raise ValueError("output shape disagrees")
    _check("splitkv_lse_rescale", lib().splitkv_lse_rescale(
        int(rows), int(d), _ptr(o_part), _dtype_code(o_part.dtype), _ptr(lse_part), _ptr(lse),
        _ptr(out), _dtype_code(out.dtype), _stream(stream)))
    return out


def splitkv_delta(o: torch.Tensor, dout: torch.Tensor, delta: Optional[torch.Tensor] = None,
                  accumulate: bool = False,
                  stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Delta = <dout, o> per row of the last dimension (+= with accumulate)."""
    d = o.shape[-1]
    if dout.shape != o.shape:
        raise ValueError("o and dout disagree")
    rows = o.numel() // d
    if delta is None:
        delta = torch.empty(o.shape[:-1], dtype=torch.float32, device=o.device)
    if delta.numel() != rows or delta.dtype != torch.float32:
        raise ValueError("delta shape disagrees")
    _check("splitkv_delta", lib().splitkv_delta(
        int(rows), int(d), _ptr(o), _dtype_code(o.dtype), _ptr(dout), _dtype_code(dout.dtype),
        _ptr(delta), int(bool(accumulate)), _stream(stream)))
    return delta


def splitkv_gemm(layout: int, A: torch.Tensor, B: torch.Tensor, out: Optional[torch.Tensor] = None,
                 out_dtype: torch.dtype = torch.float32, bias: Optional[torch.Tensor] = None,
                 accumulate: bool = False,
                 stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """bf16 product: NT A[M,K] B[N,K]^T, NN A[M,K] B[K,N], TN A[K,M]^T B[K,N] (+ bias, += C)."""
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16 or A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-d bf16")
    if layout == SPLITKV_GEMM_NT:
        (M, K), (N, K2) = A.shape, B.shape
    elif layout == SPLITKV_GEMM_NN:
        (M, K), (K2, N) = A.shape, B.shape
    elif layout == SPLITKV_GEMM_TN:
        (K, M), (K2, N) = A.shape, B.shape
    else:
        raise ValueError("unknown layout")
    if K != K2:
        raise ValueError("inner dimensions differ")
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs out")
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    if out.shape != (M, N):
        raise ValueError("output shape disagrees")
    if bias is not None and (bias.dtype != torch.float32 or bias.numel() != N):
        raise ValueError("bias must be fp32 [N]")
    _check("splitkv_gemm", lib().splitkv_gemm(int(layout), int(M), int(N), int(K), _ptr(A), _ptr(B),
                                              _ptr(out), _dtype_code(out.dtype), _ptr(bias),
                                              int(bool(accumulate)), _stream(stream)))
    return out


def _gemm_shape(layout: int, A: torch.Tensor, B: torch.Tensor):
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16 or A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-d bf16")
    if layout == SPLITKV_GEMM_NT:
        (M, K), (N, K2) = A.shape, B.shape
    elif layout == SPLITKV_GEMM_NN:
        (M, K), (K2, N) = A.shape, B.shape
    elif layout == SPLITKV_GEMM_TN:
        (K, M), (K2, N) = A.shape, B.shape
    else:
        raise ValueError("unknown layout")
    if K != K2:
        raise ValueError("inner dimensions differ")
    return M, N, K


def splitkv_gemm_pair(layout: int, A1: torch.Tensor, B1: torch.Tensor, A2: torch.Tensor,
                      B2: torch.Tensor, out: Optional[torch.Tensor] = None,
                      out_dtype: torch.dtype = torch.float32,
                      bias: Optional[torch.Tensor] = None, accumulate: bool = False,
                      stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """op(A1) op(B1) + op(A2) op(B2) in one pass (both pairs of the same shape)."""
    M, N, K = _gemm_shape(layout, A1, B1)
    if _gemm_shape(layout, A2, B2) != (M, N, K):
        raise ValueError("the two products differ in shape")
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs out")
        out = torch.empty((M, N), dtype=out_dtype, device=A1.device)
    if out.shape != (M, N):
        raise ValueError("output shape disagrees")
    if bias is not None and (bias.dtype != torch.float32 or bias.numel() != N):
        raise ValueError("bias must be fp32 [N]")
    _check("splitkv_gemm_pair", lib().splitkv_gemm_pair(
        int(layout), int(M), int(N), int(K), _ptr(A1), _ptr(B1), _ptr(A2), _ptr(B2), _ptr(out),
        _dtype_code(out.dtype), _ptr(bias), int(bool(accumulate)), _stream(stream)))
    return out


def splitkv_cast_bf16(src: torch.Tensor, out: Optional[torch.Tensor] = None,
                      stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """fp32 tensor -> bf16 tensor of the same shape (round to nearest even)."""
    if src.dtype != torch.float32:
        raise ValueError("src must be fp32")
    if out is None:
        out = torch.empty(src.shape, dtype=torch.bfloat16, device=src.device)
    if out.numel() != src.numel() or out.dtype != torch.bfloat16:
        raise ValueError("output disagrees")
    _check("splitkv_cast_bf16", lib().splitkv_cast_bf16(int(src.numel()), _ptr(src), _ptr(out),
                                                        _stream(stream)))
    return out


def _bwd_args(s, a, block_size, chunk_start, chunk_len, q, k, v, o, dout, lse, dq, scale, delta,
              out):
    """Checks and outputs shared by the two backward entry points."""
    Q, hq, d = q.shape
    hkv = k.shape[1]
    if dout.shape != q.shape or dout.dtype != q.dtype:
        raise ValueError("dout must match q")
    if o is not None and (o.shape != q.shape or o.dtype != q.dtype):
        raise ValueError("o must match q")
    if lse.shape != (Q, hq) or lse.dtype != torch.float32:
        raise ValueError("lse must be fp32 [Q, hq]")
    if dq.shape != q.shape or dq.dtype != torch.float32:
        raise ValueError("dq must be fp32 [Q, hq, d]")
    if k.shape[0] != chunk_start.numel() * chunk_len:
        raise ValueError("k/v rows must equal n_chunks * chunk_len")
    if delta is None:
        if o is None:
            raise ValueError("need o or delta")
        delta = torch.empty((Q, hq), dtype=torch.float32, device=q.device)
    if out is None:
        out = (torch.empty_like(k), torch.empty_like(v))
    dk, dv = out
    an, hd, loc = make_anchors(s, a, block_size), make_heads(hq, hkv, d, q.dtype, scale), \
        make_local(chunk_start, chunk_len)
    return an, hd, loc, delta, dk, dv


def splitkv_attn_bwd(s, a, block_size: int, chunk_start, chunk_len: int, q, k, v, o, dout, lse,
                     dq: torch.Tensor, scale: Optional[float] = None,
                     delta: Optional[torch.Tensor] = None,
                     out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                     workspace: Optional[torch.Tensor] = None,
                     stream: Optional[torch.cuda.Stream] = None):
    """Backward of the local partial with the global lse (and Delta = <do, o>).

    dq (fp32 [Q, hq, d]) is accumulated in place. Pass o=None and delta=... to
    supply Delta directly. A workspace past the minimum (bwd_workspace) holds
    dS from the dK/dV pass, so that dq need not recompute it. Returns (dk, dv,
    delta)."""
    an, hd, loc, delta, dk, dv = _bwd_args(s, a, block_size, chunk_start, chunk_len, q, k, v, o,
                                           dout, lse, dq, scale, delta, out)
    nbytes = splitkv_workspace_bytes(SPLITKV_OP_BWD, an, hd, loc)
    ws_ptr, ws_bytes = _workspace(nbytes, q.device, workspace)
    _check("splitkv_attn_bwd", lib().splitkv_attn_bwd(
        ctypes.byref(an), ctypes.byref(hd), ctypes.byref(loc), _ptr(q), _ptr(k), _ptr(v),
        _ptr(o), _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv),
        ws_ptr, ws_bytes, _stream(stream)))
    return dk, dv, delta


def splitkv_attn_bwd_ds_bytes(s, a, block_size: int, chunk_start, chunk_len: int, hq: int,
                              hkv: int, d: int, dtype: torch.dtype,
                              stream: Optional[torch.cuda.Stream] = None) -> int:
    """Bytes of stored dS (past the minimum backward workspace) that cover every
    query row. Runs on the device and waits for the result."""
    an, hd, loc = make_anchors(s, a, block_size), make_heads(hq, hkv, d, dtype), \
        make_local(chunk_start, chunk_len)
    nbytes = splitkv_workspace_bytes(SPLITKV_OP_BWD, an, hd, loc)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=s.device)
    need = torch.zeros(1, dtype=torch.int64, device=s.device)
    _check("splitkv_attn_bwd_ds_bytes", lib().splitkv_attn_bwd_ds_bytes(
        ctypes.byref(an), ctypes.byref(hd), ctypes.byref(loc), _ptr(ws), nbytes, _ptr(need),
        _stream(stream)))
    (stream if stream is not None else torch.cuda.current_stream()).synchronize()
    return int(need.item())


def bwd_workspace(s, a, block_size: int, chunk_start, chunk_len: int, hq: int, hkv: int, d: int,
                  dtype: torch.dtype, ds_bytes: Optional[int] = None) -> torch.Tensor:
    """A workspace for splitkv_attn_bwd with room for ds_bytes of stored dS
    (default: enough for every query row, from splitkv_attn_bwd_ds_bytes)."""
    if ds_bytes is None:
        ds_bytes = splitkv_attn_bwd_ds_bytes(s, a, block_size, chunk_start, chunk_len, hq, hkv, d,
                                             dtype)
    an, hd, loc = make_anchors(s, a, block_size), make_heads(hq, hkv, d, dtype), \
        make_local(chunk_start, chunk_len)
    nbytes = splitkv_workspace_bytes(SPLITKV_OP_BWD, an, hd, loc)
    return torch.empty(max(nbytes + int(ds_bytes), 1), dtype=torch.uint8, device=s.device)


def splitkv_attn_bwd_noalloc(s, a, block_size: int, chunk_start, chunk_len: int, q, k, v, o,
                             dout, lse, dq: torch.Tensor, scale: Optional[float] = None,
                             delta: torch.Tensor = None,
                             out: Tuple[torch.Tensor, torch.Tensor] = None,
                             stream: Optional[torch.cuda.Stream] = None):
    """splitkv_attn_bwd on the library's fixed per-device scratch: no workspace.
    Allocates nothing, so delta and out (dk, dv) must be given. Returns (dk,
    dv, delta)."""
    if delta is None or out is None:
        raise ValueError("the no-allocation backward needs delta and out=(dk, dv)")
    an, hd, loc, delta, dk, dv = _bwd_args(s, a, block_size, chunk_start, chunk_len, q, k, v, o,
                                           dout, lse, dq, scale, delta, out)
    _check("splitkv_attn_bwd_noalloc", lib().splitkv_attn_bwd_noalloc(
        ctypes.byref(an), ctypes.byref(hd), ctypes.byref(loc), _ptr(q), _ptr(k), _ptr(v),
        _ptr(o), _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv),
        _stream(stream)))
    return dk, dv, delta
