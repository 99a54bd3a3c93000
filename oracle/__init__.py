"""Python face of the fp64 CPU oracle (liboracle.so, built from oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the package smoke check
and the CPU-baseline leg of the benchmark, never by the product path. It shares
no code with the HIP library; only the seeded input generators are common.

Each wrapper converts numpy inputs to the C types and returns numpy outputs;
all arithmetic is in oracle.c (see its header for the equations followed),
except that full_mask_bwd adds the two key sets' dq contributions and the
draft-layer composition (draft_layer_forward / draft_layer_backward) takes its
projections as numpy fp64 matrix products around the C attention routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib: Optional[ctypes.CDLL] = None

i64p = ctypes.POINTER(ctypes.c_int64)
i32p = ctypes.POINTER(ctypes.c_int32)
f64p = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True, sanitize_to: Optional[str] = None) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, IEEE semantics: no fast-math).
    With sanitize_to, build instead an AddressSanitizer + UndefinedBehavior-
    Sanitizer copy at that path (any finding aborts); load it by running with
    SPLITKV_ORACLE_LIB=<path> and gcc's libasan preloaded."""
    out = sanitize_to or _LIB
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        san = (["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                "-fno-omit-frame-pointer", "-g"] if sanitize_to else [])
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-fno-fast-math"] + san + ["-o", tmp, _SRC, "-lm"])
        os.replace(tmp, out)
    return out


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = os.environ.get("SPLITKV_ORACLE_LIB") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(path)
        L.oracle_validate_anchors.argtypes = [ctypes.c_int64, i64p, i64p, ctypes.c_int64, i64p]
        L.oracle_locality_match.argtypes = [i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                            i32p, i64p, i64p]
        L.oracle_locality_match.restype = ctypes.c_int
        L.oracle_placement_rows.argtypes = [i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                            i32p, i64p, i64p]
        L.oracle_placement_rows.restype = ctypes.c_int
        L.oracle_omp_threads.argtypes = []
        L.oracle_omp_threads.restype = ctypes.c_int
        L.oracle_anchor_profile.argtypes = [ctypes.c_int64, i64p, i64p, ctypes.c_int64,
                                            ctypes.c_int64, i64p]
        for name in ("oracle_chunk_costs", "oracle_chunk_costs_prefix"):
            getattr(L, name).argtypes = [ctypes.c_int64, i64p, i64p, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int64, i64p]
        L.oracle_lpt.argtypes = [ctypes.c_int64, i64p, ctypes.c_int32, ctypes.c_int32,
                                 i32p, i32p, i64p]
        L.oracle_lpt.restype = ctypes.c_int
        L.oracle_zigzag_loads.argtypes = [ctypes.c_int64, i64p, i64p, i64p, ctypes.c_int32, i64p]
        L.oracle_zigzag_loads.restype = ctypes.c_int
        L.oracle_contiguous_loads.argtypes = [ctypes.c_int64, i64p, ctypes.c_int32, i64p]
        L.oracle_contiguous_loads.restype = ctypes.c_int
        L.oracle_baseline_plan.argtypes = [ctypes.c_int32, ctypes.c_int64, i64p, i64p, i64p,
                                           ctypes.c_int32, i64p, i64p]
        L.oracle_baseline_plan.restype = ctypes.c_int64
        L.oracle_lse_reduce.argtypes = [ctypes.c_int32, ctypes.c_int64, f64p, f64p]
        L.oracle_lse_reduce.restype = None
        L.oracle_lse_rescale.argtypes = [ctypes.c_int64, ctypes.c_int32, f64p, f64p, f64p, f64p]
        L.oracle_lse_rescale.restype = None
        L.oracle_imbalance.argtypes = [ctypes.c_int32, i64p, ctypes.c_int64, ctypes.c_int64]
        L.oracle_imbalance.restype = ctypes.c_double
        L.oracle_partial_attn.argtypes = [ctypes.c_int64, i64p, ctypes.c_int64, i64p, i64p,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_double, f64p, ctypes.c_int64, i64p,
                                          f64p, f64p, f64p, f64p]
        L.oracle_merge.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, f64p, f64p,
                                   f64p, f64p]
        L.oracle_delta.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, f64p, f64p,
                                   f64p]
        L.oracle_attn_bwd.argtypes = [ctypes.c_int64, ctypes.c_int64, i64p, i64p,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_double, f64p, f64p, f64p, f64p,
                                      ctypes.c_int64, i64p, f64p, f64p,
                                      ctypes.c_int64, i64p, f64p, ctypes.c_int64, i64p,
                                      f64p, f64p]
        _lib = L
    return _lib


def _p(x: np.ndarray, ctype):
    return x.ctypes.data_as(ctypes.POINTER(ctype))


def _i64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.int64)


def _f64(x) -> np.ndarray:
    if getattr(x, "dtype", None) == np.uint16:
        raise TypeError("pass widened values, not raw bf16 bits")
    return np.ascontiguousarray(x, dtype=np.float64)


# ---------------------------------------------------------------- planner --
def validate_anchors(s, a, S: int) -> Tuple[int, int]:
    """(number of blocks whose window [s_i, a_i) is not inside [0, S), index of
    the first such block or -1): §3.1 / Figure 1 of the Split-KV paper."""
    s, a = _i64(s), _i64(a)
    if len(s) != len(a):
        raise ValueError("s and a differ in length")
    out = np.zeros(2, np.int64)
    lib().oracle_validate_anchors(len(s), _p(s, ctypes.c_int64), _p(a, ctypes.c_int64), int(S),
                                  _p(out, ctypes.c_int64))
    return int(out[0]), int(out[1])


def anchor_profile(s, a, B: int, S: int) -> np.ndarray:
    s, a = _i64(s), _i64(a)
    out = np.zeros(S, dtype=np.int64)
    lib().oracle_anchor_profile(len(s), _p(s, ctypes.c_int64), _p(a, ctypes.c_int64), B, S,
                                _p(out, ctypes.c_int64))
    return out


def chunk_costs(s, a, B: int, n_chunks: int, m: int, form: str = "direct") -> np.ndarray:
    s, a = _i64(s), _i64(a)
    out = np.zeros(n_chunks, dtype=np.int64)
    fn = lib().oracle_chunk_costs if form == "direct" else lib().oracle_chunk_costs_prefix
    fn(len(s), _p(s, ctypes.c_int64), _p(a, ctypes.c_int64), B, n_chunks, m,
       _p(out, ctypes.c_int64))
    return out


def lpt(cost, P: int, J: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Returns (owner [PJ] int32, bundles [P, J] int32, load [P] int64)."""
    cost = _i64(cost)
    owner = np.zeros(len(cost), dtype=np.int32)
    bundles = np.zeros((P, J), dtype=np.int32)
    load = np.zeros(P, dtype=np.int64)
    rc = lib().oracle_lpt(len(cost), _p(cost, ctypes.c_int64), P, J, _p(owner, ctypes.c_int32),
                          _p(bundles, ctypes.c_int32), _p(load, ctypes.c_int64))
    if rc != 0:
        raise ValueError("oracle_lpt: number of chunks must equal P*J")
    return owner, bundles, load


def plan(s, a, B: int, S: int, m: int, P: int, J: int):
    """Eq. 6 costs then LPT; returns (cost, owner, bundles, load)."""
    cost = chunk_costs(s, a, B, S // m, m)
    owner, bundles, load = lpt(cost, P, J)
    return cost, owner, bundles, load


def locality_match(bundles, m: int):
    """Locality matching of §4.2: place the LPT bundles (int [P][J] chunk ids)
    on physical ranks keeping the most context rows in place, where rank r
    first holds chunks r*J .. r*J + J - 1. Returns (perm [P]: bundle -> rank,
    send int64 [P][P]: rows rank src sends to rank dst, kept, moved)."""
    b = np.ascontiguousarray(bundles, dtype=np.int32)
    P, J = b.shape
    perm = np.zeros(P, np.int32)
    send = np.zeros((P, P), np.int64)
    km = np.zeros(2, np.int64)
    rc = lib().oracle_locality_match(_p(b, ctypes.c_int32), P, J, int(m),
                                     _p(perm, ctypes.c_int32), _p(send, ctypes.c_int64),
                                     _p(km, ctypes.c_int64))
    if rc != 0:
        raise ValueError("oracle_locality_match: invalid arguments")
    return perm, send, int(km[0]), int(km[1])


def omp_threads() -> int:
    """Threads the oracle's parallel loops use on this host."""
    return int(lib().oracle_omp_threads())


def placement_rows(bundles, perm, m: int):
    """The all-to-all that one placement of the bundles implies (§4.2): chunk j
    of bundle b moves from its home rank j // J to rank perm[b]. Returns (send
    int64 [P][P]: rows rank src sends to rank dst, kept, moved). Raises if perm
    is not a permutation."""
    b = np.ascontiguousarray(bundles, dtype=np.int32)
    P, J = b.shape
    pm = np.ascontiguousarray(perm, dtype=np.int32)
    if pm.shape != (P,):
        raise ValueError("perm must have one entry per bundle")
    send = np.zeros((P, P), np.int64)
    km = np.zeros(2, np.int64)
    rc = lib().oracle_placement_rows(_p(b, ctypes.c_int32), P, J, int(m), _p(pm, ctypes.c_int32),
                                     _p(send, ctypes.c_int64), _p(km, ctypes.c_int64))
    if rc != 0:
        raise ValueError("oracle_placement_rows: perm is not a permutation")
    return send, int(km[0]), int(km[1])


def zigzag_loads(sample_start, sample_len, prof, P: int) -> np.ndarray:
    st, ln, pr = _i64(sample_start), _i64(sample_len), _i64(prof)
    out = np.zeros(P, dtype=np.int64)
    rc = lib().oracle_zigzag_loads(len(st), _p(st, ctypes.c_int64), _p(ln, ctypes.c_int64),
                                   _p(pr, ctypes.c_int64), P, _p(out, ctypes.c_int64))
    if rc != 0:
        raise ValueError("zigzag needs sample lengths divisible by 2P")
    return out


def contiguous_loads(prof, P: int) -> np.ndarray:
    pr = _i64(prof)
    out = np.zeros(P, dtype=np.int64)
    if lib().oracle_contiguous_loads(len(pr), _p(pr, ctypes.c_int64), P,
                                     _p(out, ctypes.c_int64)) != 0:
        raise ValueError("context length must be divisible by P")
    return out


def baseline_plan(strategy: int, sample_start, sample_len, prof, P: int):
    """No balance (strategy 0) or Zigzag (1) as ranges: (range_cost [R], load [P])."""
    st, ln, pr = _i64(sample_start), _i64(sample_len), _i64(prof)
    R = P if strategy == 0 else 2 * P * len(st)
    cost = np.zeros(R, dtype=np.int64)
    load = np.zeros(P, dtype=np.int64)
    got = lib().oracle_baseline_plan(int(strategy), len(st), _p(st, ctypes.c_int64),
                                     _p(ln, ctypes.c_int64), _p(pr, ctypes.c_int64), P,
                                     _p(cost, ctypes.c_int64), _p(load, ctypes.c_int64))
    if got < 0:
        raise ValueError("sample lengths do not divide into the assignment's ranges")
    assert got == R
    return cost, load


def imbalance(ctx_load, n_blocks: int, B: int) -> float:
    ld = _i64(ctx_load)
    return float(lib().oracle_imbalance(len(ld), _p(ld, ctypes.c_int64), n_blocks, B))


# -------------------------------------------------------------- attention --
def partial_attn(rows, B: int, s, a, q_sel, key_pos, k, v, scale: float):
    """Eq. 3 for the given rows. q_sel [n, hq, d]; k, v [n_keys, hkv, d] (widened to fp64).

    Returns (o [n, hq, d] fp64, lse [n, hq] fp64)."""
    rows, s, a, key_pos = _i64(rows), _i64(s), _i64(a), _i64(key_pos)
    q_sel, k, v = _f64(q_sel), _f64(k), _f64(v)
    n, hq, d = q_sel.shape
    hkv = k.shape[1]
    assert k.shape == v.shape and k.shape[0] == len(key_pos) and len(rows) == n
    o = np.zeros((n, hq, d), dtype=np.float64)
    lse = np.zeros((n, hq), dtype=np.float64)
    lib().oracle_partial_attn(n, _p(rows, ctypes.c_int64), B, _p(s, ctypes.c_int64),
                              _p(a, ctypes.c_int64), hq, hkv, d, float(scale),
                              _p(q_sel, ctypes.c_double), len(key_pos),
                              _p(key_pos, ctypes.c_int64), _p(k, ctypes.c_double),
                              _p(v, ctypes.c_double), _p(o, ctypes.c_double),
                              _p(lse, ctypes.c_double))
    return o, lse


def merge(o_parts, lse_parts):
    """Eq. 4. o_parts [P, rows, d], lse_parts [P, rows] -> (o [rows, d], lse [rows])."""
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    P, rows, d = o_parts.shape
    o = np.zeros((rows, d), dtype=np.float64)
    lse = np.zeros(rows, dtype=np.float64)
    lib().oracle_merge(P, rows, d, _p(o_parts, ctypes.c_double), _p(lse_parts, ctypes.c_double),
                       _p(o, ctypes.c_double), _p(lse, ctypes.c_double))
    return o, lse


def lse_reduce(lse_parts) -> np.ndarray:
    """lse_parts [P, rows] -> lse [rows] (the LSE half of Eq. 4)."""
    lp = _f64(lse_parts)
    P, rows = lp.shape
    out = np.zeros(rows, dtype=np.float64)
    lib().oracle_lse_reduce(P, rows, _p(lp, ctypes.c_double), _p(out, ctypes.c_double))
    return out


def lse_rescale(o_part, lse_part, lse) -> np.ndarray:
    """o_part [rows, d], lse_part, lse [rows] -> exp(lse_part - lse) o_part (0 if empty)."""
    o_part, lp, l = _f64(o_part), _f64(lse_part), _f64(lse)
    rows, d = o_part.shape
    out = np.zeros((rows, d), dtype=np.float64)
    lib().oracle_lse_rescale(rows, d, _p(o_part, ctypes.c_double), _p(lp, ctypes.c_double),
                             _p(l, ctypes.c_double), _p(out, ctypes.c_double))
    return out


def delta(o, dout) -> np.ndarray:
    """Delta[r, h] = <do[r, h], o[r, h]> for o, do [rows, hq, d]."""
    o, dout = _f64(o), _f64(dout)
    rows, hq, d = o.shape
    out = np.zeros((rows, hq), dtype=np.float64)
    lib().oracle_delta(rows, hq, d, _p(o, ctypes.c_double), _p(dout, ctypes.c_double),
                       _p(out, ctypes.c_double))
    return out


def attn_bwd(B: int, s, a, q, dout, lse, dlt, key_pos, k, v, scale: float,
             dq_rows, dkv_keys):
    """Backward of the local partial given global lse and Delta.

    q, dout [Q, hq, d]; lse, dlt [Q, hq]; k, v [n_keys, hkv, d].
    Returns (dq [len(dq_rows), hq, d], dk, dv [len(dkv_keys), hkv, d]) in fp64."""
    s, a, key_pos = _i64(s), _i64(a), _i64(key_pos)
    q, dout, k, v = _f64(q), _f64(dout), _f64(k), _f64(v)
    lse, dlt = _f64(lse), _f64(dlt)
    dq_rows, dkv_keys = _i64(dq_rows), _i64(dkv_keys)
    Q, hq, d = q.shape
    hkv = k.shape[1]
    dq = np.zeros((len(dq_rows), hq, d), dtype=np.float64)
    dk = np.zeros((len(dkv_keys), hkv, d), dtype=np.float64)
    dv = np.zeros((len(dkv_keys), hkv, d), dtype=np.float64)
    lib().oracle_attn_bwd(Q, B, _p(s, ctypes.c_int64), _p(a, ctypes.c_int64), hq, hkv, d,
                          float(scale), _p(q, ctypes.c_double), _p(dout, ctypes.c_double),
                          _p(lse, ctypes.c_double), _p(dlt, ctypes.c_double), len(key_pos),
                          _p(key_pos, ctypes.c_int64), _p(k, ctypes.c_double),
                          _p(v, ctypes.c_double), len(dq_rows), _p(dq_rows, ctypes.c_int64),
                          _p(dq, ctypes.c_double), len(dkv_keys), _p(dkv_keys, ctypes.c_int64),
                          _p(dk, ctypes.c_double), _p(dv, ctypes.c_double))
    return dq, dk, dv


# ------------------------------------------------- full mask (own blocks) --
def own_block_windows(n_blocks: int, B: int):
    """Windows of the own-block part of the mask (Figure 1 and §3.1 of the Split-KV
    paper: a block's rows also see all B tokens of their own block). With the
    block keys in block order at positions 0 .. n_blocks*B - 1, block i's window
    is [iB, (i+1)B). Returns (s', a', key positions)."""
    i = np.arange(n_blocks, dtype=np.int64)
    return i * B, (i + 1) * B, np.arange(n_blocks * B, dtype=np.int64)


def full_mask_attn(B: int, s, a, q, ctx_pos, k, v, kb, vb, scale: float):
    """Attention under the whole block-sparse mask of Figure 1 for every query
    row: the context window [s_i, a_i) of the context keys (positions ctx_pos)
    and the own block's B block keys (kb, vb [Q, hkv, d], block order). Written
    as the method writes it: the two partials (Eq. 3) merged by Eq. 4.
    Returns (o [Q, hq, d], lse [Q, hq]) in fp64."""
    q = _f64(q)
    Q, hq, d = q.shape
    rows = np.arange(Q, dtype=np.int64)
    o_c, l_c = partial_attn(rows, B, s, a, q, ctx_pos, k, v, scale)
    sb, ab, pb = own_block_windows(Q // B, B)
    o_b, l_b = partial_attn(rows, B, sb, ab, q, pb, kb, vb, scale)
    o, lse = merge(np.stack([o_c.reshape(Q * hq, d), o_b.reshape(Q * hq, d)]),
                   np.stack([l_c.reshape(-1), l_b.reshape(-1)]))
    return o.reshape(Q, hq, d), lse.reshape(Q, hq)


def full_mask_bwd(B: int, s, a, q, dout, o, lse, ctx_pos, k, v, kb, vb, scale: float):
    """Backward of full_mask_attn given its output o and lse (Algorithm 1: the
    global lse and Delta = <do, o>, then each key set's local backward; dq sums
    the two). Returns (dq [Q, hq, d], dk, dv [n_ctx, hkv, d], dkb, dvb [Q, hkv, d])."""
    q = _f64(q)
    Q = q.shape[0]
    dl = delta(o, dout)
    rows = np.arange(Q, dtype=np.int64)
    dq_c, dk, dv = attn_bwd(B, s, a, q, dout, lse, dl, ctx_pos, k, v, scale, rows,
                            np.arange(len(_i64(ctx_pos)), dtype=np.int64))
    sb, ab, pb = own_block_windows(Q // B, B)
    dq_b, dkb, dvb = attn_bwd(B, sb, ab, q, dout, lse, dl, pb, kb, vb, scale, rows,
                              np.arange(Q, dtype=np.int64))
    return dq_c + dq_b, dk, dv, dkb, dvb


def local_key_positions(chunk_ids, m: int) -> np.ndarray:
    """Global context position of each row of a local buffer made of the given chunks
    (chunk j covers [j*m, (j+1)*m)), in buffer order."""
    ids = _i64(chunk_ids)
    return (ids[:, None] * m + np.arange(m, dtype=np.int64)[None, :]).reshape(-1)


# -------------------------------------------------------------- draft layer --
def draft_layer_forward(X, U, Wq, Wk, Wv, Wo, bo, s, a, B: int, hq: int, hkv: int, d: int,
                        scale: float, bundles, m: int, own_blocks: bool = False):
    """One draft layer's attention block in Split-KV form (Algorithm 1, forward):
    q = QProj(X) = X Wq^T (all query rows on every rank); rank p projects its own
    context rows k_p = U_p Wk^T, v_p = U_p Wv^T (U_p: the rows of its chunks,
    `bundles[p]`, each of m positions); Attn gives (o_p, l_p) (Eq. 3); the LSE
    statistics are reduced and each rank rescales its partial (Eq. 4); OProj is
    applied to every rescaled partial and the results summed, the bias added once
    (Eq. 5). Shapes: X [Q, H], U [S, H], Wq [hq d, H], Wk, Wv [hkv d, H],
    Wo [H, hq d], bo [H]. With own_blocks, the whole mask of Figure 1: every
    block's rows also attend their block's B tokens, whose keys and values are
    the same projections of the block rows' own hidden states (kb = X Wk^T,
    vb = X Wv^T), one more partial in the merge. Returns a dict of the fp64
    intermediates and Y [Q, H]."""
    X, U, Wq, Wk, Wv, Wo, bo = (_f64(x) for x in (X, U, Wq, Wk, Wv, Wo, bo))
    Q = X.shape[0]
    q = (X @ Wq.T).reshape(Q, hq, d)
    rows = np.arange(Q)
    parts = []
    for chunks in bundles:
        pos = local_key_positions(chunks, m)
        k = (U[pos] @ Wk.T).reshape(len(pos), hkv, d)
        v = (U[pos] @ Wv.T).reshape(len(pos), hkv, d)
        o_p, l_p = partial_attn(rows, B, s, a, q, pos, k, v, scale)
        parts.append({"pos": pos, "k": k, "v": v, "o": o_p, "l": l_p})
    if own_blocks:
        bs, ba, bpos = own_block_windows(len(s), B)
        kb = (X @ Wk.T).reshape(Q, hkv, d)
        vb = (X @ Wv.T).reshape(Q, hkv, d)
        o_b, l_b = partial_attn(rows, B, bs, ba, q, bpos, kb, vb, scale)
        parts.append({"pos": None, "k": kb, "v": vb, "o": o_b, "l": l_b, "own": True})
    lse = lse_reduce(np.stack([pt["l"].reshape(-1) for pt in parts]))
    Y = np.zeros((Q, Wo.shape[0]), dtype=np.float64)
    for pt in parts:
        pt["obar"] = lse_rescale(pt["o"].reshape(-1, d), pt["l"].reshape(-1), lse).reshape(Q, hq, d)
        Y += pt["obar"].reshape(Q, hq * d) @ Wo.T
    Y += bo[None, :]
    return {"q": q, "parts": parts, "lse": lse.reshape(Q, hq), "Y": Y}


def draft_layer_backward(fwd, dY, X, U, Wq, Wk, Wv, Wo, s, a, B: int, hq: int, hkv: int,
                         d: int, scale: float):
    """Backward of draft_layer_forward (Algorithm 1, backward): OProjBwd gives the
    output-gradient do = dY Wo (the same for every rank, since Y sums the ranks'
    projections), dWo = sum_p dY^T obar_p and dbo = the column sums of dY;
    MERGE_BWD all-reduces Delta = sum_p <do, obar_p>; each rank's AttnBwd_p with
    the global lse and Delta gives its dq contribution (summed over ranks), dk_p
    and dv_p; QProjBwd and KeyValueProjBwd give dX, dWq and each rank's dU_p
    (its own context rows), dWk, dWv (with the own-block partial, its key and
    value gradients flow back through the same projections into dX). Returns a
    dict of fp64 gradients; dU is assembled over the ranks' rows."""
    dY, X, U, Wq, Wk, Wv, Wo = (_f64(x) for x in (dY, X, U, Wq, Wk, Wv, Wo))
    Q = X.shape[0]
    q, lse, parts = fwd["q"], fwd["lse"], fwd["parts"]
    do = (dY @ Wo).reshape(Q, hq, d)
    dWo = sum(dY.T @ pt["obar"].reshape(Q, hq * d) for pt in parts)
    dbo = dY.sum(axis=0)
    dlt = sum(delta(pt["obar"], do) for pt in parts)
    rows = np.arange(Q)
    dq = np.zeros((Q, hq, d))
    dU = np.zeros_like(U)
    dWk = np.zeros_like(Wk)
    dWv = np.zeros_like(Wv)
    dX = np.zeros_like(X)
    for pt in parts:
        if pt.get("own"):
            # own-block partial: keys are the block rows' projections of X
            bs, ba, bpos = own_block_windows(len(s), B)
            dq_p, dk, dv = attn_bwd(B, bs, ba, q, do, lse, dlt, bpos, pt["k"], pt["v"], scale,
                                    rows, np.arange(Q))
            dq += dq_p
            dk2, dv2 = dk.reshape(Q, hkv * d), dv.reshape(Q, hkv * d)
            dX += dk2 @ Wk + dv2 @ Wv
            dWk += dk2.T @ X
            dWv += dv2.T @ X
            continue
        n = len(pt["pos"])
        dq_p, dk, dv = attn_bwd(B, s, a, q, do, lse, dlt, pt["pos"], pt["k"], pt["v"], scale,
                                rows, np.arange(n))
        dq += dq_p
        dk2, dv2 = dk.reshape(n, hkv * d), dv.reshape(n, hkv * d)
        dU[pt["pos"]] += dk2 @ Wk + dv2 @ Wv
        dWk += dk2.T @ U[pt["pos"]]
        dWv += dv2.T @ U[pt["pos"]]
    dq2 = dq.reshape(Q, hq * d)
    dX += dq2 @ Wq
    return {"dX": dX, "dWq": dq2.T @ X, "dU": dU, "dWk": dWk, "dWv": dWv, "dWo": dWo,
            "dbo": dbo, "do": do, "delta": dlt, "dq": dq}

