"""Seeded synthetic workloads for the Split-KV per-device hot path.

This module only draws inputs; it holds none of the method's arithmetic (no
costs, no plans, no attention). Both the HIP path's tests and the oracle's
tests take their inputs from here.

Workload shapes follow the systems evaluation of "Split-KV: Efficient Context
Parallelism for Training Diffusion Drafters" (arXiv 2611.05926), §5.1
(Workload): randomly generated fixed-length samples with a 1:3
prompt-to-response ratio, diffusion block size B=16, an anchor budget A per
sample, micro-batch b packed into S = b*L context positions and Q = b*A*B
query rows; head layouts from Table 2 (n_q=32, n_kv=8, d_h=128).

Readings of points the paper leaves open:
  * s_i is the packed start of anchor i's sample (§3.1, Figure 1).
  * anchors are distinct positions drawn uniformly from the sample's response
    span [s + L/4, s + L), sorted ascending, blocks ordered sample-major.
  * values are fp32 normals times a scale, rounded to bf16 with
    round-to-nearest-even; the rounded bits are the ground truth for both sides.

Random streams are keyed: numpy.random.default_rng([seed, tensor_id, unit]),
so any block of q/do or any 256-row segment of k/v can be regenerated alone.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

# tensor ids of the keyed random streams
T_ANCHORS, T_Q, T_K, T_V, T_DO, T_O, T_LSE, T_OPART, T_LPART, T_KB, T_VB = range(11)
# draft-layer tensors around the attention (hidden states, context features,
# projection weights, output bias, output gradient) and plain test matrices
T_X, T_CTX, T_WQ, T_WK, T_WV, T_WO, T_BO, T_DY, T_MAT = range(11, 20)

KV_UNIT = 256  # rows of k/v per keyed random stream


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload (packed micro-batch + head layout + chunking)."""

    name: str
    b: int                 # samples per micro-batch
    L: int                 # per-sample length (context positions)
    A: int                 # anchors per sample
    B: int                 # diffusion block size
    hq: int                # query heads
    hkv: int               # key/value heads
    d: int                 # head dim
    dtype: str             # "bf16" or "fp32"
    scale: float           # std of q/k/v/do values
    P: int                 # CP size (emulated ranks)
    m: int                 # chunk length
    prompt_frac: Tuple[int, int] = (1, 4)   # prompt = first L*num/den positions
    # explicit anchor range [lo, hi) within a sample (overrides the response span)
    anchor_lo: Optional[int] = None
    anchor_hi: Optional[int] = None

    @property
    def S(self) -> int:
        return self.b * self.L

    @property
    def N(self) -> int:
        return self.b * self.A

    @property
    def Q(self) -> int:
        return self.N * self.B

    @property
    def n_chunks(self) -> int:
        return self.S // self.m

    @property
    def J(self) -> int:
        return self.n_chunks // self.P


# The five workloads (sizes from the paper's §5 experiments, one GPU's share).
WORKLOADS = {
    # tiny fp32 correctness case: 1 sample of 1024, 4 anchors in [256,1024),
    # 2 heads of dim 64, chunks of 256 (4 partials) and LPT onto 2 ranks
    "tiny": Workload("tiny", b=1, L=1024, A=4, B=16, hq=2, hkv=2, d=64,
                     dtype="fp32", scale=1.0, P=2, m=256,
                     anchor_lo=256, anchor_hi=1024),
    # weak-scaling share at P=8 (Fig. 6 point): 128k context, 8k queries
    "weak8": Workload("weak8", b=1, L=131072, A=512, B=16, hq=32, hkv=8,
                      d=128, dtype="bf16", scale=128 ** -0.5, P=8, m=4096),
    # strong-scaling share (Fig. 7 at P=8): 4 x 256k, 32k queries
    "strong8": Workload("strong8", b=4, L=262144, A=512, B=16, hq=32, hkv=8,
                        d=128, dtype="bf16", scale=128 ** -0.5, P=8, m=4096),
    # Q:S sweep shares (Fig. 8, P=32, Q=64k, per-sample context 128k)
    "qs4": Workload("qs4", b=2, L=131072, A=2048, B=16, hq=32, hkv=8, d=128,
                    dtype="bf16", scale=128 ** -0.5, P=32, m=4096),
    "qs8": Workload("qs8", b=4, L=131072, A=1024, B=16, hq=32, hkv=8, d=128,
                    dtype="bf16", scale=128 ** -0.5, P=32, m=4096),
    "qs16": Workload("qs16", b=8, L=131072, A=512, B=16, hq=32, hkv=8, d=128,
                     dtype="bf16", scale=128 ** -0.5, P=32, m=4096),
    "qs32": Workload("qs32", b=16, L=131072, A=256, B=16, hq=32, hkv=8, d=128,
                     dtype="bf16", scale=128 ** -0.5, P=32, m=4096),
    # weak-scaling share at P=64: 1M context, 8k queries, 16k local keys
    "weak64": Workload("weak64", b=1, L=1048576, A=512, B=16, hq=32, hkv=8,
                       d=128, dtype="bf16", scale=128 ** -0.5, P=64, m=4096),
}


def rng(seed: int, tensor_id: int, unit: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tensor_id), int(unit)])


# ----------------------------------------------------------------------------
# bf16 helpers (bit-level; numpy has no bfloat16)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_values(g: np.random.Generator, shape, scale: float, dtype: str) -> np.ndarray:
    """fp32 N(0,1)*scale; for bf16 returns uint16 bits, for fp32 float32."""
    x = g.standard_normal(size=shape, dtype=np.float32) * np.float32(scale)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x.astype(np.float32)


def as_f32(x: np.ndarray) -> np.ndarray:
    """Exact fp32 values of a generated array (bf16 bits or fp32)."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x)
    return np.asarray(x, dtype=np.float32)


# ----------------------------------------------------------------------------
# anchors
# ----------------------------------------------------------------------------
def sample_anchors(g: np.random.Generator, sample_start: int, lo: int, hi: int,
                   count: int) -> np.ndarray:
    """`count` distinct positions uniform in [sample_start+lo, sample_start+hi), sorted."""
    span = hi - lo
    if count > span:
        raise ValueError("more anchors than positions in the span")
    pos = g.choice(span, size=count, replace=False)
    pos.sort()
    return (pos + lo + sample_start).astype(np.int64)


def workload_anchors(w: Workload, seed: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """(s, a) int64 arrays of length N for a workload; blocks are sample-major."""
    if w.anchor_lo is not None:
        lo, hi = w.anchor_lo, w.anchor_hi
    else:
        num, den = w.prompt_frac
        lo, hi = w.L * num // den, w.L
    s_all, a_all = [], []
    for u in range(w.b):
        start = u * w.L
        a = sample_anchors(rng(seed, T_ANCHORS, u), start, lo, hi, w.A)
        s_all.append(np.full(w.A, start, dtype=np.int64))
        a_all.append(a)
    return np.concatenate(s_all), np.concatenate(a_all)


def sample_bounds(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """Packed sample starts and lengths."""
    starts = np.arange(w.b, dtype=np.int64) * w.L
    return starts, np.full(w.b, w.L, dtype=np.int64)


# ----------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------
def gen_rows_by_block(w: Workload, seed: int, tensor_id: int, blocks) -> np.ndarray:
    """q- or do-shaped values [len(blocks)*B, hq, d] for the given blocks."""
    out = [normal_values(rng(seed, tensor_id, int(i)), (w.B, w.hq, w.d), w.scale, w.dtype)
           for i in blocks]
    return np.concatenate(out, axis=0)


def gen_q(w: Workload, seed: int = 0, blocks=None) -> np.ndarray:
    blocks = range(w.N) if blocks is None else blocks
    return gen_rows_by_block(w, seed, T_Q, blocks)


def gen_do(w: Workload, seed: int = 0, blocks=None) -> np.ndarray:
    blocks = range(w.N) if blocks is None else blocks
    return gen_rows_by_block(w, seed, T_DO, blocks)


def gen_kv_rows(w: Workload, seed: int, which: str, start: int, count: int) -> np.ndarray:
    """k or v values [count, hkv, d] for global context rows [start, start+count)."""
    tid = {"k": T_K, "v": T_V}[which]
    u0, u1 = start // KV_UNIT, (start + count + KV_UNIT - 1) // KV_UNIT
    parts = [normal_values(rng(seed, tid, u), (KV_UNIT, w.hkv, w.d), w.scale, w.dtype)
             for u in range(u0, u1)]
    full = np.concatenate(parts, axis=0)
    off = start - u0 * KV_UNIT
    return np.ascontiguousarray(full[off:off + count])


def gen_block_kv(w: Workload, seed: int, which: str, blocks=None) -> np.ndarray:
    """Keys or values of the draft blocks' own B tokens [len(blocks)*B, hkv, d]
    (the "block keys" of Figure 1: one row per query row, in block order)."""
    tid = {"k": T_KB, "v": T_VB}[which]
    blocks = range(w.N) if blocks is None else blocks
    return np.concatenate([normal_values(rng(seed, tid, int(i)), (w.B, w.hkv, w.d), w.scale,
                                         w.dtype) for i in blocks], axis=0)


def gen_local_kv(w: Workload, seed: int, chunk_ids, which: str) -> np.ndarray:
    """A rank's local buffer [len(chunk_ids)*m, hkv, d]: its chunks in the given order."""
    return np.concatenate([gen_kv_rows(w, seed, which, int(j) * w.m, w.m) for j in chunk_ids],
                          axis=0)


def gen_partials(P: int, rows: int, d: int, seed: int, dtype: str,
                 ninf_frac: float = 0.1, lse_spread: float = 4.0):
    """Synthetic (o_parts [P,rows,d], lse_parts [P,rows] fp32) for merge tests.

    A fraction of (p, row) entries are empty partials (lse = -inf, o = 0) and
    one row in 16 is empty in every partial.
    """
    g = rng(seed, T_OPART, 0)
    o = g.standard_normal(size=(P, rows, d), dtype=np.float32)
    lse = (g.standard_normal(size=(P, rows), dtype=np.float32) * np.float32(lse_spread)
           + np.float32(8.0))
    empty = g.random(size=(P, rows)) < ninf_frac
    empty[:, ::16] = True
    lse[empty] = -np.inf
    o[empty] = 0.0
    if dtype == "bf16":
        return f32_to_bf16_bits(o), lse
    return o, lse


def gen_lse_like(rows: int, hq: int, seed: int, center: float = 10.0) -> np.ndarray:
    """Synthetic log-sum-exp values [rows, hq] fp32 for backward inputs."""
    g = rng(seed, T_LSE, 0)
    return (center + 0.5 * g.standard_normal(size=(rows, hq))).astype(np.float32)


def gen_o_like(w: Workload, seed: int, rows: int) -> np.ndarray:
    """Synthetic forward output [rows, hq, d] (same dtype as the workload)."""
    return normal_values(rng(seed, T_O, 0), (rows, w.hq, w.d), w.scale, w.dtype)


def random_tiny_anchors(g: np.random.Generator, n_samples: int, L: int, A: int,
                        prompt: int) -> Tuple[np.ndarray, np.ndarray]:
    """Small random packed batch: per sample, A distinct anchors in [prompt, L)."""
    s_all, a_all = [], []
    for u in range(n_samples):
        a = sample_anchors(g, u * L, prompt, L, A)
        s_all.append(np.full(A, u * L, dtype=np.int64))
        a_all.append(a)
    return np.concatenate(s_all), np.concatenate(a_all)


def gen_matrix(rows: int, cols: int, seed: int, tensor_id: int, scale: float = 1.0,
               dtype: str = "bf16", first_row: int = 0) -> np.ndarray:
    """Rows [first_row, first_row + rows) of a seeded [*, cols] N(0,1)*scale matrix,
    drawn in units of 256 rows so that any row range regenerates on its own."""
    out = []
    r = first_row
    end = first_row + rows
    while r < end:
        unit = r // KV_UNIT
        u0 = unit * KV_UNIT
        block = normal_values(rng(seed, tensor_id, unit), (KV_UNIT, cols), scale, dtype)
        take = min(end, u0 + KV_UNIT) - r
        out.append(block[r - u0:r - u0 + take])
        r += take
    if not out:
        return normal_values(rng(seed, tensor_id, 0), (0, cols), scale, dtype)
    return np.ascontiguousarray(np.concatenate(out, axis=0))


def list_workloads() -> List[str]:
    return list(WORKLOADS)
