"""One draft layer's attention block in Split-KV form on one GPU (Algorithm 1 of
"Split-KV: Efficient Context Parallelism for Training Diffusion Drafters"),
with all P ranks emulated in sequence.

Forward: q = QProj(X) = X Wq^T for all query rows; rank p projects its own
context rows, k_p = U_p Wk^T and v_p = U_p Wv^T; Attn gives (o_p, lse_p)
(Eq. 3); the LSE statistics are reduced (the all-reduce's local stand-in) and
each rank rescales its partial, obar_p = exp(lse_p - lse) o_p (Eq. 4); the
output projection is applied to each rescaled partial and the results summed,
with the bias added once (Eq. 5): Y = sum_p obar_p Wo^T + bo.

Backward (dY): dbo = column sums of dY; do = dY Wo (the same for every rank);
dWo = sum_p dY^T obar_p; Delta = sum_p <do, obar_p> (MERGE_BWD's all-reduce);
each rank's AttnBwd_p with the global lse and Delta adds its dq share and gives
dk_p, dv_p; then dX = dq Wq, dWq = dq^T X, dU_p = dk_p Wk + dv_p Wv,
dWk = sum_p dk_p^T U_p, dWv = sum_p dv_p^T U_p.

With own_blocks, the whole mask of Figure 1: every block's rows also attend
their block's B tokens, whose keys and values are the same projections of the
block rows' hidden states (kb = X Wk^T, vb = X Wv^T). They form one more local
segment (windows [iB, (i+1)B) over the block keys in block order) whose
partial joins the merge and the output projection, and whose key and value
gradients flow back through Wk, Wv into dX, dWk and dWv.

Every step is a library call (argument marshalling only): the products run in
splitkv_gemm / splitkv_gemm_pair, the attention in splitkv_attn_fwd / splitkv_attn_bwd, the merge
halves in splitkv_lse_reduce / splitkv_lse_rescale, Delta in splitkv_delta.
Operands of the products are bf16; Y and the weight and input gradients fp32.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import torch

from . import binding

NT, NN, TN = binding.SPLITKV_GEMM_NT, binding.SPLITKV_GEMM_NN, binding.SPLITKV_GEMM_TN


class DraftLayer:
    """Buffers and the call sequence of one draft layer (all ranks on one GPU).

    s, a: device int64 anchors [N]; B: block size; chunk_starts[p]: device int64
    chunk starts of rank p (ascending); m: chunk length; weights: bf16 Wq
    [hq d, H], Wk, Wv [hkv d, H], Wo [H, hq d] and fp32 bo [H]. store_ds: the
    backward's workspace holds each partial's dS, so that dq is not
    recomputed."""

    def __init__(self, s: torch.Tensor, a: torch.Tensor, B: int, hq: int, hkv: int, d: int,
                 chunk_starts: Sequence[torch.Tensor], m: int, Wq: torch.Tensor,
                 Wk: torch.Tensor, Wv: torch.Tensor, Wo: torch.Tensor, bo: torch.Tensor,
                 scale: Optional[float] = None, own_blocks: bool = False,
                 store_ds: bool = True):
        self.s, self.a, self.B = s, a, B
        self.hq, self.hkv, self.d, self.m = hq, hkv, d, m
        self.cs = list(chunk_starts)
        self.P = len(self.cs)
        self.Wq, self.Wk, self.Wv, self.Wo, self.bo = Wq, Wk, Wv, Wo, bo
        self.H = Wo.shape[0]
        self.scale = d ** -0.5 if scale is None else scale
        self.Q = s.numel() * B
        self.own = own_blocks
        dev = s.device
        Q = self.Q
        P = self.P + (1 if own_blocks else 0)    # partials in the merge
        self.n_parts = P
        bf, f32 = dict(dtype=torch.bfloat16, device=dev), dict(dtype=torch.float32, device=dev)
        self.q = torch.empty((Q, hq * d), **bf)
        self.o_parts = torch.empty((P, Q, hq, d), **bf)     # o_p, then obar_p in place
        self.l_parts = torch.empty((P, Q, hq), **f32)
        self.lse = torch.empty((Q, hq), **f32)
        self.Y = torch.empty((Q, self.H), **f32)
        self.do = torch.empty((Q, hq * d), **bf)
        self.delta = torch.empty((Q, hq), **f32)
        self.dq = torch.empty((Q, hq, d), **f32)
        self.dq16 = torch.empty((Q, hq * d), **bf)
        self.ones = torch.ones((Q, 8), **bf)
        self.dbo8 = torch.empty((self.H, 8), **f32)
        n_keys = [c.numel() * m for c in self.cs] + ([Q] if own_blocks else [])
        if own_blocks:
            self.bs, self.ba, self.bcs, self.blen = binding.own_block_local(s, B)
        self.k = [torch.empty((n, hkv * d), **bf) for n in n_keys]
        self.v = [torch.empty((n, hkv * d), **bf) for n in n_keys]
        self.dk = [torch.empty((n, hkv, d), **bf) for n in n_keys]
        self.dv = [torch.empty((n, hkv, d), **bf) for n in n_keys]
        an = binding.make_anchors(s, a, B)
        hd = binding.make_heads(hq, hkv, d, torch.bfloat16, self.scale)
        # room for the largest partial's stored dS (dq then needs no recompute)
        ds = 0
        if store_ds:
            ds = max(binding.splitkv_attn_bwd_ds_bytes(*self._segment(p)[:2], B,
                                                       *self._segment(p)[2:], hq, hkv, d,
                                                       torch.bfloat16)
                     for p in range(self.n_parts))
        ws = max(binding.splitkv_workspace_bytes(binding.SPLITKV_OP_FWD, an, hd, None),
                 binding.splitkv_workspace_bytes(binding.SPLITKV_OP_BWD, an, hd, None) + ds)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)

    # ------------------------------------------------------------- forward --
    def forward(self, X: torch.Tensor, U: Sequence[torch.Tensor]) -> torch.Tensor:
        """X bf16 [Q, H]; U[p] bf16 [J m, H] (rank p's context rows). Returns Y fp32."""
        hq, hkv, d, Q = self.hq, self.hkv, self.d, self.Q
        self.X, self.U = X, list(U)
        binding.splitkv_gemm(NT, X, self.Wq, out=self.q)
        q3 = self.q.view(Q, hq, d)
        for p in range(self.n_parts):
            src = self.U[p] if p < self.P else X      # the own-block keys come from X
            binding.splitkv_gemm(NT, src, self.Wk, out=self.k[p])
            binding.splitkv_gemm(NT, src, self.Wv, out=self.v[p])
            n = self.k[p].shape[0]
            s, a, cs, m = self._segment(p)
            binding.splitkv_attn_fwd(s, a, self.B, cs, m, q3,
                                     self.k[p].view(n, hkv, d), self.v[p].view(n, hkv, d),
                                     scale=self.scale, out=(self.o_parts[p], self.l_parts[p]),
                                     workspace=self.ws)
        binding.splitkv_lse_reduce(self.l_parts, out=self.lse)
        for p in range(self.n_parts):
            binding.splitkv_lse_rescale(self.o_parts[p], self.l_parts[p], self.lse,
                                        out=self.o_parts[p])
            binding.splitkv_gemm(NT, self.o_parts[p].view(Q, hq * d), self.Wo, out=self.Y,
                                 bias=self.bo if p == 0 else None, accumulate=p > 0)
        return self.Y

    def _segment(self, p: int):
        """(windows s, a, chunk starts, chunk length) of partial p."""
        if p < self.P:
            return self.s, self.a, self.cs[p], self.m
        return self.bs, self.ba, self.bcs, self.blen

    # ------------------------------------------------------------ backward --
    def backward(self, dY: torch.Tensor, grads: Optional[Dict[str, torch.Tensor]] = None
                 ) -> Dict[str, torch.Tensor]:
        """dY bf16 [Q, H] -> fp32 gradients dX, dU (list per rank), dWq, dWk, dWv, dWo, dbo."""
        hq, hkv, d, Q, H = self.hq, self.hkv, self.d, self.Q, self.H
        dev = dY.device
        if grads is None:
            f32 = dict(dtype=torch.float32, device=dev)
            grads = {"dX": torch.empty((Q, H), **f32),
                     "dU": [torch.empty((u.shape[0], H), **f32) for u in self.U],
                     "dWq": torch.empty(self.Wq.shape, **f32),
                     "dWk": torch.empty(self.Wk.shape, **f32),
                     "dWv": torch.empty(self.Wv.shape, **f32),
                     "dWo": torch.empty(self.Wo.shape, **f32)}
        binding.splitkv_gemm(TN, dY, self.ones, out=self.dbo8)
        grads["dbo"] = self.dbo8[:, 0]
        binding.splitkv_gemm(NN, dY, self.Wo, out=self.do)
        do3 = self.do.view(Q, hq, d)
        for p in range(self.n_parts):
            binding.splitkv_gemm(TN, dY, self.o_parts[p].view(Q, hq * d), out=grads["dWo"],
                                 accumulate=p > 0)
            binding.splitkv_delta(self.o_parts[p], do3, delta=self.delta, accumulate=p > 0)
        self.dq.zero_()
        q3 = self.q.view(Q, hq, d)
        for p in range(self.n_parts):
            n = self.k[p].shape[0]
            s, a, cs, m = self._segment(p)
            binding.splitkv_attn_bwd(s, a, self.B, cs, m, q3,
                                     self.k[p].view(n, hkv, d), self.v[p].view(n, hkv, d), None,
                                     do3, self.lse, self.dq, scale=self.scale, delta=self.delta,
                                     out=(self.dk[p], self.dv[p]), workspace=self.ws)
        binding.splitkv_cast_bf16(self.dq, out=self.dq16)
        binding.splitkv_gemm(NN, self.dq16, self.Wq, out=grads["dX"])
        binding.splitkv_gemm(TN, self.dq16, self.X, out=grads["dWq"])
        for p in range(self.n_parts):
            n = self.dk[p].shape[0]
            dk2, dv2 = self.dk[p].view(n, hkv * d), self.dv[p].view(n, hkv * d)
            # a rank's context rows get dU_p = dk Wk + dv Wv (one paired product);
            # the own-block keys' gradient adds into dX
            dst, src = (grads["dU"][p], self.U[p]) if p < self.P else (grads["dX"], self.X)
            binding.splitkv_gemm_pair(NN, dk2, self.Wk, dv2, self.Wv, out=dst,
                                      accumulate=p >= self.P)
            binding.splitkv_gemm(TN, dk2, src, out=grads["dWk"], accumulate=p > 0)
            binding.splitkv_gemm(TN, dv2, src, out=grads["dWv"], accumulate=p > 0)
        return grads

    def gemm_flops(self) -> float:
        """Matrix-product FLOPs of one forward + backward."""
        Q, H, P = self.Q, self.H, self.n_parts
        nq, nkv = self.hq * self.d, self.hkv * self.d
        S_loc = sum(k.shape[0] for k in self.k)     # every partial's key rows
        fwd = 2.0 * Q * H * nq + 2.0 * S_loc * H * 2 * nkv + P * 2.0 * Q * nq * H
        bwd = (2.0 * Q * H * nq                      # do
               + P * 2.0 * Q * H * nq                # dWo
               + 2.0 * 2.0 * Q * nq * H              # dX, dWq
               + 2.0 * 2.0 * S_loc * nkv * H * 2)    # dU (k and v), dWk, dWv
        return fwd + bwd
