/*
 * splitkv.h -- C ABI of the Split-KV per-device hot path for MI355X (gfx950).
 *
 * Method: "Split-KV: Efficient Context Parallelism for Training Diffusion
 * Drafters" (arXiv 2611.05926v1). One device (rank p) holds the globally
 * gathered draft queries q (all N blocks of B rows) and J local context chunks
 * of m positions each. Block i's rows attend the context window [s_i, a_i) of
 * their own sample (§3.1, Figure 1), restricted here to the local chunks.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless stated otherwise; the caller owns all
 *     memory. The library allocates nothing and keeps no state between calls.
 *   - Scalars and struct fields are validated on the host before anything is
 *     enqueued; on any error nothing is enqueued and a negative status returns.
 *     Device-resident contents (anchors, chunk starts) are not validated: the
 *     kernels stay in bounds for any contents, results are then unspecified.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without synchronising. Kernel launch failures return
 *     SPLITKV_ERR_HIP.
 *   - Tensors are dense row-major. Query rows are block-major: row r belongs to
 *     block r / B. Query tensors are [Q, hq, d] with Q = N*B; key/value tensors
 *     are [J*m, hkv, d], the local chunks in ascending chunk_start order. Query
 *     head h reads key/value head h / (hq / hkv).
 *   - LSE values are natural logarithms. A (row, head) with no live key gets
 *     lse = -inf and o = 0.
 *   - Supported: d in {64, 128}; hq % hkv == 0; q/k/v dtype bf16 (matrix-core
 *     path) or fp32; J*m < 2^31; N*B*hq < 2^31; hq*d < 2^25.
 *   - Alignment: every tensor of query, key/value, output, gradient or
 *     product-operand shape (q, k, v, o, o_part(s), o_bar, dout, dq, dk, dv,
 *     the products' A, B, C and the conversion's src, dst) must start on a
 *     16-byte boundary (the kernels move them 16 bytes per lane); otherwise
 *     the call returns SPLITKV_ERR_INVALID_ARG with nothing enqueued. Anchor,
 *     chunk, LSE, Delta and plan arrays need only their element alignment.
 */
#ifndef SPLITKV_H
#define SPLITKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPLITKV_OK = 0,
    SPLITKV_ERR_INVALID_ARG = -1, /* a scalar, a size or a required pointer is wrong */
    SPLITKV_ERR_UNSUPPORTED = -2, /* valid but not implemented (d, dtype, limits)      */
    SPLITKV_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required       */
    SPLITKV_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed        */
} splitkv_status;

typedef enum { SPLITKV_BF16 = 0, SPLITKV_FP32 = 1 } splitkv_dtype;

typedef enum {
    SPLITKV_OP_PLAN = 0,
    SPLITKV_OP_FWD = 1,
    SPLITKV_OP_BWD = 2,
    SPLITKV_OP_MERGE = 3
} splitkv_op;

/* Global anchor metadata A = {(s_i, a_i)} (§4.2: every rank holds it).
 * s, a: device int64 [n_blocks]; block i's window is [s[i], a[i]). */
typedef struct {
    const int64_t* s;
    const int64_t* a;
    int64_t n_blocks;    /* N */
    int32_t block_size;  /* B (16 in the paper's runs) */
} splitkv_anchors;

/* Head layout (Table 2: n_q, n_kv, d_h) and the input dtype of q, k, v, do. */
typedef struct {
    int32_t hq;
    int32_t hkv;
    int32_t d;
    int32_t dtype;       /* splitkv_dtype */
    float scale;         /* softmax scale of Eq. 3, normally 1/sqrt(d); finite, > 0 */
} splitkv_heads;

/* The rank's local context chunks (§4.2 global chunking: chunk j covers
 * [lambda_j, lambda_j + m)). chunk_start: device int64 [n_chunks], strictly
 * ascending with chunk_start[j+1] >= chunk_start[j] + m (a plan's bundle,
 * times m, satisfies this). */
typedef struct {
    const int64_t* chunk_start;
    int32_t n_chunks;    /* J */
    int64_t chunk_len;   /* m */
} splitkv_local;

/* Bytes of device workspace an entry point needs (0 if none). `op` is a
 * splitkv_op; arguments it does not use may be NULL. */
size_t splitkv_workspace_bytes(int op, const splitkv_anchors* an, const splitkv_heads* hd,
                               const splitkv_local* loc);

/* Device-side check of the anchor metadata (a debugging aid; no other entry
 * point reads anchors on the host). Block i's rows attend [s_i, a_i) of their
 * own sample (§3.1, Figure 1), so block i is valid when
 *   0 <= s[i] <= a[i] <= S     (an empty window, s[i] == a[i], is valid).
 * result: device int64 [2], overwritten with the number of invalid blocks and
 * the index of the first one (-1 if none); read it once the stream has reached
 * the call. Requires S >= 0 and result != NULL; n_blocks == 0 gives {0, -1}. */
int splitkv_validate_anchors(const splitkv_anchors* an, int64_t S, int64_t* result, void* stream);

/* The own-block part of the mask (Figure 1: each block's rows also attend
 * all B tokens of their own block, in both directions; the D term of §4.2).
 * The block tokens' keys and values are laid out in block order as one local
 * segment of n_blocks * B positions, so block i sees [i*B, (i+1)*B) of it.
 * Writes that layout for splitkv_attn_fwd / splitkv_attn_bwd: s_out, a_out
 * device int64 [n_blocks] (the windows), chunk_start_out device int64 [1]
 * (= 0) and *chunk_len (HOST int64, = n_blocks * B: the segment is one chunk).
 * Requires n_blocks * B < 2^31 (else SPLITKV_ERR_UNSUPPORTED). */
int splitkv_own_block_local(int64_t n_blocks, int32_t block_size, int64_t* s_out,
                            int64_t* a_out, int64_t* chunk_start_out, int64_t* chunk_len,
                            void* stream);

/* Chunk pricing (Eq. 6) and cost-aware LPT (§4.2).
 *   cost[j]  = B * sum_i ( min(a_i, j*m + m) - max(s_i, j*m) )^+, j < P*J   (int64)
 *   Chunks are taken by cost, highest first (equal costs: lower j first); each
 *   goes to the least-loaded rank holding fewer than J chunks (equal loads:
 *   lower rank first).
 * Outputs (device): chunk_cost int64 [P*J], chunk_owner int32 [P*J],
 *   rank_chunks int32 [P][J] (each rank's chunks ascending), rank_load int64 [P]
 *   (= C_p, the context work of rank p).
 * Requires P*J*m == S, P <= 1024, P*J <= 4096, B*N*S < 2^53 (else
 * SPLITKV_ERR_UNSUPPORTED). Integer only: the result is unique and
 * reproducible bit for bit. */
int splitkv_plan(const splitkv_anchors* an, int64_t S, int64_t m, int32_t P, int32_t J,
                 int64_t* chunk_cost, int32_t* chunk_owner, int32_t* rank_chunks,
                 int64_t* rank_load, void* stream);

/* Locality matching (§4.2): places the plan's bundles (rank_chunks of
 * splitkv_plan: device int32 [P][J] chunk ids) on physical ranks without
 * changing any load, so that the step's all-to-all moves as few context rows
 * as possible. Before the all-to-all, physical rank r holds the r-th of P
 * equal contiguous parts of [0, S), S = P*J*m (chunks r*J .. r*J + J - 1);
 * placing bundle b on rank r keeps m * #{chunks of b whose home is r} rows in
 * place. The placement maximises the rows kept (a linear assignment, solved
 * exactly). Several placements often keep the same number of rows; which of
 * them is returned is not specified (the same input gives the same one), and
 * send_rows and kept_moved always describe the placement returned.
 * Outputs (device): phys_rank int32 [P] (bundle b runs on rank phys_rank[b]),
 *   send_rows int64 [P][P] (rows rank src sends to rank dst, zero diagonal),
 *   kept_moved int64 [2] = {rows kept in place, rows moved}.
 * Requires P <= 256, P*J <= 4096, (P+1)*P*J*m < 2^54. Chunk ids outside
 * [0, P*J) count as neither kept nor sent. Integer only. */
int splitkv_locality_match(const int32_t* rank_chunks, int32_t P, int32_t J, int64_t m,
                           int32_t* phys_rank, int64_t* send_rows, int64_t* kept_moved,
                           void* stream);

/* The two position-based assignments the cost-aware plan is measured against
 * (§3.3 and Figure 5(b) for Zigzag; §5.5 and Figure 9 for No balance). */
typedef enum {
    SPLITKV_BASELINE_NO_BALANCE = 0, /* rank p owns the p-th of P equal contiguous parts of [0, S) */
    SPLITKV_BASELINE_ZIGZAG = 1      /* each sample in 2P equal chunks; rank p owns p and 2P-1-p  */
} splitkv_baseline;

/* Context work of a position-based assignment, priced like Eq. 6 but over the
 * assignment's own ranges:
 *   range_cost[r] = B * sum_i |[s_i, a_i) ∩ [lo_r, hi_r)|   (int64)
 *   rank_load[p]  = sum of range_cost over the ranges rank p owns (= C_p).
 * Ranges, in output order:
 *   NO_BALANCE: R = P ranges; range p = [p*S/P, (p+1)*S/P), owned by rank p,
 *     where S = sample_start[n-1] + sample_len[n-1].
 *   ZIGZAG: R = 2P * n_samples ranges; range u*2P + c is chunk c of sample u,
 *     [st_u + c*L_u/(2P), st_u + (c+1)*L_u/(2P)), owned by rank c for c < P and
 *     by rank 2P-1-c otherwise.
 * sample_start, sample_len: HOST int64 [n_samples], the packed samples in order
 * (sample_start[0] == 0, each sample starts where the previous one ends, every
 * length >= 1); 1 <= n_samples <= 128. P <= 1024. NO_BALANCE requires S % P == 0,
 * ZIGZAG requires every L_u % (2P) == 0 (else SPLITKV_ERR_INVALID_ARG).
 * Outputs (device): range_cost int64 [R], rank_load int64 [P]. Integer only. */
int splitkv_plan_baseline(int strategy, const splitkv_anchors* an, int32_t n_samples,
                          const int64_t* sample_start, const int64_t* sample_len, int32_t P,
                          int64_t* range_cost, int64_t* rank_load, void* stream);

/* Local partial attention, Eq. 3: for every query row r (block i) and head h,
 * over the local keys whose global position lies in [s_i, a_i):
 *   lse_p = log sum_x exp(scale <q, k_x>),  o_p = sum_x exp(scale <q, k_x> - lse_p) v_x.
 * q [Q, hq, d], k, v [J*m, hkv, d] in hd->dtype; o_part [Q, hq, d] in o_dtype
 * (bf16 or fp32); lse_part fp32 [Q, hq]. Both outputs are fully overwritten.
 * workspace: splitkv_workspace_bytes(SPLITKV_OP_FWD, ...) bytes. */
int splitkv_attn_fwd(const splitkv_anchors* an, const splitkv_heads* hd,
                     const splitkv_local* loc, const void* q, const void* k, const void* v,
                     void* o_part, int o_dtype, float* lse_part,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Exact merge of P partials, Eq. 4, row by row (rows = Q*hq):
 *   lse = log sum_p exp(lse_p),  o = sum_p exp(lse_p - lse) o_p.
 * Partials with lse_p = -inf contribute nothing; a row whose partials are all
 * empty gets (o = 0, lse = -inf).
 * o_parts [P][rows][d] in in_dtype, lse_parts fp32 [P][rows]; o [rows][d] in
 * out_dtype, lse fp32 [rows]. P >= 1. d % 8 == 0. */
int splitkv_lse_merge(int32_t P, int64_t rows, int32_t d, const void* o_parts, int in_dtype,
                      const float* lse_parts, void* o, int out_dtype, float* lse, void* stream);

/* Eq. 4 in the two halves each rank applies when the partials sit on
 * different devices (Algorithm 1, MERGE after the all-reduce of the LSE
 * statistics). Rows = Q*hq.
 * splitkv_lse_reduce: lse = log sum_p exp(lse_p) per row; all partials empty
 *   gives -inf. lse_parts fp32 [P][rows], lse fp32 [rows]. P >= 1.
 * splitkv_lse_rescale: o_bar = exp(lse_p - lse) o_p for one rank's partial
 *   (o_bar = 0 where lse_p = -inf); summed over the ranks, the o_bar are the
 *   merged output of splitkv_lse_merge. o_part [rows][d] in in_dtype, lse_part
 *   and lse fp32 [rows], o_bar [rows][d] in out_dtype; d % 8 == 0. lse must be
 *   the reduction of the partials (so lse >= lse_p). o_bar may alias o_part
 *   when the two dtypes agree (in place). */
int splitkv_lse_reduce(int32_t P, int64_t rows, const float* lse_parts, float* lse,
                       void* stream);
int splitkv_lse_rescale(int64_t rows, int32_t d, const void* o_part, int in_dtype,
                        const float* lse_part, const float* lse, void* o_bar, int out_dtype,
                        void* stream);

/* Delta of Algorithm 1's MERGE_BWD: delta[r] = <do[r], o[r]> (accumulate == 0)
 * or delta[r] += <do[r], o[r]> (accumulate != 0), over rows of d elements.
 * With a rank's rescaled partial o_bar_p as `o` this is the rank's share of
 * Delta, and accumulating over the ranks is the all-reduce; the result can be
 * handed to splitkv_attn_bwd with o == NULL. o [rows][d] in o_dtype, dout
 * [rows][d] in do_dtype, delta fp32 [rows]. d % 8 == 0 and d/8 a power of two
 * <= 64. */
int splitkv_delta(int64_t rows, int32_t d, const void* o, int o_dtype, const void* dout,
                  int do_dtype, float* delta, int accumulate, void* stream);

/* Dense projections around the attention of one draft layer (Algorithm 1:
 * QProj, KeyValueProj, OProj and their gradients). bf16 operands, fp32
 * accumulation:
 *   C[M][N] = op(A) op(B) + bias     (accumulate == 0)
 *   C[M][N] += op(A) op(B) + bias    (accumulate != 0)
 *   SPLITKV_GEMM_NT: A [M][K], B [N][K], op(B) = B^T   (x W^T)
 *   SPLITKV_GEMM_NN: A [M][K], B [K][N]                (dY W)
 *   SPLITKV_GEMM_TN: A [K][M], B [K][N], op(A) = A^T   (dY^T X)
 * All matrices dense row-major; C in c_dtype (fp32 or bf16); bias NULL or fp32
 * [N]. With OProj linear, Eq. 5 sums each rank's projected partial and adds the
 * bias once: accumulate the P products into one fp32 C, passing bias on one of
 * them. M, N, K multiples of 8 (16-byte rows), K >= 8; M*K and N*K below 2^31
 * (else SPLITKV_ERR_UNSUPPORTED). */
typedef enum {
    SPLITKV_GEMM_NT = 0,
    SPLITKV_GEMM_NN = 1,
    SPLITKV_GEMM_TN = 2
} splitkv_gemm_layout;
int splitkv_gemm(int layout, int64_t M, int64_t N, int64_t K, const void* A, const void* B,
                 void* C, int c_dtype, const float* bias, int accumulate, void* stream);

/* Two products of the same layout and shape summed into one output:
 *   C (+)= op(A1) op(B1) + op(A2) op(B2) (+ bias)
 * in one pass over C (KeyValueProj's backward: dU_p = dk_p Wk + dv_p Wv).
 * Same conventions as splitkv_gemm; additionally K % 64 == 0 and K >= 64. */
int splitkv_gemm_pair(int layout, int64_t M, int64_t N, int64_t K, const void* A1,
                      const void* B1, const void* A2, const void* B2, void* C, int c_dtype,
                      const float* bias, int accumulate, void* stream);

/* fp32 -> bf16 conversion (round to nearest even) of n elements, n % 8 == 0:
 * the rank-summed dq becomes the bf16 operand of QProj's backward products. */
int splitkv_cast_bf16(int64_t n, const float* src, void* dst, void* stream);

/* Backward of the local partial, Algorithm 1 (MERGE_BWD then AttnBwd_p), with
 * the GLOBAL (merged) lse and Delta = <do, o>:
 *   P = exp(scale <q, k_x> - lse[r,h]);  dv_x += P do;  ds = P (<do, v_x> - Delta[r,h]);
 *   dq_r += scale ds k_x;  dk_x += scale ds q_r   (dk, dv summed over the q heads of a kv head).
 * o: merged output [Q, hq, d] (hd->dtype). If o != NULL, Delta is computed and
 *   written to `delta` (fp32 [Q, hq]); if o == NULL, `delta` must hold Delta.
 * dout [Q, hq, d] (hd->dtype); lse fp32 [Q, hq] (rows with -inf contribute 0).
 * dq: fp32 [Q, hq, d], ACCUMULATED (+=) so that P emulated ranks sum into one
 *   buffer (the reduce-scatter of Algorithm 1); the caller zeroes it first.
 * dk, dv: [J*m, hkv, d] in hd->dtype, overwritten (local to the rank).
 * workspace: at least splitkv_workspace_bytes(SPLITKV_OP_BWD, ...) bytes
 *   (W). With bf16, bytes past W (workspace 16-byte aligned) hold the ds of
 *   the pairs as the dK/dV pass computes them (2 bytes per (q head, row, local
 *   key) pair the key union of a 64-vector query chunk spans), so that dq
 *   comes from them instead of recomputing S and dP; the query rows are taken
 *   256 (row, head) vectors of a kv head at a time, in order, as far as the
 *   room goes, and the rest recompute. splitkv_attn_bwd_ds_bytes gives the
 *   room that covers every row. Both ways compute the same sums; the rounding
 *   of dq may differ in the last bits between them. */
int splitkv_attn_bwd(const splitkv_anchors* an, const splitkv_heads* hd,
                     const splitkv_local* loc, const void* q, const void* k, const void* v,
                     const void* o, const void* dout, const float* lse, float* delta,
                     float* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Room for the stored ds of splitkv_attn_bwd (bytes past W) that covers every
 * query row of these anchors, heads and local chunks: enqueued on `stream`,
 * written to *ds_bytes (DEVICE int64, 8-byte aligned) as the pair count above
 * times 2, rounded up to whole 32-key groups. 0 for fp32 (that path stores
 * nothing). workspace: W bytes, overwritten. */
int splitkv_attn_bwd_ds_bytes(const splitkv_anchors* an, const splitkv_heads* hd,
                              const splitkv_local* loc, void* workspace, size_t workspace_bytes,
                              int64_t* ds_bytes, void* stream);

/* The backward above without a workspace argument, for callers that cannot
 * allocate device memory at all (code under stream capture, tight serving
 * loops, harnesses that forbid allocation). Same arguments, results and
 * kernels as splitkv_attn_bwd with a workspace of exactly W bytes (dq
 * recomputed, no stored ds); its scratch (the per-block key ranges, the
 * per-vector records and the per-chunk ranges of the workspace) lives in a
 * fixed device array of SPLITKV_NOALLOC_SCRATCH_BYTES that the library holds
 * on every device it runs on until the process ends. The call allocates and
 * frees nothing. Inputs larger than the array can hold (when
 * splitkv_workspace_bytes(SPLITKV_OP_BWD, ...) exceeds it; about 16 bytes per
 * query row and head) return SPLITKV_ERR_WORKSPACE with nothing enqueued.
 * The array is the current device's (hipGetDevice), so `stream` must belong
 * to the current device. Every call on one device shares that device's
 * array: calls that overlap in time on one device (several streams or host
 * threads) race; serialise them. No state carries over between calls. */
#define SPLITKV_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
int splitkv_attn_bwd_noalloc(const splitkv_anchors* an, const splitkv_heads* hd,
                             const splitkv_local* loc, const void* q, const void* k,
                             const void* v, const void* o, const void* dout, const float* lse,
                             float* delta, float* dq, void* dk, void* dv, void* stream);

/* Human-readable name of a status code (static string). */
const char* splitkv_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* SPLITKV_H */
