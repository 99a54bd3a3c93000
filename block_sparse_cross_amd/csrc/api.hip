// C ABI of the Split-KV per-device hot path (declared in include/splitkv.h).
// Validates every scalar on the host, sizes the workspace, and enqueues the
// kernels on the caller's stream. Nothing is enqueued when validation fails.
#include <mutex>

#include "common.hpp"
#include "internal.hpp"

using namespace splitkv;

namespace splitkv {

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

FwdWorkspace fwd_workspace_layout(int64_t n_blocks) {
  FwdWorkspace w;
  w.block_range = 0;
  w.total = align256((size_t)n_blocks * sizeof(int2));
  return w;
}

BwdWorkspace bwd_workspace_layout(int64_t n_blocks, int32_t block_size, int32_t hq, int32_t hkv) {
  BwdWorkspace w;
  w.block_range = 0;
  w.meta = align256((size_t)n_blocks * sizeof(int2));
  const int64_t n_vec = n_blocks * block_size * (hq / hkv);
  const int64_t n_qc = (n_vec + kBwdChunk - 1) / kBwdChunk;
  // 4 fp32 fields per vector, per (kv head, query chunk)
  w.chunk_range = w.meta + align256((size_t)hkv * n_qc * 4 * kBwdChunk * sizeof(float));
  w.ds_off = w.chunk_range + align256((size_t)n_qc * sizeof(int4));
  w.total = w.ds_off + align256((size_t)n_qc * sizeof(int));
  return w;
}

}  // namespace splitkv

namespace {

int hip_status(hipError_t e) { return e == hipSuccess ? SPLITKV_OK : SPLITKV_ERR_HIP; }

// Tensors the kernels touch with 16-byte vector loads, copies or stores must
// start on a 16-byte boundary (NULL passes: presence is checked separately).
bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_anchors(const splitkv_anchors* an) {
  if (an == nullptr) return SPLITKV_ERR_INVALID_ARG;
  if (an->n_blocks < 0 || an->block_size < 1) return SPLITKV_ERR_INVALID_ARG;
  if (an->n_blocks > 0 && (an->s == nullptr || an->a == nullptr)) return SPLITKV_ERR_INVALID_ARG;
  return SPLITKV_OK;
}

int check_heads(const splitkv_heads* hd) {
  if (hd == nullptr) return SPLITKV_ERR_INVALID_ARG;
  if (hd->hq < 1 || hd->hkv < 1 || hd->d < 1) return SPLITKV_ERR_INVALID_ARG;
  if (hd->hq % hd->hkv != 0) return SPLITKV_ERR_INVALID_ARG;
  // positive and finite (NaN fails the first test)
  if (!(hd->scale > 0.f) || hd->scale > 3.0e38f) return SPLITKV_ERR_INVALID_ARG;
  if (hd->dtype != SPLITKV_BF16 && hd->dtype != SPLITKV_FP32) return SPLITKV_ERR_UNSUPPORTED;
  if (hd->d != 64 && hd->d != 128) return SPLITKV_ERR_UNSUPPORTED;
  return SPLITKV_OK;
}

int check_local(const splitkv_local* loc) {
  if (loc == nullptr) return SPLITKV_ERR_INVALID_ARG;
  if (loc->n_chunks < 0 || loc->chunk_len < 1) return SPLITKV_ERR_INVALID_ARG;
  if (loc->n_chunks > 0 && loc->chunk_start == nullptr) return SPLITKV_ERR_INVALID_ARG;
  if ((int64_t)loc->n_chunks * loc->chunk_len >= (int64_t(1) << 31)) return SPLITKV_ERR_UNSUPPORTED;
  return SPLITKV_OK;
}

int check_attn_common(const splitkv_anchors* an, const splitkv_heads* hd, const splitkv_local* loc) {
  int st = check_anchors(an);
  if (st != SPLITKV_OK) return st;
  if ((st = check_heads(hd)) != SPLITKV_OK) return st;
  if ((st = check_local(loc)) != SPLITKV_OK) return st;
  const int64_t Q = an->n_blocks * (int64_t)an->block_size;
  if (Q * hd->hq >= (int64_t(1) << 31)) return SPLITKV_ERR_UNSUPPORTED;
  // a 64-row tile of q or k (all heads) must span less than 2^32 bytes (the
  // kernels copy tiles through 32-bit buffer ranges)
  if ((int64_t)hd->hq * hd->d >= (int64_t(1) << 25)) return SPLITKV_ERR_UNSUPPORTED;
  return SPLITKV_OK;
}

int check_bwd_args(const splitkv_anchors* an, const splitkv_heads* hd, const splitkv_local* loc,
                   const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, const float* delta, const float* dq, const void* dk,
                   const void* dv) {
  int st = check_attn_common(an, hd, loc);
  if (st != SPLITKV_OK) return st;
  const int64_t n_keys = (int64_t)loc->n_chunks * loc->chunk_len;
  const int64_t Q = an->n_blocks * (int64_t)an->block_size;
  if (Q > 0 && (q == nullptr || dout == nullptr || lse == nullptr || delta == nullptr ||
                dq == nullptr))
    return SPLITKV_ERR_INVALID_ARG;
  if (n_keys > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr))
    return SPLITKV_ERR_INVALID_ARG;
  if (!a16(q) || !a16(k) || !a16(v) || !a16(o) || !a16(dout) || !a16(dq) || !a16(dk) || !a16(dv))
    return SPLITKV_ERR_INVALID_ARG;
  return SPLITKV_OK;
}

// The backward's kernels on a workspace laid out as `ws` at `base` (device),
// ds_bytes past ws.total of it free for stored dS.
int run_bwd(const splitkv_anchors* an, const splitkv_heads* hd, const splitkv_local* loc,
            const void* q, const void* k, const void* v, const void* o, const void* dout,
            const float* lse, float* delta, float* dq, void* dk, void* dv, char* base,
            const BwdWorkspace& ws, size_t ds_bytes, hipStream_t s) {
  const int64_t n_keys = (int64_t)loc->n_chunks * loc->chunk_len;
  int2* block_range = reinterpret_cast<int2*>(base + ws.block_range);
  hipError_t e = launch_block_ranges(an->s, an->a, an->n_blocks, loc->chunk_start, loc->n_chunks,
                                     loc->chunk_len, block_range, s);
  if (e != hipSuccess) return SPLITKV_ERR_HIP;
  return hip_status(launch_bwd(*an, *hd, n_keys, block_range, base + ws.meta,
                               base + ws.chunk_range, reinterpret_cast<int*>(base + ws.ds_off),
                               ds_bytes > 0 ? base + ws.total : nullptr, ds_bytes, q, k, v, o,
                               dout, lse, delta, dq, dk, dv, s));
}

// Fixed device scratch of splitkv_attn_bwd_noalloc, for callers that cannot
// allocate. Each device that loads the library holds its own copy until the
// process ends. Host code never uses the array's name as an address (on the
// host it is only a stand-in for the symbol): the device address is looked up
// once per device with that device current and kept in scratch_addr.
static __device__ __align__(256) unsigned char scratch[SPLITKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mu;
char* scratch_addr[kMaxScratchDevices] = {};

// The scratch address on the current device (looked up on the first call).
int device_scratch(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SPLITKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return SPLITKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return SPLITKV_ERR_HIP;
    scratch_addr[dev] = static_cast<char*>(p);
  }
  *out = scratch_addr[dev];
  return SPLITKV_OK;
}

}  // namespace

extern "C" {

const char* splitkv_status_str(int status) {
  switch (status) {
    case SPLITKV_OK: return "ok";
    case SPLITKV_ERR_INVALID_ARG: return "invalid argument";
    case SPLITKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case SPLITKV_ERR_WORKSPACE: return "workspace missing or too small";
    case SPLITKV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t splitkv_workspace_bytes(int op, const splitkv_anchors* an, const splitkv_heads* hd,
                               const splitkv_local* loc) {
  (void)loc;
  switch (op) {
    case SPLITKV_OP_FWD:
      if (an == nullptr) return 0;
      return fwd_workspace_layout(an->n_blocks).total;
    case SPLITKV_OP_BWD:
      if (an == nullptr || hd == nullptr || hd->hkv < 1) return 0;
      return bwd_workspace_layout(an->n_blocks, an->block_size, hd->hq, hd->hkv).total;
    default:
      return 0;
  }
}

int splitkv_validate_anchors(const splitkv_anchors* an, int64_t S, int64_t* result, void* stream) {
  int st = check_anchors(an);
  if (st != SPLITKV_OK) return st;
  if (S < 0 || result == nullptr) return SPLITKV_ERR_INVALID_ARG;
  return hip_status(launch_validate_anchors(an->s, an->a, an->n_blocks, S, result,
                                            static_cast<hipStream_t>(stream)));
}

int splitkv_own_block_local(int64_t n_blocks, int32_t block_size, int64_t* s_out,
                            int64_t* a_out, int64_t* chunk_start_out, int64_t* chunk_len,
                            void* stream) {
  if (n_blocks < 0 || block_size < 1 || chunk_len == nullptr || chunk_start_out == nullptr)
    return SPLITKV_ERR_INVALID_ARG;
  if (n_blocks > 0 && (s_out == nullptr || a_out == nullptr)) return SPLITKV_ERR_INVALID_ARG;
  // the segment is one local chunk: its length must stay below 2^31 keys
  if ((__int128)n_blocks * block_size >= ((__int128)1 << 31)) return SPLITKV_ERR_UNSUPPORTED;
  *chunk_len = n_blocks * (int64_t)block_size;
  return hip_status(launch_own_block_windows(n_blocks, block_size, s_out, a_out, chunk_start_out,
                                             static_cast<hipStream_t>(stream)));
}

int splitkv_plan(const splitkv_anchors* an, int64_t S, int64_t m, int32_t P, int32_t J,
                 int64_t* chunk_cost, int32_t* chunk_owner, int32_t* rank_chunks,
                 int64_t* rank_load, void* stream) {
  int st = check_anchors(an);
  if (st != SPLITKV_OK) return st;
  if (S < 1 || m < 1 || P < 1 || J < 1) return SPLITKV_ERR_INVALID_ARG;
  if ((int64_t)P * J * m != S) return SPLITKV_ERR_INVALID_ARG;
  if (chunk_cost == nullptr || chunk_owner == nullptr || rank_chunks == nullptr ||
      rank_load == nullptr)
    return SPLITKV_ERR_INVALID_ARG;
  if (P > kMaxPlanRanks || (int64_t)P * J > kMaxPlanChunks) return SPLITKV_ERR_UNSUPPORTED;
  // every chunk cost is at most B * N * m, so a rank's load is below B * N * S
  if ((__int128)an->block_size * an->n_blocks * S >= ((__int128)1 << 53))
    return SPLITKV_ERR_UNSUPPORTED;
  return hip_status(launch_plan(an->s, an->a, an->n_blocks, an->block_size, m, P, J, chunk_cost,
                                chunk_owner, rank_chunks, rank_load,
                                static_cast<hipStream_t>(stream)));
}

int splitkv_locality_match(const int32_t* rank_chunks, int32_t P, int32_t J, int64_t m,
                           int32_t* phys_rank, int64_t* send_rows, int64_t* kept_moved,
                           void* stream) {
  if (P < 1 || J < 1 || m < 1) return SPLITKV_ERR_INVALID_ARG;
  if (rank_chunks == nullptr || phys_rank == nullptr || send_rows == nullptr ||
      kept_moved == nullptr)
    return SPLITKV_ERR_INVALID_ARG;
  if (P > kMaxMatchRanks || (int64_t)P * J > kMaxPlanChunks) return SPLITKV_ERR_UNSUPPORTED;
  // slacks stay below (P + 1) * J * m and are packed above 9 column bits
  if ((__int128)(P + 1) * P * J * m >= ((__int128)1 << 54)) return SPLITKV_ERR_UNSUPPORTED;
  return hip_status(launch_locality_match(rank_chunks, P, J, m, phys_rank, send_rows, kept_moved,
                                          static_cast<hipStream_t>(stream)));
}

int splitkv_plan_baseline(int strategy, const splitkv_anchors* an, int32_t n_samples,
                          const int64_t* sample_start, const int64_t* sample_len, int32_t P,
                          int64_t* range_cost, int64_t* rank_load, void* stream) {
  int st = check_anchors(an);
  if (st != SPLITKV_OK) return st;
  if (strategy != SPLITKV_BASELINE_NO_BALANCE && strategy != SPLITKV_BASELINE_ZIGZAG)
    return SPLITKV_ERR_INVALID_ARG;
  if (P < 1 || n_samples < 1 || sample_start == nullptr || sample_len == nullptr ||
      range_cost == nullptr || rank_load == nullptr)
    return SPLITKV_ERR_INVALID_ARG;
  if (P > kMaxPlanRanks || n_samples > kMaxBaselineSamples) return SPLITKV_ERR_UNSUPPORTED;
  BaselineSamples smp;
  smp.n = n_samples;
  int64_t next = 0;
  for (int32_t u = 0; u < n_samples; ++u) {
    // packed in order from 0; the sum stays far below 2^62 for valid lengths
    if (sample_start[u] != next || sample_len[u] < 1 || sample_len[u] > (int64_t(1) << 48))
      return SPLITKV_ERR_INVALID_ARG;
    if (strategy == SPLITKV_BASELINE_ZIGZAG && sample_len[u] % (2 * (int64_t)P) != 0)
      return SPLITKV_ERR_INVALID_ARG;
    smp.start[u] = sample_start[u];
    smp.len[u] = sample_len[u];
    next += sample_len[u];
  }
  const int64_t S = next;
  if (strategy == SPLITKV_BASELINE_NO_BALANCE && S % P != 0) return SPLITKV_ERR_INVALID_ARG;
  return hip_status(launch_plan_baseline(strategy, an->s, an->a, an->n_blocks, an->block_size,
                                         smp, P, S, range_cost, rank_load,
                                         static_cast<hipStream_t>(stream)));
}

int splitkv_attn_fwd(const splitkv_anchors* an, const splitkv_heads* hd,
                     const splitkv_local* loc, const void* q, const void* k, const void* v,
                     void* o_part, int o_dtype, float* lse_part, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check_attn_common(an, hd, loc);
  if (st != SPLITKV_OK) return st;
  if (o_dtype != SPLITKV_BF16 && o_dtype != SPLITKV_FP32) return SPLITKV_ERR_UNSUPPORTED;
  const int64_t n_keys = (int64_t)loc->n_chunks * loc->chunk_len;
  if (an->n_blocks == 0) return SPLITKV_OK;
  if (q == nullptr || o_part == nullptr || lse_part == nullptr) return SPLITKV_ERR_INVALID_ARG;
  if (n_keys > 0 && (k == nullptr || v == nullptr)) return SPLITKV_ERR_INVALID_ARG;
  if (!a16(q) || !a16(k) || !a16(v) || !a16(o_part)) return SPLITKV_ERR_INVALID_ARG;
  const FwdWorkspace ws = fwd_workspace_layout(an->n_blocks);
  if (ws.total > 0 && (workspace == nullptr || workspace_bytes < ws.total))
    return SPLITKV_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int2* block_range = reinterpret_cast<int2*>(static_cast<char*>(workspace) + ws.block_range);
  hipError_t e = launch_block_ranges(an->s, an->a, an->n_blocks, loc->chunk_start, loc->n_chunks,
                                     loc->chunk_len, block_range, s);
  if (e != hipSuccess) return SPLITKV_ERR_HIP;
  return hip_status(launch_fwd(*an, *hd, n_keys, block_range, q, k, v, o_part, o_dtype,
                               lse_part, s));
}

int splitkv_lse_merge(int32_t P, int64_t rows, int32_t d, const void* o_parts, int in_dtype,
                      const float* lse_parts, void* o, int out_dtype, float* lse, void* stream) {
  if (P < 1 || rows < 0 || d < 8 || d % 8 != 0) return SPLITKV_ERR_INVALID_ARG;
  if ((in_dtype != SPLITKV_BF16 && in_dtype != SPLITKV_FP32) ||
      (out_dtype != SPLITKV_BF16 && out_dtype != SPLITKV_FP32))
    return SPLITKV_ERR_UNSUPPORTED;
  if (rows == 0) return SPLITKV_OK;
  if (o_parts == nullptr || lse_parts == nullptr || o == nullptr || lse == nullptr)
    return SPLITKV_ERR_INVALID_ARG;
  if (!a16(o_parts) || !a16(o)) return SPLITKV_ERR_INVALID_ARG;
  if ((rows * (d / 8) + 255) / 256 >= (int64_t(1) << 31)) return SPLITKV_ERR_UNSUPPORTED;
  return hip_status(launch_merge(P, rows, d, o_parts, in_dtype, lse_parts, o, out_dtype, lse,
                                 static_cast<hipStream_t>(stream)));
}

int splitkv_lse_reduce(int32_t P, int64_t rows, const float* lse_parts, float* lse,
                       void* stream) {
  if (P < 1 || rows < 0) return SPLITKV_ERR_INVALID_ARG;
  if (rows == 0) return SPLITKV_OK;
  if (lse_parts == nullptr || lse == nullptr) return SPLITKV_ERR_INVALID_ARG;
  if ((rows + 255) / 256 >= (int64_t(1) << 31)) return SPLITKV_ERR_UNSUPPORTED;
  return hip_status(launch_lse_reduce(P, rows, lse_parts, lse, static_cast<hipStream_t>(stream)));
}

int splitkv_lse_rescale(int64_t rows, int32_t d, const void* o_part, int in_dtype,
                        const float* lse_part, const float* lse, void* o_bar, int out_dtype,
                        void* stream) {
  if (rows < 0 || d < 8 || d % 8 != 0) return SPLITKV_ERR_INVALID_ARG;
  if ((in_dtype != SPLITKV_BF16 && in_dtype != SPLITKV_FP32) ||
      (out_dtype != SPLITKV_BF16 && out_dtype != SPLITKV_FP32))
    return SPLITKV_ERR_UNSUPPORTED;
  if (rows == 0) return SPLITKV_OK;
  if (o_part == nullptr || lse_part == nullptr || lse == nullptr || o_bar == nullptr)
    return SPLITKV_ERR_INVALID_ARG;
  if (!a16(o_part) || !a16(o_bar)) return SPLITKV_ERR_INVALID_ARG;
  // in place only when the element types agree
  if (o_part == o_bar && in_dtype != out_dtype) return SPLITKV_ERR_INVALID_ARG;
  if ((rows * (d / 8) + 255) / 256 >= (int64_t(1) << 31)) return SPLITKV_ERR_UNSUPPORTED;
  return hip_status(launch_lse_rescale(rows, d, o_part, in_dtype, lse_part, lse, o_bar,
                                       out_dtype, static_cast<hipStream_t>(stream)));
}

int splitkv_delta(int64_t rows, int32_t d, const void* o, int o_dtype, const void* dout,
                  int do_dtype, float* delta, int accumulate, void* stream) {
  if (rows < 0 || d < 8 || d % 8 != 0 || d / 8 > 64 || ((d / 8) & (d / 8 - 1)) != 0)
    return SPLITKV_ERR_INVALID_ARG;
  if ((o_dtype != SPLITKV_BF16 && o_dtype != SPLITKV_FP32) ||
      (do_dtype != SPLITKV_BF16 && do_dtype != SPLITKV_FP32))
    return SPLITKV_ERR_UNSUPPORTED;
  if (rows == 0) return SPLITKV_OK;
  if (o == nullptr || dout == nullptr || delta == nullptr) return SPLITKV_ERR_INVALID_ARG;
  if (!a16(o) || !a16(dout)) return SPLITKV_ERR_INVALID_ARG;
  if ((rows * (d / 8) + 255) / 256 >= (int64_t(1) << 31)) return SPLITKV_ERR_UNSUPPORTED;
  return hip_status(launch_delta(rows, d, o, o_dtype, dout, do_dtype, delta, accumulate != 0,
                                 static_cast<hipStream_t>(stream)));
}

int splitkv_cast_bf16(int64_t n, const float* src, void* dst, void* stream) {
  if (n < 0 || n % 8 != 0) return SPLITKV_ERR_INVALID_ARG;
  if (n == 0) return SPLITKV_OK;
  if (src == nullptr || dst == nullptr) return SPLITKV_ERR_INVALID_ARG;
  if (!a16(src) || !a16(dst)) return SPLITKV_ERR_INVALID_ARG;
  if ((n / 8 + 255) / 256 >= (int64_t(1) << 31)) return SPLITKV_ERR_UNSUPPORTED;
  return hip_status(launch_cast_bf16(n, src, dst, static_cast<hipStream_t>(stream)));
}

int splitkv_gemm(int layout, int64_t M, int64_t N, int64_t K, const void* A, const void* B,
                 void* C, int c_dtype, const float* bias, int accumulate, void* stream) {
  if (layout != SPLITKV_GEMM_NT && layout != SPLITKV_GEMM_NN && layout != SPLITKV_GEMM_TN)
    return SPLITKV_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K < 1 || M % 8 != 0 || N % 8 != 0 || K % 8 != 0)
    return SPLITKV_ERR_INVALID_ARG;
  if (c_dtype != SPLITKV_BF16 && c_dtype != SPLITKV_FP32) return SPLITKV_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return SPLITKV_OK;
  if (A == nullptr || B == nullptr || C == nullptr) return SPLITKV_ERR_INVALID_ARG;
  if (!a16(A) || !a16(B) || !a16(C)) return SPLITKV_ERR_INVALID_ARG;
  // tile count; the kernel addresses each operand with 32-bit byte offsets
  if (((M + 255) / 256) * ((N + 255) / 256) >= (int64_t(1) << 31)) return SPLITKV_ERR_UNSUPPORTED;
  if (M * K >= (int64_t(1) << 31) || N * K >= (int64_t(1) << 31)) return SPLITKV_ERR_UNSUPPORTED;
  return hip_status(launch_gemm(layout, M, N, K, A, B, nullptr, nullptr, C, c_dtype, bias,
                                accumulate != 0, static_cast<hipStream_t>(stream)));
}

int splitkv_gemm_pair(int layout, int64_t M, int64_t N, int64_t K, const void* A1,
                      const void* B1, const void* A2, const void* B2, void* C, int c_dtype,
                      const float* bias, int accumulate, void* stream) {
  if (layout != SPLITKV_GEMM_NT && layout != SPLITKV_GEMM_NN && layout != SPLITKV_GEMM_TN)
    return SPLITKV_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K < 64 || M % 8 != 0 || N % 8 != 0 || K % 64 != 0)
    return SPLITKV_ERR_INVALID_ARG;
  if (c_dtype != SPLITKV_BF16 && c_dtype != SPLITKV_FP32) return SPLITKV_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return SPLITKV_OK;
  if (A1 == nullptr || B1 == nullptr || A2 == nullptr || B2 == nullptr || C == nullptr)
    return SPLITKV_ERR_INVALID_ARG;
  if (!a16(A1) || !a16(B1) || !a16(A2) || !a16(B2) || !a16(C)) return SPLITKV_ERR_INVALID_ARG;
  if (((M + 255) / 256) * ((N + 255) / 256) >= (int64_t(1) << 31)) return SPLITKV_ERR_UNSUPPORTED;
  if (M * K >= (int64_t(1) << 31) || N * K >= (int64_t(1) << 31)) return SPLITKV_ERR_UNSUPPORTED;
  return hip_status(launch_gemm(layout, M, N, K, A1, B1, A2, B2, C, c_dtype, bias,
                                accumulate != 0, static_cast<hipStream_t>(stream)));
}

int splitkv_attn_bwd(const splitkv_anchors* an, const splitkv_heads* hd,
                     const splitkv_local* loc, const void* q, const void* k, const void* v,
                     const void* o, const void* dout, const float* lse, float* delta, float* dq,
                     void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_bwd_args(an, hd, loc, q, k, v, o, dout, lse, delta, dq, dk, dv);
  if (st != SPLITKV_OK) return st;
  const BwdWorkspace ws = bwd_workspace_layout(an->n_blocks, an->block_size, hd->hq, hd->hkv);
  if (ws.total > 0 && (workspace == nullptr || workspace_bytes < ws.total))
    return SPLITKV_ERR_WORKSPACE;
  if (workspace_bytes > ws.total && !a16(workspace)) return SPLITKV_ERR_INVALID_ARG;
  return run_bwd(an, hd, loc, q, k, v, o, dout, lse, delta, dq, dk, dv,
                 static_cast<char*>(workspace), ws,
                 workspace == nullptr ? 0 : workspace_bytes - ws.total,
                 static_cast<hipStream_t>(stream));
}

int splitkv_attn_bwd_ds_bytes(const splitkv_anchors* an, const splitkv_heads* hd,
                              const splitkv_local* loc, void* workspace, size_t workspace_bytes,
                              int64_t* ds_bytes, void* stream) {
  int st = check_attn_common(an, hd, loc);
  if (st != SPLITKV_OK) return st;
  if (ds_bytes == nullptr || (reinterpret_cast<uintptr_t>(ds_bytes) & 7) != 0)
    return SPLITKV_ERR_INVALID_ARG;
  const BwdWorkspace ws = bwd_workspace_layout(an->n_blocks, an->block_size, hd->hq, hd->hkv);
  if (ws.total > 0 && (workspace == nullptr || workspace_bytes < ws.total))
    return SPLITKV_ERR_WORKSPACE;
  char* base = static_cast<char*>(workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int2* block_range = reinterpret_cast<int2*>(base + ws.block_range);
  hipError_t e = launch_block_ranges(an->s, an->a, an->n_blocks, loc->chunk_start, loc->n_chunks,
                                     loc->chunk_len, block_range, s);
  if (e != hipSuccess) return SPLITKV_ERR_HIP;
  return hip_status(launch_bwd_ds_need(*an, *hd, block_range, base + ws.chunk_range,
                                       reinterpret_cast<int*>(base + ws.ds_off), ds_bytes, s));
}

int splitkv_attn_bwd_noalloc(const splitkv_anchors* an, const splitkv_heads* hd,
                             const splitkv_local* loc, const void* q, const void* k,
                             const void* v, const void* o, const void* dout, const float* lse,
                             float* delta, float* dq, void* dk, void* dv, void* stream) {
  int st = check_bwd_args(an, hd, loc, q, k, v, o, dout, lse, delta, dq, dk, dv);
  if (st != SPLITKV_OK) return st;
  const BwdWorkspace ws = bwd_workspace_layout(an->n_blocks, an->block_size, hd->hq, hd->hkv);
  if (ws.total > SPLITKV_NOALLOC_SCRATCH_BYTES) return SPLITKV_ERR_WORKSPACE;
  char* base = nullptr;
  if ((st = device_scratch(&base)) != SPLITKV_OK) return st;
  // the scratch past the fixed part stays unused: every dQ is recomputed
  return run_bwd(an, hd, loc, q, k, v, o, dout, lse, delta, dq, dk, dv, base, ws, 0,
                 static_cast<hipStream_t>(stream));
}

}  // extern "C"
