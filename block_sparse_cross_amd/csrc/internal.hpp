// Host-side launchers shared between the C-ABI layer and the kernel files.
// Every launcher assumes its arguments were validated by the caller and
// returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "splitkv.h"

namespace splitkv {

constexpr int kMaxPlanRanks = 1024;
constexpr int kMaxPlanChunks = 4096;
constexpr int kBwdChunk = 64;  // query vectors per chunk of the dK/dV kernel
constexpr int kMaxBaselineSamples = 128;
constexpr int kMaxMatchRanks = 256;  // ranks of a locality matching

// Packed sample table of a position-based assignment, passed by value.
struct BaselineSamples {
  int32_t n;
  int64_t start[kMaxBaselineSamples];
  int64_t len[kMaxBaselineSamples];
};

// Workspace layout (device bytes), 256-byte aligned segments.
struct FwdWorkspace {
  size_t block_range;  // int2 [N]
  size_t total;
};
struct BwdWorkspace {
  size_t block_range;  // int2 [N]
  size_t meta;         // fp32 [hkv][n_qc][4][kBwdChunk]: lse*log2e, Delta, lo, hi
  size_t chunk_range;  // int4 [n_qc], n_qc = ceil(Q*G / kBwdChunk)
  size_t ds_off;       // int32 [n_qc]: first stored-dS tile of each chunk
  size_t total;        // bytes past total (if any) hold stored dS tiles
};
FwdWorkspace fwd_workspace_layout(int64_t n_blocks);
BwdWorkspace bwd_workspace_layout(int64_t n_blocks, int32_t block_size, int32_t hq, int32_t hkv);

hipError_t launch_plan(const int64_t* s, const int64_t* a, int64_t n_blocks, int32_t B,
                       int64_t m, int32_t P, int32_t J, int64_t* cost, int32_t* owner,
                       int32_t* rank_chunks, int64_t* rank_load, hipStream_t stream);

hipError_t launch_plan_baseline(int strategy, const int64_t* s, const int64_t* a,
                                int64_t n_blocks, int32_t B, const BaselineSamples& samples,
                                int32_t P, int64_t S, int64_t* range_cost, int64_t* rank_load,
                                hipStream_t stream);

hipError_t launch_locality_match(const int32_t* rank_chunks, int32_t P, int32_t J, int64_t m,
                                 int32_t* phys_rank, int64_t* send_rows, int64_t* kept_moved,
                                 hipStream_t stream);

hipError_t launch_own_block_windows(int64_t n_blocks, int32_t B, int64_t* s, int64_t* a,
                                    int64_t* chunk_start, hipStream_t stream);

hipError_t launch_validate_anchors(const int64_t* s, const int64_t* a, int64_t n_blocks,
                                   int64_t S, int64_t* result, hipStream_t stream);

hipError_t launch_block_ranges(const int64_t* s, const int64_t* a, int64_t n_blocks,
                               const int64_t* chunk_start, int32_t n_chunks, int64_t m,
                               int2* block_range, hipStream_t stream);

hipError_t launch_fwd(const splitkv_anchors& an, const splitkv_heads& hd, int64_t n_keys,
                      const int2* block_range, const void* q, const void* k, const void* v,
                      void* o, int o_dtype, float* lse, hipStream_t stream);

hipError_t launch_merge(int32_t P, int64_t rows, int32_t d, const void* o_parts, int in_dtype,
                        const float* lse_parts, void* o, int out_dtype, float* lse,
                        hipStream_t stream);

hipError_t launch_lse_reduce(int32_t P, int64_t rows, const float* lse_parts, float* lse,
                             hipStream_t stream);

hipError_t launch_lse_rescale(int64_t rows, int32_t d, const void* o_part, int in_dtype,
                              const float* lse_part, const float* lse, void* o_bar,
                              int out_dtype, hipStream_t stream);

hipError_t launch_delta(int64_t rows, int32_t d, const void* o, int o_dtype, const void* dout,
                        int do_dtype, float* delta, int accumulate, hipStream_t stream);

hipError_t launch_cast_bf16(int64_t n, const float* src, void* dst, hipStream_t stream);

hipError_t launch_gemm(int layout, int64_t M, int64_t N, int64_t K, const void* A, const void* B,
                       const void* A2, const void* B2, void* C, int c_dtype, const float* bias,
                       int accumulate, hipStream_t stream);

// ds_area / ds_bytes: room for stored dS tiles (may be empty: then every dQ
// is recomputed).
hipError_t launch_bwd(const splitkv_anchors& an, const splitkv_heads& hd, int64_t n_keys,
                      const int2* block_range, void* meta, void* chunk_range, int* ds_off,
                      void* ds_area, size_t ds_bytes, const void* q, const void* k,
                      const void* v, const void* o, const void* dout, const float* lse,
                      float* delta, float* dq, void* dk, void* dv, hipStream_t stream);

// Bytes of stored dS that cover every chunk, written to *need (device).
hipError_t launch_bwd_ds_need(const splitkv_anchors& an, const splitkv_heads& hd,
                              const int2* block_range, void* chunk_range, int* ds_off,
                              int64_t* need, hipStream_t stream);

}  // namespace splitkv
