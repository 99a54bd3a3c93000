// Device-side helpers shared by the Split-KV kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "splitkv.h"

namespace splitkv {

// Matrix-core operand and accumulator types.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint16_t bf16_t;  // raw bf16 bits in memory

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Element loads/stores for the two supported storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float x) { *p = x; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store(bf16_t* p, float x) { *p = f32_to_bf16(x); }
};

// Wave-wide reductions (64 lanes) through cross-lane shuffles.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = min(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off));
  return x;
}

// ---------------------------------------------------------------------------
// LDS staging primitives (gfx950).
//
// async_copy16: one 16-byte global -> LDS copy per lane that bypasses VGPRs
// (global_load_lds_dwordx4). The LDS destination of a wave is contiguous:
// lane l writes bytes [base + 16 l, base + 16 l + 16), with `base` uniform
// across the wave; each lane picks its own global source. Completion is
// tracked by vmcnt: wait_async() then a barrier makes the data visible.
//
// read_tr4: ds_read_b64_tr_b16. Within each 16-lane group, lane i receives
// element (i % 4) of the 8-byte words addressed by lanes i/4, i/4 + 4,
// i/4 + 8 and i/4 + 12 (in that order). If lane s of the group addresses
// row r0 + s/4, column c0 + 4 (s % 4) of a row-major bf16 tile, lane i gets
// column c0 + i of rows r0 .. r0 + 3: a transposed 4-element fragment.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void async_copy16(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void_t*)lds_wave_base, 16, 0, 0);
}

__device__ __forceinline__ void wait_async() { __builtin_amdgcn_s_waitcnt(0); }
// Wait until at most N of this wave's vector-memory operations are still in
// flight (they complete in issue order for this count), leaving the LDS and
// export counters alone: copies issued after the ones needed stay in flight.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  // vmcnt in bits 3:0 and 15:14; expcnt 7 and lgkmcnt 15: no wait
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ u32x2 read_tr4(const bf16_t* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// Two floats -> packed bf16 pair (round to nearest even) in one
// v_cvt_pk_bf16_f32; converting the pair as a vector keeps the compiler from
// splitting it into two single conversions plus a shift and an or.
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
  const f32x2_v f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_v));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// XOR swizzles of the 16-byte slots of a row-major [row][D] bf16 tile
// (NS = D / 8 slots per row). Rows read 16 bytes at a time by 32 different
// rows (row-major MFMA operands) use slot ^ (row mod NS); rows read through
// read_tr4 (4 consecutive rows x 2 slots per 16-lane group) use
// slot ^ 4 (row mod 4). Both keep a wave's reads free of bank conflicts for
// D = 128.
template <int NS> __device__ __forceinline__ int swz_rows(int row) { return row & (NS - 1); }
template <int NS> __device__ __forceinline__ int swz_tr(int row) { return (4 * (row & 3)) & (NS - 1); }
// One swizzle for tiles read both ways: 16 consecutive rows take 16 distinct
// values (row-major reads) and 4 consecutive rows take 4 distinct 4-slot
// blocks (transposing reads).
template <int NS> __device__ __forceinline__ int swz_both(int row) {
  return (((row & 3) << 2) | ((row >> 2) & 3)) & (NS - 1);
}

enum SwzKind { kSwzRows = 0, kSwzTr = 1, kSwzBoth = 2 };
template <int NS, int KIND> __device__ __forceinline__ int swz(int row) {
  return KIND == kSwzRows ? swz_rows<NS>(row) : (KIND == kSwzTr ? swz_tr<NS>(row) : swz_both<NS>(row));
}

// Asynchronous copy of ROWS consecutive local key rows k0 .. k0 + ROWS - 1 of
// kv head g (D bf16 each; rows past the end repeat the last key: finite
// filler that the masks never use) into a row-major LDS tile whose 16-byte
// slots are permuted by the swizzle KIND. All THREADS threads take part.
template <int D, int ROWS, int THREADS, int KIND>
__device__ __forceinline__ void issue_rows_async(const bf16_t* __restrict__ src, int hkv, int g,
                                                 int k0, int n_keys, bf16_t* tile, int tid) {
  constexpr int NS = D / 8;
  constexpr int PASSES = ROWS * NS / THREADS;
  static_assert(PASSES * THREADS == ROWS * NS, "tile must split evenly over the threads");
  const int wave = tid >> 6;
  int t = tid;
  asm volatile("" : "+v"(t));  // opaque: nothing here is hoisted out of a caller's loop
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    const int u = pass * THREADS + t;
    const int row = u / NS, phys = u % NS;
    const int key = min(k0 + row, n_keys - 1);
    async_copy16(src + ((int64_t)key * hkv + g) * D + (phys ^ swz<NS, KIND>(row)) * 8,
                 tile + (pass * THREADS + wave * 64) * 8);
  }
}

// The same copy through a buffer resource: buffer_load_dwordx4 ... lds, with
// a scalar base and a 32-bit range (`bytes`; a raw buffer, byte offsets,
// loads past the range read zero), a per-lane offset and a scalar offset.
// As fast as the global form in the attention kernels (0-2% faster), and the
// hardware checks every load against the tile's range.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // word 3 = 0x00020000: the raw-buffer format of the gfx9 family
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ void async_copy16_buf(__amdgpu_buffer_rsrc_t r, uint32_t lane_off,
                                                 uint32_t scalar_off, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_wave_base, 16, lane_off,
                                           scalar_off, 0, 0);
}
// The same copy written as inline assembly, so that the compiler does not
// know of it and inserts no waits of its own before later LDS reads (its
// alias tracking of asynchronous LDS writes is conservative across a loop of
// three stages and waited for every copy in flight). The caller waits for the
// copies itself (wait_vmcnt / wait_async) and must not use M0 or the
// compiler's own LDS copies in the same kernel: the assembly sets M0 to the
// wave's LDS destination, given as a 32-bit LDS byte address (lds_addr of a
// __shared__ array plus an offset: a generic pointer would cost a null check
// and 64-bit registers per copy). NT marks data read once (non-temporal: not
// kept in the caches).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const lds_void_t*)p);
}
template <bool NT = false>
__device__ __forceinline__ void async_copy16_buf_asm(__amdgpu_buffer_rsrc_t r, uint32_t lane_off,
                                                     uint32_t scalar_off, uint32_t lds_wave) {
  const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_wave);
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :: "s"(lds), "v"(lane_off), "s"(r), "s"(scalar_off) : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(lane_off), "s"(r), "s"(scalar_off) : "memory");
}
// async_copy16 as inline assembly (same conventions).
__device__ __forceinline__ void async_copy16_asm(const void* gsrc, uint32_t lds_wave) {
  const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_wave);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds), "v"(gsrc) : "memory");
}
// A 64-bit address that is the same in every lane, read from the first lane
// into scalar registers (readfirstlane returns a signed int: each half goes
// through uint32_t so that it is zero-extended).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | (uint64_t)lo);
}

// The same copy for a tile that lies wholly inside the buffer. Row r of the
// tile sits r * row_stride elements after `first`, its 16-byte slot permuted
// by the swizzle KIND; rows of pass p sit p * THREADS / NS rows below those
// of pass 0, a multiple of 16, and the swizzles depend on the row modulo 16
// only, so one per-lane byte offset (tile_lane_offset, computed once by the
// caller and kept in one register) serves every pass. The tile's first
// address is the same in every lane and becomes a buffer resource over the
// tile's ROWS rows (ROWS * row_stride * 2 bytes, below 2^32); each pass adds
// its step as the scalar offset, so a pass costs no vector instruction. The
// lane offset is made opaque at each call so that the compiler keeps it in
// one register.
template <int D, int THREADS, int KIND>
__device__ __forceinline__ uint32_t tile_lane_offset(int64_t row_stride, int tid) {
  constexpr int NS = D / 8;
  const int row = tid / NS, phys = tid % NS;
  return (uint32_t)(row * (uint32_t)row_stride * 2u + (phys ^ swz<NS, KIND>(row)) * 16);
}
template <int D, int ROWS, int THREADS>
__device__ __forceinline__ void issue_tile_async_off(const bf16_t* first, int64_t row_stride,
                                                     uint32_t lane_off, bf16_t* tile, int tid,
                                                     int valid_rows = ROWS) {
  constexpr int NS = D / 8;
  constexpr int PASSES = ROWS * NS / THREADS;
  constexpr int ROWS_PER_PASS = THREADS / NS;
  static_assert(PASSES * THREADS == ROWS * NS, "tile must split evenly over the threads");
  static_assert(ROWS_PER_PASS % 16 == 0, "pass step must keep the swizzle");
  uint32_t off = lane_off;
  asm volatile("" : "+v"(off));
  // rows from valid_rows on lie outside the range: they read as zero
  const __amdgpu_buffer_rsrc_t r =
      make_rsrc(uniform_ptr(first), (uint32_t)(min(valid_rows, ROWS) * row_stride * 2));
  const uint32_t step = (uint32_t)(ROWS_PER_PASS * row_stride * 2);
  const int lds_off = __builtin_amdgcn_readfirstlane((tid >> 6) * 64 * 8);
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass)
    async_copy16_buf(r, off, pass * step, tile + pass * THREADS * 8 + lds_off);
}

// issue_tile_async_off through async_copy16_buf_asm (tile: LDS byte address).
template <int D, int ROWS, int THREADS>
__device__ __forceinline__ void issue_tile_async_asm(const bf16_t* first, int64_t row_stride,
                                                     uint32_t lane_off, uint32_t tile, int tid,
                                                     int valid_rows) {
  constexpr int NS = D / 8;
  constexpr int PASSES = ROWS * NS / THREADS;
  constexpr int ROWS_PER_PASS = THREADS / NS;
  static_assert(PASSES * THREADS == ROWS * NS, "tile must split evenly over the threads");
  static_assert(ROWS_PER_PASS % 16 == 0, "pass step must keep the swizzle");
  const __amdgpu_buffer_rsrc_t r =
      make_rsrc(uniform_ptr(first), (uint32_t)(min(valid_rows, ROWS) * row_stride * 2));
  const uint32_t step = (uint32_t)(ROWS_PER_PASS * row_stride * 2);
  const int lds_off = __builtin_amdgcn_readfirstlane((tid >> 6) * 64 * 8);
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass)
    async_copy16_buf_asm(r, lane_off, pass * step, tile + (pass * THREADS * 8 + lds_off) * 2);
}

// Local (per-rank) key range of one block. The local buffer holds the rank's
// chunks in ascending global position, so the keys a window [s, a) reaches
// form one contiguous local interval [lo, hi): lo counts local keys before s,
// hi counts local keys before a.
struct KeyRange {
  int lo, hi;
};

}  // namespace splitkv
