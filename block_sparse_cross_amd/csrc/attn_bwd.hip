// Backward of the local partial (Algorithm 1 of "Split-KV: Efficient Context
// Parallelism for Training Diffusion Drafters", §4.1: MERGE_BWD, then
// AttnBwd_p). With the merged (global) lse and Delta = <do, o>, every live pair
// (query vector r, key x) contributes
//   P = exp(scale <q_r, k_x> - lse_r),  dv_x += P do_r,
//   ds = P (<do_r, v_x> - Delta_r),     dq_r += scale ds k_x,  dk_x += scale ds q_r.
// dk and dv stay local to the rank; dq is accumulated (+=) so that the P
// emulated ranks of one device sum into one buffer.
//
// bf16 path:
//  1. bwd_prep_delta_kernel (Delta from o and do) or bwd_prep_kernel (Delta
//     given): per query vector, a record {-lse * log2 e, -Delta, lo, hi} with
//     the row's local key interval (lse = -inf stays -inf so that
//     P = exp2(. - inf) = 0), laid out per (kv head, 64-vector chunk) as four
//     64-wide arrays.
//  2. chunk_range_kernel: per 64-vector query chunk (one wave), the union of its
//     intervals and the interval that every vector of the chunk covers;
//     ds_offsets_kernel: where each chunk's dS goes in the workspace (if it
//     fits; see the stored-dS layout below).
//  3. attn_bwd_dkdv_kernel: a workgroup owns 128 local keys of one kv head (32
//     per wave; K and V fragments and the dK, dV accumulators in registers)
//     and walks the query chunks whose union reaches those keys. Q, dO and the
//     records of the next chunk are copied global -> LDS asynchronously
//     (double-buffered, row-major, XOR-swizzled) while the current chunk is
//     computed. Per 32-vector half of a chunk, with v_mfma_f32_32x32x16_bf16:
//     S = Q K^T and dP = dO V^T so that a lane owns one key and 16 vectors;
//     dV^T += dO^T P and dK^T += Q^T dS, the Q^T and dO^T fragments read by
//     the transposing LDS read. Chunks whose vectors all cover a wave's 32
//     keys skip the per-key mask. With room in the workspace it also stores
//     the packed dS (bf16) as it feeds dK^T.
//  4. dq, either way deterministic and without atomics:
//     attn_bwd_dq_ds_kernel: from the stored dS, dQ^T += K^T dS^T (one
//       d-contraction per pair, bound by streaming the dS from HBM);
//     attn_bwd_dq_kernel: query-outer like the forward, recomputing S and dP
//       per key tile (three d-contractions per pair), for the vector groups
//       whose dS was not stored.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace splitkv {

namespace {

constexpr int kBwdThreads = 256;  // 4 waves
constexpr int kBwdKeys = 128;     // keys per workgroup, 32 per wave
constexpr int kQC = kBwdChunk;    // query vectors per chunk (dK/dV kernel)
constexpr int kListCap = 1024;    // chunk indices buffered per scan
constexpr int kDqThreads = 512;  // dQ kernels: 8 waves, two per SIMD
constexpr int kDqWaves = kDqThreads / 64;
constexpr int kDqVecPerWG = 32 * kDqWaves;
constexpr int kDqKT = 64;

// Stored dS. For kv head g and query chunk c (64 vectors) whose key union is
// [ulo, uhi), each 32-key group kg = ulo / 32 .. ceil(uhi / 32) - 1 gets one
// 4 KB tile: two 2 KB halves (vectors 0-31, 32-63 of the chunk), each 32 key
// rows of 64 bytes. A row holds the half's 32 vectors as four 16-byte slots,
// slot 2 h2 + h = vectors 16 h2 + 4 h + (0..3) and 16 h2 + 8 + 4 h + (0..3):
// exactly the 8 values one lane of the dK/dV kernel packs for a 16-vector step
// (one 16-byte store), which the dQ kernel reads back transposed (8 keys of
// one vector) with ds_read_b64_tr_b16. Tile (g, c, kg) is number
// g cap + ds_off[c] + kg of the dS area (cap tiles per kv head); ds_off[c] is
// the exclusive prefix sum of the chunks' group counts minus ulo / 32, or
// kDsNone when the chunk's dQ-from-dS workgroup (8 chunks) does not fit and
// recomputes S and dP instead.
constexpr int kDsKeys = 32;
constexpr int kDsTileBytes = kQC * kDsKeys * 2;
constexpr int kDsVecPerWG = 512;                  // vectors per workgroup of the dQ-from-dS kernel
constexpr int kDsChunksPerWG = kDsVecPerWG / kQC;  // stored or not together
constexpr int kDsNone = -0x7fffffff - 1;
// Byte offset, in a half tile's 64-byte key row, of the 4 vectors u .. u + 3
// (u a multiple of 4 below 32).
__device__ __forceinline__ int ds_word_off(int u) {
  return 16 * (2 * (u >> 4) + ((u >> 2) & 1)) + 8 * ((u >> 3) & 1);
}

// Delta[r, h] = <do[r, h], o[r, h]>, one thread per (row, head). fp32 path.
template <int D, typename T>
__global__ void __launch_bounds__(256)
delta_kernel(const T* __restrict__ o, const T* __restrict__ dout, float* __restrict__ delta,
             int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  float acc = 0.f;
#pragma unroll 8
  for (int c = 0; c < D; ++c) acc = fmaf(Elem<T>::load(o + t * D + c), Elem<T>::load(dout + t * D + c), acc);
  delta[t] = acc;
}

// bf16 path: one record slot per (kv head g, 64-vector chunk c, t < 64), laid
// out as [g][c][field][t] with fields {-lse * log2 e, -Delta, lo, hi} (the
// starting values of the S and dP accumulators of the dK/dV kernel), so that
// one 1 KB copy stages a chunk's records as four 64-wide arrays. Rows without
// live keys and slots past the last vector start S at -inf (P = 0); dead slots
// have an empty interval.
//
// Delta from o and do: D/16 lanes per (row, head) in memory order (each lane
// two 16-byte pieces of o and of do, then a shuffle reduction), so the reads
// sweep o and do front to back, and the item's record goes to its slot.
// Threads past the last item fill the dead slots of every kv head's last
// chunk (vectors n_vec .. n_qc * 64 - 1). (Walking the slots instead read o
// and do one 1 KB piece per 8 KB row per kv head, at 40% of HBM bandwidth.)
template <int D>
__global__ void __launch_bounds__(256)
bwd_prep_delta_kernel(const bf16_t* __restrict__ o, const bf16_t* __restrict__ dout,
                      const float* __restrict__ lse, float* __restrict__ delta,
                      const int2* __restrict__ block_range, float* __restrict__ meta,
                      int64_t n_items, int64_t n_vec, int64_t n_qc, int G, int hq, int hkv,
                      int B) {
  constexpr int L = D / 16;  // lanes per item, two 16-byte pieces of o and of do each
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t item = gt / L;
  const int part = (int)(gt % L);
  const bool ok = item < n_items;
  float acc = 0.f;
  if (ok) {
    const u32x4* op = reinterpret_cast<const u32x4*>(o + item * D) + part;
    const u32x4* dp = reinterpret_cast<const u32x4*>(dout + item * D) + part;
    const u32x4 a0 = __builtin_nontemporal_load(op), a1 = __builtin_nontemporal_load(op + L);
    const u32x4 b0 = __builtin_nontemporal_load(dp), b1 = __builtin_nontemporal_load(dp + L);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(__uint_as_float(a0[w] << 16), __uint_as_float(b0[w] << 16), acc);
      acc = fmaf(__uint_as_float(a0[w] & 0xffff0000u), __uint_as_float(b0[w] & 0xffff0000u), acc);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(__uint_as_float(a1[w] << 16), __uint_as_float(b1[w] << 16), acc);
      acc = fmaf(__uint_as_float(a1[w] & 0xffff0000u), __uint_as_float(b1[w] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int off = L / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (part != 0) return;
  if (ok) {
    const int64_t row = item / hq;
    const int h = (int)(item - row * hq), g = h / G;
    const int64_t vec = row * G + (h - g * G);
    float* rec = meta + ((int64_t)g * n_qc + vec / kQC) * (4 * kQC) + vec % kQC;
    delta[item] = acc;
    const float l = lse[item];
    const int2 r = block_range[row / B];
    rec[0] = l == -INFINITY ? -INFINITY : -l * kLog2e;
    rec[kQC] = -acc;
    rec[2 * kQC] = __int_as_float(r.x);
    rec[3 * kQC] = __int_as_float(r.y);
    return;
  }
  const int64_t pad = n_qc * kQC - n_vec;  // dead slots per kv head
  const int64_t d = item - n_items;
  if (d >= pad * hkv) return;
  const int g = (int)(d / pad);
  const int64_t vec = n_vec + d % pad;
  float* rec = meta + ((int64_t)g * n_qc + vec / kQC) * (4 * kQC) + vec % kQC;
  rec[0] = -INFINITY;
  rec[kQC] = 0.f;
  rec[2 * kQC] = __int_as_float(0);
  rec[3 * kQC] = __int_as_float(0);
}

// Delta given: one lane per slot, in slot order (the record writes coalesce).
template <int D>
__global__ void __launch_bounds__(256)
bwd_prep_kernel(const float* __restrict__ lse, const float* __restrict__ delta,
                const int2* __restrict__ block_range, float* __restrict__ meta, int64_t n_vec,
                int64_t n_qc, int G, int gshift, int hq, int hkv, int B) {
  const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n_slots = (int64_t)hkv * n_qc * kQC;
  if (slot >= n_slots) return;
  const int64_t gc = slot / kQC;
  const int g = (int)(gc / n_qc);
  const uint32_t vec = (uint32_t)((gc % n_qc) * kQC + slot % kQC);
  float* rec = meta + gc * (4 * kQC) + slot % kQC;
  if (vec >= n_vec) {
    rec[0] = -INFINITY;
    rec[kQC] = 0.f;
    rec[2 * kQC] = __int_as_float(0);
    rec[3 * kQC] = __int_as_float(0);
    return;
  }
  const uint32_t rw = gshift >= 0 ? vec >> gshift : vec / (uint32_t)G;
  const int64_t item = (int64_t)rw * hq + g * G + (vec - rw * G);
  const float l = lse[item];
  const int2 r = block_range[rw / B];
  rec[0] = l == -INFINITY ? -INFINITY : -l * kLog2e;
  rec[kQC] = -delta[item];
  rec[2 * kQC] = __int_as_float(r.x);
  rec[3 * kQC] = __int_as_float(r.y);
}

// Per 64-vector chunk c: {min lo, max hi} over its non-empty vectors (union),
// {max lo, min hi} over all 64 slots (what every vector covers; vectors past
// the end count as empty). One wave per chunk, lane t = vector 64 c + t, the
// four extremes by wave reductions.
constexpr int kRangeThreads = 256;
__global__ void __launch_bounds__(kRangeThreads)
chunk_range_kernel(const int2* __restrict__ block_range, int64_t n_vec, int G, int B,
                   int64_t n_qc, int4* __restrict__ out) {
  static_assert(kQC == kWave, "one lane per vector of a chunk");
  const int64_t c = ((int64_t)blockIdx.x * kRangeThreads + threadIdx.x) / kWave;
  const int lane = threadIdx.x % kWave;
  if (c >= n_qc) return;  // whole waves: c is the same in every lane of a wave
  const int64_t vec = c * kQC + lane;
  int2 r = make_int2(0, 0);
  if (vec < n_vec) r = block_range[(vec / G) / B];
  const bool live = r.x < r.y;
  const int ulo = wave_min_i(live ? r.x : 0x7fffffff);
  const int uhi = wave_max_i(live ? r.y : -1);
  const int clo = wave_max_i(r.x);
  const int chi = wave_min_i(r.y);
  if (lane == 0) out[c] = uhi < 0 ? make_int4(0, 0, 0, 0) : make_int4(ulo, uhi, clo, chi);
}

// ds_off (see kDsNone) for every chunk: one workgroup scans the group counts
// in pieces of 1024 chunks with a running carry. A dQ-from-dS workgroup's 8 chunks
// are stored when the prefix sum at their end fits in cap tiles per kv head,
// so the stored workgroups are a prefix in vector order. need (if not null)
// receives the bytes that store every chunk: hkv tiles_total kDsTileBytes.
constexpr int kDsScanThreads = 1024;
__global__ void __launch_bounds__(kDsScanThreads)
ds_offsets_kernel(const int4* __restrict__ chunk_range, int64_t n_qc, int64_t cap, int hkv,
                  int* __restrict__ ds_off, int64_t* __restrict__ need) {
  static_assert(kWave % kDsChunksPerWG == 0, "a dQ workgroup's chunks lie in one wave");
  __shared__ int64_t wsum[kDsScanThreads / kWave];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  int64_t carry = 0;
  for (int64_t base = 0; base < n_qc; base += kDsScanThreads) {
    const int64_t c = base + tid;
    int4 cr = make_int4(0, 0, 0, 0);
    if (c < n_qc) cr = chunk_range[c];
    const int64_t n = cr.x < cr.y ? ((cr.y + kDsKeys - 1) / kDsKeys) - cr.x / kDsKeys : 0;
    int64_t incl = n;  // inclusive scan within the wave
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int64_t o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int64_t before = carry, total = 0;
#pragma unroll
    for (int w = 0; w < kDsScanThreads / kWave; ++w) {
      before += w < wave ? wsum[w] : 0;
      total += wsum[w];
    }
    incl += before;
    // prefix sum at the end of this chunk's dQ workgroup (chunks past n_qc
    // count zero, so the last lane of the group holds it)
    const int64_t end = __shfl(incl, lane | (kDsChunksPerWG - 1));
    if (c < n_qc)
      ds_off[c] = end <= cap ? (int)(incl - n - cr.x / kDsKeys) : kDsNone;
    carry += total;
    __syncthreads();  // wsum is rewritten by the next piece
  }
  if (need != nullptr && tid == 0) *need = carry * hkv * kDsTileBytes;
}

template <int D>
__global__ void __launch_bounds__(kBwdThreads, 1)
attn_bwd_dkdv_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                     const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
                     const float* __restrict__ meta, bf16_t* __restrict__ dk,
                     bf16_t* __restrict__ dv, const int4* __restrict__ chunk_range,
                     bf16_t* __restrict__ ds, const int* __restrict__ ds_off, int64_t ds_cap,
                     int64_t n_vec, int64_t n_qc, int G, int gshift, int hq, int hkv,
                     int n_keys, float scale, float scale_log2) {
  constexpr int NS = D / 8;
  constexpr int NW = kBwdThreads / 64;
  // Double buffers as distinct arrays: the chunk loop is unrolled by two so
  // the compiler can tell the next chunk's asynchronous LDS writes from the
  // current chunk's reads (and does not wait for the copies to land). The Q
  // and dO tiles of one stage share an array (dO 16 KB after Q), so one
  // per-lane read offset serves both with an immediate displacement; with
  // four arrays the compiler kept a register per (array, offset) and spilled.
  __shared__ __attribute__((aligned(16))) bf16_t QD0[2 * kQC * D];
  __shared__ __attribute__((aligned(16))) bf16_t QD1[2 * kQC * D];
  bf16_t* const Qs0 = QD0;
  bf16_t* const dOs0 = QD0 + kQC * D;
  bf16_t* const Qs1 = QD1;
  bf16_t* const dOs1 = QD1 + kQC * D;
  __shared__ __attribute__((aligned(16))) float Ms0[4 * kQC];
  __shared__ __attribute__((aligned(16))) float Ms1[4 * kQC];
  __shared__ int list[kListCap];
  __shared__ int4 lrange[kListCap];
  __shared__ int ldsoff[kListCap];
  __shared__ int wave_cnt[NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int g = blockIdx.x % hkv;  // kv head fastest: one kv head per XCD
  const int k0 = (blockIdx.x / hkv) * kBwdKeys;
  const int kend = min(k0 + kBwdKeys, n_keys);
  const int kw0 = k0 + wave * 32;
  const int krow = wave * 32 + (lane & 31);  // this lane's key row in Kl
  const int mykey = k0 + krow;
  const int s16 = lane & 15;

  // K, V fragments of this wave's 32 keys (B operands of S and dP: lane = key,
  // 8 d values).
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (mykey < n_keys) {
      const int64_t off = ((int64_t)mykey * hkv + g) * D + ks * 16 + half * 8;
      a = *reinterpret_cast<const u32x4*>(k + off);
      b = *reinterpret_cast<const u32x4*>(v + off);
    }
    // K times scale * log2 e (rounded to bf16): S is then the exponent of P
#pragma unroll
    for (int w = 0; w < 4; ++w)
      a[w] = pack_bf16x2_hw(__uint_as_float(a[w] << 16) * scale_log2,
                            __uint_as_float(a[w] & 0xffff0000u) * scale_log2);
    kf[ks] = as_bf16x8(a);
    vf[ks] = as_bf16x8(b);
  }

  f32x16 dvt[D / 32], dkt[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dvt[dt][r] = 0.f; dkt[dt][r] = 0.f; }

  // Stage chunk c (kQC vectors): Q, dO rows and the records by asynchronous
  // copies (inline assembly the compiler does not track: the chunk step's own
  // waits are the only ones, and may leave the last chunk's dS stores in
  // flight). Vectors past the end reuse the last vector's rows (their records
  // are dead, so they add exact zeros).
  //
  // Fast path (G a power of two dividing kQC, chunk inside the buffer): a
  // chunk is kQC / G whole rows times G heads, so vector vec0 + r sits at
  // element ((vec0 / G + r / G) hq + g G + r % G) D. With r = RPP p + t (t the
  // lane's row within pass p, RPP = rows per pass) the offset splits into a
  // per-lane part fixed for the kernel and a part uniform per pass.
  constexpr int RPP = kBwdThreads / NS;         // vector rows per copy pass
  constexpr int QPASSES = kQC * NS / kBwdThreads;  // passes per tensor
  const bool fast_chunks = gshift >= 0 && gshift <= 6 && (kQC % G) == 0;
  uint32_t lane_off = 0;
  {
    const int t = tid / NS, phys = tid % NS;
    const int tg = fast_chunks ? (t >> gshift) : 0, th = fast_chunks ? (t & (G - 1)) : 0;
    lane_off = (uint32_t)(((int64_t)tg * hq + th) * D * 2 + ((phys ^ swz_both<NS>(t)) * 16));
  }
  const int lds_wave = __builtin_amdgcn_readfirstlane(wave * 64 * 8);
  auto issue_chunk = [&](int64_t c, bf16_t* Qd, bf16_t* Dd, float* Md) {
    const uint32_t qa = lds_addr(Qd), da = lds_addr(Dd), ma = lds_addr(Md);
    const int64_t vec0 = c * kQC;
    if (fast_chunks && vec0 + kQC <= n_vec) {
      // the chunk's kQC / G rows of all hq heads, as buffer resources
      const int64_t first = ((vec0 >> gshift) * hq + (int64_t)g * G) * D;
      const uint32_t span = (uint32_t)((kQC >> gshift) * (int64_t)hq * D * 2);
      const __amdgpu_buffer_rsrc_t qr = make_rsrc(uniform_ptr(q + first), span);
      const __amdgpu_buffer_rsrc_t dr = make_rsrc(uniform_ptr(dout + first), span);
#pragma unroll
      for (int pp = 0; pp < QPASSES; ++pp) {
        const int r0 = RPP * pp;
        const uint32_t step = (uint32_t)((((int64_t)(r0 >> gshift)) * hq + (r0 & (G - 1))) * D * 2);
        async_copy16_buf_asm(qr, lane_off, step, qa + (pp * kBwdThreads * 8 + lds_wave) * 2);
        async_copy16_buf_asm(dr, lane_off, step, da + (pp * kBwdThreads * 8 + lds_wave) * 2);
      }
      if (wave == NW - 1 && lane < kQC)
        async_copy16_asm(meta + ((int64_t)g * n_qc + c) * (4 * kQC) + lane * 4, ma);
      return;
    }
#pragma unroll
    for (int pass = 0; pass < 2 * kQC * NS / kBwdThreads; ++pass) {
      const int u = pass * kBwdThreads + tid;      // over [tensor][row][slot]
      const int tsel = u / (kQC * NS);
      const int uu = u % (kQC * NS);
      const int row = uu / NS, phys = uu % NS;
      const uint32_t vec = (uint32_t)min(vec0 + row, n_vec - 1);
      const uint32_t rw = gshift >= 0 ? vec >> gshift : vec / (uint32_t)G;
      const int64_t idx = (int64_t)rw * hq + g * G + (vec - rw * G);
      const bf16_t* src = (tsel ? dout : q) + idx * D + (phys ^ swz_both<NS>(row)) * 8;
      async_copy16_asm(src, (tsel ? da : qa) + (uu - lane) * 16);
    }
    if (wave == NW - 1 && lane < kQC)
      async_copy16_asm(meta + ((int64_t)g * n_qc + c) * (4 * kQC) + lane * 4, ma);
  };

  // Element offsets of this lane's transposing reads of Q and dO (rows t and
  // t + 8 of each 16-vector step, t = 4 half + s16 / 4), per 32-column block
  // dt; opaque so that step offsets and buffer bases become immediates.
  int tr_off[D / 32][2];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int t = 4 * half + (s16 >> 2);
    const int dcol = dt * 32 + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
    tr_off[dt][0] = t * D + (((dcol >> 3) ^ swz_both<NS>(t)) * 8) + (dcol & 7);
    tr_off[dt][1] = (t + 8) * D + (((dcol >> 3) ^ swz_both<NS>(t + 8)) * 8) + (dcol & 7);
    asm volatile("" : "+v"(tr_off[dt][0]), "+v"(tr_off[dt][1]));
  }

  // Element offsets of this lane's row-major reads of Q and dO (row lane % 32
  // of a half, d-step ks; the second half adds 32 rows) and of its first record
  // in a 4-vector group. Opaque, like tr_off, so that each buffer's base
  // becomes an immediate instead of one register per (buffer, offset).
  int row_off[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const int qrow = lane & 31;
    row_off[ks] = qrow * D + (((2 * ks + half) ^ swz_both<NS>(qrow)) * 8);
    asm volatile("" : "+v"(row_off[ks]));
  }
  int rec_off = 4 * half;
  asm volatile("" : "+v"(rec_off));

  // Byte offset of this lane's dS slot in a stored tile: its key's row, slot
  // `half` (the vector half and h2 add 2048 hv + 32 h2 as immediates).
  int ds_lane = (lane & 31) * (kDsKeys * 2) + 16 * half;
  asm volatile("" : "+v"(ds_lane));
  bool stored_last = false;  // the last computed chunk issued its 4 dS stores

  // S = Q K^T and dP = dO V^T (lane = key, 16 vectors per lane), P, dS,
  // dV^T += dO^T P, dK^T += Q^T dS, for the chunk's 32-vector halves. The
  // products of all halves are issued before the elementwise work, so one
  // half's softmax overlaps the other half's matrix-core work.
  constexpr int NH = kQC / 32;
  // MASKED: some vector's interval cuts this wave's 32 keys (per-key test);
  // otherwise every vector of the chunk covers them all. The two variants are
  // separate code so that the common unmasked one has no branches inside.
  auto compute_chunk = [&](auto masked, const bf16_t* Qb, const bf16_t* Db, const float* Mb,
                           int dso) {
    constexpr bool MASKED = decltype(masked)::value;
    static_assert(NH == 2, "chunk = two 32-vector halves");
    f32x16 sacc[NH], pacc[NH];
    // operands of a piece (two products), read three pieces ahead: Q and dO
    // rows for S / dP, dO^T and Q^T fragments for dV^T / dK^T
    u32x4 opa[4], opb[4];
    int4 mlo[2], mhi[2];     // key intervals of 4 vectors (masked chunks only)
    u32x4 pu, su;            // P and dS of the current 16-vector step, bf16
    // this wave's stored dS tile of the chunk as a buffer resource (scalar),
    // of zero range when the chunk is not stored: the hardware then drops
    // the stores, and every computed chunk issues the same 4 stores
    const bool st = dso != kDsNone;
    const int64_t tile = (int64_t)g * ds_cap + (st ? dso : 0) + (kw0 / kDsKeys);
    const __amdgpu_buffer_rsrc_t dsr =
        make_rsrc(st ? uniform_ptr(ds + tile * (kDsTileBytes / 2)) : (const void*)ds,
                  st ? (uint32_t)kDsTileBytes : 0u);
    stored_last = true;
    // dS of the current 16-vector step: one 16-byte store (lane offset in a
    // VGPR, the step's offset as the scalar offset; a plain store: the
    // non-temporal form was 5% slower here)
    auto store_ds = [&](int hv, int h2) {
      __builtin_amdgcn_raw_buffer_store_b128(su, dsr, ds_lane, hv * (kDsTileBytes / 2) + 32 * h2,
                                             0);
    };

    auto load_sd = [&](int hv, int ks, int b) {
      opa[b] = *reinterpret_cast<const u32x4*>(&Qb[hv * 32 * D + row_off[ks]]);
      opb[b] = *reinterpret_cast<const u32x4*>(&Db[hv * 32 * D + row_off[ks]]);
    };
    auto load_upd = [&](int hv, int h2, int dt, int b) {
      const int vbase = (hv * 32 + 16 * h2) * D;
      const int o0 = vbase + tr_off[dt][0], o1 = vbase + tr_off[dt][1];
      const u32x2 d0 = read_tr4(&Db[o0]), d1 = read_tr4(&Db[o1]);
      const u32x2 q0 = read_tr4(&Qb[o0]), q1 = read_tr4(&Qb[o1]);
      opa[b] = u32x4{d0.x, d0.y, d1.x, d1.y};
      opb[b] = u32x4{q0.x, q0.y, q1.x, q1.y};
    };
    // The accumulators of S and dP of half hv start from the records'
    // -lse log2 e and -Delta (element r of a lane is vector 8 (r / 4) +
    // 4 half + r % 4 of the half), so that P = exp2(S) and dS = P dP after
    // the products.
    auto load_init = [&](int hv) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int q0 = hv * 32 + 8 * jj + rec_off;
        const float4 l = *reinterpret_cast<const float4*>(&Mb[q0]);
        const float4 d = *reinterpret_cast<const float4*>(&Mb[kQC + q0]);
        sacc[hv][4 * jj + 0] = l.x; sacc[hv][4 * jj + 1] = l.y;
        sacc[hv][4 * jj + 2] = l.z; sacc[hv][4 * jj + 3] = l.w;
        pacc[hv][4 * jj + 0] = d.x; pacc[hv][4 * jj + 1] = d.y;
        pacc[hv][4 * jj + 2] = d.z; pacc[hv][4 * jj + 3] = d.w;
      }
    };
    auto load_meta = [&](int hv, int jj) {
      const int q0 = hv * 32 + 8 * jj + rec_off, b = jj & 1;
      mlo[b] = *reinterpret_cast<const int4*>(&Mb[2 * kQC + q0]);
      mhi[b] = *reinterpret_cast<const int4*>(&Mb[3 * kQC + q0]);
    };
    // The chunk runs in pieces: NP = D / 16 per phase, and the P, dS work of
    // a half is spread over NP pieces, EPP elements each.
    constexpr int NP = D / 16, DT = D / 32, EPP = 16 / NP;
    // P and dS of elements EPP w .. EPP w + EPP - 1 of half hv, in place.
    auto weigh = [&](int hv, int w) {
#pragma unroll
      for (int e = 0; e < EPP; ++e) {
        const int r = EPP * w + e, jj = r >> 2, i = r & 3, b = jj & 1;
        float pk = fast_exp2(sacc[hv][r]);
        if constexpr (MASKED) {
          const int lo = i == 0 ? mlo[b].x : i == 1 ? mlo[b].y : i == 2 ? mlo[b].z : mlo[b].w;
          const int hi = i == 0 ? mhi[b].x : i == 1 ? mhi[b].y : i == 2 ? mhi[b].z : mhi[b].w;
          pk = (mykey >= lo && mykey < hi) ? pk : 0.f;
        }
        sacc[hv][r] = pk;
        pacc[hv][r] = pk * pacc[hv][r];
      }
    };
    auto pack = [&](int hv, int h2) {
      pu.x = pack_bf16x2_hw(sacc[hv][8 * h2 + 0], sacc[hv][8 * h2 + 1]);
      pu.y = pack_bf16x2_hw(sacc[hv][8 * h2 + 2], sacc[hv][8 * h2 + 3]);
      pu.z = pack_bf16x2_hw(sacc[hv][8 * h2 + 4], sacc[hv][8 * h2 + 5]);
      pu.w = pack_bf16x2_hw(sacc[hv][8 * h2 + 6], sacc[hv][8 * h2 + 7]);
      su.x = pack_bf16x2_hw(pacc[hv][8 * h2 + 0], pacc[hv][8 * h2 + 1]);
      su.y = pack_bf16x2_hw(pacc[hv][8 * h2 + 2], pacc[hv][8 * h2 + 3]);
      su.z = pack_bf16x2_hw(pacc[hv][8 * h2 + 4], pacc[hv][8 * h2 + 5]);
      su.w = pack_bf16x2_hw(pacc[hv][8 * h2 + 6], pacc[hv][8 * h2 + 7]);
    };

    // One wave per SIMD, so matrix-core and vector work overlap only as far
    // as the instruction order lets them. The chunk runs as 4 NP pieces of two
    // products each, fenced so that the compiler keeps them in this order
    // (nothing moves across __builtin_amdgcn_sched_barrier(0)):
    //   phase 0: S, dP of half 0 (d-step ks = piece)
    //   phase 1: S, dP of half 1, with P, dS of half 0
    //   phase 2: dV^T, dK^T of half 0 (16-vector step h2, column block dt),
    //            with P, dS of half 1
    //   phase 3: dV^T, dK^T of half 1
    // A piece issues the LDS reads of the piece three later (operand slot =
    // piece mod 4): reading one piece ahead in the phases with vector work
    // (and two in the others) left the matrix core waiting on LDS latency;
    // three ahead everywhere was 1-4% faster per call.
    auto load_piece = [&](int x) {
      const int ph = x / NP, i = x % NP;
      if (ph < 2) load_sd(ph, i, x % 4);
      else if (ph < 4) load_upd(ph - 2, i / DT, i % DT, x % 4);
    };
    // The key intervals of 8-vector group jj of half hv (masked chunks) are
    // first used in piece NP (hv + 1) + 4 jj / EPP; they are loaded G = 4 / EPP
    // pieces earlier, when the group two back (same register slot) is done.
    // Half 0's accumulator starts are read before the first piece, half 1's
    // two pieces before its products begin.
    constexpr int G = 4 / EPP;
    load_init(0);
    load_piece(0);
    load_piece(1);
    load_piece(2);
#pragma unroll
    for (int pc = 0; pc < 4 * NP; ++pc) {
      if (pc + 3 < 4 * NP) load_piece(pc + 3);
      if constexpr (MASKED) {
#pragma unroll
        for (int hv = 0; hv < NH; ++hv)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            if (NP * (hv + 1) + (4 * jj) / EPP - G == pc) load_meta(hv, jj);
      }
      if (pc == NP - 2) load_init(1);
      const int ph = pc / NP, i = pc % NP, b = pc % 4;
      if (ph < 2) {
        sacc[ph] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(opa[b]), kf[i], sacc[ph], 0, 0, 0);
        pacc[ph] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(opb[b]), vf[i], pacc[ph], 0, 0, 0);
      } else {
        const int hv = ph - 2, h2 = i / DT, dt = i % DT;
        if (dt == 0) {
          pack(hv, h2);
          store_ds(hv, h2);
        }
        dvt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(opa[b]), as_bf16x8(pu), dvt[dt], 0, 0, 0);
        dkt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(opb[b]), as_bf16x8(su), dkt[dt], 0, 0, 0);
      }
      if (ph == 1 || ph == 2) weigh(ph - 1, i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto compute_phase = [&](const int4 cr, const bf16_t* Qb, const bf16_t* Db, const float* Mb,
                           int dso) {
    const bool active = cr.x < kw0 + 32 && cr.y > kw0;
    if (!active) return;
    if (cr.z <= kw0 && cr.w >= kw0 + 32)
      compute_chunk(std::false_type{}, Qb, Db, Mb, dso);
    else
      compute_chunk(std::true_type{}, Qb, Db, Mb, dso);
  };

  for (int64_t scan = 0; scan < n_qc;) {
    // ---- collect (in order) the chunks whose union reaches this workgroup ----
    int n = 0;
    while (scan < n_qc && n + kBwdThreads <= kListCap) {
      const int64_t c = scan + tid;
      int4 cr = make_int4(0, 0, 0, 0);
      bool live = false;
      int dso = kDsNone;
      if (c < n_qc) {
        cr = chunk_range[c];
        live = cr.x < cr.y && cr.x < kend && cr.y > k0;
        dso = ds_off[c];
      }
      const unsigned long long bal = __ballot(live);
      if (lane == 0) wave_cnt[wave] = __popcll(bal);
      __syncthreads();
      int off = n, total = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) { off += (w < wave) ? wave_cnt[w] : 0; total += wave_cnt[w]; }
      if (live) {
        const int slot = off + __popcll(bal & ((1ull << lane) - 1ull));
        list[slot] = (int)c;
        lrange[slot] = cr;
        ldsoff[slot] = dso;
      }
      n += total;
      scan += kBwdThreads;
      __syncthreads();
    }

    // ---- software pipeline over the list: per chunk `it`, one barrier, the
    // copies of chunk it+1, then the compute of chunk it. Workgroups of one kv
    // head (one XCD) walk their lists in the same ascending order, so the
    // query chunks they share are read from that XCD's L2. ----
    auto at = [](int it) { return it; };
    auto step = [&](int it, const bf16_t* Qb, const bf16_t* Db, const float* Mb, bf16_t* Qn,
                    bf16_t* Dn, float* Mn) {
      // the copies of chunk it; the 4 dS stores of the last chunk (issued
      // after them, counted by vmcnt too) may stay in flight
      if (stored_last)
        wait_vmcnt<4>();
      else
        wait_async();
      stored_last = false;
      // a bare barrier (__syncthreads' fence would wait for the stores)
      asm volatile("s_barrier" ::: "memory");
      if (it + 1 < n) issue_chunk(__builtin_amdgcn_readfirstlane(list[at(it + 1)]), Qn, Dn, Mn);
      const int4 cr = lrange[at(it)];
      compute_phase(make_int4(__builtin_amdgcn_readfirstlane(cr.x), __builtin_amdgcn_readfirstlane(cr.y),
                              __builtin_amdgcn_readfirstlane(cr.z), __builtin_amdgcn_readfirstlane(cr.w)),
                    Qb, Db, Mb, __builtin_amdgcn_readfirstlane(ldsoff[at(it)]));
    };
    stored_last = false;  // no store follows the copies of chunk 0
    if (n > 0) issue_chunk(__builtin_amdgcn_readfirstlane(list[at(0)]), Qs0, dOs0, Ms0);
    for (int it = 0; it < n; it += 2) {
      step(it, Qs0, dOs0, Ms0, Qs1, dOs1, Ms1);
      if (it + 1 < n) step(it + 1, Qs1, dOs1, Ms1, Qs0, dOs0, Ms0);
    }
    __syncthreads();  // the list and the buffers are reused by the next scan
  }

  // ---- write dK = scale * dK^T, dV = dV^T for this wave's keys ----
  wait_async();  // no copy into this workgroup's LDS may outlive it
  if (mykey < n_keys) {
    bf16_t* dkp = dk + ((int64_t)mykey * hkv + g) * D;
    bf16_t* dvp = dv + ((int64_t)mykey * hkv + g) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = dt * 32 + 8 * jj + 4 * half;
        u32x2 a, b;
        a.x = pack_bf16x2_hw(dkt[dt][4 * jj] * scale, dkt[dt][4 * jj + 1] * scale);
        a.y = pack_bf16x2_hw(dkt[dt][4 * jj + 2] * scale, dkt[dt][4 * jj + 3] * scale);
        b.x = pack_bf16x2_hw(dvt[dt][4 * jj], dvt[dt][4 * jj + 1]);
        b.y = pack_bf16x2_hw(dvt[dt][4 * jj + 2], dvt[dt][4 * jj + 3]);
        *reinterpret_cast<u32x2*>(dkp + d0) = a;
        *reinterpret_cast<u32x2*>(dvp + d0) = b;
      }
  }
}

// dQ, query-outer (no atomics): a workgroup takes 256 consecutive query
// vectors of one kv head (32 per wave, lane % 32 = the lane's vector) and
// walks the 64-key tiles of their key intervals, like the forward kernel. With
// the global lse the weights need no running statistics:
//   S^T = K Q^T, dP^T = V dO^T, dS^T = P (dP - Delta), dQ^T += K^T dS^T,
// the K^T fragments coming from the row-major K tile through the transposing
// read. dq += scale * dQ once at the end (each (row, head) has one owner).
template <int D>
__global__ void __launch_bounds__(kDqThreads, 1)
attn_bwd_dq_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                   const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
                   const float* __restrict__ lse, const float* __restrict__ delta,
                   float* __restrict__ dq, const int2* __restrict__ block_range,
                   const int* __restrict__ ds_off, int64_t n_vec, int G, int hq, int hkv, int B,
                   int n_keys, float scale, float scale_log2) {
  constexpr int NS = D / 8;
  // vector groups in reverse (longest windows first), as in the forward
  const int64_t group = (gridDim.x / hkv) - 1 - blockIdx.x / hkv;
  // a group whose dS the dK/dV kernel stored is attn_bwd_dq_ds_kernel's (the
  // decision is the same for all chunks of its larger groups)
  if (ds_off[group * (kDqVecPerWG / kQC)] != kDsNone) return;
  __shared__ __attribute__((aligned(16))) bf16_t K0[kDqKT * D];
  __shared__ __attribute__((aligned(16))) bf16_t V0[kDqKT * D];
  __shared__ __attribute__((aligned(16))) bf16_t K1[kDqKT * D];
  __shared__ __attribute__((aligned(16))) bf16_t V1[kDqKT * D];
  __shared__ int wave_lo[kDqWaves], wave_hi[kDqWaves];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int s16 = lane & 15;
  const int g = __builtin_amdgcn_readfirstlane(blockIdx.x % hkv);
  const int64_t vec = group * kDqVecPerWG + wave * 32 + (lane & 31);
  const bool valid = vec < n_vec;
  int64_t row = 0;
  int hh = 0, qlo = 0, qhi = 0;
  float lse2 = INFINITY, dl = 0.f;
  if (valid) {
    row = vec / G;
    hh = (int)(vec % G);
    const int64_t idx = row * hq + (int64_t)g * G + hh;
    const float l = lse[idx];
    if (l != -INFINITY) {
      const int2 r = block_range[row / B];
      qlo = r.x;
      qhi = r.y;
      lse2 = l * kLog2e;
    }
    dl = delta[idx];
  }
  const bool live_lane = valid && qlo < qhi;
  const int64_t head_off = (row * hq + (int64_t)g * G + hh) * D;
  // (the same in every lane; readfirstlane keeps the tile tests scalar)
  const int wlo = __builtin_amdgcn_readfirstlane(wave_min_i(live_lane ? qlo : 0x7fffffff));
  const int whi = __builtin_amdgcn_readfirstlane(wave_max_i(live_lane ? qhi : -1));
  const int wall_lo = __builtin_amdgcn_readfirstlane(wave_max_i(live_lane ? qlo : 0x7fffffff));
  const int wall_hi = __builtin_amdgcn_readfirstlane(wave_min_i(live_lane ? qhi : -1));
  if (lane == 0) { wave_lo[wave] = wlo; wave_hi[wave] = whi; }

  // Q and dO fragments (B operands of S^T = K Q^T and dP^T = V dO^T). The Q
  // fragment is taken times scale * log2 e (rounded to bf16), so the product
  // gives the exponent of P directly.
  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (valid) {
      a = *reinterpret_cast<const u32x4*>(q + head_off + ks * 16 + half * 8);
      b = *reinterpret_cast<const u32x4*>(dout + head_off + ks * 16 + half * 8);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w)
      a[w] = pack_bf16x2_hw(__uint_as_float(a[w] << 16) * scale_log2,
                            __uint_as_float(a[w] & 0xffff0000u) * scale_log2);
    qf[ks] = as_bf16x8(a);
    df[ks] = as_bf16x8(b);
  }
  // Accumulator starts: S^T from -lse log2 e (so P = exp2 of the product;
  // -inf for a row without live keys gives P = 0) and dP^T from -Delta (so
  // dS = P times the product). A lane's 16 accumulator values all belong to
  // its own query vector.
  f32x16 s_init, p_init;
#pragma unroll
  for (int r = 0; r < 16; ++r) { s_init[r] = -lse2; p_init[r] = -dl; }
  __syncthreads();
  int lo = 0x7fffffff, hi = -1;
#pragma unroll
  for (int w = 0; w < kDqWaves; ++w) { lo = min(lo, wave_lo[w]); hi = max(hi, wave_hi[w]); }
  lo = __builtin_amdgcn_readfirstlane(lo);
  hi = __builtin_amdgcn_readfirstlane(hi);

  const uint32_t k_off = tile_lane_offset<D, kDqThreads, kSwzBoth>((int64_t)hkv * D, tid);
  // V takes K's swizzle, so one per-lane offset table serves the row-major
  // reads of both
  const uint32_t v_off = tile_lane_offset<D, kDqThreads, kSwzBoth>((int64_t)hkv * D, tid);
  auto issue_tile = [&](int k0, bf16_t* Kn, bf16_t* Vn) {
    if (k0 + kDqKT <= n_keys) {
      const int64_t first = ((int64_t)k0 * hkv + g) * D;
      issue_tile_async_off<D, kDqKT, kDqThreads>(k + first, (int64_t)hkv * D, k_off, Kn, tid);
      issue_tile_async_off<D, kDqKT, kDqThreads>(v + first, (int64_t)hkv * D, v_off, Vn, tid);
    } else {
      issue_rows_async<D, kDqKT, kDqThreads, kSwzBoth>(k, hkv, g, k0, n_keys, Kn, tid);
      issue_rows_async<D, kDqKT, kDqThreads, kSwzBoth>(v, hkv, g, k0, n_keys, Vn, tid);
    }
  };

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[dt][r] = 0.f;

  // Element offsets of this lane's transposing reads of K (rows t and t + 8
  // of each 16-key step, t = 4 half + s16 / 4), per 32-column block dt. They
  // are opaque to the compiler so that it adds the step's row offset and the
  // buffer's base as immediates instead of rebuilding each address.
  int tr_off[D / 32][2];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int t = 4 * half + (s16 >> 2);
    const int dcol = dt * 32 + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
    tr_off[dt][0] = t * D + (((dcol >> 3) ^ swz_both<NS>(t)) * 8) + (dcol & 7);
    tr_off[dt][1] = (t + 8) * D + (((dcol >> 3) ^ swz_both<NS>(t + 8)) * 8) + (dcol & 7);
    asm volatile("" : "+v"(tr_off[dt][0]), "+v"(tr_off[dt][1]));
  }

  // Element offsets of this lane's row-major reads of K and V (key row
  // lane % 32 of a 32-key half, d-step ks); the swizzle depends on the row
  // modulo 16 only, so the second half adds 32 D. Opaque, like tr_off.
  int kro[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const int kr = lane & 31;
    kro[ks] = kr * D + (((2 * ks + half) ^ swz_both<NS>(kr)) * 8);
    asm volatile("" : "+v"(kro[ks]));
  }

  auto tile_step = [&](int k0, const bf16_t* Kt, const bf16_t* Vt, bf16_t* Kn, bf16_t* Vn) {
    wait_async();
    __syncthreads();
    if (k0 + kDqKT < hi) issue_tile(k0 + kDqKT, Kn, Vn);
    if (!(k0 < whi && k0 + kDqKT > wlo)) return;
    const bool tile_masked = k0 < wall_lo || k0 + kDqKT > wall_hi;
    // The tile's two 32-key halves one after the other: S^T, dP^T (16
    // products), the weights, dQ^T (8 products); only one half's scores are
    // live at a time.
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int hb = mt * 32 * D;
      f32x16 sacc = s_init, pacc = p_init;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&Kt[hb + kro[ks]]);
        const u32x4 b = *reinterpret_cast<const u32x4*>(&Vt[hb + kro[ks]]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qf[ks], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(b), df[ks], pacc, 0, 0, 0);
      }
      // dS^T = P (dP - Delta) (both already in the accumulators: the exponent
      // of P and dP - Delta); the per-key test only on tiles that cut some
      // lane's interval (a separate copy of the loop, so the common case has
      // no per-element branches)
      auto weights = [&](auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(sacc[r]);
          if constexpr (MASKED) {
            const int key = k0 + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            p = (key >= qlo && key < qhi) ? p : 0.f;
          }
          sacc[r] = p * pacc[r];
        }
      };
      if (tile_masked)
        weights(std::true_type{});
      else
        weights(std::false_type{});
      // dQ^T += K^T dS^T, two 16-key steps
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        u32x4 su;
        su.x = pack_bf16x2_hw(sacc[8 * h2 + 0], sacc[8 * h2 + 1]);
        su.y = pack_bf16x2_hw(sacc[8 * h2 + 2], sacc[8 * h2 + 3]);
        su.z = pack_bf16x2_hw(sacc[8 * h2 + 4], sacc[8 * h2 + 5]);
        su.w = pack_bf16x2_hw(sacc[8 * h2 + 6], sacc[8 * h2 + 7]);
        const int kbase = (mt * 32 + 16 * h2) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const u32x2 x0 = read_tr4(&Kt[kbase + tr_off[dt][0]]);
          const u32x2 x1 = read_tr4(&Kt[kbase + tr_off[dt][1]]);
          const u32x4 au = {x0.x, x0.y, x1.x, x1.y};
          dqacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(au), as_bf16x8(su), dqacc[dt], 0, 0, 0);
        }
      }
    }
  };

  if (lo < hi) issue_tile(lo, K0, V0);
  for (int k0 = lo; k0 < hi; k0 += 2 * kDqKT) {
    tile_step(k0, K0, V0, K1, V1);
    if (k0 + kDqKT < hi) tile_step(k0 + kDqKT, K1, V1, K0, V0);
  }

  if (live_lane) {
    float* dp = dq + head_off;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = dt * 32 + 8 * jj + 4 * half;
        float4 cur = *reinterpret_cast<float4*>(dp + d0);
        cur.x = fmaf(dqacc[dt][4 * jj], scale, cur.x);
        cur.y = fmaf(dqacc[dt][4 * jj + 1], scale, cur.y);
        cur.z = fmaf(dqacc[dt][4 * jj + 2], scale, cur.z);
        cur.w = fmaf(dqacc[dt][4 * jj + 3], scale, cur.w);
        *reinterpret_cast<float4*>(dp + d0) = cur;
      }
  }
}

// dQ from the stored dS, for the vector groups whose dS the dK/dV kernel
// stored: a workgroup takes 512 consecutive vectors of one kv head, one
// 64-vector chunk per wave (groups in reverse order, longest windows first).
// Per tile of KT keys (KT / 32 stored groups), dQ^T += K^T dS^T with the K^T
// fragments read from the row-major K tile by the transposing read (each one
// serves both 32-vector halves of the wave's chunk) and the dS^T fragments (8
// keys of the lane's vector) likewise from the stored key rows. Each wave
// copies its own chunk's tiles (4 KB per group) and all waves the shared K
// tile, global -> LDS asynchronously into a ring of NSTAGE stages, NSTAGE - 1
// tiles ahead. The kernel streams 2 bytes of dS per live (vector, key) pair
// from HBM and does one d-contraction per pair.
template <int D>
__global__ void __launch_bounds__(kDqThreads, 1)
attn_bwd_dq_ds_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ ds,
                      const float* __restrict__ lse, float* __restrict__ dq,
                      const int2* __restrict__ block_range, const int4* __restrict__ chunk_range,
                      const int* __restrict__ ds_off, int64_t ds_cap, int64_t n_vec,
                      int64_t n_qc, int G, int hq, int hkv, int B, int n_keys, float scale) {
  constexpr int NS = D / 8;
  constexpr int KT = D == 128 ? kDsKeys : 2 * kDsKeys;  // keys per tile (one K copy pass)
  constexpr int NG = KT / kDsKeys;                       // stored groups per tile
  constexpr int TE = kDsTileBytes / 2;         // elements of a stored tile (a chunk's group)
  constexpr int KPASS = KT * NS / kDqThreads;  // K copies per lane per tile
  constexpr int GCOPY = kDsTileBytes / (kWave * 16);  // dS copies per lane per group
  constexpr int NCOPY = KPASS + NG * GCOPY;    // copies per lane per tile
  constexpr int SE = KT * D + kDqWaves * NG * TE;       // stage: K tile, then the waves' dS
  constexpr int NSTAGE = (150 * 1024) / (SE * 2) < 3 ? (150 * 1024) / (SE * 2) : 3;
  constexpr int LA = NSTAGE - 1;               // tiles in flight ahead of the computed one
  static_assert(KPASS == 1 && GCOPY == 4 && NSTAGE >= 2 && NCOPY * LA < 64, "ring");
  static_assert(kDsVecPerWG == kQC * kDqWaves, "one chunk per wave");

  const int64_t group = (gridDim.x / hkv) - 1 - blockIdx.x / hkv;
  const int64_t c0 = group * kDsChunksPerWG;
  if (ds_off[c0] == kDsNone) return;  // recomputed by attn_bwd_dq_kernel

  // one ring (the copies are assembly the compiler does not see: the waits
  // below are the only ones, so one array with a run-time stage serves)
  __shared__ __attribute__((aligned(16))) bf16_t ring[NSTAGE * SE];
  __shared__ int wave_lo[kDqWaves], wave_hi[kDqWaves];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s16 = lane & 15;
  const int g = __builtin_amdgcn_readfirstlane(blockIdx.x % hkv);
  const int64_t c = c0 + wave;  // this wave's chunk

  // the wave's stored groups [glo, ghi)
  int glo = 0, ghi = 0, dso = 0;
  if (c < n_qc) {
    const int4 cr = chunk_range[c];
    if (cr.x < cr.y) {
      glo = cr.x / kDsKeys;
      ghi = (cr.y + kDsKeys - 1) / kDsKeys;
      dso = ds_off[c];
    }
  }
  glo = __builtin_amdgcn_readfirstlane(glo);
  ghi = __builtin_amdgcn_readfirstlane(ghi);
  dso = __builtin_amdgcn_readfirstlane(dso);
  if (lane == 0) {
    wave_lo[wave] = glo < ghi ? glo : 0x7fffffff;
    wave_hi[wave] = glo < ghi ? ghi : -1;
  }

  // the lane's two vectors (one per 32-vector half of the chunk)
  bool live_lane[2];
  int64_t head_off[2];
#pragma unroll
  for (int hv = 0; hv < 2; ++hv) {
    const int64_t vec = c * kQC + hv * 32 + (lane & 31);
    live_lane[hv] = false;
    head_off[hv] = 0;
    if (vec < n_vec) {
      const int64_t row = vec / G;
      const int64_t idx = row * hq + (int64_t)g * G + (int)(vec % G);
      head_off[hv] = idx * D;
      if (lse[idx] != -INFINITY) {
        const int2 r = block_range[row / B];
        live_lane[hv] = r.x < r.y;
      }
    }
  }

  __syncthreads();
  int lo = 0x7fffffff, hi = -1;
#pragma unroll
  for (int w = 0; w < kDqWaves; ++w) { lo = min(lo, wave_lo[w]); hi = max(hi, wave_hi[w]); }
  lo = __builtin_amdgcn_readfirstlane(lo);
  hi = __builtin_amdgcn_readfirstlane(hi);
  const int n_t = lo < hi ? (hi - lo + NG - 1) / NG : 0;

  const uint32_t k_off = tile_lane_offset<D, kDqThreads, kSwzBoth>((int64_t)hkv * D, tid);
  // a stored tile is copied as it lies (copy j takes bytes 1024 j + 16 lane)
  const uint32_t ds_src = (uint32_t)(lane * 16);
  auto issue = [&](int t, uint32_t sa) {  // sa: the stage's LDS byte address
    const int kg0 = lo + NG * t;
    const int k0 = kg0 * kDsKeys;
    // rows past the last key read as zero (their dS is zero)
    issue_tile_async_asm<D, KT, kDqThreads>(k + ((int64_t)k0 * hkv + g) * D, (int64_t)hkv * D,
                                            k_off, sa, tid, n_keys - k0);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int kg = kg0 + gi;
      const bool present = kg >= glo && kg < ghi;
      const int64_t tile = (int64_t)g * ds_cap + dso + kg;
      // an absent group is a zero-range copy into the wave's own slot: every
      // wave counts the same copies per tile (the waits count copies)
      const __amdgpu_buffer_rsrc_t r =
          make_rsrc(present ? uniform_ptr(ds + tile * TE) : (const void*)ds,
                    present ? (uint32_t)kDsTileBytes : 0u);
#pragma unroll
      for (int j = 0; j < GCOPY; ++j)
        async_copy16_buf_asm<true>(r, ds_src, (uint32_t)(j * kWave * 16),
                                   sa + (KT * D + (wave * NG + gi) * TE + j * kWave * 8) * 2);
    }
  };

  // transposing reads of K (rows t and t + 8 of each 16-key step) and of the
  // lane's dS (opaque offsets, so that step offsets become immediates): lane s
  // of each 16-lane group addresses key row 4 half + s / 4 and the 4 vectors
  // 16 ((lane / 16) % 2) + 4 (s % 4) of a half (rows 8 further for the second
  // read, 16 further per 16-key step, 1024 elements further for the second
  // half); the read hands lane l the 4 keys of vector l % 32
  int tr_off[D / 32][2];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int t = 4 * half + (s16 >> 2);
    const int dcol = dt * 32 + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
    tr_off[dt][0] = t * D + (((dcol >> 3) ^ swz_both<NS>(t)) * 8) + (dcol & 7);
    tr_off[dt][1] = (t + 8) * D + (((dcol >> 3) ^ swz_both<NS>(t + 8)) * 8) + (dcol & 7);
    asm volatile("" : "+v"(tr_off[dt][0]), "+v"(tr_off[dt][1]));
  }
  int rd_off;
  {
    const int s = lane & 15;
    const int u = 16 * ((lane >> 4) & 1) + 4 * (s & 3);
    rd_off = KT * D + wave * NG * TE + (4 * half + (s >> 2)) * kDsKeys + ds_word_off(u) / 2;
    asm volatile("" : "+v"(rd_off));
  }

  f32x16 dqacc[2][D / 32];
#pragma unroll
  for (int hv = 0; hv < 2; ++hv)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) dqacc[hv][dt][r] = 0.f;

  auto compute = [&](int t, const bf16_t* St) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int kg = lo + NG * t + gi;
      if (!(kg >= glo && kg < ghi)) continue;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        u32x4 su[2];
#pragma unroll
        for (int hv = 0; hv < 2; ++hv) {
          const int sb = gi * TE + hv * (TE / 2) + h2 * 16 * kDsKeys;
          const u32x2 y0 = read_tr4(&St[sb + rd_off]);
          const u32x2 y1 = read_tr4(&St[sb + 8 * kDsKeys + rd_off]);
          su[hv] = u32x4{y0.x, y0.y, y1.x, y1.y};
        }
        const int kbase = (gi * kDsKeys + 16 * h2) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const u32x2 x0 = read_tr4(&St[kbase + tr_off[dt][0]]);
          const u32x2 x1 = read_tr4(&St[kbase + tr_off[dt][1]]);
          const u32x4 au = {x0.x, x0.y, x1.x, x1.y};
#pragma unroll
          for (int hv = 0; hv < 2; ++hv)
            dqacc[hv][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                as_bf16x8(au), as_bf16x8(su[hv]), dqacc[hv][dt], 0, 0, 0);
        }
      }
    }
  };

  // Step u: wait until this wave's copies of tile t = u - LA have landed (the
  // later tiles' copies, NCOPY each, stay in flight), barrier (tile t visible
  // to all waves; every wave is done with tile u - NSTAGE, whose stage tile u
  // takes), copies of tile u, compute tile t.
  int s_issue = 0, s_comp = 0;  // stages of tiles u and t
  for (int u = 0; u < n_t + LA; ++u) {
    const int t = u - LA;
    if (t >= 0) {
      const int later = min(u - 1, n_t - 1) - t;  // tiles issued after t
      if (later >= 2)
        wait_vmcnt<(LA >= 3 ? 2 : 0) * NCOPY>();
      else if (later == 1)
        wait_vmcnt<NCOPY>();
      else
        wait_async();
    }
    // a bare barrier: __syncthreads' fence would wait for every copy in flight
    asm volatile("s_barrier" ::: "memory");
    if (u < n_t) issue(u, lds_addr(ring) + s_issue * SE * 2);
    if (t >= 0) compute(t, ring + s_comp * SE);
    s_issue = s_issue + 1 == NSTAGE ? 0 : s_issue + 1;
    if (t >= 0) s_comp = s_comp + 1 == NSTAGE ? 0 : s_comp + 1;
  }

#pragma unroll
  for (int hv = 0; hv < 2; ++hv) {
    if (!live_lane[hv]) continue;
    float* dp = dq + head_off[hv];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = dt * 32 + 8 * jj + 4 * half;
        float4 cur = *reinterpret_cast<float4*>(dp + d0);
        cur.x = fmaf(dqacc[hv][dt][4 * jj], scale, cur.x);
        cur.y = fmaf(dqacc[hv][dt][4 * jj + 1], scale, cur.y);
        cur.z = fmaf(dqacc[hv][dt][4 * jj + 2], scale, cur.z);
        cur.w = fmaf(dqacc[hv][dt][4 * jj + 3], scale, cur.w);
        *reinterpret_cast<float4*>(dp + d0) = cur;
      }
  }
}

// fp32 path, part 1: dq per (row, head), one thread each, plain loops.
template <int D>
__global__ void __launch_bounds__(128)
bwd_dq_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                  const float* __restrict__ v, const float* __restrict__ dout,
                  const float* __restrict__ lse, const float* __restrict__ delta,
                  float* __restrict__ dq, const int2* __restrict__ block_range, int64_t n_rows,
                  int hq, int hkv, int B, float scale) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_rows * hq) return;
  const int64_t row = t / hq;
  const int h = (int)(t % hq), g = h / (hq / hkv);
  const float l = lse[t];
  if (l == -INFINITY) return;
  const int2 r = block_range[row / B];
  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;
  for (int x = r.x; x < r.y; ++x) {
    const float* kv = k + ((int64_t)x * hkv + g) * D;
    const float* vv = v + ((int64_t)x * hkv + g) * D;
    float z = 0.f, dp = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      z = fmaf(q[t * D + c], kv[c], z);
      dp = fmaf(dout[t * D + c], vv[c], dp);
    }
    const float p = __expf(z * scale - l);
    const float ds = p * (dp - delta[t]);
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] = fmaf(ds * scale, kv[c], acc[c]);
  }
#pragma unroll
  for (int c = 0; c < D; ++c) dq[t * D + c] += acc[c];
}

// fp32 path, part 2: dk, dv per (key, kv head), one thread each, scanning the
// blocks whose interval holds the key.
template <int D>
__global__ void __launch_bounds__(128)
bwd_dkdv_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                    const float* __restrict__ v, const float* __restrict__ dout,
                    const float* __restrict__ lse, const float* __restrict__ delta,
                    float* __restrict__ dk, float* __restrict__ dv,
                    const int2* __restrict__ block_range, int64_t n_blocks, int n_keys, int hq,
                    int hkv, int B, float scale) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)n_keys * hkv) return;
  const int x = (int)(t / hkv), g = (int)(t % hkv), G = hq / hkv;
  const float* kv = k + t * D;
  const float* vv = v + t * D;
  float ak[D], av[D];
#pragma unroll
  for (int c = 0; c < D; ++c) { ak[c] = 0.f; av[c] = 0.f; }
  for (int64_t i = 0; i < n_blocks; ++i) {
    const int2 r = block_range[i];
    if (x < r.x || x >= r.y) continue;
    for (int64_t row = i * B; row < (i + 1) * B; ++row)
      for (int h = g * G; h < (g + 1) * G; ++h) {
        const int64_t idx = row * hq + h;
        const float l = lse[idx];
        if (l == -INFINITY) continue;
        const float* qv = q + idx * D;
        const float* gv = dout + idx * D;
        float z = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
          z = fmaf(qv[c], kv[c], z);
          dp = fmaf(gv[c], vv[c], dp);
        }
        const float p = __expf(z * scale - l);
        const float ds = p * (dp - delta[idx]);
#pragma unroll
        for (int c = 0; c < D; ++c) {
          av[c] = fmaf(p, gv[c], av[c]);
          ak[c] = fmaf(ds * scale, qv[c], ak[c]);
        }
      }
  }
#pragma unroll
  for (int c = 0; c < D; ++c) { dk[t * D + c] = ak[c]; dv[t * D + c] = av[c]; }
}

// Stored-dS tiles per kv head that ds_bytes hold (0 when fewer than one per
// head; at most 2^30 so that tile numbers stay in int range).
int64_t ds_capacity(size_t ds_bytes, int hkv) {
  const int64_t cap = (int64_t)(ds_bytes / ((size_t)kDsTileBytes * (size_t)hkv));
  return cap < (int64_t(1) << 30) ? cap : (int64_t(1) << 30);
}

template <int D>
hipError_t launch_bwd_t(const splitkv_anchors& an, const splitkv_heads& hd, int64_t n_keys,
                        const int2* block_range, void* meta_ws, void* chunk_ws, int* ds_off,
                        void* ds_area, size_t ds_bytes, const void* q, const void* k,
                        const void* v, const void* o, const void* dout, const float* lse,
                        float* delta, float* dq, void* dk, void* dv, hipStream_t stream) {
  const int64_t Q = an.n_blocks * an.block_size;
  const int64_t n_rh = Q * hd.hq;
  hipError_t err;
  if (hd.dtype == SPLITKV_BF16) {
    const int G = hd.hq / hd.hkv;
    const int64_t n_vec = Q * G;
    const int64_t n_qc = (n_vec + kQC - 1) / kQC;
    float* meta = static_cast<float*>(meta_ws);
    const int gshift = (G & (G - 1)) == 0 ? __builtin_ctz(G) : -1;
    int4* chunk_range = static_cast<int4*>(chunk_ws);
    const int64_t cap = ds_capacity(ds_bytes, hd.hkv);
    bf16_t* ds_bf16 = static_cast<bf16_t*>(ds_area);
    if (n_rh > 0) {
      const int64_t slots = (int64_t)hd.hkv * n_qc * kQC;
      if (o != nullptr) {
        // every (row, head), then the dead slots of each kv head's last chunk
        const int64_t threads = (n_rh + (n_qc * kQC - n_vec) * hd.hkv) * (D / 16);
        hipLaunchKernelGGL((bwd_prep_delta_kernel<D>), dim3((unsigned)((threads + 255) / 256)),
                           dim3(256), 0, stream, static_cast<const bf16_t*>(o),
                           static_cast<const bf16_t*>(dout), lse, delta, block_range, meta,
                           n_rh, n_vec, n_qc, G, hd.hq, hd.hkv, an.block_size);
      } else {  // Delta given: one lane per slot
        hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)((slots + 255) / 256)),
                           dim3(256), 0, stream, lse, delta, block_range, meta, n_vec, n_qc, G,
                           gshift, hd.hq, hd.hkv, an.block_size);
      }
      if ((err = hipGetLastError()) != hipSuccess) return err;
      const int64_t per_wg = kRangeThreads / kWave;  // chunks per workgroup
      hipLaunchKernelGGL(chunk_range_kernel, dim3((unsigned)((n_qc + per_wg - 1) / per_wg)),
                         dim3(kRangeThreads), 0, stream, block_range, n_vec, G, an.block_size,
                         n_qc, chunk_range);
      if ((err = hipGetLastError()) != hipSuccess) return err;
      hipLaunchKernelGGL(ds_offsets_kernel, dim3(1), dim3(kDsScanThreads), 0, stream,
                         chunk_range, n_qc, cap, hd.hkv, ds_off, static_cast<int64_t*>(nullptr));
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (n_keys == 0) return hipSuccess;
    const int64_t n_tiles = (n_keys + kBwdKeys - 1) / kBwdKeys;
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D>), dim3((unsigned)(n_tiles * hd.hkv)),
                       dim3(kBwdThreads), 0, stream, static_cast<const bf16_t*>(q),
                       static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),
                       static_cast<const bf16_t*>(dout), meta, static_cast<bf16_t*>(dk),
                       static_cast<bf16_t*>(dv), chunk_range, ds_bf16, ds_off, cap, n_vec, n_qc,
                       G, gshift, hd.hq, hd.hkv, (int)n_keys, hd.scale, hd.scale * kLog2e);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (n_rh == 0) return hipSuccess;
    // each vector group takes exactly one of the two dQ kernels (ds_off)
    const int64_t n_groups = (n_vec + kDqVecPerWG - 1) / kDqVecPerWG;
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D>), dim3((unsigned)(n_groups * hd.hkv)),
                       dim3(kDqThreads), 0, stream, static_cast<const bf16_t*>(q),
                       static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),
                       static_cast<const bf16_t*>(dout), lse, delta, dq, block_range, ds_off,
                       n_vec, G, hd.hq, hd.hkv, an.block_size, (int)n_keys, hd.scale,
                       hd.scale * kLog2e);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (cap == 0) return hipSuccess;  // only groups without keys count as stored
    const int64_t n_ds_groups = (n_vec + kDsVecPerWG - 1) / kDsVecPerWG;
    hipLaunchKernelGGL((attn_bwd_dq_ds_kernel<D>), dim3((unsigned)(n_ds_groups * hd.hkv)),
                       dim3(kDqThreads), 0, stream, static_cast<const bf16_t*>(k), ds_bf16, lse,
                       dq, block_range, chunk_range, ds_off, cap, n_vec, n_qc, G, hd.hq, hd.hkv,
                       an.block_size, (int)n_keys, hd.scale);
    return hipGetLastError();
  }
  if (o != nullptr && n_rh > 0) {
    hipLaunchKernelGGL((delta_kernel<D, float>), dim3((unsigned)((n_rh + 255) / 256)), dim3(256),
                       0, stream, static_cast<const float*>(o), static_cast<const float*>(dout),
                       delta, n_rh);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (n_rh > 0) {
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D>), dim3((unsigned)((n_rh + 127) / 128)), dim3(128),
                       0, stream, static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), static_cast<const float*>(dout), lse, delta,
                       dq, block_range, Q, hd.hq, hd.hkv, an.block_size, hd.scale);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const int64_t n_kg = n_keys * hd.hkv;
  if (n_kg == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D>), dim3((unsigned)((n_kg + 127) / 128)), dim3(128),
                     0, stream, static_cast<const float*>(q), static_cast<const float*>(k),
                     static_cast<const float*>(v), static_cast<const float*>(dout), lse, delta,
                     static_cast<float*>(dk), static_cast<float*>(dv), block_range, an.n_blocks,
                     (int)n_keys, hd.hq, hd.hkv, an.block_size, hd.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const splitkv_anchors& an, const splitkv_heads& hd, int64_t n_keys,
                      const int2* block_range, void* meta, void* chunk_range, int* ds_off,
                      void* ds_area, size_t ds_bytes, const void* q, const void* k,
                      const void* v, const void* o, const void* dout, const float* lse,
                      float* delta, float* dq, void* dk, void* dv, hipStream_t stream) {
  if (hd.d == 128)
    return launch_bwd_t<128>(an, hd, n_keys, block_range, meta, chunk_range, ds_off, ds_area,
                             ds_bytes, q, k, v, o, dout, lse, delta, dq, dk, dv, stream);
  return launch_bwd_t<64>(an, hd, n_keys, block_range, meta, chunk_range, ds_off, ds_area,
                          ds_bytes, q, k, v, o, dout, lse, delta, dq, dk, dv, stream);
}

hipError_t launch_bwd_ds_need(const splitkv_anchors& an, const splitkv_heads& hd,
                              const int2* block_range, void* chunk_ws, int* ds_off,
                              int64_t* need, hipStream_t stream) {
  const int G = hd.hq / hd.hkv;
  const int64_t n_vec = an.n_blocks * an.block_size * G;
  const int64_t n_qc = (n_vec + kQC - 1) / kQC;
  int4* chunk_range = static_cast<int4*>(chunk_ws);
  if (n_qc > 0) {
    const int64_t per_wg = kRangeThreads / kWave;
    hipLaunchKernelGGL(chunk_range_kernel, dim3((unsigned)((n_qc + per_wg - 1) / per_wg)),
                       dim3(kRangeThreads), 0, stream, block_range, n_vec, G, an.block_size,
                       n_qc, chunk_range);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // the bf16 path alone stores dS; fp32 needs none (hkv 0 makes need 0)
  hipLaunchKernelGGL(ds_offsets_kernel, dim3(1), dim3(kDsScanThreads), 0, stream, chunk_range,
                     n_qc, (int64_t)0, hd.dtype == SPLITKV_BF16 ? hd.hkv : 0, ds_off, need);
  return hipGetLastError();
}

}  // namespace splitkv
