// Dense bf16 matrix products for the projections around the attention of one
// draft layer (QProj, KeyValueProj, OProj and their backward; Algorithm 1 of
// "Split-KV: Efficient Context Parallelism for Training Diffusion Drafters").
// With OProj linear, each rank's rescaled partial is projected on its own and
// the results summed with the bias added once (Eq. 5): the accumulate flag and
// the optional bias of the epilogue express exactly that.
//
//   C[M][N] (+)= op(A) op(B) (+ bias)    fp32 accumulation, C in fp32 or bf16
//   NT: A [M][K], B [N][K]  (x W^T: forward projections)
//   NN: A [M][K], B [K][N]  (dY W: gradient of a projection's input)
//   TN: A [K][M], B [K][N]  (dY^T X: gradient of a projection's weight)
//
// Work decomposition. A workgroup of 8 waves (two per SIMD) computes a
// 256 x 256 tile of C; wave (wm, wn) owns 64 rows x 128 columns as 2 x 4
// blocks of the 32x32x16 bf16 matrix-core product (128 fp32 accumulators per
// lane). K advances 64 at a time through two LDS stage buffers (A and B
// slices, 64 KB per stage, declared as separate arrays): the A and B slices of
// step k + 1 are copied global -> LDS with asynchronous 16-byte loads while
// step k is multiplied, one copy per fenced piece of two products, from
// per-lane 32-bit offsets fixed per workgroup plus a scalar slice base; one
// barrier per step.
//
// Operand tiles in LDS. A slice whose rows run along K ("k-major": A in NT and
// NN, B in NT) is stored [256][64], 128-byte rows, and read 8 k-values per
// lane with one 16-byte LDS read; its 16-byte slots are XOR-permuted by
// (row / 2) mod 8, so the 16 rows a quarter-wave reads land on 16 distinct
// bank groups. A slice whose rows run along M or N ("mn-major": B in NN and
// TN, A in TN) is stored [64][256] and read transposed (ds_read_b64_tr_b16,
// 4 k-values per read, two per fragment); its slots are permuted by
// 4 (row mod 4), so the 4 rows of a transposing read hit distinct banks. The
// fragments of the next 16-deep step are read behind the current step's
// products.
//
// Paired products. C (+)= op(A1) op(B1) + op(A2) op(B2) with both pairs of the
// same shape runs the second product's K slices after the first's in the same
// accumulators (one output pass instead of a second read-modify-write): the
// gradient of a rank's context rows is dk Wk + dv Wv.
//
// Split K. When C is fp32 and the tiles leave a round of the chip part-filled,
// the tiles of that last round have K cut into splits of at least 8 slices;
// each (tile, split) workgroup adds its partial product into C with atomic
// fp32 adds (C zeroed first unless the call accumulates; the bias comes with
// split 0), while the tiles of the full rounds before it keep all of K and a
// plain store. With fewer tiles than one round (a rank's weight gradient
// 1024 x 5120 from K = 16384 rows is 80 tiles) every tile is split; with 320
// tiles (5120 x 4096) the last 64 take four splits each, so the launch lasts
// 1.25 tile-times instead of 2 (the launcher's rule says when it pays). The order of the atomic adds varies from run
// to run, so split tiles are reproducible to rounding only.
//
// Edges. M and N need not be multiples of the tile: rows and columns past the
// end are read from the last valid row or 8-column group (finite filler) and
// never stored. The last K step zero-fills the slots past K (K is a multiple
// of 8, so a 16-byte slot is wholly inside or outside), so they add nothing.
// The grid is ordered so that each XCD (workgroups are dealt round-robin over
// the 8 XCDs) takes a contiguous run of tiles, grouped 8 tile-rows at a time,
// so tiles that share A rows or B columns meet in the same L2.
#include "common.hpp"
#include "internal.hpp"

namespace splitkv {

namespace {

constexpr int kWM = 4;                      // waves along M (2 along N): 8 waves, two per SIMD
constexpr int kGemmThreads = 64 * 2 * kWM;
constexpr int kMI = 256 / kWM / 32;         // 32-row blocks per wave (2)
constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kNSK = kBK / 8;               // 16-byte slots per k-major row
constexpr int kKS = kBK / 16;               // 16-deep product steps per slice
constexpr int kTileElems = kBM * kBK;       // both operand slices hold 256 x kBK elements
constexpr int kPasses = kTileElems / 8 / kGemmThreads;  // 16-byte copies per thread per slice
constexpr int kGroupRows = 8;               // tile-rows per group of the grid order
constexpr int kXcds = 8;

// k-major slice [256][kBK]: kNSK slots per row; 16 consecutive rows span
// 16 kNSK slots, and slot ^ ((row / (16 / kNSK)) mod kNSK) puts the same
// logical slot of those rows on 16 distinct bank groups
__device__ __forceinline__ int kmaj_swz(int row) { return (row / (16 / kNSK)) & (kNSK - 1); }
// mn-major slice [kBK][256]: 32 slots per row, slot ^ 4 (row & 3)
__device__ __forceinline__ int mnmaj_swz(int row) { return 4 * (row & 3); }

// Copy one k-major slice: rows r0 .. r0 + 255 (clamped to < R) of a row-major
// [R][ld] matrix, columns k0 .. k0 + kBK - 1 (slots at or past K zero-filled
// when TAIL). Thread t, pass p handles LDS slot u = kGemmThreads p + t: row
// u / kNSK, physical slot u % kNSK, holding logical slot phys ^ swz(row).
template <bool TAIL>
__device__ __forceinline__ void copy_kmajor(const bf16_t* __restrict__ src, int64_t R, int64_t ld,
                                            int64_t r0, int64_t k0, int64_t K, bf16_t* tile,
                                            int tid) {
  const int lds_off = __builtin_amdgcn_readfirstlane((tid >> 6) * 64 * 8);
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int u = pass * kGemmThreads + tid;
    const int row = u / kNSK, phys = u % kNSK;
    const int lslot = phys ^ kmaj_swz(row);
    const int64_t r = min(r0 + row, R - 1);
    const int64_t k = k0 + 8 * lslot;
    bf16_t* dst = tile + pass * kGemmThreads * 8 + lds_off;
    if (!TAIL || k < K) {
      async_copy16(src + r * ld + k, dst);
    } else {
      *reinterpret_cast<u32x4*>(tile + (int64_t)u * 8) = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Copy one mn-major slice: rows k0 .. k0 + kBK - 1 (rows at or past K zero-filled
// when TAIL) of a row-major [K][C] matrix, columns c0 .. c0 + 255 (8-column
// groups past C read from the last group). LDS slot u: row u / 32, physical
// slot u % 32.
template <bool TAIL>
__device__ __forceinline__ void copy_mnmajor(const bf16_t* __restrict__ src, int64_t C, int64_t c0,
                                             int64_t k0, int64_t K, bf16_t* tile, int tid) {
  const int lds_off = __builtin_amdgcn_readfirstlane((tid >> 6) * 64 * 8);
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int u = pass * kGemmThreads + tid;
    const int row = u >> 5, phys = u & 31;
    const int lslot = phys ^ mnmaj_swz(row);
    const int64_t c = min(c0 + 8 * lslot, C - 8);
    const int64_t k = k0 + row;
    bf16_t* dst = tile + pass * kGemmThreads * 8 + lds_off;
    if (!TAIL || k < K) {
      async_copy16(src + k * C + c, dst);
    } else {
      *reinterpret_cast<u32x4*>(tile + (int64_t)u * 8) = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Fragment of 32 rows (r0 ..) x 16 k (step ks) from a k-major slice: lane l
// holds row r0 + (l mod 32), k-values 16 ks + 8 (l / 32) .. + 8.
__device__ __forceinline__ bf16x8 frag_kmajor(const bf16_t* tile, int r0, int ks, int lane) {
  const int row = r0 + (lane & 31);
  const int lslot = 2 * ks + (lane >> 5);
  return as_bf16x8(*reinterpret_cast<const u32x4*>(tile + row * kBK + ((lslot ^ kmaj_swz(row)) * 8)));
}

// The same fragment from an mn-major slice (columns c0 .. c0 + 31 of rows =
// k): two transposing reads of 4 k-values. In 16-lane group g (lanes 16 g ..),
// lane s addresses k-row kb + s / 4 and columns cb + 4 (s mod 4), where
// kb = 16 ks + 8 (g / 2) (+ 4 for the second read) and cb = c0 + 16 (g mod 2).
__device__ __forceinline__ bf16x8 frag_mnmajor(const bf16_t* tile, int c0, int ks, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int kb = 16 * ks + 8 * (g >> 1) + (s >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (s & 3);
  const int slot = col >> 3, within = col & 7;
  const int row0 = kb, row1 = kb + 4;
  const u32x2 lo = read_tr4(tile + row0 * kBN + (((slot ^ mnmaj_swz(row0)) * 8) + within));
  const u32x2 hi = read_tr4(tile + row1 * kBN + (((slot ^ mnmaj_swz(row1)) * 8) + within));
  return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
}

template <int LAYOUT>
struct Layout {
  static constexpr bool A_KMAJOR = LAYOUT != SPLITKV_GEMM_TN;
  static constexpr bool B_KMAJOR = LAYOUT == SPLITKV_GEMM_NT;
};

template <int LAYOUT>
__device__ __forceinline__ bf16x8 frag_a(const bf16_t* ta, int wm, int i, int ks, int lane) {
  return Layout<LAYOUT>::A_KMAJOR ? frag_kmajor(ta, wm * (kMI * 32) + 32 * i, ks, lane)
                                  : frag_mnmajor(ta, wm * (kMI * 32) + 32 * i, ks, lane);
}
template <int LAYOUT>
__device__ __forceinline__ bf16x8 frag_b(const bf16_t* tb, int wn, int j, int ks, int lane) {
  return Layout<LAYOUT>::B_KMAJOR ? frag_kmajor(tb, wn * 128 + 32 * j, ks, lane)
                                  : frag_mnmajor(tb, wn * 128 + 32 * j, ks, lane);
}

template <int LAYOUT, bool TAIL>
__device__ __forceinline__ void copy_step(const bf16_t* A, const bf16_t* B, int64_t M, int64_t N,
                                          int64_t K, int64_t m0, int64_t n0, int64_t k0,
                                          bf16_t* ta, bf16_t* tb, int tid) {
  if constexpr (Layout<LAYOUT>::A_KMAJOR)
    copy_kmajor<TAIL>(A, M, K, m0, k0, K, ta, tid);
  else
    copy_mnmajor<TAIL>(A, M, m0, k0, K, ta, tid);
  if constexpr (Layout<LAYOUT>::B_KMAJOR)
    copy_kmajor<TAIL>(B, N, K, n0, k0, K, tb, tid);
  else
    copy_mnmajor<TAIL>(B, N, n0, k0, K, tb, tid);
}

// Per-lane byte offsets of a thread's copies within a full slice (k0 = 0),
// computed once per workgroup; a step adds the uniform base of its slice.
// k-major: row r0 + row (clamped), logical slot lslot: (r * ld + 8 lslot) * 2.
__device__ __forceinline__ void kmajor_offsets(int64_t R, int64_t ld, int64_t r0, int tid,
                                               uint32_t* off) {
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int u = pass * kGemmThreads + tid;
    const int row = u / kNSK, lslot = (u % kNSK) ^ kmaj_swz(row);
    const int64_t r = min(r0 + row, R - 1);
    off[pass] = (uint32_t)((r * ld + 8 * lslot) * 2);
  }
}
// mn-major: k-row row, column c0 + 8 lslot (clamped): (row * C + c) * 2.
__device__ __forceinline__ void mnmajor_offsets(int64_t C, int64_t c0, int tid, uint32_t* off) {
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int u = pass * kGemmThreads + tid;
    const int row = u >> 5, lslot = (u & 31) ^ mnmaj_swz(row);
    const int64_t c = min(c0 + 8 * lslot, C - 8);
    off[pass] = (uint32_t)((row * C + c) * 2);
  }
}

// A full slice from precomputed offsets: `base` is the slice's first element
// (uniform). The offsets are made opaque so that the compiler keeps one 32-bit
// register per copy instead of hoisting a 64-bit address per copy and slice.
__device__ __forceinline__ void copy_offsets(const bf16_t* base, const uint32_t* off, bf16_t* tile,
                                             int tid) {
  const int lds_off = __builtin_amdgcn_readfirstlane((tid >> 6) * 64 * 8);
  const char* b = reinterpret_cast<const char*>(base);
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    uint32_t o = off[pass];
    asm volatile("" : "+v"(o));
    async_copy16(b + o, tile + pass * kGemmThreads * 8 + lds_off);
  }
}

template <int LAYOUT>
__device__ __forceinline__ void issue_stage_fast(const bf16_t* A, const bf16_t* B, int64_t M,
                                                 int64_t N, int kt, const uint32_t* aoff,
                                                 const uint32_t* boff, bf16_t* ta, bf16_t* tb,
                                                 int tid) {
  const int64_t k0 = (int64_t)kt * kBK;
  copy_offsets(Layout<LAYOUT>::A_KMAJOR ? A + k0 : A + k0 * M, aoff, ta, tid);
  copy_offsets(Layout<LAYOUT>::B_KMAJOR ? B + k0 : B + k0 * N, boff, tb, tid);
}

template <int LAYOUT>
__device__ __forceinline__ void issue_stage(const bf16_t* A, const bf16_t* B, int64_t M, int64_t N,
                                            int64_t K, int64_t m0, int64_t n0, int kt,
                                            bf16_t* ta, bf16_t* tb, int tid) {
  const int64_t k0 = (int64_t)kt * kBK;
  if (k0 + kBK > K)
    copy_step<LAYOUT, true>(A, B, M, N, K, m0, n0, k0, ta, tb, tid);
  else
    copy_step<LAYOUT, false>(A, B, M, N, K, m0, n0, k0, ta, tb, tid);
}

// One K slice: wait for its copies (issued one slice earlier into `cur`),
// pass the barrier, then run the slice's products while the copies of the next
// full slice go out into `nxt`, spread one per fenced piece. The two stage
// buffers are distinct arrays so the compiler can tell the transposing LDS
// reads of `cur` from the copies landing in `nxt` (with one indexed array it
// must assume they alias and drains every copy before each such read).
template <int LAYOUT>
__device__ __forceinline__ void gemm_slice(f32x16 (&acc)[kMI][4], const bf16_t* A,
                                           const bf16_t* B, int64_t M, int64_t N, int64_t K,
                                           int64_t m0, int64_t n0, int kt, int kt_end,
                                           int n_full, const bf16_t* A2, const bf16_t* B2,
                                           int n_k1, const uint32_t* aoff,
                                           const uint32_t* boff, const bf16_t* ta,
                                           const bf16_t* tb, bf16_t* ta_next, bf16_t* tb_next,
                                           int tid, int lane, int wm, int wn) {
  wait_async();  // this thread's copies of slice kt (and any zero-filling writes)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();  // slice kt visible to all; every wave is done with kt - 1
  asm volatile("" ::: "memory");
  const int kn = kt + 1;
  // slices past n_k1 belong to the second product of a pair
  const bool second = kn >= n_k1;
  const bf16_t* An = second ? A2 : A;
  const bf16_t* Bn = second ? B2 : B;
  const int kl = second ? kn - n_k1 : kn;
  const bool fast_next = kn < min(n_full, kt_end);
  if (!fast_next && kn < kt_end) issue_stage<LAYOUT>(An, Bn, M, N, K, m0, n0, kl, ta_next, tb_next, tid);
  const int64_t kn0 = (int64_t)kl * kBK;
  const char* a_next = reinterpret_cast<const char*>(Layout<LAYOUT>::A_KMAJOR ? An + kn0 : An + kn0 * M);
  const char* b_next = reinterpret_cast<const char*>(Layout<LAYOUT>::B_KMAJOR ? Bn + kn0 : Bn + kn0 * N);
  const int lds_off = __builtin_amdgcn_readfirstlane((tid >> 6) * 64 * 8);
  // kKS 16-deep steps of 2 x 4 products, issued as fenced pieces of two
  // products. A piece also issues at most one copy of the next slice and
  // reads part of the next step's fragments (A_0 B_0, A_1 B_1, B_2, B_3 in
  // the step's four pieces), so the LDS and memory pipes stay busy between
  // the products instead of in bursts.
  static_assert(kMI == 2 && 2 * kPasses <= 4 * kKS, "piece layout: 2 x 4 products per step");
  bf16x8 a[2][kMI], b[2][4];
#pragma unroll
  for (int i = 0; i < kMI; ++i) a[0][i] = frag_a<LAYOUT>(ta, wm, i, 0, lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) b[0][j] = frag_b<LAYOUT>(tb, wn, j, 0, lane);
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    const int c = ks & 1, nx = c ^ 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int piece = ks * 4 + q;
      if (fast_next && piece < 2 * kPasses) {
        const bool is_a = piece < kPasses;
        const int pass = is_a ? piece : piece - kPasses;
        uint32_t o = is_a ? aoff[pass] : boff[pass];
        asm volatile("" : "+v"(o));
        async_copy16((is_a ? a_next : b_next) + o,
                     (is_a ? ta_next : tb_next) + pass * kGemmThreads * 8 + lds_off);
      }
      if (ks + 1 < kKS) {
        if (q < kMI) a[nx][q] = frag_a<LAYOUT>(ta, wm, q, ks + 1, lane);
        b[nx][q] = frag_b<LAYOUT>(tb, wn, q, ks + 1, lane);
      }
      const int i = q >> 1, j0 = 2 * (q & 1);
#pragma unroll
      for (int j = j0; j < j0 + 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c][i], b[c][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int LAYOUT, typename Tc>
__global__ void __launch_bounds__(kGemmThreads, 1)
gemm_bf16_kernel(int64_t M, int64_t N, int64_t K, const bf16_t* __restrict__ A,
                 const bf16_t* __restrict__ B, const bf16_t* __restrict__ A2,
                 const bf16_t* __restrict__ B2, Tc* __restrict__ Cm,
                 const float* __restrict__ bias, int accumulate, int full_tiles, int splits,
                 int slices_per_split) {
  // two stage buffers (A and B slices each), declared apart
  __shared__ __attribute__((aligned(16))) bf16_t lds_a0[kTileElems];
  __shared__ __attribute__((aligned(16))) bf16_t lds_b0[kTileElems];
  __shared__ __attribute__((aligned(16))) bf16_t lds_a1[kTileElems];
  __shared__ __attribute__((aligned(16))) bf16_t lds_b1[kTileElems];

  // Items 0 .. full_tiles - 1 are whole tiles (all of K); each later tile is
  // `splits` items, one per K split. Grid order: the whole tiles first, then
  // the split items; within each part every XCD (workgroups are dealt to the
  // XCDs round-robin) takes a contiguous run of items, tiles grouped
  // kGroupRows tile-rows, so each XCD gets its share of both parts.
  const int n_tm = (int)((M + kBM - 1) / kBM), n_tn = (int)((N + kBN - 1) / kBN);
  const int nb = n_tm * n_tn;
  const int total = full_tiles + (nb - full_tiles) * splits;
  int item = blockIdx.x;
  if (item < full_tiles) {
    if (full_tiles % kXcds == 0) item = (item % kXcds) * (full_tiles / kXcds) + item / kXcds;
  } else if ((total - full_tiles) % kXcds == 0 && full_tiles % kXcds == 0) {
    const int r = item - full_tiles, part = (total - full_tiles) / kXcds;
    item = full_tiles + (r % kXcds) * part + r / kXcds;
  }
  const bool split_tile = item >= full_tiles && splits > 1;
  const int split = item < full_tiles ? 0 : (item - full_tiles) % splits;
  const int bid = item < full_tiles ? item : full_tiles + (item - full_tiles) / splits;
  const int group = bid / (kGroupRows * n_tn);
  const int first = group * kGroupRows;
  const int rows_in_group = min(n_tm - first, kGroupRows);
  const int tm = first + (bid % (kGroupRows * n_tn)) % rows_in_group;
  const int tn = (bid % (kGroupRows * n_tn)) / rows_in_group;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[kMI][4];
#pragma unroll
  for (int i = 0; i < kMI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // With a second product (A2, B2; then K % kBK == 0) its slices follow the
  // first product's n_k1 slices in the same accumulators.
  const int n_k1 = (int)((K + kBK - 1) / kBK);
  const int n_k = A2 != nullptr ? 2 * n_k1 : n_k1;
  const int n_full = A2 != nullptr ? n_k : (int)(K / kBK);  // slices wholly inside K
  // this workgroup's K slices (all of them unless its tile is split)
  const int kt_begin = split_tile ? split * slices_per_split : 0;
  const int kt_end = split_tile ? min(n_k, kt_begin + slices_per_split) : n_k;
  uint32_t aoff[kPasses], boff[kPasses];
  if constexpr (Layout<LAYOUT>::A_KMAJOR)
    kmajor_offsets(M, K, m0, tid, aoff);
  else
    mnmajor_offsets(M, m0, tid, aoff);
  if constexpr (Layout<LAYOUT>::B_KMAJOR)
    kmajor_offsets(N, K, n0, tid, boff);
  else
    mnmajor_offsets(N, n0, tid, boff);
  // slice kt_begin + r lands in buffer r mod 2
  {
    const bool second = kt_begin >= n_k1;
    const bf16_t* Ab = second ? A2 : A;
    const bf16_t* Bb = second ? B2 : B;
    const int kl = second ? kt_begin - n_k1 : kt_begin;
    if (kt_begin < min(n_full, kt_end))
      issue_stage_fast<LAYOUT>(Ab, Bb, M, N, kl, aoff, boff, lds_a0, lds_b0, tid);
    else if (kt_begin < kt_end)
      issue_stage<LAYOUT>(Ab, Bb, M, N, K, m0, n0, kl, lds_a0, lds_b0, tid);
  }

  for (int kt = kt_begin; kt < kt_end; kt += 2) {
    gemm_slice<LAYOUT>(acc, A, B, M, N, K, m0, n0, kt, kt_end, n_full, A2, B2, n_k1, aoff, boff,
                       lds_a0, lds_b0, lds_a1, lds_b1, tid, lane, wm, wn);
    if (kt + 1 < kt_end)
      gemm_slice<LAYOUT>(acc, A, B, M, N, K, m0, n0, kt + 1, kt_end, n_full, A2, B2, n_k1, aoff,
                         boff, lds_a1, lds_b1, lds_a0, lds_b0, tid, lane, wm, wn);
  }

  // Epilogue: lane l of block (i, j) holds column 32 j + (l mod 32) of rows
  // 32 i + 8 (e / 4) + 4 (l / 32) + (e mod 4), e = 0 .. 15.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + wn * 128 + 32 * j + (lane & 31);
    if (n >= N) continue;
    const float bn = (bias != nullptr && split == 0) ? bias[n] : 0.f;
#pragma unroll
    for (int i = 0; i < kMI; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm * (kMI * 32) + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (m < M) {
          Tc* p = Cm + m * N + n;
          float x = acc[i][j][e] + bn;
          if constexpr (sizeof(Tc) == 4) {
            if (split_tile) {  // K split: the partial sums meet in C (zeroed first if needed)
              atomicAdd(reinterpret_cast<float*>(p), x);
              continue;
            }
          }
          if (accumulate) x += Elem<Tc>::load(p);
          Elem<Tc>::store(p, x);
        }
      }
    }
  }
}

__global__ void __launch_bounds__(256)
zero_f32_kernel(int64_t n4, float4* __restrict__ p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// K is split only for the tiles of a part-filled last round of the 256 CUs,
// into as many splits as fill that round (at least 8 slices each). Measured on
// the per-rank weight gradient 1024 x 5120 from K = 16384 (80 tiles, all in
// the last round): 3 splits 241 us, 2: 280 us, 13: 442 us, none: 483 us.
// Splitting every tile of a larger output cost more in atomic adds than the
// fuller round saved. With more than one round, the last round's tiles are
// split when that round is at most a quarter full (320 tiles, 5120 x 4096 from
// K = 8192: 389 -> 350 us, accumulating 462 -> 383 us), or half full when C is
// accumulated (640 tiles, 8192 x 5120 from K = 4096: 511 -> 480 us; without
// accumulation the zeroing pass made it 342 -> 390 us, so it stays whole).
constexpr int kCus = 256;
constexpr int kMinSlicesPerSplit = 8;

template <int LAYOUT>
hipError_t launch_gemm_l(int64_t M, int64_t N, int64_t K, const void* A, const void* B,
                         const void* A2, const void* B2, void* C, int c_dtype, const float* bias,
                         int accumulate, hipStream_t stream) {
  const int64_t nb = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  const int n_k = (int)((K + kBK - 1) / kBK) * (A2 != nullptr ? 2 : 1);
  // tiles of the full rounds keep all of K; the rest (fp32 output only) split it
  int64_t full = nb;
  int splits = 1;
  if (c_dtype == SPLITKV_FP32) {
    // a last round at most a quarter full (half full when C is accumulated
    // anyway): the split's zeroing pass and atomic adds cost less than the
    // idle part of that round
    const int64_t tail = nb % kCus;
    const bool split_tail = nb > kCus && (4 * tail <= kCus || (accumulate && 2 * tail <= kCus));
    if (tail != 0 && (nb < kCus / 2 || split_tail)) {
      full = nb - tail;
      splits = max(1, min((int)(kCus / tail), n_k / kMinSlicesPerSplit));
    }
  }
  const int sps = (n_k + splits - 1) / splits;
  splits = (n_k + sps - 1) / sps;
  if (splits == 1) full = nb;
  if (splits > 1 && !accumulate) {
    const int64_t n4 = M * N / 4;  // N % 8 == 0
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                       n4, static_cast<float4*>(C));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bf16_t* a = static_cast<const bf16_t*>(A);
  const bf16_t* b = static_cast<const bf16_t*>(B);
  const bf16_t* a2 = static_cast<const bf16_t*>(A2);
  const bf16_t* b2 = static_cast<const bf16_t*>(B2);
  const dim3 grid((unsigned)(full + (nb - full) * splits));
  if (c_dtype == SPLITKV_FP32)
    hipLaunchKernelGGL((gemm_bf16_kernel<LAYOUT, float>), grid, dim3(kGemmThreads), 0, stream, M,
                       N, K, a, b, a2, b2, static_cast<float*>(C), bias, accumulate, (int)full,
                       splits, sps);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<LAYOUT, bf16_t>), grid, dim3(kGemmThreads), 0, stream,
                       M, N, K, a, b, a2, b2, static_cast<bf16_t*>(C), bias, accumulate, (int)nb, 1,
                       n_k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int layout, int64_t M, int64_t N, int64_t K, const void* A, const void* B,
                       const void* A2, const void* B2, void* C, int c_dtype, const float* bias,
                       int accumulate, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  switch (layout) {
    case SPLITKV_GEMM_NT:
      return launch_gemm_l<SPLITKV_GEMM_NT>(M, N, K, A, B, A2, B2, C, c_dtype, bias, accumulate,
                                            stream);
    case SPLITKV_GEMM_NN:
      return launch_gemm_l<SPLITKV_GEMM_NN>(M, N, K, A, B, A2, B2, C, c_dtype, bias, accumulate,
                                            stream);
    default:
      return launch_gemm_l<SPLITKV_GEMM_TN>(M, N, K, A, B, A2, B2, C, c_dtype, bias, accumulate,
                                            stream);
  }
}

}  // namespace splitkv
