// Local partial attention, Eq. 3 of "Split-KV: Efficient Context Parallelism
// for Training Diffusion Drafters" (§4.1): for every query row (block i) and
// head, softmax over the rank's local keys whose global position lies in the
// block's window [s_i, a_i); emits o_p and the natural-log LSE l_p.
//
// Work decomposition (bf16 path). A "query vector" is one (row, q-head) pair;
// vectors are numbered v = row * G + hh, where G = hq / hkv and hh indexes the
// q heads sharing kv head g, so consecutive vectors share a row (and so a
// block and a key range) and sit contiguously in q. A workgroup takes 256
// consecutive vectors of one kv head; each of its 8 waves (two per SIMD) owns
// 32 of them, and each K and V tile copied into LDS serves all 256 (half the
// copies per product of a 128-vector workgroup: 1.5% faster at the
// strong-scaling share).
// Because the local buffer is sorted by global position, every block reaches
// one contiguous local key interval [lo, hi); the workgroup walks only the
// 64-key tiles of the union of its vectors' intervals.
//
// Pipeline. K and V tiles are copied global -> LDS with asynchronous 16-byte
// direct loads (no VGPR staging), double-buffered: the copy of tile t+1 is in
// flight while tile t is computed, with one barrier per tile. Both tiles stay
// row-major in LDS with XOR-swizzled 16-byte slots.
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16). Scores are computed
// transposed, S^T = K Q^T, so a lane's 16 accumulator values all belong to its
// own query vector (lane % 32) and softmax statistics are per lane, with one
// exchange between the two half-waves holding the two key halves. The output
// is accumulated transposed, O^T = V^T P^T: P feeds the product straight from
// registers, and the V^T fragments come from the row-major V tile through the
// transposing LDS read (ds_read_b64_tr_b16).
//
// Softmax: fp32, log2 domain (scale * log2 e folded into one FMA with the
// running max); the per-key mask is applied only on tiles that cut some
// vector's interval; the running max is raised (and O, l rescaled) only when a
// new score exceeds it by more than 8 (so unnormalised weights stay <= 2^8).
// LSE is returned in natural log.
#include "common.hpp"
#include "internal.hpp"

namespace splitkv {

namespace {

constexpr int kFwdThreads = 512;  // 8 waves, two per SIMD
constexpr int kVecPerWave = 32;
constexpr int kVecPerWG = 256;
constexpr int kKT = 64;           // keys per tile
constexpr float kRescaleSlack = 8.f;

// Per block: local key interval [lo, hi) = [#local keys before s_i, #local
// keys before a_i). Empty windows give lo == hi.
__global__ void block_range_kernel(const int64_t* __restrict__ s, const int64_t* __restrict__ a,
                                   int64_t n_blocks, const int64_t* __restrict__ chunk_start,
                                   int32_t n_chunks, int64_t m, int2* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_blocks) return;
  const int64_t si = s[i], ai = a[i];
  int64_t lo = 0, hi = 0;
  for (int j = 0; j < n_chunks; ++j) {
    const int64_t lam = chunk_start[j];
    lo += min(max(si - lam, (int64_t)0), m);
    hi += min(max(ai - lam, (int64_t)0), m);
  }
  if (hi < lo) hi = lo;
  out[i] = make_int2((int)lo, (int)hi);
}

template <typename Tout> struct Store4;
template <> struct Store4<float> {
  __device__ __forceinline__ static void run(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
};
template <> struct Store4<bf16_t> {
  __device__ __forceinline__ static void run(bf16_t* p, float a, float b, float c, float d) {
    u32x2 u;
    u.x = pack_bf16x2_hw(a, b);
    u.y = pack_bf16x2_hw(c, d);
    *reinterpret_cast<u32x2*>(p) = u;
  }
};

template <int D, typename Tout>
__global__ void __launch_bounds__(kFwdThreads, 1)
attn_fwd_bf16_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                     const bf16_t* __restrict__ v, Tout* __restrict__ o, float* __restrict__ lse,
                     const int2* __restrict__ block_range, int64_t n_vec, int G, int hq, int hkv,
                     int B, int n_keys, float scale_log2) {
  constexpr int NS = D / 8;
  // two buffer pairs, as distinct arrays (see tile_step)
  __shared__ __attribute__((aligned(16))) bf16_t K0[kKT * D];
  __shared__ __attribute__((aligned(16))) bf16_t V0[kKT * D];
  __shared__ __attribute__((aligned(16))) bf16_t K1[kKT * D];
  __shared__ __attribute__((aligned(16))) bf16_t V1[kKT * D];
  __shared__ int wave_lo[kFwdThreads / 64], wave_hi[kFwdThreads / 64];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  // kv head fastest across workgroup ids: consecutive ids land on different
  // XCDs, so each XCD keeps serving the same kv head's keys from its L2.
  const int g = blockIdx.x % hkv;
  // Vector groups in reverse: blocks are ordered by ascending anchor within a
  // sample, so late groups have the longest windows; starting them first
  // shortens the tail of the launch.
  const int64_t vgroup = (gridDim.x / hkv) - 1 - blockIdx.x / hkv;
  const int64_t vec = vgroup * kVecPerWG + wave * kVecPerWave + (lane & 31);
  const bool valid = vec < n_vec;
  int64_t row = 0;
  int hh = 0, qlo = 0, qhi = 0;
  if (valid) {
    row = vec / G;
    hh = (int)(vec % G);
    const int2 r = block_range[row / B];
    qlo = r.x;
    qhi = r.y;
  }
  const bool live_lane = valid && qlo < qhi;
  const int64_t head_off = (row * hq + (int64_t)g * G + hh) * D;

  // Key interval union of this wave / workgroup, and the interval every lane
  // of the wave covers (tiles inside it need no per-key mask).
  // (the same in every lane after the reductions; readfirstlane makes that
  // visible to the compiler, so tests on them are scalar branches)
  const int wlo = __builtin_amdgcn_readfirstlane(wave_min_i(live_lane ? qlo : 0x7fffffff));
  const int whi = __builtin_amdgcn_readfirstlane(wave_max_i(live_lane ? qhi : -1));
  const int wall_lo = __builtin_amdgcn_readfirstlane(wave_max_i(live_lane ? qlo : 0x7fffffff));
  const int wall_hi = __builtin_amdgcn_readfirstlane(wave_min_i(live_lane ? qhi : -1));
  if (lane == 0) { wave_lo[wave] = wlo; wave_hi[wave] = whi; }

  // Query fragment (B operand of S^T = K Q^T): d-slices [16 ks + 8 half, +8).
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 u = {0u, 0u, 0u, 0u};
    if (valid) u = *reinterpret_cast<const u32x4*>(q + head_off + ks * 16 + half * 8);
    qf[ks] = as_bf16x8(u);
  }
  __syncthreads();
  int lo = 0x7fffffff, hi = -1;
#pragma unroll
  for (int w = 0; w < kFwdThreads / 64; ++w) { lo = min(lo, wave_lo[w]); hi = max(hi, wave_hi[w]); }
  // the same in every lane: keep the tile loop and its addressing scalar
  lo = __builtin_amdgcn_readfirstlane(lo);
  hi = __builtin_amdgcn_readfirstlane(hi);

  // K or V tile: rows k0 .. k0 + 63 of kv head g (row stride hkv * D); the
  // last tile of the buffer may run past it and takes the clamped copy.
  const uint32_t k_off = tile_lane_offset<D, kFwdThreads, kSwzRows>((int64_t)hkv * D, tid);
  const uint32_t v_off = tile_lane_offset<D, kFwdThreads, kSwzTr>((int64_t)hkv * D, tid);
  auto issue_k = [&](int k0, bf16_t* dst) {
    if (k0 + kKT <= n_keys)
      issue_tile_async_off<D, kKT, kFwdThreads>(k + ((int64_t)k0 * hkv + g) * D, (int64_t)hkv * D,
                                                k_off, dst, tid);
    else
      issue_rows_async<D, kKT, kFwdThreads, kSwzRows>(k, hkv, g, k0, n_keys, dst, tid);
  };
  auto issue_v = [&](int k0, bf16_t* dst) {
    if (k0 + kKT <= n_keys)
      issue_tile_async_off<D, kKT, kFwdThreads>(v + ((int64_t)k0 * hkv + g) * D, (int64_t)hkv * D,
                                                v_off, dst, tid);
    else
      issue_rows_async<D, kKT, kFwdThreads, kSwzTr>(v, hkv, g, k0, n_keys, dst, tid);
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Software pipeline over the key tiles t = 0 .. n_tiles - 1 (keys lo + 64 t
  // ..): iteration t computes the scores of tile t + 1 while it exponentiates
  // tile t, then multiplies P(t) V(t) while it takes the row maximum of tile
  // t + 1. K(j) and V(j) live in slot j % 2 of their double buffers; the copy
  // of K(t + 2) and V(t + 1) is issued at the top of iteration t, after the
  // barrier that ends every use of K(t) and V(t - 1).
  //
  // The pieces of a phase are fenced (__builtin_amdgcn_sched_barrier(0)) so
  // that each keeps its two products next to its share of the vector work,
  // and each issues the LDS reads of the next piece.
  constexpr int NP = D / 16;    // pieces per phase
  constexpr int DT = D / 32;    // 32-column blocks of O
  constexpr int EPP = 32 / NP;  // of a lane's 32 scores, handled per piece
  const int n_tiles = lo < hi ? (hi - lo + kKT - 1) / kKT : 0;

  f32x16 sa[2], sb[2];  // scores (then weights) of tiles t and t + 1, alternating
  u32x4 ka[2][2];       // K operands (mt) for a piece, double-buffered by piece
  u32x4 va[2][2];       // V^T operands (two products) for a piece
  u32x4 pu[2][2];       // P of tile t as bf16, per (mt, 16-key step h2)
  float mloc = -INFINITY;

  auto load_k = [&](const bf16_t* Kt, int ks, int b) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int krow = mt * 32 + (lane & 31);
      const int slot = (2 * ks + half) ^ swz_rows<NS>(krow);
      ka[b][mt] = *reinterpret_cast<const u32x4*>(&Kt[krow * D + slot * 8]);
    }
  };
  // products 2 j, 2 j + 1 of P V: (mt, h2) = (2 j) / DT split, dt = (2 j) % DT + {0, 1}
  auto load_v = [&](const bf16_t* Vt, int j, int b) {
    const int u0 = 2 * j, mh = u0 / DT, mt = mh >> 1, h2 = mh & 1;
    const int s16 = lane & 15;
    const int vrow = mt * 32 + 16 * h2 + 4 * half + (s16 >> 2);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int dt = u0 % DT + e;
      const int dcol = dt * 32 + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
      const int slot = dcol >> 3, off = dcol & 7;
      const u32x2 x0 = read_tr4(&Vt[vrow * D + ((slot ^ swz_tr<NS>(vrow)) * 8) + off]);
      const u32x2 x1 = read_tr4(&Vt[(vrow + 8) * D + ((slot ^ swz_tr<NS>(vrow + 8)) * 8) + off]);
      va[b][e] = u32x4{x0.x, x0.y, x1.x, x1.y};
    }
  };
  auto zero2 = [](f32x16 (&x)[2]) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[mt][r] = 0.f;
  };
  // keys outside a lane's interval -> -inf (tiles that cut some interval)
  auto mask_scores = [&](int k0, f32x16 (&x)[2]) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        x[mt][r] = (key >= qlo && key < qhi) ? x[mt][r] : -INFINITY;
      }
  };
  auto tile_k0 = [&](int t) { return lo + t * kKT; };
  auto needs_mask = [&](int t) { return tile_k0(t) < wall_lo || tile_k0(t) + kKT > wall_hi; };

  // one pipeline iteration; Kn = K(t + 1), Vc = V(t), Kf / Vf = free slots
  auto iteration = [&](int t, const bf16_t* Kn, const bf16_t* Vc, bf16_t* Kf, bf16_t* Vf,
                       f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    wait_async();
    __syncthreads();
    if (t + 2 < n_tiles) issue_k(tile_k0(t + 2), Kf);
    if (t + 1 < n_tiles) issue_v(tile_k0(t + 1), Vf);

    // lazy rescale: raise the running max only when tile t exceeds it by > 8
    if (__any(mloc > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
    const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;

    // phase B: S(t + 1) = K(t + 1) Q^T with P(t) = exp2(S(t) c - m)
    // (scores past the last tile are computed from a stale slot and unused)
    zero2(sn);
    float psum = 0.f;
    load_k(Kn, 0, 0);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (i + 1 < NP) load_k(Kn, i + 1, (i + 1) & 1);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        sn[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[i & 1][mt]), qf[i], sn[mt], 0, 0, 0);
#pragma unroll
      for (int e = 0; e < EPP; ++e) {
        const int x = EPP * i + e, mt = x >> 4, r = x & 15;
        const float pv = fast_exp2(fmaf(sc[mt][r], scale_log2, neg_m));
        sc[mt][r] = pv;
        psum += pv;
        asm volatile("" : "+v"(psum));  // keep the sum in this piece
        if ((r & 7) == 7) {
          const int h2 = r >> 3;
          pu[mt][h2].x = pack_bf16x2_hw(sc[mt][8 * h2 + 0], sc[mt][8 * h2 + 1]);
          pu[mt][h2].y = pack_bf16x2_hw(sc[mt][8 * h2 + 2], sc[mt][8 * h2 + 3]);
          pu[mt][h2].z = pack_bf16x2_hw(sc[mt][8 * h2 + 4], sc[mt][8 * h2 + 5]);
          pu[mt][h2].w = pack_bf16x2_hw(sc[mt][8 * h2 + 6], sc[mt][8 * h2 + 7]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += psum;

    // phase C: O^T += V(t)^T P(t) with the row maximum of S(t + 1). No
    // branch may separate the phases (the compiler would sink phase B's
    // vector work past it), so boundary tiles are masked afterwards and
    // their maximum taken again.
    float mx = -INFINITY;
    load_v(Vc, 0, 0);
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (j + 1 < NP) load_v(Vc, j + 1, (j + 1) & 1);
      const int u0 = 2 * j, mh = u0 / DT, mt = mh >> 1, h2 = mh & 1;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int dt = u0 % DT + e;
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[j & 1][e]), as_bf16x8(pu[mt][h2]),
                                                           oacc[dt], 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < EPP; ++e) {
        const int x = EPP * j + e;
        mx = fmaxf(mx, sn[x >> 4][x & 15]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (t + 1 < n_tiles && needs_mask(t + 1)) {
      mask_scores(tile_k0(t + 1), sn);
      mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sn[mt][r]);
    }
    mloc = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
  };

  if (n_tiles > 0) {
    issue_k(tile_k0(0), K0);
    issue_v(tile_k0(0), V0);
    if (n_tiles > 1) issue_k(tile_k0(1), K1);
    wait_async();
    __syncthreads();
    // scores and row maximum of tile 0
    zero2(sa);
#pragma unroll
    for (int ks = 0; ks < NP; ++ks) {
      load_k(K0, ks, 0);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        sa[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[0][mt]), qf[ks], sa[mt], 0, 0, 0);
    }
    if (needs_mask(0)) mask_scores(tile_k0(0), sa);
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sa[mt][r]);
    mloc = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
  }
  for (int t = 0; t < n_tiles; t += 2) {
    iteration(t, K1, V0, K0, V1, sa, sb);
    if (t + 1 < n_tiles) iteration(t + 1, K0, V1, K1, V0, sb, sa);
  }

  // ---- epilogue: normalise, store o_p and lse_p ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (valid) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    Tout* op = o + head_off;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = dt * 32 + 8 * jj + 4 * half;
        Store4<Tout>::run(op + d0, oacc[dt][4 * jj] * inv, oacc[dt][4 * jj + 1] * inv,
                          oacc[dt][4 * jj + 2] * inv, oacc[dt][4 * jj + 3] * inv);
      }
    if (half == 0)
      lse[row * hq + (int64_t)g * G + hh] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// fp32 path: one thread per (row, head), a plain online softmax over the
// row's local interval. Used for fp32 inputs (small correctness workloads).
template <int D, typename Tout>
__global__ void __launch_bounds__(128)
attn_fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                    const float* __restrict__ v, Tout* __restrict__ o, float* __restrict__ lse,
                    const int2* __restrict__ block_range, int64_t n_rows, int hq, int hkv, int B,
                    float scale) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_rows * hq) return;
  const int64_t row = t / hq;
  const int h = (int)(t % hq), g = h / (hq / hkv);
  const int2 r = block_range[row / B];
  const float* qv = q + t * D;
  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;
  float mx = -INFINITY, sum = 0.f;
  for (int x = r.x; x < r.y; ++x) {
    const float* kv = k + ((int64_t)x * hkv + g) * D;
    const float* vv = v + ((int64_t)x * hkv + g) * D;
    float z = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) z = fmaf(qv[c], kv[c], z);
    z *= scale;
    const float m_new = fmaxf(mx, z);
    const float alpha = __expf(mx - m_new), p = __expf(z - m_new);
    sum = sum * alpha + p;
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] = fmaf(p, vv[c], acc[c] * alpha);
    mx = m_new;
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
  for (int c = 0; c < D; ++c) Elem<Tout>::store(o + t * D + c, acc[c] * inv);
  lse[t] = sum > 0.f ? mx + __logf(sum) : -INFINITY;
}

template <int D, typename Tout>
hipError_t launch_fwd_t(const splitkv_anchors& an, const splitkv_heads& hd, int64_t n_keys,
                        const int2* block_range, const void* q, const void* k, const void* v,
                        void* o, float* lse, hipStream_t stream) {
  const int64_t Q = an.n_blocks * an.block_size;
  if (hd.dtype == SPLITKV_BF16) {
    const int G = hd.hq / hd.hkv;
    const int64_t n_vec = Q * G;
    const int64_t n_groups = (n_vec + kVecPerWG - 1) / kVecPerWG;
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, Tout>), dim3((unsigned)(n_groups * hd.hkv)),
                       dim3(kFwdThreads), 0, stream, static_cast<const bf16_t*>(q),
                       static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),
                       static_cast<Tout*>(o), lse, block_range, n_vec, G, hd.hq, hd.hkv,
                       an.block_size, (int)n_keys, hd.scale * kLog2e);
  } else {
    const int64_t n = Q * hd.hq;
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, Tout>), dim3((unsigned)((n + 127) / 128)),
                       dim3(128), 0, stream, static_cast<const float*>(q),
                       static_cast<const float*>(k), static_cast<const float*>(v),
                       static_cast<Tout*>(o), lse, block_range, Q, hd.hq, hd.hkv, an.block_size,
                       hd.scale);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_ranges(const int64_t* s, const int64_t* a, int64_t n_blocks,
                               const int64_t* chunk_start, int32_t n_chunks, int64_t m,
                               int2* block_range, hipStream_t stream) {
  if (n_blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(block_range_kernel, dim3((unsigned)((n_blocks + 255) / 256)), dim3(256), 0,
                     stream, s, a, n_blocks, chunk_start, n_chunks, m, block_range);
  return hipGetLastError();
}

hipError_t launch_fwd(const splitkv_anchors& an, const splitkv_heads& hd, int64_t n_keys,
                      const int2* block_range, const void* q, const void* k, const void* v,
                      void* o, int o_dtype, float* lse, hipStream_t stream) {
  if (an.n_blocks == 0) return hipSuccess;
  const bool f32o = o_dtype == SPLITKV_FP32;
  if (hd.d == 128)
    return f32o ? launch_fwd_t<128, float>(an, hd, n_keys, block_range, q, k, v, o, lse, stream)
                : launch_fwd_t<128, bf16_t>(an, hd, n_keys, block_range, q, k, v, o, lse, stream);
  return f32o ? launch_fwd_t<64, float>(an, hd, n_keys, block_range, q, k, v, o, lse, stream)
              : launch_fwd_t<64, bf16_t>(an, hd, n_keys, block_range, q, k, v, o, lse, stream);
}

}  // namespace splitkv
