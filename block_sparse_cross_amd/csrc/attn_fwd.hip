// Local partial attention, Eq. 3 of "Split-KV: Efficient Context Parallelism
// for Training Diffusion Drafters" (§4.1): for every query row (block i) and
// head, softmax over the rank's local keys whose global position lies in the
// block's window [s_i, a_i); emits o_p and the natural-log LSE l_p.
//
// Work decomposition (bf16 path). A "query vector" is one (row, q-head) pair;
// vectors are numbered v = row * G + hh, where G = hq / hkv and hh indexes the
// q heads sharing kv head g, so consecutive vectors share a row (and so a
// block and a key range) and sit contiguously in q. A workgroup takes 128
// consecutive vectors of one kv head; each of its 4 waves owns 32 of them.
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

constexpr int kFwdThreads = 256;  // 4 waves
constexpr int kVecPerWave = 32;
constexpr int kVecPerWG = 128;
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
__global__ void __launch_bounds__(kFwdThreads, 2)
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
  __shared__ int wave_lo[4], wave_hi[4];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  // kv head fastest across workgroup ids: consecutive ids land on different
  // XCDs, so each XCD keeps serving the same kv head's keys from its L2.
  const int g = blockIdx.x % hkv;
  const int64_t vgroup = blockIdx.x / hkv;
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
  const int wlo = wave_min_i(live_lane ? qlo : 0x7fffffff);
  const int whi = wave_max_i(live_lane ? qhi : -1);
  const int wall_lo = wave_max_i(live_lane ? qlo : 0x7fffffff);
  const int wall_hi = wave_min_i(live_lane ? qhi : -1);
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
  for (int w = 0; w < 4; ++w) { lo = min(lo, wave_lo[w]); hi = max(hi, wave_hi[w]); }
  // the same in every lane: keep the tile loop and its addressing scalar
  lo = __builtin_amdgcn_readfirstlane(lo);
  hi = __builtin_amdgcn_readfirstlane(hi);

  // K and V tiles: rows k0 .. k0 + 63 of kv head g (row stride hkv * D); the
  // last tile of the buffer may run past it and takes the clamped copy.
  auto issue_tile = [&](int k0, bf16_t* Kn, bf16_t* Vn) {
    if (k0 + kKT <= n_keys) {
      const int64_t first = ((int64_t)k0 * hkv + g) * D;
      issue_tile_async<D, kKT, kFwdThreads, kSwzRows, false>(k + first, (int64_t)hkv * D, Kn, tid);
      issue_tile_async<D, kKT, kFwdThreads, kSwzTr, false>(v + first, (int64_t)hkv * D, Vn, tid);
    } else {
      issue_rows_async<D, kKT, kFwdThreads, kSwzRows>(k, hkv, g, k0, n_keys, Kn, tid);
      issue_rows_async<D, kKT, kFwdThreads, kSwzTr>(v, hkv, g, k0, n_keys, Vn, tid);
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // One tile: wait for its copy, start the copy of the next tile into the
  // other buffer pair, compute. The buffer pairs are distinct LDS arrays and
  // the loop below is unrolled by two, so the compiler can tell the copy's LDS
  // writes from this tile's reads and does not wait for the copy to land.
  auto tile_step = [&](int k0, const bf16_t* Kt, const bf16_t* Vt, bf16_t* Kn, bf16_t* Vn) {
    wait_async();
    __syncthreads();
    if (k0 + kKT < hi) issue_tile(k0 + kKT, Kn, Vn);
    if (!(k0 < whi && k0 + kKT > wlo)) return;  // nothing live for this wave

    // ---- S^T = K Q^T for two 32-key halves ----
    f32x16 sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[mt][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {  // two independent accumulation chains
        const int krow = mt * 32 + (lane & 31);
        const int slot = (2 * ks + half) ^ swz_rows<NS>(krow);
        const u32x4 a = *reinterpret_cast<const u32x4*>(&Kt[krow * D + slot * 8]);
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qf[ks], sacc[mt], 0, 0, 0);
      }
    // ---- mask (boundary tiles only), running max ----
    const bool need_mask = k0 < wall_lo || k0 + kKT > wall_hi;
    float mloc = -INFINITY;
    if (need_mask) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const float x = (key >= qlo && key < qhi) ? sacc[mt][r] : -INFINITY;
          sacc[mt][r] = x;
          mloc = fmaxf(mloc, x);
        }
    } else {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[mt][r]);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32)) * scale_log2;
    // ---- lazy rescale: raise the running max only when exceeded by > 8 ----
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
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sacc[mt][r], scale_log2, neg_m));
        sacc[mt][r] = p;
        psum += p;
      }
    l_run += psum;

    // ---- O^T += V^T P^T, four 16-key steps ----
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        u32x4 pu;
        pu.x = pack_bf16x2_hw(sacc[mt][8 * h2 + 0], sacc[mt][8 * h2 + 1]);
        pu.y = pack_bf16x2_hw(sacc[mt][8 * h2 + 2], sacc[mt][8 * h2 + 3]);
        pu.z = pack_bf16x2_hw(sacc[mt][8 * h2 + 4], sacc[mt][8 * h2 + 5]);
        pu.w = pack_bf16x2_hw(sacc[mt][8 * h2 + 6], sacc[mt][8 * h2 + 7]);
        const bf16x8 pb = as_bf16x8(pu);
        // keys of this step held by the lane: base + 4 half + {0..3}, +8
        const int s16 = lane & 15;
        const int vrow = mt * 32 + 16 * h2 + 4 * half + (s16 >> 2);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int dcol = dt * 32 + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
          const int slot = dcol >> 3, off = dcol & 7;
          const u32x2 x0 = read_tr4(&Vt[vrow * D + ((slot ^ swz_tr<NS>(vrow)) * 8) + off]);
          const u32x2 x1 = read_tr4(&Vt[(vrow + 8) * D + ((slot ^ swz_tr<NS>(vrow + 8)) * 8) + off]);
          const u32x4 au = {x0.x, x0.y, x1.x, x1.y};
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(au), pb, oacc[dt], 0, 0, 0);
        }
      }
  };

  if (lo < hi) issue_tile(lo, K0, V0);
  for (int k0 = lo; k0 < hi; k0 += 2 * kKT) {
    tile_step(k0, K0, V0, K1, V1);
    if (k0 + kKT < hi) tile_step(k0 + kKT, K1, V1, K0, V0);
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
