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
// 64-key tiles of the union of its vectors' intervals, and masks per lane.
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16, gfx950). Scores are computed
// transposed, S^T = K Q^T, so that a lane's 16 accumulator values all belong
// to its own query vector (lane % 32); softmax statistics are per lane, with
// one exchange between the two half-waves holding the two key halves. The
// output is also accumulated transposed, O^T = V^T P^T, so the P tile feeds
// the second product straight from registers and rescaling is per lane. V is
// staged transposed in LDS ([d][key]) so that both products read 16-byte (or
// 2x8-byte) fragments. Softmax runs in fp32 in the log2 domain (scale * log2 e
// folded into one multiply of the fp32 scores); LSE is returned in natural log.
#include "common.hpp"
#include "internal.hpp"

namespace splitkv {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kFwdThreads = 256;  // 4 waves
constexpr int kVecPerWave = 32;
constexpr int kVecPerWG = 128;
constexpr int kKT = 64;           // keys per tile

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  __bf16 a = static_cast<__bf16>(lo), b = static_cast<__bf16>(hi);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
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
    u.x = pack2(a, b);
    u.y = pack2(c, d);
    *reinterpret_cast<u32x2*>(p) = u;
  }
};

template <int D, typename Tout>
__global__ void __launch_bounds__(kFwdThreads)
attn_fwd_bf16_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                     const bf16_t* __restrict__ v, Tout* __restrict__ o, float* __restrict__ lse,
                     const int2* __restrict__ block_range, int64_t n_vec, int G, int hq, int hkv,
                     int B, int n_keys, float scale_log2) {
  constexpr int KS = D + 8;    // K tile row stride (elements): conflict-free 16-byte reads
  constexpr int VS = kKT + 4;  // V^T tile row stride: conflict-free 8-byte reads
  __shared__ __attribute__((aligned(16))) bf16_t Ks[kKT * KS];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[D * VS];
  __shared__ int wave_lo[4], wave_hi[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int g = blockIdx.y;
  const int64_t vec = (int64_t)blockIdx.x * kVecPerWG + wave * kVecPerWave + (lane & 31);
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
  const int64_t head_off = (row * hq + (int64_t)g * G + hh) * D;

  // Key range of this wave and of the workgroup (union of non-empty ranges).
  int wlo = wave_min_i(qlo < qhi ? qlo : 0x7fffffff);
  int whi = wave_max_i(qlo < qhi ? qhi : -1);
  if (lane == 0) { wave_lo[wave] = wlo; wave_hi[wave] = whi; }

  // Query fragment (B operand of S^T = K Q^T): lane holds d-slices
  // [16 ks + 8 half, +8) of its own vector.
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

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int k0 = lo; k0 < hi; k0 += kKT) {
    // ---- stage K (row-major) and V (transposed) tiles in LDS ----
#pragma unroll
    for (int c = tid; c < kKT * (D / 8); c += kFwdThreads) {
      const int key = c / (D / 8), col = (c % (D / 8)) * 8;
      const int kg = k0 + key;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (kg < n_keys) val = *reinterpret_cast<const u32x4*>(k + ((int64_t)kg * hkv + g) * D + col);
      *reinterpret_cast<u32x4*>(&Ks[key * KS + col]) = val;
    }
#pragma unroll
    for (int c = tid; c < (kKT / 4) * (D / 8); c += kFwdThreads) {
      const int col = (c % (D / 8)) * 8, kq = (c / (D / 8)) * 4;
      u32x4 r[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kg = k0 + kq + u;
        r[u] = u32x4{0u, 0u, 0u, 0u};
        if (kg < n_keys) r[u] = *reinterpret_cast<const u32x4*>(v + ((int64_t)kg * hkv + g) * D + col);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1, sh = (e & 1) * 16;
        u32x2 t;
        t.x = ((r[0][w] >> sh) & 0xffffu) | (((r[1][w] >> sh) & 0xffffu) << 16);
        t.y = ((r[2][w] >> sh) & 0xffffu) | (((r[3][w] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<u32x2*>(&Vt[(col + e) * VS + kq]) = t;
      }
    }
    __syncthreads();

    if (k0 < whi && k0 + kKT > wlo) {
      // ---- S^T = K Q^T for two 32-key halves ----
      f32x16 sacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[mt][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(&Ks[(mt * 32 + (lane & 31)) * KS + ks * 16 + half * 8]);
          sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qf[ks], sacc[mt], 0, 0, 0);
        }
      }
      // ---- mask, online softmax (log2 domain) ----
      float mloc = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          float x = sacc[mt][r] * scale_log2;
          x = (key >= qlo && key < qhi) ? x : -INFINITY;
          sacc[mt][r] = x;
          mloc = fmaxf(mloc, x);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(sacc[mt][r] - m_use);
          sacc[mt][r] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;

      // ---- O^T += V^T P^T, four 16-key steps ----
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          u32x4 pu;
          pu.x = pack2(sacc[mt][8 * h2 + 0], sacc[mt][8 * h2 + 1]);
          pu.y = pack2(sacc[mt][8 * h2 + 2], sacc[mt][8 * h2 + 3]);
          pu.z = pack2(sacc[mt][8 * h2 + 4], sacc[mt][8 * h2 + 5]);
          pu.w = pack2(sacc[mt][8 * h2 + 6], sacc[mt][8 * h2 + 7]);
          const bf16x8 pb = as_bf16x8(pu);
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const bf16_t* vr = &Vt[(dt * 32 + (lane & 31)) * VS + mt * 32 + 16 * h2 + 4 * half];
            const u32x2 x0 = *reinterpret_cast<const u32x2*>(vr);
            const u32x2 x1 = *reinterpret_cast<const u32x2*>(vr + 8);
            const u32x4 au = {x0.x, x0.y, x1.x, x1.y};
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(au), pb, oacc[dt], 0, 0, 0);
          }
        }
    }
    __syncthreads();
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
    const dim3 grid((unsigned)((n_vec + kVecPerWG - 1) / kVecPerWG), (unsigned)hd.hkv);
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, Tout>), grid, dim3(kFwdThreads), 0, stream,
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                       static_cast<const bf16_t*>(v), static_cast<Tout*>(o), lse, block_range,
                       n_vec, G, hd.hq, hd.hkv, an.block_size, (int)n_keys,
                       hd.scale * kLog2e);
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
