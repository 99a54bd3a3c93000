// Backward of the local partial (Algorithm 1 of "Split-KV: Efficient Context
// Parallelism for Training Diffusion Drafters", §4.1: MERGE_BWD, then
// AttnBwd_p). With the merged (global) lse and Delta = <do, o>, every live pair
// (query vector r, key x) contributes
//   P = exp(scale <q_r, k_x> - lse_r),  dv_x += P do_r,
//   ds = P (<do_r, v_x> - Delta_r),     dq_r += scale ds k_x,  dk_x += scale ds q_r.
// dk and dv stay local to the rank; dq is accumulated (+=) so that the P
// emulated ranks of one device sum into one buffer.
//
// bf16 path: a workgroup owns 128 local keys of one kv head (32 per wave) and
// walks the 32-vector query chunks whose key intervals reach those keys. Per
// chunk each wave forms S = Q K^T and dP = dO V^T with v_mfma_f32_32x32x16_bf16
// so that a lane owns one key and 16 query vectors, then accumulates
// dV^T += dO^T P and dK^T += Q^T dS in registers (Q^T, dO^T staged transposed
// in LDS). dS goes through LDS so that dQ = dS K (K^T staged once in LDS) is
// formed per 32-wide d slice and added to dq with fp32 atomics.
#include "common.hpp"
#include "internal.hpp"

namespace splitkv {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBwdThreads = 256;  // 4 waves
constexpr int kBwdKeys = 128;     // keys per workgroup, 32 per wave
constexpr int kQC = 32;           // query vectors per chunk

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  __bf16 a = static_cast<__bf16>(lo), b = static_cast<__bf16>(hi);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}
__device__ __forceinline__ bf16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Delta[r, h] = <do[r, h], o[r, h]>, one thread per (row, head).
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

// Key interval of each 32-vector query chunk: union of its rows' block ranges.
__global__ void chunk_range_kernel(const int2* __restrict__ block_range, int64_t n_vec, int G,
                                   int B, int64_t n_qc, int2* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= n_qc) return;
  const int64_t v0 = c * kQC, v1 = min(v0 + kQC, n_vec);
  int lo = 0x7fffffff, hi = -1;
  for (int64_t row = v0 / G; row <= (v1 - 1) / G; ++row) {
    const int2 r = block_range[row / B];
    if (r.x < r.y) { lo = min(lo, r.x); hi = max(hi, r.y); }
  }
  out[c] = hi < 0 ? make_int2(0, 0) : make_int2(lo, hi);
}

template <int D>
__global__ void __launch_bounds__(kBwdThreads)
attn_bwd_bf16_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                     const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
                     const float* __restrict__ lse, const float* __restrict__ delta,
                     float* __restrict__ dq, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv,
                     const int2* __restrict__ block_range, const int2* __restrict__ chunk_range,
                     int64_t n_vec, int64_t n_qc, int G, int hq, int hkv, int B, int n_keys,
                     float scale, float scale_log2) {
  constexpr int QS = D + 8;          // [vec][d] tiles
  constexpr int TS = kQC + 4;        // [d][vec] tiles
  constexpr int SS = kBwdKeys + 8;   // dS [vec][key]
  constexpr int KTS = kBwdKeys + 8;  // K^T [d][key]
  __shared__ __attribute__((aligned(16))) bf16_t Qs[kQC * QS];
  __shared__ __attribute__((aligned(16))) bf16_t dOs[kQC * QS];
  __shared__ __attribute__((aligned(16))) bf16_t Qt[D * TS];
  __shared__ __attribute__((aligned(16))) bf16_t dOt[D * TS];
  __shared__ __attribute__((aligned(16))) bf16_t dSs[kQC * SS];
  __shared__ __attribute__((aligned(16))) bf16_t Kt[D * KTS];
  __shared__ float lse_s[kQC], dlt_s[kQC];
  __shared__ int lo_s[kQC], hi_s[kQC];
  __shared__ long long dq_off[kQC];
  __shared__ int list[kBwdThreads];
  __shared__ int wave_cnt[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int g = blockIdx.y;
  const int k0 = blockIdx.x * kBwdKeys;
  const int kend = min(k0 + kBwdKeys, n_keys);
  const int kw0 = k0 + wave * 32;
  const int mykey = kw0 + (lane & 31);

  // K, V fragments of this wave's 32 keys (B operands: lane = key, 8 d values).
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (mykey < n_keys) {
      const int64_t off = ((int64_t)mykey * hkv + g) * D + ks * 16 + half * 8;
      a = *reinterpret_cast<const u32x4*>(k + off);
      b = *reinterpret_cast<const u32x4*>(v + off);
    }
    kf[ks] = as_bf16x8(a);
    vf[ks] = as_bf16x8(b);
  }
  // K^T of the workgroup's 128 keys in LDS (B operand of dQ = dS K).
  for (int c = tid; c < (kBwdKeys / 4) * (D / 8); c += kBwdThreads) {
    const int col = (c % (D / 8)) * 8, kq = (c / (D / 8)) * 4;
    u32x4 r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kg = k0 + kq + u;
      r[u] = u32x4{0u, 0u, 0u, 0u};
      if (kg < n_keys) r[u] = *reinterpret_cast<const u32x4*>(k + ((int64_t)kg * hkv + g) * D + col);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1, sh = (e & 1) * 16;
      u32x2 t;
      t.x = ((r[0][w] >> sh) & 0xffffu) | (((r[1][w] >> sh) & 0xffffu) << 16);
      t.y = ((r[2][w] >> sh) & 0xffffu) | (((r[3][w] >> sh) & 0xffffu) << 16);
      *reinterpret_cast<u32x2*>(&Kt[(col + e) * KTS + kq]) = t;
    }
  }

  f32x16 dvt[D / 32], dkt[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dvt[dt][r] = 0.f; dkt[dt][r] = 0.f; }

  for (int64_t base = 0; base < n_qc; base += kBwdThreads) {
    // ---- collect the query chunks that reach this workgroup's keys ----
    const int64_t c = base + tid;
    bool live = false;
    if (c < n_qc) {
      const int2 cr = chunk_range[c];
      live = cr.x < cr.y && cr.x < kend && cr.y > k0;
    }
    const unsigned long long bal = __ballot(live);
    if (lane == 0) wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int off = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) { off += (w < wave) ? wave_cnt[w] : 0; total += wave_cnt[w]; }
    if (live) list[off + __popcll(bal & ((1ull << lane) - 1ull))] = (int)(c - base);
    __syncthreads();

    for (int it = 0; it < total; ++it) {
      const int64_t vec0 = (base + list[it]) * kQC;
      // ---- stage Q, dO (row-major and transposed), lse, Delta, ranges ----
      {
        const int tsel = tid / 128;                     // 0: q, 1: do
        const int t = tid % 128;
        const int col = (t % (D / 8)) * 8, vq = (t / (D / 8)) * 4;
        if (vq < kQC) {
          const bf16_t* src = tsel ? dout : q;
          bf16_t* nat = tsel ? dOs : Qs;
          bf16_t* tr = tsel ? dOt : Qt;
          u32x4 r[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int64_t vec = vec0 + vq + u;
            r[u] = u32x4{0u, 0u, 0u, 0u};
            if (vec < n_vec) {
              const int64_t row = vec / G;
              const int hh = (int)(vec % G);
              r[u] = *reinterpret_cast<const u32x4*>(src + (row * hq + (int64_t)g * G + hh) * D + col);
            }
            *reinterpret_cast<u32x4*>(&nat[(vq + u) * QS + col]) = r[u];
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int w = e >> 1, sh = (e & 1) * 16;
            u32x2 tt;
            tt.x = ((r[0][w] >> sh) & 0xffffu) | (((r[1][w] >> sh) & 0xffffu) << 16);
            tt.y = ((r[2][w] >> sh) & 0xffffu) | (((r[3][w] >> sh) & 0xffffu) << 16);
            *reinterpret_cast<u32x2*>(&tr[(col + e) * TS + vq]) = tt;
          }
        }
        if (tid < kQC) {
          const int64_t vec = vec0 + tid;
          float l2 = -INFINITY, dl = 0.f;
          int lo = 0, hi = 0;
          long long doff = -1;
          if (vec < n_vec) {
            const int64_t row = vec / G;
            const int hh = (int)(vec % G);
            const int64_t idx = row * hq + (int64_t)g * G + hh;
            const float l = lse[idx];
            if (l != -INFINITY) {
              const int2 rg = block_range[row / B];
              lo = rg.x;
              hi = rg.y;
              l2 = l * kLog2e;
            }
            dl = delta[idx];
            doff = idx * D;
          }
          lse_s[tid] = l2;
          dlt_s[tid] = dl;
          lo_s[tid] = lo;
          hi_s[tid] = hi;
          dq_off[tid] = doff;
        }
      }
      __syncthreads();

      // ---- per wave: S, dP, P, dS; dV^T, dK^T updates; dS to LDS ----
      int wlo = 0x7fffffff, whi = -1;
#pragma unroll
      for (int t = 0; t < kQC; ++t)
        if (lo_s[t] < hi_s[t]) { wlo = min(wlo, lo_s[t]); whi = max(whi, hi_s[t]); }
      const bool active = kw0 < whi && kw0 + 32 > wlo && kw0 < n_keys;
      f32x16 sacc, pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) { sacc[r] = 0.f; pacc[r] = 0.f; }
      if (active) {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const u32x4 aq = *reinterpret_cast<const u32x4*>(&Qs[(lane & 31) * QS + ks * 16 + half * 8]);
          const u32x4 ad = *reinterpret_cast<const u32x4*>(&dOs[(lane & 31) * QS + ks * 16 + half * 8]);
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aq), kf[ks], sacc, 0, 0, 0);
          pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ad), vf[ks], pacc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qv = 8 * (r >> 2) + 4 * half + (r & 3);
          const bool ok = mykey >= lo_s[qv] && mykey < hi_s[qv];
          const float p = ok ? fast_exp2(sacc[r] * scale_log2 - lse_s[qv]) : 0.f;
          sacc[r] = p;
          pacc[r] = p * (pacc[r] - dlt_s[qv]);
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          u32x4 pu, su;
          pu.x = pack2(sacc[8 * h2 + 0], sacc[8 * h2 + 1]);
          pu.y = pack2(sacc[8 * h2 + 2], sacc[8 * h2 + 3]);
          pu.z = pack2(sacc[8 * h2 + 4], sacc[8 * h2 + 5]);
          pu.w = pack2(sacc[8 * h2 + 6], sacc[8 * h2 + 7]);
          su.x = pack2(pacc[8 * h2 + 0], pacc[8 * h2 + 1]);
          su.y = pack2(pacc[8 * h2 + 2], pacc[8 * h2 + 3]);
          su.z = pack2(pacc[8 * h2 + 4], pacc[8 * h2 + 5]);
          su.w = pack2(pacc[8 * h2 + 6], pacc[8 * h2 + 7]);
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const int rowd = (dt * 32 + (lane & 31));
            const bf16_t* dr = &dOt[rowd * TS + 16 * h2 + 4 * half];
            const bf16_t* qr = &Qt[rowd * TS + 16 * h2 + 4 * half];
            const u32x2 d0 = *reinterpret_cast<const u32x2*>(dr);
            const u32x2 d1 = *reinterpret_cast<const u32x2*>(dr + 8);
            const u32x2 q0 = *reinterpret_cast<const u32x2*>(qr);
            const u32x2 q1 = *reinterpret_cast<const u32x2*>(qr + 8);
            const u32x4 ad = {d0.x, d0.y, d1.x, d1.y};
            const u32x4 aq = {q0.x, q0.y, q1.x, q1.y};
            dvt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ad), as_bf16x8(pu), dvt[dt], 0, 0, 0);
            dkt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aq), as_bf16x8(su), dkt[dt], 0, 0, 0);
          }
        }
      }
      // dS (bf16) into LDS as [vec][key]; inactive waves write zeros.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qv = 8 * (r >> 2) + 4 * half + (r & 3);
        dSs[qv * SS + wave * 32 + (lane & 31)] = to_bf16(pacc[r]);
      }
      __syncthreads();

      // ---- dQ = dS K for one 32-wide d slice per wave, atomically added ----
      {
        constexpr int NDT = D / 32;                  // d slices
        constexpr int KSPLIT = 4 / NDT;              // waves sharing a slice
        constexpr int KSTEPS = kBwdKeys / 16 / KSPLIT;
        const int dt = wave % NDT, kpart = wave / NDT;
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          const int kb = (kpart * KSTEPS + kk) * 16 + half * 8;
          const u32x4 a = *reinterpret_cast<const u32x4*>(&dSs[(lane & 31) * SS + kb]);
          const u32x4 b = *reinterpret_cast<const u32x4*>(&Kt[(dt * 32 + (lane & 31)) * KTS + kb]);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qv = 8 * (r >> 2) + 4 * half + (r & 3);
          const long long doff = dq_off[qv];
          if (doff >= 0) atomicAdd(dq + doff + dt * 32 + (lane & 31), acc[r] * scale);
        }
      }
      __syncthreads();
    }
  }

  // ---- write dK = scale * dK^T, dV = dV^T for this wave's keys ----
  if (mykey < n_keys) {
    bf16_t* dkp = dk + ((int64_t)mykey * hkv + g) * D;
    bf16_t* dvp = dv + ((int64_t)mykey * hkv + g) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = dt * 32 + 8 * jj + 4 * half;
        u32x2 a, b;
        a.x = pack2(dkt[dt][4 * jj] * scale, dkt[dt][4 * jj + 1] * scale);
        a.y = pack2(dkt[dt][4 * jj + 2] * scale, dkt[dt][4 * jj + 3] * scale);
        b.x = pack2(dvt[dt][4 * jj], dvt[dt][4 * jj + 1]);
        b.y = pack2(dvt[dt][4 * jj + 2], dvt[dt][4 * jj + 3]);
        *reinterpret_cast<u32x2*>(dkp + d0) = a;
        *reinterpret_cast<u32x2*>(dvp + d0) = b;
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

template <int D>
hipError_t launch_bwd_t(const splitkv_anchors& an, const splitkv_heads& hd, int64_t n_keys,
                        const int2* block_range, int2* chunk_range, const void* q,
                        const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, float* delta, float* dq, void* dk, void* dv,
                        hipStream_t stream) {
  const int64_t Q = an.n_blocks * an.block_size;
  const int64_t n_rh = Q * hd.hq;
  if (o != nullptr && n_rh > 0) {
    const unsigned grid = (unsigned)((n_rh + 255) / 256);
    if (hd.dtype == SPLITKV_BF16)
      hipLaunchKernelGGL((delta_kernel<D, bf16_t>), dim3(grid), dim3(256), 0, stream,
                         static_cast<const bf16_t*>(o), static_cast<const bf16_t*>(dout), delta,
                         n_rh);
    else
      hipLaunchKernelGGL((delta_kernel<D, float>), dim3(grid), dim3(256), 0, stream,
                         static_cast<const float*>(o), static_cast<const float*>(dout), delta,
                         n_rh);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (hd.dtype == SPLITKV_BF16) {
    const int G = hd.hq / hd.hkv;
    const int64_t n_vec = Q * G;
    const int64_t n_qc = (n_vec + kQC - 1) / kQC;
    if (n_qc > 0) {
      hipLaunchKernelGGL(chunk_range_kernel, dim3((unsigned)((n_qc + 255) / 256)), dim3(256), 0,
                         stream, block_range, n_vec, G, an.block_size, n_qc, chunk_range);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    if (n_keys == 0) return hipSuccess;
    const dim3 grid((unsigned)((n_keys + kBwdKeys - 1) / kBwdKeys), (unsigned)hd.hkv);
    hipLaunchKernelGGL((attn_bwd_bf16_kernel<D>), grid, dim3(kBwdThreads), 0, stream,
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                       static_cast<const bf16_t*>(v), static_cast<const bf16_t*>(dout), lse,
                       delta, dq, static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv),
                       block_range, chunk_range, n_vec, n_qc, G, hd.hq, hd.hkv, an.block_size,
                       (int)n_keys, hd.scale, hd.scale * kLog2e);
    return hipGetLastError();
  }
  if (n_rh > 0)
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D>), dim3((unsigned)((n_rh + 127) / 128)), dim3(128), 0,
                     stream, static_cast<const float*>(q), static_cast<const float*>(k),
                     static_cast<const float*>(v), static_cast<const float*>(dout), lse, delta,
                     dq, block_range, Q, hd.hq, hd.hkv, an.block_size, hd.scale);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
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
                      const int2* block_range, int2* chunk_range, const void* q, const void* k,
                      const void* v, const void* o, const void* dout, const float* lse,
                      float* delta, float* dq, void* dk, void* dv, hipStream_t stream) {
  if (hd.d == 128)
    return launch_bwd_t<128>(an, hd, n_keys, block_range, chunk_range, q, k, v, o, dout, lse,
                             delta, dq, dk, dv, stream);
  return launch_bwd_t<64>(an, hd, n_keys, block_range, chunk_range, q, k, v, o, dout, lse, delta,
                          dq, dk, dv, stream);
}

}  // namespace splitkv
