// Exact LSE merge of P partials (Eq. 4 of "Split-KV: Efficient Context
// Parallelism for Training Diffusion Drafters", §4.1):
//   lse = log sum_p exp(lse_p),   o = sum_p exp(lse_p - lse) o_p.
//
// Bandwidth-bound: every byte of the P partial outputs is read once. One
// thread owns 8 consecutive output elements of one row and streams the P
// partials with 16-byte (bf16) or 2x16-byte (fp32) loads; the d/8 threads of a
// row are adjacent, so each partial's row segment is read fully coalesced.
// The lse_p of a row are read by all its threads (cache broadcast). The
// partials are read with non-temporal loads (they are not read again); on
// MI355X that alone took the weak-scaling share's merge (P = 8, 262144 rows of
// 128) from 5.49 to 6.28 TB/s, and P = 64 from 5.40 to 5.98 TB/s.
#include "common.hpp"
#include "internal.hpp"

namespace splitkv {

namespace {

constexpr int kMergeThreads = 256;
constexpr int kMergeGroup = 8;  // partial loads kept in flight per thread

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Eight elements of a row: `load`/`store` convert to and from fp32; `ld`
// fetches the raw bytes with a non-temporal (streaming) load and `cvt`
// converts them later, so loads can be issued well ahead of their use.
template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
  using Raw = uint4;
  __device__ __forceinline__ static Raw ld(const bf16_t* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return uint4{v.x, v.y, v.z, v.w};
  }
  __device__ __forceinline__ static void cvt(const Raw& u, float* x) {
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void load(const bf16_t* p, float* x) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void store(bf16_t* p, const float* x) {
    uint4 u;
    u.x = pack_bf16x2(x[0], x[1]);
    u.y = pack_bf16x2(x[2], x[3]);
    u.z = pack_bf16x2(x[4], x[5]);
    u.w = pack_bf16x2(x[6], x[7]);
    *reinterpret_cast<uint4*>(p) = u;
  }
};
template <> struct Vec8<float> {
  struct Raw {
    float4 a, b;
  };
  __device__ __forceinline__ static Raw ld(const float* p) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
    return Raw{make_float4(a.x, a.y, a.z, a.w), make_float4(b.x, b.y, b.z, b.w)};
  }
  __device__ __forceinline__ static void cvt(const Raw& r, float* x) {
    x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
    x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
  }
  __device__ __forceinline__ static void load(const float* p, float* x) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  __device__ __forceinline__ static void store(float* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
  }
};

template <typename Tin, typename Tout>
__global__ void __launch_bounds__(kMergeThreads)
lse_merge_kernel(int P, int64_t rows, int d, const Tin* __restrict__ o_parts,
                 const float* __restrict__ lse_parts, Tout* __restrict__ o,
                 float* __restrict__ lse) {
  using Raw = typename Vec8<Tin>::Raw;
  constexpr int G = kMergeGroup;
  const int segs = d / 8;
  const int64_t units = rows * segs;
  const int64_t unit = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  if (unit >= units) return;
  int64_t row;
  int seg;
  if (units <= INT32_MAX) {  // uniform: 32-bit division when the index fits
    const uint32_t u32 = (uint32_t)unit;
    row = u32 / (uint32_t)segs;
    seg = (int)(u32 - (uint32_t)row * (uint32_t)segs);
  } else {
    row = unit / segs;
    seg = (int)(unit % segs);
  }
  const Tin* src = o_parts + row * d + seg * 8;
  const int64_t pstride = rows * (int64_t)d;
  const float* lrow = lse_parts + row;

  // Partials are taken G at a time: a group's lse_p and its o_p segments are
  // loaded together (LSEs first, so they arrive first), and the next group's
  // loads are in flight while the current one is summed. Indices past the
  // last partial load partial P-1 again (unused), so every load is issued
  // unconditionally and the waits can count them.
  auto pidx = [P](int p) -> int64_t { return p < P ? p : P - 1; };
  float lcur[G];
  Raw cur[G];
#pragma unroll
  for (int u = 0; u < G; ++u) lcur[u] = lrow[pidx(u) * rows];
#pragma unroll
  for (int u = 0; u < G; ++u) cur[u] = Vec8<Tin>::ld(src + pidx(u) * pstride);

  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < G; ++u)
    if (u < P) mx = fmaxf(mx, lcur[u]);
  for (int p0 = G; p0 < P; p0 += G) {
    float l[G];
#pragma unroll
    for (int u = 0; u < G; ++u) l[u] = lrow[pidx(p0 + u) * rows];
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (p0 + u < P) mx = fmaxf(mx, l[u]);
  }

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  Tout* orow = o + row * d + seg * 8;
  if (mx == -INFINITY) {  // every partial empty
    Vec8<Tout>::store(orow, acc);
    if (seg == 0) lse[row] = -INFINITY;
    return;
  }
  // Unnormalised sum with weights exp(lse_p - max), p ascending; empty
  // partials weigh 0.
  float wsum = 0.f;
  auto sum_group = [&](int g, const float* l, const Raw* x8) {
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (g + u < P) {
        const float w = __expf(l[u] - mx);
        float x[8];
        Vec8<Tin>::cvt(x8[u], x);
        wsum += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, x[e], acc[e]);
      }
    }
  };
  auto load_group = [&](int g, float* l, Raw* x8) {
#pragma unroll
    for (int u = 0; u < G; ++u) l[u] = lrow[pidx(g + u) * rows];
#pragma unroll
    for (int u = 0; u < G; ++u) x8[u] = Vec8<Tin>::ld(src + pidx(g + u) * pstride);
  };
  // Two register buffers in turn, so a group's loads are issued before the
  // group ahead of it is summed and no buffer is copied.
  float lnx[G];
  Raw nxt[G];
  for (int g = 0; g < P; g += 2 * G) {
    if (g + G < P) load_group(g + G, lnx, nxt);
    sum_group(g, lcur, cur);
    if (g + 2 * G < P) load_group(g + 2 * G, lcur, cur);
    if (g + G < P) sum_group(g + G, lnx, nxt);
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= inv;
  Vec8<Tout>::store(orow, acc);
  if (seg == 0) lse[row] = mx + __logf(wsum);
}

// Eq. 4 split into the two halves each rank applies when the partials sit on
// different devices (Algorithm 1's MERGE after the LSE all-reduce). First the
// LSE statistics: lse = log sum_p exp(lse_p), one thread per row, the P reads
// of a row strided by `rows` so a wave's loads are coalesced.
__global__ void __launch_bounds__(kMergeThreads)
lse_reduce_kernel(int P, int64_t rows, const float* __restrict__ lse_parts,
                  float* __restrict__ lse) {
  const int64_t row = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  if (row >= rows) return;
  float mx = -INFINITY;
  for (int p = 0; p < P; ++p) mx = fmaxf(mx, lse_parts[(int64_t)p * rows + row]);
  if (mx == -INFINITY) {
    lse[row] = -INFINITY;
    return;
  }
  float sum = 0.f;
  for (int p = 0; p < P; ++p) sum += __expf(lse_parts[(int64_t)p * rows + row] - mx);
  lse[row] = mx + __logf(sum);
}

// Then each rank's own partial: o_bar = exp(lse_p - lse) o_p, zero where the
// partial is empty (lse_p = -inf). One thread per 8 consecutive elements.
template <typename Tin, typename Tout>
__global__ void __launch_bounds__(kMergeThreads)
lse_rescale_kernel(int64_t rows, int d, const Tin* o_part, const float* __restrict__ lse_part,
                   const float* __restrict__ lse, Tout* o_bar) {
  // o_bar may alias o_part (in place): each thread loads its 8 elements
  // before it stores them, and no other thread touches them
  const int segs = d / 8;
  const int64_t unit = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  if (unit >= rows * segs) return;
  const int64_t row = unit / segs;
  const float lp = lse_part[row];
  const float w = lp == -INFINITY ? 0.f : __expf(lp - lse[row]);
  float x[8];
  Vec8<Tin>::load(o_part + unit * 8, x);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] *= w;
  Vec8<Tout>::store(o_bar + unit * 8, x);
}

// Delta[r] (+)= <do[r], o[r]> over rows of d elements (the quantity Algorithm
// 1's MERGE_BWD all-reduces; from a rank's rescaled partial it is that rank's
// share). One thread per 8 elements; the d/8 threads of a row (a power of two
// <= 64, so they share a wave) sum with lane exchanges.
template <typename To, typename Td>
__global__ void __launch_bounds__(kMergeThreads)
delta_rows_kernel(int64_t rows, int d, const To* __restrict__ o, const Td* __restrict__ dout,
                  float* __restrict__ delta, int accumulate) {
  const int segs = d / 8;
  const int64_t unit = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  if (unit >= rows * segs) return;
  float x[8], y[8];
  Vec8<To>::load(o + unit * 8, x);
  Vec8<Td>::load(dout + unit * 8, y);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = fmaf(x[e], y[e], acc);
  for (int off = segs / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (unit % segs == 0) {
    const int64_t row = unit / segs;
    delta[row] = accumulate ? delta[row] + acc : acc;
  }
}

// fp32 -> bf16 (round to nearest even), 8 elements per thread.
__global__ void __launch_bounds__(kMergeThreads)
cast_bf16_kernel(int64_t units, const float* __restrict__ src, bf16_t* __restrict__ dst) {
  const int64_t unit = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  if (unit >= units) return;
  float x[8];
  Vec8<float>::load(src + unit * 8, x);
  Vec8<bf16_t>::store(dst + unit * 8, x);
}

template <typename Tin, typename Tout>
hipError_t launch_rescale_t(int64_t rows, int32_t d, const void* o_part, const float* lse_part,
                            const float* lse, void* o_bar, hipStream_t stream) {
  const int64_t units = rows * (d / 8);
  const int64_t grid = (units + kMergeThreads - 1) / kMergeThreads;
  hipLaunchKernelGGL((lse_rescale_kernel<Tin, Tout>), dim3((unsigned)grid), dim3(kMergeThreads),
                     0, stream, rows, d, static_cast<const Tin*>(o_part), lse_part, lse,
                     static_cast<Tout*>(o_bar));
  return hipGetLastError();
}

template <typename To, typename Td>
hipError_t launch_delta_t(int64_t rows, int32_t d, const void* o, const void* dout, float* delta,
                          int accumulate, hipStream_t stream) {
  const int64_t units = rows * (d / 8);
  const int64_t grid = (units + kMergeThreads - 1) / kMergeThreads;
  hipLaunchKernelGGL((delta_rows_kernel<To, Td>), dim3((unsigned)grid), dim3(kMergeThreads), 0,
                     stream, rows, d, static_cast<const To*>(o), static_cast<const Td*>(dout),
                     delta, accumulate);
  return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_merge_t(int32_t P, int64_t rows, int32_t d, const void* o_parts,
                          const float* lse_parts, void* o, float* lse, hipStream_t stream) {
  const int64_t units = rows * (d / 8);
  const int64_t grid = (units + kMergeThreads - 1) / kMergeThreads;
  hipLaunchKernelGGL((lse_merge_kernel<Tin, Tout>), dim3((unsigned)grid), dim3(kMergeThreads),
                     0, stream, P, rows, d, static_cast<const Tin*>(o_parts), lse_parts,
                     static_cast<Tout*>(o), lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(int32_t P, int64_t rows, int32_t d, const void* o_parts, int in_dtype,
                        const float* lse_parts, void* o, int out_dtype, float* lse,
                        hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (in_dtype == SPLITKV_BF16 && out_dtype == SPLITKV_BF16)
    return launch_merge_t<bf16_t, bf16_t>(P, rows, d, o_parts, lse_parts, o, lse, stream);
  if (in_dtype == SPLITKV_BF16 && out_dtype == SPLITKV_FP32)
    return launch_merge_t<bf16_t, float>(P, rows, d, o_parts, lse_parts, o, lse, stream);
  if (in_dtype == SPLITKV_FP32 && out_dtype == SPLITKV_BF16)
    return launch_merge_t<float, bf16_t>(P, rows, d, o_parts, lse_parts, o, lse, stream);
  return launch_merge_t<float, float>(P, rows, d, o_parts, lse_parts, o, lse, stream);
}

hipError_t launch_lse_reduce(int32_t P, int64_t rows, const float* lse_parts, float* lse,
                             hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t grid = (rows + kMergeThreads - 1) / kMergeThreads;
  hipLaunchKernelGGL(lse_reduce_kernel, dim3((unsigned)grid), dim3(kMergeThreads), 0, stream, P,
                     rows, lse_parts, lse);
  return hipGetLastError();
}

hipError_t launch_lse_rescale(int64_t rows, int32_t d, const void* o_part, int in_dtype,
                              const float* lse_part, const float* lse, void* o_bar,
                              int out_dtype, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (in_dtype == SPLITKV_BF16 && out_dtype == SPLITKV_BF16)
    return launch_rescale_t<bf16_t, bf16_t>(rows, d, o_part, lse_part, lse, o_bar, stream);
  if (in_dtype == SPLITKV_BF16 && out_dtype == SPLITKV_FP32)
    return launch_rescale_t<bf16_t, float>(rows, d, o_part, lse_part, lse, o_bar, stream);
  if (in_dtype == SPLITKV_FP32 && out_dtype == SPLITKV_BF16)
    return launch_rescale_t<float, bf16_t>(rows, d, o_part, lse_part, lse, o_bar, stream);
  return launch_rescale_t<float, float>(rows, d, o_part, lse_part, lse, o_bar, stream);
}

hipError_t launch_delta(int64_t rows, int32_t d, const void* o, int o_dtype, const void* dout,
                        int do_dtype, float* delta, int accumulate, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (o_dtype == SPLITKV_BF16 && do_dtype == SPLITKV_BF16)
    return launch_delta_t<bf16_t, bf16_t>(rows, d, o, dout, delta, accumulate, stream);
  if (o_dtype == SPLITKV_BF16 && do_dtype == SPLITKV_FP32)
    return launch_delta_t<bf16_t, float>(rows, d, o, dout, delta, accumulate, stream);
  if (o_dtype == SPLITKV_FP32 && do_dtype == SPLITKV_BF16)
    return launch_delta_t<float, bf16_t>(rows, d, o, dout, delta, accumulate, stream);
  return launch_delta_t<float, float>(rows, d, o, dout, delta, accumulate, stream);
}

hipError_t launch_cast_bf16(int64_t n, const float* src, void* dst, hipStream_t stream) {
  const int64_t units = n / 8;
  if (units == 0) return hipSuccess;
  const int64_t grid = (units + kMergeThreads - 1) / kMergeThreads;
  hipLaunchKernelGGL(cast_bf16_kernel, dim3((unsigned)grid), dim3(kMergeThreads), 0, stream,
                     units, src, static_cast<bf16_t*>(dst));
  return hipGetLastError();
}

}  // namespace splitkv
