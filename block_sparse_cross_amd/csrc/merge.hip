// Exact LSE merge of P partials (Eq. 4 of "Split-KV: Efficient Context
// Parallelism for Training Diffusion Drafters", §4.1):
//   lse = log sum_p exp(lse_p),   o = sum_p exp(lse_p - lse) o_p.
//
// Bandwidth-bound: every byte of the P partial outputs is read once. One
// thread owns 8 consecutive output elements of one row and streams the P
// partials with 16-byte (bf16) or 2x16-byte (fp32) loads; the d/8 threads of a
// row are adjacent, so each partial's row segment is read fully coalesced.
// The lse_p of a row are read by all its threads (cache broadcast).
#include "common.hpp"
#include "internal.hpp"

namespace splitkv {

namespace {

constexpr int kMergeThreads = 256;

template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
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
  const int segs = d / 8;
  const int64_t unit = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  if (unit >= rows * segs) return;
  const int64_t row = unit / segs;
  const int seg = (int)(unit % segs);

  float mx = -INFINITY;
  for (int p = 0; p < P; ++p) mx = fmaxf(mx, lse_parts[(int64_t)p * rows + row]);

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  Tout* orow = o + row * d + seg * 8;
  if (mx == -INFINITY) {  // every partial empty
    Vec8<Tout>::store(orow, acc);
    if (seg == 0) lse[row] = -INFINITY;
    return;
  }
  // Unnormalised sum with weights exp(lse_p - max); empty partials weigh 0.
  float wsum = 0.f;
  const Tin* src = o_parts + row * d + seg * 8;
  const int64_t pstride = rows * (int64_t)d;
  int p = 0;
  for (; p + 4 <= P; p += 4) {
    float x[4][8], w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      Vec8<Tin>::load(src + (int64_t)(p + u) * pstride, x[u]);
      w[u] = __expf(lse_parts[(int64_t)(p + u) * rows + row] - mx);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      wsum += w[u];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w[u], x[u][e], acc[e]);
    }
  }
  for (; p < P; ++p) {
    float x[8];
    Vec8<Tin>::load(src + (int64_t)p * pstride, x);
    float w = __expf(lse_parts[(int64_t)p * rows + row] - mx);
    wsum += w;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, x[e], acc[e]);
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
lse_rescale_kernel(int64_t rows, int d, const Tin* __restrict__ o_part,
                   const float* __restrict__ lse_part, const float* __restrict__ lse,
                   Tout* __restrict__ o_bar) {
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
