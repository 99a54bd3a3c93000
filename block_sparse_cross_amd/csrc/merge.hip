// Exact LSE merge of P partials (Eq. 4 of "Split-KV: Efficient Context
// Parallelism for Training Diffusion Drafters", §4.1):
//   lse = log sum_p exp(lse_p),   o = sum_p exp(lse_p - lse) o_p.
//
// Bandwidth-bound: every byte of the P partial outputs is read once. A unit
// is 8 consecutive output elements of one row, read from each partial with one
// 16-byte (bf16) or two 16-byte (fp32) non-temporal loads (the partials are not
// read again); the d/8 units of a row are adjacent, so each partial's row
// segment is read fully coalesced, and the lse_p of a row are read by all its
// units' threads (cache broadcast). Each thread owns four units, 256 units
// apart, and keeps two partials (bf16) in flight for all four: on MI355X that
// took the merge at P = 32 over 2M rows of 128 from 65% to 69.5% of HBM
// bandwidth and P = 9 from 67% to 75% (the earlier kernel, one unit per thread
// with eight partials in flight, kept many DRAM rows of one bank open at once
// when the partials lie a power of two apart); P = 8 and 64 were unchanged or
// up to 3% faster. Non-temporal loads had taken the weak-scaling share's merge
// (P = 8, 262144 rows) from 5.49 to 6.28 TB/s.
#include "common.hpp"
#include "internal.hpp"

namespace splitkv {

namespace {

constexpr int kMergeThreads = 256;
constexpr int kMergeRows = 4;  // units (8 outputs of a row) per merge thread

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

// Where a thread's units lie. A unit u holds elements [8u, 8u + 8) of each
// partial (row u / (d/8)); a thread's R units are kMergeThreads apart, so each
// of its loads is part of a workgroup-wide contiguous run.
//  - Whole (d = 64, 128 or 256): all R units exist, and the r-th sits a fixed,
//    compile-time distance from the first in rows and elements, so all its
//    loads come off one address with constant offsets (a group's loads then
//    issue back to back).
//  - Edge (the tail of the rows, or any other d): units are placed one by one;
//    a unit past the end repeats the last one (loaded, never stored).
// Launched separately, so the tail's bookkeeping costs the main launch no
// registers.
template <int kSegs>
struct WholeUnits {
  static constexpr int kRowStep = kMergeThreads / kSegs;  // rows between a thread's units
  int64_t unit0, row0;
  bool head0;  // the first unit starts its row
  __device__ int64_t unit(int r) const { return unit0 + (int64_t)r * kMergeThreads; }
  __device__ int64_t row(int r) const { return row0 + r * kRowStep; }
  __device__ bool live(int) const { return true; }
  __device__ bool head(int) const { return head0; }
};
template <int R>
struct EdgeUnits {
  int64_t unit_[R], row_[R];
  bool live_[R];
  int segs;
  __device__ int64_t unit(int r) const { return unit_[r]; }
  __device__ int64_t row(int r) const { return row_[r]; }
  __device__ bool live(int r) const { return live_[r]; }
  __device__ bool head(int r) const { return row_[r] * segs == unit_[r]; }
};

template <typename Tin, typename Tout, int R, class Units>
__device__ __forceinline__ void merge_units(int P, int64_t rows, int d, const Tin* o_parts,
                                            const float* lse_parts, Tout* o, float* lse,
                                            const Units& U) {
  using Raw = typename Vec8<Tin>::Raw;
  constexpr int G = sizeof(Tin) == 2 ? 2 : 1;  // partials per group
  const int64_t pstride = rows * (int64_t)d;
  auto pidx = [P](int p) -> int64_t { return p < P ? p : P - 1; };
  auto load_group = [&](int g, float (*l)[G], Raw (*x8)[G]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int u = 0; u < G; ++u) l[r][u] = lse_parts[pidx(g + u) * rows + U.row(r)];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int u = 0; u < G; ++u)
        x8[r][u] = Vec8<Tin>::ld(o_parts + pidx(g + u) * pstride + U.unit(r) * 8);
  };

  // Partials are taken G at a time for all R units: a group's lse_p and its
  // o_p segments are loaded together (LSEs first, so they arrive first), and
  // the next group's loads are in flight while the current one is summed.
  // Indices past the last partial load partial P-1 again (unused), so every
  // load is issued unconditionally and the waits can count them.
  float lcur[R][G];
  Raw cur[R][G];
  load_group(0, lcur, cur);
  float mx[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    mx[r] = -INFINITY;
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (u < P) mx[r] = fmaxf(mx[r], lcur[r][u]);
  }
  for (int p0 = G; p0 < P; p0 += G) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float l[G];
#pragma unroll
      for (int u = 0; u < G; ++u) l[u] = lse_parts[pidx(p0 + u) * rows + U.row(r)];
#pragma unroll
      for (int u = 0; u < G; ++u)
        if (p0 + u < P) mx[r] = fmaxf(mx[r], l[u]);
    }
  }

  // Unnormalised sum with weights exp(lse_p - max), p ascending; empty
  // partials weigh 0. (A row whose partials are all empty has max = -inf; its
  // sums are discarded below.)
  float acc[R][8], wsum[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    wsum[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  }
  auto sum_group = [&](int g, float (*l)[G], Raw (*x8)[G]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int u = 0; u < G; ++u) {
        if (g + u < P) {
          const float w = __expf(l[r][u] - mx[r]);
          float x[8];
          Vec8<Tin>::cvt(x8[r][u], x);
          wsum[r] += w;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(w, x[e], acc[r][e]);
        }
      }
  };
  // Two register buffers in turn, so a group's loads are issued before the
  // group ahead of it is summed and no buffer is copied.
  float lnx[R][G];
  Raw nxt[R][G];
  for (int g = 0; g < P; g += 2 * G) {
    if (g + G < P) load_group(g + G, lnx, nxt);
    sum_group(g, lcur, cur);
    if (g + 2 * G < P) load_group(g + 2 * G, lcur, cur);
    if (g + G < P) sum_group(g + G, lnx, nxt);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (!U.live(r)) continue;
    const bool empty = mx[r] == -INFINITY;  // every partial empty
    const float inv = empty ? 0.f : 1.f / wsum[r];
    float out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = empty ? 0.f : acc[r][e] * inv;
    Vec8<Tout>::store(o + U.unit(r) * 8, out);
    if (U.head(r)) lse[U.row(r)] = empty ? -INFINITY : mx[r] + __logf(wsum[r]);
  }
}

// Units [unit_base, unit_base + gridDim.x * kMergeThreads * R), clipped to
// rows * d/8 on the Edge form (kSegs = 0); the Whole form (kSegs = d/8) takes
// only whole workgroups.
template <typename Tin, typename Tout, int R, int kSegs>
__global__ void __launch_bounds__(kMergeThreads)
lse_merge_kernel(int P, int64_t rows, int d, int64_t unit_base, const Tin* __restrict__ o_parts,
                 const float* __restrict__ lse_parts, Tout* __restrict__ o,
                 float* __restrict__ lse) {
  const int segs = d / 8;
  const int64_t units = rows * segs;
  const int64_t first = unit_base + (int64_t)blockIdx.x * (kMergeThreads * R) + threadIdx.x;
  if (first >= units) return;
  if constexpr (kSegs > 0) {
    WholeUnits<kSegs> U;
    U.unit0 = first;
    U.row0 = first / kSegs;
    U.head0 = first % kSegs == 0;
    merge_units<Tin, Tout, R>(P, rows, d, o_parts, lse_parts, o, lse, U);
  } else {
    EdgeUnits<R> U;
    U.segs = segs;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t unit = first + (int64_t)r * kMergeThreads;
      U.live_[r] = unit < units;
      U.unit_[r] = U.live_[r] ? unit : units - 1;
      U.row_[r] = units <= INT32_MAX ? (int64_t)((uint32_t)U.unit_[r] / (uint32_t)segs)
                                     : U.unit_[r] / segs;
    }
    merge_units<Tin, Tout, R>(P, rows, d, o_parts, lse_parts, o, lse, U);
  }
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
  const int segs = d / 8;
  const int64_t units = rows * segs;
  constexpr int64_t kWholeUnits = (int64_t)kMergeThreads * kMergeRows;  // per workgroup
  const int64_t whole = (segs == 8 || segs == 16 || segs == 32) ? units / kWholeUnits : 0;
  if (whole > 0) {
    const dim3 grid((unsigned)whole);
    auto kern = segs == 8    ? lse_merge_kernel<Tin, Tout, kMergeRows, 8>
                : segs == 16 ? lse_merge_kernel<Tin, Tout, kMergeRows, 16>
                             : lse_merge_kernel<Tin, Tout, kMergeRows, 32>;
    hipLaunchKernelGGL(kern, grid, dim3(kMergeThreads), 0, stream, P, rows, d, (int64_t)0,
                       static_cast<const Tin*>(o_parts), lse_parts, static_cast<Tout*>(o), lse);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t rest = units - whole * kWholeUnits;
  if (rest > 0) {
    hipLaunchKernelGGL((lse_merge_kernel<Tin, Tout, 1, 0>),
                       dim3((unsigned)((rest + kMergeThreads - 1) / kMergeThreads)),
                       dim3(kMergeThreads), 0, stream, P, rows, d, whole * kWholeUnits,
                       static_cast<const Tin*>(o_parts), lse_parts, static_cast<Tout*>(o), lse);
    return hipGetLastError();
  }
  return hipSuccess;
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
