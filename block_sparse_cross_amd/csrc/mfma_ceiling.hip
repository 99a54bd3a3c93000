// Matrix-core ceiling of the device, measured rather than taken from the spec
// sheet: a loop of v_mfma_f32_32x32x16_bf16 products with nothing else in it,
// to read the attention kernels' product rates against. Built as its own
// library (libsplitkv_ceiling.so), not part of the Split-KV entry points.
//
//   int splitkv_ceiling_mfma(const void* frags, int64_t iters, int32_t n_wg,
//                            float* out, void* stream);
//
// frags: device, 8 operand fragments of 64 lanes x 8 bf16 (8 KB, 16-byte
//   aligned), read once per wave: fragments 0-3 serve as A, 4-7 as B. Random
//   operands make the products toggle their inputs as real data does (the
//   board's power limit then sets the clock); constant ones do not.
// iters: loop trips; each trip issues 32 products per wave (4 waves per
//   workgroup), so the launch does n_wg * 4 * iters * 32 * 32768 FLOP.
// out: device, n_wg * 256 floats (one sum per lane, so nothing is dead code).
// Returns 0, or -1 for a bad argument, or the HIP error of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) mfma_loop_kernel(const u32x4* __restrict__ frags,
                                                        int64_t iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_bit_cast(bf16x8, frags[i * 64 + lane]);
    b[i] = __builtin_bit_cast(bf16x8, frags[(4 + i) * 64 + lane]);
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int64_t it = 0; it < iters; ++it) {
    // 8 independent accumulators; consecutive products take different
    // operand pairs
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + u) & 3], b[j & 3], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" int splitkv_ceiling_mfma(const void* frags, int64_t iters, int32_t n_wg, float* out,
                                    void* stream) {
  if (frags == nullptr || out == nullptr || iters < 0 || n_wg < 1) return -1;
  if ((reinterpret_cast<uintptr_t>(frags) & 15) != 0) return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)n_wg), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(frags), iters,
                     out);
  return (int)hipGetLastError();
}
