// Device-side check of the anchor metadata. Block i's rows attend the context
// window [s_i, a_i) of their own sample (§3.1 and Figure 1 of "Split-KV:
// Efficient Context Parallelism for Training Diffusion Drafters"), so a valid
// window is a sub-interval, possibly empty, of the packed context [0, S):
//   0 <= s_i <= a_i <= S.
// The other entry points never read anchors on the host and stay in bounds
// for any contents; this check is the debugging aid that tells whether their
// results mean anything.
#include "common.hpp"
#include "internal.hpp"

namespace splitkv {

namespace {

constexpr int kValidateThreads = 1024;

// One workgroup: thread t scans blocks t, t + 1024, ... in ascending order,
// counting the invalid ones and keeping the first; an LDS tree then sums the
// counts and takes the minimum index. result = {count, first index or -1}.
__global__ void __launch_bounds__(kValidateThreads)
validate_anchors_kernel(const int64_t* __restrict__ s, const int64_t* __restrict__ a,
                        int64_t n_blocks, int64_t S, int64_t* __restrict__ result) {
  __shared__ int64_t cnt[kValidateThreads];
  __shared__ int64_t first[kValidateThreads];
  const int tid = threadIdx.x;
  int64_t c = 0, f = INT64_MAX;
  for (int64_t i = tid; i < n_blocks; i += kValidateThreads) {
    const int64_t si = s[i], ai = a[i];
    if (!(0 <= si && si <= ai && ai <= S)) {
      c += 1;
      f = min(f, i);
    }
  }
  cnt[tid] = c;
  first[tid] = f;
  __syncthreads();
  for (int w = kValidateThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
      cnt[tid] += cnt[tid + w];
      first[tid] = min(first[tid], first[tid + w]);
    }
    __syncthreads();
  }
  if (tid == 0) {
    result[0] = cnt[0];
    result[1] = cnt[0] > 0 ? first[0] : -1;
  }
}

// Own-block windows: block i's rows also attend all B tokens of their own
// block (Figure 1: the block is bidirectional). With the block keys laid out
// in block order as one local segment of n_blocks * B positions starting at
// 0, block i's window over that segment is [i B, (i + 1) B).
__global__ void __launch_bounds__(256)
own_block_windows_kernel(int64_t n_blocks, int64_t B, int64_t* __restrict__ s,
                         int64_t* __restrict__ a, int64_t* __restrict__ chunk_start) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n_blocks) {
    s[i] = i * B;
    a[i] = (i + 1) * B;
  }
  if (i == 0) chunk_start[0] = 0;
}

}  // namespace

hipError_t launch_own_block_windows(int64_t n_blocks, int32_t B, int64_t* s, int64_t* a,
                                    int64_t* chunk_start, hipStream_t stream) {
  const int64_t grid = n_blocks > 0 ? (n_blocks + 255) / 256 : 1;
  hipLaunchKernelGGL(own_block_windows_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     n_blocks, (int64_t)B, s, a, chunk_start);
  return hipGetLastError();
}

hipError_t launch_validate_anchors(const int64_t* s, const int64_t* a, int64_t n_blocks,
                                   int64_t S, int64_t* result, hipStream_t stream) {
  hipLaunchKernelGGL(validate_anchors_kernel, dim3(1), dim3(kValidateThreads), 0, stream, s, a,
                     n_blocks, S, result);
  return hipGetLastError();
}

}  // namespace splitkv
