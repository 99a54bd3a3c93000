// Planner kernels: chunk pricing (Eq. 6) and cost-aware LPT (§4.2) of
// "Split-KV: Efficient Context Parallelism for Training Diffusion Drafters".
//
// Integer only (int64 costs and loads), so the plan is reproducible bit for
// bit. Ties are fixed: equal costs are taken in ascending chunk index, equal
// loads go to the lowest rank index.
#include "common.hpp"
#include "internal.hpp"

namespace splitkv {

namespace {

constexpr int kCostThreads = 256;
constexpr int kLptThreads = 1024;

// Eq. 6 for one chunk per workgroup: threads stride over the anchors and the
// overlaps |[s_i, a_i) ∩ [lam, lam + m)| are summed, then scaled by B.
__global__ void __launch_bounds__(kCostThreads)
chunk_cost_kernel(const int64_t* __restrict__ s, const int64_t* __restrict__ a,
                  int64_t n_blocks, int64_t B, int64_t m, int64_t* __restrict__ cost) {
  const int64_t j = blockIdx.x;
  const int64_t lam = j * m, lam_end = lam + m;
  long long total = 0;
  for (int64_t i = threadIdx.x; i < n_blocks; i += kCostThreads) {
    int64_t lo = max(s[i], lam), hi = min(a[i], lam_end);
    if (hi > lo) total += hi - lo;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) total += __shfl_xor(total, off);
  __shared__ long long part[kCostThreads / kWave];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  if (lane == 0) part[wave] = total;
  __syncthreads();
  if (threadIdx.x == 0) {
    long long t = 0;
    for (int w = 0; w < kCostThreads / kWave; ++w) t += part[w];
    cost[j] = B * t;
  }
}

// Bitonic sort of n (power of two) (key, idx) pairs in LDS. `desc_key`
// selects key-descending order; ties always break by ascending idx.
__device__ void bitonic_sort(long long* key, int* idx, int n, bool desc_key) {
  auto before = [desc_key](long long ka, int ia, long long kb, int ib) {
    if (ka != kb) return desc_key ? (ka > kb) : (ka < kb);
    return ia < ib;
  };
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        int partner = i ^ stride;
        if (partner > i) {
          bool up = (i & size) == 0;  // this run is sorted in `before` order
          long long ki = key[i], kp = key[partner];
          int ii = idx[i], ip = idx[partner];
          bool swap = up ? before(kp, ip, ki, ii) : before(ki, ii, kp, ip);
          if (swap) {
            key[i] = kp; key[partner] = ki;
            idx[i] = ip; idx[partner] = ii;
          }
        }
      }
      __syncthreads();
    }
  }
}

// (load, rank) lexicographic minimum across a wave; every lane gets it.
__device__ __forceinline__ void wave_argmin(long long& load, int& rank) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    long long ol = __shfl_xor(load, off);
    int orank = __shfl_xor(rank, off);
    if (ol < load || (ol == load && orank < rank)) { load = ol; rank = orank; }
  }
}

// One workgroup: sort chunks by cost (descending), hand them out greedily, then
// list each rank's chunks in ascending index by sorting on (owner, chunk).
__global__ void __launch_bounds__(kLptThreads)
lpt_kernel(const int64_t* __restrict__ cost, int n_chunks, int P, int J,
           int32_t* __restrict__ owner_out, int32_t* __restrict__ rank_chunks,
           int64_t* __restrict__ rank_load) {
  __shared__ long long key[kMaxPlanChunks];
  __shared__ int idx[kMaxPlanChunks];
  __shared__ int owner[kMaxPlanChunks];
  __shared__ long long best_load[2][kLptThreads / kWave];
  __shared__ int best_rank[2][kLptThreads / kWave];

  int n = 1;
  while (n < n_chunks) n <<= 1;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    key[i] = i < n_chunks ? (long long)cost[i] : -1;  // padding sorts last (costs >= 0)
    idx[i] = i;
  }
  __syncthreads();
  bitonic_sort(key, idx, n, /*desc_key=*/true);

  // Greedy: thread p owns rank p; argmin over ranks with < J chunks.
  const int p = threadIdx.x;
  const int lane = p % kWave, wave = p / kWave;
  const int n_waves = (P + kWave - 1) / kWave;
  long long load = 0;
  int held = 0;
  const long long kNone = 0x7fffffffffffffffLL;
  if (n_waves == 1) {
    if (wave == 0) {
      for (int t = 0; t < n_chunks; ++t) {
        long long cand = (p < P && held < J) ? load : kNone;
        int r = p;
        wave_argmin(cand, r);
        if (p == r) { load += key[t]; held += 1; }
        if (p == 0) owner[idx[t]] = r;
      }
    }
  } else {
    for (int t = 0; t < n_chunks; ++t) {
      long long cand = (p < P && held < J) ? load : kNone;
      int r = p;
      wave_argmin(cand, r);
      const int buf = t & 1;
      if (lane == 0 && wave < n_waves) { best_load[buf][wave] = cand; best_rank[buf][wave] = r; }
      __syncthreads();
      long long bl = best_load[buf][0];
      int br = best_rank[buf][0];
      for (int w = 1; w < n_waves; ++w) {
        long long l2 = best_load[buf][w];
        int r2 = best_rank[buf][w];
        if (l2 < bl || (l2 == bl && r2 < br)) { bl = l2; br = r2; }
      }
      if (p == br) { load += key[t]; held += 1; }
      if (p == 0) owner[idx[t]] = br;
    }
  }
  __syncthreads();
  if (p < P) rank_load[p] = load;
  for (int j = threadIdx.x; j < n_chunks; j += blockDim.x) owner_out[j] = owner[j];

  // Each rank's chunks in ascending order: sort (owner, chunk) ascending; every
  // rank holds exactly J chunks, so rank p's list is positions [pJ, pJ + J).
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    key[i] = i < n_chunks ? (long long)owner[i] : 0x7fffffffLL;
    idx[i] = i;
  }
  __syncthreads();
  bitonic_sort(key, idx, n, /*desc_key=*/false);
  for (int t = threadIdx.x; t < n_chunks; t += blockDim.x) rank_chunks[t] = idx[t];
}

}  // namespace

hipError_t launch_plan(const int64_t* s, const int64_t* a, int64_t n_blocks, int32_t B,
                       int64_t m, int32_t P, int32_t J, int64_t* cost, int32_t* owner,
                       int32_t* rank_chunks, int64_t* rank_load, hipStream_t stream) {
  const int n_chunks = P * J;
  hipLaunchKernelGGL(chunk_cost_kernel, dim3(n_chunks), dim3(kCostThreads), 0, stream, s, a,
                     n_blocks, (int64_t)B, m, cost);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(lpt_kernel, dim3(1), dim3(kLptThreads), 0, stream, cost, n_chunks, P, J,
                     owner, rank_chunks, rank_load);
  return hipGetLastError();
}

}  // namespace splitkv
