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

// Position-based assignments (Zigzag of §3.3 / Figure 5(b); the contiguous
// "No balance" split of §5.5). One workgroup per range prices it like Eq. 6
// (overlap of every anchor window with the range, times B); a second kernel
// sums each rank's ranges. Range order and ownership are those of the entry
// point's contract.
__global__ void __launch_bounds__(kCostThreads)
range_cost_kernel(const int64_t* __restrict__ s, const int64_t* __restrict__ a, int64_t n_blocks,
                  int64_t B, int strategy, int P, int64_t S, BaselineSamples smp,
                  int64_t* __restrict__ range_cost) {
  const int64_t r = blockIdx.x;
  int64_t lo, width;
  if (strategy == SPLITKV_BASELINE_NO_BALANCE) {
    width = S / P;
    lo = r * width;
  } else {
    const int u = (int)(r / (2 * P));
    const int c = (int)(r % (2 * P));
    width = smp.len[u] / (2 * P);
    lo = smp.start[u] + (int64_t)c * width;
  }
  const int64_t hi = lo + width;
  long long t = 0;
  for (int64_t i = threadIdx.x; i < n_blocks; i += kCostThreads) {
    const int64_t x0 = max(s[i], lo), x1 = min(a[i], hi);
    if (x1 > x0) t += x1 - x0;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off);
  __shared__ long long part[kCostThreads / kWave];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  if (lane == 0) part[wave] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    long long c = 0;
    for (int w = 0; w < kCostThreads / kWave; ++w) c += part[w];
    range_cost[r] = B * c;
  }
}

__global__ void __launch_bounds__(kCostThreads)
rank_sum_kernel(const int64_t* __restrict__ range_cost, int strategy, int P, int n_samples,
                int64_t* __restrict__ rank_load) {
  const int p = blockIdx.x * kCostThreads + threadIdx.x;
  if (p >= P) return;
  long long load = 0;
  if (strategy == SPLITKV_BASELINE_NO_BALANCE) {
    load = range_cost[p];
  } else {
    for (int u = 0; u < n_samples; ++u)
      load += range_cost[(int64_t)u * 2 * P + p] + range_cost[(int64_t)u * 2 * P + 2 * P - 1 - p];
  }
  rank_load[p] = load;
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

// Greedy keys: a rank's (load, rank) pair packed as load * 1024 + rank, so the
// lexicographic minimum (least load, then lowest rank) is the integer minimum.
// Loads stay below 2^53 (the host checks B * N * S, which bounds any chunk
// total, since every overlap is clipped to its chunk), so keys fit in 63 bits.
constexpr int kRankBits = 10;
constexpr unsigned long long kNoKey = ~0ull;

template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_min_step(unsigned long long v) {
  const int lo = (int)(unsigned)v, hi = (int)(unsigned)(v >> 32);
  const unsigned olo = (unsigned)__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xF, 0xF, false);
  const unsigned ohi = (unsigned)__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xF, 0xF, false);
  const unsigned long long o = ((unsigned long long)ohi << 32) | olo;
  return o < v ? o : v;
}

__device__ __forceinline__ unsigned long long lane_value(unsigned long long v, int lane) {
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(v >> 32), lane);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)v, lane);
  return ((unsigned long long)hi << 32) | lo;
}

// Every lane takes the value of the next lane up (wave-wide DPP shift); the
// last lane keeps its own.
__device__ __forceinline__ unsigned long long wave_shift_down(unsigned long long v) {
  const int lo = (int)(unsigned)v, hi = (int)(unsigned)(v >> 32);
  const unsigned slo = (unsigned)__builtin_amdgcn_update_dpp(lo, lo, 0x130, 0xF, 0xF, false);
  const unsigned shi = (unsigned)__builtin_amdgcn_update_dpp(hi, hi, 0x130, 0xF, 0xF, false);
  return ((unsigned long long)shi << 32) | slo;
}

// Minimum key of the wave, returned as a wave-uniform value: minima of lane
// quads (two quad permutations), of 8 lanes (half-row mirror) and of 16 lanes
// (row mirror) through DPP, then the four row minima read out.
__device__ __forceinline__ unsigned long long wave_min_key(unsigned long long v) {
  v = dpp_min_step<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_min_step<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_min_step<0x141>(v);  // row_half_mirror
  v = dpp_min_step<0x140>(v);  // row_mirror
  unsigned long long r0 = lane_value(v, 0), r1 = lane_value(v, 16);
  unsigned long long r2 = lane_value(v, 32), r3 = lane_value(v, 48);
  r0 = r0 < r1 ? r0 : r1;
  r2 = r2 < r3 ? r2 : r3;
  return r0 < r2 ? r0 : r2;
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
  __shared__ unsigned long long best_key[2][kLptThreads / kWave];

  int n = 1;
  while (n < n_chunks) n <<= 1;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    key[i] = i < n_chunks ? (long long)cost[i] : -1;  // padding sorts last (costs >= 0)
    idx[i] = i;
  }
  __syncthreads();
  bitonic_sort(key, idx, n, /*desc_key=*/true);

  // Greedy: thread p keeps rank p's load and chunk count. The sorted costs are
  // taken 64 at a time into a register (lane k holds step t0 + k) and read out
  // as uniform values; step t0 + k's owner is kept by lane k and written once
  // per 64 steps.
  const int p = threadIdx.x;
  const int lane = p % kWave, wave = p / kWave;
  const int n_waves = (P + kWave - 1) / kWave;
  long long load = 0;
  int held = 0;
  if (n_waves == 1) {
    // P <= 64: the wave also keeps the ranks in order, lane l holding the l-th
    // smallest key (ranks with J chunks hold kNoKey, at the end). The least
    // loaded open rank is lane 0; after it takes the chunk its new key is put
    // back at the slot given by the number of keys below it, the lanes before
    // that slot moving up by one.
    if (wave == 0) {
      unsigned long long sk = lane < P ? (unsigned long long)lane : kNoKey;  // all loads 0
      for (int t0 = 0; t0 < n_chunks; t0 += kWave) {
        const int cnt = min(kWave, n_chunks - t0);
        const long long kv = lane < cnt ? key[t0 + lane] : 0;
        int my_owner = 0;
        for (int k = 0; k < cnt; ++k) {
          const unsigned long long up = wave_shift_down(sk);  // lane l: key of lane l + 1
          const unsigned long long front = lane_value(sk, 0);
          const int r = (int)(front & ((1u << kRankBits) - 1));
          const long long kt = (long long)lane_value((unsigned long long)kv, k);
          if (lane == r) { load += kt; held += 1; }
          const int held_r = __builtin_amdgcn_readlane(held, r);
          const unsigned long long nk =
              held_r < J ? ((((front >> kRankBits) + (unsigned long long)kt) << kRankBits) |
                            (unsigned)r)
                         : kNoKey;
          const int pos = __builtin_popcountll(__builtin_amdgcn_ballot_w64(sk < nk) & ~1ull);
          sk = lane < pos ? up : (lane == pos ? nk : sk);
          if (lane == k) my_owner = r;
        }
        if (lane < cnt) owner[idx[t0 + lane]] = my_owner;
      }
    }
  } else {
    // P > 64: a lexicographic (load, rank) argmin over all ranks per step.
    for (int t0 = 0; t0 < n_chunks; t0 += kWave) {
      const int cnt = min(kWave, n_chunks - t0);
      const long long kv = lane < cnt ? key[t0 + lane] : 0;
      int my_owner = 0;
      for (int k = 0; k < cnt; ++k) {
        const unsigned long long cand =
            (p < P && held < J) ? ((unsigned long long)load << kRankBits) | (unsigned)p : kNoKey;
        const int buf = k & 1;
        const unsigned long long wbest = wave_min_key(cand);  // whole wave, before the lane test
        if (lane == 0) best_key[buf][wave] = wbest;
        __syncthreads();
        unsigned long long b = best_key[buf][0];
        for (int w = 1; w < n_waves; ++w) {
          const unsigned long long o = best_key[buf][w];
          b = o < b ? o : b;
        }
        const int r = (int)(b & ((1u << kRankBits) - 1));
        const long long kt = (long long)lane_value((unsigned long long)kv, k);
        if (p == r) { load += kt; held += 1; }
        if (lane == k) my_owner = r;
      }
      if (wave == 0 && lane < cnt) owner[idx[t0 + lane]] = my_owner;
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

// Locality matching (§4.2): the bundles of a plan are placed on physical
// ranks without changing any load, keeping as many context rows where they
// already are as possible. Before the step's all-to-all, physical rank r holds
// the r-th of P equal contiguous parts of [0, S) (S = P J m), i.e. chunks
// r J .. r J + J - 1; placing bundle b on rank r keeps
//   keep(b, r) = m * #{ chunks of b whose home is r }
// rows. The best placement is a linear assignment problem, solved exactly by
// the Hungarian method on the cost c(b, r) = J - keep(b, r) / m in [0, J]
// (the constant and the unit leave the best placement unchanged), with row
// (bundle) and column (rank) potentials, u(b) + v(r) <= c(b, r) everywhere and
// equality on placed pairs.
//
// Greedy start (column reduction): v(r) is the least cost in column r, and the
// bundle that attains it (lowest on ties) takes the column unless a lower
// column claims it too; all u start at 0, so the potentials are feasible and
// the placed pairs tight. Every bundle left over then enters along a shortest
// augmenting path: one Dijkstra-like scan per step over the free columns,
// potentials moved by the step's least slack.
//
// One wave. Lane l keeps, in registers, column l + 1 + 64 k and row
// l + 1 + 64 k (k < SLOTS, SLOTS = ceil(P / 64)): the column's potential,
// slack (minv), predecessor (way), used flag and matched row, and the row's
// potential and tree flag (a row is in the tree once the column it is matched
// to is used; those rows take + delta, the used columns - delta). The keep
// counts sit in LDS as a [P][P] table. A step scans the lane's unused columns
// and packs (slack, taken, column) into one 32-bit key whose wave minimum (DPP
// steps and four lane reads) is the smallest slack, among equal slacks a
// column no bundle holds yet (the path then ends at once: with costs in
// [0, J] ties are the rule, and at P = 64 this cuts the steps tenfold), then
// the lowest column: the result is unique. A free column
// keeps its starting potential (0 <= v <= J), so an entering bundle's path is
// at most J long and every potential moves by at most J per augmentation:
// slacks stay below 3 (P + 1) J <= 2^14 and keys below 2^24. Single values of
// other lanes are read with readlane at a uniform lane. Chunk ids outside
// [0, P J) count as neither kept nor sent.
constexpr int kMatchThreads = kWave;
constexpr int kColBits = 9;  // columns 1 .. 256 in the low bits of a wave-minimum key
constexpr unsigned kNoKey32 = 0xffffffffu;
constexpr int kMatchInf = 1 << 30;
static_assert(kMaxMatchRanks < (1 << kColBits), "column must fit its key bits");

template <int CTRL>
__device__ __forceinline__ unsigned dpp_min_step32(unsigned v) {
  const unsigned o = (unsigned)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
  return o < v ? o : v;
}

// Wave minimum of a 32-bit key, wave-uniform (as wave_min_key).
__device__ __forceinline__ unsigned wave_min_u32(unsigned v) {
  v = dpp_min_step32<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_min_step32<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_min_step32<0x141>(v);  // row_half_mirror
  v = dpp_min_step32<0x140>(v);  // row_mirror
  const unsigned r0 = (unsigned)__builtin_amdgcn_readlane((int)v, 0);
  const unsigned r1 = (unsigned)__builtin_amdgcn_readlane((int)v, 16);
  const unsigned r2 = (unsigned)__builtin_amdgcn_readlane((int)v, 32);
  const unsigned r3 = (unsigned)__builtin_amdgcn_readlane((int)v, 48);
  return min(min(r0, r1), min(r2, r3));
}

template <int SLOTS>
__global__ void __launch_bounds__(kMatchThreads)
locality_match_kernel(const int32_t* __restrict__ bundles, int P, int J, int64_t m,
                      int32_t* __restrict__ perm, int64_t* __restrict__ send,
                      int64_t* __restrict__ kept_moved) {
  __shared__ int32_t bl[kMaxPlanChunks];
  __shared__ uint16_t keepc[kMaxMatchRanks * kMaxMatchRanks];  // [bundle][home rank] chunk counts
  __shared__ int32_t placed[kMaxMatchRanks];
  __shared__ int32_t claim[kMaxMatchRanks];  // greedy start: lowest column taking each bundle
  const int lane = threadIdx.x;
  const int PJ = P * J;
  for (int x = lane; x < PJ; x += kMatchThreads) bl[x] = bundles[x];
  for (int x = lane; x < P * P; x += kMatchThreads) keepc[x] = 0;
  for (int x = lane; x < P; x += kMatchThreads) { placed[x] = x; claim[x] = 0x7fffffff; }
  __syncthreads();
  for (int bb = lane; bb < P; bb += kMatchThreads)  // lane owns row bb of the table
    for (int k = 0; k < J; ++k) {
      const int j = bl[bb * J + k];
      if (j >= 0 && j < PJ) keepc[bb * P + j / J] += 1;
    }
  __syncthreads();
  // cost of bundle i on rank c (both 1-based)
  auto cost = [&](int i, int c) { return J - (int)keepc[(i - 1) * P + (c - 1)]; };

  int v[SLOTS], minv[SLOTS], u[SLOTS], way[SLOTS], match[SLOTS], cand[SLOTS];
  bool used[SLOTS], tree[SLOTS];
  // ---- greedy start: column reduction ----
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) {
    const int c = lane + 1 + kWave * k;
    v[k] = 0; u[k] = 0; match[k] = 0; way[k] = 0; cand[k] = 0;
    if (c <= P) {
      int best = kMatchInf;
      for (int i = 1; i <= P; ++i) {
        const int ci = cost(i, c);
        if (ci < best) { best = ci; cand[k] = i; }
      }
      v[k] = best;
      atomicMin(&claim[cand[k] - 1], c);
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) {
    const int c = lane + 1 + kWave * k;
    if (c <= P && claim[cand[k] - 1] == c) match[k] = cand[k];
  }

  // value of register array x for global index g (1-based), read from its lane
  auto lane_of = [](int g) { return (g - 1) % kWave; };
  auto slot_of = [](int g) { return (g - 1) / kWave; };
  auto read_i = [&](const int (&x)[SLOTS], int g) {
    int val = x[0];
    if constexpr (SLOTS > 1) {
      const int k = slot_of(g);
#pragma unroll
      for (int q = 1; q < SLOTS; ++q) val = (k == q) ? x[q] : val;
    }
    return __builtin_amdgcn_readlane(val, lane_of(g));
  };

  // ---- the bundles left over enter one at a time ----
  for (int i = 1; i <= P; ++i) {
    if (claim[i - 1] != 0x7fffffff) continue;  // placed by the greedy start (uniform)
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) { minv[k] = kMatchInf; used[k] = false; tree[k] = false; }
    int j0 = 0;
    // at most P steps: every step uses up one more of the P real columns
    for (int step = 0; step <= P; ++step) {
      const int i0 = j0 == 0 ? i : read_i(match, j0);
#pragma unroll
      for (int k = 0; k < SLOTS; ++k) {
        if (j0 != 0 && lane == lane_of(j0) && k == slot_of(j0)) used[k] = true;
        if (lane == lane_of(i0) && k == slot_of(i0)) tree[k] = true;
      }
      const int ui0 = read_i(u, i0);
      unsigned key = kNoKey32;
#pragma unroll
      for (int k = 0; k < SLOTS; ++k) {
        const int c = lane + 1 + kWave * k;
        if (c > P || used[k]) continue;
        const int cur = cost(i0, c) - ui0 - v[k];
        if (cur < minv[k]) { minv[k] = cur; way[k] = j0; }
        const unsigned taken = match[k] != 0 ? (1u << kColBits) : 0u;
        key = min(key, ((unsigned)minv[k] << (kColBits + 1)) | taken | (unsigned)c);
      }
      const unsigned wkey = wave_min_u32(key);
      const int delta = (int)(wkey >> (kColBits + 1));
      const int col = wkey == kNoKey32 ? 0x7fffffff : (int)(wkey & ((1u << kColBits) - 1));
#pragma unroll
      for (int k = 0; k < SLOTS; ++k) {
        const int c = lane + 1 + kWave * k;
        if (c <= P) {
          if (used[k]) v[k] -= delta;
          else minv[k] -= delta;
          if (tree[k]) u[k] += delta;
        }
      }
      j0 = col;
      if (j0 > P || read_i(match, j0) == 0) break;
    }
    // flip the augmenting path back to column 0: p[j0] = p[way[j0]]
    for (int step = 0; step <= P && j0 >= 1 && j0 <= P; ++step) {
      const int j1 = read_i(way, j0);
      const int row = j1 == 0 ? i : read_i(match, j1);
#pragma unroll
      for (int k = 0; k < SLOTS; ++k)
        if (lane == lane_of(j0) && k == slot_of(j0)) match[k] = row;
      j0 = j1;
    }
  }

#pragma unroll
  for (int k = 0; k < SLOTS; ++k) {
    const int c = lane + 1 + kWave * k;
    const int b = match[k] - 1;  // the matching is perfect: every bundle is placed once
    if (c <= P && b >= 0 && b < P) placed[b] = c - 1;
  }
  for (int x = lane; x < P * P; x += kMatchThreads) send[x] = 0;
  __syncthreads();
  long long kept = 0;
  for (int b = lane; b < P; b += kMatchThreads) {
    const int dst = placed[b];
    perm[b] = dst;
    kept += (long long)keepc[b * P + dst] * m;
    for (int k = 0; k < J; ++k) {  // the lane placing bundle b owns column dst of send
      const int j = bl[b * J + k];
      if (j < 0 || j >= PJ) continue;
      const int src = j / J;
      if (src != dst) send[(int64_t)src * P + dst] += m;
    }
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) kept += __shfl_xor(kept, off);
  if (lane == 0) {
    kept_moved[0] = kept;
    kept_moved[1] = (long long)PJ * m - kept;
  }
}

}  // namespace

hipError_t launch_locality_match(const int32_t* rank_chunks, int32_t P, int32_t J, int64_t m,
                                 int32_t* phys_rank, int64_t* send_rows, int64_t* kept_moved,
                                 hipStream_t stream) {
  auto kern = P <= kWave       ? locality_match_kernel<1>
              : P <= 2 * kWave ? locality_match_kernel<2>
                               : locality_match_kernel<kMaxMatchRanks / kWave>;
  hipLaunchKernelGGL(kern, dim3(1), dim3(kMatchThreads), 0, stream, rank_chunks, P, J, m,
                     phys_rank, send_rows, kept_moved);
  return hipGetLastError();
}

hipError_t launch_plan_baseline(int strategy, const int64_t* s, const int64_t* a,
                                int64_t n_blocks, int32_t B, const BaselineSamples& samples,
                                int32_t P, int64_t S, int64_t* range_cost, int64_t* rank_load,
                                hipStream_t stream) {
  const int64_t n_ranges =
      strategy == SPLITKV_BASELINE_NO_BALANCE ? P : 2 * (int64_t)P * samples.n;
  hipLaunchKernelGGL(range_cost_kernel, dim3((unsigned)n_ranges), dim3(kCostThreads), 0, stream,
                     s, a, n_blocks, (int64_t)B, strategy, P, S, samples, range_cost);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(rank_sum_kernel, dim3((P + kCostThreads - 1) / kCostThreads),
                     dim3(kCostThreads), 0, stream, range_cost, strategy, P, samples.n,
                     rank_load);
  return hipGetLastError();
}

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
