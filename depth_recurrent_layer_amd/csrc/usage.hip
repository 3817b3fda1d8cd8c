// Expert-load bookkeeping around the router: selection counts per depth, the balancing
// update of the router bias, and usage statistics of the counts.
//
// counts: one block per (set, chunk of slots) builds an LDS histogram and adds its nonzero
// bins to the set's counts (at most one global atomic per bin and chunk).
// bias update: one block; the median of the counts comes from two order statistics found
// by bisection on the count value (a block-wide count of N_e <= v per step).
// usage: one block per set; distinct experts, max / mean and the Gini coefficient from the
// exact integer sum of |N_i - N_j| over all pairs.
#include "common.h"
#include "kernels.h"

namespace dreamer {

constexpr int COUNT_CHUNK = 8192;

__global__ __launch_bounds__(512) void route_counts_kernel(const int32_t* __restrict__ idx,
                                                          int64_t per_set, int E,
                                                          int32_t* __restrict__ counts) {
  extern __shared__ int lh[];
  const int set = blockIdx.y;
  for (int e = threadIdx.x; e < E; e += blockDim.x) lh[e] = 0;
  __syncthreads();
  const int32_t* src = idx + (int64_t)set * per_set;
  const int64_t s0 = (int64_t)blockIdx.x * COUNT_CHUNK;
  const int64_t s1 = min(s0 + COUNT_CHUNK, per_set);
  for (int64_t s = s0 + threadIdx.x; s < s1; s += blockDim.x)
    atomicAdd(&lh[min(max(src[s], 0), E - 1)], 1);
  __syncthreads();
  int32_t* out = counts + (int64_t)set * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    if (lh[e]) atomicAdd(&out[e], lh[e]);
}

int launch_route_counts(const int32_t* idx, int64_t n_sets, int64_t per_set, int E,
                        int32_t* counts, hipStream_t st) {
  if (E <= 0 || E > COUNT_MAX_E || n_sets <= 0 || n_sets > 65535) return -1;
  launch_fill_i32(counts, n_sets * E, 0, st);
  if (per_set <= 0) return 0;
  const dim3 grid((unsigned)((per_set + COUNT_CHUNK - 1) / COUNT_CHUNK), (unsigned)n_sets);
  dlaunch(route_counts_kernel, grid, 512, (size_t)E * sizeof(int), st, idx, per_set, E, counts);
  return 0;
}

// Block-wide sum of an int64 over 1024 threads (red: 16 slots).
DEV long long block_sum_i64(long long v, long long* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  long long s = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
  return s;
}

// The k-th smallest count (0-based) by bisection on the value.
DEV int kth_smallest(const int32_t* __restrict__ c, int E, int k, int hi, long long* red) {
  int lo = 0;
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    long long n = 0;
    for (int e = threadIdx.x; e < E; e += blockDim.x) n += c[e] <= mid;
    n = block_sum_i64(n, red);
    if (n >= k + 1) hi = mid; else lo = mid + 1;
  }
  return lo;
}

__global__ __launch_bounds__(1024) void bias_update_kernel(const int32_t* __restrict__ c, int E,
                                                          float lam, float* __restrict__ bias) {
  __shared__ long long red[16];
  __shared__ int s_max;
  if (threadIdx.x == 0) s_max = 0;
  __syncthreads();
  int m = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) m = max(m, c[e]);
  atomicMax(&s_max, m);
  __syncthreads();
  const int hi = s_max;
  // median: the middle order statistic, or the mean of the two middle ones (exact in
  // double for integer counts)
  const int a = kth_smallest(c, E, (E - 1) / 2, hi, red);
  const int b = E % 2 ? a : kth_smallest(c, E, E / 2, hi, red);
  const double med = 0.5 * ((double)a + (double)b);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const double d = med - (double)c[e];
    const float sgn = d > 0 ? 1.f : (d < 0 ? -1.f : 0.f);
    bias[e] = bias[e] + lam * sgn;
  }
}

void launch_bias_update(const int32_t* counts, int E, float lam, float* bias, hipStream_t st) {
  if (E <= 0) return;
  dlaunch(bias_update_kernel, 1, 1024, 0, st, counts, E, lam, bias);
}

// stats[set] = {distinct experts, max / mean, Gini}
__global__ __launch_bounds__(1024) void usage_kernel(const int32_t* __restrict__ counts, int E,
                                                    float* __restrict__ stats) {
  extern __shared__ int c[];  // [E]
  __shared__ long long red[16];
  const int32_t* src = counts + (int64_t)blockIdx.x * E;
  long long distinct = 0, total = 0, mx = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int v = src[e];
    c[e] = v;
    distinct += v > 0;
    total += v;
    mx = max(mx, (long long)v);
  }
  __shared__ int s_max;
  if (threadIdx.x == 0) s_max = 0;
  distinct = block_sum_i64(distinct, red);  // (its barriers also order s_max's init)
  total = block_sum_i64(total, red);
  atomicMax(&s_max, (int)mx);
  // sum over ordered pairs of |N_i - N_j| (exact in int64)
  long long pairs = 0;
  for (int i = threadIdx.x; i < E; i += blockDim.x) {
    const int ci = c[i];
    for (int j = 0; j < E; ++j) pairs += ci > c[j] ? ci - c[j] : c[j] - ci;
  }
  pairs = block_sum_i64(pairs, red);
  if (threadIdx.x == 0) {
    float* o = stats + (int64_t)blockIdx.x * 3;
    o[0] = (float)distinct;
    const double mean = (double)total / E;
    o[1] = total > 0 ? (float)((double)s_max / mean) : 0.f;
    o[2] = total > 0 ? (float)((double)pairs / (2.0 * E * (double)total)) : 0.f;
  }
}

int launch_expert_usage(const int32_t* counts, int64_t n_sets, int E, float* stats,
                        hipStream_t st) {
  if (E <= 0 || E > PERM_MAX_E || n_sets <= 0 || n_sets > 65535) return -1;
  dlaunch(usage_kernel, (unsigned)n_sets, 1024, (size_t)E * sizeof(int), st, counts, E, stats);
  return 0;
}

}  // namespace dreamer
