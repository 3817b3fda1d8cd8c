// Expert routing: scores, bias-adjusted top-k, sigmoid gates, usage counts, and the
// token permutation that groups (token, slot) pairs by expert.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dreamer {

constexpr int ROUTE_THREADS = 256;
constexpr int ROUTE_LDS_FLOATS = 16384;  // 64 KiB of biased scores per block

// z_e = rho * (u . key_e), u in LDS (float32), key in storage dtype; fixed summation order
// so that a recomputation gives the same bits.
template <typename T>
DEV float key_dot(const float* u, const T* key, int r) {
  float acc = 0.f;
  for (int i = 0; i < r; i += Vec16<T>::N) {
    float kv[Vec16<T>::N];
    load16(key + i, kv);
#pragma unroll
    for (int j = 0; j < Vec16<T>::N; ++j) acc = fmaf(u[i + j], kv[j], acc);
  }
  return acc;
}

// (value, index) ordering of the router: larger value first, then lower index.
DEV bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// One block handles TB tokens: depth-RoPE'd u rows into LDS, biased scores of all E
// experts into LDS, then per token k rounds of a wave-wide argmax.
template <typename T>
__global__ __launch_bounds__(ROUTE_THREADS) void route_kernel(
    int64_t Ttok, int r, int E, int k, int l, int L, int TB, const float* __restrict__ u,
    const T* __restrict__ keys, const float* __restrict__ bias, float rho, int normalize,
    const float* __restrict__ cs, const float* __restrict__ sn, int32_t* __restrict__ idx,
    float* __restrict__ gate, int32_t* __restrict__ counts) {
  extern __shared__ float smem[];
  float* us = smem;              // [TB, r]
  float* sc = smem + TB * r;     // [TB, E]
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * TB;
  const int nt = (int)min((int64_t)TB, Ttok - t0);
  const int half = r / 2, quarter = r / 4;

  // u rows with depth RoPE (pairs i < r/4 at depth l, the rest at L-1-l)
  for (int e = tid; e < nt * r; e += blockDim.x) {
    const int t = e / r, i = e % r;
    const float* ur = u + (t0 + t) * r;
    const int p = i < half ? i : i - half;
    const int pos = p < quarter ? l : L - 1 - l;
    const float cv = cs[pos * half + p], sv = sn[pos * half + p];
    const float x = ur[i], y = ur[i < half ? i + half : i - half];
    us[t * r + i] = i < half ? x * cv - y * sv : x * cv + y * sv;
  }
  __syncthreads();
  // biased scores
  for (int e = tid; e < E; e += blockDim.x) {
    const T* key = keys + (int64_t)e * r;
    const float be = bias[e];
    for (int t = 0; t < nt; ++t) sc[t * E + e] = rho * key_dot<T>(us + t * r, key, r) + be;
  }
  __syncthreads();
  // top-k per token, one wave per token
  const int lane = tid & 63, wv = tid >> 6, nw = blockDim.x >> 6;
  for (int t = wv; t < nt; t += nw) {
    float* row = sc + t * E;
    int isel[32];
    // lane-local best over experts lane, lane+64, ...
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int e = lane; e < E; e += 64)
      if (better(row[e], e, bv, bi)) { bv = row[e]; bi = e; }
    for (int j = 0; j < k; ++j) {
      float wvv = bv;
      int wi = bi;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {  // butterfly: every lane ends with the winner
        const float ov = __shfl_xor(wvv, o, 64);
        const int oi = __shfl_xor(wi, o, 64);
        if (better(ov, oi, wvv, wi)) { wvv = ov; wi = oi; }
      }
      isel[j] = wi;
      if ((wi & 63) == lane) {  // the owner marks it taken and rescans its slice
        row[wi] = -INFINITY;
        bv = -INFINITY;
        bi = 0x7fffffff;
        for (int e = lane; e < E; e += 64)
          if (row[e] != -INFINITY && better(row[e], e, bv, bi)) { bv = row[e]; bi = e; }
      }
    }
    // gates: sigmoid of the unbiased score, recomputed with the same dot product
    float gv = 0.f;
    int my = 0;
    if (lane < k) {
      for (int j = 0; j < k; ++j) my = j == lane ? isel[j] : my;
      const float z = rho * key_dot<T>(us + t * r, keys + (int64_t)my * r, r);
      gv = sigmoidf_(z);
    }
    const float gsum = wave_sum(gv);
    if (lane < k) {
      const int64_t o = (t0 + t) * k + lane;
      idx[o] = my;
      gate[o] = normalize ? gv / gsum : gv;
      if (counts) atomicAdd(&counts[my], 1);
    }
  }
}

// Replay of given expert choices: idx = idx_in, gates from this token's own scores with
// the same rotation and dot product as route_kernel.  One wave per token.
template <typename T>
__global__ __launch_bounds__(256) void route_forced_kernel(
    int64_t Ttok, int r, int k, int l, int L, const float* __restrict__ u,
    const T* __restrict__ keys, float rho, int normalize, const float* __restrict__ cs,
    const float* __restrict__ sn, const int32_t* __restrict__ idx_in,
    int32_t* __restrict__ idx, float* __restrict__ gate, int32_t* __restrict__ counts) {
  extern __shared__ float smem[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wv;
  if (t >= Ttok) return;
  float* us = smem + wv * r;
  const int half = r / 2, quarter = r / 4;
  const float* ur = u + t * r;
  for (int i = lane; i < r; i += 64) {
    const int p = i < half ? i : i - half;
    const int pos = p < quarter ? l : L - 1 - l;
    const float cv = cs[pos * half + p], sv = sn[pos * half + p];
    const float x = ur[i], y = ur[i < half ? i + half : i - half];
    us[i] = i < half ? x * cv - y * sv : x * cv + y * sv;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  float gv = 0.f;
  int e = 0;
  if (lane < k) {
    e = idx_in[t * k + lane];
    gv = sigmoidf_(rho * key_dot<T>(us, keys + (int64_t)e * r, r));
  }
  const float gsum = wave_sum(gv);
  if (lane < k) {
    idx[t * k + lane] = e;
    gate[t * k + lane] = normalize ? gv / gsum : gv;
    if (counts) atomicAdd(&counts[e], 1);
  }
}

int launch_route(int dtype, int64_t T, int r, int E, int k, int l, int L, const float* u,
                 const void* keys, const float* bias, float rho, int normalize,
                 const float* cos_r, const float* sin_r, int32_t* idx, float* gate,
                 int32_t* counts, const int32_t* idx_in, hipStream_t st) {
  if (T <= 0) return 0;
  if (k < 1 || k > 32 || k > E || E > ROUTE_LDS_FLOATS || r % 8) return -1;
  if (idx_in) {
    if (r > 1024) return -1;
    const unsigned grid = (unsigned)((T + 3) / 4);
    const size_t lds = 4 * (size_t)r * sizeof(float);
    if (dtype == DT_BF16)
      route_forced_kernel<bf16><<<grid, 256, lds, st>>>(T, r, k, l, L, u, (const bf16*)keys,
                                                        rho, normalize, cos_r, sin_r, idx_in,
                                                        idx, gate, counts);
    else
      route_forced_kernel<float><<<grid, 256, lds, st>>>(T, r, k, l, L, u, (const float*)keys,
                                                         rho, normalize, cos_r, sin_r, idx_in,
                                                         idx, gate, counts);
    return 0;
  }
  int TB = (ROUTE_LDS_FLOATS - 1024) / (E + r);
  TB = max(1, min(TB, 16));
  const size_t lds = (size_t)TB * (E + r) * sizeof(float);
  const unsigned grid = (unsigned)((T + TB - 1) / TB);
  if (dtype == DT_BF16)
    route_kernel<bf16><<<grid, ROUTE_THREADS, lds, st>>>(T, r, E, k, l, L, TB, u,
                                                         (const bf16*)keys, bias, rho,
                                                         normalize, cos_r, sin_r, idx, gate,
                                                         counts);
  else
    route_kernel<float><<<grid, ROUTE_THREADS, lds, st>>>(T, r, E, k, l, L, TB, u,
                                                          (const float*)keys, bias, rho,
                                                          normalize, cos_r, sin_r, idx, gate,
                                                          counts);
  return 0;
}

// ----------------------------------------------------------------------------- permute
__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

void launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st) {
  if (n <= 0) return;
  fill_i32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, n, v);
}

// Single block: exclusive scans of counts and of ceil(counts / tile_m).
__global__ __launch_bounds__(1024) void moe_scan_kernel(const int32_t* __restrict__ counts,
                                                        int E, int tile_m,
                                                        int32_t* __restrict__ goff,
                                                        int32_t* __restrict__ toff,
                                                        int32_t* __restrict__ cursor) {
  __shared__ int s_rows[1024], s_tiles[1024];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (E + nt - 1) / nt;
  const int e0 = tid * per, e1 = min(E, e0 + per);
  int rsum = 0, tsum = 0;
  for (int e = e0; e < e1; ++e) {
    const int c = counts[e];
    rsum += c;
    tsum += (c + tile_m - 1) / tile_m;
  }
  s_rows[tid] = rsum;
  s_tiles[tid] = tsum;
  __syncthreads();
  // Hillis-Steele inclusive scan over the per-thread sums
  for (int o = 1; o < nt; o <<= 1) {
    const int a = tid >= o ? s_rows[tid - o] : 0;
    const int b = tid >= o ? s_tiles[tid - o] : 0;
    __syncthreads();
    s_rows[tid] += a;
    s_tiles[tid] += b;
    __syncthreads();
  }
  int rr = s_rows[tid] - rsum, tt = s_tiles[tid] - tsum;  // exclusive prefixes
  for (int e = e0; e < e1; ++e) {
    goff[e] = rr;
    toff[e] = tt;
    cursor[e] = 0;
    const int c = counts[e];
    rr += c;
    tt += (c + tile_m - 1) / tile_m;
  }
  if (tid == nt - 1) {
    goff[E] = s_rows[nt - 1];
    toff[E] = s_tiles[nt - 1];
  }
}

void launch_moe_scan(const int32_t* counts, int E, int tile_m, int32_t* goff, int32_t* toff,
                     int32_t* cursor, hipStream_t st) {
  moe_scan_kernel<<<1, 1024, 0, st>>>(counts, E, tile_m, goff, toff, cursor);
}

__global__ void moe_histogram_kernel(const int32_t* __restrict__ idx, int64_t nslots,
                                     int32_t* __restrict__ counts) {
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s < nslots) atomicAdd(&counts[idx[s]], 1);
}

void launch_moe_histogram(const int32_t* idx, int64_t nslots, int32_t* counts, hipStream_t st) {
  if (nslots <= 0) return;
  moe_histogram_kernel<<<(unsigned)((nslots + 255) / 256), 256, 0, st>>>(idx, nslots, counts);
}

__global__ void moe_scatter_kernel(const int32_t* __restrict__ idx, int64_t nslots,
                                   const int32_t* __restrict__ goff,
                                   int32_t* __restrict__ cursor, int32_t* __restrict__ perm) {
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= nslots) return;
  const int e = idx[s];
  const int pos = goff[e] + atomicAdd(&cursor[e], 1);
  perm[pos] = (int32_t)s;
}

void launch_moe_scatter(const int32_t* idx, int64_t nslots, const int32_t* goff,
                        int32_t* cursor, int32_t* perm, hipStream_t st) {
  if (nslots <= 0) return;
  moe_scatter_kernel<<<(unsigned)((nslots + 255) / 256), 256, 0, st>>>(idx, nslots, goff,
                                                                       cursor, perm);
}

}  // namespace dreamer
