// Expert routing: scores, bias-adjusted top-k, sigmoid gates, and the permutation that
// groups (token, slot) pairs by expert.
//
// bf16 scores: one block per 16 tokens.  u = x W_r^T on MFMA (bf16 x bf16 products are
// exact in float32), depth RoPE on u in float32, then z = rho * u_rot . keys with u_rot
// split into three bf16 parts (hi + mid + lo carries 24 mantissa bits) so the scores keep
// float32 accuracy on MFMA.  Scores go to a [T, E] float32 buffer; the top-k kernel
// (one wave per token) reads them, ranks by z + b and takes gates from z.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dreamer {

// ------------------------------------------------------------------ scores (bf16, MFMA)
template <int NKS>  // r = 32 * NKS
__global__ __launch_bounds__(256) void router_scores_bf16_kernel(
    int64_t Ttok, int h, int r, int E, int l, int L, const bf16* __restrict__ x, int64_t ldx,
    const bf16* __restrict__ w_r, const bf16* __restrict__ keys, float rho,
    const float* __restrict__ cs, const float* __restrict__ sn, float* __restrict__ z) {
  extern __shared__ float smem[];
  float* us = smem;            // [16, r] u
  float* ur = smem + 16 * r;   // [16, r] rotated u
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  const bf16x8 zero8 = {};
  // u tile [16 tokens x r]: wave w owns rank columns 16 nt, nt = w, w + 4, ...
  const int64_t tr = t0 + lr;
  const bf16* xrow = tr < Ttok ? x + tr * ldx + lg * 8 : nullptr;
  for (int nt = w; nt < r / 16; nt += 4) {
    const bf16* wrow = w_r + (int64_t)(nt * 16 + lr) * h + lg * 8;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < h; k0 += 32) {
      const bf16x8 af = xrow ? *reinterpret_cast<const bf16x8*>(xrow + k0) : zero8;
      const bf16x8 bf = *reinterpret_cast<const bf16x8*>(wrow + k0);
      acc = mfma16(af, bf, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) us[(lg * 4 + i) * r + nt * 16 + lr] = acc[i];
  }
  __syncthreads();
  // depth RoPE: pairs i < r/4 at depth l, the others at L-1-l
  const int half = r / 2, quarter = r / 4;
  for (int e = tid; e < 16 * r; e += 256) {
    const int t = e / r, i = e % r;
    const int p = i < half ? i : i - half;
    const int pos = p < quarter ? l : L - 1 - l;
    const float cv = cs[pos * half + p], sv = sn[pos * half + p];
    const float a = us[t * r + i], b = us[t * r + (i < half ? i + half : i - half)];
    ur[e] = i < half ? a * cv - b * sv : a * cv + b * sv;
  }
  __syncthreads();
  // three-part bf16 split of the rotated u rows (A operand: token lr, k-group lg)
  bf16x8 ah[NKS], am[NKS], al[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = ur[lr * r + ks * 32 + lg * 8 + j];
      const bf16 hi = (bf16)v;
      const float r1 = v - (float)hi;
      const bf16 mid = (bf16)r1;
      ah[ks][j] = hi;
      am[ks][j] = mid;
      al[ks][j] = (bf16)(r1 - (float)mid);
    }
  }
  // scores: wave w takes expert tiles et = w, w + 4, ...
  for (int et = w; et < E / 16; et += 4) {
    const bf16* krow = keys + (int64_t)(et * 16 + lr) * r + lg * 8;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 bk = *reinterpret_cast<const bf16x8*>(krow + ks * 32);
      acc = mfma16(ah[ks], bk, acc);
      acc = mfma16(am[ks], bk, acc);
      acc = mfma16(al[ks], bk, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = t0 + lg * 4 + i;
      if (t < Ttok) z[t * E + et * 16 + lr] = rho * acc[i];
    }
  }
}

// ------------------------------------------------------------------- scores (float32)
// One thread per (token, expert): u rotated on the fly, plain float32 FMAs.
__global__ void router_scores_f32_kernel(int64_t Ttok, int r, int E, int l, int L,
                                         const float* __restrict__ u,
                                         const float* __restrict__ keys, float rho,
                                         const float* __restrict__ cs,
                                         const float* __restrict__ sn, float* __restrict__ z) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= Ttok * E) return;
  const int64_t t = gid / E;
  const int e = (int)(gid % E);
  const float* ut = u + t * r;
  const float* ke = keys + (int64_t)e * r;
  const int half = r / 2, quarter = r / 4;
  float acc = 0.f;
  for (int i = 0; i < r; ++i) {
    const int p = i < half ? i : i - half;
    const int pos = p < quarter ? l : L - 1 - l;
    const float cv = cs[pos * half + p], sv = sn[pos * half + p];
    const float a = ut[i], b = ut[i < half ? i + half : i - half];
    acc = fmaf(i < half ? a * cv - b * sv : a * cv + b * sv, ke[i], acc);
  }
  z[gid] = rho * acc;
}

// ------------------------------------------------------------------------------- top-k
// (value, index) order of the router: larger value first, then lower index.
DEV bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

// One wave per token.  Each lane keeps a sorted list of its KMAX best (z + b, e) over
// experts lane, lane + 64, ...; k rounds of a butterfly argmax pop the heads.  Gates are
// sigmoid(z) of the winners, divided by their sum when normalising.  With idx_in the
// given experts are adopted instead.
template <int KMAX>
__global__ __launch_bounds__(256) void router_topk_kernel(
    int64_t Ttok, int E, int k, const float* __restrict__ z, const float* __restrict__ bias,
    int normalize, const int32_t* __restrict__ idx_in, int32_t* __restrict__ idx,
    float* __restrict__ gate) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Ttok) return;
  const float* zt = z + t * E;
  int my = 0;
  if (idx_in) {
    if (lane < k) my = idx_in[t * k + lane];
  } else {
    float lv[KMAX];
    int li[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) { lv[j] = -INFINITY; li[j] = 0x7fffffff; }
    for (int e = lane; e < E; e += 64) {
      const float v = zt[e] + bias[e];
      if (!better(v, e, lv[KMAX - 1], li[KMAX - 1])) continue;
      // insert into the sorted list (unrolled bubble from the tail)
      float cv = v;
      int ci = e;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (better(cv, ci, lv[j], li[j])) {
          const float tv = lv[j];
          const int ti = li[j];
          lv[j] = cv;
          li[j] = ci;
          cv = tv;
          ci = ti;
        }
      }
    }
    for (int j = 0; j < k; ++j) {
      float bv = lv[0];
      int bi = li[0];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {  // every lane ends with the winner
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if (lane == j) my = bi;
      if (li[0] == bi) {  // the owner pops its head
#pragma unroll
        for (int q = 0; q < KMAX - 1; ++q) { lv[q] = lv[q + 1]; li[q] = li[q + 1]; }
        lv[KMAX - 1] = -INFINITY;
        li[KMAX - 1] = 0x7fffffff;
      }
    }
  }
  float gv = 0.f;
  if (lane < k) gv = sigmoidf_(zt[my]);
  const float gsum = wave_sum(gv);
  if (lane < k) {
    idx[t * k + lane] = my;
    gate[t * k + lane] = normalize ? gv / gsum : gv;
  }
}

int router_scores(int dtype, int64_t T, int h, int r, int E, int l, int L, const void* x,
                  int64_t ldx, const void* w_r, const float* u, const void* keys, float rho,
                  const float* cos_r, const float* sin_r, float* z, hipStream_t st) {
  if (T <= 0) return 0;
  if (dtype == DT_BF16) {
    if (r % 32 || r > 256 || E % 16 || h % 32) return -1;
    const unsigned grid = (unsigned)((T + 15) / 16);
    const size_t lds = 2 * 16 * r * sizeof(float);
#define RS_CASE(NK)                                                                      \
  router_scores_bf16_kernel<NK><<<grid, 256, lds, st>>>(T, h, r, E, l, L, (const bf16*)x, \
                                                        ldx, (const bf16*)w_r,            \
                                                        (const bf16*)keys, rho, cos_r, sin_r, z)
    switch (r / 32) {
      case 1: RS_CASE(1); break;
      case 2: RS_CASE(2); break;
      case 4: RS_CASE(4); break;
      case 8: RS_CASE(8); break;
      default: return -1;
    }
#undef RS_CASE
  } else {
    const int64_t n = T * E;
    router_scores_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
        T, r, E, l, L, u, (const float*)keys, rho, cos_r, sin_r, z);
  }
  return 0;
}

int router_topk(int64_t T, int E, int k, const float* z, const float* bias, int normalize,
                const int32_t* idx_in, int32_t* idx, float* gate, hipStream_t st) {
  if (T <= 0) return 0;
  if (k < 1 || k > 32 || k > E) return -1;
  const unsigned grid = (unsigned)((T + 3) / 4);
#define TK_CASE(KM) \
  router_topk_kernel<KM><<<grid, 256, 0, st>>>(T, E, k, z, bias, normalize, idx_in, idx, gate)
  if (k <= 1) TK_CASE(1);
  else if (k <= 2) TK_CASE(2);
  else if (k <= 4) TK_CASE(4);
  else if (k <= 8) TK_CASE(8);
  else if (k <= 16) TK_CASE(16);
  else TK_CASE(32);
#undef TK_CASE
  return 0;
}

// ----------------------------------------------------------------------------- permute
// Slots are cut into blocks of PERM_CHUNK; per block an LDS histogram over experts, then
// one column scan gives every (block, expert) its base position, and the scatter hands
// out positions with LDS atomics.  No global atomics.
__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

void launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st) {
  if (n <= 0) return;
  fill_i32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, n, v);
}

__global__ __launch_bounds__(1024) void perm_count_kernel(const int32_t* __restrict__ idx,
                                                         int64_t nslots, int E,
                                                         int32_t* __restrict__ hist) {
  extern __shared__ int lh[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) lh[e] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)blockIdx.x * PERM_CHUNK;
  const int64_t s1 = min(s0 + PERM_CHUNK, nslots);
  for (int64_t s = s0 + threadIdx.x; s < s1; s += blockDim.x) atomicAdd(&lh[idx[s]], 1);
  __syncthreads();
  int32_t* out = hist + (int64_t)blockIdx.x * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) out[e] = lh[e];
}

// Single block.  hist [nb, E] -> base [nb, E] (in place, absolute positions); counts,
// goff, toff over experts.
__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t* __restrict__ hist, int nb,
                                                        int E, int tile_m,
                                                        int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ goff,
                                                        int32_t* __restrict__ toff) {
  __shared__ int s_rows[1024], s_tiles[1024];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (E + nt - 1) / nt;
  const int e0 = tid * per, e1 = min(E, e0 + per);
  int rsum = 0, tsum = 0;
  for (int e = e0; e < e1; ++e) {  // column scan over blocks, per expert
    int run = 0;
    for (int b = 0; b < nb; ++b) {
      const int c = hist[(int64_t)b * E + e];
      hist[(int64_t)b * E + e] = run;
      run += c;
    }
    counts[e] = run;
    rsum += run;
    tsum += (run + tile_m - 1) / tile_m;
  }
  s_rows[tid] = rsum;
  s_tiles[tid] = tsum;
  __syncthreads();
  for (int o = 1; o < nt; o <<= 1) {
    const int a = tid >= o ? s_rows[tid - o] : 0;
    const int b = tid >= o ? s_tiles[tid - o] : 0;
    __syncthreads();
    s_rows[tid] += a;
    s_tiles[tid] += b;
    __syncthreads();
  }
  int rr = s_rows[tid] - rsum, tt = s_tiles[tid] - tsum;
  for (int e = e0; e < e1; ++e) {
    goff[e] = rr;
    toff[e] = tt;
    for (int b = 0; b < nb; ++b) hist[(int64_t)b * E + e] += rr;
    const int c = counts[e];
    rr += c;
    tt += (c + tile_m - 1) / tile_m;
  }
  if (tid == nt - 1) {
    goff[E] = s_rows[nt - 1];
    toff[E] = s_tiles[nt - 1];
  }
}

__global__ __launch_bounds__(1024) void perm_scatter_kernel(const int32_t* __restrict__ idx,
                                                           int64_t nslots, int E,
                                                           const int32_t* __restrict__ base,
                                                           int32_t* __restrict__ perm) {
  extern __shared__ int cur[];
  const int32_t* bb = base + (int64_t)blockIdx.x * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cur[e] = bb[e];
  __syncthreads();
  const int64_t s0 = (int64_t)blockIdx.x * PERM_CHUNK;
  const int64_t s1 = min(s0 + PERM_CHUNK, nslots);
  for (int64_t s = s0 + threadIdx.x; s < s1; s += blockDim.x) {
    const int pos = atomicAdd(&cur[idx[s]], 1);
    perm[pos] = (int32_t)s;
  }
}

__global__ void histogram_kernel(const int32_t* __restrict__ idx, int64_t n,
                                 int32_t* __restrict__ counts) {
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s < n) atomicAdd(&counts[idx[s]], 1);
}

void launch_histogram(const int32_t* idx, int64_t n, int32_t* counts, int E, hipStream_t st) {
  launch_fill_i32(counts, E, 0, st);
  if (n > 0) histogram_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(idx, n, counts);
}

int perm_blocks(int64_t nslots) { return (int)((nslots + PERM_CHUNK - 1) / PERM_CHUNK); }

// Whole permutation in one block (count, scan, scatter) for moderate slot counts.
constexpr int PERM_FUSED_MAX_SLOTS = 65536, PERM_FUSED_MAX_E = 8192;
__global__ __launch_bounds__(1024) void perm_fused_kernel(const int32_t* __restrict__ idx,
                                                         int nslots, int E, int tile_m,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ goff,
                                                         int32_t* __restrict__ toff,
                                                         int32_t* __restrict__ perm) {
  extern __shared__ int lh[];  // [E] counts, then cursors
  __shared__ int s_rows[1024], s_tiles[1024];
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int e = tid; e < E; e += nt) lh[e] = 0;
  __syncthreads();
  for (int s = tid; s < nslots; s += nt) atomicAdd(&lh[idx[s]], 1);
  __syncthreads();
  const int per = (E + nt - 1) / nt;
  const int e0 = tid * per, e1 = min(E, e0 + per);
  int rsum = 0, tsum = 0;
  for (int e = e0; e < e1; ++e) {
    rsum += lh[e];
    tsum += (lh[e] + tile_m - 1) / tile_m;
  }
  s_rows[tid] = rsum;
  s_tiles[tid] = tsum;
  __syncthreads();
  for (int o = 1; o < nt; o <<= 1) {
    const int a = tid >= o ? s_rows[tid - o] : 0;
    const int b = tid >= o ? s_tiles[tid - o] : 0;
    __syncthreads();
    s_rows[tid] += a;
    s_tiles[tid] += b;
    __syncthreads();
  }
  int rr = s_rows[tid] - rsum, tt = s_tiles[tid] - tsum;
  for (int e = e0; e < e1; ++e) {
    const int c = lh[e];
    counts[e] = c;
    goff[e] = rr;
    toff[e] = tt;
    lh[e] = rr;  // cursor
    rr += c;
    tt += (c + tile_m - 1) / tile_m;
  }
  if (tid == nt - 1) {
    goff[E] = s_rows[nt - 1];
    toff[E] = s_tiles[nt - 1];
  }
  __syncthreads();
  for (int s = tid; s < nslots; s += nt) perm[atomicAdd(&lh[idx[s]], 1)] = s;
}

int launch_permute(const int32_t* idx, int64_t nslots, int E, int tile_m, int32_t* hist,
                   int32_t* counts, int32_t* goff, int32_t* toff, int32_t* perm,
                   hipStream_t st) {
  if (E > 16384) return -1;
  if (nslots <= PERM_FUSED_MAX_SLOTS && E <= PERM_FUSED_MAX_E) {
    perm_fused_kernel<<<1, 1024, (size_t)E * sizeof(int), st>>>(idx, (int)nslots, E, tile_m,
                                                                 counts, goff, toff, perm);
    return 0;
  }
  const int nb = max(1, perm_blocks(nslots));
  const size_t lds = (size_t)E * sizeof(int);
  perm_count_kernel<<<nb, 1024, lds, st>>>(idx, nslots, E, hist);
  perm_scan_kernel<<<1, 1024, 0, st>>>(hist, nb, E, tile_m, counts, goff, toff);
  if (nslots > 0) perm_scatter_kernel<<<nb, 1024, lds, st>>>(idx, nslots, E, hist, perm);
  return 0;
}

}  // namespace dreamer
