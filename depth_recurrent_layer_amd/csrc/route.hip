// Expert routing: scores, bias-adjusted top-k, sigmoid gates, and the permutation that
// groups (token, slot) pairs by expert.
//
// bf16 scores: one block per 16 tokens.  u = x W_r^T on MFMA (bf16 x bf16 products are
// exact in float32), depth RoPE on u in float32, then z = rho * u_rot . keys with u_rot
// split into three bf16 parts (hi + mid + lo carries 24 mantissa bits) so the scores keep
// float32 accuracy on MFMA.  With many tokens one fused kernel also selects (scores stay
// in LDS); with few tokens and many experts the scores go to a [T, E] float32 buffer over
// a 2-D grid and a top-k kernel (one wave per token) selects.  Either way the selection
// ranks by z + b and takes gates from z, and may count selections per expert with
// global atomics, handing each selection its rank within its expert; a placement kernel
// then turns (expert, rank) into the expert-major slot order.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dreamer {

// ------------------------------------------------------------------ scores (bf16, MFMA)
// u tile [16 tokens x r] of the block's tokens, rotated by depth, split into three bf16
// parts as MFMA A operands (token lr, k-group lg).  us / ur: 2 * 16 * (r + 4) floats of
// LDS; rows are padded by 4 floats so that the 16 rows of a fragment read (and of the
// projection's stores) start in distinct banks.
// r divides 256, so each thread rotates one rank index i = tid % r (one table entry,
// loaded before the projection).
template <int NKS>
DEV void router_u_parts(int64_t Ttok, int64_t t0, int h, int r, int l, int L,
                        const bf16* __restrict__ x, int64_t ldx, const bf16* __restrict__ w_r,
                        const float* __restrict__ cs, const float* __restrict__ sn, float* us,
                        float* ur, bf16x8 (&ah)[NKS], bf16x8 (&am)[NKS], bf16x8 (&al)[NKS]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const bf16x8 zero8 = {};
  // depth RoPE: pairs i < r/4 at depth l, the others at L-1-l
  const int half = r / 2, quarter = r / 4;
  const int i = tid % r;
  const int p = i < half ? i : i - half;
  const int pos = p < quarter ? l : L - 1 - l;
  const float cv = cs[pos * half + p], sv = sn[pos * half + p];
  // wave w owns rank columns 16 nt, nt = w, w + 4, ...  Rows past the last token read
  // the last token (their u is never used).  Loads go out in batches of 8 k-steps before
  // their MFMAs, so a batch costs one memory round trip.
  const int64_t tr = t0 + lr < Ttok ? t0 + lr : Ttok - 1;
  const bf16* xrow = x + tr * ldx + lg * 8;
  for (int nt = w; nt < r / 16; nt += 4) {
    const bf16* wrow = w_r + (int64_t)(nt * 16 + lr) * h + lg * 8;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < h; k0 += 8 * 32) {
      bf16x8 af[8], bf[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool in = k0 + 32 * j < h;
        af[j] = in ? *reinterpret_cast<const bf16x8*>(xrow + k0 + 32 * j) : zero8;
        bf[j] = in ? *reinterpret_cast<const bf16x8*>(wrow + k0 + 32 * j) : zero8;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = mfma16(af[j], bf[j], acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) us[(lg * 4 + i) * (r + 4) + nt * 16 + lr] = acc[i];
  }
  __syncthreads();
  const int ip = i < half ? i + half : i - half;
  for (int e = tid; e < 16 * r; e += 256) {
    const int t = e / r;
    const float a = us[t * (r + 4) + i], b = us[t * (r + 4) + ip];
    ur[t * (r + 4) + i] = i < half ? a * cv - b * sv : a * cv + b * sv;
  }
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const float4* src = reinterpret_cast<const float4*>(ur + lr * (r + 4) + ks * 32 + lg * 8);
    const float4 q0 = src[0], q1 = src[1];
    const float uv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = uv[j];
      const bf16 hi = (bf16)v;
      const float r1 = v - (float)hi;
      const bf16 mid = (bf16)r1;
      ah[ks][j] = hi;
      am[ks][j] = mid;
      al[ks][j] = (bf16)(r1 - (float)mid);
    }
  }
}

// Keys of one tile of 16 experts (et * 16 ..) as MFMA B operands (expert lr, k-group lg).
template <int NKS>
struct KeyFrag {
  bf16x8 v[NKS];
};

template <int NKS>
DEV void load_keys(const bf16* __restrict__ keys, int r, int et, KeyFrag<NKS>& kf) {
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const bf16* krow = keys + (int64_t)(et * 16 + lr) * r + lg * 8;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) kf.v[ks] = *reinterpret_cast<const bf16x8*>(krow + ks * 32);
}

// z for one 16 x 16 tile (tokens x experts) from the split u and the tile's keys.
template <int NKS>
DEV floatx4 router_tile(const KeyFrag<NKS>& kf, const bf16x8 (&ah)[NKS],
                        const bf16x8 (&am)[NKS], const bf16x8 (&al)[NKS]) {
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    acc = mfma16(ah[ks], kf.v[ks], acc);
    acc = mfma16(am[ks], kf.v[ks], acc);
    acc = mfma16(al[ks], kf.v[ks], acc);
  }
  return acc;
}

// Scores to a [T, E] buffer; blockIdx.y takes experts [256 y, 256 y + 256).
template <int NKS>  // r = 32 * NKS
__global__ __launch_bounds__(256) void router_scores_bf16_kernel(
    int64_t Ttok, int h, int r, int E, int l, int L, const bf16* __restrict__ x, int64_t ldx,
    const bf16* __restrict__ w_r, const bf16* __restrict__ keys, float rho,
    const float* __restrict__ cs, const float* __restrict__ sn, float* __restrict__ z) {
  extern __shared__ float smem[];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 15, lg = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  const int et0 = blockIdx.y * 16, et1 = min(E / 16, et0 + 16);
  KeyFrag<NKS> kf[4];  // this wave's tiles et0 + w + 4 j, loaded before the projection
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (et0 + w + 4 * j < et1) load_keys<NKS>(keys, r, et0 + w + 4 * j, kf[j]);
  bf16x8 ah[NKS], am[NKS], al[NKS];
  router_u_parts<NKS>(Ttok, t0, h, r, l, L, x, ldx, w_r, cs, sn, smem, smem + 16 * (r + 4), ah,
                      am, al);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int et = et0 + w + 4 * j;
    if (et >= et1) break;
    const floatx4 acc = router_tile<NKS>(kf[j], ah, am, al);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = t0 + lg * 4 + i;
      if (t < Ttok) z[t * E + et * 16 + lr] = rho * acc[i];
    }
  }
}

// (value, index) order of the router: larger value first, then lower index.
DEV bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

// Insert (v, zv, e) into a sorted list of KMAX entries (best first).
template <int KMAX>
DEV void list_insert(float (&lv)[KMAX], float (&lz)[KMAX], int (&li)[KMAX], float v, float zv,
                     int e) {
  float cv = v, cz = zv;
  int ci = e;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (better(cv, ci, lv[j], li[j])) {
      const float tv = lv[j], tz = lz[j];
      const int ti = li[j];
      lv[j] = cv;
      lz[j] = cz;
      li[j] = ci;
      cv = tv;
      cz = tz;
      ci = ti;
    }
  }
}

// ------------------------------------------------------------- fused route (bf16, MFMA)
// One block per 16 tokens.  The scores of each chunk of 256 experts go to LDS; 16 lanes
// per token scan them, each keeping a sorted list of its best (z + b, z, e); k rounds of
// a 16-lane butterfly argmax pick the winners.  Gates sigmoid(z), normalised on request
// by their sum taken in selection order.
// score rows padded to RCH + 20 floats: a wave's stores of 4 x 16 fragment rows and its
// 4 x 16-lane row scans both spread over the banks (at most 2-way on the scans)
constexpr int RCH = 256, RCH_LD = RCH + 20;

template <int NKS, int KMAX>
__global__ __launch_bounds__(256) void router_fused_bf16_kernel(
    int64_t Ttok, int h, int r, int E, int k, int l, int L, const bf16* __restrict__ x,
    int64_t ldx, const bf16* __restrict__ w_r, const bf16* __restrict__ keys,
    const float* __restrict__ bias, float rho, int normalize, const float* __restrict__ cs,
    const float* __restrict__ sn, const int32_t* __restrict__ idx_in, int32_t* __restrict__ idx,
    float* __restrict__ gate) {
  extern __shared__ float smem[];
  float* zs = smem + 32 * (r + 4);  // [16][RCH_LD]
  float* bs = zs + 16 * RCH_LD;   // [RCH] bias chunk
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  // first chunk's keys (this wave's tiles w + 4 j) and biases, before the projection
  KeyFrag<NKS> kf[4];
  int n = min(RCH, E);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (w + 4 * j < n / 16) load_keys<NKS>(keys, r, w + 4 * j, kf[j]);
  if (tid < n) bs[tid] = bias[tid];
  bf16x8 ah[NKS], am[NKS], al[NKS];
  router_u_parts<NKS>(Ttok, t0, h, r, l, L, x, ldx, w_r, cs, sn, smem, smem + 16 * (r + 4), ah,
                      am, al);
  const int tl = w * 4 + (lane >> 4), g = lane & 15;
  const int64_t t = t0 + tl;
  float lv[KMAX], lz[KMAX];
  int li[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) { lv[j] = -INFINITY; lz[j] = 0.f; li[j] = 0x7fffffff; }
  int my = 0;
  float myz = 0.f;
  if (idx_in && t < Ttok && g < k) my = min(max(idx_in[t * k + g], 0), E - 1);
  for (int c0 = 0; c0 < E; c0 += RCH) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int et = w + 4 * j;
      if (et >= n / 16) break;
      const floatx4 acc = router_tile<NKS>(kf[j], ah, am, al);
#pragma unroll
      for (int i = 0; i < 4; ++i) zs[(lg * 4 + i) * RCH_LD + et * 16 + lr] = rho * acc[i];
    }
    __syncthreads();
    // next chunk's keys and biases are fetched while this chunk is scanned
    const int c1 = c0 + RCH, n1 = c1 < E ? min(RCH, E - c1) : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (w + 4 * j < n1 / 16) load_keys<NKS>(keys, r, c1 / 16 + w + 4 * j, kf[j]);
    const float bnext = tid < n1 ? bias[c1 + tid] : 0.f;
    const float* zt = zs + tl * RCH_LD;
    if (idx_in) {
      if (g < k && my >= c0 && my < c0 + n) myz = zt[my - c0];
    } else {
      for (int j = g; j < n; j += 16) {
        const float zv = zt[j], v = zv + bs[j];
        if (better(v, c0 + j, lv[KMAX - 1], li[KMAX - 1])) list_insert<KMAX>(lv, lz, li, v, zv, c0 + j);
      }
    }
    __syncthreads();
    if (tid < n1) bs[tid] = bnext;
    n = n1;
  }
  if (!idx_in) {
    for (int j = 0; j < k; ++j) {
      float bv = lv[0], bz = lz[0];
      int bi = li[0];
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) {  // every lane of the group ends with the winner
        const float ov = __shfl_xor(bv, o, 16), oz = __shfl_xor(bz, o, 16);
        const int oi = __shfl_xor(bi, o, 16);
        if (better(ov, oi, bv, bi)) { bv = ov; bz = oz; bi = oi; }
      }
      if (g == j) { my = bi; myz = bz; }
      if (li[0] == bi) {  // the owner pops its head
#pragma unroll
        for (int q = 0; q < KMAX - 1; ++q) { lv[q] = lv[q + 1]; lz[q] = lz[q + 1]; li[q] = li[q + 1]; }
        lv[KMAX - 1] = -INFINITY;
        li[KMAX - 1] = 0x7fffffff;
      }
    }
  }
  const float gv = g < k ? sigmoidf_(myz) : 0.f;
  float gsum = 0.f;  // in selection order, as the top-k kernel sums
  for (int j = 0; j < k; ++j) gsum += __shfl(gv, j, 16);
  if (t < Ttok && g < k) {
    idx[t * k + g] = my;
    gate[t * k + g] = normalize ? gv / gsum : gv;
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
    if (lane < k) my = min(max(idx_in[t * k + lane], 0), E - 1);
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
  float gsum = 0.f;  // in selection order
  for (int j = 0; j < k; ++j) gsum += __shfl(gv, j, 64);
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
    const dim3 grid((unsigned)((T + 15) / 16), (unsigned)((E + RCH - 1) / RCH));
    const size_t lds = 2 * 16 * (r + 4) * sizeof(float);
#define RS_CASE(NK)                                                                      \
  dlaunch(router_scores_bf16_kernel<NK>, grid, 256, lds, st, T, h, r, E, l, L, (const bf16*)x, \
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
    dlaunch(router_scores_f32_kernel, (unsigned)((n + 255) / 256), 256, 0, st,
        T, r, E, l, L, u, (const float*)keys, rho, cos_r, sin_r, z);
  }
  return 0;
}

int router_topk(int64_t T, int E, int k, const float* z, const float* bias, int normalize,
                const int32_t* idx_in, int32_t* idx, float* gate, hipStream_t st) {
  if (T <= 0) return 0;
  if (k < 1 || k > 32 || k > E) return -1;
  const unsigned grid = (unsigned)((T + 3) / 4);
#define TK_CASE(KM)                                                                       \
  dlaunch(router_topk_kernel<KM>, grid, 256, 0, st, T, E, k, z, bias, normalize, idx_in, idx, gate)
  if (k <= 1) TK_CASE(1);
  else if (k <= 2) TK_CASE(2);
  else if (k <= 4) TK_CASE(4);
  else if (k <= 8) TK_CASE(8);
  else if (k <= 16) TK_CASE(16);
  else TK_CASE(32);
#undef TK_CASE
  return 0;
}

bool router_fused_ok(int dtype, int64_t T, int r, int E, int k) {
  return dtype == DT_BF16 && k <= 8 && (r == 32 || r == 64 || r == 128) && E % 16 == 0 &&
         (T + 15) / 16 >= 64;
}

int router_route_fused(int64_t T, int h, int r, int E, int k, int l, int L, const void* x,
                       int64_t ldx, const void* w_r, const void* keys, const float* bias,
                       float rho, int normalize, const float* cos_r, const float* sin_r,
                       const int32_t* idx_in, int32_t* idx, float* gate, hipStream_t st) {
  if (T <= 0) return 0;
  if (!router_fused_ok(DT_BF16, T, r, E, k) || h % 32) return -1;
  const unsigned grid = (unsigned)((T + 15) / 16);
  const size_t lds = (2 * 16 * (r + 4) + 16 * RCH_LD + RCH) * sizeof(float);
#define RF_CASE(NK, KM)                                                                     \
  dlaunch(router_fused_bf16_kernel<NK, KM>, grid, 256, lds, st,                                  \
      T, h, r, E, k, l, L, (const bf16*)x, ldx, (const bf16*)w_r, (const bf16*)keys, bias,  \
      rho, normalize, cos_r, sin_r, idx_in, idx, gate)
#define RF_K(NK)                      \
  if (k <= 1) RF_CASE(NK, 1);         \
  else if (k <= 2) RF_CASE(NK, 2);    \
  else if (k <= 4) RF_CASE(NK, 4);    \
  else RF_CASE(NK, 8);
  switch (r / 32) {
    case 1: RF_K(1); break;
    case 2: RF_K(2); break;
    case 4: RF_K(4); break;
    default: return -1;
  }
#undef RF_K
#undef RF_CASE
  return 0;
}

// ----------------------------------------------------------------------------- permute
// Routed slots grouped by expert without global atomics.  The slots are cut into chunks
// of PERM_CHUNK; kernel 1 counts each chunk's slots per expert in LDS (hist [nb, E]);
// kernel 2, one block per chunk, sums the hist columns before its chunk and in total,
// scans the totals over experts (rows, and m-tiles of tile_m rows) and hands out its
// slots' positions with LDS atomics.  Block 0 publishes counts, goff and toff.  Expert
// ids outside [0, E) are clamped into range (memory safety only: they are caller errors).
__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

void launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st) {
  if (n <= 0) return;
  dlaunch(fill_i32_kernel, (unsigned)((n + 255) / 256), 256, 0, st, p, n, v);
}

int perm_blocks(int64_t nslots) { return (int)std::max<int64_t>(1, (nslots + PERM_CHUNK - 1) / PERM_CHUNK); }

__global__ __launch_bounds__(512) void perm_hist_kernel(const int32_t* __restrict__ idx,
                                                       int64_t nslots, int E,
                                                       int32_t* __restrict__ hist) {
  extern __shared__ int lh[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) lh[e] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)blockIdx.x * PERM_CHUNK;
  const int64_t s1 = min(s0 + PERM_CHUNK, nslots);
  for (int64_t s = s0 + threadIdx.x; s < s1; s += blockDim.x)
    atomicAdd(&lh[min(max(idx[s], 0), E - 1)], 1);
  __syncthreads();
  int32_t* out = hist + (int64_t)blockIdx.x * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) out[e] = lh[e];
}

// Expert offsets from the per-expert totals in base[E] (LDS): every thread owns a
// contiguous range of experts; a wavefront scan (lane shuffles) plus one pass over the
// wave totals gives each range its first row and first m-tile.  base[e] becomes e's
// first row plus prev[e] (the rows of e in earlier chunks, or nullptr); with pub,
// counts / goff / toff and the tile descriptors are written; with pad, prev[e] becomes
// the shift from e's compact positions to its tile-padded ones.  s_wave: 32 ints.
DEV void expert_offsets(int* base, int* prev, int E, int tile_m, bool pub, bool pad,
                        int32_t* __restrict__ counts, int32_t* __restrict__ goff,
                        int32_t* __restrict__ toff, int4* __restrict__ tiles, int* s_wave) {
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, w = tid >> 6;
  const int per = (E + nt - 1) / nt;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int rsum = 0, tsum = 0;
  for (int e = e0; e < e1; ++e) {
    rsum += base[e];
    tsum += (base[e] + tile_m - 1) / tile_m;
  }
  int r = rsum, t = tsum;  // inclusive scans within the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int a = __shfl_up(r, o, 64), c = __shfl_up(t, o, 64);
    if (lane >= o) {
      r += a;
      t += c;
    }
  }
  if (lane == 63) {
    s_wave[w] = r;
    s_wave[16 + w] = t;
  }
  __syncthreads();
  int rr = r - rsum, tt = t - tsum, rtot = 0, ttot = 0;
  for (int q = 0; q < (nt >> 6); ++q) {
    if (q < w) {
      rr += s_wave[q];
      tt += s_wave[16 + q];
    }
    rtot += s_wave[q];
    ttot += s_wave[16 + q];
  }
  for (int e = e0; e < e1; ++e) {
    const int tot = base[e];
    if (pub) {
      counts[e] = tot;
      goff[e] = rr;
      toff[e] = tt;
      if (tiles)  // one descriptor per m-tile: expert, first row, end of the expert's rows
        for (int q = 0; q * tile_m < tot; ++q) tiles[tt + q] = make_int4(e, rr + q * tile_m, rr + tot, 0);
    }
    base[e] = rr + (prev ? prev[e] : 0);
    if (pad) prev[e] = tt * tile_m - rr;
    rr += tot;
    tt += (tot + tile_m - 1) / tile_m;
  }
  if (pub && tid == 0) {
    goff[E] = rtot;
    toff[E] = ttot;
  }
  __syncthreads();
}

// One block of PERM_THREADS per chunk: the chunk's experts and gates are loaded first
// (their latency overlaps the histogram reads), then the totals and the rows of each
// expert in earlier chunks, the offsets, and the scatter from registers.  pad: slot ids
// and gates go to tile-padded positions (m-tile t of the expert-major order owns
// positions t * tile_m ..), the layout the expert FFN reads per tile.
constexpr int PERM_THREADS = 512, PERM_PER = PERM_CHUNK / PERM_THREADS;

__global__ __launch_bounds__(PERM_THREADS) void perm_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t nslots, int E, int nb, int tile_m,
    const int32_t* __restrict__ hist, int32_t* __restrict__ counts, int32_t* __restrict__ goff,
    int32_t* __restrict__ toff, int32_t* __restrict__ perm, const float* __restrict__ gate,
    float* __restrict__ pgate, int4* __restrict__ tiles, int pad) {
  extern __shared__ int sh[];  // base [E] (totals, then cursors), prev [E]
  int* base = sh;
  int* prev = sh + E;
  __shared__ int s_wave[32];
  const int tid = threadIdx.x, b = blockIdx.x;
  const int64_t s0 = (int64_t)b * PERM_CHUNK;
  int ex[PERM_PER];
  float gv[PERM_PER];
#pragma unroll
  for (int j = 0; j < PERM_PER; ++j) {
    const int64_t s = s0 + j * PERM_THREADS + tid;
    ex[j] = s < nslots ? min(max(idx[s], 0), E - 1) : -1;
    gv[j] = (pgate && s < nslots) ? gate[s] : 0.f;
  }
  for (int e = tid; e < E; e += PERM_THREADS) {
    int tot = 0, pre = 0;
    for (int q = 0; q < nb; ++q) {
      const int v = hist[(int64_t)q * E + e];
      tot += v;
      pre += q < b ? v : 0;
    }
    base[e] = tot;
    prev[e] = pre;
  }
  __syncthreads();
  expert_offsets(base, prev, E, tile_m, b == 0, pad != 0, counts, goff, toff, tiles, s_wave);
#pragma unroll
  for (int j = 0; j < PERM_PER; ++j)
    if (ex[j] >= 0) {
      const int pos = atomicAdd(&base[ex[j]], 1) + (pad ? prev[ex[j]] : 0);
      perm[pos] = (int32_t)(s0 + j * PERM_THREADS + tid);
      if (pgate) pgate[pos] = gv[j];
    }
}

__global__ void hist_colsum_kernel(const int32_t* __restrict__ hist, int nb, int E,
                                   int32_t* __restrict__ counts) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  int c = 0;
  for (int q = 0; q < nb; ++q) c += hist[(int64_t)q * E + e];
  counts[e] = c;
}

int launch_permute(const int32_t* idx, int64_t nslots, int E, int tile_m, int32_t* hist,
                   int32_t* counts, int32_t* goff, int32_t* toff, int32_t* perm,
                   hipStream_t st, const float* gate, float* pgate, int4* tiles, int pad) {
  if (E <= 0 || E > PERM_MAX_E) return -1;
  const size_t lds = (size_t)E * sizeof(int);
  const int nb = perm_blocks(nslots);
  dlaunch(perm_hist_kernel, nb, 512, lds, st, idx, nslots, E, hist);
  dlaunch(perm_scatter_kernel, nb, PERM_THREADS, 2 * lds, st, idx, nslots, E, nb, tile_m, hist,
                                                         counts, goff, toff, perm, gate, pgate,
                                                         tiles, pad);
  return 0;
}

int launch_counts(const int32_t* idx, int64_t nslots, int E, int32_t* hist, int32_t* counts,
                  hipStream_t st) {
  if (E <= 0 || E > COUNT_MAX_E) return -1;
  const int nb = perm_blocks(nslots);
  dlaunch(perm_hist_kernel, nb, 512, (size_t)E * sizeof(int), st, idx, nslots, E, hist);
  dlaunch(hist_colsum_kernel, (E + 255) / 256, 256, 0, st, hist, nb, E, counts);
  return 0;
}

}  // namespace dreamer
