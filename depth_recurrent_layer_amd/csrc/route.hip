// Expert routing: scores, bias-adjusted top-k, sigmoid gates, and the permutation that
// groups (token, slot) pairs by expert.
//
// bf16 scores: one block per 16 tokens.  u = x W_r^T on MFMA (bf16 x bf16 products are
// exact in float32), depth RoPE on u in float32, then z = rho * u_rot . keys with u_rot
// split into three bf16 parts (hi + mid + lo carries 24 mantissa bits) so the scores keep
// float32 accuracy on MFMA.  With many tokens one fused kernel also selects (scores stay
// in LDS); with few tokens and many experts the scores go to a [T, E] float32 buffer over
// a 2-D grid and a top-k kernel (one wave per token) selects.  Either way the selection
// ranks by z + b (ties to the lower expert index) and takes gates from z.  The fused
// kernel can also count the permutation's chunk histograms (global atomics); the
// permutation kernels then scan them and scatter the slots into expert-major order.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dreamer {

// ------------------------------------------------------------------ scores (bf16, MFMA)
// u tile [16 tokens x r] of the block's tokens, rotated by depth, split into three bf16
// parts as MFMA A operands (token lr, k-group lg).  The projection is split over the
// block's 4 waves by k: wave w takes the k-steps (of 32) w, w + 4, ..., all r / 16 column
// tiles, so each x fragment is loaded once; the 4 partial tiles go to part [4][16][r + 4]
// in LDS and are summed in wave order.  ur: [16][r + 4].  Rows are padded by 4 floats so
// that the 16 rows of a fragment read (and of the partial stores) start in distinct banks.
// r divides 256, so each thread rotates one rank index i = tid % r (one table entry,
// loaded before the projection).
template <int NKS>
DEV void router_u_parts(int64_t Ttok, int64_t t0, int h, int r, int l, int L,
                        const bf16* __restrict__ x, int64_t ldx, const bf16* __restrict__ w_r,
                        const float* __restrict__ cs, const float* __restrict__ sn, float* part,
                        float* ur, bf16x8 (&ah)[NKS], bf16x8 (&am)[NKS], bf16x8 (&al)[NKS]) {
  constexpr int NT = 2 * NKS;           // r / 16 column tiles
  constexpr int KB = NT <= 4 ? 4 : 2;   // k-steps per batch of loads (KB x (1 + NT) x 16 B)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int rp = r + 4;
  // depth RoPE: pairs i < r/4 at depth l, the others at L-1-l
  const int half = r / 2, quarter = r / 4;
  const int i = tid % r;
  const int p = i < half ? i : i - half;
  const int pos = p < quarter ? l : L - 1 - l;
  const float cv = cs[pos * half + p], sv = sn[pos * half + p];
  // Rows past the last token read the last token (their u is never used).  A batch's
  // loads all go out before its MFMAs (one memory round trip per batch); k-steps past the
  // wave's last are clamped loads that are not used.  Token block t0 / 16 starts at batch
  // (t0 / 16) % batches: concurrent blocks read different parts of W_r (the order is a
  // function of the token block alone, so every kernel computing u for a token sums in
  // the same order).
  const int64_t tr = t0 + lr < Ttok ? t0 + lr : Ttok - 1;
  const bf16* xrow = x + tr * ldx + lg * 8;
  const bf16* wrow = w_r + (int64_t)lr * h + lg * 8;
  const int nkw = (h / 32 - w + 3) / 4;  // this wave's k-steps
  const int nbat = (nkw + KB - 1) / KB;
  const int rot = nbat > 0 ? (int)((t0 / 16) % nbat) : 0;
  floatx4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int bq = 0; bq < nbat; ++bq) {
    const int b0 = ((bq + rot) % nbat) * KB;
    bf16x8 af[KB], bf[KB][NT];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int k0 = (w + 4 * min(b0 + j, nkw - 1)) * 32;
      af[j] = *reinterpret_cast<const bf16x8*>(xrow + k0);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        bf[j][nt] = *reinterpret_cast<const bf16x8*>(wrow + (int64_t)nt * 16 * h + k0);
    }
#pragma unroll
    for (int j = 0; j < KB; ++j)
      if (b0 + j < nkw) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma16(af[j], bf[j][nt], acc[nt]);
      }
  }
  float* pw = part + w * 16 * rp;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int q = 0; q < 4; ++q) pw[(lg * 4 + q) * rp + nt * 16 + lr] = acc[nt][q];
  __syncthreads();
  const int ip = i < half ? i + half : i - half;
  for (int e = tid; e < 16 * r; e += 256) {
    const float* pt = part + (e / r) * rp;
    const float a = ((pt[i] + pt[16 * rp + i]) + pt[32 * rp + i]) + pt[48 * rp + i];
    const float b = ((pt[ip] + pt[16 * rp + ip]) + pt[32 * rp + ip]) + pt[48 * rp + ip];
    ur[(e / r) * rp + i] = i < half ? rot_first(a, b, cv, sv) : rot_second(a, b, cv, sv);
  }
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const float4* src = reinterpret_cast<const float4*>(ur + lr * rp + ks * 32 + lg * 8);
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
  router_u_parts<NKS>(Ttok, t0, h, r, l, L, x, ldx, w_r, cs, sn, smem + 16 * (r + 4), smem, ah,
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

// ------------------------------------------------------------- fused route (bf16, MFMA)
// One block per 16 tokens, 16 lanes per token.  The scores of each chunk of 256 experts go
// to LDS.  The token's best k so far are held across its 16 lanes, lane g holding the g-th
// best (z + b, z, e).  Each chunk, a lane reads its 16 values (experts c0 + g + 16 q) and
// flags those that are not below tau, a value under which nothing can be selected: tau is
// the larger of the current k-th best and the k-th largest of the 16 lanes' chunk maxima
// (both leave at least k better values above anything below them).  The flagged
// candidates are then inserted one per token per step: the token's group takes its first
// flagged lane's first candidate, every lane compares it with its entry, and entries that
// lose to it move down one lane (a row shift).  Candidates are few once the list holds
// good values (about k / c of a chunk's values pass in chunk c on random data), so the
// selection costs a compare per value.  Gates sigmoid(z), normalised on request by their
// sum taken in selection order.
// score rows padded to RCH + 20 floats: a wave's stores of 4 x 16 fragment rows and its
// 4 x 16-lane row reads both spread over the banks (at most 2-way on the reads)
constexpr int RCH = 256, RCH_LD = RCH + 20;

// The value of the lane one below in the same 16-lane row; lane 0 of a row gets `first`.
DEV int row_shr1(int v, int first) { return __builtin_amdgcn_update_dpp(first, v, 0x111, 0xF, 0xF, false); }
DEV float row_shr1(float v, float first) {
  return __int_as_float(row_shr1(__float_as_int(v), __float_as_int(first)));
}

template <int NKS>
__global__ __launch_bounds__(256) void router_fused_bf16_kernel(
    int64_t Ttok, int h, int r, int E, int k, int l, int L, const bf16* __restrict__ x,
    int64_t ldx, const bf16* __restrict__ w_r, const bf16* __restrict__ keys,
    const float* __restrict__ bias, float rho, int normalize, const float* __restrict__ cs,
    const float* __restrict__ sn, const int32_t* __restrict__ idx_in, int32_t* __restrict__ idx,
    float* __restrict__ gate, int32_t* __restrict__ hist) {
  extern __shared__ float smem[];
  float* bs = smem + 16 * (r + 4);  // [RCH] bias chunk (after u's [16][r + 4])
  float* zs = bs + RCH;  // [16][RCH_LD] scores; first the projection's partial tiles
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  // Chunks of RCH experts in the order rot, rot + 1, ... (rot = block % chunks): concurrent
  // blocks read different parts of the key table (the selection does not depend on the
  // order).  The first chunk's keys (this wave's tiles w + 4 j) and biases are loaded
  // before the projection; tile indices are clamped into the key table (tiles past the
  // chunk are not used), so the loads are unconditional.
  const int nch = (E + RCH - 1) / RCH, rot = (int)(blockIdx.x % nch);
  KeyFrag<NKS> kf[4];
  int c0 = rot * RCH, n = min(RCH, E - c0);
  const int ntile = E / 16;
#pragma unroll
  for (int j = 0; j < 4; ++j) load_keys<NKS>(keys, r, min(c0 / 16 + w + 4 * j, ntile - 1), kf[j]);
  if (tid < n) bs[tid] = bias[c0 + tid];
  bf16x8 ah[NKS], am[NKS], al[NKS];
  router_u_parts<NKS>(Ttok, t0, h, r, l, L, x, ldx, w_r, cs, sn, zs, smem, ah, am, al);
  const int tl = w * 4 + (lane >> 4), g = lane & 15;
  const int64_t t = t0 + tl;
  float lv = -INFINITY, lz = 0.f;  // this lane's entry of the token's list
  int li = 0x7fffffff;
  int my = 0;
  float myz = 0.f;
  if (idx_in && t < Ttok && g < k) my = min(max(idx_in[t * k + g], 0), E - 1);
  for (int ci = 0; ci < nch; ++ci) {
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
    const int c1 = ((ci + 1 + rot) % nch) * RCH, n1 = ci + 1 < nch ? min(RCH, E - c1) : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      load_keys<NKS>(keys, r, min(c1 / 16 + w + 4 * j, ntile - 1), kf[j]);
    const float bnext = tid < n1 ? bias[c1 + tid] : 0.f;
    const float* zt = zs + tl * RCH_LD;
    if (idx_in) {
      if (g < k && my >= c0 && my < c0 + n) myz = zt[my - c0];
    } else {
      float vr[RCH / 16];
      float lmax = -INFINITY;
#pragma unroll
      for (int q = 0; q < RCH / 16; ++q) {
        const int j = min(g + 16 * q, n - 1);  // n is a multiple of 16
        vr[q] = zt[j] + bs[j];
        lmax = fmaxf(lmax, vr[q]);
      }
      // k rounds of a group max over the lane maxima, each dropping the lanes that hold
      // the round's max (equal maxima dropped together only lower the bound)
      float tau = __shfl(lv, k - 1, 16), cut = -INFINITY;
      for (int j = 0; j < k; ++j) {
        cut = group_max16(lmax);
        if (lmax == cut) lmax = -INFINITY;
      }
      tau = fmaxf(tau, cut);
      unsigned m = 0;
#pragma unroll
      for (int q = 0; q < RCH / 16; ++q)
        if (16 * q < n && vr[q] >= tau) m |= 1u << q;
      for (;;) {
        const uint64_t act = __ballot(m != 0);
        if (!act) break;  // the same in every lane
        const unsigned gm = (unsigned)(act >> (lane & 48)) & 0xFFFFu;  // my group's lanes
        const int src = gm ? __builtin_ctz(gm) : 0;
        const unsigned ms = __shfl(m, src, 16);
        const int jc = gm ? src + 16 * __builtin_ctz(ms) : 0;
        if (gm && g == src) m &= m - 1;
        const float cz = zt[jc], cv = cz + bs[jc];
        const int ce = c0 + jc;
        const bool keep = !gm || better(lv, li, cv, ce);
        const int pk = row_shr1(keep ? 1 : 0, 1);
        const float pv = row_shr1(lv, 0.f), pz = row_shr1(lz, 0.f);
        const int pi = row_shr1(li, 0);
        lv = keep ? lv : (pk ? cv : pv);
        lz = keep ? lz : (pk ? cz : pz);
        li = keep ? li : (pk ? ce : pi);
      }
    }
    __syncthreads();
    if (tid < n1) bs[tid] = bnext;
    c0 = c1;
    n = n1;
  }
  if (!idx_in) {
    my = min(max(li, 0), E - 1);  // entries past the k-th are not used
    myz = lz;
  }
  const float gv = g < k ? sigmoidf_(myz) : 0.f;
  float gsum = 0.f;  // in selection order, as the top-k kernel sums
  for (int j = 0; j < k; ++j) gsum += __shfl(gv, j, 16);
  if (t < Ttok && g < k) {
    idx[t * k + g] = my;
    gate[t * k + g] = normalize ? gv / gsum : gv;
    if (hist) atomicAdd(&hist[((t * k + g) / PERM_CHUNK) * E + my], 1);
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
    acc = fmaf(i < half ? rot_first(a, b, cv, sv) : rot_second(a, b, cv, sv), ke[i], acc);
  }
  z[gid] = rho * acc;
}

// ------------------------------------------------------------------------------- top-k
// Top-k for 16 < k <= 32.  One wave per token.  Each lane keeps a sorted list of its KMAX
// best (z + b, e) over experts lane, lane + 64, ...; k rounds of a butterfly argmax pop
// the heads.  Gates are sigmoid(z) of the winners, divided by their sum when normalising.
// With idx_in the given experts are adopted instead.
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
    // values below tau, the largest KMAX-th best of the 64 lane lists, cannot be selected
    // (see the fused kernel); tau is refreshed after every 4 values of a lane
    float tau = -INFINITY;
    for (int e0 = 0; e0 < E; e0 += 64) {  // the same iterations in every lane
      if ((e0 & 255) == 0 && e0 > 0)
        tau = fmaxf(tau, max_xor32(max_xor16(group_max16(lv[KMAX - 1]))));
      const int e = e0 + lane;
      if (e >= E) continue;
      const float v = zt[e] + bias[e];
      if (v < tau || !better(v, e, lv[KMAX - 1], li[KMAX - 1])) continue;
      // insert into the sorted list (selects: straight-line compares and moves)
      float cv = v;
      int ci = e;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        const bool b = better(cv, ci, lv[j], li[j]);
        const float nv = b ? cv : lv[j];
        const int ni = b ? ci : li[j];
        cv = b ? lv[j] : cv;
        ci = b ? li[j] : ci;
        lv[j] = nv;
        li[j] = ni;
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

// Top-k for k <= 16, one wave per token.  The wave's four 16-lane groups take the
// experts in four contiguous quarters; each group keeps its quarter's best k across its
// lanes (lane g: the g-th best) with the fused kernel's selection (chunks of 16 values per
// lane, values below tau flagged off, candidates inserted one per step by a row shift).
// A step takes one candidate in every group: each lane offers its lowest flagged value,
// and the group's first offering lane is read with readlane (the lane numbers come from
// the wave's ballot, so they are the same in every lane).  The next chunk's scores are
// loaded while a chunk is selected.  Group 0 then takes in the other groups' entries that
// are not below its k-th best: the top k of the union of the quarters' top k lists is
// the top k of all experts.
DEV void topk_row_insert(float& lv, float& lz, int& li, bool none, float cv, float cz, int ce) {
  const bool keep = none || better(lv, li, cv, ce);
  const int pk = row_shr1(keep ? 1 : 0, 1);
  const float pv = row_shr1(lv, 0.f), pz = row_shr1(lz, 0.f);
  const int pi = row_shr1(li, 0);
  lv = keep ? lv : (pk ? cv : pv);
  lz = keep ? lz : (pk ? cz : pz);
  li = keep ? li : (pk ? ce : pi);
}

// One token per block: group G of wave w (the block's 16 groups of 16 lanes) scans range
// 4 w + G of 16 equal expert ranges; each wave's group 0 merges its wave's groups, then
// wave 0 takes in the other waves' lists from LDS (a token's scan spread over four
// waves: few tokens, as in decode, still occupy as many CUs as they have tokens).
__global__ __launch_bounds__(256) void router_topk16_kernel(
    int64_t Ttok, int E, int k, const float* __restrict__ z, const float* __restrict__ bias,
    int normalize, const int32_t* __restrict__ idx_in, int32_t* __restrict__ idx,
    float* __restrict__ gate) {
  __shared__ float s_v[4][16], s_z[4][16];
  __shared__ int s_i[4][16];
  const int lane = threadIdx.x & 63, G = lane >> 4, g = lane & 15, w = threadIdx.x >> 6;
  const int64_t t = blockIdx.x;
  if (t >= Ttok) return;  // the whole block
  const float* zt = z + t * E;
  int my = 0;
  float myz = 0.f;
  if (idx_in) {
    if (w != 0) return;
    if (lane < k) {
      my = min(max(idx_in[t * k + lane], 0), E - 1);
      myz = zt[my];
    }
  } else {
    constexpr int NQ = RCH / 16;
    const int eq = (E + 255) / 256 * 16;  // range length (a multiple of 16)
    const int GG = w * 4 + G;             // this group's range
    const int e1 = min(E, (GG + 1) * eq);
    float lv = -INFINITY, lz = 0.f;
    int li = 0x7fffffff;
    float zn[NQ], bn[NQ];  // the next chunk's scores and biases (clamped reads)
    auto load = [&](int c0) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int e = min(c0 + g + 16 * q, E - 1);
        zn[q] = zt[e];
        bn[q] = bias[e];
      }
    };
    load(GG * eq);
    for (int c0 = GG * eq; c0 < (GG + 1) * eq; c0 += RCH) {  // same trip count in every group
      float vr[NQ], zr[NQ];
      float lmax = -INFINITY;
      unsigned m = 0;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const bool in = c0 + g + 16 * q < e1;
        zr[q] = zn[q];
        vr[q] = in ? zn[q] + bn[q] : -INFINITY;
        lmax = fmaxf(lmax, vr[q]);
        m |= (in ? 1u : 0u) << q;
      }
      if (c0 + RCH < (GG + 1) * eq) load(c0 + RCH);
      float tau = __shfl(lv, k - 1, 16), cut = -INFINITY;
      for (int j = 0; j < k; ++j) {
        cut = group_max16(lmax);
        if (lmax == cut) lmax = -INFINITY;
      }
      tau = fmaxf(tau, cut);
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if (!(vr[q] >= tau)) m &= ~(1u << q);
      for (;;) {
        const uint64_t act = __ballot(m != 0);
        if (!act) break;  // the same in every lane
        const int qn = m ? __builtin_ctz(m) : 0;
        float ov = vr[0], oz = zr[0];
#pragma unroll
        for (int q = 1; q < NQ; ++q)
          if (qn == q) {
            ov = vr[q];
            oz = zr[q];
          }
        const int oe = c0 + g + 16 * qn;
        float cv = 0.f, cz = 0.f;
        int ce = 0;
        bool none = true;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {  // group q4's first offering lane
          const unsigned gm = (unsigned)(act >> (16 * q4)) & 0xFFFFu;
          if (!gm) continue;
          const int sl = 16 * q4 + __builtin_ctz(gm);
          const float v4 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ov), sl));
          const float z4 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(oz), sl));
          const int e4 = __builtin_amdgcn_readlane(oe, sl);
          if (G == q4) {
            cv = v4;
            cz = z4;
            ce = e4;
            none = false;
            if (lane == sl) m &= m - 1;
          }
        }
        topk_row_insert(lv, lz, li, none, cv, cz, ce);
      }
    }
    // group 0 takes in the entries of groups 1..3 that are not below its k-th best
    const float tau0 = __shfl(lv, k - 1, 64);
    uint64_t bal = __ballot(G > 0 && g < k && lv >= tau0);
    while (bal) {  // the same in every lane
      const int sl = __builtin_ctzll(bal);
      bal &= bal - 1;
      const float cv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), sl));
      const float cz = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lz), sl));
      const int ce = __builtin_amdgcn_readlane(li, sl);
      topk_row_insert(lv, lz, li, G != 0, cv, cz, ce);
    }
    // wave 0's group 0 takes in the other waves' lists that are not below its k-th best
    if (lane < k) {
      s_v[w][lane] = lv;
      s_z[w][lane] = lz;
      s_i[w][lane] = li;
    }
    __syncthreads();
    if (w != 0) return;
    const float tau1 = __shfl(lv, k - 1, 64);
    for (int wo = 1; wo < 4; ++wo)
      for (int j = 0; j < k; ++j) {  // the same in every lane
        const float cv = s_v[wo][j];
        if (!(cv >= tau1)) continue;
        topk_row_insert(lv, lz, li, G != 0, cv, s_z[wo][j], s_i[wo][j]);
      }
    my = min(max(li, 0), E - 1);  // lanes 0..k-1 (group 0) hold the selection in order
    myz = lz;
  }
  const float gv = lane < k ? sigmoidf_(myz) : 0.f;
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
    const size_t lds = 5 * 16 * (r + 4) * sizeof(float);
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
  if (k <= 16)
    dlaunch(router_topk16_kernel, (unsigned)T, 256, 0, st, T, E, k, z, bias, normalize, idx_in,
            idx, gate);
  else
    TK_CASE(32);
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
                       const int32_t* idx_in, int32_t* idx, float* gate, hipStream_t st,
                       int32_t* hist) {
  if (T <= 0) return 0;
  if (!router_fused_ok(DT_BF16, T, r, E, k) || h % 32) return -1;
  const unsigned grid = (unsigned)((T + 15) / 16);
  const size_t lds = (16 * (r + 4) + RCH + std::max(16 * RCH_LD, 64 * (r + 4))) * sizeof(float);
#define RF_K(NK)                                                                          \
  dlaunch(router_fused_bf16_kernel<NK>, grid, 256, lds, st, T, h, r, E, k, l, L, (const bf16*)x, \
          ldx, (const bf16*)w_r, (const bf16*)keys, bias, rho, normalize, cos_r, sin_r, idx_in, \
          idx, gate, hist)
  switch (r / 32) {
    case 1: RF_K(1); break;
    case 2: RF_K(2); break;
    case 4: RF_K(4); break;
    default: return -1;
  }
#undef RF_K
  return 0;
}

// ----------------------------------------------------------------------------- permute
// Routed slots grouped by expert.  The slots are cut into chunks of PERM_CHUNK; kernel 1
// counts each chunk's slots per expert in LDS (hist [nb, E]; in the layer the fused
// router counts them instead, with global atomics, and kernel 1 is skipped); kernel 2
// turns hist, in place, into each chunk's rows of every expert in earlier chunks and
// writes the totals to counts; kernel 3, one block per chunk, scans the totals over
// experts (rows, and m-tiles of tile_m rows) and hands out its slots' positions with LDS
// atomics.  Block 0 of kernel 3 publishes goff and toff.  Expert ids outside [0, E) are
// clamped into range (memory safety only: they are caller errors).
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

// Per expert (32 per block, one lane each in 8 groups of chunk rows): the exclusive
// prefix of hist's column over the chunks, in place, and the column total into counts.
// A group sums its run of rows, the runs' sums are scanned through LDS, then the group
// rewrites its rows (the column is re-read from L2).
__global__ __launch_bounds__(256) void perm_prefix_kernel(int32_t* __restrict__ hist, int nb,
                                                          int E, int32_t* __restrict__ counts) {
  __shared__ int part[8][32];
  const int el = threadIdx.x & 31, grp = threadIdx.x >> 5;
  const int e = blockIdx.x * 32 + el;
  const int run = (nb + 7) / 8, q0 = grp * run, q1 = min(nb, q0 + run);
  const int ec = min(e, E - 1);
  int sum = 0;
  for (int q = q0; q < q1; q += 8) {  // 8 loads in flight (clamped rows, unused dropped)
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = hist[(int64_t)min(q + u, q1 - 1) * E + ec];
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += q + u < q1 ? v[u] : 0;
  }
  part[grp][el] = sum;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    pre += g < grp ? part[g][el] : 0;
    tot += part[g][el];
  }
  if (e >= E) return;
  if (grp == 0) counts[e] = tot;
  for (int q = q0; q < q1; ++q) {
    int32_t* p = hist + (int64_t)q * E + e;
    const int v = *p;
    *p = pre;
    pre += v;
  }
}

// Expert offsets from the per-expert totals in base[E] (LDS): every thread owns a
// contiguous range of experts; a wavefront scan (lane shuffles) plus one pass over the
// wave totals gives each range its first row and first m-tile.  base[e] becomes e's
// first row plus prev[e] (the rows of e in earlier chunks, or nullptr); with pub,
// goff / toff and the tile descriptors are written; with pad, prev[e] becomes the shift
// from e's compact positions to its tile-padded ones.  s_wave: 32 ints.
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
// (their latency overlaps the other reads), then the totals and the rows of each expert
// in earlier chunks, the offsets, and the scatter from registers.  pad: slot ids
// and gates go to tile-padded positions (m-tile t of the expert-major order owns
// positions t * tile_m ..), the layout the expert FFN reads per tile.
constexpr int PERM_THREADS = 512, PERM_PER = PERM_CHUNK / PERM_THREADS;

__global__ __launch_bounds__(PERM_THREADS) void perm_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t nslots, int E, int nb, int tile_m,
    const int32_t* __restrict__ hist, int32_t* __restrict__ counts, int32_t* __restrict__ goff,
    int32_t* __restrict__ toff, int32_t* __restrict__ perm, const float* __restrict__ gate,
    float* __restrict__ pgate, int4* __restrict__ tiles, int pad, int32_t* __restrict__ zero_next) {
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
  // the totals and this chunk's row of earlier-chunk counts (hist after kernel 2)
  for (int e = tid; e < E; e += PERM_THREADS) {
    base[e] = counts[e];
    prev[e] = hist[(int64_t)b * E + e];
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
  if (zero_next)
    for (int64_t i = (int64_t)b * PERM_THREADS + tid; i < (int64_t)nb * E; i += (int64_t)nb * PERM_THREADS)
      zero_next[i] = 0;
}

// The whole permutation in one block when the slots fit one chunk (nslots <= PERM_CHUNK,
// e.g. a decode step's few tokens): the chunk's histogram in LDS, the offsets, the
// scatter, and (zero_next) the clearing of the router's other histogram buffer.  The
// same outputs as the three-kernel path (rows of one expert in some order; every row's
// result is independent of its place in the group).
__global__ __launch_bounds__(PERM_THREADS) void perm_single_kernel(
    const int32_t* __restrict__ idx, int64_t nslots, int E, int tile_m,
    int32_t* __restrict__ counts, int32_t* __restrict__ goff, int32_t* __restrict__ toff,
    int32_t* __restrict__ perm, const float* __restrict__ gate, float* __restrict__ pgate,
    int4* __restrict__ tiles, int pad, int32_t* __restrict__ zero_next) {
  extern __shared__ int sh[];  // base [E] (totals, then cursors), prev [E]
  int* base = sh;
  int* prev = sh + E;
  __shared__ int s_wave[32];
  const int tid = threadIdx.x;
  int ex[PERM_PER];
  float gv[PERM_PER];
#pragma unroll
  for (int j = 0; j < PERM_PER; ++j) {
    const int64_t s = j * PERM_THREADS + tid;
    ex[j] = s < nslots ? min(max(idx[s], 0), E - 1) : -1;
    gv[j] = (pgate && s < nslots) ? gate[s] : 0.f;
  }
  for (int e = tid; e < E; e += PERM_THREADS) {
    base[e] = 0;
    prev[e] = 0;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PERM_PER; ++j)
    if (ex[j] >= 0) atomicAdd(&base[ex[j]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += PERM_THREADS) counts[e] = base[e];
  expert_offsets(base, prev, E, tile_m, true, pad != 0, counts, goff, toff, tiles, s_wave);
#pragma unroll
  for (int j = 0; j < PERM_PER; ++j)
    if (ex[j] >= 0) {
      const int pos = atomicAdd(&base[ex[j]], 1) + (pad ? prev[ex[j]] : 0);
      perm[pos] = (int32_t)(j * PERM_THREADS + tid);
      if (pgate) pgate[pos] = gv[j];
    }
  if (zero_next)
    for (int e = tid; e < E; e += PERM_THREADS) zero_next[e] = 0;
}

__global__ void hist_colsum_kernel(const int32_t* __restrict__ hist, int nb, int E,
                                   int32_t* __restrict__ counts) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  int c = 0;
  for (int q0 = 0; q0 < nb; q0 += 8) {  // 8 loads in flight
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = hist[(int64_t)min(q0 + u, nb - 1) * E + e];
#pragma unroll
    for (int u = 0; u < 8; ++u) c += q0 + u < nb ? v[u] : 0;
  }
  counts[e] = c;
}

int launch_permute(const int32_t* idx, int64_t nslots, int E, int tile_m, int32_t* hist,
                   int32_t* counts, int32_t* goff, int32_t* toff, int32_t* perm,
                   hipStream_t st, const float* gate, float* pgate, int4* tiles, int pad,
                   bool hist_ready, int32_t* zero_next) {
  if (E <= 0 || E > PERM_MAX_E) return -1;
  const size_t lds = (size_t)E * sizeof(int);
  const int nb = perm_blocks(nslots);
  if (nb == 1) {  // one chunk: one launch (a counted histogram, if any, is not needed)
    dlaunch(perm_single_kernel, 1, PERM_THREADS, 2 * lds, st, idx, nslots, E, tile_m, counts,
            goff, toff, perm, gate, pgate, tiles, pad, zero_next);
    return 0;
  }
  if (!hist_ready) dlaunch(perm_hist_kernel, nb, 512, lds, st, idx, nslots, E, hist);
  dlaunch(perm_prefix_kernel, (E + 31) / 32, 256, 0, st, hist, nb, E, counts);
  dlaunch(perm_scatter_kernel, nb, PERM_THREADS, 2 * lds, st, idx, nslots, E, nb, tile_m, hist,
          counts, goff, toff, perm, gate, pgate, tiles, pad, zero_next);
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
