// Attention kernels: depth attention (DA), causal sequence attention (SA) prefill with
// MFMA, and a row-streaming SA kernel used for decode (split over key ranges) and for
// shapes outside the MFMA kernel.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dreamer {

// ------------------------------------------------------------------------- RoPE tables
__global__ void rope_table_kernel(int D, int npos, double base, float* c, float* s) {
  const int half = D / 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)npos * half) return;
  const int p = (int)(i / half), j = (int)(i % half);
  const double theta = pow(base, -2.0 * (double)j / (double)D);
  const double ang = (double)p * theta;
  c[i] = (float)cos(ang);
  s[i] = (float)sin(ang);
}

void launch_rope_tables(int D, int npos, double base, float* c, float* s, hipStream_t st) {
  const int64_t n = (int64_t)npos * (D / 2);
  if (n <= 0) return;
  rope_table_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(D, npos, base, c, s);
}

// Rotate one 16-byte chunk in place.  The lane holds dims [c*VEC, c*VEC+VEC) of a head
// with LPH lanes per head; its rotate-half partner chunk is c ^ (LPH/2), fetched with a
// lane shuffle.  pos_fwd / pos_rev: positions used by rotary pairs below / from d/4.
template <int VEC, int LPH>
DEV void rope_chunk(float* x, int c, int d, int pos_fwd, int pos_rev, const float* cs,
                    const float* sn) {
  float other[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) other[i] = __shfl_xor(x[i], LPH / 2, 64);
  const int half = d / 2, quarter = d / 4;
  const bool lo = c < LPH / 2;
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    const int dim = c * VEC + i;
    const int p = lo ? dim : dim - half;       // rotary pair index
    const int pos = p < quarter ? pos_fwd : pos_rev;
    const float cv = cs[pos * half + p], sv = sn[pos * half + p];
    x[i] = lo ? x[i] * cv - other[i] * sv : x[i] * cv + other[i] * sv;
  }
}

// ----------------------------------------------------------------------- depth attention
// One lane per 16-byte chunk of a row; LPH = d / VEC lanes per head (aligned groups in a
// wave).  Per row and head: rotate q and k_new (depth RoPE, half reversed), store the
// rotated key and the value into cache slot l, then stream slots 0..l with an online
// softmax.  The current slot is used from registers.
template <typename T, int LPH>
__global__ __launch_bounds__(256) void depth_attn_kernel(
    int64_t rows, int H, int d, int l, int L, const T* __restrict__ q, int64_t ldq,
    const T* __restrict__ kn, int64_t ldk, const T* __restrict__ vn, int64_t ldv,
    T* __restrict__ kc, T* __restrict__ vc, T* __restrict__ out, int64_t ldo,
    const float* __restrict__ cosd, const float* __restrict__ sind, float scale) {
  constexpr int VEC = Vec16<T>::N;
  const int h = H * d;
  const int cpr = h / VEC;  // chunks per row
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / cpr;
  if (row >= rows) return;  // whole heads leave together (cpr is a multiple of LPH)
  const int chunk = (int)(gid % cpr);
  const int c = chunk % LPH;
  const int col = chunk * VEC;

  float qv[VEC], kv[VEC], vv[VEC];
  load16(q + row * ldq + col, qv);
  load16(kn + row * ldk + col, kv);
  load16(vn + row * ldv + col, vv);
  rope_chunk<VEC, LPH>(qv, c, d, l, L - 1 - l, cosd, sind);
  rope_chunk<VEC, LPH>(kv, c, d, l, L - 1 - l, cosd, sind);
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    qv[i] = round_to<T>(qv[i]);
    kv[i] = round_to<T>(kv[i]);
  }
  T* krow = kc + row * (int64_t)L * h + col;
  T* vrow = vc + row * (int64_t)L * h + col;
  store16(krow + (int64_t)l * h, kv);
  store16(vrow + (int64_t)l * h, vv);

  float m = -INFINITY, lsum = 0.f, acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
  for (int j = 0; j <= l; ++j) {
    float kj[VEC], vj[VEC];
    if (j < l) {
      load16(krow + (int64_t)j * h, kj);
      load16(vrow + (int64_t)j * h, vj);
    } else {
#pragma unroll
      for (int i = 0; i < VEC; ++i) { kj[i] = kv[i]; vj[i] = vv[i]; }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) s = fmaf(qv[i], kj[i], s);
    s = group_sum<LPH>(s) * scale;
    const float mn = fmaxf(m, s);
    const float corr = expf(m - mn);  // exp(-inf) = 0 on the first key
    const float p = expf(s - mn);
    lsum = lsum * corr + p;
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = acc[i] * corr + p * vj[i];
    m = mn;
  }
  const float inv = 1.0f / lsum;
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] *= inv;
  store16(out + row * ldo + col, acc);
}

int launch_depth_attn(int dtype, int64_t rows, int H, int d, int l, int L, const void* q,
                      int64_t ldq, const void* kn, int64_t ldk, const void* vn, int64_t ldv,
                      void* kc, void* vc, void* out, int64_t ldo, const float* cosd,
                      const float* sind, float scale, hipStream_t st) {
  const int vec = dtype == DT_BF16 ? 8 : 4;
  const int lph = d / vec;
  const int64_t threads = rows * (int64_t)(H * d / vec);
  if (threads <= 0) return 0;
  const unsigned grid = (unsigned)((threads + 255) / 256);
#define DA_CASE(T, LP)                                                                  \
  depth_attn_kernel<T, LP><<<grid, 256, 0, st>>>(                                       \
      rows, H, d, l, L, (const T*)q, ldq, (const T*)kn, ldk, (const T*)vn, ldv, (T*)kc, \
      (T*)vc, (T*)out, ldo, cosd, sind, scale)
  if (dtype == DT_BF16) {
    switch (lph) {
      case 2: DA_CASE(bf16, 2); break;
      case 4: DA_CASE(bf16, 4); break;
      case 8: DA_CASE(bf16, 8); break;
      case 16: DA_CASE(bf16, 16); break;
      default: return -1;
    }
  } else {
    switch (lph) {
      case 2: DA_CASE(float, 2); break;
      case 4: DA_CASE(float, 4); break;
      case 8: DA_CASE(float, 8); break;
      case 16: DA_CASE(float, 16); break;
      case 32: DA_CASE(float, 32); break;
      default: return -1;
    }
  }
#undef DA_CASE
  return 0;
}

// ------------------------------------------------- SA: rotate new keys into a key buffer
// dst_k[b, pos0 + i] = RoPE_seq(k_new[b, i]) (rounded), dst_v[b, pos0 + i] = v_new[b, i].
template <typename T, int LPH>
__global__ __launch_bounds__(256) void sa_rope_store_kernel(
    int B, int n, int H, int d, int64_t pos0, const T* __restrict__ kn, int64_t ldk,
    const T* __restrict__ vn, int64_t ldv, T* __restrict__ dk, T* __restrict__ dv,
    int64_t cap, const float* __restrict__ cs, const float* __restrict__ sn, int rope) {
  constexpr int VEC = Vec16<T>::N;
  const int h = H * d, cpr = h / VEC;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / cpr;  // b * n + i
  if (row >= (int64_t)B * n) return;
  const int chunk = (int)(gid % cpr), c = chunk % LPH, col = chunk * VEC;
  const int64_t b = row / n, i = row % n, pos = pos0 + i;
  float kv[VEC], vv[VEC];
  load16(kn + row * ldk + col, kv);
  load16(vn + row * ldv + col, vv);
  if (rope) rope_chunk<VEC, LPH>(kv, c, d, (int)pos, (int)pos, cs, sn);
  const int64_t drow = (b * cap + pos) * h + col;
  store16(dk + drow, kv);
  store16(dv + drow, vv);
}

// ------------------------------------------------------- SA: row-streaming (any shape)
// One block per (query row, key split).  Threads = chunks of the row (h / VEC of them).
// Query (b, i) sits at position pos0 + i and sees keys 0..pos0+i of kbuf/vbuf
// ([B, cap, H, d], already rotated).  Split s covers keys [s*span, (s+1)*span).
// nsplit == 1: writes the normalised output; else (m, lsum, acc) partials.
template <typename T, int LPH>
__global__ void sa_rows_kernel(int B, int n, int H, int d, int64_t pos0, const T* __restrict__ q,
                               int64_t ldq, const T* __restrict__ kb, const T* __restrict__ vb,
                               int64_t cap, T* __restrict__ out, int64_t ldo,
                               const float* __restrict__ cs, const float* __restrict__ sn,
                               int rope, float scale, int nsplit, int span,
                               float* __restrict__ part_acc, float* __restrict__ part_ml) {
  constexpr int VEC = Vec16<T>::N;
  const int h = H * d;
  const int split = blockIdx.x;
  const int64_t row = blockIdx.y;  // b * n + i
  const int chunk = threadIdx.x, c = chunk % LPH, col = chunk * VEC;
  const int head = chunk / LPH;
  const int64_t b = row / n, i = row % n, qpos = pos0 + i;
  const int64_t k0 = (int64_t)split * span;
  const int64_t k1 = min((int64_t)(split + 1) * span, qpos + 1);
  if (chunk >= h / VEC) return;
  float qv[VEC];
  load16(q + row * ldq + col, qv);
  if (rope) rope_chunk<VEC, LPH>(qv, c, d, (int)qpos, (int)qpos, cs, sn);
#pragma unroll
  for (int e = 0; e < VEC; ++e) qv[e] = round_to<T>(qv[e]);
  float m = -INFINITY, lsum = 0.f, acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  const T* kp = kb + (b * cap) * h + col;
  const T* vp = vb + (b * cap) * h + col;
  for (int64_t j = k0; j < k1; ++j) {
    float kj[VEC], vj[VEC];
    load16(kp + j * h, kj);
    load16(vp + j * h, vj);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) s = fmaf(qv[e], kj[e], s);
    s = group_sum<LPH>(s) * scale;
    const float mn = fmaxf(m, s);
    const float corr = expf(m - mn), p = expf(s - mn);
    lsum = lsum * corr + p;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = acc[e] * corr + p * vj[e];
    m = mn;
  }
  if (nsplit == 1) {
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] *= inv;
    store16(out + row * ldo + col, acc);
    return;
  }
  float* pa = part_acc + (row * nsplit + split) * (int64_t)h + col;
#pragma unroll
  for (int e = 0; e < VEC; ++e) pa[e] = acc[e];
  if (c == 0) {
    float* pm = part_ml + ((row * nsplit + split) * (int64_t)H + head) * 2;
    pm[0] = m;
    pm[1] = lsum;
  }
}

template <typename T>
__global__ void sa_combine_kernel(int64_t nrows, int H, int d, int nsplit,
                                  const float* __restrict__ part_acc,
                                  const float* __restrict__ part_ml, T* __restrict__ out,
                                  int64_t ldo) {
  const int h = H * d;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / h;
  if (row >= nrows) return;
  const int col = (int)(gid % h), head = col / d;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s)
    M = fmaxf(M, part_ml[((row * nsplit + s) * H + head) * 2]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float ms = part_ml[((row * nsplit + s) * H + head) * 2];
    if (ms == -INFINITY) continue;  // empty split
    const float wgt = expf(ms - M);
    num += wgt * part_acc[(row * nsplit + s) * (int64_t)h + col];
    den += wgt * part_ml[((row * nsplit + s) * H + head) * 2 + 1];
  }
  out[row * ldo + col] = from_f<T>(num / den);
}

// ------------------------------------------------------------ SA: MFMA flash prefill
// bf16, d == 64.  Block = 4 waves = 64 queries of one (batch, head); wave w owns 16.
// S^T = K Q^T (keys on rows) so that every lane owns one query column: the online
// softmax statistics stay in the lane (plus the 4 lane groups, joined by two shuffles),
// and P feeds O^T = V^T P^T straight from registers.  K tiles (64 keys) are rotated
// while being staged into LDS; V tiles are staged transposed.
namespace fa {
constexpr int BQ = 64, BKEY = 64, D = 64, LDK = D + 8, LDV = BKEY + 8;
}

__global__ __launch_bounds__(256) void sa_flash_kernel(
    int B, int S, int H, const bf16* __restrict__ q, int64_t ldq, const bf16* __restrict__ kn,
    int64_t ldk, const bf16* __restrict__ vn, int64_t ldv, bf16* __restrict__ out,
    int64_t ldo, const float* __restrict__ cs, const float* __restrict__ sn, int rope,
    float scale) {
  using namespace fa;
  __shared__ __attribute__((aligned(16))) bf16 Ks[BKEY * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Vt[D * LDV];
  const int nqb = (S + BQ - 1) / BQ;
  const int qb = nqb - 1 - (int)blockIdx.x;  // heavy (late) query blocks first
  const int head = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t tok0 = (int64_t)b * S;
  const int hoff = head * D;
  constexpr int HALF = D / 2;

  // Q^T fragments: lane (query lr of wave w, group lg) holds dims 8lg..+8 (k-step 0)
  // and 32+8lg..+8 (k-step 1): one rotate-half pair, rotated in registers.
  const int qpos = qb * BQ + w * 16 + lr;
  const int qrow = min(qpos, S - 1);
  bf16x8 qf[2];
  {
    float a[8], bb[8];
    load16(q + (tok0 + qrow) * ldq + hoff + lg * 8, a);
    load16(q + (tok0 + qrow) * ldq + hoff + HALF + lg * 8, bb);
    if (rope) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int p = lg * 8 + i;
        const float cv = cs[qrow * HALF + p], sv = sn[qrow * HALF + p];
        const float x = a[i], y = bb[i];
        a[i] = x * cv - y * sv;
        bb[i] = y * cv + x * sv;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qf[0][i] = (bf16)a[i];
      qf[1][i] = (bf16)bb[i];
    }
  }
  const float sl2 = scale * 1.44269504088896341f;  // scale * log2(e)
  float m = -INFINITY, lsum = 0.f;
  floatx4 o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) o[t] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int qlast = min(qb * BQ + BQ, S) - 1;
  const int nkt = qlast / BKEY + 1;
  for (int kt = 0; kt < nkt; ++kt) {
    const int kbase = kt * BKEY;
    __syncthreads();
    {  // stage K (rotated): thread -> key tid/4, pair part tid%4
      const int key = tid >> 2, part = tid & 3;
      const int kp = kbase + key;
      float a[8], bb[8];
      if (kp < S) {
        load16(kn + (tok0 + kp) * ldk + hoff + part * 8, a);
        load16(kn + (tok0 + kp) * ldk + hoff + HALF + part * 8, bb);
        if (rope) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int p = part * 8 + i;
            const float cv = cs[kp * HALF + p], sv = sn[kp * HALF + p];
            const float x = a[i], y = bb[i];
            a[i] = x * cv - y * sv;
            bb[i] = y * cv + x * sv;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = bb[i] = 0.f;
      }
      bf16x8 va, vb;
#pragma unroll
      for (int i = 0; i < 8; ++i) { va[i] = (bf16)a[i]; vb[i] = (bf16)bb[i]; }
      *reinterpret_cast<bf16x8*>(&Ks[key * LDK + part * 8]) = va;
      *reinterpret_cast<bf16x8*>(&Ks[key * LDK + HALF + part * 8]) = vb;
    }
    {  // stage V transposed: thread -> key tid%64, dims 16*(tid/64)..+16
      const int key = tid & 63, dp = tid >> 6;
      const int kp = kbase + key;
      bf16x8 v0 = {}, v1 = {};
      if (kp < S) {
        v0 = *reinterpret_cast<const bf16x8*>(vn + (tok0 + kp) * ldv + hoff + dp * 16);
        v1 = *reinterpret_cast<const bf16x8*>(vn + (tok0 + kp) * ldv + hoff + dp * 16 + 8);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        Vt[(dp * 16 + i) * LDV + key] = v0[i];
        Vt[(dp * 16 + 8 + i) * LDV + key] = v1[i];
      }
    }
    __syncthreads();

    // S^T tiles: 4 key tiles of 16, K = 64 dims in two steps.
    floatx4 sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sacc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(&Ks[(t * 16 + lr) * LDK + ks * 32 + lg * 8]);
        sacc[t] = mfma16(kf, qf[ks], sacc[t]);
      }
    }
    // mask + tile max (lane holds keys kbase + 16t + 4lg + i for query qpos)
    float tmax = -INFINITY;
    const int qlim = min(qpos, S - 1);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kp = kbase + t * 16 + lg * 4 + i;
        if (kp > qlim) sacc[t][i] = -INFINITY;
        tmax = fmaxf(tmax, sacc[t][i]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mn = fmaxf(m, tmax);
    const float corr = exp2f((m - mn) * sl2);
    m = mn;
    lsum *= corr;
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] *= corr;
    // P^T fragments for the two 32-key chunks (slot j < 4: tile 2c, j >= 4: tile 2c+1).
    // P = hi + lo, both bf16, so P V keeps ~16 mantissa bits of P (a single bf16 P
    // would perturb every output by up to 2^-9 max|v|).
    bf16x8 ph[2], pl[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float sv = sacc[2 * cc + (j >> 2)][j & 3];
        const float p = exp2f((sv - mn) * sl2);
        lsum += p;
        const bf16 hi = (bf16)p;
        ph[cc][j] = hi;
        pl[cc][j] = (bf16)(p - (float)hi);
      }
    // O^T += V^T P^T : 4 dim tiles x 2 key chunks
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const bf16* vrow = &Vt[(t * 16 + lr) * LDV + cc * 32 + lg * 4];
        bf16x8 vf;
        const bf16x4 lo4 = *reinterpret_cast<const bf16x4*>(vrow);
        const bf16x4 hi4 = *reinterpret_cast<const bf16x4*>(vrow + 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) { vf[j] = lo4[j]; vf[4 + j] = hi4[j]; }
        o[t] = mfma16(vf, ph[cc], o[t]);
        o[t] = mfma16(vf, pl[cc], o[t]);
      }
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (qpos >= S) return;
  const float inv = 1.0f / lsum;
  bf16* orow = out + (tok0 + qpos) * ldo + hoff;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (bf16)(o[t][i] * inv);
    *reinterpret_cast<bf16x4*>(orow + t * 16 + lg * 4) = v;
  }
}

// ------------------------------------------------------------------------------ launch
static int lph_of(int dtype, int d) { return d / (dtype == DT_BF16 ? 8 : 4); }

constexpr int SA_SPLIT_SPAN = 256;

size_t seq_attn_ws(int dtype, int B, int q_len, int H, int d, int64_t pos0) {
  const size_t es = dtype == DT_BF16 ? 2 : 4;
  const size_t h = (size_t)H * d;
  if (pos0 > 0) {  // decode: split partials
    const int nsplit = (int)((pos0 + 1 + SA_SPLIT_SPAN - 1) / SA_SPLIT_SPAN);
    const size_t rows = (size_t)B * q_len;
    return rows * nsplit * h * 4 + rows * nsplit * H * 2 * 4 + 512;
  }
  if (dtype == DT_BF16 && d == 64) return 0;  // flash kernel reads q/k/v directly
  return 2 * (size_t)B * q_len * h * es + 512;  // rotated key / value buffers
}

template <typename T>
static int sa_rope_store(int lph, int B, int n, int H, int d, int64_t pos0, const void* kn,
                         int64_t ldk, const void* vn, int64_t ldv, void* dk, void* dv,
                         int64_t cap, const float* cs, const float* sn, int rope,
                         hipStream_t st) {
  constexpr int VEC = Vec16<T>::N;
  const int64_t threads = (int64_t)B * n * (H * d / VEC);
  const unsigned grid = (unsigned)((threads + 255) / 256);
#define RS_CASE(LP)                                                                  \
  sa_rope_store_kernel<T, LP><<<grid, 256, 0, st>>>(B, n, H, d, pos0, (const T*)kn, \
                                                    ldk, (const T*)vn, ldv, (T*)dk,  \
                                                    (T*)dv, cap, cs, sn, rope)
  switch (lph) {
    case 2: RS_CASE(2); break;
    case 4: RS_CASE(4); break;
    case 8: RS_CASE(8); break;
    case 16: RS_CASE(16); break;
    default: return -1;
  }
#undef RS_CASE
  return 0;
}

template <typename T>
static int sa_rows(int lph, int B, int n, int H, int d, int64_t pos0, const void* q,
                   int64_t ldq, const void* kb, const void* vb, int64_t cap, void* out,
                   int64_t ldo, const float* cs, const float* sn, int rope, float scale,
                   int nsplit, int span, float* pa, float* pm, hipStream_t st) {
  constexpr int VEC = Vec16<T>::N;
  const int threads = H * d / VEC;
  const int blk = ((threads + 63) / 64) * 64;
  if (blk > 1024) return -1;
  dim3 grid(nsplit, (unsigned)((int64_t)B * n));
#define SR_CASE(LP)                                                                    \
  sa_rows_kernel<T, LP><<<grid, blk, 0, st>>>(B, n, H, d, pos0, (const T*)q, ldq,      \
                                              (const T*)kb, (const T*)vb, cap, (T*)out, \
                                              ldo, cs, sn, rope, scale, nsplit, span, pa, pm)
  switch (lph) {
    case 2: SR_CASE(2); break;
    case 4: SR_CASE(4); break;
    case 8: SR_CASE(8); break;
    case 16: SR_CASE(16); break;
    default: return -1;
  }
#undef SR_CASE
  if (nsplit > 1) {
    const int64_t tot = (int64_t)B * n * H * d;
    sa_combine_kernel<T><<<(unsigned)((tot + 255) / 256), 256, 0, st>>>(
        (int64_t)B * n, H, d, nsplit, pa, pm, (T*)out, ldo);
  }
  return 0;
}

int launch_seq_attn(int dtype, int B, int q_len, int H, int d, int64_t pos0, const void* q,
                    int64_t ldq, const void* kn, int64_t ldk, const void* vn, int64_t ldv,
                    void* kc, void* vc, int64_t cap, void* out, int64_t ldo,
                    const float* cos_s, const float* sin_s, float scale, int sa_rope,
                    void* ws, size_t ws_bytes, hipStream_t st) {
  const int lph = lph_of(dtype, d);
  const size_t es = dtype == DT_BF16 ? 2 : 4;
  const int64_t h = (int64_t)H * d;
  if (B <= 0 || q_len <= 0) return 0;
  if (ws_bytes < seq_attn_ws(dtype, B, q_len, H, d, pos0)) return -2;
  const bool bf = dtype == DT_BF16;
  if (pos0 > 0) {
    // decode: append the rotated new key/value at pos0, then split-K over 0..pos0
    int rc = bf ? sa_rope_store<bf16>(lph, B, q_len, H, d, pos0, kn, ldk, vn, ldv, kc, vc,
                                      cap, cos_s, sin_s, sa_rope, st)
                : sa_rope_store<float>(lph, B, q_len, H, d, pos0, kn, ldk, vn, ldv, kc, vc,
                                       cap, cos_s, sin_s, sa_rope, st);
    if (rc) return rc;
    const int nsplit = (int)((pos0 + 1 + SA_SPLIT_SPAN - 1) / SA_SPLIT_SPAN);
    float* pa = (float*)ws;
    float* pm = pa + (size_t)B * q_len * nsplit * h;
    return bf ? sa_rows<bf16>(lph, B, q_len, H, d, pos0, q, ldq, kc, vc, cap, out, ldo,
                              cos_s, sin_s, sa_rope, scale, nsplit, SA_SPLIT_SPAN, pa, pm, st)
              : sa_rows<float>(lph, B, q_len, H, d, pos0, q, ldq, kc, vc, cap, out, ldo,
                               cos_s, sin_s, sa_rope, scale, nsplit, SA_SPLIT_SPAN, pa, pm,
                               st);
  }
  // prefill
  if (kc) {
    int rc = bf ? sa_rope_store<bf16>(lph, B, q_len, H, d, 0, kn, ldk, vn, ldv, kc, vc, cap,
                                      cos_s, sin_s, sa_rope, st)
                : sa_rope_store<float>(lph, B, q_len, H, d, 0, kn, ldk, vn, ldv, kc, vc, cap,
                                       cos_s, sin_s, sa_rope, st);
    if (rc) return rc;
  }
  if (bf && d == 64) {
    dim3 grid((q_len + fa::BQ - 1) / fa::BQ, H, B);
    sa_flash_kernel<<<grid, 256, 0, st>>>(B, q_len, H, (const bf16*)q, ldq, (const bf16*)kn,
                                          ldk, (const bf16*)vn, ldv, (bf16*)out, ldo, cos_s,
                                          sin_s, sa_rope, scale);
    return 0;
  }
  // generic: rotated keys into ws, then one row-streaming pass
  char* kb = (char*)ws;
  char* vb = kb + (size_t)B * q_len * h * es;
  int rc = bf ? sa_rope_store<bf16>(lph, B, q_len, H, d, 0, kn, ldk, vn, ldv, kb, vb, q_len,
                                    cos_s, sin_s, sa_rope, st)
              : sa_rope_store<float>(lph, B, q_len, H, d, 0, kn, ldk, vn, ldv, kb, vb, q_len,
                                     cos_s, sin_s, sa_rope, st);
  if (rc) return rc;
  return bf ? sa_rows<bf16>(lph, B, q_len, H, d, 0, q, ldq, kb, vb, q_len, out, ldo, cos_s,
                            sin_s, sa_rope, scale, 1, q_len, nullptr, nullptr, st)
            : sa_rows<float>(lph, B, q_len, H, d, 0, q, ldq, kb, vb, q_len, out, ldo, cos_s,
                             sin_s, sa_rope, scale, 1, q_len, nullptr, nullptr, st);
}

}  // namespace dreamer
