// Attention kernels: depth attention (DA), causal sequence attention (SA) prefill with
// MFMA, and a row-streaming SA kernel used for decode (split over key ranges) and for
// shapes outside the MFMA kernel.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dreamer {

// ------------------------------------------------------------------------- RoPE tables
// Split tables of head dim D: c[p * D/2 + j] = cos(p th_j), s[...] = sin(p th_j), with
// th_j = base^(-2j/D), evaluated in float64 and rounded once.
// Interleaved tables of head dim 64 (the QKV epilogue's): t[p * 16 + j] =
// (cos p th_j, cos p th_{j+16}, sin p th_j, sin p th_{j+16}), the same values.
// One launch fills every table of a RopeJobs set: thread i walks the jobs in order.
__global__ void rope_jobs_kernel(RopeJobs jobs) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int q = 0; q < jobs.n; ++q) {
    const RopeJob& jb = jobs.j[q];
    const int per = jb.t4 ? 16 : jb.D / 2;
    const int64_t n = (int64_t)jb.npos * per;
    if (i >= n) {
      i -= n;
      continue;
    }
    const int p = (int)(i / per), j = (int)(i % per);
    if (jb.t4) {
      const double a0 = (double)p * pow(jobs.base, -2.0 * (double)j / 64.0);
      const double a1 = (double)p * pow(jobs.base, -2.0 * (double)(j + 16) / 64.0);
      jb.t4[i] = make_float4((float)cos(a0), (float)cos(a1), (float)sin(a0), (float)sin(a1));
    } else {
      const double ang = (double)p * pow(jobs.base, -2.0 * (double)j / (double)jb.D);
      jb.c[i] = (float)cos(ang);
      jb.s[i] = (float)sin(ang);
    }
    return;
  }
}

void launch_rope_jobs(const RopeJobs& jobs, hipStream_t st) {
  int64_t n = 0;
  for (int q = 0; q < jobs.n; ++q)
    n += (int64_t)jobs.j[q].npos * (jobs.j[q].t4 ? 16 : jobs.j[q].D / 2);
  if (n <= 0) return;
  dlaunch(rope_jobs_kernel, (unsigned)((n + 255) / 256), 256, 0, st, jobs);
}

void launch_rope_tables(int D, int npos, double base, float* c, float* s, hipStream_t st) {
  RopeJobs jobs;
  jobs.base = base;
  jobs.add_split(D, npos, c, s);
  launch_rope_jobs(jobs, st);
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
    x[i] = lo ? rot_first(x[i], other[i], cv, sv) : rot_second(x[i], other[i], cv, sv);
  }
}

// ----------------------------------------------------------------------- depth attention
// One lane per 16-byte chunk of a row; LPH = d / VEC lanes per head (aligned groups in a
// wave).  Per row and head: (ROPE) rotate q and k_new by depth, half reversed, and round
// them to storage precision; store the key and the value into cache slot l, then stream
// slots 0..l with an online softmax.  The current slot is used from registers.
// window > 0 keeps only the slots l-window+1..l and, with dilation > 0, the older slots j
// with (l - j) divisible by dilation; the skipped slots are never loaded.
// Block blk of 256 threads (the body of depth_attn_kernel and of the paired launch).
// NT: the cache's older slots are read with nontemporal loads.
template <typename T, int LPH, bool ROPE, bool NT = false, int NB_ = 2>
DEV void depth_attn_block(
    int64_t blk, int64_t rows, int H, int d, int l, int L, const T* __restrict__ q,
    int64_t ldq, const T* __restrict__ kn, int64_t ldk, const T* __restrict__ vn, int64_t ldv,
    T* __restrict__ kc, T* __restrict__ vc, T* __restrict__ out, int64_t ldo,
    const float* __restrict__ cosd, const float* __restrict__ sind, float scale, int window,
    int dilation, int64_t srow, int64_t sslot) {
  constexpr int VEC = Vec16<T>::N;
  const int h = H * d;
  const int cpr = h / VEC;  // chunks per row
  const int64_t gid = blk * 256 + threadIdx.x;
  const int64_t row = gid / cpr;
  if (row >= rows) return;  // whole heads leave together (cpr is a multiple of LPH)
  const int chunk = (int)(gid % cpr);
  const int col = chunk * VEC;

  float qv[VEC], kv[VEC], vv[VEC];
  load16(q + row * ldq + col, qv);
  load16(kn + row * ldk + col, kv);
  load16(vn + row * ldv + col, vv);
  if constexpr (ROPE) {
    const int c = chunk % LPH;
    rope_chunk<VEC, LPH>(qv, c, d, l, L - 1 - l, cosd, sind);
    rope_chunk<VEC, LPH>(kv, c, d, l, L - 1 - l, cosd, sind);
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      qv[i] = round_to<T>(qv[i]);
      kv[i] = round_to<T>(kv[i]);
    }
  }
  // the cache: row `row`'s slot j at kc + row srow + j sslot ([rows, L, h]: srow = L h,
  // sslot = h; slot-major [L, rows, h]: srow = h, sslot = rows h)
  T* krow = kc + row * srow + col;
  T* vrow = vc + row * srow + col;
  // k_new / v_new may already be the cache's slot l (the layer's projection writes them
  // there); then they are not stored again
  if (ROPE || kn + row * ldk + col != krow + (int64_t)l * sslot) store16(krow + (int64_t)l * sslot, kv);
  if (vn + row * ldv + col != vrow + (int64_t)l * sslot) store16(vrow + (int64_t)l * sslot, vv);

  // The current slot first (from registers), so the running max starts finite; then the
  // older slots in batches of NB whose loads are issued together (the key test is the
  // same for every lane, so whole waves take or skip a slot).
  float m, lsum = 1.f, acc[VEC];
  {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      s = fmaf(qv[i], kv[i], s);
      acc[i] = vv[i];
    }
    m = group_sum<LPH>(s) * scale;
  }
  // NB_ slots per batch (two batches in flight).  Two (eight 16-byte loads in flight) was
  // measured faster than four in DA's own launch (8192 rows of 32 heads, 64 depths), most
  // at the first depths, where a batch of four mostly re-reads clamped slots.
  constexpr int NB = NB_;
  // One batch of NB slots from raw 16-byte chunks: scores, one max and rescale for the
  // batch, then the weighted values (slots j >= l, or outside the key set, are skipped).
  typedef uint32_t raw16 __attribute__((ext_vector_type(4)));
  auto unpack = [&](raw16 r, float* out) {
    if constexpr (sizeof(T) == 2) {
      const bf16x8 v = __builtin_bit_cast(bf16x8, r);
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
    } else {
      const floatx4 v = __builtin_bit_cast(floatx4, r);
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = v[i];
    }
  };
  auto batch = [&](int j0, const raw16 (&kr)[NB], const raw16 (&vr)[NB]) {
    bool use[NB];
    float s[NB], bm = m;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = j0 + b;
      use[b] = j < l && !(window > 0 && l - j >= window && (dilation <= 0 || (l - j) % dilation));
      if (!use[b]) continue;
      float kj[VEC];
      unpack(kr[b], kj);
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) t = fmaf(qv[i], kj[i], t);
      s[b] = group_sum<LPH>(t) * scale;
      bm = fmaxf(bm, s[b]);
    }
    const float corr = __expf(m - bm);
    lsum *= corr;
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] *= corr;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (!use[b]) continue;
      const float p = __expf(s[b] - bm);
      lsum += p;
      float vj[VEC];
      unpack(vr[b], vj);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = fmaf(p, vj[i], acc[i]);
    }
    m = bm;
  };
  if (window <= 0) {
    // every older slot: unconditional loads (slot indices clamped into 0..l-1), the next
    // batch's loads issued before this batch's arithmetic
    auto load = [&](raw16 (&kr)[NB], raw16 (&vr)[NB], int j0) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int64_t jc = min(j0 + b, l - 1);
        const raw16* kp = reinterpret_cast<const raw16*>(krow + jc * sslot);
        const raw16* vp = reinterpret_cast<const raw16*>(vrow + jc * sslot);
        if constexpr (NT) {  // a cache far larger than the caches: stream it past them
          kr[b] = __builtin_nontemporal_load(kp);
          vr[b] = __builtin_nontemporal_load(vp);
        } else {
          kr[b] = *kp;
          vr[b] = *vp;
        }
      }
    };
    raw16 ka[NB], va[NB], kb[NB], vb[NB];
    if (l > 0) load(ka, va, 0);
    for (int j0 = 0; j0 < l; j0 += 2 * NB) {
      load(kb, vb, j0 + NB);
      batch(j0, ka, va);
      if (j0 + NB >= l) break;  // the same in every lane
      load(ka, va, j0 + 2 * NB);
      batch(j0 + NB, kb, vb);
    }
  } else {
    // a key set: the slots outside it are not loaded
    for (int j0 = 0; j0 < l; j0 += NB) {
      raw16 kr[NB], vr[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int j = j0 + b;
        if (j < l && !(l - j >= window && (dilation <= 0 || (l - j) % dilation))) {
          kr[b] = *reinterpret_cast<const raw16*>(krow + (int64_t)j * sslot);
          vr[b] = *reinterpret_cast<const raw16*>(vrow + (int64_t)j * sslot);
        }
      }
      batch(j0, kr, vr);
    }
  }
  const float inv = 1.0f / lsum;
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] *= inv;
  store16(out + row * ldo + col, acc);
}

template <typename T, int LPH, bool ROPE, bool NT>
__global__ __launch_bounds__(256) void depth_attn_kernel(
    int64_t rows, int H, int d, int l, int L, const T* __restrict__ q, int64_t ldq,
    const T* __restrict__ kn, int64_t ldk, const T* __restrict__ vn, int64_t ldv,
    T* __restrict__ kc, T* __restrict__ vc, T* __restrict__ out, int64_t ldo,
    const float* __restrict__ cosd, const float* __restrict__ sind, float scale, int window,
    int dilation, int64_t srow, int64_t sslot) {
  depth_attn_block<T, LPH, ROPE, NT>(blockIdx.x, rows, H, d, l, L, q, ldq, kn, ldk, vn, ldv, kc, vc,
                                 out, ldo, cosd, sind, scale, window, dilation, srow, sslot);
}

int launch_depth_attn(int dtype, int64_t rows, int H, int d, int l, int L, const void* q,
                      int64_t ldq, const void* kn, int64_t ldk, const void* vn, int64_t ldv,
                      void* kc, void* vc, void* out, int64_t ldo, const float* cosd,
                      const float* sind, float scale, int rope, hipStream_t st, int window,
                      int dilation, int64_t srow, int64_t sslot) {
  const int vec = dtype == DT_BF16 ? 8 : 4;
  if (srow <= 0) {  // [rows, L, h]
    srow = (int64_t)L * H * d;
    sslot = (int64_t)H * d;
  }
  const int lph = d / vec;
  const int64_t threads = rows * (int64_t)(H * d / vec);
  if (threads <= 0) return 0;
  const unsigned grid = (unsigned)((threads + 255) / 256);
  // nontemporal loads once the K and V caches exceed what the last-level caches hold well
  // (measured: faster at 4 GiB, slower at 64 MiB, where the slots stay cached)
  const bool nt = 2 * rows * (int64_t)L * H * d * (dtype == DT_BF16 ? 2 : 4) > ((int64_t)256 << 20);
#define DA_LAUNCH(T, LP, R)                                                              \
  if (nt) dlaunch(depth_attn_kernel<T, LP, R, true>, grid, 256, 0, st,                        \
      rows, H, d, l, L, (const T*)q, ldq, (const T*)kn, ldk, (const T*)vn, ldv, (T*)kc, \
      (T*)vc, (T*)out, ldo, cosd, sind, scale, window, dilation, srow, sslot);             \
  else dlaunch(depth_attn_kernel<T, LP, R, false>, grid, 256, 0, st,                          \
      rows, H, d, l, L, (const T*)q, ldq, (const T*)kn, ldk, (const T*)vn, ldv, (T*)kc, \
      (T*)vc, (T*)out, ldo, cosd, sind, scale, window, dilation, srow, sslot)
#define DA_CASE(T, LP)                 \
  if (rope) DA_LAUNCH(T, LP, true);    \
  else DA_LAUNCH(T, LP, false);        \
  break;
  if (dtype == DT_BF16) {
    switch (lph) {
      case 2: DA_CASE(bf16, 2)
      case 4: DA_CASE(bf16, 4)
      case 8: DA_CASE(bf16, 8)
      case 16: DA_CASE(bf16, 16)
      default: return -1;
    }
  } else {
    switch (lph) {
      case 2: DA_CASE(float, 2)
      case 4: DA_CASE(float, 4)
      case 8: DA_CASE(float, 8)
      case 16: DA_CASE(float, 16)
      case 32: DA_CASE(float, 32)
      default: return -1;
    }
  }
#undef DA_CASE
#undef DA_LAUNCH
  return 0;
}

// --------------------------------------------- in-place RoPE of a [T, 6h] QKV buffer
// Rotates SA q/k by sequence position (when sa_rope) and DA q/k by depth; used where
// the projection kernel does not rotate in its epilogue (float32 storage).
template <typename T, int LPH>
__global__ __launch_bounds__(256) void qkv_rope_kernel(int64_t rows, int H, int d, int seq,
                                                       int pos_fixed, int sa_rope, int l,
                                                       int L, T* __restrict__ qkv,
                                                       const float* __restrict__ cs,
                                                       const float* __restrict__ sn,
                                                       const float* __restrict__ cd,
                                                       const float* __restrict__ sd) {
  constexpr int VEC = Vec16<T>::N;
  const int h = H * d, cpr = h / VEC;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t unit = gid / cpr;  // (row, section in {SA q, SA k, DA q, DA k})
  if (unit >= rows * 4) return;
  const int64_t row = unit >> 2;
  const int sec = (int)(unit & 3);
  const int chunk = (int)(gid % cpr), c = chunk % LPH;
  const int col = (sec < 2 ? sec : sec + 1) * h + chunk * VEC;
  T* p = qkv + row * 6 * (int64_t)h + col;
  float x[VEC];
  load16(p, x);
  if (sec < 2) {
    if (!sa_rope) return;  // whole rows of a section leave together
    const int pos = pos_fixed >= 0 ? pos_fixed : (int)(row % seq);
    rope_chunk<VEC, LPH>(x, c, d, pos, pos, cs, sn);
  } else {
    rope_chunk<VEC, LPH>(x, c, d, l, L - 1 - l, cd, sd);
  }
  store16(p, x);
}

int launch_qkv_rope(int dtype, int64_t rows, int H, int d, int seq, int pos_fixed,
                    int sa_rope, int l, int L, void* qkv, const float* cs, const float* sn,
                    const float* cd, const float* sd, hipStream_t st) {
  const int vec = dtype == DT_BF16 ? 8 : 4;
  const int lph = d / vec;
  const int64_t threads = rows * 4 * (int64_t)(H * d / vec);
  if (threads <= 0) return 0;
  const unsigned grid = (unsigned)((threads + 255) / 256);
#define QR_CASE(T, LP)                                                                   \
  dlaunch(qkv_rope_kernel<T, LP>, grid, 256, 0, st, rows, H, d, seq, pos_fixed, sa_rope, l, L, \
                                               (T*)qkv, cs, sn, cd, sd);                 \
  break;
  if (dtype == DT_BF16) {
    switch (lph) {
      case 2: QR_CASE(bf16, 2)
      case 4: QR_CASE(bf16, 4)
      case 8: QR_CASE(bf16, 8)
      case 16: QR_CASE(bf16, 16)
      default: return -1;
    }
  } else {
    switch (lph) {
      case 2: QR_CASE(float, 2)
      case 4: QR_CASE(float, 4)
      case 8: QR_CASE(float, 8)
      case 16: QR_CASE(float, 16)
      default: return -1;
    }
  }
#undef QR_CASE
  return 0;
}

// ------------------------------------------------- SA: rotate new keys into a key buffer
// dst_k[b, pos0 + i] = RoPE_seq(k_new[b, i]) (rounded; a copy when rope == 0),
// dst_v[b, pos0 + i] = v_new[b, i].
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
// One wave per (query row, key split, group of 64 chunks of the row): thread = chunk of the
// row (h / VEC of them; a head's LPH chunks lie in one wave).  One-wave blocks spread the
// work evenly over the CUs (a block per row and split left some CUs one block more than
// others, all streaming at the per-CU load rate).  Query (b, i) sits at position pos0 + i
// and sees keys 0..pos0+i of kbuf/vbuf ([B, cap, H, d], already rotated).  Split s covers
// keys [s*span, (s+1)*span).  nsplit == 1: writes the normalised output; else (m, lsum,
// acc) partials.
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
  const int chunk = blockIdx.z * blockDim.x + threadIdx.x, c = chunk % LPH, col = chunk * VEC;
  const int head = chunk / LPH;
  const int64_t b = row / n, i = row % n, qpos = pos0 + i;
  const int64_t k0 = (int64_t)split * span;
  const int64_t k1 = min((int64_t)(split + 1) * span, qpos + 1);
  if (chunk >= h / VEC) return;
  float qv[VEC];
  load16(q + row * ldq + col, qv);
  if (rope) {
    rope_chunk<VEC, LPH>(qv, c, d, (int)qpos, (int)qpos, cs, sn);
#pragma unroll
    for (int e = 0; e < VEC; ++e) qv[e] = round_to<T>(qv[e]);
  }
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
// bf16, d == 64, q/k already rotated, v given transposed per (batch, head):
// vt [B][H][64][S].  Block = 4 waves = 64 queries of one (batch, head); wave w owns 16.
// S^T = K Q^T (keys on rows) so that every lane owns one query column: the online
// softmax statistics stay in the lane (plus the 4 lane groups, joined by two shuffles),
// and P feeds O^T = V^T P^T straight from registers.  K and V^T tiles of 64 keys stream
// through a 3-stage LDS ring filled by direct global->LDS loads (128-byte rows, 16-byte
// chunks XOR-swizzled by row).  The K tile's rows hold the keys in the order key_of_row,
// which makes the 8 P values a lane feeds to one MFMA 8 consecutive keys, so each V^T
// fragment is one 16-byte read.  Requires S % 8 == 0.
namespace fa {
constexpr int BQ = 64, BKEY = 64, NSTG = 3, TILE = 8192;  // bytes per K or V^T tile
}
// Largest excess (exp2 units) of a score over its query's reference maximum before the
// flash kernels rescale: P stays <= 2^8.
constexpr float SA_LAZY = 8.0f;

DEV int swz128(int row, int c) { return row * 64 + ((c ^ (row & 7)) << 3); }  // elements

// Key (within a 64-key tile) held by K-tile row r = 32 cc + 16 h + 4 g + i: the S^T tile
// t = 2 cc + h gives lane group g the keys 32 cc + 8 g + 4 h + i.
DEV int key_of_row(int r) {
  return (r & 32) + ((r >> 2) & 3) * 8 + ((r >> 4) & 1) * 4 + (r & 3);
}

// Query block qbx (counted from the last: heavy blocks first), head, batch b; stg: the
// block's 3 x 16 KiB ring in LDS (1 KiB aligned).
DEV void sa_flash_block(int qbx, int head, int b, int S, int H, const bf16* __restrict__ q,
                        int64_t ldq, const bf16* __restrict__ kk, int64_t ldk,
                        const bf16* __restrict__ vt, bf16* __restrict__ out, int64_t ldo,
                        float scale, char (*stg)[2 * fa::TILE]) {
  using namespace fa;
  const int nqb = (S + BQ - 1) / BQ;
  const int qb = nqb - 1 - qbx;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t tok0 = (int64_t)b * S;
  const int hoff = head * 64;

  // Q^T fragments: lane (query lr of wave w, group lg) holds dims 8lg..+8 (k-step 0)
  // and 32+8lg..+8 (k-step 1)
  const int qpos = qb * BQ + w * 16 + lr;
  const int qrow = min(qpos, S - 1);
  bf16x8 qf[2];
  qf[0] = *reinterpret_cast<const bf16x8*>(q + (tok0 + qrow) * ldq + hoff + lg * 8);
  qf[1] = *reinterpret_cast<const bf16x8*>(q + (tok0 + qrow) * ldq + hoff + 32 + lg * 8);

  // loads of one stage: 16 instructions of 1 KiB (8 for K rows, 8 for V^T rows); wave w
  // issues instructions j = w + 4 i (i < 2: K rows, i >= 2: V^T rows).  Lane -> (row
  // lane/8, slot lane%8) of 8 rows.  Tiles inside the sequence advance precomputed
  // pointers by one tile; the last, partial tile clamps its rows into the sequence.
  const int lrow = lane >> 3, slot = lane & 7;
  const bf16* vbase = vt + ((int64_t)(b * H + head) * 64) * S;
  auto tile_src = [&](int i, int kbase) -> const bf16* {
    const int j = w + 4 * i;
    if (i < 2) {  // K rows (keys in key_of_row order)
      const int row = j * 8 + lrow;
      const int kp = min(kbase + key_of_row(row), S - 1);
      return kk + (tok0 + kp) * ldk + hoff + (slot ^ (row & 7)) * 8;
    }
    const int dim = (j - 8) * 8 + lrow;  // V^T rows (dims)
    const int p0 = min(kbase + (slot ^ (dim & 7)) * 8, S - 8);
    return vbase + (int64_t)dim * S + p0;
  };
  // whole tiles: a base the same in every lane (advanced by the tile) plus this lane's
  // 32-bit byte offset, so the per-tile address work is scalar
  const char* kb_u = reinterpret_cast<const char*>(kk + tok0 * ldk + hoff);
  const char* vb_u = reinterpret_cast<const char*>(vbase);
  uint32_t loff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = w + 4 * i;
    if (i < 2) {
      const int row = j * 8 + lrow;
      loff[i] = (uint32_t)((key_of_row(row) * ldk + (slot ^ (row & 7)) * 8) * 2);
    } else {
      const int dim = (j - 8) * 8 + lrow;
      loff[i] = (uint32_t)(((int64_t)dim * S + (slot ^ (dim & 7)) * 8) * 2);
    }
  }
  auto issue = [&](int t) {
    char* sb = stg[t % NSTG];
    const int kbase = t * BKEY;
    const bool whole = kbase + BKEY <= S;
    const char* kt_u = kb_u + (int64_t)kbase * ldk * 2;
    const char* vt_u = vb_u + (int64_t)kbase * 2;
    if (whole) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds((const void*)((i < 2 ? kt_u : vt_u) + loff[i]),
                                         (lds_void*)(sb + (w + 4 * i) * 1024), 16, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds((const void*)tile_src(i, kbase),
                                         (lds_void*)(sb + (w + 4 * i) * 1024), 16, 0, 0);
    }
  };

  const float sl2 = scale * 1.44269504088896341f;  // scale * log2(e)
  const float lazy_thr = SA_LAZY / sl2;             // in score units
  float m = -INFINITY;
  floatx4 o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) o[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  // The softmax denominator comes from the P.V MFMAs: an extra A fragment whose row 0 is
  // all ones turns that row of the product into the sum of the (bf16) P of each query,
  // held by the lane of group 0 that owns the query (element 0 of osum).
  floatx4 osum = {0.f, 0.f, 0.f, 0.f};
  bf16x8 ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = (bf16)(lr == 0 ? 1.f : 0.f);

  const int qlast = min(qb * BQ + BQ, S) - 1;
  const int qlim = min(qpos, S - 1);
  const int nkt = qlast / BKEY + 1;
  const uint32_t stg0 = lds_off(stg[0]);
  // per-lane fragment offsets within a tile (row lr; tile rows 16t + lr follow at 2048 t)
  const uint32_t kofs0 = 2 * swz128(lr, lg), kofs1 = 2 * swz128(lr, 4 + lg);
  const uint32_t vofs0 = kofs0, vofs1 = kofs1;
  issue(0);
  if (nkt > 1) issue(1);
  // The Q fragments, loaded before the ring, are taken through an empty asm statement:
  // the compiler waits for their loads there (only the ring loads issued later stay
  // outstanding) and then sees them as plain register values, so their first use inside
  // the loop does not drain the ring.
  asm volatile("" : "+v"(qf[0]), "+v"(qf[1]));
  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) wait_vmcnt<4>();
    else wait_vmcnt<0>();
    ring_barrier();  // tile kt visible to all waves; tile kt-1 consumed by all
    if (kt + 2 < nkt) issue(kt + 2);
    const uint32_t ks0 = stg0 + (kt % NSTG) * 2 * TILE, vs0 = ks0 + TILE;
    const int kbase = kt * BKEY;

    // S^T tiles: 4 key tiles of 16, K = 64 dims in two steps.  Row 16t + lr of a tile
    // sits 2048 t bytes after row lr (kf[t]: dims 0..31, kf[4 + t]: dims 32..63).
    bf16x8 kf[8];
    lds_read_b128_2x4<2048>(kf, ks0 + kofs0, ks0 + kofs1);
    floatx4 sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sacc[t] = mfma16(kf[t], qf[0], floatx4{0.f, 0.f, 0.f, 0.f});
      sacc[t] = mfma16(kf[4 + t], qf[1], sacc[t]);
    }
    // causal mask on the diagonal tile (lane holds keys kbase + 32(t/2) + 8lg + 4(t%2) + i
    // for query qpos), then the tile max
    if (kbase + BKEY - 1 > qb * BQ) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kbase + (t >> 1) * 32 + lg * 8 + (t & 1) * 4 + i > qlim) sacc[t][i] = -INFINITY;
    }
    // Lazy rescaling: the reference m of each query moves only when one of this tile's
    // scores exceeds it by more than SA_LAZY (2^8 in exp2 units), so P <= 256; softmax
    // is invariant to the reference, and the rescale (a cross-lane max, one exp2 and 20
    // multiplications) is skipped in almost every tile.
    float lmax = -INFINITY;  // this lane's 16 scores
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) lmax = fmaxf(lmax, sacc[t][i]);
    if (__any(lmax > m + lazy_thr)) {
      const float mn = fmaxf(m, max_xor32(max_xor16(lmax)));
      const float corr = __builtin_amdgcn_exp2f((m - mn) * sl2);
      m = mn;
      osum *= corr;
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] *= corr;
    }
    // P^T fragments for the two 32-key chunks: element j of lane group lg is key
    // 32cc + 8lg + j (tile 2cc for j < 4, tile 2cc+1 for j >= 4).  P is rounded to bf16
    // (pairwise conversions) for the MFMA, numerator and denominator alike.
    bf16x8 ph[2];
    const float msl = m * sl2;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      floatx8 pv;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        pv[j] = __builtin_amdgcn_exp2f(fmaf(sacc[2 * cc + (j >> 2)][j & 3], sl2, -msl));
      ph[cc] = __builtin_convertvector(pv, bf16x8);
    }
    // O^T += V^T P^T : 4 dim tiles x 2 key chunks.  Lane (dim 16t + lr, group lg) takes
    // keys 32cc + 8lg + 0..7 of its V^T row: chunk 4cc + lg.
    bf16x8 vf[8];  // vf[t]: keys 0..31 of dim row 16t + lr, vf[4 + t]: keys 32..63
    lds_read_b128_2x4<2048>(vf, vs0 + vofs0, vs0 + vofs1);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) o[t] = mfma16(vf[cc * 4 + t], ph[cc], o[t]);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) osum = mfma16(ones, ph[cc], osum);
  }
  const float lsum = __shfl(osum[0], lr, 64);  // from the group-0 lane of this query
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

__global__ __launch_bounds__(256, 3) void sa_flash_kernel(
    int B, int S, int H, const bf16* __restrict__ q, int64_t ldq, const bf16* __restrict__ kk,
    int64_t ldk, const bf16* __restrict__ vt, bf16* __restrict__ out, int64_t ldo,
    float scale) {
  __shared__ __attribute__((aligned(1024))) char stg[fa::NSTG][2 * fa::TILE];
  sa_flash_block(blockIdx.x, blockIdx.y, blockIdx.z, S, H, q, ldq, kk, ldk, vt, out, ldo, scale,
                 stg);
}

// Flash SA with two 16-query sets per wave, 128 queries per block of 4 waves: every K and
// V^T fragment a wave reads from the LDS ring feeds the MFMAs of both sets, half the LDS
// bytes and half the per-tile ring and address work per product of the one-set kernel
// above (whose ring, fragment layout and key order it keeps).  Per query the arithmetic
// is that kernel's, in the same order (same tiles, MFMAs, and rescale decisions taken per
// 16-query set over the same 16 queries), so the outputs are the same bits.  Key tiles
// below the block's first query need no mask and run in the first loop; the (at most
// two) diagonal tiles run in a second loop with the causal mask.  Set 0 also runs the
// block's last tile when it lies past all of its queries: every score is masked there,
// nothing exceeds the reference maximum, and P = 0 adds nothing.
namespace fa2 {
constexpr int QS = 2, BQ = 64 * QS;
}

// Work item (xcd, j) of the two-set flash grid: the (batch, head) pairs p with p % 8 == xcd,
// one pair's query blocks after the other (heavy, late ones first); items past the grid
// return.  stg: the block's ring (3 x 16 KiB, 1 KiB aligned).
DEV void sa_flash2_block(int xcd, int j, int B, int S, int H, const bf16* __restrict__ q,
                         int64_t ldq, const bf16* __restrict__ kk, int64_t ldk,
                         const bf16* __restrict__ vt, bf16* __restrict__ out, int64_t ldo,
                         float scale, char (*stg)[2 * fa::TILE]) {
  using namespace fa;
  constexpr int QS = fa2::QS, BQ2 = fa2::BQ;
  const int nqb = (S + BQ2 - 1) / BQ2;
  const int npairs = B * H, ppx = (npairs + 7) / 8;
  const int pair = xcd + 8 * (j / nqb);
  if (j >= ppx * nqb || pair >= npairs) return;
  const int qb = nqb - 1 - j % nqb;
  const int head = pair % H, b = pair / H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t tok0 = (int64_t)b * S;
  const int hoff = head * 64;
  const int q0 = qb * BQ2;

  // set s of wave w: queries q0 + 64 s + 16 w + lr; Q^T fragments as in the one-set kernel
  int qpos[QS], qlim[QS];
  bf16x8 qf[QS][2];
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    qpos[s] = q0 + 64 * s + 16 * w + lr;
    qlim[s] = min(qpos[s], S - 1);
    const bf16* qr = q + (tok0 + qlim[s]) * ldq + hoff + lg * 8;
    qf[s][0] = *reinterpret_cast<const bf16x8*>(qr);
    qf[s][1] = *reinterpret_cast<const bf16x8*>(qr + 32);
  }

  // ring loads of one 64-key stage, as in the one-set kernel
  const int lrow = lane >> 3, slot = lane & 7;
  const bf16* vbase = vt + ((int64_t)(b * H + head) * 64) * S;
  auto tile_src = [&](int i, int kbase) -> const bf16* {
    const int j = w + 4 * i;
    if (i < 2) {
      const int row = j * 8 + lrow;
      const int kp = min(kbase + key_of_row(row), S - 1);
      return kk + (tok0 + kp) * ldk + hoff + (slot ^ (row & 7)) * 8;
    }
    const int dim = (j - 8) * 8 + lrow;
    const int p0 = min(kbase + (slot ^ (dim & 7)) * 8, S - 8);
    return vbase + (int64_t)dim * S + p0;
  };
  const char* kb_u = reinterpret_cast<const char*>(kk + tok0 * ldk + hoff);
  const char* vb_u = reinterpret_cast<const char*>(vbase);
  uint32_t loff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = w + 4 * i;
    if (i < 2) {
      const int row = j * 8 + lrow;
      loff[i] = (uint32_t)((key_of_row(row) * ldk + (slot ^ (row & 7)) * 8) * 2);
    } else {
      const int dim = (j - 8) * 8 + lrow;
      loff[i] = (uint32_t)(((int64_t)dim * S + (slot ^ (dim & 7)) * 8) * 2);
    }
  }
  auto issue = [&](int t) {
    char* sb = stg[t % NSTG];
    const int kbase = t * BKEY;
    const char* kt_u = kb_u + (int64_t)kbase * ldk * 2;
    const char* vt_u = vb_u + (int64_t)kbase * 2;
    if (kbase + BKEY <= S) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds((const void*)((i < 2 ? kt_u : vt_u) + loff[i]),
                                         (lds_void*)(sb + (w + 4 * i) * 1024), 16, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds((const void*)tile_src(i, kbase),
                                         (lds_void*)(sb + (w + 4 * i) * 1024), 16, 0, 0);
    }
  };

  const float sl2 = scale * 1.44269504088896341f;  // scale * log2(e)
  const float lazy_thr = SA_LAZY / sl2;             // in score units
  float m[QS];
  floatx4 o[QS][4], osum[QS];
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    m[s] = -INFINITY;
    osum[s] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) o[s][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 ones;  // row 0 all ones: the P.V MFMAs' extra product is the softmax denominator
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = (bf16)(lr == 0 ? 1.f : 0.f);

  const int nkt = (min(q0 + BQ2, S) - 1) / BKEY + 1;
  const int nfull = min(q0 / BKEY, nkt);  // tiles whose keys all precede query q0
  const uint32_t stg0 = lds_off(stg[0]);
  const uint32_t kofs0 = 2 * swz128(lr, lg), kofs1 = 2 * swz128(lr, 4 + lg);
  issue(0);
  if (nkt > 1) issue(1);
  asm volatile("" : "+v"(qf[0][0]), "+v"(qf[0][1]), "+v"(qf[1][0]), "+v"(qf[1][1]));

  auto tile = [&](int kt, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if (kt + 1 < nkt) wait_vmcnt<4>();
    else wait_vmcnt<0>();
    ring_barrier();  // tile kt visible to all waves; tile kt-1 consumed by all
    if (kt + 2 < nkt) issue(kt + 2);
    const uint32_t ks0 = stg0 + (kt % NSTG) * 2 * TILE, vs0 = ks0 + TILE;
    const int kbase = kt * BKEY;
    // kf[t] / kf[4 + t]: K rows 16t + lr, dims 0..31 / 32..63; vf[4cc + t]: V^T row
    // (dim) 16t + lr, keys 32cc + 8lg + 0..7.  K first, V^T after the score MFMAs are
    // issued (fewer live registers: three waves per SIMD).
    bf16x8 kf[8], vf[8];
    lds_read_b128_2x4<2048>(kf, ks0 + kofs0, ks0 + kofs1);
    floatx4 sacc[QS][4];
#pragma unroll
    for (int s = 0; s < QS; ++s)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        sacc[s][t] = mfma16(kf[t], qf[s][0], floatx4{0.f, 0.f, 0.f, 0.f});
        sacc[s][t] = mfma16(kf[4 + t], qf[s][1], sacc[s][t]);
      }
    lds_read_b128_2x4<2048>(vf, vs0 + kofs0, vs0 + kofs1);
    if constexpr (MASK) {
#pragma unroll
      for (int s = 0; s < QS; ++s)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kbase + (t >> 1) * 32 + lg * 8 + (t & 1) * 4 + i > qlim[s])
              sacc[s][t][i] = -INFINITY;
    }
    // lazy rescaling per 16-query set, decided as in the one-set kernel
    float lmax[QS];
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      lmax[s] = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) lmax[s] = fmaxf(lmax[s], sacc[s][t][i]);
    }
    bool need = false;
#pragma unroll
    for (int s = 0; s < QS; ++s) need = need || lmax[s] > m[s] + lazy_thr;
    if (__any(need)) {  // rare: one branch for both sets keeps the common path straight
#pragma unroll
      for (int s = 0; s < QS; ++s) {
        if (__any(lmax[s] > m[s] + lazy_thr)) {
          const float mn = fmaxf(m[s], max_xor32(max_xor16(lmax[s])));
          const float corr = __builtin_amdgcn_exp2f((m[s] - mn) * sl2);
          m[s] = mn;
          osum[s] *= corr;
#pragma unroll
          for (int t = 0; t < 4; ++t) o[s][t] *= corr;
        }
      }
    }
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      bf16x8 ph[2];
      const float msl = m[s] * sl2;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        floatx8 pv;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          pv[j] = __builtin_amdgcn_exp2f(fmaf(sacc[s][2 * cc + (j >> 2)][j & 3], sl2, -msl));
        ph[cc] = __builtin_convertvector(pv, bf16x8);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) o[s][t] = mfma16(vf[cc * 4 + t], ph[cc], o[s][t]);
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) osum[s] = mfma16(ones, ph[cc], osum[s]);
    }
  };
  int kt = 0;
  for (; kt < nfull; ++kt) tile(kt, std::false_type{});
  for (; kt < nkt; ++kt) tile(kt, std::true_type{});

#pragma unroll
  for (int s = 0; s < QS; ++s) {
    const float lsum = __shfl(osum[s][0], lr, 64);  // from the group-0 lane of this query
    if (qpos[s] >= S) continue;
    const float inv = 1.0f / lsum;
    bf16* orow = out + (tok0 + qpos[s]) * ldo + hoff;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (bf16)(o[s][t][i] * inv);
      *reinterpret_cast<bf16x4*>(orow + t * 16 + lg * 4) = v;
    }
  }
}

// Blocks reach the 8 XCDs round-robin: block b is item (b % 8, b / 8), so a pair's K and
// V^T are read into one XCD's L2 only.
__global__ __launch_bounds__(256, 3) void sa_flash2_kernel(
    int B, int S, int H, const bf16* __restrict__ q, int64_t ldq, const bf16* __restrict__ kk,
    int64_t ldk, const bf16* __restrict__ vt, bf16* __restrict__ out, int64_t ldo,
    float scale) {
  __shared__ __attribute__((aligned(1024))) char stg[fa::NSTG][2 * fa::TILE];
  sa_flash2_block((int)blockIdx.x & 7, (int)blockIdx.x >> 3, B, S, H, q, ldq, kk, ldk, vt, out,
                  ldo, scale, stg);
}

// SA (flash, prepared inputs) and DA (bf16, head dim 64, inputs already rotated) of one
// depth in one launch: blocks [0, nsa) are the flash blocks in the flash grid's order,
// the rest the depth-attention blocks.  The two write disjoint outputs and read only the
// projections, so the DA blocks fill the CUs that the causal flash grid leaves idle in
// its tail (its last query blocks are the longest).
struct SaFlashArgs {
  int S, H;
  const bf16* q;
  int64_t ldq;
  const bf16* kk;
  int64_t ldk;
  const bf16* vt;
  bf16* out;
  int64_t ldo;
  float scale;
};
struct DaArgs {
  int64_t rows;
  int H, l, L;
  const bf16 *q, *kn, *vn;
  int64_t ldq, ldk, ldv;
  bf16 *kc, *vc, *out;
  int64_t ldo;
  float scale;
  int window, dilation;
  int64_t srow, sslot;  // cache strides (see depth_attn_block)
};

__global__ __launch_bounds__(256, 3) void attn_pair_kernel(SaFlashArgs sa, DaArgs da, int nsa) {
  __shared__ __attribute__((aligned(1024))) char stg[fa::NSTG][2 * fa::TILE];
  const int bi = blockIdx.x;
  if (bi < nsa) {
    const int nqb = (sa.S + fa::BQ - 1) / fa::BQ;
    sa_flash_block(bi % nqb, (bi / nqb) % sa.H, bi / (nqb * sa.H), sa.S, sa.H, sa.q, sa.ldq,
                   sa.kk, sa.ldk, sa.vt, sa.out, sa.ldo, sa.scale, stg);
  } else {
    depth_attn_block<bf16, 8, false>(bi - nsa, da.rows, da.H, 64, da.l, da.L, da.q, da.ldq, da.kn,
                                     da.ldk, da.vn, da.ldv, da.kc, da.vc, da.out, da.ldo, nullptr,
                                     nullptr, da.scale, da.window, da.dilation, da.srow, da.sslot);
  }
}

// SA (the two-set flash grid) and DA of one depth in one launch, the two kinds of block
// interleaved over the first m blocks: block i < m is flash block k = floor(i nsa / m)
// when floor((i + 1) nsa / m) > k, else DA block i - k; the blocks from m on are DA's.
// The dispatcher hands each freed slot to the next block, so every CU keeps running both
// kinds (matrix-core and VALU work beside HBM streaming); in separate launches on two
// streams SA's blocks hold all registers of the CUs they occupy and the two split the
// CUs.  The launcher takes m = nsa + 3/5 of the DA blocks: the flash blocks, much longer
// than DA's, then all start early, so that the launch ends on DA blocks (measured with
// b = 2, s = 4096, 32 heads of 64, over 64 depths: 507 us per launch, against 536 with the
// flash blocks spread over the whole grid and 563 with all of them first).  Flash block k
// is item (k % 8, k / 8); spacings m / nsa that are not integers spread a (batch, head)
// pair's blocks over the XCDs, which was faster there than keeping them on one.  The DA blocks batch their slots as DA's own
// launch does (the same bits).
template <bool NT>
__global__ __launch_bounds__(256, 3) void attn_pair2_kernel(SaFlashArgs sa, DaArgs da, int B,
                                                            int64_t nsa, int64_t m) {
  __shared__ __attribute__((aligned(1024))) char stg[fa::NSTG][2 * fa::TILE];
  const int64_t i = blockIdx.x;
  const int64_t k = i < m ? i * nsa / m : nsa;
  if (i < m && (i + 1) * nsa / m > k) {
    sa_flash2_block((int)(k & 7), (int)(k >> 3), B, sa.S, sa.H, sa.q, sa.ldq, sa.kk, sa.ldk,
                    sa.vt, sa.out, sa.ldo, sa.scale, stg);
  } else {
    depth_attn_block<bf16, 8, false, NT>(i - k, da.rows, da.H, 64, da.l, da.L, da.q, da.ldq,
                                            da.kn, da.ldk, da.vn, da.ldv, da.kc, da.vc, da.out,
                                            da.ldo, nullptr, nullptr, da.scale, da.window,
                                            da.dilation, da.srow, da.sslot);
  }
}

// v [B, S, H, 64] (row stride ldv) -> vt [B][H][64][S] through LDS: one block per (64
// positions, head, batch); 16-byte loads of whole rows and 16-byte stores of position runs.
__global__ __launch_bounds__(256) void v_transpose_kernel(int S, int H, const bf16* __restrict__ v,
                                                          int64_t ldv, bf16* __restrict__ vt) {
  __shared__ bf16 tile[64][64 + 8];  // [position][dim]
  const int p0 = blockIdx.x * 64, head = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 2; ++u) {  // 64 rows x 8 chunks
    const int it = tid + 256 * u, r = it >> 3, ch = it & 7;
    const int p = min(p0 + r, S - 1);
    const bf16x8 x =
        *reinterpret_cast<const bf16x8*>(v + ((int64_t)b * S + p) * ldv + head * 64 + ch * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[r][ch * 8 + e] = x[e];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {  // 64 dims x 8 runs of 8 positions
    const int it = tid + 256 * u, dim = it >> 3, ch = it & 7;
    if (p0 + ch * 8 >= S) continue;  // S % 8 == 0: runs are whole or absent
    bf16x8 y;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = tile[ch * 8 + e][dim];
    *reinterpret_cast<bf16x8*>(vt + (((int64_t)b * H + head) * 64 + dim) * S + p0 + ch * 8) = y;
  }
}

// Prepares flash inputs from unrotated projections: qr/kr [B, S, H, 64] rotated (when
// rope) and rounded, vt [B][H][64][S].  Thread -> (row, head, chunk pair c < 4).
__global__ __launch_bounds__(256) void sa_prep_kernel(int B, int S, int H, const bf16* __restrict__ q,
                                                      int64_t ldq, const bf16* __restrict__ k,
                                                      int64_t ldk, const bf16* __restrict__ v,
                                                      int64_t ldv, bf16* __restrict__ qr,
                                                      bf16* __restrict__ kr, bf16* __restrict__ vt,
                                                      const float* __restrict__ cs,
                                                      const float* __restrict__ sn, int rope) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t unit = gid >> 2;  // (row, head)
  if (unit >= (int64_t)B * S * H) return;
  const int c = (int)(gid & 3);
  const int64_t row = unit / H;
  const int head = (int)(unit % H);
  const int pos = (int)(row % S);
  const int64_t h = (int64_t)H * 64;
  const bf16* srcs[2] = {q + row * ldq, k + row * ldk};
  bf16* dsts[2] = {qr + row * h, kr + row * h};
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float lo[8], hi[8];
    load16(srcs[s] + head * 64 + c * 8, lo);
    load16(srcs[s] + head * 64 + 32 + c * 8, hi);
    if (rope) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int pair = c * 8 + e;
        const float cv = cs[pos * 32 + pair], sv = sn[pos * 32 + pair];
        const float x = lo[e], y = hi[e];
        lo[e] = rot_first(x, y, cv, sv);
        hi[e] = rot_second(y, x, cv, sv);
      }
    }
    store16(dsts[s] + head * 64 + c * 8, lo);
    store16(dsts[s] + head * 64 + 32 + c * 8, hi);
  }
  // v^T: this thread writes dims c*16..c*16+15 of (row, head)
  const int64_t bb = row / S;
  const bf16* vr = v + row * ldv + head * 64 + c * 16;
  bf16* vo = vt + ((bb * H + head) * 64 + c * 16) * S + pos;
#pragma unroll
  for (int e = 0; e < 16; ++e) vo[(int64_t)e * S] = vr[e];
}

// ------------------------------------------------------------------------------ launch
static int lph_of(int dtype, int d) { return d / (dtype == DT_BF16 ? 8 : 4); }

constexpr int SA_SPLIT_SPAN = 256;

static bool flash_ok(int dtype, int d, int q_len) {
  return dtype == DT_BF16 && d == 64 && q_len % 8 == 0;
}

size_t seq_attn_ws(int dtype, int B, int q_len, int H, int d, int64_t pos0, int prepared) {
  const size_t es = dtype == DT_BF16 ? 2 : 4;
  const size_t h = (size_t)H * d;
  if (pos0 > 0) {  // decode: split partials
    const int nsplit = (int)((pos0 + 1 + SA_SPLIT_SPAN - 1) / SA_SPLIT_SPAN);
    const size_t rows = (size_t)B * q_len;
    return rows * nsplit * h * 4 + rows * nsplit * H * 2 * 4 + 512;
  }
  if (flash_ok(dtype, d, q_len)) return prepared ? 0 : 3 * (size_t)B * q_len * h * es + 1024;
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
  dlaunch(sa_rope_store_kernel<T, LP>, grid, 256, 0, st, B, n, H, d, pos0, (const T*)kn, \
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
  constexpr int SRT = 64;  // threads per block
  if (64 % lph) return -1;  // a head's chunks in one wave
  dim3 grid(nsplit, (unsigned)((int64_t)B * n), (unsigned)((threads + SRT - 1) / SRT));
#define SR_CASE(LP)                                                                    \
  dlaunch(sa_rows_kernel<T, LP>, grid, SRT, 0, st, B, n, H, d, pos0, (const T*)q, ldq,      \
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
    dlaunch(sa_combine_kernel<T>, (unsigned)((tot + 255) / 256), 256, 0, st,
        (int64_t)B * n, H, d, nsplit, pa, pm, (T*)out, ldo);
  }
  return 0;
}

int launch_seq_attn(int dtype, int B, int q_len, int H, int d, int64_t pos0, const void* q,
                    int64_t ldq, const void* kn, int64_t ldk, const void* vn, int64_t ldv,
                    const void* vt, void* kc, void* vc, int64_t cap, void* out, int64_t ldo,
                    const float* cos_s, const float* sin_s, float scale, int rope, void* ws,
                    size_t ws_bytes, hipStream_t st) {
  const int lph = lph_of(dtype, d);
  const size_t es = dtype == DT_BF16 ? 2 : 4;
  const int64_t h = (int64_t)H * d;
  if (B <= 0 || q_len <= 0) return 0;
  const bool prepared = !rope && vt;
  if (ws_bytes < seq_attn_ws(dtype, B, q_len, H, d, pos0, prepared)) return -2;
  const bool bf = dtype == DT_BF16;
  if (pos0 > 0) {
    // decode: append the (rotated) new key/value at pos0, then split-K over 0..pos0
    int rc = bf ? sa_rope_store<bf16>(lph, B, q_len, H, d, pos0, kn, ldk, vn, ldv, kc, vc,
                                      cap, cos_s, sin_s, rope, st)
                : sa_rope_store<float>(lph, B, q_len, H, d, pos0, kn, ldk, vn, ldv, kc, vc,
                                       cap, cos_s, sin_s, rope, st);
    if (rc) return rc;
    const int nsplit = (int)((pos0 + 1 + SA_SPLIT_SPAN - 1) / SA_SPLIT_SPAN);
    float* pa = (float*)ws;
    float* pm = pa + (size_t)B * q_len * nsplit * h;
    return bf ? sa_rows<bf16>(lph, B, q_len, H, d, pos0, q, ldq, kc, vc, cap, out, ldo,
                              cos_s, sin_s, rope, scale, nsplit, SA_SPLIT_SPAN, pa, pm, st)
              : sa_rows<float>(lph, B, q_len, H, d, pos0, q, ldq, kc, vc, cap, out, ldo,
                               cos_s, sin_s, rope, scale, nsplit, SA_SPLIT_SPAN, pa, pm, st);
  }
  // prefill
  if (kc) {
    int rc = bf ? sa_rope_store<bf16>(lph, B, q_len, H, d, 0, kn, ldk, vn, ldv, kc, vc, cap,
                                      cos_s, sin_s, rope, st)
                : sa_rope_store<float>(lph, B, q_len, H, d, 0, kn, ldk, vn, ldv, kc, vc, cap,
                                       cos_s, sin_s, rope, st);
    if (rc) return rc;
  }
  if (flash_ok(dtype, d, q_len)) {
    const bf16 *fq = (const bf16*)q, *fk = (const bf16*)kn, *fvt = (const bf16*)vt;
    int64_t fldq = ldq, fldk = ldk;
    if (!prepared && !rope) {  // rotated (or unrotated by choice) q / k: only v^T needed
      bf16* vtt = (bf16*)ws + 2 * (size_t)B * q_len * h;
      dlaunch(v_transpose_kernel, dim3((q_len + 63) / 64, H, B), 256, 0, st, q_len, H,
              (const bf16*)vn, ldv, vtt);
      fvt = vtt;
    } else if (!prepared) {
      bf16* qr = (bf16*)ws;
      bf16* kr = qr + (size_t)B * q_len * h;
      bf16* vtt = kr + (size_t)B * q_len * h;
      const int64_t units = (int64_t)B * q_len * H * 4;
      dlaunch(sa_prep_kernel, (unsigned)((units + 255) / 256), 256, 0, st,
          B, q_len, H, (const bf16*)q, ldq, (const bf16*)kn, ldk, (const bf16*)vn, ldv, qr,
          kr, vtt, cos_s, sin_s, rope);
      fq = qr;
      fk = kr;
      fvt = vtt;
      fldq = fldk = h;
    }
    if (q_len > fa::BQ) {  // two query sets per wave once a block has more than 64 rows
      const int64_t nqb = (q_len + fa2::BQ - 1) / fa2::BQ;
      const int64_t ppx = ((int64_t)B * H + 7) / 8;  // (batch, head) pairs per XCD
      if (8 * ppx * nqb > 0x7fffffff) return -1;
      dlaunch(sa_flash2_kernel, (unsigned)(8 * ppx * nqb), 256, 0, st, B, q_len, H, fq, fldq,
              fk, fldk, fvt, (bf16*)out, ldo, scale);
      return 0;
    }
    dim3 grid((q_len + fa::BQ - 1) / fa::BQ, H, B);
    dlaunch(sa_flash_kernel, grid, 256, 0, st, B, q_len, H, fq, fldq, fk, fldk, fvt, (bf16*)out,
                                          ldo, scale);
    return 0;
  }
  // generic: (rotated) keys into ws, then one row-streaming pass
  char* kb = (char*)ws;
  char* vb = kb + (size_t)B * q_len * h * es;
  int rc = bf ? sa_rope_store<bf16>(lph, B, q_len, H, d, 0, kn, ldk, vn, ldv, kb, vb, q_len,
                                    cos_s, sin_s, rope, st)
              : sa_rope_store<float>(lph, B, q_len, H, d, 0, kn, ldk, vn, ldv, kb, vb, q_len,
                                     cos_s, sin_s, rope, st);
  if (rc) return rc;
  return bf ? sa_rows<bf16>(lph, B, q_len, H, d, 0, q, ldq, kb, vb, q_len, out, ldo, cos_s,
                            sin_s, rope, scale, 1, q_len, nullptr, nullptr, st)
            : sa_rows<float>(lph, B, q_len, H, d, 0, q, ldq, kb, vb, q_len, out, ldo, cos_s,
                             sin_s, rope, scale, 1, q_len, nullptr, nullptr, st);
}

bool attn_pair_ok(int dtype, int B, int q_len, int H, int d, int64_t pos0, const void* vt) {
  return dtype == DT_BF16 && d == 64 && pos0 == 0 && vt && B > 0 && flash_ok(dtype, d, q_len);
}

int launch_attn_pair(int B, int S, int H, int l, int L, const void* q, const void* k,
                     const void* vt, const void* dq, const void* dk, const void* dv,
                     int64_t ldqkv, int64_t ldkv, int64_t srow, int64_t sslot, void* dkc, void* dvc, void* out_sa, void* out_da,
                     int64_t ldo, float scale, int window, int dilation, hipStream_t st) {
  if (!attn_pair_ok(DT_BF16, B, S, H, 64, 0, vt)) return -1;
  const int nqb = (S + fa::BQ - 1) / fa::BQ;
  const int64_t nsa = (int64_t)nqb * H * B;
  const int64_t rows = (int64_t)B * S;
  const int64_t nda = (rows * H * 8 + 255) / 256;  // 8 lanes per head of 64
  if (nsa + nda > 0x7fffffff) return -1;
  SaFlashArgs sa{S, H, (const bf16*)q, ldqkv, (const bf16*)k, ldqkv, (const bf16*)vt,
                 (bf16*)out_sa, ldo, scale};
  DaArgs da{rows, H, l, L, (const bf16*)dq, (const bf16*)dk, (const bf16*)dv, ldqkv, ldkv,
            ldkv, (bf16*)dkc, (bf16*)dvc, (bf16*)out_da, ldo, scale, window, dilation,
            srow, sslot};
  dlaunch(attn_pair_kernel, (unsigned)(nsa + nda), 256, 0, st, sa, da, (int)nsa);
  return 0;
}

int launch_attn_pair2(int B, int S, int H, int l, int L, const void* q, const void* k,
                      const void* vt, const void* dq, const void* dk, const void* dv,
                      int64_t ldqkv, int64_t ldkv, int64_t srow, int64_t sslot, void* dkc, void* dvc, void* out_sa, void* out_da,
                      int64_t ldo, float scale, int window, int dilation, hipStream_t st) {
  if (!attn_pair_ok(DT_BF16, B, S, H, 64, 0, vt) || S <= fa::BQ) return -1;
  const int64_t nqb = (S + fa2::BQ - 1) / fa2::BQ;
  const int64_t nsa = 8 * (((int64_t)B * H + 7) / 8) * nqb;  // the two-set flash grid
  const int64_t rows = (int64_t)B * S;
  const int64_t nda = (rows * H * 8 + 255) / 256;  // 8 lanes per head of 64
  if (nsa + nda > 0x7fffffff) return -1;
  SaFlashArgs sa{S, H, (const bf16*)q, ldqkv, (const bf16*)k, ldqkv, (const bf16*)vt,
                 (bf16*)out_sa, ldo, scale};
  DaArgs da{rows, H, l, L, (const bf16*)dq, (const bf16*)dk, (const bf16*)dv, ldqkv, ldkv,
            ldkv, (bf16*)dkc, (bf16*)dvc, (bf16*)out_da, ldo, scale, window, dilation,
            srow, sslot};
  // nontemporal cache reads once the K and V caches exceed 256 MiB (as depth_attn)
  const bool nt = 2 * rows * (int64_t)L * H * 64 * 2 > ((int64_t)256 << 20);
  const int64_t m = nsa + nda * 3 / 5;  // the flash blocks lie among the first m
  if (nt)
    dlaunch(attn_pair2_kernel<true>, (unsigned)(nsa + nda), 256, 0, st, sa, da, B, nsa, m);
  else
    dlaunch(attn_pair2_kernel<false>, (unsigned)(nsa + nda), 256, 0, st, sa, da, B, nsa, m);
  return 0;
}

}  // namespace dreamer
