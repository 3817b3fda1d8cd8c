// Expert FFNs on routed slots, the combine / residual / RMSNorm epilogue of a depth step,
// and the shared-expert absorption helper.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dreamer {

// ------------------------------------------------------------- fused expert FFN (bf16)
// One block = one 64-row tile of one expert's routed slots (tiles listed by toff).
// GEMM1 (x W1^T, x W3^T) accumulates in registers; wave w owns hidden columns
// [w F/4, (w+1) F/4) of both the gate and the up projection, so the activation is
// lane-local.  The hidden tile goes to LDS (bf16) and GEMM2 (H W2^T) streams W2 in
// 256-column chunks.  Outputs are gate-scaled and written per slot.
template <int F, int KIND>
__global__ __launch_bounds__(256) void expert_ffn_kernel(
    int k, int h_in, int h_out, int E, const bf16* __restrict__ x,
    const float* __restrict__ gate, const bf16* __restrict__ w1,
    const bf16* __restrict__ w3, const bf16* __restrict__ w2, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ goff, const int32_t* __restrict__ toff,
    bf16* __restrict__ slots) {
  constexpr int BM = FFN_TILE_M, LDH = F + 8;
  constexpr int NT1 = F / 64;  // 16-col tiles per wave per projection
  constexpr int KS2 = F / 32;  // k-steps of GEMM2
  __shared__ int s_slot[BM];
  __shared__ float s_gate[BM];
  __shared__ __attribute__((aligned(16))) bf16 Hs[BM * LDH];

  const int tile = blockIdx.x;
  if (tile >= toff[E]) return;
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (toff[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int r0 = goff[e] + (tile - toff[e]) * BM, r1 = goff[e + 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  if (tid < BM) {
    const int m = r0 + tid;
    const int s = m < r1 ? perm[m] : -1;
    s_slot[tid] = s;
    s_gate[tid] = s >= 0 ? gate[s] : 0.f;
  }
  __syncthreads();

  // A row pointers (token rows) for the 4 m-tiles this lane feeds
  const bf16* arow[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int s = s_slot[mt * 16 + lr];
    arow[mt] = s >= 0 ? x + (int64_t)(s / k) * h_in + lg * 8 : nullptr;
  }
  const bf16* W1 = w1 + (int64_t)e * F * h_in;
  const bf16* W3 = KIND == FFN_SWIGLU ? w3 + (int64_t)e * F * h_in : nullptr;
  const bf16* brow1[NT1];
  const bf16* brow3[NT1];
#pragma unroll
  for (int nt = 0; nt < NT1; ++nt) {
    const int col = w * (F / 4) + nt * 16 + lr;
    brow1[nt] = W1 + (int64_t)col * h_in + lg * 8;
    brow3[nt] = KIND == FFN_SWIGLU ? W3 + (int64_t)col * h_in + lg * 8 : nullptr;
  }
  floatx4 ag[4][NT1], au[4][NT1];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT1; ++nt) {
      ag[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
      au[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  const bf16x8 zero8 = {};
  for (int k0 = 0; k0 < h_in; k0 += 64) {
    bf16x8 af[2][4], b1[2][NT1], b3[2][NT1];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        af[ks][mt] = arow[mt] ? *reinterpret_cast<const bf16x8*>(arow[mt] + k0 + ks * 32)
                              : zero8;
#pragma unroll
      for (int nt = 0; nt < NT1; ++nt) {
        b1[ks][nt] = *reinterpret_cast<const bf16x8*>(brow1[nt] + k0 + ks * 32);
        if (KIND == FFN_SWIGLU)
          b3[ks][nt] = *reinterpret_cast<const bf16x8*>(brow3[nt] + k0 + ks * 32);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT1; ++nt) {
          ag[mt][nt] = mfma16(af[ks][mt], b1[ks][nt], ag[mt][nt]);
          if (KIND == FFN_SWIGLU) au[mt][nt] = mfma16(af[ks][mt], b3[ks][nt], au[mt][nt]);
        }
  }
  // activation -> LDS (row mt*16 + 4lg + i, col w*F/4 + nt*16 + lr)
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT1; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g = ag[mt][nt][i];
        const float hv = KIND == FFN_SWIGLU ? silu_(g) * au[mt][nt][i] : gelu_erf(g);
        Hs[(mt * 16 + lg * 4 + i) * LDH + w * (F / 4) + nt * 16 + lr] = (bf16)hv;
      }
  __syncthreads();
  bf16x8 hf[4][KS2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int ks = 0; ks < KS2; ++ks)
      hf[mt][ks] = *reinterpret_cast<const bf16x8*>(&Hs[(mt * 16 + lr) * LDH + ks * 32 + lg * 8]);

  const bf16* W2 = w2 + (int64_t)e * h_out * F;
  for (int nc = 0; nc < h_out; nc += 256) {
    const int cbase = nc + w * 64;
    if (cbase >= h_out) break;
    floatx4 acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const bf16* brow = W2 + (int64_t)(cbase + nt * 16 + lr) * F + lg * 8;
      bf16x8 bf_[KS2];
#pragma unroll
      for (int ks = 0; ks < KS2; ++ks)
        bf_[ks] = *reinterpret_cast<const bf16x8*>(brow + ks * 32);
#pragma unroll
      for (int ks = 0; ks < KS2; ++ks)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = mfma16(hf[mt][ks], bf_[ks], acc[mt][nt]);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = mt * 16 + lg * 4 + i;
        const int s = s_slot[row];
        if (s < 0) continue;
        const float gs = s_gate[row];
        bf16* out = slots + (int64_t)s * h_out + cbase + lr;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) out[nt * 16] = (bf16)(acc[mt][nt][i] * gs);
      }
  }
}

// ------------------------------------------------ per-slot expert FFN (float32, any f)
// One block per slot s = t*k + i: hidden in LDS, then the output row.
__global__ void expert_ffn_f32_kernel(int64_t nslots, int k, int kind, int h_in, int f,
                                      int h_out, const float* __restrict__ x,
                                      const int32_t* __restrict__ idx,
                                      const float* __restrict__ gate,
                                      const float* __restrict__ w1,
                                      const float* __restrict__ w3,
                                      const float* __restrict__ w2, float* __restrict__ slots) {
  extern __shared__ float hid[];
  const int64_t s = blockIdx.x;
  if (s >= nslots) return;
  const int e = idx[s];
  const float g = gate[s];
  const float* xr = x + (s / k) * h_in;
  if (kind == FFN_LINEAR) {
    const float* W = w1 + (int64_t)e * h_out * h_in;
    for (int n = threadIdx.x; n < h_out; n += blockDim.x) {
      float a = 0.f;
      for (int j = 0; j < h_in; ++j) a = fmaf(W[(int64_t)n * h_in + j], xr[j], a);
      slots[s * h_out + n] = g * a;
    }
    return;
  }
  const float* W1 = w1 + (int64_t)e * f * h_in;
  for (int j = threadIdx.x; j < f; j += blockDim.x) {
    float a = 0.f, b = 0.f;
    for (int c = 0; c < h_in; ++c) a = fmaf(W1[(int64_t)j * h_in + c], xr[c], a);
    if (kind == FFN_SWIGLU) {
      const float* W3 = w3 + (int64_t)e * f * h_in;
      for (int c = 0; c < h_in; ++c) b = fmaf(W3[(int64_t)j * h_in + c], xr[c], b);
      hid[j] = silu_(a) * b;
    } else {
      hid[j] = gelu_erf(a);
    }
  }
  __syncthreads();
  const float* W2 = w2 + (int64_t)e * h_out * f;
  for (int n = threadIdx.x; n < h_out; n += blockDim.x) {
    float a = 0.f;
    for (int j = 0; j < f; ++j) a = fmaf(W2[(int64_t)n * f + j], hid[j], a);
    slots[s * h_out + n] = g * a;
  }
}

int launch_expert_ffn(int dtype, int kind, int64_t nslots, int k, int h_in, int f, int h_out,
                      int E, const void* x, const float* gate, const void* w1,
                      const void* w3, const void* w2, const int32_t* perm,
                      const int32_t* goff, const int32_t* toff, void* slots,
                      hipStream_t st) {
  if (nslots <= 0) return 0;
  if (dtype == DT_F32) return -1;  // the f32 path uses launch_expert_ffn_f32
  if (h_in % 64 || h_out % 64) return -1;
  const unsigned grid = (unsigned)((nslots + FFN_TILE_M - 1) / FFN_TILE_M + E);
#define EF_CASE(FF, KK)                                                                    \
  expert_ffn_kernel<FF, KK><<<grid, 256, 0, st>>>(k, h_in, h_out, E, (const bf16*)x, gate, \
                                                  (const bf16*)w1, (const bf16*)w3,        \
                                                  (const bf16*)w2, perm, goff, toff,       \
                                                  (bf16*)slots)
  if (kind == FFN_SWIGLU && f == 64) EF_CASE(64, FFN_SWIGLU);
  else if (kind == FFN_SWIGLU && f == 128) EF_CASE(128, FFN_SWIGLU);
  else if (kind == FFN_GELU && f == 64) EF_CASE(64, FFN_GELU);
  else if (kind == FFN_GELU && f == 128) EF_CASE(128, FFN_GELU);
  else return -1;
#undef EF_CASE
  return 0;
}

int launch_expert_ffn_f32(int kind, int64_t nslots, int k, int h_in, int f, int h_out,
                          const float* x, const int32_t* idx, const float* gate,
                          const float* w1, const float* w3, const float* w2, float* slots,
                          hipStream_t st) {
  if (nslots <= 0) return 0;
  const size_t lds = (size_t)(kind == FFN_LINEAR ? 1 : f) * sizeof(float);
  if (lds > 65536) return -1;
  expert_ffn_f32_kernel<<<(unsigned)nslots, 256, lds, st>>>(nslots, k, kind, h_in, f, h_out,
                                                            x, idx, gate, w1, w3, w2, slots);
  return 0;
}

// -------------------------------------------------------------- combine + next RMSNorm
// Block per token, one 16-byte chunk of the row per thread.  x = y + sum_i slots[t*k+i]
// (fixed slot order), then optional x stores and xhat = x / sqrt(mean(x^2) + eps) * g.
template <typename T>
__global__ __launch_bounds__(1024) void combine_norm_kernel(
    int64_t Ttok, int h, int k, const float* __restrict__ y, const T* __restrict__ slots,
    float* __restrict__ x_out, float* __restrict__ x_out2, const T* __restrict__ g, float eps,
    T* __restrict__ xhat, float* __restrict__ xhat32) {
  constexpr int VEC = Vec16<T>::N;
  __shared__ float red[16];
  const int64_t t = blockIdx.x;
  const int c = threadIdx.x * VEC;
  const bool act = c < h;
  float v[VEC];
  float ss = 0.f;
  if (act) {
    if (y) {
      load16(y + t * h + c, v);
      if constexpr (VEC == 8) load16(y + t * h + c + 4, v + 4);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = 0.f;
    }
    for (int i = 0; i < k; ++i) {
      float sv[VEC];
      load16(slots + (t * k + i) * h + c, sv);
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] += sv[e];
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) ss += v[e] * v[e];
    float* outs[2] = {x_out, x_out2};
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      if (!outs[o]) continue;
      store16(outs[o] + t * h + c, v);
      if constexpr (VEC == 8) store16(outs[o] + t * h + c + 4, v + 4);
    }
  }
  if (!xhat) return;
  ss = block_sum(ss, red);
  if (!act) return;
  const float inv = 1.0f / sqrtf(ss / (float)h + eps);
  float gv[VEC];
  load16(g + c, gv);
#pragma unroll
  for (int e = 0; e < VEC; ++e) v[e] = v[e] * inv * gv[e];
  store16(xhat + t * h + c, v);
  if (xhat32) {
    store16(xhat32 + t * h + c, v);
    if constexpr (VEC == 8) store16(xhat32 + t * h + c + 4, v + 4);
  }
}

void launch_combine_norm(int dtype, int64_t T, int h, int k, const float* y,
                         const void* slots, float* x_out, float* x_out2, const void* g,
                         float eps, void* xhat, float* xhat32, hipStream_t st) {
  if (T <= 0) return;
  const int vec = dtype == DT_BF16 ? 8 : 4;
  const int threads = ((h / vec + 63) / 64) * 64;
  if (dtype == DT_BF16)
    combine_norm_kernel<bf16><<<(unsigned)T, threads, 0, st>>>(
        T, h, k, y, (const bf16*)slots, x_out, x_out2, (const bf16*)g, eps, (bf16*)xhat,
        xhat32);
  else
    combine_norm_kernel<float><<<(unsigned)T, threads, 0, st>>>(
        T, h, k, y, (const float*)slots, x_out, x_out2, (const float*)g, eps, (float*)xhat,
        xhat32);
}

void launch_rmsnorm(int dtype, int64_t T, int h, const float* x, const void* g, float eps,
                    void* xhat, float* xhat32, hipStream_t st) {
  launch_combine_norm(dtype, T, h, 0, x, nullptr, nullptr, nullptr, g, eps, xhat, xhat32, st);
}

// ------------------------------------------------------------------------------ absorb
template <typename T>
__global__ void absorb_kernel(int64_t ne, int64_t n, const T* __restrict__ we,
                              const T* __restrict__ wsh, T* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= ne * n) return;
  out[i] = from_f<T>(to_f(we[i]) + to_f(wsh[i % n]));
}

void launch_absorb(int dtype, int64_t ne, int64_t n, const void* we, const void* wsh,
                   void* out, hipStream_t st) {
  const int64_t tot = ne * n;
  if (tot <= 0) return;
  const unsigned grid = (unsigned)((tot + 255) / 256);
  if (dtype == DT_BF16)
    absorb_kernel<bf16><<<grid, 256, 0, st>>>(ne, n, (const bf16*)we, (const bf16*)wsh,
                                               (bf16*)out);
  else
    absorb_kernel<float><<<grid, 256, 0, st>>>(ne, n, (const float*)we, (const float*)wsh,
                                                (float*)out);
}

}  // namespace dreamer
