// Per-slot float32 expert FFN, the combine / residual / RMSNorm epilogue of a depth step,
// and the shared-expert absorption helper.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dreamer {

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

int launch_expert_ffn_f32(int kind, int64_t nslots, int k, int h_in, int f, int h_out,
                          const float* x, const int32_t* idx, const float* gate,
                          const float* w1, const float* w3, const float* w2, float* slots,
                          hipStream_t st) {
  if (nslots <= 0) return 0;
  const size_t lds = (size_t)(kind == FFN_LINEAR ? 1 : f) * sizeof(float);
  if (lds > 65536) return -1;
  dlaunch(expert_ffn_f32_kernel, (unsigned)nslots, 256, lds, st, nslots, k, kind, h_in, f, h_out,
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
    // The slots in groups of 8, all loads of a group issued before the first sum (a loop
    // over k waits for each load in turn), the first group before the residual; past k a
    // load repeats the last slot and is not summed, so no load sits behind a branch.  The
    // sums keep the order residual, slot 0, 1, ...
    using RawV = typename std::conditional<sizeof(T) == 2, bf16x8, floatx4>::type;
    auto load_group = [&](RawV (&raw)[8], int i0) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        raw[i] = *reinterpret_cast<const RawV*>(slots + (t * k + min(i0 + i, k - 1)) * h + c);
    };
    auto add_group = [&](const RawV (&raw)[8], int i0) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i0 + i < k)
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] += (float)raw[i][e];
    };
    RawV raw[8];
    if (k > 0) load_group(raw, 0);
    if (y) {
      load16(y + t * h + c, v);
      if constexpr (VEC == 8) load16(y + t * h + c + 4, v + 4);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = 0.f;
    }
    if (k > 0) add_group(raw, 0);
    for (int i0 = 8; i0 < k; i0 += 8) {
      load_group(raw, i0);
      add_group(raw, i0);
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
    dlaunch(combine_norm_kernel<bf16>, (unsigned)T, threads, 0, st,
        T, h, k, y, (const bf16*)slots, x_out, x_out2, (const bf16*)g, eps, (bf16*)xhat,
        xhat32);
  else
    dlaunch(combine_norm_kernel<float>, (unsigned)T, threads, 0, st,
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
    dlaunch(absorb_kernel<bf16>, grid, 256, 0, st, ne, n, (const bf16*)we, (const bf16*)wsh,
                                               (bf16*)out);
  else
    dlaunch(absorb_kernel<float>, grid, 256, 0, st, ne, n, (const float*)we, (const float*)wsh,
                                                (float*)out);
}

}  // namespace dreamer
