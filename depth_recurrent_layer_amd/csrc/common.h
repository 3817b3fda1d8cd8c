// Shared device helpers for the gfx950 kernels of libdreamer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define DEV __device__ __forceinline__

DEV float to_f(float x) { return x; }
DEV float to_f(bf16 x) { return (float)x; }

template <typename T>
DEV T from_f(float x);
template <>
DEV float from_f<float>(float x) { return x; }
// float -> bf16 conversion: gfx950 v_cvt_pk_bf16_f32, round to nearest even.
template <>
DEV bf16 from_f<bf16>(float x) { return (bf16)x; }

// Round a float to storage precision T and back (the value a reload would see).
template <typename T>
DEV float round_to(float x) { return to_f(from_f<T>(x)); }

// 16-byte vector of storage elements: 8 bf16 or 4 f32.
template <typename T>
struct Vec16;
template <>
struct Vec16<bf16> {
  static constexpr int N = 8;
  bf16x8 v;
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  floatx4 v;
};

template <typename T>
DEV void load16(const T* p, float* out) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
  } else {
    floatx4 v = *reinterpret_cast<const floatx4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = v[i];
  }
}

template <typename T>
DEV void store16(T* p, const float* in) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (bf16)in[i];
    *reinterpret_cast<bf16x8*>(p) = v;
  } else {
    floatx4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = in[i];
    *reinterpret_cast<floatx4*>(p) = v;
  }
}

DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over aligned groups of G lanes (G a power of two <= 64).
template <int G>
DEV float group_sum(float v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Block-wide sum (blockDim.x a multiple of 64, <= 1024); `red` holds >= 16 floats.
DEV float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

DEV float fast_exp(float x) { return __expf(x); }

DEV float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

DEV float silu_(float x) { return x / (1.0f + expf(-x)); }

DEV float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

// MFMA 16x16x32 bf16 -> f32 (gfx950).  Lane l holds A[row l%16][k 8(l/16)..+8],
// B[k 8(l/16)..+8][col l%16]; D lane l holds rows 4(l/16)+i, col l%16, i = 0..3.
DEV floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
