// Shared device helpers for the gfx950 kernels of libdreamer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
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

// Reductions across lanes l ^ 16 and l ^ 32 with the gfx950 lane-swap instructions (no
// trip through LDS as a general shuffle would take): with both operands x, the swap
// returns x of the partner half-row (half-wave) in one result and this lane's own
// half-row's x in the other, in some order, so max / sum of the pair is symmetric.
DEV float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
DEV float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
DEV float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
DEV float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// Sum over aligned groups of G lanes (G a power of two <= 64), every lane ending with its
// group's sum: within 16 lanes by DPP lane permutes on the VALU (swap neighbours, swap
// pairs, mirror within 8, mirror within 16: each step adds the partner subgroup's sum),
// across 16 and 32 lanes by the lane-swap instructions.
template <int CTRL>
DEV int dpp_get(int v) {  // the value of the partner lane CTRL selects
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
DEV float dpp_get(float v) {
  return __int_as_float(dpp_get<CTRL>(__float_as_int(v)));
}
DEV float dpp_add(float v, int ctrl) {
  switch (ctrl) {  // the control word must be an immediate
    case 0xB1: return v + dpp_get<0xB1>(v);
    case 0x4E: return v + dpp_get<0x4E>(v);
    case 0x141: return v + dpp_get<0x141>(v);
    default: return v + dpp_get<0x140>(v);
  }
}
// Max over aligned groups of 16 lanes (the same DPP steps as group_sum).
DEV float group_max16(float v) {
  v = fmaxf(v, dpp_get<0xB1>(v));
  v = fmaxf(v, dpp_get<0x4E>(v));
  v = fmaxf(v, dpp_get<0x141>(v));
  return fmaxf(v, dpp_get<0x140>(v));
}
template <int G>
DEV float group_sum(float v) {
  static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "power of two up to 64");
  if constexpr (G >= 2) v = dpp_add(v, 0xB1);   // lane ^ 1
  if constexpr (G >= 4) v = dpp_add(v, 0x4E);   // lane ^ 2 (pairs of a quad)
  if constexpr (G >= 8) v = dpp_add(v, 0x141);  // lane 7 - i of its 8: the other quad
  if constexpr (G >= 16) v = dpp_add(v, 0x140); // lane 15 - i of its 16: the other 8
  if constexpr (G >= 32) v = sum_xor16(v);
  if constexpr (G >= 64) v = sum_xor32(v);
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


// Rotary pair (x, y) turned by (c, s): x' = x c - y s and y' = y c + x s, each computed
// as one fused multiply-add whose addend is the other product rounded on its own.  Every
// kernel that rotates uses these, so that the bits never depend on which product the
// compiler would otherwise fuse.
DEV float rot_first(float x, float y, float c, float s) {
#pragma clang fp contract(off)
  const float ys = y * s;
  return __builtin_fmaf(x, c, -ys);
}
DEV float rot_second(float y, float x, float c, float s) {
#pragma clang fp contract(off)
  const float xs = x * s;
  return __builtin_fmaf(y, c, xs);
}

DEV float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

DEV float silu_(float x) { return x / (1.0f + expf(-x)); }

DEV float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

// LDS pointer type of the direct global->LDS loads (global_load_lds_dwordx4: lane L of
// one instruction lands 16 bytes at LDS base + 16 L).
typedef __attribute__((address_space(3))) void lds_void;

// Wait until at most N vector-memory operations of this wave are outstanding (gfx9
// s_waitcnt encoding: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt left at max).
template <int N>
DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Runtime count: waits until at most n (clamped to [0, 63], the counter's range) are
// outstanding; a binary search over the immediate forms (six compares).
template <int LO, int HI>
DEV void wait_vmcnt_range(int n) {
  if constexpr (LO == HI) {
    wait_vmcnt<LO>();
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (n <= MID) wait_vmcnt_range<LO, MID>(n);
    else wait_vmcnt_range<MID + 1, HI>(n);
  }
}
DEV void wait_vmcnt_upto(int n) { wait_vmcnt_range<0, 63>(n < 0 ? 0 : n > 63 ? 63 : n); }

// One 8-byte global store issued as exactly one instruction (global_store_dwordx2), for
// code that counts its outstanding vector-memory operations itself: a store is one more
// operation ahead of the loads issued after it.  Nothing stored this way is read back by
// the issuing kernel.
DEV void store_b64_counted(void* p, bf16x4 v) {
  asm volatile("global_store_dwordx2 %0, %1, off" : : "v"(p), "v"(v) : "memory");
}
// The 16-byte form (global_store_dwordx4), same conventions.
DEV void store_b128_counted(void* p, bf16x8 v) {
  asm volatile("global_store_dwordx4 %0, %1, off" : : "v"(p), "v"(v) : "memory");
}

// 8-byte LDS write that the compiler does not see as an LDS access: a plain store into
// a ring that direct global->LDS loads still fill would first wait for all of them
// (vmcnt(0)).  Completed by the next lgkmcnt wait (ring_barrier has one).
DEV void lds_write_b64(uint32_t addr, bf16x4 v) {
  asm volatile("ds_write_b64 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// Workgroup barrier for LDS rings filled by direct global->LDS loads.  __syncthreads()
// would first wait for every outstanding vector-memory load of the wave (its fence
// covers global memory), draining the loads of later ring stages; here only this wave's
// LDS operations are waited for (lgkmcnt(0)), so the caller's own vmcnt wait decides
// which stages must have landed.  The empty asm statements keep the compiler from
// moving memory accesses across the barrier.
DEV void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS tiles of 64-byte rows (32 bf16 of K): chunk c (16 bytes) of row r is stored at slot
// c ^ ((r >> 1) & 3), so the 8 rows read by 8 consecutive lanes of an MFMA fragment load
// cover all 32 banks.
DEV int swz64_slot(int row, int c) { return c ^ ((row >> 1) & 3); }
DEV int swz64(int row, int c) { return row * 64 + (swz64_slot(row, c) << 4); }

// 32-bit LDS offset of a pointer into a __shared__ array.
DEV uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// N 16-byte LDS reads (1 <= N <= 24) completed within one statement.  Ring stages
// filled by direct global->LDS loads are read this way: for a plain LDS read the
// compiler cannot tell that it misses the stages still in flight and would wait for
// every outstanding load first.  The reads are complete when the statement ends, so no
// register of it is written later (the caller's vmcnt wait and barrier made the stage
// visible before).
template <int N>
DEV void lds_read_b128(bf16x8 (&x)[N], const uint32_t (&a)[N]) {
  static_assert(N >= 1 && N <= 24, "1 to 24 reads");
  if constexpr (N == 1) {
    asm volatile(
        "ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0])
        : "v"(a[0])
        : "memory");
  } else if constexpr (N == 2) {
    asm volatile(
        "ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1])
        : "v"(a[0]), "v"(a[1])
        : "memory");
  } else if constexpr (N == 3) {
    asm volatile(
        "ds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\tds_read_b128 %2, %5\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2])
        : "v"(a[0]), "v"(a[1]), "v"(a[2])
        : "memory");
  } else if constexpr (N == 4) {
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
  } else if constexpr (N == 5) {
    asm volatile(
        "ds_read_b128 %0, %5\n\tds_read_b128 %1, %6\n\tds_read_b128 %2, %7\n\t"
        "ds_read_b128 %3, %8\n\tds_read_b128 %4, %9\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4])
        : "memory");
  } else if constexpr (N == 6) {
    asm volatile(
        "ds_read_b128 %0, %6\n\tds_read_b128 %1, %7\n\tds_read_b128 %2, %8\n\t"
        "ds_read_b128 %3, %9\n\tds_read_b128 %4, %10\n\tds_read_b128 %5, %11\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5])
        : "memory");
  } else if constexpr (N == 7) {
    asm volatile(
        "ds_read_b128 %0, %7\n\tds_read_b128 %1, %8\n\tds_read_b128 %2, %9\n\t"
        "ds_read_b128 %3, %10\n\tds_read_b128 %4, %11\n\tds_read_b128 %5, %12\n\t"
        "ds_read_b128 %6, %13\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6])
        : "memory");
  } else if constexpr (N == 8) {
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\tds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\t"
        "ds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7])
        : "memory");
  } else if constexpr (N == 9) {
    asm volatile(
        "ds_read_b128 %0, %9\n\tds_read_b128 %1, %10\n\tds_read_b128 %2, %11\n\t"
        "ds_read_b128 %3, %12\n\tds_read_b128 %4, %13\n\tds_read_b128 %5, %14\n\t"
        "ds_read_b128 %6, %15\n\tds_read_b128 %7, %16\n\tds_read_b128 %8, %17\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "v"(a[8])
        : "memory");
  } else if constexpr (N == 10) {
    asm volatile(
        "ds_read_b128 %0, %10\n\tds_read_b128 %1, %11\n\tds_read_b128 %2, %12\n\t"
        "ds_read_b128 %3, %13\n\tds_read_b128 %4, %14\n\tds_read_b128 %5, %15\n\t"
        "ds_read_b128 %6, %16\n\tds_read_b128 %7, %17\n\tds_read_b128 %8, %18\n\t"
        "ds_read_b128 %9, %19\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "v"(a[8]), "v"(a[9])
        : "memory");
  } else if constexpr (N == 11) {
    asm volatile(
        "ds_read_b128 %0, %11\n\tds_read_b128 %1, %12\n\tds_read_b128 %2, %13\n\t"
        "ds_read_b128 %3, %14\n\tds_read_b128 %4, %15\n\tds_read_b128 %5, %16\n\t"
        "ds_read_b128 %6, %17\n\tds_read_b128 %7, %18\n\tds_read_b128 %8, %19\n\t"
        "ds_read_b128 %9, %20\n\tds_read_b128 %10, %21\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10])
        : "memory");
  } else if constexpr (N == 12) {
    asm volatile(
        "ds_read_b128 %0, %12\n\tds_read_b128 %1, %13\n\tds_read_b128 %2, %14\n\t"
        "ds_read_b128 %3, %15\n\tds_read_b128 %4, %16\n\tds_read_b128 %5, %17\n\t"
        "ds_read_b128 %6, %18\n\tds_read_b128 %7, %19\n\tds_read_b128 %8, %20\n\t"
        "ds_read_b128 %9, %21\n\tds_read_b128 %10, %22\n\tds_read_b128 %11, %23\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11])
        : "memory");
  } else if constexpr (N == 13) {
    asm volatile(
        "ds_read_b128 %0, %13\n\tds_read_b128 %1, %14\n\tds_read_b128 %2, %15\n\t"
        "ds_read_b128 %3, %16\n\tds_read_b128 %4, %17\n\tds_read_b128 %5, %18\n\t"
        "ds_read_b128 %6, %19\n\tds_read_b128 %7, %20\n\tds_read_b128 %8, %21\n\t"
        "ds_read_b128 %9, %22\n\tds_read_b128 %10, %23\n\tds_read_b128 %11, %24\n\t"
        "ds_read_b128 %12, %25\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]),
          "=&v"(x[12])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12])
        : "memory");
  } else if constexpr (N == 14) {
    asm volatile(
        "ds_read_b128 %0, %14\n\tds_read_b128 %1, %15\n\tds_read_b128 %2, %16\n\t"
        "ds_read_b128 %3, %17\n\tds_read_b128 %4, %18\n\tds_read_b128 %5, %19\n\t"
        "ds_read_b128 %6, %20\n\tds_read_b128 %7, %21\n\tds_read_b128 %8, %22\n\t"
        "ds_read_b128 %9, %23\n\tds_read_b128 %10, %24\n\tds_read_b128 %11, %25\n\t"
        "ds_read_b128 %12, %26\n\tds_read_b128 %13, %27\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]),
          "=&v"(x[12]), "=&v"(x[13])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13])
        : "memory");
  } else if constexpr (N == 15) {
    asm volatile(
        "ds_read_b128 %0, %15\n\tds_read_b128 %1, %16\n\tds_read_b128 %2, %17\n\t"
        "ds_read_b128 %3, %18\n\tds_read_b128 %4, %19\n\tds_read_b128 %5, %20\n\t"
        "ds_read_b128 %6, %21\n\tds_read_b128 %7, %22\n\tds_read_b128 %8, %23\n\t"
        "ds_read_b128 %9, %24\n\tds_read_b128 %10, %25\n\tds_read_b128 %11, %26\n\t"
        "ds_read_b128 %12, %27\n\tds_read_b128 %13, %28\n\tds_read_b128 %14, %29\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]),
          "=&v"(x[12]), "=&v"(x[13]), "=&v"(x[14])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]),
          "v"(a[14])
        : "memory");
  } else if constexpr (N == 16) {
    asm volatile(
        "ds_read_b128 %0, %16\n\tds_read_b128 %1, %17\n\tds_read_b128 %2, %18\n\t"
        "ds_read_b128 %3, %19\n\tds_read_b128 %4, %20\n\tds_read_b128 %5, %21\n\t"
        "ds_read_b128 %6, %22\n\tds_read_b128 %7, %23\n\tds_read_b128 %8, %24\n\t"
        "ds_read_b128 %9, %25\n\tds_read_b128 %10, %26\n\tds_read_b128 %11, %27\n\t"
        "ds_read_b128 %12, %28\n\tds_read_b128 %13, %29\n\tds_read_b128 %14, %30\n\t"
        "ds_read_b128 %15, %31\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]),
          "=&v"(x[12]), "=&v"(x[13]), "=&v"(x[14]), "=&v"(x[15])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]),
          "v"(a[14]), "v"(a[15])
        : "memory");
  } else if constexpr (N == 17) {
    asm volatile(
        "ds_read_b128 %0, %17\n\tds_read_b128 %1, %18\n\tds_read_b128 %2, %19\n\t"
        "ds_read_b128 %3, %20\n\tds_read_b128 %4, %21\n\tds_read_b128 %5, %22\n\t"
        "ds_read_b128 %6, %23\n\tds_read_b128 %7, %24\n\tds_read_b128 %8, %25\n\t"
        "ds_read_b128 %9, %26\n\tds_read_b128 %10, %27\n\tds_read_b128 %11, %28\n\t"
        "ds_read_b128 %12, %29\n\tds_read_b128 %13, %30\n\tds_read_b128 %14, %31\n\t"
        "ds_read_b128 %15, %32\n\tds_read_b128 %16, %33\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]),
          "=&v"(x[12]), "=&v"(x[13]), "=&v"(x[14]), "=&v"(x[15]), "=&v"(x[16])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]),
          "v"(a[14]), "v"(a[15]), "v"(a[16])
        : "memory");
  } else if constexpr (N == 18) {
    asm volatile(
        "ds_read_b128 %0, %18\n\tds_read_b128 %1, %19\n\tds_read_b128 %2, %20\n\t"
        "ds_read_b128 %3, %21\n\tds_read_b128 %4, %22\n\tds_read_b128 %5, %23\n\t"
        "ds_read_b128 %6, %24\n\tds_read_b128 %7, %25\n\tds_read_b128 %8, %26\n\t"
        "ds_read_b128 %9, %27\n\tds_read_b128 %10, %28\n\tds_read_b128 %11, %29\n\t"
        "ds_read_b128 %12, %30\n\tds_read_b128 %13, %31\n\tds_read_b128 %14, %32\n\t"
        "ds_read_b128 %15, %33\n\tds_read_b128 %16, %34\n\tds_read_b128 %17, %35\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]),
          "=&v"(x[12]), "=&v"(x[13]), "=&v"(x[14]), "=&v"(x[15]), "=&v"(x[16]), "=&v"(x[17])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]),
          "v"(a[14]), "v"(a[15]), "v"(a[16]), "v"(a[17])
        : "memory");
  } else if constexpr (N == 19) {
    asm volatile(
        "ds_read_b128 %0, %19\n\tds_read_b128 %1, %20\n\tds_read_b128 %2, %21\n\t"
        "ds_read_b128 %3, %22\n\tds_read_b128 %4, %23\n\tds_read_b128 %5, %24\n\t"
        "ds_read_b128 %6, %25\n\tds_read_b128 %7, %26\n\tds_read_b128 %8, %27\n\t"
        "ds_read_b128 %9, %28\n\tds_read_b128 %10, %29\n\tds_read_b128 %11, %30\n\t"
        "ds_read_b128 %12, %31\n\tds_read_b128 %13, %32\n\tds_read_b128 %14, %33\n\t"
        "ds_read_b128 %15, %34\n\tds_read_b128 %16, %35\n\tds_read_b128 %17, %36\n\t"
        "ds_read_b128 %18, %37\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]),
          "=&v"(x[12]), "=&v"(x[13]), "=&v"(x[14]), "=&v"(x[15]), "=&v"(x[16]), "=&v"(x[17]),
          "=&v"(x[18])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]),
          "v"(a[14]), "v"(a[15]), "v"(a[16]), "v"(a[17]), "v"(a[18])
        : "memory");
  } else if constexpr (N == 20) {
    asm volatile(
        "ds_read_b128 %0, %20\n\tds_read_b128 %1, %21\n\tds_read_b128 %2, %22\n\t"
        "ds_read_b128 %3, %23\n\tds_read_b128 %4, %24\n\tds_read_b128 %5, %25\n\t"
        "ds_read_b128 %6, %26\n\tds_read_b128 %7, %27\n\tds_read_b128 %8, %28\n\t"
        "ds_read_b128 %9, %29\n\tds_read_b128 %10, %30\n\tds_read_b128 %11, %31\n\t"
        "ds_read_b128 %12, %32\n\tds_read_b128 %13, %33\n\tds_read_b128 %14, %34\n\t"
        "ds_read_b128 %15, %35\n\tds_read_b128 %16, %36\n\tds_read_b128 %17, %37\n\t"
        "ds_read_b128 %18, %38\n\tds_read_b128 %19, %39\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]),
          "=&v"(x[12]), "=&v"(x[13]), "=&v"(x[14]), "=&v"(x[15]), "=&v"(x[16]), "=&v"(x[17]),
          "=&v"(x[18]), "=&v"(x[19])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]),
          "v"(a[14]), "v"(a[15]), "v"(a[16]), "v"(a[17]), "v"(a[18]), "v"(a[19])
        : "memory");
  } else if constexpr (N == 21) {
    asm volatile(
        "ds_read_b128 %0, %21\n\tds_read_b128 %1, %22\n\tds_read_b128 %2, %23\n\t"
        "ds_read_b128 %3, %24\n\tds_read_b128 %4, %25\n\tds_read_b128 %5, %26\n\t"
        "ds_read_b128 %6, %27\n\tds_read_b128 %7, %28\n\tds_read_b128 %8, %29\n\t"
        "ds_read_b128 %9, %30\n\tds_read_b128 %10, %31\n\tds_read_b128 %11, %32\n\t"
        "ds_read_b128 %12, %33\n\tds_read_b128 %13, %34\n\tds_read_b128 %14, %35\n\t"
        "ds_read_b128 %15, %36\n\tds_read_b128 %16, %37\n\tds_read_b128 %17, %38\n\t"
        "ds_read_b128 %18, %39\n\tds_read_b128 %19, %40\n\tds_read_b128 %20, %41\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]),
          "=&v"(x[12]), "=&v"(x[13]), "=&v"(x[14]), "=&v"(x[15]), "=&v"(x[16]), "=&v"(x[17]),
          "=&v"(x[18]), "=&v"(x[19]), "=&v"(x[20])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]),
          "v"(a[14]), "v"(a[15]), "v"(a[16]), "v"(a[17]), "v"(a[18]), "v"(a[19]), "v"(a[20])
        : "memory");
  } else if constexpr (N == 22) {
    asm volatile(
        "ds_read_b128 %0, %22\n\tds_read_b128 %1, %23\n\tds_read_b128 %2, %24\n\t"
        "ds_read_b128 %3, %25\n\tds_read_b128 %4, %26\n\tds_read_b128 %5, %27\n\t"
        "ds_read_b128 %6, %28\n\tds_read_b128 %7, %29\n\tds_read_b128 %8, %30\n\t"
        "ds_read_b128 %9, %31\n\tds_read_b128 %10, %32\n\tds_read_b128 %11, %33\n\t"
        "ds_read_b128 %12, %34\n\tds_read_b128 %13, %35\n\tds_read_b128 %14, %36\n\t"
        "ds_read_b128 %15, %37\n\tds_read_b128 %16, %38\n\tds_read_b128 %17, %39\n\t"
        "ds_read_b128 %18, %40\n\tds_read_b128 %19, %41\n\tds_read_b128 %20, %42\n\t"
        "ds_read_b128 %21, %43\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]),
          "=&v"(x[12]), "=&v"(x[13]), "=&v"(x[14]), "=&v"(x[15]), "=&v"(x[16]), "=&v"(x[17]),
          "=&v"(x[18]), "=&v"(x[19]), "=&v"(x[20]), "=&v"(x[21])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]),
          "v"(a[14]), "v"(a[15]), "v"(a[16]), "v"(a[17]), "v"(a[18]), "v"(a[19]), "v"(a[20]),
          "v"(a[21])
        : "memory");
  } else if constexpr (N == 23) {
    asm volatile(
        "ds_read_b128 %0, %23\n\tds_read_b128 %1, %24\n\tds_read_b128 %2, %25\n\t"
        "ds_read_b128 %3, %26\n\tds_read_b128 %4, %27\n\tds_read_b128 %5, %28\n\t"
        "ds_read_b128 %6, %29\n\tds_read_b128 %7, %30\n\tds_read_b128 %8, %31\n\t"
        "ds_read_b128 %9, %32\n\tds_read_b128 %10, %33\n\tds_read_b128 %11, %34\n\t"
        "ds_read_b128 %12, %35\n\tds_read_b128 %13, %36\n\tds_read_b128 %14, %37\n\t"
        "ds_read_b128 %15, %38\n\tds_read_b128 %16, %39\n\tds_read_b128 %17, %40\n\t"
        "ds_read_b128 %18, %41\n\tds_read_b128 %19, %42\n\tds_read_b128 %20, %43\n\t"
        "ds_read_b128 %21, %44\n\tds_read_b128 %22, %45\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]),
          "=&v"(x[12]), "=&v"(x[13]), "=&v"(x[14]), "=&v"(x[15]), "=&v"(x[16]), "=&v"(x[17]),
          "=&v"(x[18]), "=&v"(x[19]), "=&v"(x[20]), "=&v"(x[21]), "=&v"(x[22])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]),
          "v"(a[14]), "v"(a[15]), "v"(a[16]), "v"(a[17]), "v"(a[18]), "v"(a[19]), "v"(a[20]),
          "v"(a[21]), "v"(a[22])
        : "memory");
  } else if constexpr (N == 24) {
    asm volatile(
        "ds_read_b128 %0, %24\n\tds_read_b128 %1, %25\n\tds_read_b128 %2, %26\n\t"
        "ds_read_b128 %3, %27\n\tds_read_b128 %4, %28\n\tds_read_b128 %5, %29\n\t"
        "ds_read_b128 %6, %30\n\tds_read_b128 %7, %31\n\tds_read_b128 %8, %32\n\t"
        "ds_read_b128 %9, %33\n\tds_read_b128 %10, %34\n\tds_read_b128 %11, %35\n\t"
        "ds_read_b128 %12, %36\n\tds_read_b128 %13, %37\n\tds_read_b128 %14, %38\n\t"
        "ds_read_b128 %15, %39\n\tds_read_b128 %16, %40\n\tds_read_b128 %17, %41\n\t"
        "ds_read_b128 %18, %42\n\tds_read_b128 %19, %43\n\tds_read_b128 %20, %44\n\t"
        "ds_read_b128 %21, %45\n\tds_read_b128 %22, %46\n\tds_read_b128 %23, %47\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]),
          "=&v"(x[12]), "=&v"(x[13]), "=&v"(x[14]), "=&v"(x[15]), "=&v"(x[16]), "=&v"(x[17]),
          "=&v"(x[18]), "=&v"(x[19]), "=&v"(x[20]), "=&v"(x[21]), "=&v"(x[22]), "=&v"(x[23])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]),
          "v"(a[14]), "v"(a[15]), "v"(a[16]), "v"(a[17]), "v"(a[18]), "v"(a[19]), "v"(a[20]),
          "v"(a[21]), "v"(a[22]), "v"(a[23])
        : "memory");
  }
}

// Eight 16-byte LDS reads from two base offsets, four each at steps of STRIDE bytes
// (immediate offsets), completed within the statement like lds_read_b128.
template <int STRIDE>
DEV void lds_read_b128_2x4(bf16x8 (&x)[8], uint32_t b0, uint32_t b1) {
  static_assert(3 * STRIDE < 65536, "ds offset range");
  asm volatile(
      "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:%10\n\t"
      "ds_read_b128 %2, %8 offset:%11\n\tds_read_b128 %3, %8 offset:%12\n\t"
      "ds_read_b128 %4, %9\n\tds_read_b128 %5, %9 offset:%10\n\t"
      "ds_read_b128 %6, %9 offset:%11\n\tds_read_b128 %7, %9 offset:%12\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
        "=&v"(x[6]), "=&v"(x[7])
      : "v"(b0), "v"(b1), "n"(STRIDE), "n"(2 * STRIDE), "n"(3 * STRIDE)
      : "memory");
}

// LDS writes of this wave complete and ordered before its following LDS reads (for
// exchanges between the lanes of one wave; lgkmcnt(0), then a scheduling barrier).
DEV void wave_lds_sync() {
  // the empty asm statements keep the compiler from moving memory accesses across: a
  // lane's LDS read after the sync need not touch the addresses that lane wrote before
  // it, so without them the compiler may read before the other lanes' writes
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// MFMA 16x16x32 bf16 -> f32 (gfx950).  Lane l holds A[row l%16][k 8(l/16)..+8],
// B[k 8(l/16)..+8][col l%16]; D lane l holds rows 4(l/16)+i, col l%16, i = 0..3.
DEV floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
