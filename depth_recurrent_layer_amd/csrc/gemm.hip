// C = A . B^T with fused epilogues, for the dense projections (QKV, O, router rank-r
// projection) and the grouped linear-MoE projections.
//
// bf16 path: LDS-tiled MFMA (v_mfma_f32_16x16x32_bf16), 256 threads = 2 x 2 waves,
// register prefetch of the next K tile while the current one is multiplied.
// f32 path: one thread per output element (used only for small float32 layers).
//
// Row model: the kernel walks "positions" m.  Position m reads A row
// (rows ? rows[m] / row_div : m) and writes output row (rows ? rows[m] : m); with
// groups, positions goff[g]..goff[g+1] use B + g * b_gstride.  Epilogue:
//   v = acc * (row_scale ? row_scale[out_row] : 1) + (resid ? resid[out_row, n] : 0)
//   C[out_row, n] = v (OutT);  C2[out_row, n] = bf16(v) if C2.
#include "common.h"
#include "kernels.h"

namespace dreamer {

template <typename OutT, typename ResT, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int BK = 64, LD = BK + 8;  // LDS row = 144 B (16-B aligned, spreads banks)
  constexpr int TM = BM / 32, TN = BN / 32;  // 16x16 tiles per wave (2 x 2 waves)
  constexpr int ACH = BM * 8 / 256, BCH = BN * 8 / 256;  // 16-B chunks per thread
  __shared__ __attribute__((aligned(16))) bf16 As[BM * LD];
  __shared__ __attribute__((aligned(16))) bf16 Bs[BN * LD];
  __shared__ int rows_s[BM];

  const int tid = threadIdx.x;
  int g = 0, m_begin, m_end;
  const int mtile = blockIdx.x;
  if (a.toff) {
    if (mtile >= a.toff[a.G]) return;
    int lo = 0, hi = a.G - 1;  // largest g with toff[g] <= mtile
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (a.toff[mid] <= mtile) lo = mid; else hi = mid - 1;
    }
    g = lo;
    m_begin = a.goff[g] + (mtile - a.toff[g]) * BM;
    m_end = a.goff[g + 1];
  } else {
    m_begin = mtile * BM;
    m_end = a.M;
  }
  const int n0 = blockIdx.y * BN;
  const bf16* __restrict__ A = (const bf16*)a.A;
  const bf16* __restrict__ B = (const bf16*)a.B + (int64_t)g * a.b_gstride;

  for (int i = tid; i < BM; i += 256) {
    int m = m_begin + i;
    rows_s[i] = (m < m_end) ? (a.rows ? a.rows[m] : m) : -1;
  }
  __syncthreads();

  // global -> register staging
  const bf16* aptr[ACH];
  const bf16* bptr[BCH];
#pragma unroll
  for (int j = 0; j < ACH; ++j) {
    int c = tid + 256 * j, row = c >> 3, kc = c & 7;
    int src = rows_s[row];
    aptr[j] = src >= 0 ? A + (int64_t)(src / a.row_div) * a.lda + kc * 8 : nullptr;
  }
#pragma unroll
  for (int j = 0; j < BCH; ++j) {
    int c = tid + 256 * j, row = c >> 3, kc = c & 7;
    int n = n0 + row;
    bptr[j] = n < a.N ? B + (int64_t)n * a.ldb + kc * 8 : nullptr;
  }
  bf16x8 ra[ACH], rb[BCH];
  const bf16x8 zero8 = {};
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < ACH; ++j)
      ra[j] = aptr[j] ? *reinterpret_cast<const bf16x8*>(aptr[j] + k0) : zero8;
#pragma unroll
    for (int j = 0; j < BCH; ++j)
      rb[j] = bptr[j] ? *reinterpret_cast<const bf16x8*>(bptr[j] + k0) : zero8;
  };
  auto lstore = [&]() {
#pragma unroll
    for (int j = 0; j < ACH; ++j) {
      int c = tid + 256 * j, row = c >> 3, kc = c & 7;
      *reinterpret_cast<bf16x8*>(&As[row * LD + kc * 8]) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < BCH; ++j) {
      int c = tid + 256 * j, row = c >> 3, kc = c & 7;
      *reinterpret_cast<bf16x8*>(&Bs[row * LD + kc * 8]) = rb[j];
    }
  };

  const int lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  const int lr = lane & 15, lg = lane >> 4;
  floatx4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore();
  __syncthreads();
  for (int k0 = 0; k0 < a.K; k0 += BK) {
    const bool more = k0 + BK < a.K;
    if (more) gload(k0 + BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(
            &As[(wm * (BM / 2) + i * 16 + lr) * LD + ks * 32 + lg * 8]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(
            &Bs[(wn * (BN / 2) + j * 16 + lr) * LD + ks * 32 + lg * 8]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
    }
    if (more) {
      __syncthreads();
      lstore();
      __syncthreads();
    }
  }

  // epilogue
  OutT* C = (OutT*)a.C;
  bf16* C2 = (bf16*)a.C2;
  const ResT* R = (const ResT*)a.resid;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int ml = wm * (BM / 2) + i * 16 + lg * 4 + v;
      const int orow = rows_s[ml];
      if (orow < 0) continue;
      const float sc = a.row_scale ? a.row_scale[orow] : 1.0f;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * (BN / 2) + j * 16 + lr;
        if (n >= a.N) continue;
        float val = acc[i][j][v] * sc;
        if (R) val += to_f(R[(int64_t)orow * a.ldr + n]);
        C[(int64_t)orow * a.ldc + n] = from_f<OutT>(val);
        if (C2) C2[(int64_t)orow * a.ldc2 + n] = (bf16)val;
      }
    }
  }
}

// float32 reference-style kernel: one thread per (position, column).
__global__ void gemm_f32_kernel(GemmArgs a) {
  const int n = blockIdx.x * 16 + (threadIdx.x & 15);
  const int m = blockIdx.y * 16 + (threadIdx.x >> 4);
  if (m >= a.M || n >= a.N) return;
  int g = 0;
  if (a.goff) {
    if (m >= a.goff[a.G]) return;
    int lo = 0, hi = a.G - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (a.goff[mid] <= m) lo = mid; else hi = mid - 1;
    }
    g = lo;
  }
  const int orow = a.rows ? a.rows[m] : m;
  const float* A = (const float*)a.A + (int64_t)(orow / a.row_div) * a.lda;
  const float* B = (const float*)a.B + (int64_t)g * a.b_gstride + (int64_t)n * a.ldb;
  float acc = 0.f;
  for (int k = 0; k < a.K; ++k) acc = fmaf(A[k], B[k], acc);
  float val = acc * (a.row_scale ? a.row_scale[orow] : 1.0f);
  if (a.resid) val += ((const float*)a.resid)[(int64_t)orow * a.ldr + n];
  ((float*)a.C)[(int64_t)orow * a.ldc + n] = val;
  if (a.C2) ((float*)a.C2)[(int64_t)orow * a.ldc2 + n] = val;
}

int launch_gemm(const GemmArgs& a, int dtype, int out_f32, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return 0;
  if (dtype == DT_F32) {
    dim3 grid((a.N + 15) / 16, (a.M + 15) / 16);
    gemm_f32_kernel<<<grid, 256, 0, st>>>(a);
    return 0;
  }
  if (a.K % 64 != 0) return -1;
  // Tile choice: 128x128 when that still gives >= 2 tiles per CU, else 64-row tiles.
  // Grouped launches use the m-tile size their tile offsets were built with.
  int bm, bn = a.N >= 128 ? 128 : 64;
  if (a.toff) {
    if (a.tile_m != 64) return -1;
    bm = 64;
  } else {
    const int64_t tiles128 = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128);
    bm = (bn == 128 && tiles128 >= 512) ? 128 : 64;
  }
  const int mt = (a.M + bm - 1) / bm + (a.toff ? a.G : 0);
  dim3 grid(mt, (a.N + bn - 1) / bn);
#define DREAMER_GEMM_LAUNCH(OUT)                                                    \
  if (bm == 128) gemm_bf16_kernel<OUT, float, 128, 128><<<grid, 256, 0, st>>>(a);   \
  else if (bn == 128) gemm_bf16_kernel<OUT, float, 64, 128><<<grid, 256, 0, st>>>(a); \
  else gemm_bf16_kernel<OUT, float, 64, 64><<<grid, 256, 0, st>>>(a);
  if (out_f32) {
    DREAMER_GEMM_LAUNCH(float)
  } else {
    DREAMER_GEMM_LAUNCH(bf16)
  }
#undef DREAMER_GEMM_LAUNCH
  return 0;
}

}  // namespace dreamer
