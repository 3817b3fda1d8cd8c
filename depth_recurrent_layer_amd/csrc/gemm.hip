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

// LDS tile layout: rows of BK = 64 bf16 (128 B), 16-byte chunks XOR-swizzled by row
// (chunk c of row r lives at slot c ^ (r & 7)), so the 16 rows read by one MFMA
// fragment load hit distinct banks without padding.
DEV int swz(int row, int kc) { return row * 64 + ((kc ^ (row & 7)) << 3); }

template <typename OutT, typename ResT, int BM, int BN>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int BK = 64;
  constexpr int TM = BM / 32, TN = BN / 32;              // 16x16 tiles per wave (2 x 2 waves)
  constexpr int ACH = BM * 8 / 256, BCH = BN * 8 / 256;  // 16-B chunks per thread per tile
  // A/B tiles during the K loop; the float32 C tile (rows padded by 4) in the epilogue
  constexpr int LDC = BN + 4;
  constexpr int AB_BYTES = 2 * (BM + BN) * BK * 2, C_BYTES = BM * LDC * 4;
  __shared__ __attribute__((aligned(16))) char smem[AB_BYTES > C_BYTES ? AB_BYTES : C_BYTES];
  bf16 (*As)[BM * BK] = reinterpret_cast<bf16 (*)[BM * BK]>(smem);
  bf16 (*Bs)[BN * BK] = reinterpret_cast<bf16 (*)[BN * BK]>(smem + 2 * BM * BK * 2);
  float* Cs = reinterpret_cast<float*>(smem);
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

  // Thread -> (row, chunk) of the tiles it stages; source rows as 32-bit indices.
  const int kc = tid & 7, r0 = tid >> 3;  // rows r0 + 32 j
  int arow[ACH], brow[BCH];
#pragma unroll
  for (int j = 0; j < ACH; ++j) {
    const int src = rows_s[r0 + 32 * j];
    arow[j] = src >= 0 ? src / a.row_div : -1;
  }
#pragma unroll
  for (int j = 0; j < BCH; ++j) {
    const int n = n0 + r0 + 32 * j;
    brow[j] = n < a.N ? n : -1;
  }
  bf16x8 ra[ACH], rb[BCH];
  const bf16x8 zero8 = {};
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < ACH; ++j)
      ra[j] = arow[j] >= 0
                  ? *reinterpret_cast<const bf16x8*>(A + (int64_t)arow[j] * a.lda + k0 + kc * 8)
                  : zero8;
#pragma unroll
    for (int j = 0; j < BCH; ++j)
      rb[j] = brow[j] >= 0
                  ? *reinterpret_cast<const bf16x8*>(B + (int64_t)brow[j] * a.ldb + k0 + kc * 8)
                  : zero8;
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < ACH; ++j)
      *reinterpret_cast<bf16x8*>(&As[buf][swz(r0 + 32 * j, kc)]) = ra[j];
#pragma unroll
    for (int j = 0; j < BCH; ++j)
      *reinterpret_cast<bf16x8*>(&Bs[buf][swz(r0 + 32 * j, kc)]) = rb[j];
  };

  const int lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  const int lr = lane & 15, lg = lane >> 4;
  floatx4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < a.K; k0 += BK) {
    const bool more = k0 + BK < a.K;
    if (more) gload(k0 + BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8 bfr[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(
            &Bs[buf][swz(wn * (BN / 2) + j * 16 + lr, ks * 4 + lg)]);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(
            &As[buf][swz(wm * (BM / 2) + i * 16 + lr, ks * 4 + lg)]);
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(af, bfr[j], acc[i][j]);
      }
    }
    if (more) {
      lstore(buf ^ 1);  // the other buffer was last read before the previous barrier
      __syncthreads();
      buf ^= 1;
    }
  }

  // epilogue: accumulators -> LDS (float32), then every thread handles 8-column chunks of
  // whole rows so the residual loads and the output stores are 16-byte and coalesced
  __syncthreads();  // all waves are done reading the A/B tiles
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        Cs[(wm * (BM / 2) + i * 16 + lg * 4 + v) * LDC + wn * (BN / 2) + j * 16 + lr] =
            acc[i][j][v];
  __syncthreads();
  OutT* C = (OutT*)a.C;
  bf16* C2 = (bf16*)a.C2;
  const ResT* R = (const ResT*)a.resid;
  constexpr int CPR = BN / 8;  // 8-column chunks per row
  for (int c = tid; c < BM * CPR; c += 256) {
    const int row = c / CPR, cc = c % CPR;
    const int orow = rows_s[row];
    const int n = n0 + cc * 8;
    if (orow < 0 || n >= a.N) continue;
    const float sc = a.row_scale ? a.row_scale[orow] : 1.0f;
    float val[8];
    const floatx4 c0 = *reinterpret_cast<const floatx4*>(&Cs[row * LDC + cc * 8]);
    const floatx4 c1 = *reinterpret_cast<const floatx4*>(&Cs[row * LDC + cc * 8 + 4]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      val[e] = c0[e] * sc;
      val[4 + e] = c1[e] * sc;
    }
    if (R) {
      float rv[8];
      load16(R + (int64_t)orow * a.ldr + n, rv);
      load16(R + (int64_t)orow * a.ldr + n + 4, rv + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) val[e] += rv[e];
    }
    OutT* cp = C + (int64_t)orow * a.ldc + n;
    if constexpr (sizeof(OutT) == 2) {
      store16(cp, val);
    } else {
      store16(cp, val);
      store16(cp + 4, val + 4);
    }
    if (C2) store16(C2 + (int64_t)orow * a.ldc2 + n, val);
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
  if (a.K % 64 != 0 || a.N % 8 != 0) return -1;
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
