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
  if constexpr (BN == 128 && sizeof(OutT) == 2) {
    if (a.qkv_h) {  // the tile is two heads of one section
      const int sect = n0 / a.qkv_h, hcol0 = n0 % a.qkv_h;
      const bool sa_qk = (sect == 0 || sect == 1) && a.sa_rope;
      const bool da_qk = sect == 3 || sect == 4;
      // item = (row, head of the tile, chunk c < 4): dims c*8..+8 and 32+c*8..+8 rotate
      // together (rotate-half pairs)
      for (int it = tid; it < BM * 8; it += 256) {
        const int row = it >> 3, hh = (it >> 2) & 1, c = it & 3;
        const int orow = rows_s[row];
        if (orow < 0) continue;
        const float sc = a.row_scale ? a.row_scale[orow] : 1.0f;
        const int lc = hh * 64 + c * 8;
        float lo[8], hi[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          lo[e] = Cs[row * LDC + lc + e] * sc;
          hi[e] = Cs[row * LDC + lc + 32 + e] * sc;
        }
        if (sa_qk || da_qk) {
          int pf, pr;
          const float *cs, *sn;
          if (sa_qk) {
            pf = pr = a.pos_fixed >= 0 ? a.pos_fixed : orow % a.seq;
            cs = a.cos_s;
            sn = a.sin_s;
          } else {
            pf = a.depth_l;
            pr = a.depth_L - 1 - a.depth_l;
            cs = a.cos_d;
            sn = a.sin_d;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int pair = c * 8 + e;
            const int pos = pair < 16 ? pf : pr;
            const float cv = cs[pos * 32 + pair], sv = sn[pos * 32 + pair];
            const float x = lo[e], y = hi[e];
            lo[e] = x * cv - y * sv;
            hi[e] = y * cv + x * sv;
          }
        }
        OutT* cp = C + (int64_t)orow * a.ldc + n0 + lc;
        store16(cp, lo);
        store16(cp + 32, hi);
      }
      if (sect == 2 && a.vt) {  // SA v, transposed: item = (column, 8 consecutive rows)
        constexpr int RG = BM / 8;
        bf16* vt = (bf16*)a.vt;
        const int H = a.qkv_h / 64;
        for (int it = tid; it < RG * BN; it += 256) {
          const int col = it / RG, rg = it % RG;
          const int head = (hcol0 + col) >> 6, dim = (hcol0 + col) & 63;
          const int o0 = rows_s[rg * 8];
          const bool run = o0 >= 0 && rows_s[rg * 8 + 7] == o0 + 7 && (o0 % a.seq) + 7 < a.seq;
          if (run) {
            float vv[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
              const int orow = o0 + r;
              const float sc = a.row_scale ? a.row_scale[orow] : 1.0f;
              vv[r] = Cs[(rg * 8 + r) * LDC + col] * sc;
            }
            store16(vt + (((int64_t)(o0 / a.seq) * H + head) * 64 + dim) * a.seq + o0 % a.seq,
                    vv);
          } else {
            for (int r = 0; r < 8; ++r) {
              const int orow = rows_s[rg * 8 + r];
              if (orow < 0) continue;
              const float sc = a.row_scale ? a.row_scale[orow] : 1.0f;
              vt[(((int64_t)(orow / a.seq) * H + head) * 64 + dim) * a.seq + orow % a.seq] =
                  (bf16)(Cs[(rg * 8 + r) * LDC + col] * sc);
            }
          }
        }
      }
      return;
    }
  }
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
  // Tiles: the largest of 128x128, 64x128, 64x64 that still gives >= 512 blocks (two per
  // CU); the QKV epilogue needs 128-column tiles.
  int bm, bn;
  if (a.qkv_h) {
    if (a.qkv_h % 128 || out_f32) return -1;
    bn = 128;
  } else {
    bn = a.N >= 128 ? 128 : 64;
  }
  auto tiles = [&](int tm, int tn) {
    return (int64_t)((a.M + tm - 1) / tm) * ((a.N + tn - 1) / tn);
  };
  if (a.toff) {
    if (a.tile_m != 64) return -1;
    bm = 64;
  } else if (bn == 128 && tiles(128, 128) >= 512) {
    bm = 128;
  } else {
    bm = 64;
    if (!a.qkv_h && bn == 128 && tiles(64, 128) < 512) bn = 64;
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
