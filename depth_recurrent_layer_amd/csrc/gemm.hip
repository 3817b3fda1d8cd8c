// C = A . B^T with fused epilogues, for the dense projections (QKV, O, router rank-r
// projection) and the grouped linear-MoE projections.
//
// bf16 path: MFMA (v_mfma_f32_16x16x32_bf16) over a multi-stage LDS ring, 256 threads =
// 2 x 2 waves.
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

// K streams through a ring of NS stages of 32-wide K slices filled by direct global->LDS
// loads (global_load_lds_dwordx4), NS - 1 slices in flight per block.  A stage holds
// the BM A rows then the BN B rows of one slice as 64-byte rows; the four 16-byte chunks
// of row r are XOR-swizzled (chunk c at slot c ^ ((r >> 1) & 3)) so the 8 rows read by
// 8 consecutive lanes of one MFMA fragment load cover all 32 banks.  2 x 2 waves, each
// owning a WM x WN sub-tile (WM/16 x WN/16 MFMA tiles).  After the K loop every wave
// stages its own sub-tile in LDS and writes whole rows with 16-byte stores.
#ifndef DREAMER_GEMM_RING_BYTES
#define DREAMER_GEMM_RING_BYTES 65536  // ring budget per block (two blocks per CU)
#endif

// QKVONLY: an instance for the Q/K/V projection only (bf16 output, QKV epilogue), whose
// epilogue staging is bf16 and therefore smaller.  RING: LDS budget of the K ring; OCC:
// blocks per CU the instance is built for.
template <int WM, int WN, bool QKVONLY, int RING>
struct GemmShape {
  static constexpr int BM = 2 * WM, BN = 2 * WN, TM = WM / 16, TN = WN / 16;
  static constexpr int STAGE = (BM + BN) * 64;  // bytes per K slice
  static constexpr int NI = (BM + BN) / 16;     // 1 KiB load instructions per stage
  static constexpr int LPW = NI / 4;            // per wave
  static constexpr int NS0 = RING / STAGE;
  static constexpr int NS = NS0 > 8 ? 8 : NS0;  // ring depth
  // epilogue staging per wave: float32 rows of WN (+4), or bf16 rows of WN (+8)
  static constexpr int LDF = WN + 4, LDB = WN + 8;
  static constexpr int WAVE_STAGE = QKVONLY ? WM * LDB * 2 : WM * LDF * 4;
  static constexpr int SMEM = NS * STAGE > 4 * WAVE_STAGE ? NS * STAGE : 4 * WAVE_STAGE;
  static_assert(NI % 4 == 0, "stage must split evenly over 4 waves");
  static_assert(NS >= 2, "ring too small");
};

template <typename OutT, int WM, int WN, bool QKVONLY = false,
          int RING = DREAMER_GEMM_RING_BYTES, int OCC = 2>
__global__ __launch_bounds__(256, OCC) void gemm_bf16_kernel(GemmArgs a) {
  using S = GemmShape<WM, WN, QKVONLY, RING>;
  constexpr int BM = S::BM, BN = S::BN, TM = S::TM, TN = S::TN;
  __shared__ __attribute__((aligned(1024))) char ring[S::SMEM];
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
    const int m = m_begin + i;
    rows_s[i] = (m < m_end) ? (a.rows ? a.rows[m] : m) : -1;
  }
  __syncthreads();

  // load descriptors: wave w issues instructions q = w + 4 j of every stage; lane L of
  // instruction q fills row 16 q' + L / 4, slot L % 4 of its section
  const int lane = tid & 63, w = tid >> 6;
  const bf16* src[S::LPW];
#pragma unroll
  for (int j = 0; j < S::LPW; ++j) {
    const int q = w + 4 * j, slot = lane & 3;
    if (q < BM / 16) {
      const int row = q * 16 + (lane >> 2);
      const int o = rows_s[row] >= 0 ? rows_s[row] : rows_s[0];  // pad rows repeat row 0
      src[j] = A + (int64_t)(o / a.row_div) * a.lda + (swz64_slot(row, slot) << 3);
    } else {
      const int row = (q - BM / 16) * 16 + (lane >> 2);
      const int n = min(n0 + row, a.N - 1);
      src[j] = B + (int64_t)n * a.ldb + (swz64_slot(row, slot) << 3);
    }
  }
  auto issue = [&](int s) {
    char* sb = ring + (s % S::NS) * S::STAGE;
#pragma unroll
    for (int j = 0; j < S::LPW; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(src[j] + s * 32),
                                       (lds_void*)(sb + (w + 4 * j) * 1024), 16, 0, 0);
  };

  const int wm = w >> 1, wn = w & 1, lr = lane & 15, lg = lane >> 4;
  floatx4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Epilogue operands that do not depend on the product are fetched before the K loop so
  // that their latency hides behind it: the rotary table entries of the QKV epilogue
  // (per row for sequence positions, per pair for depth), or the float32 residual of the
  // generic epilogue (the 8-column chunks this lane will write).
  constexpr bool QKV = WN == 64 && sizeof(OutT) == 2;
  constexpr int CPR = WN / 8, NIT = WM * CPR / 64;  // generic epilogue items per lane
  const int rw0 = wm * WM, cw0 = n0 + wn * WN;      // this wave's first tile row, column
  const int sect = a.qkv_h ? a.qkv_sect0 + cw0 / a.qkv_h : -1;
  const bool sa_qk = QKV && a.qkv_h && (sect == 0 || sect == 1) && a.sa_rope;
  const bool da_qk = QKV && a.qkv_h && (sect == 3 || sect == 4);
  // Rotary table entries (interleaved RopeJobs t4 layout, one 16-byte load gives a lane the
  // cos / sin of both its pairs lr and lr + 16): the sequence rotation per row position;
  // the depth rotation at l for pairs < 16 and at L-1-l for the others.  They are loaded
  // after the ring's first stages (so stage 0 does not wait for them) when registers allow,
  // else in the epilogue.
  auto row_pos = [&](int i, int v) {
    const int orow = rows_s[rw0 + i * 16 + lg * 4 + v];
    return a.pos_fixed >= 0 ? a.pos_fixed : (orow >= 0 ? orow % a.seq : 0);
  };
  constexpr bool PRE_TAB = QKV && TM * OCC <= 8;  // register room for the row entries
  float4 tq[PRE_TAB ? TM : 1][4];
  float4 td0 = {}, td1 = {};
  int n_tab = 0;  // table loads issued behind the ring's first stages
  auto load_seq_tables = [&](float4 (&t)[PRE_TAB ? TM : 1][4]) {
#pragma unroll
    for (int i = 0; i < (PRE_TAB ? TM : 1); ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) t[i][v] = a.rope_s4[row_pos(i, v) * 16 + lr];
  };
  float rres[QKV ? 1 : NIT][8];
  if constexpr (QKV) {
  } else {
    if (a.resid) {
#pragma unroll
      for (int m = 0; m < NIT; ++m) {
        const int it = lane + 64 * m, rt = it / CPR, n = cw0 + (it % CPR) * 8;
        const int orow = rows_s[rw0 + rt];
        if (orow >= 0 && n < a.N) {
          load16(a.resid + (int64_t)orow * a.ldr + n, rres[m]);
          load16(a.resid + (int64_t)orow * a.ldr + n + 4, rres[m] + 4);
        }
      }
    }
  }

  const int nst = a.K / 32;
  const uint32_t ring0 = lds_off(ring);
  for (int s = 0; s < S::NS - 1 && s < nst; ++s) issue(s);
  if constexpr (QKV) {
    if (da_qk) {
      td0 = a.rope_d4[a.depth_l * 16 + lr];
      td1 = a.rope_d4[(a.depth_L - 1 - a.depth_l) * 16 + lr];
      n_tab = 2;
    } else if (PRE_TAB && sa_qk) {
      load_seq_tables(tq);
      n_tab = TM * 4;
    }
  }
  for (int s = 0; s < nst; ++s) {
    // stage s has landed once only the loads issued after it are outstanding: the later
    // stages', and the table loads while s is one of the stages issued before them
    wait_vmcnt_upto(S::LPW * min(S::NS - 2, nst - 1 - s) + (s <= S::NS - 2 ? n_tab : 0));
    ring_barrier();  // stage s visible to every wave; stage s - 1 consumed by every wave
    if (s + S::NS - 1 < nst) issue(s + S::NS - 1);
    const uint32_t sb = ring0 + (s % S::NS) * S::STAGE;
    uint32_t ad[TM + TN];
    bf16x8 fr[TM + TN];  // A fragments, then B fragments
#pragma unroll
    for (int i = 0; i < TM; ++i) ad[i] = sb + swz64(wm * WM + i * 16 + lr, lg);
#pragma unroll
    for (int j = 0; j < TN; ++j) ad[TM + j] = sb + BM * 64 + swz64(wn * WN + j * 16 + lr, lg);
    lds_read_b128<TM + TN>(fr, ad);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(fr[i], fr[TM + j], acc[i][j]);
  }
  __syncthreads();  // every wave is done with the ring; it becomes epilogue staging

  char* wst = ring + w * S::WAVE_STAGE;
  OutT* C = (OutT*)a.C;
  if constexpr (QKV) {
    if (a.qkv_h) {
      // the wave's 64 columns are one head of one section (qkv_h % 128 == 0, BN = 128)
      const int hcol0 = cw0 % a.qkv_h;
      bf16* sw = reinterpret_cast<bf16*>(wst);  // [WM][LDB]
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        float4 ti[4];  // this m-tile's sequence-rotation entries, one per row
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if constexpr (PRE_TAB) ti[v] = tq[i][v];
          else if (sa_qk) ti[v] = a.rope_s4[row_pos(i, v) * 16 + lr];
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int rt = i * 16 + lg * 4 + v;  // row within the wave
          const int orow = rows_s[rw0 + rt];
          const float sc = (a.row_scale && orow >= 0) ? a.row_scale[orow] : 1.0f;
#pragma unroll
          for (int j = 0; j < 2; ++j) {  // rotate-half pairs (c, c + 32), c = 16 j + lr
            const int pair = j * 16 + lr;
            float x = acc[i][j][v] * sc, y = acc[i][j + 2][v] * sc;
            if (sa_qk || da_qk) {
              float cv, sv;
              if (sa_qk) {
                const float4 t = ti[v];
                cv = j == 0 ? t.x : t.y;
                sv = j == 0 ? t.z : t.w;
              } else {
                cv = j == 0 ? td0.x : td1.y;
                sv = j == 0 ? td0.z : td1.w;
              }
              const float xr = x * cv - y * sv;
              y = y * cv + x * sv;
              x = xr;
            }
            sw[rt * S::LDB + pair] = (bf16)x;
            sw[rt * S::LDB + pair + 32] = (bf16)y;
          }
        }
      }
      wave_lds_sync();
      // rows of 64 bf16 = 8 chunks of 16 bytes
      for (int it = lane; it < WM * 8; it += 64) {
        const int rt = it >> 3, ch = it & 7;
        const int orow = rows_s[rw0 + rt];
        if (orow < 0) continue;
        *reinterpret_cast<bf16x8*>(C + (int64_t)orow * a.ldc + cw0 + ch * 8) =
            *reinterpret_cast<const bf16x8*>(sw + rt * S::LDB + ch * 8);
      }
      if (sect == 2 && a.vt) {  // SA v, transposed: item = (dim, 8 consecutive rows)
        bf16* vt = (bf16*)a.vt;
        const int H = a.qkv_h / 64, head = hcol0 >> 6;
        for (int it = lane; it < 64 * (WM / 8); it += 64) {
          const int dim = it & 63, rg = it >> 6;
          const int o0 = rows_s[rw0 + rg * 8];
          const bool run = o0 >= 0 && o0 % 8 == 0 && rows_s[rw0 + rg * 8 + 7] == o0 + 7 &&
                           (o0 % a.seq) + 7 < a.seq;
          if (run) {
            bf16x8 vv;
#pragma unroll
            for (int r = 0; r < 8; ++r) vv[r] = sw[(rg * 8 + r) * S::LDB + dim];
            *reinterpret_cast<bf16x8*>(
                vt + (((int64_t)(o0 / a.seq) * H + head) * 64 + dim) * a.seq + o0 % a.seq) = vv;
          } else {
            for (int r = 0; r < 8; ++r) {
              const int orow = rows_s[rw0 + rg * 8 + r];
              if (orow < 0) continue;
              vt[(((int64_t)(orow / a.seq) * H + head) * 64 + dim) * a.seq + orow % a.seq] =
                  sw[(rg * 8 + r) * S::LDB + dim];
            }
          }
        }
      }
      return;
    }
  }
  if constexpr (QKVONLY) return;
  // generic: v = acc * row_scale + resid; C (OutT) and optional bf16 copy C2
  float* sf = reinterpret_cast<float*>(wst);  // [WM][LDF]
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) sf[(i * 16 + lg * 4 + v) * S::LDF + j * 16 + lr] = acc[i][j][v];
  wave_lds_sync();
  bf16* C2 = (bf16*)a.C2;
#pragma unroll
  for (int m = 0; m < NIT; ++m) {
    const int it = lane + 64 * m, rt = it / CPR, cc = it % CPR;
    const int orow = rows_s[rw0 + rt];
    const int n = cw0 + cc * 8;
    if (orow < 0 || n >= a.N) continue;
    const float sc = a.row_scale ? a.row_scale[orow] : 1.0f;
    const floatx4 c0 = *reinterpret_cast<const floatx4*>(sf + rt * S::LDF + cc * 8);
    const floatx4 c1 = *reinterpret_cast<const floatx4*>(sf + rt * S::LDF + cc * 8 + 4);
    float val[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      val[e] = c0[e] * sc;
      val[4 + e] = c1[e] * sc;
    }
    if constexpr (!QKV) {
      if (a.resid) {
#pragma unroll
        for (int e = 0; e < 8; ++e) val[e] += rres[m][e];
      }
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
  if (a.K % 32 != 0 || a.N % 8 != 0) return -1;
  // Tiles: 128 x 128 when that gives >= 512 blocks (two per CU), else 64 x 128, else
  // 64 x 64; the QKV epilogue needs 64-column wave tiles (one head), grouped launches the
  // 64-row m-tiles their tile offsets were built with.
  int bm, bn;
  if (a.qkv_h) {
    if (a.qkv_h % 128 || out_f32 || !a.rope_d4 || (a.sa_rope && !a.rope_s4)) return -1;
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
  // QKV projections with the rotary epilogue: 256 x 128 tiles at two blocks per CU once
  // they fill the chip, else 128 x 128 tiles at three per CU (one round for up to 768
  // tiles); small M keeps the 64 x 128 tiles chosen above.
  if (a.qkv_h && !a.toff && tiles(256, 128) >= 512) {
    dim3 g2((a.M + 255) / 256, (a.N + 127) / 128);
    gemm_bf16_kernel<bf16, 128, 64, true, 73728, 2><<<g2, 256, 0, st>>>(a);
    return 0;
  }
  if (a.qkv_h && !a.toff && tiles(128, 128) >= 256) {
    dim3 g3((a.M + 127) / 128, (a.N + 127) / 128);
    gemm_bf16_kernel<bf16, 64, 64, true, 49152, 3><<<g3, 256, 0, st>>>(a);
    return 0;
  }
#define DREAMER_GEMM_LAUNCH(OUT)                                                  \
  if (bm == 128) gemm_bf16_kernel<OUT, 64, 64><<<grid, 256, 0, st>>>(a);          \
  else if (bn == 128) gemm_bf16_kernel<OUT, 32, 64><<<grid, 256, 0, st>>>(a);     \
  else gemm_bf16_kernel<OUT, 32, 32><<<grid, 256, 0, st>>>(a);
  if (out_f32) {
    DREAMER_GEMM_LAUNCH(float)
  } else {
    DREAMER_GEMM_LAUNCH(bf16)
  }
#undef DREAMER_GEMM_LAUNCH
  return 0;
}

}  // namespace dreamer
