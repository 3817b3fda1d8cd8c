// C = A . B^T with fused epilogues, for the dense projections (QKV, O, router rank-r
// projection) and the grouped linear-MoE projections.
//
// bf16 path: MFMA (v_mfma_f32_16x16x32_bf16) over a multi-stage LDS ring; the tile,
// wave grid, slice width, ring depth and blocks per CU come from a GemmCfg instance
// chosen per launch shape (launch_gemm).
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

// K streams through a ring of NS stages filled by direct global->LDS loads
// (global_load_lds_dwordx4), NS - 1 stages in flight per block.  A stage holds a K slice
// of BKB bytes (32 or 64 elements) of the BM A rows, then of the BN B rows; the 16-byte
// chunks of row r are XOR-swizzled (chunk c at slot c ^ ((r >> 1) & (BKB/16 - 1))) so the
// rows read by consecutive lanes of one MFMA fragment load cover all banks.  128-byte
// slices read whole cache lines and stream from L2 markedly faster than 64-byte ones.
// WGM x WGN waves, each owning a WM x WN sub-tile (WM/16 x WN/16 MFMA tiles).  After the
// K loop every wave stages its own sub-tile in LDS and writes whole rows with 16-byte
// stores.  QKVONLY: an instance for the Q/K/V projection only (bf16 output, QKV
// epilogue), whose epilogue staging is bf16 and therefore smaller.  OCC: blocks per CU
// the instance is built for.
template <int WM_, int WN_, int WGM_, int WGN_, int BKB_, int NS_, int OCC_, bool QKVONLY_>
struct GemmCfg {
  static constexpr int WM = WM_, WN = WN_, WGM = WGM_, WGN = WGN_, BKB = BKB_, NS = NS_;
  static constexpr int OCC = OCC_;
  static constexpr bool QKVONLY = QKVONLY_;
  static constexpr int NW = WGM * WGN, NT = 64 * NW;
  static constexpr int BM = WGM * WM, BN = WGN * WN, TM = WM / 16, TN = WN / 16;
  static constexpr int CPR = BKB / 16, RPI = 64 / CPR;  // chunks per row, rows per load
  static constexpr int KSUB = BKB / 64;                 // 32-wide MFMA k-steps per stage
  static constexpr int STAGE = (BM + BN) * BKB;         // bytes per K slice
  static constexpr int NI = STAGE / 1024;               // 1 KiB load instructions per stage
  static constexpr int LPW = NI / NW;                   // per wave
  // epilogue staging per wave: float32 rows of WN (+4), or bf16 rows of WN (+8); the
  // float32 tile in EPASS passes of WM / EPASS rows when the whole tile of every wave
  // would not fit the LDS
  static constexpr int LDF = WN + 4, LDB = WN + 8;
  static constexpr int EPASS = QKVONLY || NW * WM * LDF * 4 + BM * 4 <= 160 * 1024 ? 1 : 2;
  static constexpr int WAVE_STAGE = QKVONLY ? WM * LDB * 2 : WM / EPASS * LDF * 4;
  // the float32 residual of the generic epilogue is fetched before the K loop only with
  // at most two waves per SIMD (it holds 2 WM WN / 64 registers through the loop)
  static constexpr bool PRE_RES = NW * OCC <= 8;
  static constexpr int SMEM = NS * STAGE > NW * WAVE_STAGE ? NS * STAGE : NW * WAVE_STAGE;
  static_assert(BKB == 64 || BKB == 128, "64- or 128-byte K slices");
  static_assert(NI % NW == 0, "stage must split evenly over the waves");
  static_assert(BM % RPI == 0, "A rows must fill whole load instructions");
  static_assert(NS >= 2 && SMEM <= 160 * 1024, "ring");
  static_assert(TM % EPASS == 0, "epilogue passes of whole m-tiles");
};

DEV int gemm_swz(int bkb, int row, int c) {
  return bkb == 64 ? (c ^ ((row >> 1) & 3)) : (c ^ ((row >> 1) & 7));
}

template <typename OutT, typename CFG>
__global__ __launch_bounds__(CFG::NT, CFG::OCC) void gemm_bf16_kernel(GemmArgs a) {
  using S = CFG;
  constexpr int BM = S::BM, BN = S::BN, TM = S::TM, TN = S::TN, WM = S::WM, WN = S::WN;
  constexpr int BKB = S::BKB, NW = S::NW;
  constexpr bool QKVONLY = S::QKVONLY;
  __shared__ __attribute__((aligned(1024))) char ring[S::SMEM];
  __shared__ int rows_s[BM];

  const int tid = threadIdx.x;
  int g = 0, m_begin, m_end;
  // grouped launches with many n-tiles run them fastest (n_fast): consecutive blocks
  // (spread over the XCDs) share one m-tile's rows, and each XCD sees the same n-tiles of
  // a group's weights for all of that group's m-tiles
  const int mtile = a.n_fast ? blockIdx.y : blockIdx.x;
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
  const int n0 = (a.n_fast ? blockIdx.x : blockIdx.y) * BN;
  // split-K partial launch: block z takes K columns [z K, (z + 1) K) and writes partial
  // product z (float32, [M, ldc]) of a stack of ksplit
  const int64_t kz = a.ksplit > 1 ? (int64_t)blockIdx.z * a.K : 0;
  const bf16* __restrict__ A = (const bf16*)a.A + kz;
  const bf16* __restrict__ B = (const bf16*)a.B + (int64_t)g * a.b_gstride + kz;
  for (int i = tid; i < BM; i += S::NT) {
    const int m = m_begin + i;
    rows_s[i] = (m < m_end) ? (a.rows ? a.rows[m] : m) : -1;
  }
  __syncthreads();

  // load descriptors: wave w issues instructions q = w + NW j of every stage; lane L of
  // instruction q fills row RPI q' + L / CPR, slot L % CPR of its section
  const int lane = tid & 63, w = tid >> 6;
  const bf16* src[S::LPW];
#pragma unroll
  for (int j = 0; j < S::LPW; ++j) {
    const int q = w + NW * j, slot = lane % S::CPR;
    if (q < BM / S::RPI) {
      const int row = q * S::RPI + lane / S::CPR;
      const int o = rows_s[row] >= 0 ? rows_s[row] : rows_s[0];  // pad rows repeat row 0
      src[j] = A + (int64_t)(o / a.row_div) * a.lda + (gemm_swz(BKB, row, slot) << 3);
    } else {
      const int row = (q - BM / S::RPI) * S::RPI + lane / S::CPR;
      const int n = min(n0 + row, a.N - 1);
      src[j] = B + (int64_t)n * a.ldb + (gemm_swz(BKB, row, slot) << 3);
    }
  }
  auto issue = [&](int s) {
    char* sb = ring + (s % S::NS) * S::STAGE;
#pragma unroll
    for (int j = 0; j < S::LPW; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(src[j] + s * (BKB / 2)),
                                       (lds_void*)(sb + (w + NW * j) * 1024), 16, 0, 0);
  };

  const int wm = w / S::WGN, wn = w % S::WGN, lr = lane & 15, lg = lane >> 4;
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
  // register room for the row entries: 4 TM float4 per lane at NW * OCC / 4 waves per SIMD
  constexpr bool PRE_TAB = QKV && TM * (NW * S::OCC / 4) <= 8;
  float4 tq[PRE_TAB ? TM : 1][4];
  float4 td0 = {}, td1 = {};
  int n_tab = 0;  // table loads issued behind the ring's first stages
  auto load_seq_tables = [&](float4 (&t)[PRE_TAB ? TM : 1][4]) {
#pragma unroll
    for (int i = 0; i < (PRE_TAB ? TM : 1); ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) t[i][v] = a.rope_s4[row_pos(i, v) * 16 + lr];
  };
  float rres[QKV || !S::PRE_RES ? 1 : NIT][8];
  if constexpr (QKV || !S::PRE_RES) {
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

  const int nst = a.K / (BKB / 2);
  const uint32_t ring0 = lds_off(ring);
  for (int s = 0; s < S::NS - 1 && s < nst; ++s) issue(s);
  // the depth-rotation entries too are fetched behind the first stages, with at most two
  // waves per SIMD (with more, their registers would be held through the K loop by too
  // many waves), else in the epilogue
  constexpr bool PRE_DTAB = NW * S::OCC <= 8;
  if constexpr (QKV) {
    if (PRE_DTAB && da_qk) {
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
#pragma unroll
    for (int kh = 0; kh < S::KSUB; ++kh) {
      // the swizzle slot depends on the row only through lr, so fragments i (j) of one
      // k-step sit 16 rows apart: one base address per operand, immediate offsets
      const int slot = gemm_swz(BKB, lr, kh * 4 + lg);
      const uint32_t abase = sb + (wm * WM + lr) * BKB + (slot << 4);
      const uint32_t bbase = sb + (BM + wn * WN + lr) * BKB + (slot << 4);
      bf16x8 fr[TM + TN];  // A fragments, then B fragments
      if constexpr (TM == 4 && TN == 4) {
        lds_read_b128_2x4<16 * BKB>(fr, abase, bbase);
      } else {
        uint32_t ad[TM + TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) ad[i] = abase + i * 16 * BKB;
#pragma unroll
        for (int j = 0; j < TN; ++j) ad[TM + j] = bbase + j * 16 * BKB;
        lds_read_b128<TM + TN>(fr, ad);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(fr[i], fr[TM + j], acc[i][j]);
    }
  }
  __syncthreads();  // every wave is done with the ring; it becomes epilogue staging

  char* wst = ring + w * S::WAVE_STAGE;
  OutT* C = (OutT*)a.C + (a.ksplit > 1 ? (int64_t)blockIdx.z * a.M * a.ldc : 0);
  if constexpr (QKV) {
    if (a.qkv_h) {
      if (!PRE_DTAB && da_qk) {
        td0 = a.rope_d4[a.depth_l * 16 + lr];
        td1 = a.rope_d4[(a.depth_L - 1 - a.depth_l) * 16 + lr];
      }
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
              const float xr = rot_first(x, y, cv, sv);
              y = rot_second(y, x, cv, sv);
              x = xr;
            }
            sw[rt * S::LDB + pair] = (bf16)x;
            sw[rt * S::LDB + pair + 32] = (bf16)y;
          }
        }
      }
      wave_lds_sync();
      // rows of 64 bf16 = 8 chunks of 16 bytes (SA v with vt_only: the transposed copy only)
      const bool plain = !(sect == 2 && a.vt && a.vt_only);
      // DA k / v straight into the depth-attention cache's slot when given
      bf16* dst = C + cw0;
      int64_t ldd = a.ldc;
      if ((sect == 4 || sect == 5) && a.da_k) {
        dst = (bf16*)(sect == 4 ? a.da_k : a.da_v) + hcol0;
        ldd = a.da_ld;
      }
      for (int it = plain ? lane : WM * 8; it < WM * 8; it += 64) {
        const int rt = it >> 3, ch = it & 7;
        const int orow = rows_s[rw0 + rt];
        if (orow < 0) continue;
        *reinterpret_cast<bf16x8*>(dst + (int64_t)orow * ldd + ch * 8) =
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
  // generic: v = acc * row_scale + resid; C (OutT) and optional bf16 copy C2.  Pass p
  // stages m-tiles p TM / EPASS .. and writes their rows (item m of the wave's tile is
  // row (lane + 64 m) / CPR, chunk (lane + 64 m) % CPR).
  constexpr int EP = S::EPASS, PTM = TM / EP, PNIT = NIT / EP;
  static_assert(NIT % EP == 0 && PNIT * 64 / CPR == PTM * 16, "a pass holds whole rows");
  float* sf = reinterpret_cast<float*>(wst);  // [WM / EPASS][LDF]
  bf16* C2 = (bf16*)a.C2;
#pragma unroll
  for (int p = 0; p < EP; ++p) {
    // The pass's row scales and residuals are loaded first, every load issued before the
    // first use (item by item, each would wait for its own); a row past the tile or a
    // chunk past N reads row 0 / the last chunk and is not stored.
    float scl[PNIT], rr[S::PRE_RES ? 1 : PNIT][8];
#pragma unroll
    for (int mm = 0; mm < PNIT; ++mm) {
      const int it = lane + 64 * (p * PNIT + mm);
      scl[mm] = 1.0f;
      if (a.row_scale) scl[mm] = a.row_scale[max(rows_s[rw0 + it / CPR], 0)];
    }
    if constexpr (!QKV && !S::PRE_RES) {
      if (a.resid) {
#pragma unroll
        for (int mm = 0; mm < PNIT; ++mm) {
          const int it = lane + 64 * (p * PNIT + mm);
          const int orow = max(rows_s[rw0 + it / CPR], 0);
          const int n = max(0, min(cw0 + (it % CPR) * 8, a.N - 8));
          load16(a.resid + (int64_t)orow * a.ldr + n, rr[mm]);
          load16(a.resid + (int64_t)orow * a.ldr + n + 4, rr[mm] + 4);
        }
      }
    }
    if (p) wave_lds_sync();  // the previous pass's rows are read before they are replaced
#pragma unroll
    for (int i = 0; i < PTM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          sf[(i * 16 + lg * 4 + v) * S::LDF + j * 16 + lr] = acc[p * PTM + i][j][v];
    wave_lds_sync();
    // all of the pass's values first, then all of its stores: with the values of one item
    // at a time the next item waits for the previous item's stores to read their registers
    float val[PNIT][8];
#pragma unroll
    for (int mm = 0; mm < PNIT; ++mm) {
      const int m = p * PNIT + mm;
      const int it = lane + 64 * m, rt = it / CPR, cc = it % CPR;
      const int rs = rt - p * PTM * 16;  // row in the staged pass
      const float sc = scl[mm];
      const floatx4 c0 = *reinterpret_cast<const floatx4*>(sf + rs * S::LDF + cc * 8);
      const floatx4 c1 = *reinterpret_cast<const floatx4*>(sf + rs * S::LDF + cc * 8 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        val[mm][e] = c0[e] * sc;
        val[mm][4 + e] = c1[e] * sc;
      }
      if constexpr (!QKV) {
        if (a.resid) {
          if constexpr (S::PRE_RES) {
#pragma unroll
            for (int e = 0; e < 8; ++e) val[mm][e] += rres[m][e];
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) val[mm][e] += rr[mm][e];
          }
        }
      }
    }
#pragma unroll
    for (int mm = 0; mm < PNIT; ++mm) {
      const int it = lane + 64 * (p * PNIT + mm), rt = it / CPR, cc = it % CPR;
      const int orow = rows_s[rw0 + rt];
      const int n = cw0 + cc * 8;
      if (orow < 0 || n >= a.N) continue;
      OutT* cp = C + (int64_t)orow * a.ldc + n;
      if constexpr (sizeof(OutT) == 2) {
        store16(cp, val[mm]);
      } else {
        store16(cp, val[mm]);
        store16(cp + 4, val[mm] + 4);
      }
      if (C2) store16(C2 + (int64_t)orow * a.ldc2 + n, val[mm]);
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

// Split-K second pass, generic epilogue: out = (sum of the ksplit partials, in order) *
// row_scale + resid; C (float32 or bf16) and optional bf16 copy C2.  One thread per 4
// columns.
template <typename OutT>
__global__ void splitk_reduce_kernel(int M, int N, int ksplit, const float* __restrict__ part,
                                     const float* __restrict__ row_scale,
                                     const float* __restrict__ resid, int64_t ldr,
                                     OutT* __restrict__ C, int64_t ldc, bf16* __restrict__ C2,
                                     int64_t ldc2) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int nq = N / 4;
  if (i >= (int64_t)M * nq) return;
  const int m = (int)(i / nq), n = (int)(i % nq) * 4;
  floatx4 v = *reinterpret_cast<const floatx4*>(part + (int64_t)m * N + n);
  for (int z = 1; z < ksplit; ++z)
    v += *reinterpret_cast<const floatx4*>(part + ((int64_t)z * M + m) * N + n);
  const float sc = row_scale ? row_scale[m] : 1.0f;
  float o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = v[e] * sc + (resid ? resid[(int64_t)m * ldr + n + e] : 0.f);
#pragma unroll
  for (int e = 0; e < 4; ++e) C[(int64_t)m * ldc + n + e] = (OutT)o[e];
  if (C2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) C2[(int64_t)m * ldc2 + n + e] = (bf16)o[e];
  }
}

// Split count for a few-row dense launch with the generic epilogue: the number of
// 64-element K slices per part stays whole, and the grid of 64 x 64 tiles reaches about
// two blocks per CU.  (A 64-row QKV projection, 96 tiles of 64 x 128, was measured no
// faster split.)
static int choose_split(const GemmArgs& a) {
  if (a.qkv_h || a.toff || a.rows || a.row_div != 1 || !a.split_ws || a.M > 64 || a.K % 64)
    return 1;
  const int64_t tiles = (a.N + 63) / 64;
  const int64_t want = 2 * (int64_t)device_cus();
  int sp = 1;
  while (sp < 32 && tiles * sp < want && (a.K / 64) % (2 * sp) == 0 &&
         (int64_t)2 * sp * a.M * a.N <= a.split_elems)
    sp *= 2;
  return sp;
}

int launch_gemm(const GemmArgs& a_in, int dtype, int out_f32, hipStream_t st) {
  GemmArgs a = a_in;
  a.n_fast = a.toff && a.N >= 16 * 128;  // grouped with many n-tiles: n fastest (see the kernel)
  if (a.M <= 0 || a.N <= 0) return 0;
  if (dtype == DT_F32) {
    dim3 grid((a.N + 15) / 16, (a.M + 15) / 16);
    dlaunch(gemm_f32_kernel, grid, 256, 0, st, a);
    return 0;
  }
  if (a.K % 32 != 0 || a.N % 8 != 0) return -1;
  if (dtype == DT_BF16 && a.ksplit == 1) {
    const int sp = choose_split(a);
    if (sp > 1) {  // partial products of K / sp columns each, then the epilogue pass
      GemmArgs p = a;
      p.K = a.K / sp;
      p.ksplit = sp;
      p.C = a.split_ws;
      p.ldc = a.N;
      p.resid = nullptr;
      p.row_scale = nullptr;
      p.C2 = nullptr;
      p.qkv_h = 0;
      dim3 grid((a.M + 63) / 64, (a.N + 63) / 64, sp);
      dlaunch(gemm_bf16_kernel<float, GemmCfg<32, 32, 2, 2, 128, 4, 2, false>>, grid, 256, 0,
              st, p);
      const int64_t n = (int64_t)a.M * (a.N / 4);
      if (out_f32)
        dlaunch(splitk_reduce_kernel<float>, (unsigned)((n + 255) / 256), 256, 0, st, a.M, a.N,
                sp, (const float*)a.split_ws, a.row_scale, a.resid, a.ldr, (float*)a.C, a.ldc,
                (bf16*)a.C2, a.ldc2);
      else
        dlaunch(splitk_reduce_kernel<bf16>, (unsigned)((n + 255) / 256), 256, 0, st, a.M, a.N,
                sp, (const float*)a.split_ws, a.row_scale, a.resid, a.ldr, (bf16*)a.C, a.ldc,
                (bf16*)a.C2, a.ldc2);
      return 0;
    }
  }
  const bool k64 = a.K % 64 == 0;  // 128-byte K slices
  auto tiles = [&](int tm, int tn) {
    return (int64_t)((a.M + tm - 1) / tm) * ((a.N + tn - 1) / tn);
  };
  auto grid_of = [&](int bm, int bn) {
    const int nm = (a.M + bm - 1) / bm + (a.toff ? a.G : 0), nn = (a.N + bn - 1) / bn;
    return a.n_fast ? dim3(nn, nm) : dim3(nm, nn);
  };
  // QKV projections with the rotary epilogue (64-column wave tiles, one head each):
  // launches of at least one 256 x 256 tile per CU take those tiles, 16 waves in one block
  // per CU on a two-stage ring of 128-byte K slices (two k-steps, 32 MFMAs per wave, per
  // barrier: measured 3% faster at the deep shape than four stages of 64-byte slices);
  // else 128 x 128 tiles of 8 waves at two blocks per CU; few rows, and grouped launches whose
  // tile offsets were built for 64-row m-tiles, take 64 x 128 tiles of 4 waves (grouped
  // launches built for 128-row m-tiles take the 128 x 128 tiles).
  if (a.qkv_h) {
    if (a.qkv_h % 128 || out_f32 || !a.rope_d4 || (a.sa_rope && !a.rope_s4)) return -1;
    if (a.toff && a.tile_m != 64 && a.tile_m != 128) return -1;
    if (!a.toff && k64 && tiles(256, 256) >= 256) {
      dlaunch(gemm_bf16_kernel<bf16, GemmCfg<64, 64, 4, 4, 128, 2, 1, true>>, grid_of(256, 256), 1024, 0, st, a);
    } else if (a.toff ? a.tile_m == 64 : tiles(128, 128) < 256) {
      if (k64)
        dlaunch(gemm_bf16_kernel<bf16, GemmCfg<32, 64, 2, 2, 128, 3, 2, false>>, grid_of(64, 128), 256, 0, st, a);
      else
        dlaunch(gemm_bf16_kernel<bf16, GemmCfg<32, 64, 2, 2, 64, 5, 2, false>>, grid_of(64, 128), 256, 0, st, a);
    } else if (k64) {
      dlaunch(gemm_bf16_kernel<bf16, GemmCfg<32, 64, 4, 2, 128, 2, 2, true>>, grid_of(128, 128), 512, 0, st, a);
    } else {
      dlaunch(gemm_bf16_kernel<bf16, GemmCfg<64, 64, 2, 2, 64, 3, 3, true>>, grid_of(128, 128), 256, 0, st, a);
    }
    return 0;
  }
  // Generic: 128 x 128 tiles when that gives >= 512 blocks (two per CU), else 64 x 128,
  // else 64 x 64; grouped launches use m-tiles of their tile_m rows (64, or 128 with
  // 128-column tiles).
  const int bn = a.N >= 128 ? 128 : 64;
  int bm = 64, bnn = bn;
  // float32 output, at least one 256 x 256 tile per CU: those tiles, as the QKV
  // projection (16 waves of 64 x 64, 128-byte slices on two stages; the epilogue in two
  // passes of 32 rows, the residual read there)
  if (out_f32 && !a.toff && k64 && a.N % 256 == 0 && tiles(256, 256) >= 256) {
    dlaunch(gemm_bf16_kernel<float, GemmCfg<64, 64, 4, 4, 128, 2, 1, false>>, grid_of(256, 256), 1024, 0, st, a);
    return 0;
  }
  if (a.toff) {
    if (a.tile_m == 128 && bn == 128) bm = 128;
    else if (a.tile_m != 64) return -1;
  } else if (bn == 128 && tiles(128, 128) >= 512) {
    bm = 128;
  } else if (bn == 128 && tiles(64, 128) < 512) {
    bnn = 64;
  }
#define DREAMER_GEMM_LAUNCH(OUT)                                                               \
  if (bm == 128) {                                                                            \
    if (k64) dlaunch(gemm_bf16_kernel<OUT, GemmCfg<64, 64, 2, 2, 128, 2, 2, false>>, grid_of(128, 128), 256, 0, st, a); \
    else dlaunch(gemm_bf16_kernel<OUT, GemmCfg<64, 64, 2, 2, 64, 4, 2, false>>, grid_of(128, 128), 256, 0, st, a);      \
  } else if (bnn == 128) {                                                                    \
    if (k64) dlaunch(gemm_bf16_kernel<OUT, GemmCfg<32, 64, 2, 2, 128, 3, 2, false>>, grid_of(64, 128), 256, 0, st, a);  \
    else dlaunch(gemm_bf16_kernel<OUT, GemmCfg<32, 64, 2, 2, 64, 5, 2, false>>, grid_of(64, 128), 256, 0, st, a);       \
  } else {                                                                                    \
    if (k64) dlaunch(gemm_bf16_kernel<OUT, GemmCfg<32, 32, 2, 2, 128, 4, 2, false>>, grid_of(64, 64), 256, 0, st, a);   \
    else dlaunch(gemm_bf16_kernel<OUT, GemmCfg<32, 32, 2, 2, 64, 8, 2, false>>, grid_of(64, 64), 256, 0, st, a);        \
  }
  if (out_f32) {
    DREAMER_GEMM_LAUNCH(float)
  } else {
    DREAMER_GEMM_LAUNCH(bf16)
  }
#undef DREAMER_GEMM_LAUNCH
  return 0;
}

}  // namespace dreamer
