// Fused expert FFN for bf16 storage (SwiGLU or GELU) over routed slots.
//
// One block = one 64-row m-tile of one expert's slots; wave w owns tile rows
// [16 w, 16 w + 16).  A single ring of LDS stages, filled by direct global->LDS loads
// (global_load_lds_dwordx4, several stages in flight), streams everything the tile
// reads: first GEMM1's K slices (the gathered token rows and the expert's W1 / W3 rows),
// then GEMM2's slices of W2 rows (output columns), so W2 is already in flight while
// GEMM1 finishes.
//
// GEMM1 runs transposed, H^T = W X^T: the weight rows are the MFMA A operand, so a lane
// ends with hidden units of one token row.  The weight rows are loaded in a permuted
// order (LDS row 16 t + 4 g + i holds hidden unit 32 (t/2) + 8 g + 4 (t%2) + i) that
// makes those hidden units exactly the 8 consecutive ones GEMM2's B fragment needs: the
// activation goes from the accumulators straight into GEMM2's operand registers.
// GEMM2 runs transposed too, O^T = W2 H^T: every lane holds 4 consecutive gate-scaled
// outputs of one slot and stores them as 8 bytes.
//
// Slices are XOR-swizzled by row in 16-byte chunks so that the 16 rows one fragment
// read touches fall into distinct banks.
#include "common.h"
#include "kernels.h"

namespace dreamer {

// Blocks per CU and the ring's LDS budget per block: narrow experts (f <= 64, 128-byte K
// slices, 24 KiB stages) run three blocks per CU on a two-stage ring (measured faster at
// the small workload's ~400 tiles than two blocks on three stages); wider ones two blocks
// on 78 KiB.
#ifndef DREAMER_FFN_NARROW_F
#define DREAMER_FFN_NARROW_F 64
#endif

template <int F, int KIND>
struct FfnCfg {
  static constexpr int NW1 = KIND == FFN_SWIGLU ? 2 : 1;  // GEMM1 weight matrices
  static constexpr bool NARROW = F <= DREAMER_FFN_NARROW_F;
  static constexpr int OCC = NARROW ? 3 : 2;                       // blocks per CU
  static constexpr int LDS = NARROW ? 52 * 1024 : 78 * 1024;       // ring budget per block
  static constexpr int BKB = NARROW ? 128 : 64;           // bytes of a GEMM1 K slice row
  static constexpr int KSUB = BKB / 64;                   // 32-wide k-steps per slice
  static constexpr int CPR = BKB / 16, RPI = 64 / CPR;    // chunks per row, rows per load
  static constexpr int XB = 64 * BKB;                     // token rows of one slice
  static constexpr int WB = F * BKB;                      // one weight's rows of one slice
  static constexpr int STAGE = XB + NW1 * WB;             // bytes per ring stage
  // GEMM2 stage: C2 W2 rows (output columns) of F elements, as many as fit a stage
  static constexpr int RB2 = 2 * F;
  static constexpr int C2 = 128 * RB2 <= STAGE ? 128 : (64 * RB2 <= STAGE ? 64 : 32);
  static constexpr int CPR2 = RB2 / 16, RPI2 = 64 / CPR2;
  static constexpr int NI1 = STAGE / 1024, LPW1 = NI1 / 4;  // load instructions
  static constexpr int NI2 = C2 * RB2 / 1024, LPW2 = NI2 / 4;
  static constexpr int NT1 = F / 16;            // GEMM1 m-tiles (16 hidden units) per weight
  static constexpr int KS2 = F / 32;            // GEMM2 k-steps
  static constexpr int NT2 = C2 / 16;           // GEMM2 output-column tiles per stage
  // ring depth: what the LDS budget holds, at most 8, and few enough stages that the
  // operations outstanding behind a stage (the loads of NS - 2 stages, the output stores
  // of NS - 1 iterations) stay within the vmcnt counter's range
  static constexpr int LPWM = LPW1 > LPW2 ? LPW1 : LPW2;
  static constexpr int fit_ns(int ns) {
    return ns <= 2 || (ns - 2) * LPWM + (ns - 1) * NT2 <= 63 ? ns : fit_ns(ns - 1);
  }
  static constexpr int NS0 = LDS / STAGE;
  static constexpr int NS = fit_ns(NS0 > 8 ? 8 : NS0);
  static_assert(NI1 % 4 == 0 && NI2 % 4 == 0, "stages must split evenly over 4 waves");
  static_assert(NS >= 2, "LDS ring too small");
};

// slot of 16-byte chunk c in a ring row of rb bytes
DEV int ffn_swz(int rb, int row, int c) {
  return rb == 64 ? (c ^ ((row >> 1) & 3)) : rb == 128 ? (c ^ ((row >> 1) & 7)) : (c ^ (row & 15));
}

template <int F, int KIND>
__global__ __launch_bounds__(256, (FfnCfg<F, KIND>::OCC)) void expert_ffn_kernel(
    int k, int h_in, int h_out, const bf16* __restrict__ x, const bf16* __restrict__ w1,
    const bf16* __restrict__ w3, const bf16* __restrict__ w2, const int32_t* __restrict__ perm,
    const float* __restrict__ pgate, const int4* __restrict__ tiles, int tile_cap,
    const int32_t* __restrict__ ntiles, bf16* __restrict__ slots) {
  using S = FfnCfg<F, KIND>;
  constexpr int BKB = S::BKB, RB2 = S::RB2;
  __shared__ __attribute__((aligned(1024))) char stg[S::NS * S::STAGE];
  __shared__ int s_slot[64];

  // Blocks reach the 8 XCDs round-robin; block b takes tile (b % 8) * per + b / 8, so each
  // XCD works through one contiguous range of tiles, where consecutive tiles mostly share
  // an expert whose weights then stay in that XCD's L2.  The tile count, the descriptor
  // and the tile's slot ids and gates (tile-padded by the permutation) come in one round
  // trip; indices are clamped into the arrays and the values used only for a real tile.
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int n_tiles = *ntiles;
  const int b = blockIdx.x, per = (n_tiles + 7) / 8;
  const int tile = (b & 7) * per + (b >> 3);
  const int tc = min(tile, tile_cap - 1);
  const int4 td = tiles[tc];
  const int pslot = perm[tc * 64 + (tid & 63)];          // row tid (first wave)
  const int oslot = perm[tc * 64 + w * 16 + lr];         // this lane's output row
  float gate = pgate[tc * 64 + w * 16 + lr];
  if ((b >> 3) >= per || tile >= n_tiles) return;
  const int e = td.x, nrows = min(64, td.z - td.y);
  const int sl = w * 16 + lr < nrows ? oslot : -1;
  if (tid < 64) s_slot[tid] = tid < nrows ? pslot : -1;
  // the gate is taken through an empty asm statement: the compiler waits for it here,
  // before the ring starts, instead of draining the ring at its first use
  asm volatile("" : "+v"(gate));
  __syncthreads();

  // load descriptors: wave w issues instructions q = w + 4 j of every stage
  const bf16* src1[S::LPW1];  // GEMM1: token rows, then W1 (and W3) rows, permuted
#pragma unroll
  for (int j = 0; j < S::LPW1; ++j) {
    const int q = w + 4 * j, slot = lane % S::CPR;
    const int row = q * S::RPI + lane / S::CPR;  // row of the stage
    if (row < 64) {
      const int s = s_slot[row] >= 0 ? s_slot[row] : s_slot[0];  // pad rows repeat row 0
      src1[j] = x + (int64_t)(s / k) * h_in + ffn_swz(BKB, row, slot) * 8;
    } else {
      const int wr = (row - 64) % F, m = (row - 64) / F;
      const int t = wr >> 4, g = (wr >> 2) & 3, i = wr & 3;
      const int hu = 32 * (t >> 1) + 8 * g + 4 * (t & 1) + i;  // hidden unit of LDS row wr
      const bf16* W = m == 0 ? w1 : w3;
      src1[j] = W + ((int64_t)e * F + hu) * h_in + ffn_swz(BKB, wr, slot) * 8;
    }
  }
  const bf16* src2[S::LPW2];  // GEMM2: W2 rows (output columns) of the first chunk
#pragma unroll
  for (int j = 0; j < S::LPW2; ++j) {
    const int q = w + 4 * j, slot = lane % S::CPR2;
    const int row = q * S::RPI2 + lane / S::CPR2;
    src2[j] = w2 + ((int64_t)e * h_out + row) * F + ffn_swz(RB2, row, slot) * 8;
  }
  const int n1 = h_in * 2 / BKB, n2 = h_out / S::C2, ntot = n1 + n2;
  auto issue = [&](int s) {
    char* sb = stg + (s % S::NS) * S::STAGE;
    if (s < n1) {
#pragma unroll
      for (int j = 0; j < S::LPW1; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(src1[j] + s * (BKB / 2)),
                                         (lds_void*)(sb + (w + 4 * j) * 1024), 16, 0, 0);
    } else {
      const int64_t o = (int64_t)(s - n1) * S::C2 * F;
#pragma unroll
      for (int j = 0; j < S::LPW2; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(src2[j] + o),
                                         (lds_void*)(sb + (w + 4 * j) * 1024), 16, 0, 0);
    }
  };

  floatx4 ag[S::NT1], au[S::NT1];
#pragma unroll
  for (int t = 0; t < S::NT1; ++t) {
    ag[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    au[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 hf[S::KS2];  // GEMM2 B operand: this lane's row, hidden units 32 s + 8 lg + j
  const uint32_t stg0 = lds_off(stg);
  // Stage s has landed once at most the operations issued after its loads are
  // outstanding: the loads of stages s+1 .. s+NS-2 and the output stores of the GEMM2
  // iterations from the one that issued stage s on (NT2 counted store instructions per
  // iteration, in waves that own a slot row).
  const int nst_w = w * 16 < nrows ? S::NT2 : 0;
  for (int s = 0; s < S::NS - 1 && s < ntot; ++s) issue(s);
  for (int s = 0; s < ntot; ++s) {
    int later = 0;
    for (int t = s + 1; t < s + S::NS - 1 && t < ntot; ++t) later += t < n1 ? S::LPW1 : S::LPW2;
    later += nst_w * max(0, s - max(n1, s - S::NS + 1));
    wait_vmcnt_upto(later);
    ring_barrier();  // stage s visible to all waves; stage s-1 fully consumed
    if (s + S::NS - 1 < ntot) issue(s + S::NS - 1);
    const uint32_t sb = stg0 + (s % S::NS) * S::STAGE;
    if (s < n1) {
      // every fragment of the stage in one read group (one LDS round trip per stage):
      // per k-step the X fragment, then NT1 fragments of each weight
      constexpr int PER = 1 + S::NW1 * S::NT1, NR = S::KSUB * PER;
      bf16x8 fr[NR];
      uint32_t ad[NR];
#pragma unroll
      for (int kh = 0; kh < S::KSUB; ++kh) {
        // fragments 16 rows apart share the swizzle slot (it depends on lr only)
        const int slot = ffn_swz(BKB, lr, kh * 4 + lg);
        const uint32_t wa = sb + S::XB + lr * BKB + (slot << 4);
        ad[kh * PER] = sb + (w * 16 + lr) * BKB + (slot << 4);
#pragma unroll
        for (int m = 0; m < S::NW1; ++m)
#pragma unroll
          for (int t = 0; t < S::NT1; ++t)
            ad[kh * PER + 1 + m * S::NT1 + t] = wa + m * S::WB + t * 16 * BKB;
      }
      lds_read_b128<NR>(fr, ad);
#pragma unroll
      for (int kh = 0; kh < S::KSUB; ++kh)
#pragma unroll
        for (int t = 0; t < S::NT1; ++t) {
          ag[t] = mfma16(fr[kh * PER + 1 + t], fr[kh * PER], ag[t]);
          if constexpr (KIND == FFN_SWIGLU)
            au[t] = mfma16(fr[kh * PER + 1 + S::NT1 + t], fr[kh * PER], au[t]);
        }
      continue;
    }
    if (s == n1) {
      // activation: accumulator tile t, element i is hidden unit 32 (t/2) + 8 lg +
      // 4 (t%2) + i of row w*16 + lr, i.e. element 4 (t%2) + i of GEMM2 k-step t/2
#pragma unroll
      for (int t = 0; t < S::NT1; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = ag[t][i];
          const float hv = KIND == FFN_SWIGLU ? silu_(g) * au[t][i] : gelu_erf(g);
          hf[t >> 1][4 * (t & 1) + i] = (bf16)hv;
        }
    }
    // GEMM2 stage: output columns nc .. nc + C2 of this wave's 16 rows
    const int nc = (s - n1) * S::C2;
    floatx4 acc[S::NT2];
#pragma unroll
    for (int nt = 0; nt < S::NT2; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    {
      constexpr int NR = S::KS2 * S::NT2;  // all W2 fragments of the stage in one group
      bf16x8 fw[NR];
      uint32_t ad[NR];
#pragma unroll
      for (int ks = 0; ks < S::KS2; ++ks) {
        const int slot = ffn_swz(RB2, lr, ks * 4 + lg);
        const uint32_t base = sb + lr * RB2 + (slot << 4);
#pragma unroll
        for (int nt = 0; nt < S::NT2; ++nt) ad[ks * S::NT2 + nt] = base + nt * 16 * RB2;
      }
      lds_read_b128<NR>(fw, ad);
#pragma unroll
      for (int ks = 0; ks < S::KS2; ++ks)
#pragma unroll
        for (int nt = 0; nt < S::NT2; ++nt)
          acc[nt] = mfma16(fw[ks * S::NT2 + nt], hf[ks], acc[nt]);
    }
    if (nst_w) {  // wave-uniform; row 16 w is a slot row, so some lanes store
      if (sl >= 0) {
        bf16* orow = slots + (int64_t)sl * h_out + nc + lg * 4;
#pragma unroll
        for (int nt = 0; nt < S::NT2; ++nt) {
          bf16x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (bf16)(acc[nt][i] * gate);
          store_b64_counted(orow + nt * 16, v);
        }
      }
    }
  }
}

int launch_expert_ffn(int dtype, int kind, int64_t nslots, int k, int h_in, int f, int h_out,
                      int E, const void* x, const void* w1, const void* w3, const void* w2,
                      const int32_t* perm, const float* pgate, const int4* tiles,
                      const int32_t* toff, void* slots, hipStream_t st) {
  if (nslots <= 0) return 0;
  if (dtype == DT_F32) return -1;  // the f32 path uses launch_expert_ffn_f32
  if (h_in % 64 || h_out % 128) return -1;
  // every tile index below the bound has a block (a multiple of the 8 XCDs)
  const int64_t cap = tile_bound(nslots, E, FFN_TILE_M);
  const unsigned grid = (unsigned)((cap + 7) / 8 * 8);
#define EF_CASE(FF, KK)                                                                     \
  dlaunch(expert_ffn_kernel<FF, KK>, grid, 256, 0, st, k, h_in, h_out, (const bf16*)x,           \
                                                  (const bf16*)w1, (const bf16*)w3,         \
                                                  (const bf16*)w2, perm, pgate, tiles,      \
                                                  (int)cap, toff + E, (bf16*)slots)
  if (kind == FFN_SWIGLU && f == 64) EF_CASE(64, FFN_SWIGLU);
  else if (kind == FFN_SWIGLU && f == 128) EF_CASE(128, FFN_SWIGLU);
  else if (kind == FFN_GELU && f == 64) EF_CASE(64, FFN_GELU);
  else if (kind == FFN_GELU && f == 128) EF_CASE(128, FFN_GELU);
  else return -1;
#undef EF_CASE
  return 0;
}

}  // namespace dreamer
