// Fused expert FFN for bf16 storage (SwiGLU or GELU) over routed slots.
//
// One block = one 64-row m-tile of one expert's slots, four waves.  A single ring of LDS
// stages, filled by direct global->LDS loads (global_load_lds_dwordx4, several stages in
// flight), streams everything the tile reads: first GEMM1's K slices (the gathered token
// rows and the expert's W1 / W3 rows), then GEMM2's slices of W2 rows (output columns),
// so W2 is already in flight while GEMM1 finishes.
//
// The waves split the weights, not the token rows, so that every weight fragment is read
// from LDS by one wave only: in GEMM1, H^T = W X^T, wave w owns F/4 hidden units (the
// weight rows are the MFMA A operand) for all 64 token rows; the activation goes through
// LDS once (64 x F bf16, in the ring stage GEMM1 has just finished with) and every wave
// keeps all of it in registers as GEMM2's B operand.  In GEMM2, O^T = W2 H^T, wave w owns
// a quarter of each stage's output columns for all token rows; every lane holds 4
// consecutive gate-scaled outputs of one slot per column tile, and with two column tiles
// per wave, neighbouring lanes trade one tile each so that every lane stores 8
// consecutive outputs as 16 bytes.
//
// Slices are XOR-swizzled by row in 16-byte chunks so that the 16 rows one fragment
// read touches fall into distinct banks.
#include "common.h"
#include "kernels.h"

namespace dreamer {

// Blocks per CU and the ring's LDS budget per block: narrow experts (f <= 64, 128-byte K
// slices, 24 KiB stages) run three blocks per CU on a two-stage ring (measured faster over
// ~400 tiles than two blocks on three stages, and than 64-byte slices on four stages); wider ones two blocks on 80 KiB, two stages of 128-byte slices
// (whole cache lines: half the L2 requests of 64-byte slices for the same bytes).
#ifndef DREAMER_FFN_NARROW_F
#define DREAMER_FFN_NARROW_F 64
#endif

template <int F, int KIND>
struct FfnCfg {
  static constexpr int NW1 = KIND == FFN_SWIGLU ? 2 : 1;  // GEMM1 weight matrices
  static constexpr bool NARROW = F <= DREAMER_FFN_NARROW_F;
  static constexpr int OCC = NARROW ? 3 : 2;                       // blocks per CU
  static constexpr int LDS = NARROW ? 52 * 1024 : 80 * 1024;       // ring budget per block
  static constexpr int BKB = 128;                         // bytes of a GEMM1 K slice row
  static constexpr int KSUB = BKB / 64;                   // 32-wide k-steps per slice
  static constexpr int CPR = BKB / 16, RPI = 64 / CPR;    // chunks per row, rows per load
  static constexpr int XB = 64 * BKB;                     // token rows of one slice
  static constexpr int WB = F * BKB;                      // one weight's rows of one slice
  static constexpr int STAGE1 = XB + NW1 * WB;            // bytes GEMM1 loads per stage
  // GEMM2 stage: C2 W2 rows (output columns) of F elements, 16 or 32 per wave
  static constexpr int RB2 = 2 * F;
  static constexpr int C2 = 128 * RB2 <= STAGE1 ? 128 : 64;
  static constexpr int CT = C2 / 64;                      // column tiles per wave and stage
  // the activation exchange: 64 token rows of F bf16, rows padded by 16 bytes
  static constexpr int HS = 2 * F + 16;
  static constexpr int HB = (64 * HS + 1023) / 1024 * 1024;
  static constexpr int STAGE = STAGE1 > C2 * RB2 ? (STAGE1 > HB ? STAGE1 : HB)
                                                 : (C2 * RB2 > HB ? C2 * RB2 : HB);
  static constexpr int CPR2 = RB2 / 16, RPI2 = 64 / CPR2;
  static constexpr int NI1 = STAGE1 / 1024, LPW1 = NI1 / 4;  // load instructions
  static constexpr int NI2 = C2 * RB2 / 1024, LPW2 = NI2 / 4;
  static constexpr int HT = F / 64;             // GEMM1 hidden tiles per wave and weight
  static constexpr int KS2 = F / 32;            // GEMM2 k-steps
  static constexpr int NT2 = 4 * CT;            // GEMM2 stores per wave and stage (at most)
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
  static_assert(STAGE1 % 1024 == 0 && STAGE % 1024 == 0, "stages are whole load rows");
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
  // the tile's slot ids: the rows this lane gathers (GEMM1 instructions j < XROWS of the
  // token section), then its output rows 16 tt + lr; pad rows (past nrows) are resolved
  // below
  constexpr int XROWS = (64 / S::RPI + 3) / 4;  // token-row instructions per wave (at most)
  int xs[XROWS], sl[4];
#pragma unroll
  for (int j = 0; j < XROWS; ++j) xs[j] = perm[tc * 64 + min(63, (w + 4 * j) * S::RPI + lane / S::CPR)];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) sl[tt] = perm[tc * 64 + tt * 16 + lr];
  int slot0 = perm[tc * 64];
  float gate[4];  // gates of this lane's output rows 16 tt + lr
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) gate[tt] = pgate[tc * 64 + tt * 16 + lr];
  if ((b >> 3) >= per || tile >= n_tiles) return;
  const int e = td.x, nrows = min(64, td.z - td.y);
  // the slot ids and gates are taken through empty asm statements: the compiler waits for
  // them here, before the ring starts, instead of draining the ring at their first use
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    asm volatile("" : "+v"(gate[tt]), "+v"(sl[tt]));
    if (tt * 16 + lr >= nrows) sl[tt] = -1;  // pad row
  }
#pragma unroll
  for (int j = 0; j < XROWS; ++j) asm volatile("" : "+v"(xs[j]));
  asm volatile("" : "+v"(slot0));

  // load descriptors: wave w issues instructions q = w + 4 j of every stage
  const bf16* src1[S::LPW1];  // GEMM1: token rows, then W1 (and W3) rows
#pragma unroll
  for (int j = 0; j < S::LPW1; ++j) {
    const int q = w + 4 * j, slot = lane % S::CPR;
    const int row = q * S::RPI + lane / S::CPR;  // row of the stage
    if (row < 64) {
      // (row < 64 only for j < XROWS; pad rows repeat row 0)
      const int s = row < nrows ? xs[j < XROWS ? j : 0] : slot0;
      src1[j] = x + (int64_t)(s / k) * h_in + ffn_swz(BKB, row, slot) * 8;
    } else {
      const int hu = (row - 64) % F, m = (row - 64) / F;  // hidden unit, weight
      const bf16* W = m == 0 ? w1 : w3;
      src1[j] = W + ((int64_t)e * F + hu) * h_in + ffn_swz(BKB, hu, slot) * 8;
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

  // Stage s has landed once at most the operations issued after its loads are
  // outstanding: the loads of stages s+1 .. s+NS-2 and the output stores of the GEMM2
  // iterations from the one that issued stage s on (per iteration one store instruction
  // per token tile that holds a slot row, or CT of them with one column tile per wave;
  // the same count in every wave).
  const int nst_w = (S::CT == 2 ? 1 : S::CT) * ((nrows + 15) / 16);
  auto wait_stage = [&](int s) {
    int later = 0;
    for (int t = s + 1; t < s + S::NS - 1 && t < ntot; ++t) later += t < n1 ? S::LPW1 : S::LPW2;
    later += nst_w * max(0, s - max(n1, s - S::NS + 1));
    wait_vmcnt_upto(later);
    ring_barrier();  // stage s visible to all waves; stage s-1 fully consumed
  };
  const uint32_t stg0 = lds_off(stg);
  for (int s = 0; s < S::NS - 1 && s < ntot; ++s) issue(s);

  // GEMM1 accumulators: hidden tile w * HT + j of weight 1 (ag) and 3 (au), token tile tt
  floatx4 ag[S::HT][4], au[S::HT][4];
#pragma unroll
  for (int j = 0; j < S::HT; ++j)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      ag[j][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
      au[j][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  for (int s = 0; s < n1; ++s) {
    wait_stage(s);
    if (s + S::NS - 1 < ntot) issue(s + S::NS - 1);
    const uint32_t sb = stg0 + (s % S::NS) * S::STAGE;
    // every fragment of the stage in one read group (one LDS round trip per stage):
    // per k-step the 4 token-row fragments, then HT fragments of each weight
    constexpr int PER = 4 + S::NW1 * S::HT, NR = S::KSUB * PER;
    bf16x8 fr[NR];
    uint32_t ad[NR];
#pragma unroll
    for (int kh = 0; kh < S::KSUB; ++kh) {
      // fragments 16 rows apart share the swizzle slot (it depends on lr only)
      const int slot = ffn_swz(BKB, lr, kh * 4 + lg);
      const uint32_t xa = sb + lr * BKB + (slot << 4);
      const uint32_t wa = sb + S::XB + (w * S::HT * 16 + lr) * BKB + (slot << 4);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) ad[kh * PER + tt] = xa + tt * 16 * BKB;
#pragma unroll
      for (int m = 0; m < S::NW1; ++m)
#pragma unroll
        for (int j = 0; j < S::HT; ++j)
          ad[kh * PER + 4 + m * S::HT + j] = wa + m * S::WB + j * 16 * BKB;
    }
    lds_read_b128<NR>(fr, ad);
#pragma unroll
    for (int kh = 0; kh < S::KSUB; ++kh)
#pragma unroll
      for (int j = 0; j < S::HT; ++j)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          ag[j][tt] = mfma16(fr[kh * PER + 4 + j], fr[kh * PER + tt], ag[j][tt]);
          if constexpr (KIND == FFN_SWIGLU)
            au[j][tt] = mfma16(fr[kh * PER + 4 + S::HT + j], fr[kh * PER + tt], au[j][tt]);
        }
  }

  // Activation through LDS, in the stage GEMM1 finished last (slot (n1 - 1) % NS, whose
  // next load, stage n1 + NS - 1, is issued by the first GEMM2 iteration, after a barrier
  // that follows every wave's read of the activation): accumulator element i of (j, tt)
  // is hidden unit 16 (w HT + j) + 4 lg + i of row 16 tt + lr; four consecutive units are
  // written as 8 bytes.
  bf16x8 hf[4][S::KS2];  // GEMM2 B operand: row 16 tt + lr, hidden units 32 ks + 8 lg + i
  {
    const int hs = (n1 + S::NS - 1) % S::NS;
    const uint32_t hb = stg0 + hs * S::STAGE;
    ring_barrier();  // every wave is done with GEMM1's last stage
#pragma unroll
    for (int j = 0; j < S::HT; ++j)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        bf16x4 hv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = ag[j][tt][i];
          hv[i] = (bf16)(KIND == FFN_SWIGLU ? silu_(g) * au[j][tt][i] : gelu_erf(g));
        }
        lds_write_b64(hb + (tt * 16 + lr) * S::HS + ((w * S::HT + j) * 16 + lg * 4) * 2, hv);
      }
    ring_barrier();  // the whole activation written
    constexpr int NR = 4 * S::KS2;
    uint32_t ad[NR];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int ks = 0; ks < S::KS2; ++ks)
        ad[tt * S::KS2 + ks] = hb + (tt * 16 + lr) * S::HS + (ks * 32 + lg * 8) * 2;
    lds_read_b128<NR>(reinterpret_cast<bf16x8(&)[NR]>(hf), ad);
  }

  for (int s = n1; s < ntot; ++s) {
    wait_stage(s);  // at s = n1 also: every wave holds the activation
    if (s + S::NS - 1 < ntot) issue(s + S::NS - 1);
    const uint32_t sb = stg0 + (s % S::NS) * S::STAGE;
    // GEMM2 stage: output columns nc + 16 (w CT + c) .. + 16 of all token rows
    const int nc = (s - n1) * S::C2;
    floatx4 acc[S::CT][4];
#pragma unroll
    for (int c = 0; c < S::CT; ++c)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc[c][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
    {
      constexpr int NR = S::KS2 * S::CT;  // this wave's W2 fragments of the stage
      bf16x8 fw[NR];
      uint32_t ad[NR];
#pragma unroll
      for (int ks = 0; ks < S::KS2; ++ks) {
        const int slot = ffn_swz(RB2, lr, ks * 4 + lg);
        const uint32_t base = sb + (w * S::CT * 16 + lr) * RB2 + (slot << 4);
#pragma unroll
        for (int c = 0; c < S::CT; ++c) ad[ks * S::CT + c] = base + c * 16 * RB2;
      }
      lds_read_b128<NR>(fw, ad);
#pragma unroll
      for (int ks = 0; ks < S::KS2; ++ks)
#pragma unroll
        for (int c = 0; c < S::CT; ++c)
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
            acc[c][tt] = mfma16(fw[ks * S::CT + c], hf[tt][ks], acc[c][tt]);
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      if (tt * 16 < nrows) {  // uniform; row 16 tt is a slot row, so some lanes store
        if constexpr (S::CT == 2) {
          // Lane (lr, lg) holds columns 4 lg .. 4 lg + 3 of both column tiles (c = 0: the
          // wave's columns 0..15, c = 1: 16..31).  Lanes lg and lg ^ 1 swap one tile each,
          // so that an even lg holds columns 4 lg .. 4 lg + 7 and an odd lg columns
          // 16 + 4 (lg - 1) .. + 7: every lane stores 16 bytes and the four lanes of a row
          // write its 64 bytes with one instruction (8-byte stores split them in two).
          bf16x4 v0, v1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v0[i] = (bf16)(acc[0][tt][i] * gate[tt]);
            v1[i] = (bf16)(acc[1][tt][i] * gate[tt]);
          }
          const bool even = (lg & 1) == 0;
          const uint2 snd = __builtin_bit_cast(uint2, even ? v1 : v0);
          uint2 rcv;
          rcv.x = (uint32_t)__shfl_xor((int)snd.x, 16, 64);
          rcv.y = (uint32_t)__shfl_xor((int)snd.y, 16, 64);
          const bf16x4 vr = __builtin_bit_cast(bf16x4, rcv);
          const bf16x4 lo = even ? v0 : vr, hi = even ? vr : v1;
          const bf16x8 v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          if (sl[tt] >= 0)
            store_b128_counted(slots + (int64_t)sl[tt] * h_out + nc + w * 32 +
                                   (even ? lg * 4 : 16 + (lg - 1) * 4), v8);
        } else if (sl[tt] >= 0) {
          bf16* orow = slots + (int64_t)sl[tt] * h_out + nc + w * S::CT * 16 + lg * 4;
#pragma unroll
          for (int c = 0; c < S::CT; ++c) {
            bf16x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (bf16)(acc[c][tt][i] * gate[tt]);
            store_b64_counted(orow + c * 16, v);
          }
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
