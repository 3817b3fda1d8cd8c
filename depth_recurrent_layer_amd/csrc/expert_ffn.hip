// Fused expert FFN for bf16 storage (SwiGLU or GELU) over routed slots.
//
// One block = one 64-row tile of one expert's slots (tiles listed by toff).  GEMM1
// (x W1^T and, for SwiGLU, x W3^T) streams 32-wide K slices of the gathered token rows and
// of the expert's weight rows through a multi-stage LDS ring filled by direct
// global->LDS loads (global_load_lds_dwordx4: no staging registers, several slices in
// flight per wave).  Slices are stored as 64-byte rows whose 16-byte chunks are
// XOR-swizzled by row (swz64), so the rows one MFMA fragment read touches fall into
// distinct banks.  Wave w owns hidden columns
// [w F/4, (w+1) F/4) of both projections, so the activation is lane-local.  The hidden
// tile goes to LDS (bf16); GEMM2 runs transposed (W2 H^T) over 64-column chunks so every
// lane holds 4 consecutive gate-scaled outputs of one slot and stores them directly.
#include "common.h"
#include "kernels.h"

namespace dreamer {

template <int F, int KIND>
struct FfnShape {
  static constexpr int NW1 = KIND == FFN_SWIGLU ? 2 : 1;  // GEMM1 weight matrices
  static constexpr int XB = 64 * 64;                       // X slice: 64 rows x 32 bf16
  static constexpr int WB = F * 64;                        // one weight slice
  static constexpr int STAGE = XB + NW1 * WB;
  static constexpr int NI = STAGE / 1024;                  // 1 KiB load instructions
  static constexpr int LPW = NI / 4;                       // per wave per stage
  static constexpr int LDH = F + 8;
  static constexpr int HS_BYTES = 64 * LDH * 2;
  static constexpr int NS0 = (78 * 1024 - HS_BYTES) / STAGE;
  static constexpr int NS = NS0 > 8 ? 8 : NS0;             // ring depth (2 blocks / CU)
  static_assert(NI % 4 == 0, "stage must split evenly over 4 waves");
  static_assert(NS >= 2, "LDS ring too small");
};

template <int F, int KIND>
__global__ __launch_bounds__(256, 2) void expert_ffn_kernel(
    int k, int h_in, int h_out, int E, const bf16* __restrict__ x,
    const bf16* __restrict__ w1, const bf16* __restrict__ w3, const bf16* __restrict__ w2,
    const int32_t* __restrict__ perm, const float* __restrict__ pgate,
    const int4* __restrict__ tiles, int tile_cap, const int32_t* __restrict__ ntiles,
    bf16* __restrict__ slots) {
  using S = FfnShape<F, KIND>;
  constexpr int NT1 = F / 64;  // 16-col tiles per wave per projection
  constexpr int KS2 = F / 32;  // k-steps of GEMM2
  __shared__ __attribute__((aligned(1024))) char stg[S::NS * S::STAGE];
  __shared__ __attribute__((aligned(16))) bf16 Hs[64 * S::LDH];
  __shared__ int s_slot[64];
  __shared__ float s_gate[64];

  // Blocks reach the 8 XCDs round-robin; block b takes tile (b % 8) * per + b / 8, so each
  // XCD works through one contiguous range of tiles, where consecutive tiles mostly share
  // an expert whose weights then stay in that XCD's L2.  The tile count and a descriptor
  // (clamped into the array, used only for a real tile) come in one round trip, then the
  // slot ids and gates (stored in expert-major order by the permutation) in another.
  const int n_tiles = *ntiles;
  const int b = blockIdx.x, per = (n_tiles + 7) / 8;
  const int tile = (b & 7) * per + (b >> 3);
  const int4 td = tiles[min(tile, tile_cap - 1)];
  if ((b >> 3) >= per || tile >= n_tiles) return;
  const int e = td.x, r0 = td.y, r1 = td.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  if (tid < 64) {
    const int m = r0 + tid;
    const bool in = m < r1;
    s_slot[tid] = in ? perm[m] : -1;
    s_gate[tid] = in ? pgate[m] : 0.f;
  }
  // GEMM2's first W2 fragments depend on the expert only: fetched now, used after GEMM1
  constexpr bool PREFETCH = KS2 <= 2;  // register room for two chunks' fragments
  const bf16* W2 = w2 + (int64_t)e * h_out * F;
  auto load_w2 = [&](int nc, bf16x8 (&fr)[4][KS2]) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int ks = 0; ks < KS2; ++ks)
        fr[nt][ks] = *reinterpret_cast<const bf16x8*>(
            W2 + (int64_t)(nc + nt * 16 + lr) * F + ks * 32 + lg * 8);
  };
  bf16x8 wf[4][KS2];
  if (PREFETCH && w * 64 < h_out) load_w2(w * 64, wf);
  // the W2 fragments are taken through an empty asm statement: the compiler waits for
  // them here, before the ring starts, instead of draining the ring at their first use
  if constexpr (PREFETCH) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int ks = 0; ks < KS2; ++ks) asm volatile("" : "+v"(wf[nt][ks]));
  }
  __syncthreads();

  // load descriptors: wave w issues instructions q = w + 4 j of every stage
  const bf16* src[S::LPW];
#pragma unroll
  for (int j = 0; j < S::LPW; ++j) {
    const int q = w + 4 * j;
    const int slot = lane & 3;
    if (q < 4) {  // gathered token rows
      const int row = q * 16 + (lane >> 2);
      const int s = s_slot[row] >= 0 ? s_slot[row] : s_slot[0];
      src[j] = x + (int64_t)(s / k) * h_in + swz64_slot(row, slot) * 8;
    } else {      // expert weight rows
      const int wq = q - 4, m = wq / (F / 16);
      const int mr = (wq % (F / 16)) * 16 + (lane >> 2);
      const bf16* W = m == 0 ? w1 : w3;
      src[j] = W + ((int64_t)e * F + mr) * h_in + swz64_slot(mr, slot) * 8;
    }
  }
  auto issue = [&](int s) {
    char* sb = stg + (s % S::NS) * S::STAGE;
#pragma unroll
    for (int j = 0; j < S::LPW; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(src[j] + s * 32),
                                       (lds_void*)(sb + (w + 4 * j) * 1024), 16, 0, 0);
  };

  floatx4 ag[4][NT1], au[4][NT1];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT1; ++nt) {
      ag[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
      au[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  const int nst = h_in / 32;
  const uint32_t stg0 = lds_off(stg);
  // fragments read per stage: 4 of X, then NT1 of W1 (and NT1 of W3); a GELU tile of
  // F = 64 reads its single weight fragment twice to make an even count
  constexpr int NB = NT1 * S::NW1, NR = 4 + (NB == 1 ? 2 : NB);
  for (int s = 0; s < S::NS - 1 && s < nst; ++s) issue(s);
  for (int s = 0; s < nst; ++s) {
    wait_vmcnt_upto(S::LPW * min(S::NS - 2, nst - 1 - s));
    ring_barrier();  // stage s visible to all waves; stage s-1 fully consumed
    if (s + S::NS - 1 < nst) issue(s + S::NS - 1);
    const uint32_t sb = stg0 + (s % S::NS) * S::STAGE;
    uint32_t ad[NR];
    bf16x8 fr[NR];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) ad[mt] = sb + swz64(mt * 16 + lr, lg);
#pragma unroll
    for (int nt = 0; nt < NT1; ++nt) {
      const int col = w * (F / 4) + nt * 16 + lr;
      ad[4 + nt] = sb + S::XB + swz64(col, lg);
      if constexpr (S::NW1 == 2) ad[4 + NT1 + nt] = sb + S::XB + S::WB + swz64(col, lg);
    }
    if constexpr (NB == 1) ad[5] = ad[4];
    lds_read_b128<NR>(fr, ad);
#pragma unroll
    for (int nt = 0; nt < NT1; ++nt) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) ag[mt][nt] = mfma16(fr[mt], fr[4 + nt], ag[mt][nt]);
      if constexpr (KIND == FFN_SWIGLU) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          au[mt][nt] = mfma16(fr[mt], fr[4 + NT1 + nt], au[mt][nt]);
      }
    }
  }
  // activation -> LDS (row mt*16 + 4lg + i, col w*F/4 + nt*16 + lr)
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT1; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g = ag[mt][nt][i];
        const float hv = KIND == FFN_SWIGLU ? silu_(g) * au[mt][nt][i] : gelu_erf(g);
        Hs[(mt * 16 + lg * 4 + i) * S::LDH + w * (F / 4) + nt * 16 + lr] = (bf16)hv;
      }
  __syncthreads();
  bf16x8 hf[4][KS2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int ks = 0; ks < KS2; ++ks)
      hf[mt][ks] =
          *reinterpret_cast<const bf16x8*>(&Hs[(mt * 16 + lr) * S::LDH + ks * 32 + lg * 8]);

  // GEMM2 transposed, O^T = W2 H^T: the A operand is W2's rows (output columns), the B
  // operand the hidden rows, so a lane ends with 4 consecutive output columns of one slot,
  // scaled by the slot's gate and stored as 8 bytes straight into the slot row.  Wave w
  // takes the 64-column chunks w, w + 4, ...; the next chunk's W2 fragments are loaded
  // while the current one is multiplied.
  int sl[4];
  float gs[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    sl[mt] = s_slot[mt * 16 + lr];
    gs[mt] = s_gate[mt * 16 + lr];
  }
  for (int nc = w * 64; nc < h_out; nc += 256) {
    bf16x8 cur[4][KS2];
    if constexpr (PREFETCH) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int ks = 0; ks < KS2; ++ks) cur[nt][ks] = wf[nt][ks];
      if (nc + 256 < h_out) load_w2(nc + 256, wf);
    } else {
      load_w2(nc, cur);
    }
    floatx4 acc[4][4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS2; ++ks)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[nt][mt] = mfma16(cur[nt][ks], hf[mt][ks], acc[nt][mt]);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (sl[mt] < 0) continue;
      bf16* orow = slots + (int64_t)sl[mt] * h_out + nc + lg * 4;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (bf16)(acc[nt][mt][i] * gs[mt]);
        *reinterpret_cast<bf16x4*>(orow + nt * 16) = v;
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
  if (h_in % 64 || h_out % 64) return -1;
  // every tile index below the bound has a block (a multiple of the 8 XCDs)
  const int64_t cap = tile_bound(nslots, E, FFN_TILE_M);
  const unsigned grid = (unsigned)((cap + 7) / 8 * 8);
#define EF_CASE(FF, KK)                                                                  \
  expert_ffn_kernel<FF, KK><<<grid, 256, 0, st>>>(k, h_in, h_out, E, (const bf16*)x,     \
                                                  (const bf16*)w1, (const bf16*)w3,      \
                                                  (const bf16*)w2, perm, pgate, tiles,   \
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
