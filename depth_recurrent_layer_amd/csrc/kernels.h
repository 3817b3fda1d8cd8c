// Internal launcher interface between the C-ABI layer (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dreamer {

// Every kernel of the library is launched through dlaunch (one place to hook launches).
template <typename... P, typename... A>
void dlaunch(void (*kernel)(P...), dim3 grid, dim3 block, size_t shm, hipStream_t st,
             A... args) {
  kernel<<<grid, block, shm, st>>>(args...);
}

enum { DT_F32 = 0, DT_BF16 = 1 };
enum { FFN_GELU = 0, FFN_SWIGLU = 1, FFN_LINEAR = 2 };

struct GemmArgs {
  int M = 0, N = 0, K = 0;           // positions, columns, reduction length
  const void* A = nullptr;           // storage dtype, row stride lda
  int64_t lda = 0;
  const void* B = nullptr;           // [N, K] per group, row stride ldb
  int64_t ldb = 0;
  int64_t b_gstride = 0;             // elements between group matrices
  const int* rows = nullptr;         // position -> output row (A row = rows[m] / row_div)
  int row_div = 1;
  const float* row_scale = nullptr;  // per output row
  const int* goff = nullptr;         // [G+1] position offsets of groups (device)
  const int* toff = nullptr;         // [G+1] m-tile offsets of groups (device, tile_m rows)
  int G = 1;
  int tile_m = 64;                   // rows per m-tile used to build toff
  int n_fast = 0;                    // set by launch_gemm: grouped grid runs n-tiles fastest
  void* C = nullptr;                 // OutT, row stride ldc
  int64_t ldc = 0;
  const float* resid = nullptr;      // float32 residual, row stride ldr
  int64_t ldr = 0;
  void* C2 = nullptr;                // optional bf16 (f32 in f32 mode) copy, row stride ldc2
  int64_t ldc2 = 0;
  // QKV epilogue (bf16, head dim 64, BN = 128): columns are six blocks of qkv_h =
  // [SA q | SA k | SA v | DA q | DA k | DA v].  SA q/k are rotated by sequence position
  // (pos_fixed >= 0 ? pos_fixed : out_row % seq) when sa_rope, DA q/k by depth
  // (pairs < 16 at depth_l, the rest at depth_L-1-depth_l), before the bf16 rounding.
  // vt (optional): SA v also written transposed, [out_row / seq][head][64][seq].
  int qkv_h = 0;
  int qkv_sect0 = 0;                 // section of output column 0 (3: a DA-only projection)
  int seq = 1;
  int pos_fixed = -1;
  int sa_rope = 0;
  int depth_l = 0, depth_L = 1;
  const float4* rope_s4 = nullptr;  // interleaved rotary tables (RopeJobs t4): sequence positions,
  const float4* rope_d4 = nullptr;  // and depths 0..depth_L-1
  void* vt = nullptr;
  int vt_only = 0;                   // with vt: SA v only transposed (its plain rows unread)
  // optional: DA k and v (sections 4 and 5) written to these rows instead (row stride
  // da_ld; the depth-attention cache's current slot) and not into C
  void* da_k = nullptr;
  void* da_v = nullptr;
  int64_t da_ld = 0;
  // Split-K for few rows (dense, no row gather, generic epilogue): float32 scratch of
  // split_elems elements for partial products; launch_gemm splits K when the grid would
  // leave CUs idle and the partials fit, and then sums them in a fixed order in a second
  // pass that applies the epilogue.  ksplit: set by launch_gemm for the partial launch.
  float* split_ws = nullptr;
  int64_t split_elems = 0;
  int ksplit = 1;
};

// out_f32: C is float32 (else storage dtype).  Returns -1 on an unsupported shape.
int launch_gemm(const GemmArgs& a, int dtype, int out_f32, hipStream_t st);
// Compute units of the current device (cached per device).
int device_cus();

// RoPE tables in float64 math: cos/sin [npos, D/2].
void launch_rope_tables(int D, int npos, double base, float* c, float* s, hipStream_t st);
// The same values for D = 64, interleaved [npos][16] float4 (cos j, cos j+16, sin j, sin j+16).
// Rotary tables built in one launch (up to four): split cos / sin tables of head dim D, or
// (t4 set) the interleaved head-dim-64 table of the QKV epilogue.
struct RopeJob {
  int D = 0, npos = 0;
  float *c = nullptr, *s = nullptr;
  float4* t4 = nullptr;
};
struct RopeJobs {
  RopeJob j[4];
  int n = 0;
  double base = 10000.0;
  void add_split(int D, int npos, float* c, float* s) { j[n++] = RopeJob{D, npos, c, s, nullptr}; }
  void add_t4(int npos, float4* t) { j[n++] = RopeJob{64, npos, nullptr, nullptr, t}; }
};
void launch_rope_jobs(const RopeJobs& jobs, hipStream_t st);

// Depth attention (row strides in elements for q/k/v/out).  Cache: row r's slot j at
// r srow + j sslot elements; srow = 0 selects [rows, L, H, d] (srow = L h, sslot = h).
// rope: rotate q and k_new by depth here (else they arrive rotated and rounded).
int launch_depth_attn(int dtype, int64_t rows, int H, int d, int l, int L, const void* q,
                      int64_t ldq, const void* kn, int64_t ldk, const void* vn, int64_t ldv,
                      void* kc, void* vc, void* out, int64_t ldo, const float* cosd,
                      const float* sind, float scale, int rope, hipStream_t st,
                      int window = 0, int dilation = 0, int64_t srow = 0, int64_t sslot = 0);

// In-place RoPE of a [rows, 6h] QKV buffer (SA q/k by sequence position, DA q/k by depth).
int launch_qkv_rope(int dtype, int64_t rows, int H, int d, int seq, int pos_fixed,
                    int sa_rope, int l, int L, void* qkv, const float* cs, const float* sn,
                    const float* cd, const float* sd, hipStream_t st);

// Sequence attention.  rope: rotate q/k here by sequence position (else they arrive
// rotated, or no RoPE is wanted).  vt: v transposed [B][H][64][q_len] when available
// (prefill, bf16, d = 64); with rope == 0 and vt given the flash kernel needs no ws.
size_t seq_attn_ws(int dtype, int B, int q_len, int H, int d, int64_t pos0, int prepared);
int launch_seq_attn(int dtype, int B, int q_len, int H, int d, int64_t pos0, const void* q,
                    int64_t ldq, const void* kn, int64_t ldk, const void* vn, int64_t ldv,
                    const void* vt, void* kc, void* vc, int64_t cap, void* out, int64_t ldo,
                    const float* cos_s, const float* sin_s, float scale, int rope, void* ws,
                    size_t ws_bytes, hipStream_t st);
// SA and DA of one depth in one launch (bf16 prefill, head dim 64, flash-prepared SA
// inputs: rotated q / k rows and v transposed; DA q / k already rotated): the flash grid's
// blocks first, then the DA blocks.  q, k: SA rows; dq, dk, dv: the DA projections; all
// with row stride ldqkv; outputs with stride ldo.  attn_pair_ok says when it applies.
bool attn_pair_ok(int dtype, int B, int q_len, int H, int d, int64_t pos0, const void* vt);
int launch_attn_pair(int B, int S, int H, int l, int L, const void* q, const void* k,
                     const void* vt, const void* dq, const void* dk, const void* dv,
                     int64_t ldqkv, int64_t ldkv, int64_t srow, int64_t sslot, void* dkc, void* dvc, void* out_sa, void* out_da,
                     int64_t ldo, float scale, int window, int dilation, hipStream_t st);
// The same for query blocks of more than 64 rows (the two-set flash grid), the two kinds
// of block interleaved in proportion in one launch; -1 when S <= 64 or unsupported.
int launch_attn_pair2(int B, int S, int H, int l, int L, const void* q, const void* k,
                      const void* vt, const void* dq, const void* dk, const void* dv,
                      int64_t ldqkv, int64_t ldkv, int64_t srow, int64_t sslot, void* dkc, void* dvc, void* out_sa, void* out_da,
                      int64_t ldo, float scale, int window, int dilation, hipStream_t st);

// Router scores z [T, E] f32 = rho * RoPE_depth(x W_r^T) . keys.  bf16: u computed inside
// (u ignored; needs r % 32 == 0, E % 16 == 0); f32: reads u = x W_r^T [T, r].
int router_scores(int dtype, int64_t T, int h, int r, int E, int l, int L, const void* x,
                  int64_t ldx, const void* w_r, const float* u, const void* keys, float rho,
                  const float* cos_r, const float* sin_r, float* z, hipStream_t st);
// Top-k of z + bias (ties to the lower index), gates sigmoid(z), normalised on request by
// their sum in selection order.  idx_in (optional, [T, k]): adopt these experts instead of
// selecting (entries clamped into [0, E)).
int router_topk(int64_t T, int E, int k, const float* z, const float* bias, int normalize,
                const int32_t* idx_in, int32_t* idx, float* gate, hipStream_t st);
// Scores and top-k in one kernel (bf16 only; router_fused_ok says when it applies).
// hist (optional, [perm_blocks(T * k), E], zero on entry): the permutation's chunk
// histograms are counted here with global atomics (slot t * k + j in chunk
// (t * k + j) / PERM_CHUNK), so launch_permute can skip its histogram kernel.
bool router_fused_ok(int dtype, int64_t T, int r, int E, int k);
int router_route_fused(int64_t T, int h, int r, int E, int k, int l, int L, const void* x,
                       int64_t ldx, const void* w_r, const void* keys, const float* bias,
                       float rho, int normalize, const float* cos_r, const float* sin_r,
                       const int32_t* idx_in, int32_t* idx, float* gate, hipStream_t st,
                       int32_t* hist = nullptr);

// Fill n ints with a value (graph-safe replacement of memset).
void launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st);

// Permutation of routed slots by expert: hist [perm_blocks(nslots), E] scratch; outputs
// counts [E], goff [E+1], toff [E+1] (tiles of tile_m rows), perm [nslots] (perm[goff[e]+j]
// = slot id t*k+i of the j-th slot routed to e; order within an expert unspecified).
// Optional: pgate [nslots] = gate in the same order (gate given), and tiles
// [tile_bound(nslots, E, tile_m)] = {expert, first row, end of the expert's rows, 0} per
// m-tile (the first toff[E] entries are written).  pad: perm and pgate are tile-padded
// instead ([tile_bound * tile_m]: row j of m-tile t at t * tile_m + j; the rows past an
// expert's end in its last tile are left unwritten).  hist_ready: hist already holds the
// chunk histograms (counted by the fused router); zero_next (optional): another buffer
// of the hist shape that the scatter clears, ready for the next histogram.
constexpr int PERM_CHUNK = 1024, PERM_MAX_E = 8192, COUNT_MAX_E = 16384;
int perm_blocks(int64_t nslots);
int launch_permute(const int32_t* idx, int64_t nslots, int E, int tile_m, int32_t* hist,
                   int32_t* counts, int32_t* goff, int32_t* toff, int32_t* perm,
                   hipStream_t st, const float* gate = nullptr, float* pgate = nullptr,
                   int4* tiles = nullptr, int pad = 0, bool hist_ready = false,
                   int32_t* zero_next = nullptr);
inline int64_t tile_bound(int64_t nslots, int E, int tile_m) { return nslots / tile_m + E + 1; }
// counts [E] of routed slots per expert (hist as above).
int launch_counts(const int32_t* idx, int64_t nslots, int E, int32_t* hist, int32_t* counts,
                  hipStream_t st);

// counts [n_sets, E] (zeroed here) of the expert ids idx [n_sets, per_set] (E <= COUNT_MAX_E).
int launch_route_counts(const int32_t* idx, int64_t n_sets, int64_t per_set, int E,
                        int32_t* counts, hipStream_t st);
// bias[e] += lam * sign(median(counts) - counts[e]).
void launch_bias_update(const int32_t* counts, int E, float lam, float* bias, hipStream_t st);
// stats [n_sets, 3] = {distinct experts, max / mean, Gini} of counts [n_sets, E] (E <= PERM_MAX_E).
int launch_expert_usage(const int32_t* counts, int64_t n_sets, int E, float* stats,
                        hipStream_t st);

// Fused expert FFN (GELU / SWIGLU): slots[s] = gate[s] * FFN_e(x[s / k]) for every
// routed slot s, written in storage dtype [T*k, h_out].
// perm / pgate / tiles / toff from launch_permute (tile_m = FFN_TILE_M).
int launch_expert_ffn(int dtype, int kind, int64_t nslots, int k, int h_in, int f, int h_out,
                      int E, const void* x, const void* w1, const void* w3, const void* w2,
                      const int32_t* perm, const float* pgate, const int4* tiles,
                      const int32_t* toff, void* slots, hipStream_t st);
constexpr int FFN_TILE_M = 64;
// m-tile rows of the grouped (top-1 linear-MoE) Q/K/V/O projections
constexpr int PROJ_TILE_M = 128;
// float32 per-slot expert FFN (any kind, any f): slots[s] = gate[s] * FFN_idx[s](x[s/k]).
int launch_expert_ffn_f32(int kind, int64_t nslots, int k, int h_in, int f, int h_out,
                          const float* x, const int32_t* idx, const float* gate,
                          const float* w1, const float* w3, const float* w2, float* slots,
                          hipStream_t st);

// x_next[t] = y[t] + sum_i slots[t*k+i] (k may be 0, y may be null = 0); optional stores
// of x_next (f32, up to two destinations) and of xhat = RMSNorm(x_next) * g in storage
// dtype (xhat) and in float32 (xhat32, optional).
void launch_combine_norm(int dtype, int64_t T, int h, int k, const float* y,
                         const void* slots, float* x_out, float* x_out2, const void* g,
                         float eps, void* xhat, float* xhat32, hipStream_t st);
// xhat = RMSNorm(x) * g from an f32 stream.
void launch_rmsnorm(int dtype, int64_t T, int h, const float* x, const void* g, float eps,
                    void* xhat, float* xhat32, hipStream_t st);

// out[e*n + i] = w_e[e*n + i] + w_sh[i]
void launch_absorb(int dtype, int64_t ne, int64_t n, const void* we, const void* wsh,
                   void* out, hipStream_t st);

// Kernel-class timing hooks (api.cpp).
void timing_begin(int kclass, hipStream_t st);
void timing_end(int kclass, hipStream_t st);
// Records the thread's error text (dreamer_last_error) and returns `code`.
int api_fail(int code, const char* fmt, ...);

}  // namespace dreamer
