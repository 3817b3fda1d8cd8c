/*
 * dreamer_ref.h -- C ABI of libdreamer_ref, the CPU oracle of one Dreamer depth-recurrent
 * attention-mixture layer (arXiv 2601.21582), forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark may load this library.  It shares no code, header, table or constant with
 * the GPU library (libdreamer); the two only see the same seeded inputs.
 *
 * Plain C++17 with OpenMP over independent rows: float64 arithmetic, written in the
 * order the pages describe the method, slow and obvious on purpose.  Every output element
 * is computed by one thread in a fixed order, so results do not depend on the number of
 * threads.
 *
 * Pages cited (all describe arXiv 2601.21582):
 *   [PN]    papernotes.org paper notes (Chinese): "Method / overall framework" (loop
 *           flowchart, DA-cache remark), "Key design 1" (depth attention, half-reversed
 *           depth RoPE, parallel-residual equation), "Key design 2" (expert attention,
 *           gate equation, bias update), "Key design 3" (linear-MoE projections and the
 *           shared-expert identity), "Loss / training" (RMSNorm on the residual stream),
 *           ablation table (mixture wirings), analysis of expert usage (Gini, Lorenz),
 *           "Limitations and outlook" (windowed / dilated depth attention).
 *   [GS-de] gist.science German technical summary, "Methodik: Dreamer-Framework".
 *
 * Conventions
 *   - Every pointer is HOST memory owned by the caller; arrays are row-major, contiguous.
 *   - Activations, caches and outputs are float64.  Weight matrices are float64 or
 *     float32 (a flag says which; bf16 and f32 storage values are exact in float32), and
 *     are stored [out_features, in_features], y = x W^T.
 *   - bf16 = 1 switches on storage emulation: the values the GPU path stores in bfloat16
 *     are rounded to bfloat16 (round to nearest, ties to even) at the same named points
 *     (x_hat as projection input, rotated q/k, v, attention outputs, the bf16 copy of y,
 *     the expert hidden state, the gated expert outputs).  Everything else stays float64.
 *   - Return value: 0 on success, 1 for an invalid argument (null pointer, bad size).
 */
#ifndef DREAMER_REF_H
#define DREAMER_REF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Threads used by the parallel loops (OpenMP); n <= 0 keeps the current setting.
 * Returns the number in use. */
int dreamer_ref_threads(int n);

/* ---------------------------------------------------------------- pieces ---------- */

/* out[i] = x[i] rounded to the nearest bfloat16 (through float32, both steps ties to even). */
void dreamer_ref_bf16_round(const double* x, int64_t n, double* out);

/* Residual-stream RMSNorm ([PN] "Loss / training"):
 * out[t] = x[t] / sqrt(mean_j x[t,j]^2 + eps) * g.   x, out: [rows, h]; g: [h]. */
int dreamer_ref_rmsnorm(const double* x, const double* g, int64_t rows, int h, double eps,
                        double* out);

/* Rotary embedding, rotate-half pairs (i, i + D/2), theta_i = base^(-2 i / D):
 *   out_i = u_i cos(p_i theta_i) - u_{i+D/2} sin(p_i theta_i)
 *   out_{i+D/2} = u_{i+D/2} cos(p_i theta_i) + u_i sin(p_i theta_i)
 * u, out: [n, D]; pos: [n, D/2], one position per vector and rotary pair. */
int dreamer_ref_rope(const double* u, const double* pos, int64_t n, int D, double base,
                     double* out);

/* Depth RoPE ([PN] "Key design 1": half of the rotary dims run in reversed depth order):
 * rotary pairs i < D/4 at position l, pairs i >= D/4 at position L-1-l.  u, out: [n, D]. */
int dreamer_ref_depth_rope(const double* u, int64_t n, int D, int l, int L, double base,
                           double* out);

/* Depth slots read by DA at depth l: all of 0..l when window <= 0; otherwise the window
 * most recent depths plus, when dilation > 0, every older j with (l - j) % dilation == 0
 * ([PN] "Limitations and outlook").  Writes them ascending to keys[] (room for l + 1) and
 * returns their number. */
int dreamer_ref_depth_keys(int l, int window, int dilation, int* keys);

/* ------------------------------------------------------------- attention ---------- */

/* Causal sequence attention at one depth ([PN] parallel-residual equation, SA(x_l)):
 *   q, k_new, v_new : [B, n, H, d], tokens at positions pos0..pos0+n-1
 *   k_cache, v_cache: [B, cap, H, d] (float64, or float32 when cache_f32) rotated keys and
 *                     values of positions 0..pos0-1; read only; may be NULL when pos0 == 0
 *   sa_rope         : plain RoPE on q and k_new at their positions
 *   out             : [B, n, H, d]; k_rot, v_out : [B, n, H, d] the entries to append
 * Scale 1/sqrt(d); token i sees keys 0..pos0+i. */
int dreamer_ref_seq_attn(int B, int n, int H, int d, int64_t pos0, const double* q,
                         const double* k_new, const double* v_new, const void* k_cache,
                         const void* v_cache, int64_t cap, int cache_f32, int sa_rope,
                         double base, int bf16, double* out, double* k_rot, double* v_out);

/* Depth attention at depth l ([PN] "Key design 1"): every row attends over its own keys
 * at the depths dreamer_ref_depth_keys(l, window, dilation) (0..l, inclusive of l).
 *   q, k_new, v_new : [R, H, d]; with use_rope, depth RoPE is applied to q and k_new
 *   k_cache, v_cache: [R, L, H, d]; the (rotated) key and the value are written into
 *                     slot l first; other slots are read, slots > l never
 *   out             : [R, H, d]    scale 1/sqrt(d). */
int dreamer_ref_depth_attn(int64_t R, int H, int d, int l, int L, const double* q,
                           const double* k_new, const double* v_new, double* k_cache,
                           double* v_cache, double base, int bf16, int use_rope, int window,
                           int dilation, double* out);

/* --------------------------------------------------------------- routing ---------- */

/* The k largest entries of every row of key[T, E], descending; equal keys go to the lower
 * index (a stable sort of the indices).  idx: [T, k]. */
int dreamer_ref_topk_select(const double* key, int64_t T, int E, int k, int64_t* idx);

/* Expert-attention router ([PN] "Key design 2"):
 *   u = x W_r^T (rank r), depth RoPE on u, z_e = rho * (u . keys_e),
 *   sel = TopK by z + bias, gate = sigmoid(z_sel), divided by its sum when normalize.
 *   x [T, h]; w_r [r, h], keys [E, r] (float32 when w_f32); bias [E]
 *   idx [T, k], gate [T, k], counts [E] or NULL, z [T, E] or NULL */
int dreamer_ref_expert_route(int64_t T, int h, int r, int E, int k, int l, int L,
                             const double* x, const void* w_r, const void* keys, int w_f32,
                             const double* bias, double rho, int normalize, double base,
                             int64_t* idx, double* gate, int64_t* counts, double* z);

/* Balancing update b <- b + lambda * sign(median(N) - N) ([PN] "Key design 2"); the
 * median of an even count is the mean of the two middle values.  out may alias bias. */
int dreamer_ref_bias_update(const double* bias, const int64_t* counts, int E, double lambda,
                            double* out);

/* counts[s, e] = number of entries equal to e in idx[s * per_set .. (s+1) * per_set). */
int dreamer_ref_route_counts(const int64_t* idx, int64_t n_sets, int64_t per_set, int E,
                             int64_t* counts);

/* Usage statistics of counts[E] ([PN] analysis of expert usage): number of experts used,
 * max / mean, Gini = sum_i sum_j |N_i - N_j| / (2 E^2 mean), and the Lorenz curve
 * lorenz[E] (share of all selections held by the 1, 2, .., E least used experts). */
int dreamer_ref_expert_usage(const int64_t* counts, int E, int* distinct,
                             double* max_over_mean, double* gini, double* lorenz);

/* --------------------------------------------------------------- experts ---------- */

#define DREAMER_REF_GELU 0
#define DREAMER_REF_SWIGLU 1
#define DREAMER_REF_LINEAR 2

/* Sparse experts, value side ([PN] "Key design 2"; dropless):
 *   out[t] = residual[t] + sum_{i<k} gate[t,i] * FFN_{idx[t,i]}(x[t])   (i in order)
 *   GELU:   FFN(x) = W2 gelu_erf(W1 x);  SWIGLU: W2 (silu(W1 x) * (W3 x));
 *   LINEAR: FFN(x) = W1 x.
 *   x [T, h_in]; idx, gate [T, k]; w1 (w3) [E, f, h_in], w2 [E, h_out, f]
 *   (LINEAR: w1 [E, h_out, h_in]); float32 when w_f32; residual [T, h_out] or NULL;
 *   out [T, h_out].
 *   slots [T, k, h_out] (gated, stored expert outputs) and hidden [T, k, f] (the stored
 *   hidden state; not for LINEAR) receive the intermediate values, or are NULL. */
int dreamer_ref_expert_ffn(int kind, int64_t T, int h_in, int f, int h_out, int E, int k,
                           const double* x, const int64_t* idx, const double* gate,
                           const void* w1, const void* w3, const void* w2, int w_f32,
                           const double* residual, int bf16, double* out, double* slots,
                           double* hidden);

/* ----------------------------------------------------------------- layer ---------- */

#define DREAMER_REF_PARTIAL 0   /* y = xh + DA(xh) + SA(xh); x' = y + EA(y)       */
#define DREAMER_REF_SERIAL 1    /* u = xh + DA(xh); v = u + SA(u); x' = v + EA(v) */
#define DREAMER_REF_PARALLEL 2  /* x' = xh + DA(xh) + SA(xh) + EA(xh)             */

typedef struct dreamer_ref_cfg {
  int bf16;                 /* storage emulation                                    */
  int b, s, h, H, d, L;     /* decode: b sequences, s == 1                          */
  int E, k, f, r;
  int ffn;                  /* DREAMER_REF_GELU / DREAMER_REF_SWIGLU                */
  int normalize;            /* normalise the EA gates                               */
  int use_da, use_ea, sa_rope;
  int proj_experts;         /* 0 dense projections; > 0 top-1 linear MoE            */
  int mixture;              /* DREAMER_REF_PARTIAL / _SERIAL / _PARALLEL            */
  int decode;               /* one new token per sequence at position sa_pos        */
  int64_t sa_pos;
  int da_window, da_dilation;
  double rope_base, rms_eps, rho;
} dreamer_ref_cfg;

/* Weights.  f32 = 1: every matrix is float32, else float64.  Dense projections use w_qkv
 * [6h, h] (rows: SA q, k, v then DA q, k, v) and w_o [h, 2h] (columns: SA output then DA
 * output).  Linear MoE (proj_experts = Ep > 0) uses w_qkv_e [Ep, 6h, h], w_qkv_sh [6h, h],
 * w_o_e [Ep, h, 2h], w_o_sh [h, 2h] unabsorbed, with router w_pr [r, h], pkeys [Ep, r].
 * EA: w_r [r, h], keys [E, r], bias [E] (float64), w1, w3 [E, f, h], w2 [E, h, f]. */
typedef struct dreamer_ref_weights {
  int f32;
  const void *g, *w_qkv, *w_o;
  const void *w_qkv_e, *w_qkv_sh, *w_o_e, *w_o_sh, *w_pr, *pkeys;
  const void *w_r, *keys, *w1, *w3, *w2;
  const double* bias;
} dreamer_ref_weights;

/* Per-step outputs; every pointer may be NULL except x_next.
 *   x_next, y, yb [T, h]   (y: the stream after the attention (SERIAL: v), the residual
 *                           EA adds to; yb: the storage copy of the stream EA reads,
 *                           that is of y, or of x_hat in PARALLEL)
 *   idx, gate [T, k], counts [E], z [T, E]      EA routing (use_ea)
 *   pidx, pgate [T], pz [T, Ep]                 projection routing (proj_experts) */
typedef struct dreamer_ref_step_out {
  double *x_next, *y, *yb;
  int64_t *idx;
  double *gate;
  int64_t *counts;
  double *z;
  int64_t *pidx;
  double *pgate, *pz;
} dreamer_ref_step_out;

/* One depth step l ([PN] flowchart: RMSNorm, then DA and SA, residual, then EA):
 *   x [T, h] the stream x_l (T = b*s; decode T = b)
 *   da_k, da_v [T, L, H, d]: slot l written, the slots of the key set read
 *   sa_k, sa_v [L, b, sa_cap, H, d] (float32 when sa_f32) or NULL.  Decode: positions
 *     0..sa_pos-1 of depth l read, sa_pos written.  Prefill: positions 0..s-1 written.
 *   force_idx [T, k] / force_pidx [T] or NULL: adopt these expert choices (the gates still
 *     come from this step's own scores). */
int dreamer_ref_layer_step(const dreamer_ref_cfg* cfg, const dreamer_ref_weights* w,
                           const double* x, int l, double* da_k, double* da_v, void* sa_k,
                           void* sa_v, int64_t sa_cap, int sa_f32, const int64_t* force_idx,
                           const int64_t* force_pidx, const dreamer_ref_step_out* out);

/* The unrolled layer x_0 -> x_L ([PN] flowchart: one shared layer applied L times):
 *   x0 [T, h] -> x_out [T, h].  da_k, da_v [T, L, H, d] (their old contents are never read).
 *   steps: per-depth outputs, each field [L, ...] of the step_out shapes, or NULL;
 *   steps->x_next (if given) receives x_1..x_L.
 *   force_idx [L, T, k] / force_pidx [L, T] or NULL. */
int dreamer_ref_layer_forward(const dreamer_ref_cfg* cfg, const dreamer_ref_weights* w,
                              const double* x0, double* x_out, double* da_k, double* da_v,
                              void* sa_k, void* sa_v, int64_t sa_cap, int sa_f32,
                              const int64_t* force_idx, const int64_t* force_pidx,
                              const dreamer_ref_step_out* steps);

/* n consecutive decode steps ([PN]: the SA cache persists per depth, the DA cache is
 * overwritten by the next token): token j runs at position cfg->sa_pos + j with a fresh
 * DA cache and appends to sa_k / sa_v.  xs, x_out [n, b, h]; steps (or NULL): fields
 * [n, L, ...]. */
int dreamer_ref_decode_tokens(const dreamer_ref_cfg* cfg, const dreamer_ref_weights* w,
                              int n, const double* xs, double* x_out, void* sa_k, void* sa_v,
                              int64_t sa_cap, int sa_f32, const dreamer_ref_step_out* steps);

#ifdef __cplusplus
}
#endif
#endif /* DREAMER_REF_H */
