/*
 * dreamer.h -- C ABI of libdreamer: forward pass of one Dreamer depth-recurrent
 * attention-mixture layer (arXiv 2601.21582) on AMD MI355X (gfx950).
 *
 * Pages cited (all about arXiv 2601.21582):
 *   [PN]    papernotes.org paper notes: "Method / overall framework" (loop flowchart,
 *           DA-cache remark), "Key design 1" (depth attention, half-reversed depth RoPE,
 *           parallel-residual equation), "Key design 2" (expert attention, gate
 *           equation, bias update), "Key design 3" (linear-MoE projections, shared
 *           expert identity), "Loss / training" (RMSNorm on the residual stream).
 *   [GS-de] gist.science German technical summary, "Methodik: Dreamer-Framework".
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is DEVICE memory owned by the caller.  No entry point
 *     allocates or frees device memory: scratch space is passed in as `ws`/`ws_bytes`
 *     (query the size with the matching *_ws_bytes function).  No entry point waits for
 *     the device, except dreamer_timing_read, which synchronises on its timing events.
 *     Tables and weights are read only.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = null stream).  The
 *     return value reports host-side validation and launch errors only; a fault inside
 *     a kernel surfaces at the caller's next synchronisation.
 *   - Layouts are row-major and contiguous unless stated.  `dtype` selects the storage
 *     type of activations and weights: DREAMER_F32 or DREAMER_BF16.  Accumulation is
 *     always float32; softmax, RoPE, routing scores and gates are float32.  Biases, gates
 *     and RoPE tables are float32 in both modes.
 *   - Weight matrices are stored [out_features, in_features] (y = x W^T).
 *   - RoPE tables are plain rotary tables cos/sin[pos][i] = cos/sin(pos * base^(-2i/D)),
 *     i < D/2, pairs (i, i + D/2) ("rotate half"); fill them with dreamer_rope_tables.
 *   - Status: DREAMER_OK, or DREAMER_E_INVAL (null pointer, negative or inconsistent
 *     size), DREAMER_E_UNSUPPORTED (a shape the kernels do not cover), DREAMER_E_WORKSPACE
 *     (ws too small), DREAMER_E_HIP (launch error).  dreamer_last_error() then returns a
 *     static, thread-local description.
 *   - Library state, process-wide and kept until the process ends: (1) per device, two
 *     side streams (default priority) and one fork/join event, created by the first
 *     layer call that forks with branch_streams (see below) and guarded by a mutex; (2) the
 *     kernel-timing state of dreamer_timing_* (one harness at a time, not thread-safe);
 *     (3) the thread-local error text.  Nothing else is kept between calls: calls on
 *     different streams may run concurrently, but calls that share output or ws buffers
 *     race.
 */
#ifndef DREAMER_H
#define DREAMER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DREAMER_OK 0
#define DREAMER_E_INVAL 1
#define DREAMER_E_UNSUPPORTED 2
#define DREAMER_E_WORKSPACE 3
#define DREAMER_E_HIP 4

#define DREAMER_F32 0
#define DREAMER_BF16 1

#define DREAMER_FFN_GELU 0   /* FFN(x) = W2 gelu_erf(W1 x)                 */
#define DREAMER_FFN_SWIGLU 1 /* FFN(x) = W2 (silu(W1 x) * (W3 x))           */
#define DREAMER_FFN_LINEAR 2 /* FFN(x) = W1 x   (linear-MoE projection expert) */

typedef void* dreamer_stream_t;

/* Description of the last error on this thread ("" if none). */
const char* dreamer_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int dreamer_version(void);

/*
 * Plain rotary tables for positions 0..npos-1: cos_out/sin_out [npos, D/2] float32,
 * entry (p, i) = cos/sin(p * base^(-2i/D)) evaluated in float64 on the device and rounded.
 * D must be even.  Used for sequence RoPE (positions = token positions) and depth RoPE
 * (positions = depths 0..L-1).
 */
int dreamer_rope_tables(int D, int npos, double base, float* cos_out, float* sin_out,
                        dreamer_stream_t stream);

/*
 * Depth attention DA at depth l ([PN] "Key design 1"; [GS-de] "Depth Attention"):
 * each of `rows` rows (b*s tokens in prefill, b sequences in decode) attends over its
 * own keys at depths 0..l, inclusive of l.
 *   q, k_new, v_new : [rows, H, d]  this depth's projections (not rotated)
 *   k_cache, v_cache: [rows, L, H, d] in/out.  Depth RoPE is applied to q and k_new,
 *                     then the rotated key and the value are written into slot l;
 *                     slots 0..l-1 are read, slots > l are never touched.  In decode the
 *                     same buffers are reused for every token, slot l being overwritten,
 *                     so DA memory does not grow with the sequence ([PN] overall
 *                     framework: the DA cache is overwritten at the next token).
 *   out             : [rows, H, d]
 *   cos_d, sin_d    : [L, d/2] rotary tables of positions 0..L-1.  Depth RoPE uses, for
 *                     rotary pair i, position l when i < d/4 and L-1-l otherwise (half of
 *                     the rotary dims run in reversed depth order).
 *   scale           : score scale (1/sqrt(d) in the layer).
 * Requires d % 16 == 0 (bf16) or d % 8 == 0 (f32), 0 <= l < L.
 */
int dreamer_depth_attn(int dtype, int64_t rows, int H, int d, int l, int L, const void* q,
                       const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                       void* out, const float* cos_d, const float* sin_d, float scale,
                       dreamer_stream_t stream);

/*
 * Windowed / dilated depth attention ([PN] "Limitations and outlook" proposes local
 * sliding windows combined with dilated sparse depth attention to cut the memory traffic
 * of deep recurrences; the pages give no formula, this is the plainest reading):
 * as dreamer_depth_attn, but depth l reads only the slots j <= l with l - j < window, and,
 * when dilation > 0, the older slots with (l - j) % dilation == 0.  The current slot is
 * always read; window == 0 is dreamer_depth_attn (dilation ignored).  Skipped slots are
 * never loaded, and slot l is still written, so the cache layout is unchanged.
 * Errors: DREAMER_E_INVAL for window < 0 or dilation < 0, otherwise as dreamer_depth_attn.
 */
int dreamer_depth_attn_windowed(int dtype, int64_t rows, int H, int d, int l, int L,
                                const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, void* out, const float* cos_d,
                                const float* sin_d, float scale, int window, int dilation,
                                dreamer_stream_t stream);

/*
 * Causal sequence attention SA at one depth ([PN] parallel-residual equation, SA(x_l);
 * [GS-de] "standard self-attention along the token sequence").
 *   q, k_new, v_new : [B, q_len, H, d] projections of tokens at positions pos0..pos0+q_len-1
 *   k_cache, v_cache: [B, cap, H, d] rotated keys / values by position, or NULL.
 *                     Prefill (pos0 == 0): optional; if given, the rotated keys and the
 *                     values of the q_len tokens are written at positions 0..q_len-1.
 *                     Decode (pos0 > 0): required, q_len must be 1; positions 0..pos0-1
 *                     are read and the new token is appended at pos0 (cap > pos0).
 *   out             : [B, q_len, H, d]
 *   cos_s, sin_s    : [>= pos0 + q_len, d/2] rotary tables (ignored if sa_rope == 0)
 *   ws, ws_bytes    : scratch, at least dreamer_seq_attn_ws_bytes(...) bytes.
 */
size_t dreamer_seq_attn_ws_bytes(int dtype, int B, int q_len, int H, int d, int64_t pos0);
int dreamer_seq_attn(int dtype, int B, int q_len, int H, int d, int64_t pos0, const void* q,
                     const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                     int64_t cap, void* out, const float* cos_s, const float* sin_s,
                     float scale, int sa_rope, void* ws, size_t ws_bytes,
                     dreamer_stream_t stream);

/*
 * dreamer_seq_attn without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, semantics and results as dreamer_seq_attn; its scratch
 * is a fixed device array inside the library of DREAMER_NOALLOC_SCRATCH_BYTES (64 MiB),
 * one copy per GPU, kept until the process ends (its address is looked up on the first
 * call on each device).  Shapes whose dreamer_seq_attn_ws_bytes exceeds that limit are
 * rejected with DREAMER_E_WORKSPACE before anything is launched (for example decode of
 * 64 sequences x 32 heads x 64 over 4096 cached positions needs about 9 MB; bf16 prefill
 * with RoPE needs 6 * B * q_len * H * d bytes).  Nothing is allocated or freed.  Every
 * call on one GPU shares that GPU's array: calls that may overlap on one GPU (different
 * streams, or host threads) race and must be serialised by the caller.
 */
#define DREAMER_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int dreamer_seq_attn_noalloc(int dtype, int B, int q_len, int H, int d, int64_t pos0,
                             const void* q, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, int64_t cap, void* out,
                             const float* cos_s, const float* sin_s, float scale, int sa_rope,
                             dreamer_stream_t stream);

/*
 * Expert-attention router ([PN] "Key design 2"; [GS-de] "Routing"):
 *   u = x W_r^T (rank r, float32), depth RoPE on u at depth l of L (same half-reversed
 *   rule as DA), z_e = rho * (u . keys_e); the k experts with the largest z_e + bias_e
 *   are selected (descending; ties to the lower index) and their gates are sigmoid(z_e),
 *   divided by the sum of the k gates (taken in selection order) when `normalize` != 0:
 *   sigma = norm(TopK(sigmoid(z), z + b, k)).
 *   x      : [T, h] storage dtype     w_r : [r, h]     keys : [E, r]     bias : [E] f32
 *   cos_r, sin_r : [L, r/2] rotary tables of positions 0..L-1
 *   idx    : [T, k] int32 out         gate : [T, k] f32 out
 *   counts : [E] int32 out (set to the number of selections of each expert) or NULL
 * Requires r % 8 == 0, h % 64 == 0 (bf16) or h % 4 == 0 (f32), 1 <= k <= min(E, 32),
 * E <= 16384.
 */
size_t dreamer_expert_route_ws_bytes(int64_t T, int r, int E);
int dreamer_expert_route(int dtype, int64_t T, int h, int r, int E, int k, int l, int L,
                         const void* x, const void* w_r, const void* keys, const float* bias,
                         float rho, int normalize, const float* cos_r, const float* sin_r,
                         int32_t* idx, float* gate, int32_t* counts, void* ws,
                         size_t ws_bytes, dreamer_stream_t stream);

/*
 * Sparse experts, value side ([PN] "Key design 2": each expert's FFN is the value
 * transform; dropless routing -- every selected (token, expert) pair is computed):
 *   out[t] = residual[t] + sum_{i<k} gate[t,i] * FFN_{idx[t,i]}(x[t])   (i in order)
 *   x : [T, h_in] storage dtype;  idx, gate : [T, k] (idx entries in [0, E));
 *   residual : [T, h_out] f32 or NULL
 *   GELU/SWIGLU: w1 (and w3) [E, f, h_in], w2 [E, h_out, f]; LINEAR: w1 [E, h_out, h_in],
 *   f ignored, w2/w3 unused.   out : [T, h_out] f32.
 * Tokens are grouped by expert on the device (count, scan, scatter); no capacity limit.
 * bf16 GELU/SWIGLU needs f in {64, 128} and h_in, h_out % 64 == 0.  E <= 8192.
 */
size_t dreamer_expert_ffn_ws_bytes(int dtype, int kind, int64_t T, int h_in, int f,
                                   int h_out, int E, int k);
int dreamer_expert_ffn(int dtype, int kind, int64_t T, int h_in, int f, int h_out, int E,
                       int k, const void* x, const int32_t* idx, const float* gate,
                       const void* w1, const void* w3, const void* w2, const float* residual,
                       float* out, void* ws, size_t ws_bytes, dreamer_stream_t stream);

/*
 * Expert-load bookkeeping ([PN] "Key design 2": the router bias is nudged by the sign of
 * the difference between the median usage count and each expert's count; [PN] analysis
 * of expert usage: unique experts per depth, Lorenz curve and Gini coefficient).
 *
 * dreamer_route_counts: counts[s, e] = #{j : idx[s * per_set + j] == e} for every set s
 *   (e.g. one set per depth of a [L, T, k] routing, per_set = T * k; or one set over all
 *   depths).  idx entries must lie in [0, E) (others are clamped into it).
 *   counts : [n_sets, E] int32 out (overwritten).  E <= 16384, n_sets <= 65535.
 * dreamer_bias_update: bias[e] += lambda * sign(median(counts) - counts[e]), in place;
 *   the median of an even count is the mean of the two middle values.  counts : [E].
 * dreamer_expert_usage: stats[s] = {number of experts with count > 0, max / mean count,
 *   Gini = sum_i sum_j |N_i - N_j| / (2 E^2 mean)} (0 for an all-zero set; the pair sum
 *   is exact in 64-bit integers).  counts : [n_sets, E], stats : [n_sets, 3] f32.
 *   E <= 8192, n_sets <= 65535.
 */
int dreamer_route_counts(const int32_t* idx, int64_t n_sets, int64_t per_set, int E,
                         int32_t* counts, dreamer_stream_t stream);
int dreamer_bias_update(const int32_t* counts, int E, float lambda, float* bias,
                        dreamer_stream_t stream);
int dreamer_expert_usage(const int32_t* counts, int64_t n_sets, int E, float* stats,
                         dreamer_stream_t stream);

/*
 * Offline absorption of the shared projection expert ([PN] "Key design 3"):
 *   out[e] = W_e + W_shared for e < n_experts; w_e/out: [n_experts, n], w_shared: [n].
 * bf16: out = bf16(float(W_e) + float(W_shared)).  out may alias w_e.
 */
int dreamer_absorb_shared(int dtype, int64_t n_experts, int64_t n, const void* w_e,
                          const void* w_shared, void* out, dreamer_stream_t stream);

/* Mixture wirings of one depth step ([PN] ablation of the mixture's parallelism; the
 * pages name the three wirings and their relative step throughput, not the formulas;
 * these are the plainest readings with one RMSNorm per step, xh = RMSNorm(x_l) * g):
 *   PARTIAL   y = xh + DA(xh) + SA(xh);       x' = y + EA(y)        (default)
 *   SERIAL    u = xh + DA(xh);  v = u + SA(u);  x' = v + EA(v)     (DA -> SA -> EA)
 *   PARALLEL  x' = xh + DA(xh) + SA(xh) + EA(xh)                   (all three at once)
 * DA(.) / SA(.) include their halves of the output projection.  With branch_streams set,
 * the independent branches of a step run concurrently on side streams of the library
 * (two per device, created once, default priority) forked from and joined back into the
 * caller's stream: in PARTIAL and PARALLEL prefill, DA beside SA (unless the two share
 * one launch, see fuse_attn); in PARALLEL, also the EA chain (router, grouping, experts)
 * beside the attention.  Otherwise, and for SERIAL, everything runs in order on the
 * caller's stream.  Results are the same bits either way.  Calls that fork on one device
 * serialise their enqueueing on a host mutex. */
#define DREAMER_MIX_PARTIAL 0
#define DREAMER_MIX_SERIAL 1
#define DREAMER_MIX_PARALLEL 2

typedef struct dreamer_layer_cfg {
  int dtype;            /* DREAMER_F32 / DREAMER_BF16                                */
  int b, s;             /* batch and sequence length; decode: b sequences, s == 1    */
  int h, H, d;          /* hidden size, heads, head dim (h == H * d), shared by SA/DA */
  int L;                /* depth steps                                               */
  int E, k, f, r;       /* experts, top-k, expert width, router rank                 */
  int ffn_kind;         /* DREAMER_FFN_GELU / DREAMER_FFN_SWIGLU                     */
  int normalize_gates;  /* divide the k gates by their sum                           */
  int use_da, use_ea;   /* 0 disables depth attention / expert attention             */
  int sa_rope;          /* sequence RoPE on SA q and k                               */
  int proj_experts;     /* 0: dense Q/K/V/O; >0: top-1 linear MoE with this many experts */
  int mixture;          /* DREAMER_MIX_PARTIAL / _SERIAL / _PARALLEL                  */
  int decode;           /* 0: prefill of s tokens; 1: one new token per sequence      */
  int64_t sa_pos;       /* decode: position of the new token (positions 0..sa_pos-1 cached) */
  int64_t sa_cap;       /* SA cache capacity per sequence (decode: > sa_pos; prefill: >= s) */
  double rope_base;     /* rotary base (SA, DA and routers)                           */
  float rms_eps;        /* RMSNorm epsilon                                           */
  float rho;            /* router score scale                                        */
  int branch_streams;   /* 1: independent branches on side streams (see above)         */
  int da_window;        /* 0: DA over every depth 0..l; w > 0: only the w most recent  */
  int da_dilation;      /* with da_window > 0 and this > 0: also every da_dilation-th
                           older depth (see dreamer_depth_attn_windowed)               */
  int fuse_attn;        /* 1: SA and DA of a depth may share one launch (bf16 prefill,
                           PARTIAL / PARALLEL, head dim 64, no SA cache output, and the
                           causal flash grid fits the GPU in one round): the DA blocks
                           fill the CUs the flash grid's tail leaves idle.  Same bits
                           either way; timed as DREAMER_KC_ATTN.  0: separate launches */
} dreamer_layer_cfg;

typedef struct dreamer_layer_weights {
  const void* g;         /* [h] RMSNorm gain                                           */
  const void* w_qkv;     /* dense [6h, h] rows = SA q,k,v then DA q,k,v; MoE [Ep, 6h, h]  */
  const void* w_o;       /* dense [h, 2h] columns = SA heads then DA heads; MoE [Ep, h, 2h] */
  const void* w_pr;      /* MoE only: projection router [r, h]                          */
  const void* pkeys;     /* MoE only: projection expert keys [Ep, r]                    */
  const float* pbias;    /* MoE only: projection router bias [Ep] f32, or NULL (zeros)  */
  const void* w_r;       /* EA router [r, h]                                           */
  const void* keys;      /* EA expert keys [E, r]                                      */
  const float* bias;     /* EA router bias [E] f32                                     */
  const void* w1;        /* [E, f, h] GELU W1 / SwiGLU gate                             */
  const void* w3;        /* [E, f, h] SwiGLU up, NULL for GELU                          */
  const void* w2;        /* [E, h, f] down                                             */
} dreamer_layer_weights;

/*
 * The whole layer, unrolled over L depth steps with one shared set of parameters
 * ([PN] overall framework flowchart; parallel-residual equation of "Key design 1"):
 *   for l in 0..L-1:
 *     xh = RMSNorm(x_l) * g                          (the stream itself is normalised)
 *     [proj MoE: e*, sigma = top-1 projection router on xh; every projection below is
 *      sigma * xh W_{e*} with the shared expert already absorbed into W_{e*}]
 *     a_SA = SA(xh) at depth l,  a_DA = DA(xh) over depths 0..l
 *     y = xh + [a_SA | a_DA] W_o^T
 *     x_{l+1} = y + sum_i gate_i FFN_{idx_i}(y)   (router on y)
 *   (that is the PARTIAL wiring; SERIAL and PARALLEL as defined above)
 *   x_in  : [T, h] f32 (T = b*s; decode T = b)     x_out : [T, h] f32 = x_L
 *   route_idx, route_gate : [L, T, k] per-depth EA routing, or NULL
 *   proj_idx, proj_gate   : [L, T] per-depth projection routing (MoE), or NULL
 *   x_steps : [L, T, h] f32, x_{l+1} after every step, or NULL
 *   y_steps : [L, T, h] storage dtype, the EA router input of every step (the storage
 *             copy of y; of xh in the PARALLEL wiring), or NULL
 *   da_k, da_v : [T, L, H, d] DA caches, or NULL (then kept in ws); their old contents
 *                are never read
 *   sa_k, sa_v : [L, b, sa_cap, H, d] per-depth SA caches of rotated keys / values.
 *                Decode: required, positions 0..sa_pos-1 read, sa_pos written.
 *                Prefill: optional, positions 0..s-1 written (hand-off to decode).
 *   route_in, proj_route_in : [L, T, k] / [L, T] int32 expert choices to replay instead
 *                of selecting (gates are still computed from this run's own scores), or
 *                NULL.  Replaying the choices of another run (another precision, a
 *                reference) removes the discrete top-k flips that last-bit differences
 *                cause, so the continuous parts can be compared alone.  Entries must lie
 *                in [0, E); out-of-range entries are clamped into it.
 *   ws, ws_bytes : scratch of at least dreamer_layer_ws_bytes(cfg) bytes.
 * Precision (bf16 storage): xh is stored in bf16 as the projection input and kept in
 * float32 for the residual; y and x stay float32; EA reads a bf16 copy of y.
 */
size_t dreamer_layer_ws_bytes(const dreamer_layer_cfg* cfg);
int dreamer_layer_forward(const dreamer_layer_cfg* cfg, const dreamer_layer_weights* w,
                          const float* x_in, float* x_out, int32_t* route_idx,
                          float* route_gate, int32_t* proj_idx, float* proj_gate,
                          float* x_steps, void* y_steps, void* da_k, void* da_v, void* sa_k,
                          void* sa_v, const int32_t* route_in, const int32_t* proj_route_in,
                          void* ws, size_t ws_bytes, dreamer_stream_t stream);

/*
 * Multi-token decode ([PN] inference: the SA key/value cache persists across tokens, one
 * per depth; the DA cache is addressed only within one token's depth steps and the next
 * token overwrites it): n_tokens consecutive decode steps of b sequences, token j at
 * position cfg->sa_pos + j.  The same as n_tokens calls of dreamer_layer_forward with
 * decode = 1 and sa_pos incremented (same bits); the rotary tables are built once.
 *   cfg   : decode = 1, s = 1, sa_pos = P0 > 0 (positions 0..P0-1 cached),
 *           sa_cap >= P0 + n_tokens
 *   x_in  : [n_tokens, b, h] f32, token j of every sequence (its embedding; this layer
 *           has no head, so the caller supplies the next inputs)
 *   x_out : [n_tokens, b, h] f32, x_L of every token
 *   route_idx, route_gate : [n_tokens, L, b, k] per-token EA routing, or NULL
 *   da_k, da_v : [b, L, H, d] DA caches reused by every token, or NULL (kept in ws)
 *   sa_k, sa_v : [L, b, sa_cap, H, d]; positions P0..P0+n_tokens-1 are appended
 *   ws, ws_bytes : scratch of at least dreamer_decode_ws_bytes(cfg, n_tokens) bytes
 * Errors as dreamer_layer_forward; a failure part-way leaves the earlier tokens done.
 */
size_t dreamer_decode_ws_bytes(const dreamer_layer_cfg* cfg, int n_tokens);
int dreamer_decode_tokens(const dreamer_layer_cfg* cfg, const dreamer_layer_weights* w,
                          int n_tokens, const float* x_in, float* x_out, int32_t* route_idx,
                          float* route_gate, void* da_k, void* da_v, void* sa_k, void* sa_v,
                          void* ws, size_t ws_bytes, dreamer_stream_t stream);

/*
 * Kernel timing, for measurement harnesses.  When enabled, every launch of the kernel
 * class `kclass` (DREAMER_KC_*) made by the library on a stream is bracketed by two HIP
 * events recorded on that stream (timing-only events, without a system-scope fence; the
 * bracket holds the kernel's dispatch as well as its execution); dreamer_timing_read
 * returns the number of bracketed launches and their summed duration in milliseconds (it
 * synchronises on the events).  Disabled by default; not reentrant (one harness at a
 * time).
 */
#define DREAMER_KC_GEMM 1       /* Q/K/V projection (and the float32 router projection) */
#define DREAMER_KC_SEQ_ATTN 2
#define DREAMER_KC_DEPTH_ATTN 3
#define DREAMER_KC_ROUTE 4      /* router scores + top-k                               */
#define DREAMER_KC_PERMUTE 5
#define DREAMER_KC_EXPERT_FFN 6
#define DREAMER_KC_COMBINE 7    /* combine + RMSNorm (and the first RMSNorm)           */
#define DREAMER_KC_OUT_PROJ 8   /* output projection + residual                        */
#define DREAMER_KC_ATTN 9       /* SA and DA in one launch (dreamer_layer_cfg.fuse_attn) */
int dreamer_timing_enable(int kclass, int max_launches);
int dreamer_timing_read(int* n_launches, double* total_ms);
int dreamer_timing_disable(void);

#ifdef __cplusplus
}
#endif
#endif /* DREAMER_H */
