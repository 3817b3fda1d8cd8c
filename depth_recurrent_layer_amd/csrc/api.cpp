// C ABI of libdreamer (declared in include/dreamer.h): argument validation, workspace
// planning and the depth loop of the layer forward.  All device work is enqueued on the
// caller's stream through the launchers in kernels.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/dreamer.h"
#include "kernels.h"

using namespace dreamer;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return DREAMER_OK;
}

// Checks the launch queue after enqueuing kernels.
int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DREAMER_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

size_t esize(int dtype) { return dtype == DREAMER_BF16 ? 2 : 4; }

bool dtype_ok(int dtype) { return dtype == DREAMER_F32 || dtype == DREAMER_BF16; }

// Bump allocator over the caller's workspace (base == nullptr: size planning only).
struct Bump {
  char* base;
  size_t off = 0;
  explicit Bump(void* b) : base((char*)b) {}
  void* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
  template <typename T>
  T* take_n(size_t n) { return (T*)take(n * sizeof(T)); }
};

hipStream_t S(dreamer_stream_t s) { return (hipStream_t)s; }

// ---------------------------------------------------------------------------- timing
struct Timing {
  int kclass = 0;
  int max = 0;
  int n = 0;
  std::vector<hipEvent_t> ev0, ev1;
} g_tm;

}  // namespace

namespace dreamer {
int api_fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

void timing_begin(int kclass, hipStream_t st) {
  if (g_tm.kclass == kclass && g_tm.n < g_tm.max) (void)hipEventRecord(g_tm.ev0[g_tm.n], st);
}
void timing_end(int kclass, hipStream_t st) {
  if (g_tm.kclass == kclass && g_tm.n < g_tm.max) {
    (void)hipEventRecord(g_tm.ev1[g_tm.n], st);
    ++g_tm.n;
  }
}
}  // namespace dreamer

// compute units of the current device (cached per device)
int dreamer::device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
static int cu_count() { return dreamer::device_cus(); }

#define TB(kc) timing_begin(kc, st)
#define TE(kc) timing_end(kc, st)

// ------------------------------------------------------------------------ side streams
// Non-blocking side streams (default priority) and a fork/join event per device,
// created on first use and kept until the process ends.  side_fork makes `side` wait for
// the work queued on `st` so far; side_join makes `st` wait for the work queued on
// `side`.  A call that forks holds `mu` while it enqueues, so concurrent calls on one
// device never interleave their event records.
namespace {
struct SideStreams {
  hipStream_t s[2];  // [0]: the fully parallel wiring's EA chain, [1]: depth attention
  hipEvent_t ev;
  std::mutex mu;
};
std::mutex g_side_mu;
SideStreams* g_side[64];

SideStreams* side_streams() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(g_side_mu);
  if (!g_side[dev]) {
    SideStreams* ss = new SideStreams();
    for (hipStream_t& x : ss->s)
      if (hipStreamCreateWithFlags(&x, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&ss->ev, hipEventDisableTiming) != hipSuccess) return nullptr;
    g_side[dev] = ss;
  }
  return g_side[dev];
}

void side_fork(SideStreams* ss, hipStream_t st, hipStream_t side) {
  (void)hipEventRecord(ss->ev, st);
  (void)hipStreamWaitEvent(side, ss->ev, 0);
}

void side_join(SideStreams* ss, hipStream_t st, hipStream_t side) {
  (void)hipEventRecord(ss->ev, side);
  (void)hipStreamWaitEvent(st, ss->ev, 0);
}
}  // namespace

extern "C" {

const char* dreamer_last_error(void) { return g_err; }

int dreamer_version(void) { return 100; }

int dreamer_timing_enable(int kclass, int max_launches) {
  dreamer_timing_disable();
  if (kclass < DREAMER_KC_GEMM || kclass > DREAMER_KC_ATTN || max_launches <= 0)
    return fail(DREAMER_E_INVAL, "timing_enable: bad class or count");
  g_tm.ev0.resize(max_launches);
  g_tm.ev1.resize(max_launches);
  // timing-only events: no system-scope fence (cache writeback) at each record, which
  // would both inflate and perturb the bracketed launch
  for (int i = 0; i < max_launches; ++i) {
    if (hipEventCreateWithFlags(&g_tm.ev0[i], hipEventDisableSystemFence) != hipSuccess ||
        hipEventCreateWithFlags(&g_tm.ev1[i], hipEventDisableSystemFence) != hipSuccess)
      return fail(DREAMER_E_HIP, "timing_enable: hipEventCreate failed");
  }
  g_tm.max = max_launches;
  g_tm.n = 0;
  g_tm.kclass = kclass;
  return ok();
}

int dreamer_timing_read(int* n_launches, double* total_ms) {
  double tot = 0.0;
  for (int i = 0; i < g_tm.n; ++i) {
    if (hipEventSynchronize(g_tm.ev1[i]) != hipSuccess)
      return fail(DREAMER_E_HIP, "timing_read: event sync failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_tm.ev0[i], g_tm.ev1[i]) != hipSuccess)
      return fail(DREAMER_E_HIP, "timing_read: elapsed time failed");
    tot += ms;
  }
  if (n_launches) *n_launches = g_tm.n;
  if (total_ms) *total_ms = tot;
  return ok();
}

int dreamer_timing_disable(void) {
  for (auto e : g_tm.ev0) (void)hipEventDestroy(e);
  for (auto e : g_tm.ev1) (void)hipEventDestroy(e);
  g_tm.ev0.clear();
  g_tm.ev1.clear();
  g_tm.kclass = 0;
  g_tm.max = g_tm.n = 0;
  return ok();
}

int dreamer_rope_tables(int D, int npos, double base, float* cos_out, float* sin_out,
                        dreamer_stream_t stream) {
  if (D <= 0 || D % 2 || npos < 0 || !(base > 0.0)) return fail(DREAMER_E_INVAL, "rope_tables: bad D/npos/base");
  if (npos > 0 && (!cos_out || !sin_out)) return fail(DREAMER_E_INVAL, "rope_tables: null output");
  launch_rope_tables(D, npos, base, cos_out, sin_out, S(stream));
  return check_launch("rope_tables");
}

int dreamer_depth_attn(int dtype, int64_t rows, int H, int d, int l, int L, const void* q,
                       const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                       void* out, const float* cos_d, const float* sin_d, float scale,
                       dreamer_stream_t stream) {
  return dreamer_depth_attn_windowed(dtype, rows, H, d, l, L, q, k_new, v_new, k_cache,
                                     v_cache, out, cos_d, sin_d, scale, 0, 0, stream);
}

int dreamer_depth_attn_windowed(int dtype, int64_t rows, int H, int d, int l, int L,
                                const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, void* out, const float* cos_d,
                                const float* sin_d, float scale, int window, int dilation,
                                dreamer_stream_t stream) {
  if (!dtype_ok(dtype)) return fail(DREAMER_E_INVAL, "depth_attn: bad dtype");
  if (window < 0 || dilation < 0)
    return fail(DREAMER_E_INVAL, "depth_attn: negative window (%d) or dilation (%d)", window,
                dilation);
  if (rows < 0 || H <= 0 || d <= 0 || L <= 0 || l < 0 || l >= L)
    return fail(DREAMER_E_INVAL, "depth_attn: bad sizes (rows=%lld H=%d d=%d l=%d L=%d)",
                (long long)rows, H, d, l, L);
  if (rows == 0) return ok();
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !out || !cos_d || !sin_d)
    return fail(DREAMER_E_INVAL, "depth_attn: null pointer");
  const int vec = dtype == DREAMER_BF16 ? 8 : 4;
  if (d % (2 * vec) || (d / vec) > 64 || ((d / vec) & (d / vec - 1)))
    return fail(DREAMER_E_UNSUPPORTED, "depth_attn: head dim %d unsupported", d);
  const int64_t h = (int64_t)H * d;
  hipStream_t st = S(stream);
  TB(DREAMER_KC_DEPTH_ATTN);
  int rc = launch_depth_attn(dtype, rows, H, d, l, L, q, h, k_new, h, v_new, h, k_cache,
                             v_cache, out, h, cos_d, sin_d, scale, 1, st, window, dilation);
  TE(DREAMER_KC_DEPTH_ATTN);
  if (rc) return fail(DREAMER_E_UNSUPPORTED, "depth_attn: head dim %d unsupported", d);
  return check_launch("depth_attn");
}

size_t dreamer_seq_attn_ws_bytes(int dtype, int B, int q_len, int H, int d, int64_t pos0) {
  return seq_attn_ws(dtype, B, q_len, H, d, pos0, 0);
}

static int validate_seq(int dtype, int B, int q_len, int H, int d, int64_t pos0, int64_t cap,
                        bool has_cache) {
  if (!dtype_ok(dtype)) return fail(DREAMER_E_INVAL, "seq_attn: bad dtype");
  if (B < 0 || q_len < 0 || H <= 0 || d <= 0 || pos0 < 0)
    return fail(DREAMER_E_INVAL, "seq_attn: bad sizes");
  const int vec = dtype == DREAMER_BF16 ? 8 : 4;
  if (d % (2 * vec) || (d / vec) > 16 || ((d / vec) & (d / vec - 1)))
    return fail(DREAMER_E_UNSUPPORTED, "seq_attn: head dim %d unsupported", d);
  if ((int64_t)H * d / vec > 1024) return fail(DREAMER_E_UNSUPPORTED, "seq_attn: hidden too large");
  if (pos0 > 0) {
    if (q_len != 1) return fail(DREAMER_E_UNSUPPORTED, "seq_attn: decode needs q_len == 1");
    if (!has_cache) return fail(DREAMER_E_INVAL, "seq_attn: decode needs k_cache/v_cache");
    if (cap <= pos0) return fail(DREAMER_E_INVAL, "seq_attn: cap must exceed pos0");
  } else if (has_cache && cap < q_len) {
    return fail(DREAMER_E_INVAL, "seq_attn: cap < q_len");
  }
  return ok();
}

int dreamer_seq_attn(int dtype, int B, int q_len, int H, int d, int64_t pos0, const void* q,
                     const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                     int64_t cap, void* out, const float* cos_s, const float* sin_s,
                     float scale, int sa_rope, void* ws, size_t ws_bytes,
                     dreamer_stream_t stream) {
  int rc = validate_seq(dtype, B, q_len, H, d, pos0, cap, k_cache && v_cache);
  if (rc) return rc;
  if (B == 0 || q_len == 0) return ok();
  if (!q || !k_new || !v_new || !out) return fail(DREAMER_E_INVAL, "seq_attn: null pointer");
  if (sa_rope && (!cos_s || !sin_s)) return fail(DREAMER_E_INVAL, "seq_attn: null rope table");
  const size_t need = seq_attn_ws(dtype, B, q_len, H, d, pos0, 0);
  if (ws_bytes < need || (need && !ws))
    return fail(DREAMER_E_WORKSPACE, "seq_attn: workspace %zu < %zu", ws_bytes, need);
  const int64_t h = (int64_t)H * d;
  hipStream_t st = S(stream);
  TB(DREAMER_KC_SEQ_ATTN);
  rc = launch_seq_attn(dtype, B, q_len, H, d, pos0, q, h, k_new, h, v_new, h, nullptr,
                       k_cache, v_cache, cap, out, h, cos_s, sin_s, scale, sa_rope, ws,
                       ws_bytes, st);
  TE(DREAMER_KC_SEQ_ATTN);
  if (rc) return fail(DREAMER_E_UNSUPPORTED, "seq_attn: unsupported shape (%d)", rc);
  return check_launch("seq_attn");
}

static int validate_route(int dtype, int64_t T, int h, int r, int E, int k, int l, int L) {
  if (!dtype_ok(dtype)) return fail(DREAMER_E_INVAL, "expert_route: bad dtype");
  if (T < 0 || h <= 0 || r <= 0 || E <= 0 || k <= 0 || L <= 0 || l < 0 || l >= L)
    return fail(DREAMER_E_INVAL, "expert_route: bad sizes");
  if (k > E || k > 32) return fail(DREAMER_E_UNSUPPORTED, "expert_route: k=%d (E=%d) unsupported", k, E);
  if (r % 8) return fail(DREAMER_E_UNSUPPORTED, "expert_route: r %% 8 != 0");
  if (E > 16384) return fail(DREAMER_E_UNSUPPORTED, "expert_route: E > 16384");
  if (dtype == DREAMER_BF16) {
    if (h % 64) return fail(DREAMER_E_UNSUPPORTED, "expert_route: h %% 64 != 0");
    if (r != 32 && r != 64 && r != 128 && r != 256)
      return fail(DREAMER_E_UNSUPPORTED, "expert_route: bf16 needs r in {32, 64, 128, 256}");
    if (E % 16) return fail(DREAMER_E_UNSUPPORTED, "expert_route: bf16 needs E %% 16 == 0");
  }
  return ok();
}

size_t dreamer_expert_route_ws_bytes(int64_t T, int r, int E) {
  if (T < 0 || r <= 0 || E <= 0) return 0;
  Bump b(nullptr);
  b.take_n<float>((size_t)T * r);
  b.take_n<float>((size_t)T * E);
  b.take_n<int32_t>((size_t)perm_blocks(T * 32) * E);  // count chunks for any k <= 32
  return b.off + 256;
}

// u = x W_r^T (f32), then the routing kernels (fused scores + selection when it applies).
static int route_impl(int dtype, int64_t T, int h, int r, int E, int k, int l, int L,
                      const void* x, int64_t ldx, const void* w_r, const void* keys,
                      const float* bias, float rho, int normalize, const float* cos_r,
                      const float* sin_r, int32_t* idx, float* gate, float* u, float* z,
                      hipStream_t st, const int32_t* idx_in = nullptr,
                      int32_t* hist = nullptr) {
  int rc;
  if (router_fused_ok(dtype, T, r, E, k)) {  // counts the permutation's histograms if hist
    TB(DREAMER_KC_ROUTE);
    rc = router_route_fused(T, h, r, E, k, l, L, x, ldx, w_r, keys, bias, rho, normalize,
                            cos_r, sin_r, idx_in, idx, gate, st, hist);
    TE(DREAMER_KC_ROUTE);
    if (rc) return fail(DREAMER_E_UNSUPPORTED, "expert_route: unsupported shape");
    return ok();
  }
  if (dtype == DREAMER_F32) {  // bf16 computes u inside the scores kernel
    GemmArgs ga;
    ga.M = (int)T;
    ga.N = r;
    ga.K = h;
    ga.A = x;
    ga.lda = ldx;
    ga.B = w_r;
    ga.ldb = h;
    ga.C = u;
    ga.ldc = r;
    TB(DREAMER_KC_GEMM);
    rc = launch_gemm(ga, dtype, 1, st);
    TE(DREAMER_KC_GEMM);
    if (rc) return fail(DREAMER_E_UNSUPPORTED, "router projection: unsupported shape");
  }
  TB(DREAMER_KC_ROUTE);
  rc = router_scores(dtype, T, h, r, E, l, L, x, ldx, w_r, u, keys, rho, cos_r, sin_r, z, st);
  if (!rc) rc = router_topk(T, E, k, z, bias, normalize, idx_in, idx, gate, st);
  TE(DREAMER_KC_ROUTE);
  if (rc) return fail(DREAMER_E_UNSUPPORTED, "expert_route: unsupported shape");
  return ok();
}

int dreamer_expert_route(int dtype, int64_t T, int h, int r, int E, int k, int l, int L,
                         const void* x, const void* w_r, const void* keys, const float* bias,
                         float rho, int normalize, const float* cos_r, const float* sin_r,
                         int32_t* idx, float* gate, int32_t* counts, void* ws,
                         size_t ws_bytes, dreamer_stream_t stream) {
  int rc = validate_route(dtype, T, h, r, E, k, l, L);
  if (rc) return rc;
  if (T == 0) return ok();
  if (!x || !w_r || !keys || !bias || !cos_r || !sin_r || !idx || !gate)
    return fail(DREAMER_E_INVAL, "expert_route: null pointer");
  const size_t need = dreamer_expert_route_ws_bytes(T, r, E);
  if (!ws || ws_bytes < need) return fail(DREAMER_E_WORKSPACE, "expert_route: workspace %zu < %zu", ws_bytes, need);
  hipStream_t st = S(stream);
  Bump b(ws);
  float* u = b.take_n<float>((size_t)T * r);
  float* z = b.take_n<float>((size_t)T * E);
  int32_t* hist = b.take_n<int32_t>((size_t)perm_blocks(T * 32) * E);
  rc = route_impl(dtype, T, h, r, E, k, l, L, x, h, w_r, keys, bias, rho, normalize, cos_r,
                  sin_r, idx, gate, u, z, st);
  if (rc) return rc;
  if (counts && launch_counts(idx, T * k, E, hist, counts, st))
    return fail(DREAMER_E_UNSUPPORTED, "expert_route: E too large for counts");
  return check_launch("expert_route");
}

// ------------------------------------------------------------------------ expert FFN
struct FfnWs {
  int32_t *counts, *goff, *toff, *hist, *perm;
  float* pgate;  // gates in expert-major order (tile-padded for the fused FFN)
  int4* tiles;   // m-tile descriptors
  void* slots;
};

static FfnWs plan_ffn(Bump& b, int dtype, int64_t T, int h_out, int E, int k) {
  FfnWs w;
  w.counts = b.take_n<int32_t>(E);
  w.goff = b.take_n<int32_t>(E + 1);
  w.toff = b.take_n<int32_t>(E + 1);
  w.hist = b.take_n<int32_t>((size_t)std::max(1, perm_blocks(T * k)) * E);
  // compact (grouped GEMM) or tile-padded (fused FFN) expert-major order
  const size_t npad = (size_t)tile_bound(T * k, E, FFN_TILE_M) * FFN_TILE_M;
  w.perm = b.take_n<int32_t>(npad);
  w.pgate = b.take_n<float>(npad);
  w.tiles = b.take_n<int4>((size_t)tile_bound(T * k, E, FFN_TILE_M));
  w.slots = b.take((size_t)T * k * h_out * esize(dtype));
  return w;
}

size_t dreamer_expert_ffn_ws_bytes(int dtype, int kind, int64_t T, int h_in, int f,
                                   int h_out, int E, int k) {
  (void)kind; (void)h_in; (void)f;
  if (T < 0 || E <= 0 || k <= 0 || h_out <= 0) return 0;
  Bump b(nullptr);
  plan_ffn(b, dtype, T, h_out, E, k);
  return b.off + 256;
}

// Routed slots for (idx, gate): slots[t*k+i] = gate * FFN_idx(x[t]).  bf16 groups the
// slots by expert first (histogram unless the counts are already there, scan, scatter).
static int ffn_slots(int dtype, int kind, int64_t T, int h_in, int f, int h_out, int E, int k,
                     const void* x, const int32_t* idx, const float* gate, const void* w1,
                     const void* w3, const void* w2, const FfnWs& w, hipStream_t st,
                     int32_t* hist_ready = nullptr, int32_t* zero_next = nullptr) {
  const int64_t ns = T * k;
  if (dtype == DREAMER_F32) {
    TB(DREAMER_KC_EXPERT_FFN);
    int rc = launch_expert_ffn_f32(kind, ns, k, h_in, f, h_out, (const float*)x, idx, gate,
                                   (const float*)w1, (const float*)w3, (const float*)w2,
                                   (float*)w.slots, st);
    TE(DREAMER_KC_EXPERT_FFN);
    return rc ? fail(DREAMER_E_UNSUPPORTED, "expert_ffn: f32 shape unsupported") : ok();
  }
  TB(DREAMER_KC_PERMUTE);
  const bool fused = kind != DREAMER_FFN_LINEAR;
  // hist_ready: the router has counted the chunk histograms into that buffer
  int prc = launch_permute(idx, ns, E, FFN_TILE_M, hist_ready ? hist_ready : w.hist, w.counts,
                           w.goff, w.toff, w.perm, st, fused ? gate : nullptr,
                           fused ? w.pgate : nullptr, fused ? w.tiles : nullptr, fused ? 1 : 0,
                           hist_ready != nullptr, zero_next);
  TE(DREAMER_KC_PERMUTE);
  if (prc) return fail(DREAMER_E_UNSUPPORTED, "expert_ffn: E too large for the permutation");
  int rc;
  if (kind == DREAMER_FFN_LINEAR) {
    GemmArgs ga;
    ga.M = (int)ns;
    ga.N = h_out;
    ga.K = h_in;
    ga.A = x;
    ga.lda = h_in;
    ga.B = w1;
    ga.ldb = h_in;
    ga.b_gstride = (int64_t)h_out * h_in;
    ga.rows = w.perm;
    ga.row_div = k;
    ga.row_scale = gate;
    ga.goff = w.goff;
    ga.toff = w.toff;
    ga.G = E;
    ga.tile_m = FFN_TILE_M;
    ga.C = w.slots;
    ga.ldc = h_out;
    TB(DREAMER_KC_EXPERT_FFN);
    rc = launch_gemm(ga, dtype, 0, st);
    TE(DREAMER_KC_EXPERT_FFN);
  } else {
    TB(DREAMER_KC_EXPERT_FFN);
    rc = launch_expert_ffn(dtype, kind, ns, k, h_in, f, h_out, E, x, w1, w3, w2, w.perm,
                           w.pgate, w.tiles, w.toff, w.slots, st);
    TE(DREAMER_KC_EXPERT_FFN);
  }
  return rc ? fail(DREAMER_E_UNSUPPORTED, "expert_ffn: shape unsupported (f=%d h_in=%d h_out=%d)",
                   f, h_in, h_out)
            : ok();
}

static int validate_ffn(int dtype, int kind, int64_t T, int h_in, int f, int h_out, int E,
                        int k) {
  if (!dtype_ok(dtype)) return fail(DREAMER_E_INVAL, "expert_ffn: bad dtype");
  if (kind < DREAMER_FFN_GELU || kind > DREAMER_FFN_LINEAR) return fail(DREAMER_E_INVAL, "expert_ffn: bad kind");
  if (T < 0 || h_in <= 0 || h_out <= 0 || E <= 0 || k <= 0 || (kind != DREAMER_FFN_LINEAR && f <= 0))
    return fail(DREAMER_E_INVAL, "expert_ffn: bad sizes");
  if (h_out > 4096) return fail(DREAMER_E_UNSUPPORTED, "expert_ffn: h_out > 4096");
  if (E > PERM_MAX_E) return fail(DREAMER_E_UNSUPPORTED, "expert_ffn: E > %d", PERM_MAX_E);
  if (T * k > INT32_MAX / 2) return fail(DREAMER_E_UNSUPPORTED, "expert_ffn: too many slots");
  if (dtype == DREAMER_BF16) {
    if (h_in % 64 || h_out % 64) return fail(DREAMER_E_UNSUPPORTED, "expert_ffn: bf16 needs h %% 64 == 0");
    if (kind != DREAMER_FFN_LINEAR && f != 64 && f != 128)
      return fail(DREAMER_E_UNSUPPORTED, "expert_ffn: bf16 needs f in {64, 128}");
  } else if (kind != DREAMER_FFN_LINEAR && f > 16384) {
    return fail(DREAMER_E_UNSUPPORTED, "expert_ffn: f too large");
  }
  return ok();
}

int dreamer_expert_ffn(int dtype, int kind, int64_t T, int h_in, int f, int h_out, int E,
                       int k, const void* x, const int32_t* idx, const float* gate,
                       const void* w1, const void* w3, const void* w2, const float* residual,
                       float* out, void* ws, size_t ws_bytes, dreamer_stream_t stream) {
  int rc = validate_ffn(dtype, kind, T, h_in, f, h_out, E, k);
  if (rc) return rc;
  if (T == 0) return ok();
  if (!x || !idx || !gate || !w1 || !out || (kind == DREAMER_FFN_SWIGLU && !w3) ||
      (kind != DREAMER_FFN_LINEAR && !w2))
    return fail(DREAMER_E_INVAL, "expert_ffn: null pointer");
  const size_t need = dreamer_expert_ffn_ws_bytes(dtype, kind, T, h_in, f, h_out, E, k);
  if (!ws || ws_bytes < need) return fail(DREAMER_E_WORKSPACE, "expert_ffn: workspace %zu < %zu", ws_bytes, need);
  hipStream_t st = S(stream);
  Bump b(ws);
  FfnWs w = plan_ffn(b, dtype, T, h_out, E, k);
  rc = ffn_slots(dtype, kind, T, h_in, f, h_out, E, k, x, idx, gate, w1, w3, w2, w, st);
  if (rc) return rc;
  TB(DREAMER_KC_COMBINE);
  launch_combine_norm(dtype, T, h_out, k, residual, w.slots, out, nullptr, nullptr, 0.f,
                      nullptr, nullptr, st);
  TE(DREAMER_KC_COMBINE);
  return check_launch("expert_ffn");
}

int dreamer_absorb_shared(int dtype, int64_t n_experts, int64_t n, const void* w_e,
                          const void* w_shared, void* out, dreamer_stream_t stream) {
  if (!dtype_ok(dtype) || n_experts < 0 || n < 0) return fail(DREAMER_E_INVAL, "absorb_shared: bad args");
  if (n_experts * n == 0) return ok();
  if (!w_e || !w_shared || !out) return fail(DREAMER_E_INVAL, "absorb_shared: null pointer");
  launch_absorb(dtype, n_experts, n, w_e, w_shared, out, S(stream));
  return check_launch("absorb_shared");
}

// ------------------------------------------------------------------------------ layer
struct LayerWs {
  float *cos_s, *sin_s, *cos_d, *sin_d, *cos_r, *sin_r;
  float4 *rope_s4, *rope_d4;  // interleaved head-dim-64 tables of the bf16 QKV epilogue
  void *xh, *qkv, *att, *yb;
  float* xh32;  // float32 copy of xhat for the residual (bf16 storage only)
  float *y, *u, *z, *rgate, *pgate, *zero_pbias;
  int32_t *ridx, *pidx;
  FfnWs ffn;
  int32_t* hist2;  // second chunk-histogram buffer (depths alternate; see layer_run)
  int32_t *pcounts, *pgoff, *ptoff, *phist, *pperm;
  void *da_k, *da_v, *sa_ws, *vt;
  size_t sa_ws_bytes;
  float* split_ws;  // decode: split-K partial products of the projections
  int64_t split_elems;
};

static int64_t sa_npos(const dreamer_layer_cfg* c) { return c->decode ? c->sa_pos + 1 : c->s; }

static LayerWs plan_layer(Bump& b, const dreamer_layer_cfg* c, bool need_yb, bool need_route,
                          bool need_proj_route, bool need_da) {
  LayerWs w{};
  const int64_t T = (int64_t)c->b * c->s;
  const size_t es = esize(c->dtype);
  const int64_t h = c->h;
  const int64_t npos = sa_npos(c);
  // rotary tables: the router's (depth, rank r); q / k rotate in the bf16 QKV epilogue
  // (interleaved tables) or in a float32 pass (split tables)
  w.cos_r = b.take_n<float>((size_t)c->L * (c->r / 2));
  w.sin_r = b.take_n<float>((size_t)c->L * (c->r / 2));
  if (c->dtype == DREAMER_BF16) {
    w.rope_s4 = b.take_n<float4>(npos * 16);
    w.rope_d4 = b.take_n<float4>((size_t)c->L * 16);
  } else {
    w.cos_s = b.take_n<float>(npos * (c->d / 2));
    w.sin_s = b.take_n<float>(npos * (c->d / 2));
    w.cos_d = b.take_n<float>((size_t)c->L * (c->d / 2));
    w.sin_d = b.take_n<float>((size_t)c->L * (c->d / 2));
  }
  w.xh = b.take(T * h * es);
  w.xh32 = c->dtype == DREAMER_BF16 ? b.take_n<float>(T * h) : nullptr;
  w.qkv = b.take(T * 6 * h * es);
  w.att = b.take(T * 2 * h * es);
  w.y = b.take_n<float>(T * h);
  w.yb = need_yb ? b.take(T * h * es) : nullptr;
  w.u = b.take_n<float>(T * c->r);
  if (c->use_ea) {
    if (need_route) {
      w.ridx = b.take_n<int32_t>(T * c->k);
      w.rgate = b.take_n<float>(T * c->k);
    }
    w.ffn = plan_ffn(b, c->dtype, T, c->h, c->E, c->k);
    w.hist2 = b.take_n<int32_t>((size_t)std::max(1, perm_blocks(T * c->k)) * c->E);
  }
  if (c->proj_experts) {
    const int Ep = c->proj_experts;
    if (need_proj_route) {
      w.pidx = b.take_n<int32_t>(T);
      w.pgate = b.take_n<float>(T);
    }
    w.zero_pbias = b.take_n<float>(Ep);
    w.pcounts = b.take_n<int32_t>(Ep);
    w.pgoff = b.take_n<int32_t>(Ep + 1);
    w.ptoff = b.take_n<int32_t>(Ep + 1);
    w.phist = b.take_n<int32_t>((size_t)perm_blocks(T) * Ep);
    w.pperm = b.take_n<int32_t>(T);
  }
  w.z = b.take_n<float>((size_t)T * std::max(c->use_ea ? c->E : 1, c->proj_experts));
  if (need_da) {
    w.da_k = b.take(T * c->L * h * es);
    w.da_v = b.take(T * c->L * h * es);
  }
  // bf16 prefill: q/k arrive rotated and v transposed from the QKV epilogue (not with the
  // grouped linear-MoE projections: their rows are in expert order, so the transposed v
  // would be written element by element; SA then transposes v in its own preparation pass)
  const bool vt_ok = c->dtype == DREAMER_BF16 && !c->decode && c->d == 64 && c->s % 8 == 0 &&
                     c->proj_experts == 0;
  w.vt = vt_ok ? b.take((size_t)T * h * es) : nullptr;
  // decode: the output projection of a few rows splits K over the CUs (up to 16 partial
  // products [T, h])
  if (c->decode && c->dtype == DREAMER_BF16) {
    w.split_elems = 16 * T * h;
    w.split_ws = b.take_n<float>((size_t)w.split_elems);
  }
  w.sa_ws_bytes = seq_attn_ws(c->dtype, c->b, c->s, c->H, c->d, c->decode ? c->sa_pos : 0,
                              vt_ok ? 1 : 0);
  w.sa_ws = w.sa_ws_bytes ? b.take(w.sa_ws_bytes) : nullptr;
  return w;
}

static int validate_layer(const dreamer_layer_cfg* c, const dreamer_layer_weights* w) {
  if (!c || !w) return fail(DREAMER_E_INVAL, "layer: null cfg or weights");
  if (!dtype_ok(c->dtype)) return fail(DREAMER_E_INVAL, "layer: bad dtype");
  if (c->b <= 0 || c->s <= 0 || c->h <= 0 || c->H <= 0 || c->d <= 0 || c->L <= 0 || c->r <= 0)
    return fail(DREAMER_E_INVAL, "layer: non-positive size");
  if ((int64_t)c->H * c->d != c->h) return fail(DREAMER_E_INVAL, "layer: h != H * d");
  if (c->mixture < DREAMER_MIX_PARTIAL || c->mixture > DREAMER_MIX_PARALLEL)
    return fail(DREAMER_E_INVAL, "layer: mixture %d", c->mixture);
  if (c->da_window < 0 || c->da_dilation < 0)
    return fail(DREAMER_E_INVAL, "layer: negative da_window (%d) or da_dilation (%d)",
                c->da_window, c->da_dilation);
  if (c->decode && (c->s != 1 || c->sa_pos <= 0 || c->sa_cap <= c->sa_pos))
    return fail(DREAMER_E_INVAL, "layer: decode needs s == 1, sa_pos > 0, sa_cap > sa_pos");
  if (!c->decode && c->sa_cap < 0) return fail(DREAMER_E_INVAL, "layer: bad sa_cap");
  if (c->h > 4096) return fail(DREAMER_E_UNSUPPORTED, "layer: h > 4096");
  if ((int64_t)c->b * c->s * 6 * c->h > INT32_MAX) return fail(DREAMER_E_UNSUPPORTED, "layer: T * 6h too large");
  if (c->r % 8) return fail(DREAMER_E_UNSUPPORTED, "layer: r %% 8 != 0");
  int rc = validate_seq(c->dtype, c->b, c->s, c->H, c->d, c->decode ? c->sa_pos : 0,
                        c->sa_cap, c->decode != 0);
  if (rc) return rc;
  if (c->use_ea) {
    rc = validate_route(c->dtype, (int64_t)c->b * c->s, c->h, c->r, c->E, c->k, 0, c->L);
    if (rc) return rc;

    if (c->ffn_kind != DREAMER_FFN_GELU && c->ffn_kind != DREAMER_FFN_SWIGLU)
      return fail(DREAMER_E_INVAL, "layer: ffn_kind must be GELU or SWIGLU");
    rc = validate_ffn(c->dtype, c->ffn_kind, (int64_t)c->b * c->s, c->h, c->f, c->h, c->E, c->k);
    if (rc) return rc;
    if (!w->w_r || !w->keys || !w->bias || !w->w1 || !w->w2 ||
        (c->ffn_kind == DREAMER_FFN_SWIGLU && !w->w3))
      return fail(DREAMER_E_INVAL, "layer: null expert weights");
  }
  if (c->proj_experts) {
    rc = validate_route(c->dtype, (int64_t)c->b * c->s, c->h, c->r, c->proj_experts, 1, 0, c->L);
    if (rc) return rc;
    if (!w->w_pr || !w->pkeys) return fail(DREAMER_E_INVAL, "layer: null projection router");
  }
  if (c->dtype == DREAMER_BF16 && (c->h % 128 || c->d != 64))
    return fail(DREAMER_E_UNSUPPORTED, "layer: bf16 needs head dim 64 and h %% 128 == 0");
  if (c->dtype == DREAMER_F32 && c->h % 8) return fail(DREAMER_E_UNSUPPORTED, "layer: h %% 8 != 0");
  if (!w->g || !w->w_qkv || !w->w_o) return fail(DREAMER_E_INVAL, "layer: null projection weights");
  if (!(c->rope_base > 0.0)) return fail(DREAMER_E_INVAL, "layer: rope_base must be > 0");
  return ok();
}

size_t dreamer_layer_ws_bytes(const dreamer_layer_cfg* cfg) {
  if (!cfg || cfg->b <= 0 || cfg->s <= 0 || cfg->h <= 0 || cfg->d <= 0 || cfg->L <= 0) return 0;
  Bump b(nullptr);
  plan_layer(b, cfg, true, true, true, true);
  return b.off + 256;
}

// The L depth steps of one call on a planned workspace.  table_npos > 0: build the rotary
// tables first (sequence table with table_npos positions); 0: they are already there.
static int layer_run(const dreamer_layer_cfg* cfg, const dreamer_layer_weights* w,
                     const LayerWs& lw, int64_t table_npos, const float* x_in, float* x_out,
                     int32_t* route_idx, float* route_gate, int32_t* proj_idx,
                     float* proj_gate, float* x_steps, void* y_steps, void* da_k, void* da_v,
                     void* sa_k, void* sa_v, const int32_t* route_in,
                     const int32_t* proj_route_in, hipStream_t st) {
  const dreamer_layer_cfg& c = *cfg;
  int rc = 0;
  const int dt = c.dtype;
  const size_t es = esize(dt);
  const int64_t T = (int64_t)c.b * c.s, h = c.h;
  const int L = c.L, k = c.k;
  const float scale = 1.0f / sqrtf((float)c.d);
  void* DAk = da_k ? da_k : lw.da_k;
  void* DAv = da_v ? da_v : lw.da_v;
  const int64_t cap = sa_k ? c.sa_cap : 0;
  const int64_t pos0 = c.decode ? c.sa_pos : 0;

  if (table_npos > 0) {  // rotary tables (and the zero projection bias), once per call
    RopeJobs jobs;
    jobs.base = c.rope_base;
    jobs.add_split(c.r, L, lw.cos_r, lw.sin_r);
    if (lw.rope_s4) {
      jobs.add_t4((int)table_npos, lw.rope_s4);
      jobs.add_t4(L, lw.rope_d4);
    } else {
      jobs.add_split(c.d, (int)table_npos, lw.cos_s, lw.sin_s);
      jobs.add_split(c.d, L, lw.cos_d, lw.sin_d);
    }
    launch_rope_jobs(jobs, st);
    if (c.proj_experts) launch_fill_i32((int32_t*)lw.zero_pbias, c.proj_experts, 0, st);
  }
  TB(DREAMER_KC_COMBINE);
  launch_rmsnorm(dt, T, c.h, x_in, w->g, c.rms_eps, lw.xh, lw.xh32, st);
  const float* resid = lw.xh32 ? lw.xh32 : (const float*)lw.xh;
  TE(DREAMER_KC_COMBINE);

  const bool serial = c.mixture == DREAMER_MIX_SERIAL;
  const bool parallel = c.mixture == DREAMER_MIX_PARALLEL;
  // With branch_streams, the fully parallel wiring runs its EA chain on a side stream beside
  // the attention (DA beside SA is not forked: at these sizes the cross-stream
  // synchronisation costs more than the overlap gains).
  // SA and DA in one launch where the flash grid alone would leave CUs idle in its tail:
  // its blocks (query blocks x heads x batch) fit the GPU at three per CU
  const bool pair_attn = c.fuse_attn && c.use_da && !serial && !sa_k && !c.decode &&
                         attn_pair_ok(dt, c.b, c.s, c.H, c.d, 0, lw.vt) &&
                         (int64_t)((c.s + 63) / 64) * c.H * c.b <= 3 * (int64_t)cu_count();
  // Larger flash grids (query blocks of 128 rows): SA and DA blocks interleaved in one
  // launch, so that every CU runs both (DA streams HBM while SA keeps the matrix cores
  // and the VALU busy)
  const bool pair2_attn = c.fuse_attn && c.use_da && !serial && !sa_k && !c.decode &&
                          !pair_attn && c.s > 64 &&
                          attn_pair_ok(dt, c.b, c.s, c.H, c.d, 0, lw.vt);
  // Otherwise, with branch_streams, DA (bound by memory bandwidth) runs on a side stream
  // beside SA (bound by the matrix cores and the vector ALU) in prefill: the two read
  // only the projections and write disjoint outputs.
  const bool da_side = c.branch_streams && c.use_da && !serial && !pair_attn && !pair2_attn &&
                       !c.decode;
  SideStreams* ss = nullptr;
  std::unique_lock<std::mutex> side_lock;
  if ((c.branch_streams && parallel && c.use_ea) || da_side) {
    ss = side_streams();
    if (!ss) return fail(DREAMER_E_HIP, "layer: side streams unavailable");
    side_lock = std::unique_lock<std::mutex>(ss->mu);  // the fork/join event is shared
  }
  hipStream_t sd_ea = (ss && parallel && c.use_ea) ? ss->s[0] : st;
  hipStream_t sd_da = da_side ? ss->s[1] : st;
  // the fused router (bf16) counts the permutation's histograms
  const bool fused_hist = c.use_ea && router_fused_ok(dt, T, c.r, c.E, k);
  if (fused_hist)
    launch_fill_i32(lw.ffn.hist, (int64_t)std::max(1, perm_blocks(T * k)) * c.E, 0, st);
  char* qkv = (char*)lw.qkv;
  char* att = (char*)lw.att;
  // The DA cache: the caller's [T, L, H, d] when given; the layer's own is slot-major
  // [L, T, h], so that a depth's slot is one contiguous block (the projection writes it
  // whole) -- the same values and the same DA reads either way.
  const int64_t da_srow = da_k ? (int64_t)L * h : (int64_t)h;
  const int64_t da_sslot = da_k ? (int64_t)h : (int64_t)T * h;

  for (int l = 0; l < L; ++l) {
    int32_t* pidx = nullptr;
    float* pgate = nullptr;
    if (c.proj_experts) {  // top-1 projection router shared by every Q/K/V/O projection
      const int Ep = c.proj_experts;
      pidx = proj_idx ? proj_idx + (int64_t)l * T : lw.pidx;
      pgate = proj_gate ? proj_gate + (int64_t)l * T : lw.pgate;
      rc = route_impl(dt, T, c.h, c.r, Ep, 1, l, L, lw.xh, h, w->w_pr, w->pkeys,
                      w->pbias ? w->pbias : lw.zero_pbias, c.rho, 0, lw.cos_r, lw.sin_r, pidx,
                      pgate, lw.u, lw.z, st,
                      proj_route_in ? proj_route_in + (int64_t)l * T : nullptr);
      if (rc) return rc;
      TB(DREAMER_KC_PERMUTE);
      rc = launch_permute(pidx, T, Ep, PROJ_TILE_M, lw.phist, lw.pcounts, lw.pgoff, lw.ptoff, lw.pperm,
                          st);
      TE(DREAMER_KC_PERMUTE);
      if (rc) return fail(DREAMER_E_UNSUPPORTED, "layer: projection permutation");
    }
    const bool last = l == L - 1;
    // bf16: DA's k / v of this depth are written by the QKV projection straight into the
    // cache's slot l, where DA reads them with the older slots
    const bool kv_bf = dt == DREAMER_BF16 && c.use_da;
    void* dak_l = kv_bf ? (char*)DAk + (size_t)l * da_sslot * es : nullptr;
    void* dav_l = kv_bf ? (char*)DAv + (size_t)l * da_sslot * es : nullptr;
    // the storage copy of y feeds the router (PARTIAL, SERIAL); the fully parallel wiring's
    // router reads xh, so no copy of y is stored there
    void* y_out = y_steps ? (char*)y_steps + (size_t)l * T * h * es : nullptr;
    void* yb = parallel ? nullptr : (y_out ? y_out : lw.yb);
    int32_t* ridx = nullptr;
    float* rgate = nullptr;
    if (c.use_ea) {
      ridx = route_idx ? route_idx + (size_t)l * T * k : lw.ridx;
      rgate = route_gate ? route_gate + (size_t)l * T * k : lw.rgate;
    }
    // EA on `in` (storage dtype), leaving the gate-scaled expert outputs in the slots
    // With the fused router the permutation's chunk histograms are counted during the
    // selection, into the buffer of this depth's parity; the scatter then clears the
    // other buffer for the next depth (the first was cleared before depth 0).
    auto ea = [&](const void* in, hipStream_t es_) -> int {
      int32_t* hcur = fused_hist ? ((l & 1) ? lw.hist2 : lw.ffn.hist) : nullptr;
      int32_t* hnext = fused_hist ? ((l & 1) ? lw.ffn.hist : lw.hist2) : nullptr;
      int r2 = route_impl(dt, T, c.h, c.r, c.E, k, l, L, in, h, w->w_r, w->keys, w->bias,
                          c.rho, c.normalize_gates, lw.cos_r, lw.sin_r, ridx, rgate, lw.u,
                          lw.z, es_, route_in ? route_in + (size_t)l * T * k : nullptr, hcur);
      if (r2) return r2;
      return ffn_slots(dt, c.ffn_kind, T, c.h, c.f, c.h, c.E, k, in, ridx, rgate, w->w1,
                       w->w3, w->w2, lw.ffn, es_, hcur, hnext);
    };
    // Q/K/V projection of sections [sect0, sect0 + nsect) from `in` into qkv
    auto project_qkv = [&](const void* in, int sect0, int nsect) -> int {
      GemmArgs gq;
      gq.M = (int)T;
      gq.N = nsect * (int)h;
      gq.K = (int)h;
      gq.A = in;
      gq.lda = h;
      gq.B = (const char*)w->w_qkv + (size_t)sect0 * h * h * es;
      gq.ldb = h;
      gq.C = qkv + (size_t)sect0 * h * es;
      gq.ldc = 6 * h;
      if (c.proj_experts) {
        gq.b_gstride = 6 * h * h;
        gq.rows = lw.pperm;
        gq.row_scale = pgate;
        gq.goff = lw.pgoff;
        gq.toff = lw.ptoff;
        gq.G = c.proj_experts;
        gq.tile_m = PROJ_TILE_M;
      }
      // q/k leave the projection rotated (SA by position, DA by depth) and rounded once
      if (dt == DREAMER_BF16) {
        gq.qkv_h = (int)h;
        gq.qkv_sect0 = sect0;
        gq.seq = c.s;
        gq.pos_fixed = c.decode ? (int)c.sa_pos : -1;
        gq.sa_rope = c.sa_rope;
        gq.depth_l = l;
        gq.depth_L = L;
        gq.rope_s4 = lw.rope_s4;
        gq.rope_d4 = lw.rope_d4;
        gq.vt = lw.vt;
        // the paired attention launches read SA v transposed only
        gq.vt_only = pair_attn || pair2_attn;
        // DA k / v go straight into the cache's slot l, where DA reads them
        gq.da_k = dak_l;
        gq.da_v = dav_l;
        gq.da_ld = da_srow;
      }
      TB(DREAMER_KC_GEMM);
      int r2 = launch_gemm(gq, dt, 0, st);
      TE(DREAMER_KC_GEMM);
      if (r2) return fail(DREAMER_E_UNSUPPORTED, "layer: QKV projection shape");
      if (dt == DREAMER_F32) {  // rotates every section of the buffer in place
        r2 = launch_qkv_rope(dt, T, c.H, c.d, c.s, c.decode ? (int)c.sa_pos : -1, c.sa_rope,
                             l, L, lw.qkv, lw.cos_s, lw.sin_s, lw.cos_d, lw.sin_d, st);
        if (r2) return fail(DREAMER_E_UNSUPPORTED, "layer: head dim for RoPE");
      }
      return ok();
    };
    auto run_sa = [&]() -> int {
      void* sk = sa_k ? (char*)sa_k + (size_t)l * c.b * cap * h * es : nullptr;
      void* sv = sa_v ? (char*)sa_v + (size_t)l * c.b * cap * h * es : nullptr;
      TB(DREAMER_KC_SEQ_ATTN);
      int r2 = launch_seq_attn(dt, c.b, c.s, c.H, c.d, pos0, qkv, 6 * h, qkv + h * es, 6 * h,
                               qkv + 2 * h * es, 6 * h, lw.vt, sk, sv, cap, att, 2 * h,
                               lw.cos_s, lw.sin_s, scale, 0, lw.sa_ws, lw.sa_ws_bytes, st);
      TE(DREAMER_KC_SEQ_ATTN);
      return r2 ? fail(DREAMER_E_UNSUPPORTED, "layer: sequence attention shape (%d)", r2)
                : ok();
    };
    auto run_da = [&](hipStream_t s_) -> int {
      timing_begin(DREAMER_KC_DEPTH_ATTN, s_);
      int r2 = launch_depth_attn(dt, T, c.H, c.d, l, L, qkv + 3 * h * es, 6 * h,
                                 kv_bf ? dak_l : qkv + 4 * h * es, kv_bf ? da_srow : 6 * h,
                                 kv_bf ? dav_l : qkv + 5 * h * es, kv_bf ? da_srow : 6 * h,
                                 DAk, DAv,
                                 att + h * es, 2 * h, lw.cos_d, lw.sin_d, scale, 0, s_,
                                 c.da_window, c.da_dilation, da_srow, da_sslot);
      timing_end(DREAMER_KC_DEPTH_ATTN, s_);  // s_: the stream DA runs on
      return r2 ? fail(DREAMER_E_UNSUPPORTED, "layer: depth attention shape") : ok();
    };
    // out = res + a W_o^T over attention columns [col0, col0 + K) (f32, plus a copy in
    // storage dtype, C2)
    auto project_o = [&](int col0, int K, const float* res, void* C2) -> int {
      GemmArgs go;
      go.M = (int)T;
      go.N = (int)h;
      go.K = K;
      go.A = att + (size_t)col0 * es;
      go.lda = 2 * h;
      go.B = (const char*)w->w_o + (size_t)col0 * es;
      go.ldb = 2 * h;
      go.C = lw.y;
      go.ldc = h;
      go.resid = res;
      go.ldr = h;
      go.C2 = C2;
      go.ldc2 = h;
      go.split_ws = lw.split_ws;
      go.split_elems = lw.split_elems;
      if (c.proj_experts) {
        go.b_gstride = 2 * h * h;
        go.rows = lw.pperm;
        go.row_scale = pgate;
        go.goff = lw.pgoff;
        go.toff = lw.ptoff;
        go.G = c.proj_experts;
        go.tile_m = PROJ_TILE_M;
      }
      TB(DREAMER_KC_OUT_PROJ);
      int r2 = launch_gemm(go, dt, 1, st);
      TE(DREAMER_KC_OUT_PROJ);
      return r2 ? fail(DREAMER_E_UNSUPPORTED, "layer: output projection shape") : ok();
    };

    if (parallel && c.use_ea) {  // EA reads xh: it starts with the step
      if (ss) side_fork(ss, st, sd_ea);
      if ((rc = ea(lw.xh, sd_ea))) return rc;
    }
    if (serial) {
      // u = xh + DA(xh) into y (f32) and its storage copy into xh; then v = u + SA(u)
      const float* res = resid;
      if (c.use_da) {
        if ((rc = project_qkv(lw.xh, 3, 3)) || (rc = run_da(st)) ||
            (rc = project_o((int)h, (int)h, resid, lw.xh)))
          return rc;
        res = lw.y;
      }
      if ((rc = project_qkv(lw.xh, 0, 3)) || (rc = run_sa()) ||
          (rc = project_o(0, (int)h, res, yb)))
        return rc;
    } else {
      // y = xh + [a_SA | a_DA] W_o^T
      if ((rc = project_qkv(lw.xh, 0, c.use_da ? 6 : 3))) return rc;
      if (pair_attn) {
        TB(DREAMER_KC_ATTN);
        int r2 = launch_attn_pair(c.b, c.s, c.H, l, L, qkv, qkv + h * es, lw.vt,
                                  qkv + 3 * h * es, dak_l, dav_l, 6 * h, da_srow, da_srow,
                                  da_sslot,
                                  DAk, DAv, att, att + h * es, 2 * h, scale, c.da_window,
                                  c.da_dilation, st);
        TE(DREAMER_KC_ATTN);
        if (r2) return fail(DREAMER_E_UNSUPPORTED, "layer: paired attention shape");
      } else if (pair2_attn) {
        TB(DREAMER_KC_ATTN);
        int r2 = launch_attn_pair2(c.b, c.s, c.H, l, L, qkv, qkv + h * es, lw.vt,
                                   qkv + 3 * h * es, dak_l, dav_l, 6 * h, da_srow, da_srow,
                                   da_sslot,
                                   DAk, DAv, att, att + h * es, 2 * h, scale, c.da_window,
                                   c.da_dilation, st);
        TE(DREAMER_KC_ATTN);
        if (r2) return fail(DREAMER_E_UNSUPPORTED, "layer: paired attention shape");
      } else if (da_side) {
        side_fork(ss, st, sd_da);  // after the projection
        if ((rc = run_da(sd_da))) return rc;
        if ((rc = run_sa())) return rc;
        side_join(ss, st, sd_da);  // before the output projection
      } else {
        if ((rc = run_sa())) return rc;
        if (c.use_da && (rc = run_da(st))) return rc;
      }
      if ((rc = project_o(0, c.use_da ? 2 * (int)h : (int)h, resid, yb))) return rc;
    }
    if (c.use_ea) {
      if (parallel) {
        if (ss) side_join(ss, st, sd_ea);
      }
      else if ((rc = ea(yb, st))) return rc;
    }
    if (parallel && y_out &&  // the router input of this step (xh) before it is replaced
        hipMemcpyAsync(y_out, lw.xh, (size_t)T * h * es, hipMemcpyDeviceToDevice, st) !=
            hipSuccess)
      return fail(DREAMER_E_HIP, "layer: copy of the router input");
    // x_{l+1} = y + sum of the slots; the next step's RMSNorm
    float* xs = x_steps ? x_steps + (size_t)l * T * h : nullptr;
    TB(DREAMER_KC_COMBINE);
    launch_combine_norm(dt, T, c.h, c.use_ea ? k : 0, lw.y, c.use_ea ? lw.ffn.slots : nullptr,
                        last ? x_out : nullptr, xs, w->g, c.rms_eps, last ? nullptr : lw.xh,
                        last ? nullptr : lw.xh32, st);
    TE(DREAMER_KC_COMBINE);
  }
  return ok();
}

int dreamer_layer_forward(const dreamer_layer_cfg* cfg, const dreamer_layer_weights* w,
                          const float* x_in, float* x_out, int32_t* route_idx,
                          float* route_gate, int32_t* proj_idx, float* proj_gate,
                          float* x_steps, void* y_steps, void* da_k, void* da_v, void* sa_k,
                          void* sa_v, const int32_t* route_in, const int32_t* proj_route_in,
                          void* ws, size_t ws_bytes, dreamer_stream_t stream) {
  int rc = validate_layer(cfg, w);
  if (rc) return rc;
  const dreamer_layer_cfg& c = *cfg;
  if (!x_in || !x_out) return fail(DREAMER_E_INVAL, "layer: null x_in / x_out");
  if (c.decode && (!sa_k || !sa_v)) return fail(DREAMER_E_INVAL, "layer: decode needs sa_k / sa_v");
  if ((da_k == nullptr) != (da_v == nullptr)) return fail(DREAMER_E_INVAL, "layer: da_k / da_v must both be given");
  if ((sa_k == nullptr) != (sa_v == nullptr)) return fail(DREAMER_E_INVAL, "layer: sa_k / sa_v must both be given");
  if ((route_idx == nullptr) != (route_gate == nullptr) ||
      (proj_idx == nullptr) != (proj_gate == nullptr))
    return fail(DREAMER_E_INVAL, "layer: routing outputs must come in (idx, gate) pairs");
  if (sa_k && !c.decode && c.sa_cap < c.s) return fail(DREAMER_E_INVAL, "layer: sa_cap < s");
  const size_t need = dreamer_layer_ws_bytes(cfg);
  if (!ws || ws_bytes < need) return fail(DREAMER_E_WORKSPACE, "layer: workspace %zu < %zu", ws_bytes, need);

  Bump b(ws);
  LayerWs lw = plan_layer(b, cfg, y_steps == nullptr, route_idx == nullptr,
                          proj_idx == nullptr, da_k == nullptr);
  rc = layer_run(cfg, w, lw, sa_npos(cfg), x_in, x_out, route_idx, route_gate, proj_idx,
                 proj_gate, x_steps, y_steps, da_k, da_v, sa_k, sa_v, route_in, proj_route_in,
                 S(stream));
  if (rc) return rc;
  return check_launch("layer_forward");
}

// ------------------------------------------------------------ expert-load bookkeeping
int dreamer_route_counts(const int32_t* idx, int64_t n_sets, int64_t per_set, int E,
                         int32_t* counts, dreamer_stream_t stream) {
  if (n_sets <= 0 || per_set < 0 || E <= 0 || !counts || (per_set > 0 && !idx))
    return fail(DREAMER_E_INVAL, "route_counts: bad arguments");
  if (E > COUNT_MAX_E || n_sets > 65535)
    return fail(DREAMER_E_UNSUPPORTED, "route_counts: E > %d or more than 65535 sets", COUNT_MAX_E);
  if (launch_route_counts(idx, n_sets, per_set, E, counts, S(stream)))
    return fail(DREAMER_E_UNSUPPORTED, "route_counts: unsupported shape");
  return check_launch("route_counts");
}

int dreamer_bias_update(const int32_t* counts, int E, float lambda, float* bias,
                        dreamer_stream_t stream) {
  if (E <= 0 || !counts || !bias) return fail(DREAMER_E_INVAL, "bias_update: bad arguments");
  launch_bias_update(counts, E, lambda, bias, S(stream));
  return check_launch("bias_update");
}

int dreamer_expert_usage(const int32_t* counts, int64_t n_sets, int E, float* stats,
                         dreamer_stream_t stream) {
  if (n_sets <= 0 || E <= 0 || !counts || !stats)
    return fail(DREAMER_E_INVAL, "expert_usage: bad arguments");
  if (launch_expert_usage(counts, n_sets, E, stats, S(stream)))
    return fail(DREAMER_E_UNSUPPORTED, "expert_usage: E > %d or more than 65535 sets", PERM_MAX_E);
  return check_launch("expert_usage");
}

// Multi-token decode: n_tokens consecutive decode steps; token j sits at position
// sa_pos + j, appends its keys / values to the SA caches and overwrites the DA slots.  The
// workspace is planned for the last token's position (every buffer covers the earlier
// ones) and the rotary tables are built once.
static dreamer_layer_cfg last_token_cfg(const dreamer_layer_cfg* cfg, int n_tokens) {
  dreamer_layer_cfg m = *cfg;
  m.sa_pos = cfg->sa_pos + n_tokens - 1;
  return m;
}

size_t dreamer_decode_ws_bytes(const dreamer_layer_cfg* cfg, int n_tokens) {
  if (!cfg || n_tokens <= 0) return 0;
  const dreamer_layer_cfg m = last_token_cfg(cfg, n_tokens);
  return dreamer_layer_ws_bytes(&m);
}

int dreamer_decode_tokens(const dreamer_layer_cfg* cfg, const dreamer_layer_weights* w,
                          int n_tokens, const float* x_in, float* x_out, int32_t* route_idx,
                          float* route_gate, void* da_k, void* da_v, void* sa_k, void* sa_v,
                          void* ws, size_t ws_bytes, dreamer_stream_t stream) {
  if (!cfg || n_tokens <= 0) return fail(DREAMER_E_INVAL, "decode_tokens: null cfg or n_tokens <= 0");
  if (!cfg->decode) return fail(DREAMER_E_INVAL, "decode_tokens: cfg.decode must be 1");
  const dreamer_layer_cfg m = last_token_cfg(cfg, n_tokens);
  int rc = validate_layer(cfg, w);
  if (rc) return rc;
  if ((rc = validate_layer(&m, w))) return rc;  // sa_cap covers the last position
  if (!x_in || !x_out || !sa_k || !sa_v) return fail(DREAMER_E_INVAL, "decode_tokens: null x_in / x_out / SA caches");
  if ((da_k == nullptr) != (da_v == nullptr)) return fail(DREAMER_E_INVAL, "decode_tokens: da_k / da_v must both be given");
  if ((route_idx == nullptr) != (route_gate == nullptr))
    return fail(DREAMER_E_INVAL, "decode_tokens: route_idx / route_gate must both be given");
  const size_t need = dreamer_decode_ws_bytes(cfg, n_tokens);
  if (!ws || ws_bytes < need) return fail(DREAMER_E_WORKSPACE, "decode_tokens: workspace %zu < %zu", ws_bytes, need);
  Bump b(ws);
  LayerWs lw = plan_layer(b, &m, true, route_idx == nullptr, true, da_k == nullptr);
  const int64_t bh = (int64_t)cfg->b * cfg->h, blk = (int64_t)cfg->L * cfg->b * cfg->k;
  for (int j = 0; j < n_tokens; ++j) {
    dreamer_layer_cfg cj = *cfg;
    cj.sa_pos = cfg->sa_pos + j;
    rc = layer_run(&cj, w, lw, j == 0 ? sa_npos(&m) : 0, x_in + j * bh, x_out + j * bh,
                   route_idx ? route_idx + j * blk : nullptr,
                   route_gate ? route_gate + j * blk : nullptr, nullptr, nullptr, nullptr,
                   nullptr, da_k, da_v, sa_k, sa_v, nullptr, nullptr, S(stream));
    if (rc) return rc;
  }
  return check_launch("decode_tokens");
}

}  // extern "C"
