// dreamer_ref.cpp -- CPU oracle of one Dreamer depth-recurrent attention-mixture layer
// (arXiv 2601.21582), forward pass.  TEST INFRASTRUCTURE ONLY (see dreamer_ref.h).
//
// Plain float64 C++17, written from the method description in the pages' order:
// RMSNorm of the stream -> SA and DA on the normalised stream -> parallel residual ->
// EA (router, then the selected tiny experts).  No blocking, no fusion, no reordering:
// every matrix product is a row-by-row dot product, every softmax is max / exp / sum /
// divide, every top-k is a stable sort.  OpenMP only splits independent rows (or
// (row, output) pairs) between threads; each value is computed by one thread in a fixed
// order, so the thread count never changes a result.
//
// Pages cited by section (all describe arXiv 2601.21582):
//   [PN]    papernotes.org paper notes: "Method / overall framework" (loop flowchart,
//           DA-cache remark), "Key design 1" (depth attention, depth RoPE with half the
//           dims reversed, parallel-residual equation y = x_l + DA(x_{:l}) + SA(x_l)),
//           "Key design 2" (expert attention, gate equation
//           sigma = norm(TopK(sigmoid(x), x + b, k)), bias update), "Key design 3"
//           (linear-MoE projections, shared-expert identity), "Loss / training" (RMSNorm
//           on the residual stream), ablation table (mixture wirings), analysis of expert
//           usage, "Limitations and outlook" (windowed / dilated depth attention).
//   [GS-de] gist.science German technical summary, "Methodik: Dreamer-Framework".
//
// Readings where the pages leave a step open (each is named where it is used):
//   R1  DA keys are the depths 0..l, inclusive of the current one.
//   R2  one RMSNorm per step, on the stream itself, at the loop head; x_hat is both the
//       attention input and the residual.  R3: eps inside the root, gain g.
//   R4  depth RoPE: rotary pairs i < D/4 at depth l, pairs i >= D/4 at L-1-l (the
//       reversed half), same theta ladder, on q and k alike (router: on the query only).
//   R5  SA uses plain RoPE over token positions.  R6: scale 1/sqrt(d); separate SA and
//       DA projections; no biases.
//   R7  EA reads y (no second norm).  R8: router u = RoPE_depth(y W_r), z = rho u.keys.
//   R10 experts are ranked by z + b, gate values are sigmoid(z), ties go to the lower
//       index, output in descending order.  R11: "norm" divides by the sum of the k gates.
//   R12 the shared expert lives only in the linear-MoE projections; for top-1,
//       max(sigma_hat) = sigma; projection gate = raw sigmoid; one projection router per
//       token and depth, on x_hat, bias 0.
//   R13 GELU is the erf form; SwiGLU = W2 (silu(W1 x) * (W3 x)).
//   R14 decode: the SA cache is per depth, holds rotated keys, the new token is appended
//       at sa_pos.
//   R20 the residual keeps x_hat unrounded; the projections read its storage copy.
//   R21 q and k are rotated from the unrounded projection and stored once, rotated.
//   R22 serial and fully parallel wirings: see dreamer_ref.h.
//   R26 windowed / dilated depth attention key sets: see dreamer_ref_depth_keys.

#include "dreamer_ref.h"

#include <omp.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <numeric>
#include <vector>

namespace {

using ::int64_t;
using vec = std::vector<double>;

// ------------------------------------------------------------------------ rounding

// Nearest bfloat16 (ties to even), through float32 (also ties to even).
double bf16_round(double v) {
  float f = static_cast<float>(v);
  if (std::isnan(f)) return v;
  uint32_t u;
  std::memcpy(&u, &f, 4);
  uint64_t w = u;
  w = (w + 0x7FFFu + ((w >> 16) & 1u)) & 0xFFFF0000u;
  u = static_cast<uint32_t>(w);
  std::memcpy(&f, &u, 4);
  return static_cast<double>(f);
}

// A storage point: rounds to bfloat16 when the storage emulation is on.
void store(bool bf16, double* a, int64_t n) {
  if (!bf16) return;
  for (int64_t i = 0; i < n; ++i) a[i] = bf16_round(a[i]);
}

// ------------------------------------------------------------------ small algebra

template <class WT>
double dot(const double* x, const WT* w, int64_t n) {
  double acc = 0.0;
#pragma omp simd reduction(+ : acc)
  for (int64_t p = 0; p < n; ++p) acc += x[p] * static_cast<double>(w[p]);
  return acc;
}

// Y[t, j] = sum_p X[t, p] W[j, p]   (W stored [N, K]: y = x W^T)
template <class WT>
void linear(const double* X, int64_t T, int64_t K, const WT* W, int64_t N, double* Y) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < N; ++j) Y[t * N + j] = dot(X + t * K, W + j * K, K);
}

double sigmoid(double x) { return 1.0 / (1.0 + std::exp(-x)); }
double silu(double x) { return x * sigmoid(x); }
double gelu(double x) { return 0.5 * x * (1.0 + std::erf(x / std::sqrt(2.0))); }

// --------------------------------------------------------------------------- RoPE

// One vector of length D, rotary pairs (i, i + D/2) with theta_i = base^(-2i/D) and a
// position per pair.  out may alias u.
void rope_vec(const double* u, const double* pos, int D, double base, double* out) {
  const int half = D / 2;
  for (int i = 0; i < half; ++i) {
    const double theta = std::pow(base, -2.0 * i / D);
    const double ang = pos[i] * theta;
    const double c = std::cos(ang), s = std::sin(ang);
    const double a = u[i], b = u[i + half];
    out[i] = a * c - b * s;
    out[i + half] = b * c + a * s;
  }
}

// R4: pairs i < D/4 sit at depth l, the others at L-1-l ([PN] "Key design 1").
vec depth_positions(int l, int L, int D) {
  vec pos(D / 2);
  for (int i = 0; i < D / 2; ++i) pos[i] = (i < D / 4) ? double(l) : double(L - 1 - l);
  return pos;
}

void depth_rope_rows(const double* u, int64_t n, int D, int l, int L, double base,
                     double* out) {
  const vec pos = depth_positions(l, L, D);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) rope_vec(u + t * D, pos.data(), D, base, out + t * D);
}

// R26 ([PN] "Limitations and outlook"): window <= 0 -> every depth 0..l (R1).
std::vector<int> depth_keys(int l, int window, int dilation) {
  std::vector<int> keys;
  for (int j = 0; j <= l; ++j) {
    if (window <= 0 || l - j < window || (dilation > 0 && (l - j) % dilation == 0))
      keys.push_back(j);
  }
  return keys;
}

// ------------------------------------------------------------------------ softmax

// p_j = exp(s_j - max) / sum_i exp(s_i - max), in place.
void softmax(double* s, int n) {
  double m = -std::numeric_limits<double>::infinity();
  for (int j = 0; j < n; ++j) m = std::max(m, s[j]);
  double sum = 0.0;
  for (int j = 0; j < n; ++j) {
    s[j] = std::exp(s[j] - m);
    sum += s[j];
  }
  for (int j = 0; j < n; ++j) s[j] = s[j] / sum;
}

// ------------------------------------------------------------- sequence attention

// Causal SA ([PN] parallel-residual equation, SA(x_l); [GS-de] standard self-attention
// along the tokens).  R5: plain RoPE at positions pos0 + i; R6: scale 1/sqrt(d).
template <class CT>
void seq_attn(int B, int n, int H, int d, int64_t pos0, const double* q, const double* k_new,
              const double* v_new, const CT* k_cache, const CT* v_cache, int64_t cap,
              bool sa_rope, double base, bool bf16, double* out, double* k_rot,
              double* v_out) {
  const int64_t hd = int64_t(H) * d;
  const int64_t N = int64_t(B) * n * hd;
  vec qr(q, q + N);
  std::memcpy(k_rot, k_new, sizeof(double) * N);
  std::memcpy(v_out, v_new, sizeof(double) * N);
  if (sa_rope) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
      for (int i = 0; i < n; ++i) {
        const vec pos(d / 2, double(pos0 + i));
        for (int hh = 0; hh < H; ++hh) {
          const int64_t o = (int64_t(b) * n + i) * hd + int64_t(hh) * d;
          rope_vec(qr.data() + o, pos.data(), d, base, qr.data() + o);
          rope_vec(k_rot + o, pos.data(), d, base, k_rot + o);
        }
      }
    store(bf16, qr.data(), N);
    store(bf16, k_rot, N);
  }
#pragma omp parallel for collapse(3) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int hh = 0; hh < H; ++hh)
      for (int i = 0; i < n; ++i) {
        const int64_t nk = pos0 + i + 1;  // keys 0..pos0+i (causal)
        vec s(nk);
        const double* qv = qr.data() + (int64_t(b) * n + i) * hd + int64_t(hh) * d;
        auto key = [&](int64_t j, int c) -> double {
          if (j < pos0) return double(k_cache[((int64_t(b) * cap + j) * H + hh) * d + c]);
          return k_rot[(int64_t(b) * n + (j - pos0)) * hd + int64_t(hh) * d + c];
        };
        auto val = [&](int64_t j, int c) -> double {
          if (j < pos0) return double(v_cache[((int64_t(b) * cap + j) * H + hh) * d + c]);
          return v_out[(int64_t(b) * n + (j - pos0)) * hd + int64_t(hh) * d + c];
        };
        for (int64_t j = 0; j < nk; ++j) {
          double acc = 0.0;
          for (int c = 0; c < d; ++c) acc += qv[c] * key(j, c);
          s[j] = acc / std::sqrt(double(d));
        }
        softmax(s.data(), int(nk));
        double* o = out + (int64_t(b) * n + i) * hd + int64_t(hh) * d;
        for (int c = 0; c < d; ++c) {
          double acc = 0.0;
          for (int64_t j = 0; j < nk; ++j) acc += s[j] * val(j, c);
          o[c] = acc;
        }
      }
  store(bf16, out, N);
}

// ---------------------------------------------------------------- depth attention

// DA at depth l ([PN] "Key design 1"; [GS-de] DA: every token attends over its own
// activations at earlier depths, the depth axis taking the place of the sequence axis).
// R1: the key set includes depth l; R4: depth RoPE on q and the new key; the rotated key
// and the value go into slot l before the attention reads the key set (R26).
void depth_attn(int64_t R, int H, int d, int l, int L, const double* q, const double* k_new,
                const double* v_new, double* k_cache, double* v_cache, double base, bool bf16,
                bool use_rope, int window, int dilation, double* out) {
  const int64_t hd = int64_t(H) * d;
  const int64_t N = R * hd;
  vec qr(q, q + N), kr(k_new, k_new + N);
  if (use_rope) {
    depth_rope_rows(qr.data(), R * H, d, l, L, base, qr.data());
    depth_rope_rows(kr.data(), R * H, d, l, L, base, kr.data());
    store(bf16, qr.data(), N);
    store(bf16, kr.data(), N);
  }
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    std::memcpy(k_cache + (r * L + l) * hd, kr.data() + r * hd, sizeof(double) * hd);
    std::memcpy(v_cache + (r * L + l) * hd, v_new + r * hd, sizeof(double) * hd);
  }
  const std::vector<int> keys = depth_keys(l, window, dilation);
  const int nk = int(keys.size());
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t r = 0; r < R; ++r)
    for (int hh = 0; hh < H; ++hh) {
      const double* qv = qr.data() + r * hd + int64_t(hh) * d;
      vec s(nk);
      for (int j = 0; j < nk; ++j) {
        const double* kv = k_cache + (r * L + keys[j]) * hd + int64_t(hh) * d;
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += qv[c] * kv[c];
        s[j] = acc / std::sqrt(double(d));
      }
      softmax(s.data(), nk);
      double* o = out + r * hd + int64_t(hh) * d;
      for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int j = 0; j < nk; ++j) acc += s[j] * v_cache[(r * L + keys[j]) * hd + hh * d + c];
        o[c] = acc;
      }
    }
  store(bf16, out, N);
}

// ------------------------------------------------------------------------ routing

// R10: descending by key, equal keys in index order (stable sort), first k.
void topk_row(const double* key, int E, int k, int64_t* idx) {
  std::vector<int> order(E);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return key[a] > key[b]; });
  for (int i = 0; i < k; ++i) idx[i] = order[i];
}

// Router ([PN] "Key design 2"): low-rank query, depth RoPE on the query only (R8),
// z = rho * u . keys_e; sigma = norm(TopK(sigmoid(z), z + b, k)) (R10, R11).
template <class WT>
void expert_route(int64_t T, int h, int r, int E, int k, int l, int L, const double* x,
                  const WT* w_r, const WT* keys, const double* bias, double rho,
                  bool normalize, double base, int64_t* idx, double* gate, int64_t* counts,
                  double* z_out, const int64_t* force_idx) {
  vec u(T * r);
  linear(x, T, h, w_r, r, u.data());
  depth_rope_rows(u.data(), T, r, l, L, base, u.data());
  vec z(T * E);
  linear(u.data(), T, r, keys, E, z.data());
  for (int64_t i = 0; i < T * E; ++i) z[i] = rho * z[i];
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    if (force_idx) {
      for (int i = 0; i < k; ++i) idx[t * k + i] = force_idx[t * k + i];
    } else {
      vec keyv(E);
      for (int e = 0; e < E; ++e) keyv[e] = z[t * E + e] + bias[e];
      topk_row(keyv.data(), E, k, idx + t * k);
    }
    double sum = 0.0;
    for (int i = 0; i < k; ++i) {
      gate[t * k + i] = sigmoid(z[t * E + idx[t * k + i]]);
      sum += gate[t * k + i];
    }
    if (normalize)
      for (int i = 0; i < k; ++i) gate[t * k + i] = gate[t * k + i] / sum;
  }
  if (counts) {
    std::fill(counts, counts + E, int64_t(0));
    for (int64_t i = 0; i < T * k; ++i) counts[idx[i]] += 1;
  }
  if (z_out) std::memcpy(z_out, z.data(), sizeof(double) * T * E);
}

// ------------------------------------------------------------------------ experts

// Value side of EA ([PN] "Key design 2": each tiny expert's FFN is the value transform;
// dropless): every selected (token, expert) pair is computed, gated, stored (bf16
// emulation), then summed onto the residual in slot order.  R13 activations.
template <class WT>
void expert_ffn(int kind, int64_t T, int h_in, int f, int h_out, int k, const double* x,
                const int64_t* idx, const double* gate, const WT* w1, const WT* w3,
                const WT* w2, const double* residual, bool bf16, double* out,
                double* slots_out = nullptr, double* hidden_out = nullptr) {
  vec slots(T * k * h_out);
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t sl = 0; sl < T * k; ++sl) {
    const int64_t t = sl / k;
    const int64_t e = idx[sl];
    const double* xt = x + t * h_in;
    double* o = slots.data() + sl * h_out;
    if (kind == DREAMER_REF_LINEAR) {
      const WT* W = w1 + e * int64_t(h_out) * h_in;
      for (int m = 0; m < h_out; ++m) o[m] = dot(xt, W + int64_t(m) * h_in, h_in);
    } else {
      const WT* W1 = w1 + e * int64_t(f) * h_in;
      vec hid(f);
      for (int j = 0; j < f; ++j) {
        const double a = dot(xt, W1 + int64_t(j) * h_in, h_in);
        if (kind == DREAMER_REF_SWIGLU) {
          const WT* W3 = w3 + e * int64_t(f) * h_in;
          hid[j] = silu(a) * dot(xt, W3 + int64_t(j) * h_in, h_in);
        } else {
          hid[j] = gelu(a);
        }
      }
      store(bf16, hid.data(), f);
      if (hidden_out) std::copy(hid.begin(), hid.end(), hidden_out + sl * f);
      const WT* W2 = w2 + e * int64_t(h_out) * f;
      for (int m = 0; m < h_out; ++m) o[m] = dot(hid.data(), W2 + int64_t(m) * f, f);
    }
    for (int m = 0; m < h_out; ++m) o[m] = gate[sl] * o[m];
    store(bf16, o, h_out);
  }
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int m = 0; m < h_out; ++m) {
      double acc = residual ? residual[t * h_out + m] : 0.0;
      for (int i = 0; i < k; ++i) acc = acc + slots[(t * k + i) * h_out + m];
      out[t * h_out + m] = acc;
    }
  }
  if (slots_out) std::copy(slots.begin(), slots.end(), slots_out);
}

// --------------------------------------------------------------------------- layer

template <class WT>
struct Weights {
  const WT *g, *w_qkv, *w_o, *w_qkv_e, *w_qkv_sh, *w_o_e, *w_o_sh, *w_pr, *pkeys;
  const WT *w_r, *keys, *w1, *w3, *w2;
  const double* bias;
};

template <class WT>
Weights<WT> cast_weights(const dreamer_ref_weights* w) {
  auto c = [](const void* p) { return static_cast<const WT*>(p); };
  return {c(w->g),     c(w->w_qkv),    c(w->w_o),  c(w->w_qkv_e), c(w->w_qkv_sh),
          c(w->w_o_e), c(w->w_o_sh),   c(w->w_pr), c(w->pkeys),   c(w->w_r),
          c(w->keys),  c(w->w1),       c(w->w3),   c(w->w2),      w->bias};
}

// Q/K/V (is_qkv, X = x_hat [T, h] -> [T, 6h]) or output (X = [a_SA | a_DA] [T, 2h] ->
// [T, h]) projection.  Dense, or the top-1 linear MoE of [PN] "Key design 3" in its
// unabsorbed form: sigma x W_{e*} + max(sigma_hat) x W_shared, max(sigma_hat) = sigma
// for top-1 (R12).
template <class WT>
void project(const dreamer_ref_cfg& c, const Weights<WT>& w, bool is_qkv, const double* X,
             int64_t T, const int64_t* pidx, const double* pgate, double* Y) {
  const int64_t h = c.h;
  const int64_t K = is_qkv ? h : 2 * h, N = is_qkv ? 6 * h : h;
  if (!c.proj_experts) {
    linear(X, T, K, is_qkv ? w.w_qkv : w.w_o, N, Y);
    return;
  }
  const WT* We = is_qkv ? w.w_qkv_e : w.w_o_e;
  const WT* Wsh = is_qkv ? w.w_qkv_sh : w.w_o_sh;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < N; ++j) {
      const double a = dot(X + t * K, We + (pidx[t] * N + j) * K, K);
      const double b = dot(X + t * K, Wsh + j * K, K);
      Y[t * N + j] = pgate[t] * a + pgate[t] * b;
    }
}

// Columns [sec*h, (sec+1)*h) of a [T, 6h] projection.
vec columns(const double* qkv, int64_t T, int64_t h, int sec) {
  vec out(T * h);
  for (int64_t t = 0; t < T; ++t)
    std::memcpy(out.data() + t * h, qkv + t * 6 * h + sec * h, sizeof(double) * h);
  return out;
}

// SA at depth l from the SA columns [q | k | v] (R5, R21: rotated, then stored once).
template <class CT>
vec sa_branch(const dreamer_ref_cfg& c, const double* qkv, int l, CT* sa_k, CT* sa_v,
              int64_t cap) {
  const int64_t T = int64_t(c.b) * c.s, h = c.h;
  const int H = c.H, d = c.d;
  const bool bf = c.bf16 != 0;
  vec q = columns(qkv, T, h, 0), k = columns(qkv, T, h, 1), v = columns(qkv, T, h, 2);
  if (c.sa_rope) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      const double p = c.decode ? double(c.sa_pos) : double(t % c.s);
      const vec pos(d / 2, p);
      for (int hh = 0; hh < H; ++hh) {
        rope_vec(q.data() + t * h + hh * d, pos.data(), d, c.rope_base, q.data() + t * h + hh * d);
        rope_vec(k.data() + t * h + hh * d, pos.data(), d, c.rope_base, k.data() + t * h + hh * d);
      }
    }
  }
  store(bf, q.data(), T * h);
  store(bf, k.data(), T * h);
  store(bf, v.data(), T * h);
  vec a(T * h), krot(T * h), vapp(T * h);
  const int64_t cache_per_depth = int64_t(c.b) * cap * h;
  if (c.decode) {
    // R14: keys = the cached positions 0..sa_pos-1 of depth l, then this token.
    const int64_t P = c.sa_pos;
    seq_attn<CT>(c.b, 1, H, d, P, q.data(), k.data(), v.data(), sa_k + l * cache_per_depth,
                 sa_v + l * cache_per_depth, cap, false, c.rope_base, bf, a.data(),
                 krot.data(), vapp.data());
    for (int b = 0; b < c.b; ++b)
      for (int64_t j = 0; j < h; ++j) {
        sa_k[l * cache_per_depth + (int64_t(b) * cap + P) * h + j] = CT(krot[b * h + j]);
        sa_v[l * cache_per_depth + (int64_t(b) * cap + P) * h + j] = CT(vapp[b * h + j]);
      }
  } else {
    seq_attn<CT>(c.b, c.s, H, d, 0, q.data(), k.data(), v.data(), nullptr, nullptr, 0, false,
                 c.rope_base, bf, a.data(), krot.data(), vapp.data());
    if (sa_k) {  // prefill -> decode hand-off: positions 0..s-1 of depth l
      for (int b = 0; b < c.b; ++b)
        for (int64_t i = 0; i < c.s; ++i)
          for (int64_t j = 0; j < h; ++j) {
            sa_k[l * cache_per_depth + (int64_t(b) * cap + i) * h + j] =
                CT(krot[(int64_t(b) * c.s + i) * h + j]);
            sa_v[l * cache_per_depth + (int64_t(b) * cap + i) * h + j] =
                CT(vapp[(int64_t(b) * c.s + i) * h + j]);
          }
    }
  }
  return a;
}

// DA over the key set of depth l from the DA columns [q | k | v] (R1, R4, R21, R26).
vec da_branch(const dreamer_ref_cfg& c, const double* qkv, int l, double* da_k,
              double* da_v) {
  const int64_t T = int64_t(c.b) * c.s, h = c.h;
  if (!c.use_da) return vec(T * h, 0.0);
  const bool bf = c.bf16 != 0;
  vec q = columns(qkv, T, h, 3), k = columns(qkv, T, h, 4), v = columns(qkv, T, h, 5);
  depth_rope_rows(q.data(), T * c.H, c.d, l, c.L, c.rope_base, q.data());
  depth_rope_rows(k.data(), T * c.H, c.d, l, c.L, c.rope_base, k.data());
  store(bf, q.data(), T * h);
  store(bf, k.data(), T * h);
  store(bf, v.data(), T * h);
  vec a(T * h);
  depth_attn(T, c.H, c.d, l, c.L, q.data(), k.data(), v.data(), da_k, da_v, c.rope_base, bf,
             false, c.da_window, c.da_dilation, a.data());
  return a;
}

// [a | b] row by row: [T, 2h].
vec concat(const vec& a, const vec& b, int64_t T, int64_t h) {
  vec out(T * 2 * h);
  for (int64_t t = 0; t < T; ++t) {
    std::memcpy(out.data() + t * 2 * h, a.data() + t * h, sizeof(double) * h);
    std::memcpy(out.data() + t * 2 * h + h, b.data() + t * h, sizeof(double) * h);
  }
  return out;
}

// One depth step l ([PN] flowchart: RMSNorm -> DA and SA -> residual -> EA).
template <class WT, class CT>
void layer_step(const dreamer_ref_cfg& c, const Weights<WT>& w, const double* x, int l,
                double* da_k, double* da_v, CT* sa_k, CT* sa_v, int64_t cap,
                const int64_t* force_idx, const int64_t* force_pidx,
                const dreamer_ref_step_out& out) {
  const int64_t T = int64_t(c.b) * c.s, h = c.h;
  const bool bf = c.bf16 != 0;
  // R2, R3: x_hat = x / sqrt(mean(x^2) + eps) * g, the stream itself ([PN] "Loss /
  // training": RMSNorm on the residual stream).  R20: the residual keeps x_hat unrounded.
  vec xh(T * h), g(h);
  for (int64_t j = 0; j < h; ++j) g[j] = double(w.g[j]);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double ms = 0.0;
    for (int64_t j = 0; j < h; ++j) ms += x[t * h + j] * x[t * h + j];
    ms = ms / double(h);
    const double inv = std::sqrt(ms + c.rms_eps);
    for (int64_t j = 0; j < h; ++j) xh[t * h + j] = x[t * h + j] / inv * g[j];
  }
  vec xhb(xh);
  store(bf, xhb.data(), T * h);

  // R12: one top-1 projection router per token and depth on x_hat, bias 0, raw sigmoid.
  std::vector<int64_t> pidx;
  vec pgate, pz;
  if (c.proj_experts) {
    const int Ep = c.proj_experts;
    pidx.resize(T);
    pgate.resize(T);
    pz.resize(T * Ep);
    const vec pbias(Ep, 0.0);
    expert_route<WT>(T, c.h, c.r, Ep, 1, l, c.L, xhb.data(), w.w_pr, w.pkeys, pbias.data(),
                     c.rho, false, c.rope_base, pidx.data(), pgate.data(), nullptr, pz.data(),
                     force_pidx);
    if (out.pidx) std::copy(pidx.begin(), pidx.end(), out.pidx);
    if (out.pgate) std::copy(pgate.begin(), pgate.end(), out.pgate);
    if (out.pz) std::copy(pz.begin(), pz.end(), out.pz);
  }
  const int64_t* pi = c.proj_experts ? pidx.data() : nullptr;
  const double* pg = c.proj_experts ? pgate.data() : nullptr;

  const vec zero(T * h, 0.0);
  vec y(T * h);
  if (c.mixture == DREAMER_REF_SERIAL) {
    // R22: u = x_hat + DA(x_hat); v = u + SA(u) through u's storage copy.
    vec qkv(T * 6 * h), o(T * h);
    project(c, w, true, xhb.data(), T, pi, pg, qkv.data());
    const vec a_da = da_branch(c, qkv.data(), l, da_k, da_v);
    project(c, w, false, concat(zero, a_da, T, h).data(), T, pi, pg, o.data());
    vec u(T * h);
    for (int64_t i = 0; i < T * h; ++i) u[i] = xh[i] + o[i];
    vec ub(u);
    store(bf, ub.data(), T * h);
    project(c, w, true, ub.data(), T, pi, pg, qkv.data());
    const vec a_sa = sa_branch<CT>(c, qkv.data(), l, sa_k, sa_v, cap);
    project(c, w, false, concat(a_sa, zero, T, h).data(), T, pi, pg, o.data());
    for (int64_t i = 0; i < T * h; ++i) y[i] = u[i] + o[i];
  } else {
    // Parallel residual y = x_l + DA(x_{:l}) + SA(x_l) ([PN] "Key design 1"); R6: the SA
    // and DA output projections act on [a_SA | a_DA].
    vec qkv(T * 6 * h), o(T * h);
    project(c, w, true, xhb.data(), T, pi, pg, qkv.data());
    const vec a_sa = sa_branch<CT>(c, qkv.data(), l, sa_k, sa_v, cap);
    const vec a_da = da_branch(c, qkv.data(), l, da_k, da_v);
    project(c, w, false, concat(a_sa, a_da, T, h).data(), T, pi, pg, o.data());
    for (int64_t i = 0; i < T * h; ++i) y[i] = xh[i] + o[i];
  }
  vec yb(y);
  store(bf, yb.data(), T * h);
  // R7: EA reads y (serial: v); the fully parallel wiring reads x_hat.
  const vec& ea_in = (c.mixture == DREAMER_REF_PARALLEL) ? xhb : yb;
  if (out.y) std::copy(y.begin(), y.end(), out.y);
  if (out.yb) std::copy(ea_in.begin(), ea_in.end(), out.yb);

  if (!c.use_ea) {
    std::copy(y.begin(), y.end(), out.x_next);
    return;
  }
  std::vector<int64_t> idx(T * c.k);
  vec gate(T * c.k), z(T * int64_t(c.E));
  std::vector<int64_t> counts(c.E);
  expert_route<WT>(T, c.h, c.r, c.E, c.k, l, c.L, ea_in.data(), w.w_r, w.keys, w.bias, c.rho,
                   c.normalize != 0, c.rope_base, idx.data(), gate.data(), counts.data(),
                   z.data(), force_idx);
  expert_ffn<WT>(c.ffn, T, c.h, c.f, c.h, c.k, ea_in.data(), idx.data(), gate.data(), w.w1,
                 w.w3, w.w2, y.data(), bf, out.x_next);
  if (out.idx) std::copy(idx.begin(), idx.end(), out.idx);
  if (out.gate) std::copy(gate.begin(), gate.end(), out.gate);
  if (out.counts) std::copy(counts.begin(), counts.end(), out.counts);
  if (out.z) std::copy(z.begin(), z.end(), out.z);
}

// Offsets a step_out to depth (or token) slot n.
dreamer_ref_step_out step_at(const dreamer_ref_step_out* s, const dreamer_ref_cfg& c,
                             int64_t n) {
  dreamer_ref_step_out o{};
  if (!s) return o;
  const int64_t T = int64_t(c.b) * c.s, h = c.h, k = c.k, E = c.E, Ep = c.proj_experts;
  auto off = [&](auto* p, int64_t per) { return p ? p + n * per : p; };
  o.x_next = off(s->x_next, T * h);
  o.y = off(s->y, T * h);
  o.yb = off(s->yb, T * h);
  o.idx = off(s->idx, T * k);
  o.gate = off(s->gate, T * k);
  o.counts = off(s->counts, E);
  o.z = off(s->z, T * E);
  o.pidx = off(s->pidx, T);
  o.pgate = off(s->pgate, T);
  o.pz = off(s->pz, T * Ep);
  return o;
}

bool cfg_ok(const dreamer_ref_cfg* c) {
  if (!c) return false;
  if (c->b < 1 || c->s < 1 || c->h < 1 || c->H < 1 || c->d < 2 || c->L < 1) return false;
  if (c->H * c->d != c->h || c->d % 2 || c->r % 2) return false;
  if (c->use_ea && (c->E < 1 || c->k < 1 || c->k > c->E || c->f < 1 || c->r < 2)) return false;
  if (c->decode && (c->s != 1 || c->sa_pos < 1)) return false;
  return true;
}

// The unrolled layer ([PN] flowchart: one shared layer, repeated until depth L).
template <class WT, class CT>
void layer_forward(const dreamer_ref_cfg& c, const Weights<WT>& w, const double* x0,
                   double* x_out, double* da_k, double* da_v, CT* sa_k, CT* sa_v, int64_t cap,
                   const int64_t* force_idx, const int64_t* force_pidx,
                   const dreamer_ref_step_out* steps) {
  const int64_t T = int64_t(c.b) * c.s, h = c.h;
  vec x(x0, x0 + T * h), nx(T * h);
  for (int l = 0; l < c.L; ++l) {
    dreamer_ref_step_out o = step_at(steps, c, l);
    o.x_next = nx.data();
    layer_step<WT, CT>(c, w, x.data(), l, da_k, da_v, sa_k, sa_v, cap,
                       force_idx ? force_idx + l * T * c.k : nullptr,
                       force_pidx ? force_pidx + l * T : nullptr, o);
    if (steps && steps->x_next) std::copy(nx.begin(), nx.end(), steps->x_next + l * T * h);
    x.swap(nx);
  }
  std::copy(x.begin(), x.end(), x_out);
}

template <class F>
int dispatch(int w_f32, int sa_f32, F&& f) {
  if (w_f32 && sa_f32) return f(float(), float());
  if (w_f32) return f(float(), double());
  if (sa_f32) return f(double(), float());
  return f(double(), double());
}

}  // namespace

// ============================================================================ C ABI

extern "C" {

int dreamer_ref_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
}

void dreamer_ref_bf16_round(const double* x, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_round(x[i]);
}

int dreamer_ref_rmsnorm(const double* x, const double* g, int64_t rows, int h, double eps,
                        double* out) {
  if (!x || !g || !out || rows < 0 || h < 1) return 1;
  for (int64_t t = 0; t < rows; ++t) {
    double ms = 0.0;
    for (int j = 0; j < h; ++j) ms += x[t * h + j] * x[t * h + j];
    ms = ms / double(h);
    const double inv = std::sqrt(ms + eps);
    for (int j = 0; j < h; ++j) out[t * h + j] = x[t * h + j] / inv * g[j];
  }
  return 0;
}

int dreamer_ref_rope(const double* u, const double* pos, int64_t n, int D, double base,
                     double* out) {
  if (!u || !pos || !out || n < 0 || D < 2 || D % 2) return 1;
  for (int64_t t = 0; t < n; ++t) rope_vec(u + t * D, pos + t * (D / 2), D, base, out + t * D);
  return 0;
}

int dreamer_ref_depth_rope(const double* u, int64_t n, int D, int l, int L, double base,
                           double* out) {
  if (!u || !out || n < 0 || D < 2 || D % 2 || l < 0 || l >= L) return 1;
  depth_rope_rows(u, n, D, l, L, base, out);
  return 0;
}

int dreamer_ref_depth_keys(int l, int window, int dilation, int* keys) {
  if (l < 0 || !keys) return -1;
  const std::vector<int> k = depth_keys(l, window, dilation);
  std::copy(k.begin(), k.end(), keys);
  return int(k.size());
}

int dreamer_ref_seq_attn(int B, int n, int H, int d, int64_t pos0, const double* q,
                         const double* k_new, const double* v_new, const void* k_cache,
                         const void* v_cache, int64_t cap, int cache_f32, int sa_rope,
                         double base, int bf16, double* out, double* k_rot, double* v_out) {
  if (!q || !k_new || !v_new || !out || !k_rot || !v_out) return 1;
  if (B < 1 || n < 1 || H < 1 || d < 2 || d % 2 || pos0 < 0) return 1;
  if (pos0 > 0 && (!k_cache || !v_cache || cap < pos0)) return 1;
  if (cache_f32)
    seq_attn<float>(B, n, H, d, pos0, q, k_new, v_new, static_cast<const float*>(k_cache),
                    static_cast<const float*>(v_cache), cap, sa_rope != 0, base, bf16 != 0,
                    out, k_rot, v_out);
  else
    seq_attn<double>(B, n, H, d, pos0, q, k_new, v_new, static_cast<const double*>(k_cache),
                     static_cast<const double*>(v_cache), cap, sa_rope != 0, base, bf16 != 0,
                     out, k_rot, v_out);
  return 0;
}

int dreamer_ref_depth_attn(int64_t R, int H, int d, int l, int L, const double* q,
                           const double* k_new, const double* v_new, double* k_cache,
                           double* v_cache, double base, int bf16, int use_rope, int window,
                           int dilation, double* out) {
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !out) return 1;
  if (R < 0 || H < 1 || d < 2 || d % 2 || l < 0 || l >= L) return 1;
  depth_attn(R, H, d, l, L, q, k_new, v_new, k_cache, v_cache, base, bf16 != 0,
             use_rope != 0, window, dilation, out);
  return 0;
}

int dreamer_ref_topk_select(const double* key, int64_t T, int E, int k, int64_t* idx) {
  if (!key || !idx || T < 0 || k < 1 || k > E) return 1;
  for (int64_t t = 0; t < T; ++t) topk_row(key + t * E, E, k, idx + t * k);
  return 0;
}

int dreamer_ref_expert_route(int64_t T, int h, int r, int E, int k, int l, int L,
                             const double* x, const void* w_r, const void* keys, int w_f32,
                             const double* bias, double rho, int normalize, double base,
                             int64_t* idx, double* gate, int64_t* counts, double* z) {
  if (!x || !w_r || !keys || !bias || !idx || !gate) return 1;
  if (T < 0 || h < 1 || r < 2 || r % 2 || E < 1 || k < 1 || k > E || l < 0 || l >= L) return 1;
  if (w_f32)
    expert_route<float>(T, h, r, E, k, l, L, x, static_cast<const float*>(w_r),
                        static_cast<const float*>(keys), bias, rho, normalize != 0, base, idx,
                        gate, counts, z, nullptr);
  else
    expert_route<double>(T, h, r, E, k, l, L, x, static_cast<const double*>(w_r),
                         static_cast<const double*>(keys), bias, rho, normalize != 0, base,
                         idx, gate, counts, z, nullptr);
  return 0;
}

int dreamer_ref_bias_update(const double* bias, const int64_t* counts, int E, double lambda,
                            double* out) {
  if (!bias || !counts || !out || E < 1) return 1;
  std::vector<int64_t> srt(counts, counts + E);
  std::sort(srt.begin(), srt.end());
  const double med = (E % 2) ? double(srt[E / 2])
                             : (double(srt[E / 2 - 1]) + double(srt[E / 2])) / 2.0;
  for (int e = 0; e < E; ++e) {
    const double diff = med - double(counts[e]);
    const double sgn = (diff > 0) ? 1.0 : (diff < 0 ? -1.0 : 0.0);
    out[e] = bias[e] + lambda * sgn;
  }
  return 0;
}

int dreamer_ref_route_counts(const int64_t* idx, int64_t n_sets, int64_t per_set, int E,
                             int64_t* counts) {
  if (!idx || !counts || n_sets < 0 || per_set < 0 || E < 1) return 1;
  std::fill(counts, counts + n_sets * E, int64_t(0));
  for (int64_t s = 0; s < n_sets; ++s)
    for (int64_t j = 0; j < per_set; ++j) {
      const int64_t e = idx[s * per_set + j];
      if (e < 0 || e >= E) return 1;
      counts[s * E + e] += 1;
    }
  return 0;
}

int dreamer_ref_expert_usage(const int64_t* counts, int E, int* distinct,
                             double* max_over_mean, double* gini, double* lorenz) {
  if (!counts || !distinct || !max_over_mean || !gini || !lorenz || E < 1) return 1;
  double sum = 0.0, mx = 0.0;
  int used = 0;
  for (int e = 0; e < E; ++e) {
    sum += double(counts[e]);
    mx = std::max(mx, double(counts[e]));
    used += counts[e] > 0;
  }
  const double mean = sum / double(E);
  double pair = 0.0;
  for (int i = 0; i < E; ++i)
    for (int j = 0; j < E; ++j) pair += std::fabs(double(counts[i]) - double(counts[j]));
  *distinct = used;
  *max_over_mean = mx / mean;
  *gini = pair / (2.0 * E * E * mean);
  std::vector<int64_t> srt(counts, counts + E);
  std::sort(srt.begin(), srt.end());
  double cum = 0.0;
  for (int e = 0; e < E; ++e) {
    cum += double(srt[e]);
    lorenz[e] = cum / sum;
  }
  return 0;
}

int dreamer_ref_expert_ffn(int kind, int64_t T, int h_in, int f, int h_out, int E, int k,
                           const double* x, const int64_t* idx, const double* gate,
                           const void* w1, const void* w3, const void* w2, int w_f32,
                           const double* residual, int bf16, double* out, double* slots,
                           double* hidden) {
  if (!x || !idx || !gate || !w1 || !out || T < 0 || h_in < 1 || h_out < 1 || k < 1) return 1;
  if (kind != DREAMER_REF_LINEAR && (!w2 || f < 1)) return 1;
  if (kind == DREAMER_REF_SWIGLU && !w3) return 1;
  for (int64_t i = 0; i < T * k; ++i)
    if (idx[i] < 0 || idx[i] >= E) return 1;
  if (w_f32)
    expert_ffn<float>(kind, T, h_in, f, h_out, k, x, idx, gate, static_cast<const float*>(w1),
                      static_cast<const float*>(w3), static_cast<const float*>(w2), residual,
                      bf16 != 0, out, slots, hidden);
  else
    expert_ffn<double>(kind, T, h_in, f, h_out, k, x, idx, gate,
                       static_cast<const double*>(w1), static_cast<const double*>(w3),
                       static_cast<const double*>(w2), residual, bf16 != 0, out, slots,
                       hidden);
  return 0;
}

int dreamer_ref_layer_step(const dreamer_ref_cfg* cfg, const dreamer_ref_weights* w,
                           const double* x, int l, double* da_k, double* da_v, void* sa_k,
                           void* sa_v, int64_t sa_cap, int sa_f32, const int64_t* force_idx,
                           const int64_t* force_pidx, const dreamer_ref_step_out* out) {
  if (!cfg_ok(cfg) || !w || !x || !da_k || !da_v || !out || !out->x_next) return 1;
  if (l < 0 || l >= cfg->L) return 1;
  if (cfg->decode && (!sa_k || !sa_v || sa_cap <= cfg->sa_pos)) return 1;
  return dispatch(w->f32, sa_f32, [&](auto wt, auto ct) {
    using WT = decltype(wt);
    using CT = decltype(ct);
    layer_step<WT, CT>(*cfg, cast_weights<WT>(w), x, l, da_k, da_v, static_cast<CT*>(sa_k),
                       static_cast<CT*>(sa_v), sa_cap, force_idx, force_pidx, *out);
    return 0;
  });
}

int dreamer_ref_layer_forward(const dreamer_ref_cfg* cfg, const dreamer_ref_weights* w,
                              const double* x0, double* x_out, double* da_k, double* da_v,
                              void* sa_k, void* sa_v, int64_t sa_cap, int sa_f32,
                              const int64_t* force_idx, const int64_t* force_pidx,
                              const dreamer_ref_step_out* steps) {
  if (!cfg_ok(cfg) || !w || !x0 || !x_out || !da_k || !da_v) return 1;
  if (cfg->decode && (!sa_k || !sa_v || sa_cap <= cfg->sa_pos)) return 1;
  if (!cfg->decode && sa_k && sa_cap < cfg->s) return 1;
  return dispatch(w->f32, sa_f32, [&](auto wt, auto ct) {
    using WT = decltype(wt);
    using CT = decltype(ct);
    layer_forward<WT, CT>(*cfg, cast_weights<WT>(w), x0, x_out, da_k, da_v,
                          static_cast<CT*>(sa_k), static_cast<CT*>(sa_v), sa_cap, force_idx,
                          force_pidx, steps);
    return 0;
  });
}

int dreamer_ref_decode_tokens(const dreamer_ref_cfg* cfg, const dreamer_ref_weights* w,
                              int n, const double* xs, double* x_out, void* sa_k, void* sa_v,
                              int64_t sa_cap, int sa_f32, const dreamer_ref_step_out* steps) {
  if (!cfg_ok(cfg) || !cfg->decode || !w || !xs || !x_out || n < 0) return 1;
  if (!sa_k || !sa_v || sa_cap < cfg->sa_pos + n) return 1;
  const int64_t T = cfg->b, h = cfg->h;
  const int64_t cache = T * int64_t(cfg->L) * cfg->h;
  for (int j = 0; j < n; ++j) {
    dreamer_ref_cfg cj = *cfg;
    cj.sa_pos = cfg->sa_pos + j;
    // a fresh DA cache per token: slots are written before they are read ([PN] the DA
    // cache is overwritten at the next token)
    vec dk(cache, std::numeric_limits<double>::quiet_NaN()), dv(dk);
    dreamer_ref_step_out sj{};
    const dreamer_ref_step_out* sp = nullptr;
    if (steps) {
      sj = step_at(steps, cj, int64_t(j) * cfg->L);
      sp = &sj;
    }
    const int rc = dreamer_ref_layer_forward(&cj, w, xs + j * T * h, x_out + j * T * h,
                                             dk.data(), dv.data(), sa_k, sa_v, sa_cap, sa_f32,
                                             nullptr, nullptr, sp);
    if (rc) return rc;
  }
  return 0;
}

}  // extern "C"
