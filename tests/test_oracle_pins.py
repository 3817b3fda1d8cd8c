"""Pins of the CPU oracle against facts fixed outside the oracle itself: published
generator values, library routines (torch float64 SDPA, rms_norm, bfloat16 casts),
closed forms (RoPE as complex rotation), invariants and brute force.  No GPU."""
import itertools
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synth import CONFIGS, make_weights, make_x0, rng

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- generator

def test_splitmix64_published_value():
    # SplitMix64 (Steele-Lea-Flood 2014, Vigna's splitmix64.c): state 0 -> first output.
    with open(os.path.join(GOLDEN, "splitmix64.txt")) as fh:
        lines = [l.split("#")[0].strip() for l in fh if l.split("#")[0].strip()]
    state, first = (int(v, 16) for v in lines[0].split())
    assert rng.mix_int(state + rng.GAMMA) == first


def test_rng_torch_matches_python_and_random_access():
    n = torch.arange(1000, dtype=torch.int64)
    raw = rng.raw_at(n, 5, 9)
    base = rng.stream_base(5, 9)
    for i in (0, 1, 17, 999):
        assert (int(raw[i]) & rng.MASK64) == rng.mix_int(base + (i + 1) * rng.GAMMA)
    full = rng.normal((40, 30), 3, 4)
    part = rng.normal((10, 30), 3, 4, offset=25 * 30)
    assert torch.equal(full[25:35], part)


def test_rng_normal_moments():
    x = rng.normal((1 << 20,), 11, 2).double()
    assert abs(x.mean().item()) < 5e-3
    assert abs(x.std().item() - 1.0) < 5e-3
    u = rng.uniform((1 << 18,), 11, 3, -0.2, 0.2).double()
    assert u.min() >= -0.2 and u.max() < 0.2 and abs(u.mean().item()) < 2e-3


# ------------------------------------------------------------------------------ rounding

def test_bf16_round_matches_torch_cast():
    x = (torch.randn(200000, dtype=torch.float64) * 3).float()
    ref = x.to(torch.bfloat16).double().numpy()
    got = oracle.bf16_round(x.double().numpy())
    assert np.array_equal(ref, got)
    # ties to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert oracle.bf16_round(1.0 + 2 ** -8) == 1.0
    assert oracle.bf16_round(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6


# ---------------------------------------------------------------------------------- RoPE

def _rope_complex(u, pos, base):
    """RoPE written as complex multiplication of the pairs (u_i, u_{i+D/2})."""
    D = u.shape[-1]
    half = D // 2
    z = u[..., :half] + 1j * u[..., half:]
    theta = np.array([base ** (-(2.0 * i) / D) for i in range(half)])
    z = z * np.exp(1j * np.asarray(pos, np.float64) * theta)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_is_complex_rotation():
    r = np.random.default_rng(0)
    u = r.standard_normal((5, 16))
    pos = r.integers(0, 50, size=(5, 1)).astype(np.float64)
    assert np.allclose(oracle.rope(u, pos, 10000.0), _rope_complex(u, pos, 10000.0),
                       atol=1e-13)
    # D = 2: theta_0 = 1, so the angle equals the position exactly
    v = np.array([[1.0, 0.0]])
    assert np.allclose(oracle.rope(v, 0.5, 10000.0), [[math.cos(0.5), math.sin(0.5)]])


def test_rope_norm_and_relative_position():
    r = np.random.default_rng(1)
    q, k = r.standard_normal((2, 32))
    for m, n in [(0, 3), (7, 2)]:
        s1 = oracle.rope(q, m, 1e4) @ oracle.rope(k, n, 1e4)
        s2 = oracle.rope(q, m + 11, 1e4) @ oracle.rope(k, n + 11, 1e4)
        assert abs(s1 - s2) < 1e-12
    assert abs(np.linalg.norm(oracle.rope(q, 9, 1e4)) - np.linalg.norm(q)) < 1e-12


def _halves(u):
    D = u.shape[-1]
    q4 = D // 4
    fwd = np.r_[0:q4, D // 2:D // 2 + q4]
    rev = np.r_[q4:D // 2, D // 2 + q4:D]
    return fwd, rev


def test_depth_rope_forward_half_relative_reversed_half_distance_to_L():
    r = np.random.default_rng(2)
    D, L = 64, 16
    q, k = r.standard_normal((2, D))
    fwd, rev = _halves(q)
    def parts(m, n, LL):
        a = oracle.depth_rope(q, m, LL, 1e4)
        b = oracle.depth_rope(k, n, LL, 1e4)
        return a[fwd] @ b[fwd], a[rev] @ b[rev]
    f1, r1 = parts(5, 2, L)
    f2, r2 = parts(9, 6, L)      # same offset, shifted
    assert abs(f1 - f2) < 1e-12 and abs(r1 - r2) < 1e-12
    # reversed half at (m, n; L) == plain RoPE score of that half at (L-1-m, L-1-n)
    m, n = 3, 11
    a = oracle.depth_rope(q, m, L, 1e4)
    b = oracle.depth_rope(k, n, L, 1e4)
    pa = _rope_complex(q, L - 1 - m, 1e4)
    pb = _rope_complex(k, L - 1 - n, 1e4)
    assert abs(a[rev] @ b[rev] - pa[rev] @ pb[rev]) < 1e-12
    assert abs(a[fwd] @ b[fwd] - _rope_complex(q, m, 1e4)[fwd] @ _rope_complex(k, n, 1e4)[fwd]) < 1e-12
    # position-less key (router): the reversed half depends only on L-1-l
    sa = oracle.depth_rope(q, 4, 10, 1e4)[rev] @ k[rev]
    sb = oracle.depth_rope(q, 9, 15, 1e4)[rev] @ k[rev]
    assert abs(sa - sb) < 1e-12
    fa = oracle.depth_rope(q, 4, 10, 1e4)[fwd] @ k[fwd]
    fb = oracle.depth_rope(q, 9, 15, 1e4)[fwd] @ k[fwd]
    assert abs(fa - fb) > 1e-6
    # the reversed half sees the depth offset with its sign flipped: its score at
    # (m, n) is the plain-RoPE score of the same dims at (n, m)
    a = oracle.depth_rope(q, 7, L, 1e4)
    b = oracle.depth_rope(k, 4, L, 1e4)
    pa = _rope_complex(q, 4, 1e4)
    pb = _rope_complex(k, 7, 1e4)
    assert abs(a[rev] @ b[rev] - pa[rev] @ pb[rev]) < 1e-12


# ------------------------------------------------------------------------------ attention

def _sdpa(q, k, v, causal=True):
    """torch float64 SDPA with [B, n, H, d] layout."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float64).transpose(0, 2, 1, 3)))
    o = F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal)
    return o.numpy().transpose(0, 2, 1, 3)


def test_depth_attn_first_depth_returns_v_exactly():
    r = np.random.default_rng(3)
    R, H, d, L = 7, 4, 16, 5
    q, k, v = r.standard_normal((3, R, H, d))
    for bf16 in (False, True):
        vv = oracle.bf16_round(v) if bf16 else v
        kc, vc = np.full((R, L, H, d), np.nan), np.full((R, L, H, d), np.nan)
        out = oracle.depth_attn(q, k, vv, kc, vc, 0, L, bf16=bf16)
        assert np.array_equal(out, vv)


def test_depth_attn_equals_causal_sdpa_over_depth():
    r = np.random.default_rng(4)
    R, H, d, L = 6, 2, 8, 7
    q, k, v = r.standard_normal((3, R, L, H, d))
    kc, vc = np.full((R, L, H, d), np.nan), np.full((R, L, H, d), np.nan)
    outs = np.stack([oracle.depth_attn(q[:, l], k[:, l], v[:, l], kc, vc, l, L, use_rope=False)
                     for l in range(L)], axis=1)
    ref = _sdpa(q, k, v, causal=True)   # rows as batch, depth as the sequence axis
    assert np.allclose(outs, ref, atol=1e-12)


def test_depth_attn_ignores_future_slots_and_constant_values():
    r = np.random.default_rng(5)
    R, H, d, L, l = 4, 2, 8, 6, 3
    kc = r.standard_normal((R, L, H, d))
    vc = np.ones((R, L, H, d)) * 0.75
    kc[:, l + 1:] = np.nan
    vc[:, l + 1:] = np.nan
    q, k = r.standard_normal((2, R, H, d))
    out = oracle.depth_attn(q, k, np.full((R, H, d), 0.75), kc, vc, l, L)
    assert np.allclose(out, 0.75, atol=1e-14)


# Windowed / dilated depth attention (R26): keys of depth l are the `window` most recent
# depths plus every `dilation`-th older one.  Key sets written out by hand for L = 10,
# window 2, dilation 3.
_KEYS_W2_D3 = [[0], [0, 1], [1, 2], [0, 2, 3], [1, 3, 4], [2, 4, 5], [0, 3, 5, 6],
               [1, 4, 6, 7], [2, 5, 7, 8], [0, 3, 6, 8, 9]]


def test_depth_keys_hand_enumerated():
    for l, keys in enumerate(_KEYS_W2_D3):
        assert list(oracle.depth_keys(l, 2, 3)) == keys
    assert list(oracle.depth_keys(5)) == [0, 1, 2, 3, 4, 5]
    assert list(oracle.depth_keys(5, 3)) == [3, 4, 5]
    assert list(oracle.depth_keys(7, 1, 2)) == [1, 3, 5, 7]
    assert list(oracle.depth_keys(2, 5)) == [0, 1, 2]          # window wider than l + 1
    assert list(oracle.depth_keys(6, 2, 1)) == list(range(7))  # dilation 1: every depth
    assert list(oracle.depth_keys(0, 1, 4)) == [0]


def test_windowed_depth_attn_equals_masked_sdpa():
    r = np.random.default_rng(41)
    R, H, d, L = 5, 2, 8, 10
    q, k, v = r.standard_normal((3, R, L, H, d))
    kc, vc = np.full((R, L, H, d), np.nan), np.full((R, L, H, d), np.nan)
    outs = np.stack([oracle.depth_attn(q[:, l], k[:, l], v[:, l], kc, vc, l, L, use_rope=False,
                                       window=2, dilation=3) for l in range(L)], axis=1)
    mask = torch.zeros((L, L), dtype=torch.bool)
    for l, keys in enumerate(_KEYS_W2_D3):
        mask[l, keys] = True
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3)))
    ref = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask)
    assert np.allclose(outs, ref.numpy().transpose(0, 2, 1, 3), atol=1e-12)


def test_window_one_depth_attn_returns_v_exactly():
    r = np.random.default_rng(42)
    R, H, d, L, l = 6, 2, 16, 8, 5
    kc, vc = r.standard_normal((2, R, L, H, d))
    q, k, v = r.standard_normal((3, R, H, d))
    for bf16 in (False, True):
        vv = oracle.bf16_round(v) if bf16 else v
        out = oracle.depth_attn(q, k, vv, kc.copy(), vc.copy(), l, L, bf16=bf16, window=1)
        assert np.array_equal(out, vv)


def test_seq_attn_equals_sdpa_and_causality():
    r = np.random.default_rng(6)
    B, n, H, d = 2, 9, 3, 8
    q, k, v = r.standard_normal((3, B, n, H, d))
    out, _, _ = oracle.seq_attn(q, k, v, sa_rope=False)
    assert np.allclose(out, _sdpa(q, k, v), atol=1e-12)
    # with RoPE: equals SDPA on q, k rotated by the complex formulation
    pos = np.arange(n, dtype=np.float64)[None, :, None, None]
    out2, krot, _ = oracle.seq_attn(q, k, v, sa_rope=True)
    qr, kr = _rope_complex(q, pos, 1e4), _rope_complex(k, pos, 1e4)
    assert np.allclose(out2, _sdpa(qr, kr, v), atol=1e-12)
    assert np.allclose(krot, kr, atol=1e-12)
    # causality: perturbing token p+1 leaves rows <= p unchanged
    k2, v2 = k.copy(), v.copy()
    k2[:, 5] += 1.0
    v2[:, 5] -= 2.0
    out3, _, _ = oracle.seq_attn(q, k2, v2)
    assert np.array_equal(out3[:, :5], out2[:, :5])


def test_seq_attn_decode_equals_prefill_last_row():
    r = np.random.default_rng(7)
    B, n, H, d = 2, 6, 2, 8
    q, k, v = r.standard_normal((3, B, n, H, d))
    full, krot, vv = oracle.seq_attn(q, k, v)
    cap = n + 2
    kc, vc = np.full((B, cap, H, d), np.nan), np.full((B, cap, H, d), np.nan)
    kc[:, :n - 1], vc[:, :n - 1] = krot[:, :n - 1], vv[:, :n - 1]
    dec, _, _ = oracle.seq_attn(q[:, n - 1:], k[:, n - 1:], v[:, n - 1:], pos0=n - 1,
                                k_cache=kc, v_cache=vc)
    assert np.allclose(dec[:, 0], full[:, n - 1], atol=1e-12)


# -------------------------------------------------------------------------------- routing

def _topk_bruteforce(key, k):
    """Rank by counting the experts that beat e: higher key, or equal key and lower index."""
    E = key.shape[0]
    rank = [sum(1 for f in range(E) if key[f] > key[e] or (key[f] == key[e] and f < e))
            for e in range(E)]
    sel = sorted([e for e in range(E) if rank[e] < k], key=lambda e: rank[e])
    return sel


def test_topk_matches_bruteforce_with_ties():
    r = np.random.default_rng(8)
    for trial in range(300):
        E = int(r.integers(1, 13))
        k = int(r.integers(1, min(3, E) + 1))
        key = np.round(r.standard_normal(E), 1)          # many exact ties
        got = list(oracle.topk_select(key[None], k)[0])
        assert got == _topk_bruteforce(key, k)
        # the set is the best k-subset by key sum (among subsets, lexicographic ties aside)
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(key[list(c)]))
        assert abs(sum(key[got]) - sum(key[list(best)])) < 1e-12


def test_route_gate_properties():
    r = np.random.default_rng(9)
    T, h, rr, E = 11, 16, 8, 10
    x = r.standard_normal((T, h))
    w_r = r.standard_normal((rr, h)) * 0.3
    keys = r.standard_normal((E, rr)) * 0.3
    bias = r.uniform(-0.2, 0.2, E)
    idx, gate, counts, z = oracle.expert_route(x, w_r, keys, bias, 3, 2, 6)
    assert np.allclose(gate.sum(-1), 1.0, atol=1e-12)
    assert counts.sum() == T * 3
    idx1, g1, _, z1 = oracle.expert_route(x, w_r, keys, bias, 1, 2, 6, normalize=False)
    assert np.allclose(g1[:, 0], 1 / (1 + np.exp(-z1[np.arange(T), idx1[:, 0]])))
    idxE, _, cE, _ = oracle.expert_route(x, w_r, keys, bias, E, 2, 6)
    assert (cE == T).all()
    # relabelling the experts permutes the indices, leaves the gates unchanged
    perm = r.permutation(E)
    inv = np.argsort(perm)
    idx_p, gate_p, _, _ = oracle.expert_route(x, w_r, keys[perm], bias[perm], 3, 2, 6)
    assert np.array_equal(perm[idx_p], idx) and np.allclose(gate_p, gate)
    assert np.array_equal(inv[idx], idx_p)


def test_route_scores_closed_form_small_rank():
    # r = 4: pairs (0,2) and (1,3); pair 0 at depth l with theta 1, pair 1 reversed at
    # L-1-l with theta = base^-1/2.  Written as two complex rotations.
    x = np.array([[1.0, 0.0, 0.0]])
    w_r = np.array([[2.0, 0, 0], [0, 0, 0], [0, 0, 0], [1.0, 0, 0]])  # u = (2, 0, 0, 1)
    keys = np.eye(4)
    l, L, base = 2, 5, 100.0
    _, _, _, z = oracle.expert_route(x, w_r, keys, np.zeros(4), 1, l, L, base=base)
    c0 = 2.0 * np.exp(1j * l * 1.0)                          # (u0 + i u2) e^{i l}
    c1 = (0.0 + 1j * 1.0) * np.exp(1j * (L - 1 - l) * base ** -0.5)
    assert np.allclose(z[0], [c0.real, c1.real, c0.imag, c1.imag], atol=1e-14)


def test_bias_update_zero_sum_sign():
    # odd E: median 4 -> experts above it lose lam, below gain lam, the median one stays
    N = np.array([5, 1, 9, 3, 4, 7, 2])
    b = oracle.bias_update(np.zeros(7), N, 0.1)
    assert np.allclose(b, [-0.1, 0.1, -0.1, 0.1, 0.0, -0.1, 0.1], atol=1e-15)
    assert np.isclose(b.sum(), 0.0)  # distinct counts: as many above as below the median
    # even E: the median is the mean of the two middle counts (2.5 here)
    b = oracle.bias_update(np.array([1.0, -1.0, 0.5, 0.0]), np.array([1, 2, 3, 10]), 0.25)
    assert np.allclose(b, [1.25, -0.75, 0.25, -0.25], atol=1e-15)
    # all loads equal: nothing moves
    assert np.array_equal(oracle.bias_update(np.ones(5), np.full(5, 7), 0.3), np.ones(5))


def test_usage_statistics_closed_forms():
    u = oracle.expert_usage([0, 0, 1, 3])   # hand count: sum |Ni - Nj| = 20, E = 4, mean 1
    assert np.isclose(u["gini"], 20 / 32) and u["distinct"] == 2 and u["max_over_mean"] == 3
    assert np.allclose(u["lorenz"], [0, 0, 0.25, 1.0])
    assert oracle.expert_usage(np.full(64, 5))["gini"] == 0.0         # perfectly even
    one = np.zeros(50)
    one[7] = 100
    assert np.isclose(oracle.expert_usage(one)["gini"], 49 / 50)       # one expert holds all
    # two other definitions agree on random loads: 1 - 2 * (area under the Lorenz curve,
    # trapezoids from (0, 0)), and the sorted-rank form 2 sum i x_(i) / (E sum x) - (E+1)/E
    r = np.random.default_rng(5)
    N = r.integers(0, 300, size=257)
    u = oracle.expert_usage(N)
    E = N.size
    Lz = np.concatenate([[0.0], u["lorenz"]])
    area = np.sum((Lz[1:] + Lz[:-1]) / 2) / E
    assert np.isclose(u["gini"], 1 - 2 * area, atol=1e-12)
    xs = np.sort(N).astype(np.float64)
    rank_form = 2 * np.sum(np.arange(1, E + 1) * xs) / (E * xs.sum()) - (E + 1) / E
    assert np.isclose(u["gini"], rank_form, atol=1e-12)


def test_route_counts_per_depth():
    idx = np.array([[[0, 2], [2, 1]], [[3, 3], [0, 1]]])     # [L=2, T=2, k=2]
    assert np.array_equal(oracle.route_counts(idx, 4), [[1, 1, 2, 0], [1, 1, 0, 2]])
    assert np.array_equal(oracle.route_counts(idx[0], 4), [1, 1, 2, 0])


# -------------------------------------------------------------------------------- experts

def test_single_expert_is_dense_mlp():
    r = np.random.default_rng(10)
    T, h, f = 9, 12, 6
    y = r.standard_normal((T, h))
    w1, w3 = r.standard_normal((2, 1, f, h)) * 0.4
    w2 = r.standard_normal((1, h, f)) * 0.4
    w_r, keys = r.standard_normal((4, h)) * 0.3, r.standard_normal((1, 4))
    idx, gate, _, z = oracle.expert_route(y, w_r, keys, np.zeros(1), 1, 0, 3, normalize=False)
    yt = torch.from_numpy(y)
    for kind in ("swiglu", "gelu"):
        out = oracle.expert_ffn(kind, y, idx, gate, w1, w3, w2)
        if kind == "swiglu":
            hid = F.silu(F.linear(yt, torch.from_numpy(w1[0]))) * F.linear(yt, torch.from_numpy(w3[0]))
        else:
            hid = F.gelu(F.linear(yt, torch.from_numpy(w1[0])))
        mlp = F.linear(hid, torch.from_numpy(w2[0])).numpy()
        sig = 1.0 / (1.0 + np.exp(-z[:, 0]))
        assert np.allclose(out, sig[:, None] * mlp, atol=1e-12)


def test_grouped_experts_equal_per_token_loop():
    r = np.random.default_rng(11)
    T, h, f, E, k = 13, 8, 4, 5, 2
    x = r.standard_normal((T, h))
    w1, w3 = r.standard_normal((2, E, f, h))
    w2 = r.standard_normal((E, h, f))
    idx = np.stack([r.choice(E, k, replace=False) for _ in range(T)])
    gate = r.uniform(0.1, 1, (T, k))
    res = r.standard_normal((T, h))
    out = oracle.expert_ffn("swiglu", x, idx, gate, w1, w3, w2, residual=res)
    ref = res.copy()
    for t in range(T):
        for i in range(k):
            e = idx[t, i]
            a = w1[e] @ x[t]
            u = w3[e] @ x[t]
            ref[t] += gate[t, i] * (w2[e] @ (a / (1 + np.exp(-a)) * u))
    assert np.allclose(out, ref, atol=1e-12)
    wl = r.standard_normal((E, 3, h))
    lin = oracle.expert_ffn("linear", x, idx[:, :1], gate[:, :1], wl)
    ref_l = np.stack([gate[t, 0] * (wl[idx[t, 0]] @ x[t]) for t in range(T)])
    assert np.allclose(lin, ref_l, atol=1e-12)


def test_shared_expert_identity_top1():
    """sigma x W_e + max(sigma_hat) x W_sh == sigma x (W_e + W_sh) for top-1 ([PN] key design 3)."""
    cfg = CONFIGS["linear_moe"].replace(b=1, s=8, h=32, H=2, d=16, L=3, E=8, k=2, f=8, r=8,
                                        proj_experts=4, dtype="f32")
    W = oracle.prepare_weights(make_weights(cfg))
    x0 = make_x0(cfg).numpy()
    ref = oracle.layer_forward(cfg, W, x0)
    Wa = dict(W)
    for nm in ("qkv", "o"):
        Wa["w_%s_e" % nm] = W["w_%s_e" % nm] + W["w_%s_sh" % nm][None]
        Wa["w_%s_sh" % nm] = np.zeros_like(W["w_%s_sh" % nm])
    got = oracle.layer_forward(cfg, Wa, x0)
    assert np.array_equal(got["pidx"], ref["pidx"])
    assert np.allclose(got["x_out"], ref["x_out"], atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------------- layer

def test_layer_without_da_ea_is_plain_recurrent_attention_block():
    cfg = CONFIGS["tiny"].replace(use_da=False, use_ea=False, sa_rope=False, b=2, s=10)
    W = oracle.prepare_weights(make_weights(cfg))
    x0 = make_x0(cfg).numpy()
    got = oracle.layer_forward(cfg, W, x0)["x_out"]
    x = torch.from_numpy(x0.reshape(cfg.T, cfg.h).astype(np.float64))
    g = torch.from_numpy(W["g"])
    wq, wk, wv = (torch.from_numpy(W["w_qkv"][j * cfg.h:(j + 1) * cfg.h]) for j in range(3))
    wo = torch.from_numpy(W["w_o"][:, :cfg.h])
    for _ in range(cfg.L):
        xh = F.rms_norm(x, (cfg.h,), g, eps=cfg.rms_eps)
        sh = lambda a: a.reshape(cfg.b, cfg.s, cfg.H, cfg.d).transpose(1, 2)
        att = F.scaled_dot_product_attention(sh(F.linear(xh, wq)), sh(F.linear(xh, wk)),
                                             sh(F.linear(xh, wv)), is_causal=True)
        x = xh + F.linear(att.transpose(1, 2).reshape(cfg.T, cfg.h), wo)
    assert np.allclose(got, x.numpy(), atol=1e-11)


def test_layer_batch_independence():
    cfg = CONFIGS["tiny"].replace(b=3, s=6)
    W = oracle.prepare_weights(make_weights(cfg))
    x0 = make_x0(cfg).numpy()
    a = oracle.layer_forward(cfg, W, x0)["x_out"].reshape(3, 6, -1)
    b = oracle.layer_forward(cfg, W, x0[[2, 0, 1]])["x_out"].reshape(3, 6, -1)
    assert np.allclose(b, a[[2, 0, 1]], atol=1e-13)


def test_layer_depth_window_special_cases():
    # a window covering every depth is the full DA; a window of one makes DA return the
    # token's own value, the same layer as DA with keys restricted to the current slot
    cfg = CONFIGS["tiny"].replace(b=2, s=5, L=5)
    W = oracle.prepare_weights(make_weights(cfg))
    x0 = make_x0(cfg).numpy()
    full = oracle.layer_forward(cfg, W, x0)["x_out"]
    wide = oracle.layer_forward(cfg.replace(da_window=cfg.L, da_dilation=2), W, x0)["x_out"]
    assert np.array_equal(full, wide)
    one = oracle.layer_forward(cfg.replace(da_window=1), W, x0)["x_out"]
    dil = oracle.layer_forward(cfg.replace(da_window=2, da_dilation=2), W, x0)["x_out"]
    assert not np.allclose(one, full) and not np.allclose(dil, full)


@pytest.mark.parametrize("bf16", [False, True])
def test_prefill_then_decode_equals_longer_prefill(bf16):
    base_cfg = CONFIGS["decode"].replace(h=64, H=4, d=16, L=4, E=16, k=2, f=16, r=16,
                                         dtype="bf16" if bf16 else "f32")
    s = 7
    pre = base_cfg.replace(decode=False, b=2, s=s + 1, sa_pos=0)
    W = oracle.prepare_weights(make_weights(pre))
    x0 = make_x0(pre).numpy()                     # [2, s+1, h]
    full = oracle.layer_forward(pre, W, x0)["x_out"].reshape(2, s + 1, -1)
    short = pre.replace(s=s)
    cap = s + 1
    sk = np.full((short.L, 2, cap, short.H, short.d), np.nan)
    sv = np.full_like(sk, np.nan)
    oracle.layer_forward(short, W, x0[:, :s], sa_k=sk, sa_v=sv)
    dec = base_cfg.replace(b=2, s=1, decode=True, sa_pos=s)
    out = oracle.layer_forward(dec, W, x0[:, s], sa_k=sk, sa_v=sv)["x_out"]
    # float32 storage: identical up to float64 summation order; bf16 storage: one
    # rounding flip can move a value by a bf16 ulp, so compare at bf16 resolution
    assert np.allclose(out, full[:, s], atol=3e-2 if bf16 else 1e-11)


@pytest.mark.parametrize("bf16", [False, True])
def test_decode_loop_equals_longer_prefill(bf16):
    """Prefill of s tokens (writing the SA caches), then n decode steps = a prefill of
    s + n tokens, token by token (causality), and one step = one decode call."""
    base_cfg = CONFIGS["decode"].replace(h=64, H=4, d=16, L=3, E=16, k=2, f=16, r=16,
                                         dtype="bf16" if bf16 else "f32")
    s, n, b = 6, 4, 2
    pre = base_cfg.replace(decode=False, b=b, s=s + n, sa_pos=0)
    W = oracle.prepare_weights(make_weights(pre))
    x0 = make_x0(pre).numpy()                      # [b, s+n, h]
    full = oracle.layer_forward(pre, W, x0)["x_out"].reshape(b, s + n, -1)
    cap = s + n
    sk = np.full((pre.L, b, cap, pre.H, pre.d), np.nan)
    sv = np.full_like(sk, np.nan)
    oracle.layer_forward(pre.replace(s=s), W, x0[:, :s], sa_k=sk, sa_v=sv)
    dec = base_cfg.replace(b=b, s=1, decode=True, sa_pos=s)
    k0, v0 = sk.copy(), sv.copy()
    got = oracle.decode_tokens(dec, W, x0[:, s:].transpose(1, 0, 2), sk, sv)["x_out"]
    assert np.allclose(got.transpose(1, 0, 2), full[:, s:], atol=3e-2 if bf16 else 1e-11)
    assert np.isfinite(sk[:, :, :cap]).all()       # every position appended
    one = oracle.layer_forward(dec, W, x0[:, s], sa_k=k0, sa_v=v0)["x_out"]
    assert np.array_equal(one, got[0])


def test_decode_da_cache_overwritten_before_read():
    cfg = CONFIGS["decode"].replace(h=64, H=4, d=16, L=3, E=8, k=2, f=8, r=16, b=2, sa_pos=3,
                                    dtype="f32")
    W = oracle.prepare_weights(make_weights(cfg))
    x0 = make_x0(cfg).numpy()
    r = np.random.default_rng(12)
    sk = r.standard_normal((cfg.L, 2, 4, cfg.H, cfg.d))
    sv = r.standard_normal((cfg.L, 2, 4, cfg.H, cfg.d))
    out = oracle.layer_forward(cfg, W, x0, sa_k=sk.copy(), sa_v=sv.copy())["x_out"]
    assert np.isfinite(out).all()   # layer_forward starts from NaN DA caches


def test_bf16_emulation_rounds_storage_points():
    cfg = CONFIGS["small"].replace(b=1, s=8, L=2)
    W = oracle.prepare_weights(make_weights(cfg))
    x0 = make_x0(cfg).numpy()
    out = oracle.layer_forward(cfg, W, x0, return_steps=True)
    yb = out["steps"][1]["yb"]
    assert np.array_equal(yb, oracle.bf16_round(yb))
    assert not np.array_equal(out["steps"][1]["y"], yb)


def test_golden_tiny_regression():
    """Stored oracle output of the tiny workload (written by tests/golden/make_golden.py,
    which calls only the oracle): guards the oracle against silent drift."""
    data = np.load(os.path.join(GOLDEN, "tiny_oracle.npz"))
    cfg = CONFIGS["tiny"]
    W = oracle.prepare_weights(make_weights(cfg))
    r = oracle.layer_forward(cfg, W, make_x0(cfg).numpy())
    assert np.allclose(r["x_out"], data["x_out"], atol=1e-12, rtol=0)
    assert np.array_equal(r["idx"], data["idx"])


# ------------------------------------------------------------------------ mixture wirings

def _layer(cfg, W=None, x0=None):
    W = make_weights(cfg) if W is None else W
    x0 = make_x0(cfg) if x0 is None else x0
    return oracle.layer_forward(cfg, oracle.prepare_weights(W), x0.numpy())["x_out"]


def test_mixtures_coincide_where_their_definitions_do():
    base = CONFIGS["tiny"].replace(b=2, s=9, L=3)
    # no DA: serial (DA -> SA -> EA) is the default wiring; no EA: so is the fully
    # parallel one
    for mix, kw in (("serial", dict(use_da=False)), ("parallel", dict(use_ea=False))):
        c = base.replace(**kw)
        assert np.array_equal(_layer(c.replace(mixture=mix)), _layer(c))
    # zero output projections: every wiring reduces to x' = x^ + EA(x^) at every depth
    W = make_weights(base)
    W["w_o"] = torch.zeros_like(W["w_o"])
    outs = [_layer(base.replace(mixture=m), W) for m in ("partial", "serial", "parallel")]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    # in general the three differ
    outs = [_layer(base.replace(mixture=m)) for m in ("partial", "serial", "parallel")]
    for i, j in ((0, 1), (0, 2), (1, 2)):
        assert np.abs(outs[i] - outs[j]).max() > 1e-3


def _sa_torch(u, W, cfg):
    """Causal SDPA over RoPE'd q, k (complex-rotation form) from rows 0..3h of w_qkv."""
    h = cfg.h
    return _sa_torch_qkv(*(u @ W["w_qkv"][j * h:(j + 1) * h].T for j in range(3)), cfg)


def _sa_torch_qkv(q, k, v, cfg):
    """Causal SDPA of projections q, k, v [T, h] after RoPE (complex-rotation form)."""
    h, H, d = cfg.h, cfg.H, cfg.d
    pos = (np.arange(cfg.T) % cfg.s).astype(np.float64)[:, None, None]
    q = _rope_complex(q.reshape(cfg.T, H, d), pos, cfg.rope_base)
    k = _rope_complex(k.reshape(cfg.T, H, d), pos, cfg.rope_base)
    sh = lambda a: torch.from_numpy(np.ascontiguousarray(
        a.reshape(cfg.b, cfg.s, H, d).transpose(0, 2, 1, 3)))
    att = F.scaled_dot_product_attention(sh(q), sh(k), sh(v), is_causal=True)
    return att.numpy().transpose(0, 2, 1, 3).reshape(cfg.T, h)


def test_serial_wiring_one_depth_closed_form():
    """L = 1, float32 storage, no EA: DA over one depth returns its value projection, so
    u = x^ + (x^ W_V^DA) W_O^DA; then x_1 = u + SA(u) W_O^SA with SA as torch SDPA."""
    cfg = CONFIGS["tiny"].replace(b=2, s=7, L=1, use_ea=False, mixture="serial")
    W = oracle.prepare_weights(make_weights(cfg))
    x0 = make_x0(cfg).numpy().reshape(cfg.T, cfg.h)
    got = oracle.layer_forward(cfg, W, x0)["x_out"]
    h = cfg.h
    xh = F.rms_norm(torch.from_numpy(x0.astype(np.float64)), (h,),
                    torch.from_numpy(W["g"]), eps=cfg.rms_eps).numpy()
    u = xh + (xh @ W["w_qkv"][5 * h:6 * h].T) @ W["w_o"][:, h:].T
    ref = u + _sa_torch(u, W, cfg) @ W["w_o"][:, :h].T
    assert np.allclose(got, ref, atol=1e-11)


def test_parallel_wiring_one_depth_closed_form():
    """L = 1, float32 storage, no DA: x_1 = x^ + SA(x^) W_O^SA + g * FFN_e(x^), with the
    top-1 expert e and its gate g computed here from the router's definition (depth RoPE
    at l = 0, L = 1 is the identity)."""
    cfg = CONFIGS["tiny"].replace(b=2, s=7, L=1, use_da=False, mixture="parallel")
    W = oracle.prepare_weights(make_weights(cfg))
    x0 = make_x0(cfg).numpy().reshape(cfg.T, cfg.h)
    got = oracle.layer_forward(cfg, W, x0)["x_out"]
    h = cfg.h
    xh = F.rms_norm(torch.from_numpy(x0.astype(np.float64)), (h,),
                    torch.from_numpy(W["g"]), eps=cfg.rms_eps).numpy()
    z = cfg.rho * (xh @ W["w_r"].T) @ W["keys"].T
    e = np.argmax(z + W["bias"][None, :], axis=1)
    g = 1.0 / (1.0 + np.exp(-z[np.arange(cfg.T), e]))
    ffn = np.stack([W["w2"][e[t]] @ (0.5 * (W["w1"][e[t]] @ xh[t]) *
                                     (1 + np.vectorize(math.erf)((W["w1"][e[t]] @ xh[t]) /
                                                                 math.sqrt(2))))
                    for t in range(cfg.T)])
    ref = xh + _sa_torch(xh, W, cfg) @ W["w_o"][:, :h].T + g[:, None] * ffn
    assert np.allclose(got, ref, atol=1e-11)


# ------------------------------------------------------------ linear-MoE projections

def test_linear_moe_one_depth_closed_form():
    """L = 1, float32 storage, no EA ([PN] "Key design 3"; reading R12).  The projection
    router's scores come from its definition, z = rho (x^ W_P^T) K_P^T (depth RoPE at
    l = 0 of L = 1 rotates by zero); each token takes e* = argmax z with gate
    sigma = sigmoid(z_e*), and every projection is sigma x (W_e* + W_sh).  DA over one
    depth returns its value projection; SA is torch SDPA.  Dropping sigma, or using the
    gate of another expert, fails this."""
    cfg = CONFIGS["linear_moe"].replace(b=2, s=7, h=32, H=2, d=16, L=1, E=8, k=2, f=8, r=8,
                                        proj_experts=4, dtype="f32", use_ea=False)
    W = oracle.prepare_weights(make_weights(cfg))
    x0 = make_x0(cfg).numpy().reshape(cfg.T, cfg.h)
    got = oracle.layer_forward(cfg, W, x0)
    h, T = cfg.h, cfg.T
    xh = F.rms_norm(torch.from_numpy(x0.astype(np.float64)), (h,),
                    torch.from_numpy(W["g"]), eps=cfg.rms_eps).numpy()
    z = cfg.rho * (xh @ W["w_pr"].T) @ W["pkeys"].T
    e = np.argmax(z, axis=1)
    assert len(set(e.tolist())) > 1            # the per-token expert choice matters here
    sig = 1.0 / (1.0 + np.exp(-z[np.arange(T), e]))
    assert np.array_equal(got["pidx"][0], e)
    assert np.allclose(got["pgate"][0], sig, atol=1e-15)

    def layer(gate):
        Wq = W["w_qkv_e"][e] + W["w_qkv_sh"][None]           # [T, 6h, h], per token
        qkv = gate[:, None] * np.einsum("tnj,tj->tn", Wq, xh)
        a_sa = _sa_torch_qkv(qkv[:, :h], qkv[:, h:2 * h], qkv[:, 2 * h:3 * h], cfg)
        att = np.concatenate([a_sa, qkv[:, 5 * h:6 * h]], axis=1)
        Wo = W["w_o_e"][e] + W["w_o_sh"][None]              # [T, h, 2h]
        return xh + gate[:, None] * np.einsum("tnj,tj->tn", Wo, att)

    assert np.allclose(got["x_out"], layer(sig), atol=1e-11)
    assert np.abs(layer(np.ones(T)) - got["x_out"]).max() > 1e-3     # sigma is not vacuous
