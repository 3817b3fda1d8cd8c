"""GPU parity of each C-ABI entry point against the CPU oracle (same seeded inputs).

Tolerances: float32 storage -> max|err| / max|ref| <= 1e-5.  bf16 storage -> the oracle
rounds at the same storage points, so outputs must agree to 1-2 bf16 ulps, plus a term
for the one internal rounding the oracle does not model (bf16 softmax weights inside the
MFMA attention kernel: |dP| <= 2^-8 P, hence a per-element |dO| <= 2^-8 (sum p|v| / sum p
+ |o|) / (1 - 2^-8)), and, in depth attention, a term of 2^-8 max|v| for one-ulp
differences of the independently rounded rotated q and k.  Routing: the selected
sets must be identical except where the oracle's k-th and (k+1)-th biased scores are within
1e-6; gates to 1e-5 relative."""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close_ulps, bf16_ulp, rel_err, routing_mismatch
from synth import CONFIGS, make_bias, rng

pytestmark = pytest.mark.gpu


def _t(shape, seed, tid, std=1.0, dtype=torch.bfloat16):
    return rng.normal(shape, seed, tid, std, dtype).cuda()


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


TD = {"bf16": torch.bfloat16, "f32": torch.float32}


# ------------------------------------------------------------------------ depth attention

@pytest.mark.parametrize("dt,H,d,rows,L", [("bf16", 8, 64, 300, 8), ("f32", 4, 16, 37, 4),
                                           ("bf16", 32, 64, 70, 64), ("bf16", 4, 16, 50, 5),
                                           ("f32", 2, 64, 9, 3)])
def test_depth_attn(gpu_lib, dt, H, d, rows, L):
    _depth_attn_case(gpu_lib, dt, H, d, rows, L)


# windowed / dilated key sets: window 3 dilation 4 over 12 depths, window 2 dilation 3,
# window 1 (DA returns v), a window without dilation, a window wider than L
@pytest.mark.parametrize("dt,H,d,rows,L,window,dilation", [
    ("bf16", 8, 64, 300, 12, 3, 4), ("f32", 4, 16, 37, 10, 2, 3), ("bf16", 4, 64, 70, 9, 1, 0),
    ("f32", 2, 16, 20, 6, 3, 0), ("bf16", 8, 64, 100, 8, 9, 2)])
def test_depth_attn_windowed(gpu_lib, dt, H, d, rows, L, window, dilation):
    _depth_attn_case(gpu_lib, dt, H, d, rows, L, window, dilation)


def _depth_attn_case(D, dt, H, d, rows, L, window=None, dilation=0):
    tdt, bf = TD[dt], dt == "bf16"
    print(f"depth_attn {dt} H={H} d={d} rows={rows} L={L} window={window} dilation={dilation}",
          flush=True)
    cos, sin = D.dreamer_rope_tables(d, L)
    kc = torch.full((rows, L, H, d), float("nan"), dtype=tdt, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    kc_full, vc_full = kc.clone(), vc.clone()
    rk = np.full((rows, L, H, d), np.nan)
    rv = np.full_like(rk, np.nan)
    for l in range(L):
        q, k, v = (_t((rows, H, d), 7, 100 + 3 * l + j, dtype=tdt) for j in range(3))
        out = D.dreamer_depth_attn(q, k, v, kc, vc, l, L, cos, sin, window=window,
                                   dilation=dilation)
        ref = oracle.depth_attn(_np(q), _np(k), _np(v), rk, rv, l, L, bf16=bf,
                                window=window or 0, dilation=dilation)
        torch.cuda.synchronize()
        g = _np(out)
        if l == 0 or window == 1:
            assert torch.equal(out, v), "a single key must return v exactly"
        if window is not None and window >= L:
            full = D.dreamer_depth_attn(q, k, v, kc_full, vc_full, l, L, cos, sin)
            assert torch.equal(out, full), "a window over every depth is the full DA"
        assert np.isfinite(g).all()
        if bf:
            # rotated q and k are a bf16 storage point rounded independently on each side;
            # a one-ulp flip moves a score by <= |q_i k_i| 2^-7 / sqrt(d), which moves the
            # output by a small multiple of 2^-8 max|v|
            vmax = np.abs(_np(v)).max()
            assert_close_ulps(g, ref, ulps=2, atol=2.0 ** -8 * vmax, what=f"DA out l={l}")
            # x cos - y sin in float32 is off by <= 2^-23 (|x| + |y|) before rounding, which
            # matters where the two products cancel; inputs here are |x|, |y| < 8
            assert_close_ulps(_np(kc[:, l]), rk[:, l], ulps=1, atol=2.0 ** -20,
                              what="rotated key")
        else:
            assert rel_err(g, ref) <= 1e-5
            assert rel_err(_np(kc[:, l]), rk[:, l]) <= 1e-6
        assert torch.equal(vc[:, l], v)


# ---------------------------------------------------------------------- sequence attention

@pytest.mark.parametrize("dt,B,S,H,d,rope", [("bf16", 2, 200, 4, 64, True),
                                             ("bf16", 1, 64, 2, 64, False),
                                             ("bf16", 3, 1, 2, 64, True),
                                             ("f32", 2, 37, 4, 16, True),
                                             ("bf16", 2, 45, 2, 16, True),
                                             # two query sets per wave (> 64 rows): a
                                             # ragged last block, one set past the end,
                                             # and a long sequence of 32 blocks
                                             ("bf16", 2, 300, 4, 64, True),
                                             ("bf16", 1, 72, 2, 64, False),
                                             ("bf16", 1, 4096, 2, 64, True)])
def test_seq_attn_prefill(gpu_lib, dt, B, S, H, d, rope):
    D = gpu_lib
    tdt, bf = TD[dt], dt == "bf16"
    print(f"seq_attn prefill {dt} B={B} S={S} H={H} d={d} rope={rope}", flush=True)
    q, k, v = (_t((B, S, H, d), 11, j, dtype=tdt) for j in range(3))
    cos, sin = D.dreamer_rope_tables(d, S)
    cap = S + 3
    kc = torch.full((B, cap, H, d), float("nan"), dtype=tdt, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    out = D.dreamer_seq_attn(q, k, v, 0, kc, vc, cos, sin, sa_rope=rope)
    ref, krot, _ = oracle.seq_attn(_np(q), _np(k), _np(v), 0, None, None, rope, 1e4, bf)
    torch.cuda.synchronize()
    g = _np(out)
    if bf:
        # Every softmax weight enters P.V rounded to bf16 (relative error <= u = 2^-8), and
        # the denominator is summed from the same rounded weights, so out = sum p~ v / sum p~
        # lies within u / (1 - u) * (sum p |v| / sum p + |o|) of the exact o, per element;
        # sum p |v| / sum p is the oracle's attention over |v|.  With RoPE, q and k are
        # rounded after the rotation on each side, and a rare one-ulp difference moves a
        # score by up to about as much again.
        vabs, _, _ = oracle.seq_attn(_np(q), _np(k), np.abs(_np(v)), 0, None, None, rope, 1e4,
                                     bf)
        u = 2.0 ** -8
        bound = (2.0 if rope else 1.0) * u / (1 - u) * (vabs + np.abs(ref))
        assert_close_ulps(g, ref, ulps=2, atol=bound, what="SA prefill")
        lim = 2 * bf16_ulp(ref) + bound
        print(f"  worst err / bound {(np.abs(g - ref) / lim).max():.3f}", flush=True)
        assert_close_ulps(_np(kc[:, :S]), krot, ulps=1, atol=2.0 ** -20, what="SA cache keys")
    else:
        assert rel_err(g, ref) <= 1e-5
        assert rel_err(_np(kc[:, :S]), krot) <= 1e-6
    assert torch.equal(vc[:, :S], v)
    assert torch.isnan(kc[:, S:]).all()


def test_seq_attn_causal_perturbation(gpu_lib):
    D = gpu_lib
    B, S, H, d = 1, 150, 2, 64
    q, k, v = (_t((B, S, H, d), 12, j) for j in range(3))
    cos, sin = D.dreamer_rope_tables(d, S)
    a = D.dreamer_seq_attn(q, k, v, cos_s=cos, sin_s=sin)
    k2, v2 = k.clone(), v.clone()
    k2[:, 100:] += 1.0
    v2[:, 100:] -= 1.0
    b = D.dreamer_seq_attn(q, k2, v2, cos_s=cos, sin_s=sin)
    torch.cuda.synchronize()
    assert torch.equal(a[:, :100], b[:, :100])


@pytest.mark.parametrize("dt,B,P,H,d", [("bf16", 3, 300, 4, 64), ("bf16", 2, 1000, 32, 64),
                                        ("f32", 2, 50, 4, 16)])
def test_seq_attn_decode(gpu_lib, dt, B, P, H, d):
    D = gpu_lib
    tdt, bf = TD[dt], dt == "bf16"
    print(f"seq_attn decode {dt} B={B} P={P} H={H} d={d}", flush=True)
    kc = _t((B, P + 2, H, d), 13, 0, dtype=tdt)
    vc = _t((B, P + 2, H, d), 13, 1, dtype=tdt)
    kc[:, P:] = float("nan")
    vc[:, P:] = float("nan")
    q, k, v = (_t((B, 1, H, d), 13, 2 + j, dtype=tdt) for j in range(3))
    cos, sin = D.dreamer_rope_tables(d, P + 1)
    rkc, rvc = _np(kc), _np(vc)
    out = D.dreamer_seq_attn(q, k, v, P, kc, vc, cos, sin)
    ref, krot, _ = oracle.seq_attn(_np(q), _np(k), _np(v), P, rkc, rvc, True, 1e4, bf)
    torch.cuda.synchronize()
    if bf:
        assert_close_ulps(_np(out), ref, ulps=2, atol=2.0 ** -20, what="SA decode")
        assert_close_ulps(_np(kc[:, P:P + 1]), krot, ulps=1, atol=2.0 ** -20,
                          what="appended key")
    else:
        assert rel_err(_np(out), ref) <= 1e-5
    assert torch.equal(vc[:, P:P + 1], v)
    assert torch.isnan(kc[:, P + 1]).all()


# ------------------------------------------------------------------------------- routing

@pytest.mark.parametrize("dt,T,h,r,E,k,norm,bias", [
    ("bf16", 333, 512, 64, 256, 4, True, 0.2),
    ("f32", 16, 64, 16, 16, 1, False, 0.1),
    ("bf16", 200, 2048, 64, 4096, 8, True, 0.2),
    ("bf16", 150, 1024, 64, 16, 1, False, 0.0),
    ("bf16", 64, 256, 32, 32, 32, True, 0.2),      # k == E: every expert selected
    ("bf16", 120, 512, 64, 112, 16, True, 0.2),    # k = 16, a partial last expert quarter
    ("f32", 50, 64, 16, 100, 13, True, 0.1),       # E not a multiple of 16, odd k
    ("bf16", 100, 512, 64, 8192, 8, True, 0.2),    # few tokens: two chunks per expert range
    # >= 1024 tokens: scores and selection in one kernel (ragged last block of 16 tokens)
    ("bf16", 1037, 512, 64, 256, 4, True, 0.2),
    ("bf16", 1030, 1024, 128, 1024, 8, True, 0.2),  # four chunks of 256 experts
    ("bf16", 1100, 512, 64, 272, 2, True, 0.2),     # a last chunk of 16 experts
    ("bf16", 1024, 256, 32, 48, 1, False, 0.0),     # one partial chunk, top-1
    ("bf16", 1040, 1024, 64, 16, 1, False, 0.0),    # the linear-MoE projection router
    # the deep workload's router: h = 2048, E = 2048 top-8, Zipf-skewed bias, its weight
    # scale, at depth 40 of 64 (fused scores + selection, T >= 1024)
    ("bf16", 1100, 2048, 64, 2048, 8, True, "zipf"),
])
def test_expert_route(gpu_lib, dt, T, h, r, E, k, norm, bias):
    D = gpu_lib
    tdt = TD[dt]
    print(f"route {dt} T={T} h={h} r={r} E={E} k={k} bias={bias}", flush=True)
    x = _t((T, h), 21, 0, 1.0, tdt)
    std = 0.02 if bias == "zipf" else 0.05
    w_r = _t((r, h), 21, 1, std, tdt)
    keys = _t((E, r), 21, 2, std, tdt)
    l, L = 2, 5
    if bias == "zipf":
        b = make_bias(CONFIGS["deep"]).cuda()
        l, L = 40, 64
    elif bias:
        b = rng.uniform((E,), 21, 3, -bias, bias).cuda()
    else:
        b = torch.zeros(E, device="cuda")
    cos, sin = D.dreamer_rope_tables(r, L)
    idx, gate, counts = D.dreamer_expert_route(x, w_r, keys, b, k, l, L, cos, sin, 1.0, norm)
    ridx, rgate, rcounts, z = oracle.expert_route(_np(x), _np(w_r), _np(keys), _np(b), k, l, L,
                                                  1.0, norm)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    n_bad, n_ex = routing_mismatch(gi, z, _np(b), k)
    assert n_bad == 0, f"{n_bad} tokens routed differently ({n_ex} exempt ties)"
    assert np.array_equal(counts.cpu().numpy(), np.bincount(gi.reshape(-1), minlength=E))
    # gates by expert id, on tokens with the same set
    gg = gate.cpu().numpy()
    for t in range(T):
        if set(gi[t]) != set(ridx[t]):
            continue
        gmap = dict(zip(gi[t], gg[t]))
        for e, rv in zip(ridx[t], rgate[t]):
            assert abs(gmap[e] - rv) <= 1e-5 * abs(rv) + 1e-7
    # descending order of the biased score on the GPU side
    key = z + _np(b)[None, :]
    ks = np.take_along_axis(key, gi.astype(np.int64), axis=1)
    assert (np.diff(ks, axis=1) <= 1e-6).all()


@pytest.mark.parametrize("T,E,tied", [(40, 16, (3, 7, 9)), (1040, 16, (3, 7, 9)),
                                       (40, 256, (5, 70, 200)), (1040, 512, (5, 300, 260)),
                                       (40, 1024, (700, 5, 300))])
def test_expert_route_ties_go_to_lower_index(gpu_lib, T, E, tied):
    """Identical experts (same key, same bias) in one or in different expert chunks or
    quarters of the selection: they win in index order."""
    D = gpu_lib
    h, r = 128, 32
    x = _t((T, h), 22, 0)
    w_r = _t((r, h), 22, 1, 0.05)
    keys = _t((E, r), 22, 2, 0.05)
    for e in tied[1:]:
        keys[e] = keys[tied[0]]
    b = torch.zeros(E, device="cuda")
    for e in tied:
        b[e] = 5.0  # the identical experts win, in index order
    cos, sin = D.dreamer_rope_tables(r, 3)
    idx, _, _ = D.dreamer_expert_route(x, w_r, keys, b, 2, 1, 3, cos, sin)
    torch.cuda.synchronize()
    first, second = sorted(tied)[:2]
    assert (idx[:, 0] == first).all() and (idx[:, 1] == second).all()


# ------------------------------------------------------------------------------- experts

def _routing(T, E, k, seed, skew=False):
    g = torch.Generator().manual_seed(seed)
    idx = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)
    if skew:  # a third of the tokens send their first slot to expert 0 (one big group)
        idx[: T // 3, 0] = 0
        for t in range(T // 3):
            row = idx[t]
            dup = (row[1:] == 0).nonzero()
            for j in dup.flatten().tolist():
                row[1 + j] = (E - 1) if row[0] != E - 1 else 1
    gate = torch.rand((T, k), generator=g) * 0.9 + 0.1
    return idx.cuda(), gate.cuda()


@pytest.mark.parametrize("dt,kind,T,h,f,E,k,skew", [
    ("bf16", "swiglu", 300, 512, 64, 256, 4, False),
    ("bf16", "swiglu", 100, 1024, 128, 64, 8, True),
    ("bf16", "gelu", 77, 256, 64, 8, 2, False),
    ("bf16", "gelu", 150, 512, 128, 16, 4, True),     # wide GELU: activation-sized stages
    ("bf16", "swiglu", 64, 2048, 128, 8, 2, False),   # long GEMM1 K loop
    ("bf16", "linear", 130, 256, 0, 16, 1, True),
    ("f32", "gelu", 16, 64, 32, 16, 1, False),
    ("f32", "swiglu", 20, 64, 32, 8, 2, False),
    ("bf16", "swiglu", 4500, 256, 64, 64, 8, True),   # > 32768 slots: chunked grouping
])
def test_expert_ffn(gpu_lib, dt, kind, T, h, f, E, k, skew):
    D = gpu_lib
    tdt, bf = TD[dt], dt == "bf16"
    print(f"expert_ffn {dt} {kind} T={T} h={h} f={f} E={E} k={k}", flush=True)
    x = _t((T, h), 31, 0, 1.0, tdt)
    idx, gate = _routing(T, E, k, 31, skew)
    res = _t((T, h), 31, 1, 1.0, torch.float32)
    if kind == "linear":
        w1, w3, w2 = _t((E, h, h), 31, 2, 0.05, tdt), None, None
    else:
        w1 = _t((E, f, h), 31, 2, 0.05, tdt)
        w3 = _t((E, f, h), 31, 3, 0.05, tdt) if kind == "swiglu" else None
        w2 = _t((E, h, f), 31, 4, 0.05, tdt)
    out = D.dreamer_expert_ffn(kind, x, idx, gate, w1, w3, w2, res)
    ref, slots, hid = oracle.expert_ffn(kind, _np(x), idx.cpu().numpy(), _np(gate), _np(w1),
                                        None if w3 is None else _np(w3),
                                        None if w2 is None else _np(w2), residual=_np(res),
                                        bf16=bf, return_parts=True)
    torch.cuda.synchronize()
    g = _np(out)
    if bf:
        # Per element, from the oracle's own stored values.  Both sides round the hidden
        # state and the gated slot outputs to bf16 at the same points.  A stored hidden
        # element h differs by at most one rounding step (<= 2^-7 |h|) plus the float32
        # error of its GEMM (<= one more such step unless the GEMM's terms cancel, so
        # 2^-6 |h| in all), which moves an output by <= 2^-6 sum_j |h_j| |W2_mj| times the
        # gate; a LINEAR slot carries the float32 error of its one GEMM instead
        # (<= h_in 2^-24 sum_c |x_c| |W1_mc|).  A slot differs by one more rounding step
        # (<= 2^-7 |slot|); the float32 sum of residual and k slots adds (k+1) 2^-24 of its
        # absolute terms.
        ii = idx.cpu().numpy()
        gt = _np(gate)
        xa = np.abs(_np(x))
        Wa = np.abs(_np(w1) if kind == "linear" else _np(w2))    # [E, h_out, h_in or f]
        gemm = np.zeros_like(slots)
        for e in np.unique(ii):
            tt, kk = np.nonzero(ii == e)
            if kind == "linear":
                gemm[tt, kk] = (xa[tt] @ Wa[e].T) * (h * 2.0 ** -24)
            else:
                gemm[tt, kk] = (np.abs(hid[tt, kk]) @ Wa[e].T) * 2.0 ** -6
        bound = (2.0 ** -7 * np.abs(slots) + gt[..., None] * gemm).sum(axis=1)
        bound += (k + 1) * 2.0 ** -24 * (np.abs(_np(res)) + np.abs(slots).sum(axis=1))
        err = np.abs(g - ref)
        bad = err > bound
        assert not bad.any(), (f"{bad.sum()} of {bad.size} elements beyond their bound; "
                               f"worst err/bound {(err / bound).max():.2f}")
        print(f"  worst err/bound {(err / bound).max():.3f}", flush=True)
    else:
        assert rel_err(g, ref) <= 1e-5
    # no routing: out == residual exactly when every gate is zero
    out0 = D.dreamer_expert_ffn(kind, x, idx, torch.zeros_like(gate), w1, w3, w2, res)
    torch.cuda.synchronize()
    assert torch.equal(out0, res)


@pytest.mark.parametrize("T,n", [(4500, 4000), (129, 128)])
def test_expert_ffn_grouping_paths_same_bits(gpu_lib, T, n):
    # T tokens x top-8 and their first n tokens are grouped with different chunk counts
    # (36 vs 32 chunks of 1024 slots; 1032 slots in two chunks vs 1024 in the one-block
    # launch): every token's output is the same bits either way
    D = gpu_lib
    h, f, E, k = 256, 64, 64, 8
    x = _t((T, h), 33, 0, 1.0, torch.bfloat16)
    idx, gate = _routing(T, E, k, 33, True)
    res = _t((T, h), 33, 1, 1.0, torch.float32)
    w1, w3 = _t((E, f, h), 33, 2, 0.05, torch.bfloat16), _t((E, f, h), 33, 3, 0.05, torch.bfloat16)
    w2 = _t((E, h, f), 33, 4, 0.05, torch.bfloat16)
    full = D.dreamer_expert_ffn("swiglu", x, idx, gate, w1, w3, w2, res)
    part = D.dreamer_expert_ffn("swiglu", x[:n].contiguous(), idx[:n].contiguous(),
                                gate[:n].contiguous(), w1, w3, w2, res[:n].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(full[:n], part)


def test_absorb_shared_exact(gpu_lib):
    D = gpu_lib
    we = _t((4, 64, 32), 41, 0, 0.02)
    ws = _t((64, 32), 41, 1, 0.02)
    got = D.dreamer_absorb_shared(we, ws)
    torch.cuda.synchronize()
    ref = (we.float() + ws.float()[None]).to(torch.bfloat16)
    assert torch.equal(got, ref)


def test_errors_are_reported(gpu_lib):
    D = gpu_lib
    q = torch.zeros((4, 2, 64), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((4, 3, 2, 64), dtype=torch.bfloat16, device="cuda")
    cos, sin = D.dreamer_rope_tables(64, 3)
    with pytest.raises(D.DreamerError) as ei:
        D.dreamer_depth_attn(q, q, q, kc, kc, 3, 3, cos, sin)   # l >= L
    assert ei.value.code == D.E_INVAL
    q2 = torch.zeros((4, 2, 24), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(D.DreamerError) as ei:
        D.dreamer_depth_attn(q2, q2, q2, kc[..., :24].contiguous(), kc[..., :24].contiguous(),
                             0, 3, cos, sin)
    assert ei.value.code == D.E_UNSUPPORTED
    with pytest.raises(D.DreamerError) as ei:
        D.dreamer_depth_attn(q, q, q, kc, kc, 1, 3, cos, sin, window=-1)
    assert ei.value.code == D.E_INVAL


# ------------------------------------------------------------- expert-load bookkeeping

def test_route_counts_match_oracle(gpu_lib):
    D = gpu_lib
    g = torch.Generator().manual_seed(3)
    L, n, E = 3, 5000, 300
    idx = torch.randint(0, E, (L, n), generator=g, dtype=torch.int32)
    idx[1, :2000] = 7                                         # one hot expert
    got = D.dreamer_route_counts(idx.cuda(), E, n_sets=L).cpu().numpy()
    assert np.array_equal(got, oracle.route_counts(idx.numpy()[:, None, :], E))
    one = D.dreamer_route_counts(idx.reshape(-1).cuda(), E).cpu().numpy()[0]
    assert np.array_equal(one, np.bincount(idx.numpy().reshape(-1), minlength=E))


@pytest.mark.parametrize("E", [257, 256, 4096])
def test_bias_update_matches_oracle(gpu_lib, E):
    D = gpu_lib
    g = torch.Generator().manual_seed(E)
    counts = torch.randint(0, 40, (E,), generator=g, dtype=torch.int32)   # many ties
    bias = (torch.rand(E, generator=g) - 0.5) * 0.4
    lam = 0.01
    got = D.dreamer_bias_update(counts.cuda(), bias.clone().cuda(), lam).cpu().numpy()
    sgn = np.sign(np.median(counts.numpy()) - counts.numpy())
    want32 = (bias.numpy() + np.float32(lam) * sgn.astype(np.float32)).astype(np.float32)
    assert np.array_equal(got, want32)                        # same float32 operations
    ref = oracle.bias_update(bias.numpy().astype(np.float64), counts.numpy(), lam)
    assert np.abs(got - ref).max() <= 1e-7


def test_expert_usage_matches_oracle(gpu_lib):
    D = gpu_lib
    g = torch.Generator().manual_seed(9)
    sets = [torch.randint(0, 50, (256,), generator=g), torch.zeros(256, dtype=torch.int64),
            torch.full((256,), 4)]
    sets[1][17] = 1000                                        # one expert holds everything
    counts = torch.stack(sets).to(torch.int32)
    got = D.dreamer_expert_usage(counts.cuda()).cpu().numpy()
    for s in range(3):
        ref = oracle.expert_usage(counts[s].numpy())
        assert got[s, 0] == ref["distinct"]
        assert abs(got[s, 1] - ref["max_over_mean"]) <= 1e-6 * ref["max_over_mean"]
        assert abs(got[s, 2] - ref["gini"]) <= 1e-6 * max(ref["gini"], 1e-6)
    assert got[2, 2] == 0.0


def test_bias_balancing_reduces_imbalance(gpu_lib):
    """Repeated b <- b + lam sign(median(N) - N) on a fixed batch evens the load out."""
    D = gpu_lib
    T, h, r, E, k = 2048, 256, 64, 64, 2
    x = _t((T, h), 31, 0, 1.0, torch.bfloat16)
    w_r = _t((r, h), 31, 1, 0.05, torch.bfloat16)
    keys = _t((E, r), 31, 2, 0.3, torch.bfloat16)
    bias = torch.zeros(E, device="cuda")
    cos, sin = D.dreamer_rope_tables(r, 4)
    ginis = []
    for it in range(40):
        idx, _, counts = D.dreamer_expert_route(x, w_r, keys, bias, k, 1, 4, cos, sin, 1.0, True)
        ginis.append(float(D.dreamer_expert_usage(counts.reshape(1, E))[0, 2]))
        D.dreamer_bias_update(counts, bias, 0.02)
    torch.cuda.synchronize()
    print(f"Gini {ginis[0]:.3f} -> {ginis[-1]:.3f}")
    assert ginis[0] > 0.1 and min(ginis[-5:]) < 0.6 * ginis[0]
