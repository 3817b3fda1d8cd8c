"""Shared test plumbing: workload -> library config, weight upload, comparisons."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from synth import make_weights, make_x0


def bf16_ulp(ref):
    """One bf16 ulp of each reference value (for |v| >= 2^-126)."""
    a = np.maximum(np.abs(np.asarray(ref, np.float64)), 1e-30)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def assert_close_ulps(got, ref, ulps=1.0, atol=0.0, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    lim = ulps * bf16_ulp(ref) + atol
    bad = err > lim
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} beyond {ulps} ulp + {atol}; "
                           f"worst err {err.max():.3e} at ref {ref.flat[np.argmax(err - lim)]:.4e}")


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def rms_normed(x):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-6)


def lib_cfg(D, cfg, sa_cap=0, streams=False, fuse_attn=True):
    return D.make_layer_cfg(dtype=cfg.dtype, b=cfg.b, s=cfg.s, h=cfg.h, H=cfg.H, d=cfg.d, L=cfg.L,
                            E=cfg.E, k=cfg.k, f=cfg.f, r=cfg.r, ffn=cfg.ffn,
                            normalize=cfg.normalize, use_da=cfg.use_da, use_ea=cfg.use_ea,
                            sa_rope=cfg.sa_rope, proj_experts=cfg.proj_experts,
                            decode=cfg.decode, sa_pos=cfg.sa_pos, sa_cap=sa_cap,
                            rope_base=cfg.rope_base, rms_eps=cfg.rms_eps, rho=cfg.rho,
                            mixture=D.MIXTURES[cfg.mixture], branch_streams=streams,
                            da_window=cfg.da_window, da_dilation=cfg.da_dilation,
                            fuse_attn=fuse_attn)


def gpu_weights(D, cfg, W):
    """Device copies of a synth weight dict; linear-MoE stacks get the shared expert
    absorbed by the library (W_e + W_shared)."""
    dev = "cuda"
    G = {}
    for k_, v in W.items():
        G[k_] = v.to(dev).contiguous()
    if cfg.proj_experts:
        G["w_qkv"] = D.dreamer_absorb_shared(G.pop("w_qkv_e"), G.pop("w_qkv_sh"))
        G["w_o"] = D.dreamer_absorb_shared(G.pop("w_o_e"), G.pop("w_o_sh"))
    return G


def routing_mismatch(idx_gpu, z_ref, bias, k, tie=1e-6):
    """Tokens whose selected expert set differs from the oracle's, excluding tokens whose
    k-th and (k+1)-th biased oracle scores are within `tie`.  Returns (n_bad, n_exempt)."""
    key = np.asarray(z_ref, np.float64) + np.asarray(bias, np.float64)[None, :]
    srt = -np.sort(-key, axis=1)
    ref_idx = oracle.topk_select(key, k)
    exempt = np.zeros(key.shape[0], bool)
    if key.shape[1] > k:
        exempt = (srt[:, k - 1] - srt[:, k]) < tie
    same = np.array([set(a) == set(b) for a, b in zip(np.asarray(idx_gpu), ref_idx)])
    return int((~same & ~exempt).sum()), int(exempt.sum())


# --------------------------------------------------------------------- routing checks
#
# The router's scores are linear in its input: z = RoPE_depth(x W_r^T) K^T * rho is a
# fixed linear map at depth l, so z(x) = x @ c.T with c [E, h] (the router's Jacobian,
# taken here by running the oracle's router on the unit vectors).  That gives three
# checks of a selection, each of which a single wrong expert on a non-tied token fails:
#   exact    - the oracle's router on the GPU's own router input (y_steps): identical sets
#              except oracle ties within `tie` (the float32 evaluation of the scores);
#   margin   - against the free-running oracle at the same depth: the scores of the two
#              runs differ by dz = (in_gpu - in_ref) @ c.T exactly, so a token whose
#              k-th vs (k+1)-th margin exceeds max(dz) - min(dz) + tie cannot change;
#   midpoint - the projection router reads x_hat, which the GPU does not export: it is
#              recomputed from the GPU's float32 stream x_l; the GPU's float32 RMSNorm is
#              within a relative XHAT_REL of the exact value, so only elements whose exact
#              value lies that close to a bf16 rounding midpoint can round differently
#              (by one bf16 ulp), which bounds each token's score change.

TIE = 1e-6
XHAT_REL = 2.0 ** -16   # float32 RMSNorm error bound (a tree sum of squares, rsqrt, mul)


def router_jacobian(Wn, which, l, cfg):
    """c [E, h]: z = x @ c.T for the EA router ("ea") or the projection router ("proj")."""
    w_r, keys = (Wn["w_r"], Wn["keys"]) if which == "ea" else (Wn["w_pr"], Wn["pkeys"])
    E = keys.shape[0]
    _, _, _, z = oracle.expert_route(np.eye(cfg.h), w_r, keys, np.zeros(E), 1, l, cfg.L,
                                     cfg.rho, False, cfg.rope_base)
    return z.T


def _sets_equal(a, b):
    a, b = np.sort(np.asarray(a), axis=1), np.sort(np.asarray(b), axis=1)
    return (a == b).all(axis=1)


def _margins(key, k):
    srt = -np.sort(-key, axis=1)
    if key.shape[1] <= k:
        return np.full(key.shape[0], np.inf)
    return srt[:, k - 1] - srt[:, k]


def routing_exact_on_own_input(cfg, Wn, ea_in, idx_gpu, l, tie=TIE):
    """Oracle router on the GPU's own EA input of depth l.  Returns (n_bad, n_tie)."""
    _, _, _, z = oracle.expert_route(ea_in, Wn["w_r"], Wn["keys"], Wn["bias"], cfg.k, l,
                                     cfg.L, cfg.rho, cfg.normalize, cfg.rope_base)
    return routing_mismatch(idx_gpu, z, Wn["bias"], cfg.k, tie)


def routing_margin_rule(cfg, Wn, l, in_gpu, in_ref, idx_gpu, z_ref, tie=TIE):
    """Free-running GPU vs free-running oracle at depth l.  Returns (n_bad, n_diff,
    n_exempt, margins of the differing tokens)."""
    c = router_jacobian(Wn, "ea", l, cfg)
    dz = (np.asarray(in_gpu, np.float64) - np.asarray(in_ref, np.float64)) @ c.T
    delta = dz.max(axis=1) - dz.min(axis=1) + tie
    key = z_ref + Wn["bias"][None, :]
    margin = _margins(key, cfg.k)
    same = _sets_equal(idx_gpu, oracle.topk_select(key, cfg.k))
    must = margin > delta
    return (int((~same & must).sum()), int((~same).sum()), int((~must).sum()),
            np.sort(margin[~same]))


def proj_routing_midpoint_rule(cfg, Wn, l, x_l, pidx_gpu, tie=TIE):
    """Top-1 projection routing of depth l from the GPU's float32 stream x_l [T, h].
    Returns (n_bad, n_exempt)."""
    xh = oracle.rmsnorm(x_l, Wn["g"], cfg.rms_eps)
    lo = oracle.bf16_round(xh * (1 - XHAT_REL))
    hi = oracle.bf16_round(xh * (1 + XHAT_REL))
    xhb = oracle.bf16_round(xh)
    dmax = np.maximum(np.abs(hi - xhb), np.abs(lo - xhb))     # 0 unless near a midpoint
    Ep = Wn["pkeys"].shape[0]
    _, _, _, z = oracle.expert_route(xhb, Wn["w_pr"], Wn["pkeys"], np.zeros(Ep), 1, l, cfg.L,
                                     cfg.rho, False, cfg.rope_base)
    c = router_jacobian(Wn, "proj", l, cfg)
    delta = 2.0 * (dmax @ np.abs(c).T).max(axis=1) + tie
    margin = _margins(z, 1)
    same = np.asarray(pidx_gpu).reshape(-1) == np.argmax(z, axis=1)
    must = margin > delta
    return int((~same & must).sum()), int((~must).sum())


def check_free_routing(cfg, W, gpu, ref):
    """The three selection checks of a free-running bf16 GPU run (see the module text);
    prints the later-depth disagreements with the free-running oracle and their margins."""
    Wn = oracle.prepare_weights(W, big_as_f32=True)
    for l in range(cfg.L):
        if cfg.use_ea:
            n_bad, n_tie = routing_exact_on_own_input(cfg, Wn, gpu["y_steps"][l],
                                                      gpu["idx"][l], l)
            assert n_bad == 0, f"depth {l}: {n_bad} tokens off the oracle's selection on the " \
                               f"GPU's own router input ({n_tie} ties exempt)"
            n_bad, n_diff, n_ex, marg = routing_margin_rule(
                cfg, Wn, l, gpu["y_steps"][l], ref["steps"][l]["yb"], gpu["idx"][l],
                ref["steps"][l]["z"])
            if l == 0:
                assert n_bad == 0, f"depth 0: {n_bad} wide-margin tokens differ from the " \
                                   f"free-running oracle ({n_ex} within their bound)"
            elif n_diff:
                print(f"  depth {l}: {n_diff} of {cfg.T} tokens differ from the free-running "
                      f"oracle (cascade), margins {marg[:4]}", flush=True)
        if cfg.proj_experts:
            x_l = gpu["x0"] if l == 0 else gpu["x_steps"][l - 1]
            n_bad, n_ex = proj_routing_midpoint_rule(cfg, Wn, l, x_l, gpu["pidx"][l])
            assert n_bad == 0, f"depth {l}: {n_bad} projection selections off ({n_ex} exempt)"
