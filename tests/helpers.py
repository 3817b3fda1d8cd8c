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
