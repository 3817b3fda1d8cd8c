"""The five workloads at full size, in the launch configuration the benchmark times.

Prefill: the full-size GPU run's rows of batch 0, positions 0..P-1, must be bit-identical
to a GPU run of that prefix alone (causality in s and batch independence: no token's
result may depend on later tokens or other sequences, whatever the launch shapes), and
the prefix run must match the CPU oracle: RMSNorm'd x_L within 2e-2 with the oracle's
expert choices replayed, and in a free-running run the selection checks of
helpers.check_free_routing (exact on the GPU's own router inputs; the margin rule against
the free-running oracle at depth 0; the projection midpoint rule).  Decode: the same with
the first sequences of the batch.  The small workload is also compared with the oracle
whole.  Every full-size run's routing is also checked exactly, at every depth and for
every token, against the oracle's router applied to the GPU's own router inputs.
Weights and inputs are drawn on the device."""
import numpy as np
import pytest
import torch

import oracle
from helpers import (check_free_routing, gpu_weights, lib_cfg, proj_routing_midpoint_rule,
                     rms_normed, routing_exact_on_own_input)
from synth import CONFIGS, make_weights, make_x0
from synth.configs import make_sa_cache

pytestmark = pytest.mark.gpu


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def gpu_forward(D, cfg, G, x0, sa_cache=None, sa_cap=0, replay=None, steps=False):
    """The benchmark's launch configuration (independent branches on side streams, SA and
    DA in one launch where that applies).  steps: also return x_steps (f32) and y_steps
    (EA router inputs) on the device."""
    lc = lib_cfg(D, cfg, sa_cap=sa_cap, streams=True)
    T = cfg.T
    x = x0.reshape(T, cfg.h).float().contiguous()
    route = (torch.empty((cfg.L, T, cfg.k), dtype=torch.int32, device="cuda"),
             torch.empty((cfg.L, T, cfg.k), dtype=torch.float32, device="cuda"))
    proj = None
    if cfg.proj_experts:
        proj = (torch.empty((cfg.L, T), dtype=torch.int32, device="cuda"),
                torch.empty((cfg.L, T), dtype=torch.float32, device="cuda"))
    rin = pin = None
    if replay is not None:
        rin = torch.from_numpy(np.ascontiguousarray(replay["idx"]).astype(np.int32)).cuda()
        if cfg.proj_experts:
            pin = torch.from_numpy(np.ascontiguousarray(replay["pidx"]).astype(np.int32)).cuda()
    xs = ys = None
    if steps:
        ys = torch.empty((cfg.L, T, cfg.h), dtype=cfg.torch_dtype, device="cuda")
        if cfg.proj_experts:
            xs = torch.empty((cfg.L, T, cfg.h), dtype=torch.float32, device="cuda")
    out = D.dreamer_layer_forward(lc, G, x, route=route, proj_route=proj, sa_cache=sa_cache,
                                  route_in=rin, proj_route_in=pin, x_steps=xs, y_steps=ys)
    torch.cuda.synchronize()
    return out, route, proj, xs, ys


def oracle_run(cfg, W_dev, x0_cpu, sa_k=None, sa_v=None):
    Wn = oracle.prepare_weights({k: v.cpu() for k, v in W_dev.items()}, big_as_f32=True)
    return oracle.layer_forward(cfg, Wn, x0_cpu.reshape(cfg.T, cfg.h).numpy(), sa_k, sa_v,
                                return_steps=True)


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def compare_with_oracle(D, cfg, W, G, x0, ref, sa_cache_fn=None, sa_cap=0):
    """GPU (prefix shape) with the oracle's choices replayed, and free-running."""
    sc = sa_cache_fn() if sa_cache_fn else None
    rep = gpu_forward(D, cfg, G, x0, sa_cache=sc, sa_cap=sa_cap, replay=ref)[0]
    err = np.abs(rms_normed(rep.cpu().double().numpy()) - rms_normed(ref["x_out"])).max()
    sc = sa_cache_fn() if sa_cache_fn else None
    free, route, proj, xs, ys = gpu_forward(D, cfg, G, x0, sa_cache=sc, sa_cap=sa_cap,
                                            steps=True)
    err_free = np.abs(rms_normed(free.cpu().double().numpy()) - rms_normed(ref["x_out"])).max()
    print(f"{cfg.name}: replay err {err:.3e}, free err {err_free:.3e}", flush=True)
    assert err <= 2e-2
    gpu = {"idx": route[0].cpu().numpy(), "y_steps": _host(ys),
           "x0": _host(x0.reshape(cfg.T, cfg.h))}
    if cfg.proj_experts:
        gpu["pidx"] = proj[0].cpu().numpy()
        gpu["x_steps"] = _host(xs)
    check_free_routing(cfg, {k: v.cpu() for k, v in W.items()}, gpu, ref)


def routing_exact_full(cfg, W, x0, route, proj, xs, ys):
    """Every depth of a full-size run: the oracle's router on the GPU's own router input
    selects the same sets (ties within 1e-6 exempt); projection routing by the midpoint
    rule from the GPU's float32 stream.  Depth by depth, on the host."""
    Wn = oracle.prepare_weights({k: v.cpu() for k, v in W.items()}, big_as_f32=True)
    ties = 0
    for l in range(cfg.L):
        n_bad, n_tie = routing_exact_on_own_input(cfg, Wn, _host(ys[l]),
                                                  route[0][l].cpu().numpy(), l)
        assert n_bad == 0, f"depth {l}: {n_bad} tokens off the oracle's selection"
        ties += n_tie
        if cfg.proj_experts:
            x_l = _host(x0.reshape(cfg.T, cfg.h)) if l == 0 else _host(xs[l - 1])
            n_bad, _ = proj_routing_midpoint_rule(cfg, Wn, l, x_l, proj[0][l].cpu().numpy())
            assert n_bad == 0, f"depth {l}: {n_bad} projection selections off"
    print(f"{cfg.name}: routing exact at all {cfg.L} depths x {cfg.T} tokens "
          f"({ties} tie exemptions)", flush=True)


@pytest.mark.parametrize("mixture", ["partial", "serial", "parallel"])
def test_small_full_vs_oracle(gpu_lib, mixture):
    D = gpu_lib
    cfg = CONFIGS["small"].replace(mixture=mixture)
    print(f"full small workload, {mixture} wiring", flush=True)
    W = make_weights(cfg, device="cuda")
    G = gpu_weights(D, cfg, W)
    x0 = make_x0(cfg, device="cuda")
    ref = oracle_run(cfg, W, x0.cpu())
    compare_with_oracle(D, cfg, W, G, x0, ref)
    del W, G
    _free()


@pytest.mark.parametrize("name,prefix", [("linear_moe", 128), ("deep", 128)])
def test_prefill_full_prefix(gpu_lib, name, prefix):
    D = gpu_lib
    cfg = CONFIGS[name]
    print(f"full {name}: b={cfg.b} s={cfg.s} h={cfg.h} L={cfg.L} E={cfg.E}", flush=True)
    W = make_weights(cfg, device="cuda")
    G = gpu_weights(D, cfg, W)
    x0 = make_x0(cfg, device="cuda")
    full, route_full, _, _, _ = gpu_forward(D, cfg, G, x0)
    assert torch.isfinite(full).all()
    pcfg = cfg.replace(b=1, s=prefix)
    # bit-identical prefixes: causality and batch independence of the whole GPU path; the
    # last sequence's prefix lies in other row tiles of every full-size launch
    for bi in sorted({0, cfg.b - 1}):
        xb = x0[bi:bi + 1, :prefix].contiguous()
        part_b, route_b, _, _, _ = gpu_forward(D, pcfg, G, xb)
        r0 = bi * cfg.s
        assert torch.equal(full[r0:r0 + prefix], part_b), f"sequence {bi}"
        assert torch.equal(route_full[0][:, r0:r0 + prefix], route_b[0]), f"sequence {bi}"
        del part_b, route_b
    x0p = x0[:1, :prefix].contiguous()
    del full, route_full
    _free()
    ref = oracle_run(pcfg, W, x0p.cpu())
    compare_with_oracle(D, pcfg, W, G, x0p, ref)
    del W, G
    _free()


@pytest.mark.parametrize("name", ["small", "linear_moe", "deep"])
def test_prefill_full_routing_exact(gpu_lib, name):
    D = gpu_lib
    cfg = CONFIGS[name]
    print(f"full {name}: routing of every depth on the GPU's own router inputs", flush=True)
    W = make_weights(cfg, device="cuda")
    G = gpu_weights(D, cfg, W)
    x0 = make_x0(cfg, device="cuda")
    out, route, proj, xs, ys = gpu_forward(D, cfg, G, x0, steps=True)
    assert torch.isfinite(out).all()
    del G, out
    routing_exact_full(cfg, W, x0, route, proj, xs, ys)
    del W, xs, ys
    _free()


def _decode_caches(cfg):
    cap = cfg.sa_pos + 1
    shape = (cfg.L, cfg.b, cap, cfg.H, cfg.d)
    sk = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    sv = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    for l in range(cfg.L):   # cache contents N(0,1), drawn on the device depth by depth
        sk[l, :, :cfg.sa_pos] = make_sa_cache(cfg, "k", "cuda", l0=l, nl=1)[0]
        sv[l, :, :cfg.sa_pos] = make_sa_cache(cfg, "v", "cuda", l0=l, nl=1)[0]
    return sk, sv, cap


def test_decode_full_first_sequences(gpu_lib):
    D = gpu_lib
    cfg = CONFIGS["decode"]
    nseq = 4
    print(f"full decode: {cfg.b} sequences, cache {cfg.sa_pos}, L={cfg.L}, E={cfg.E}", flush=True)
    W = make_weights(cfg, device="cuda")
    G = gpu_weights(D, cfg, W)
    x0 = make_x0(cfg, device="cuda")
    sk, sv, cap = _decode_caches(cfg)
    sub_k = sk[:, :nseq].clone()
    sub_v = sv[:, :nseq].clone()
    full, route_full, proj, xs, ys = gpu_forward(D, cfg, G, x0, sa_cache=(sk, sv), sa_cap=cap,
                                                 steps=True)
    assert torch.isfinite(full).all()
    # the appended position of every depth was written
    assert torch.isfinite(sk[:, :, cfg.sa_pos]).all()
    del sk, sv
    _free()
    routing_exact_full(cfg, W, x0, route_full, proj, xs, ys)
    pcfg = cfg.replace(b=nseq)
    x0p = x0[:nseq].contiguous()
    part, route_part, _, _, _ = gpu_forward(D, pcfg, G, x0p,
                                            sa_cache=(sub_k.clone(), sub_v.clone()),
                                            sa_cap=cap)
    assert torch.equal(full[:nseq], part)
    assert torch.equal(route_full[0][:, :nseq], route_part[0])
    del full, ys
    _free()
    rk = sub_k.float().cpu().numpy()
    rv = sub_v.float().cpu().numpy()
    ref = oracle_run(pcfg, W, x0p.cpu(), rk, rv)
    compare_with_oracle(D, pcfg, W, G, x0p, ref,
                        sa_cache_fn=lambda: (sub_k.clone(), sub_v.clone()), sa_cap=cap)
    del W, G, sub_k, sub_v
    _free()
