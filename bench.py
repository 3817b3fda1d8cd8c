"""Throughput of the Dreamer layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload deep] [--no-cpu-baseline]

One step = one dreamer_layer_forward over the whole workload (all L depth steps of
RMSNorm, projections, SA, DA, routing, permutation, expert FFNs and combine) on inputs
already resident in HBM.  The default workload is the largest one that fits one GPU, the
deep recurrence (b=2, s=4096, h=2048, 32 heads x 64, L=64, E=2048 top-8, Zipf-skewed
router bias).  Prints one JSON line.  Inputs are seeded synthetic tensors of the
workload's shapes (weights N(0, 0.02), tokens N(0, 1)), drawn on the device.

Timed region: exactly K forwards between two device synchronisations (value and
ms_per_step from the wall clock), with a HIP event pair around every forward (the median
is reported too) and the launches of the dominant kernel class bracketed by HIP events on
their stream (roofline.achieved).  Before it, one instrumented forward per kernel class
gives each class's time and its fraction of its binding roofline (classes).  The line
also carries the per-step time of the three mixture wirings (serial, the default partial
one, fully parallel) and their throughput relative to the serial wiring, windowed depth
attention, the expert-usage statistics, and the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # fp32 vector
METRIC = "token-depth-steps/sec, Dreamer layer fwd; % of HBM BW / MFMA peak"
CLASSES = ["qkv_proj", "out_proj", "seq_attn", "depth_attn", "attention", "route", "permute",
           "expert_ffn", "combine"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="deep")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--kernel-class", default=None, help="time this class live (default: dominant)")
    p.add_argument("--decode-tokens", type=int, default=8,
                   help="decode workloads: tokens per step (one multi-token decode call)")
    p.add_argument("--no-usage", action="store_true", help="skip the expert-usage report")
    p.add_argument("--no-mixtures", action="store_true",
                   help="skip timing the serial / partial / fully parallel wirings")
    p.add_argument("--no-depth-windows", action="store_true",
                   help="skip timing windowed / dilated depth attention")
    p.add_argument("--da-window", type=int, default=None,
                   help="DA over the most recent depths only (0: all; default: workload's)")
    p.add_argument("--da-dilation", type=int, default=None,
                   help="with a window: also every N-th older depth")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (read + write), for scaling "
                        "the FETCH_SIZE / WRITE_SIZE counters")
    return p.parse_args()


def calibrate_copy(mib):
    """A plain elementwise copy of known size: mib MiB read, mib MiB written per launch."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n * 4}), flush=True)


def stored_traffic(kclass, workload):
    """HBM bytes per launch of one kernel class, from the committed counter summary, or None
    when the summary is missing or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kclass}_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    try:
        blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (IndexError, ValueError):
        return None
    from depth_recurrent_layer_amd.profiling import source_digest
    if blob.get("source_sha256") != source_digest(kclass):
        return None
    return blob["bytes_per_launch"]


def algorithmic_work(cfg, counts_per_depth, reps=1):
    """Algorithmic bytes / flops per step for each kernel class (what the method must move
    or compute, not what the kernels happen to move).  Decode: a step is `reps` tokens,
    token j attending over sa_pos + j + 1 cached positions."""
    es = 2 if cfg.dtype == "bf16" else 4
    T, h, L, k, f, r, E = cfg.T, cfg.h, cfg.L, cfg.k, cfg.f, cfg.r, cfg.E
    nq = 6 if cfg.use_da else 3
    w = {}
    w["qkv_proj"] = dict(bound="mfma", flops=L * 2 * T * h * nq * h, launches=L)
    w["out_proj"] = dict(bound="mfma", flops=L * 2 * T * (nq // 3) * h * h, launches=L)
    if cfg.decode:  # every cached key and value of every depth read once per token
        w["seq_attn"] = dict(bound="hbm", bytes=sum(L * cfg.b * (cfg.sa_pos + j + 1) * 2 * h * es
                                                    for j in range(reps)), launches=L * reps)
    else:
        w["seq_attn"] = dict(bound="mfma", flops=L * 4 * cfg.b * h * (cfg.s * (cfg.s + 1) // 2),
                             launches=L)
    # bf16: q in and the output out (2 rows), the key and value of every slot read, the
    # current one included (the projection writes it into the cache); float32: q, k, v in,
    # key and value stored, output out (6 rows), 2 per older slot read
    if cfg.dtype == "bf16":
        da_bytes = sum(T * h * es * (2 + 2 * n_depth_keys(l, cfg.da_window, cfg.da_dilation))
                       for l in range(L))
    else:
        da_bytes = sum(T * h * es * (6 + 2 * (n_depth_keys(l, cfg.da_window, cfg.da_dilation) - 1))
                       for l in range(L))
    w["depth_attn"] = dict(bound="hbm", bytes=da_bytes, launches=L)
    # SA and DA in one launch: priced by its SA flops against the MFMA peak, and (reported
    # beside it) by its DA bytes against the HBM peak; each is a lower bound of the
    # launch's use of that resource
    w["attention"] = dict(bound="mfma", flops=w["seq_attn"].get("flops", 0), launches=L,
                          bytes=da_bytes)
    nw = 3 if cfg.ffn == "swiglu" else 2
    w["expert_ffn"] = dict(bound="hbm", bytes=L * 2 * T * k * h * es,
                           flops=L * 2 * T * k * nw * h * f, launches=L)
    w["combine"] = dict(bound="hbm", bytes=L * T * h * (k * es + 4 + es), launches=L + 1)
    w["route"] = dict(bound="alu", flops=L * 2 * T * (h * r + r * E), launches=L)
    w["permute"] = dict(bound="hbm", bytes=L * T * k * 12, launches=L)
    for name, v in w.items():
        if name != "seq_attn" or not cfg.decode:
            for key in ("bytes", "flops", "launches"):
                if key in v:
                    v[key] *= reps
    # expert weights: each (token pass, depth) reads the matrices of the experts it touches
    touched = sum(int((c > 0).sum()) for c in counts_per_depth)
    w["expert_ffn"]["bytes"] += touched * nw * h * f * es
    return w


def class_report(work, per_class):
    """Per kernel class: ms per step from its instrumented forward (the event brackets add
    a few microseconds per launch), and the fraction of its binding roofline that its
    average launch reaches."""
    out = {}
    for c, (n, ms) in per_class.items():
        if n == 0:
            continue
        e = {"ms_per_step": round(ms, 4), "launches": n}
        if c in work and ("bytes" in work[c] or "flops" in work[c]):
            r = roofline_entry(work[c], ms / n)
            e.update(bound=r["bound"], achieved=r["achieved"], unit=r["unit"], frac=r["frac"])
            if r["bound"] != "hbm" and "bytes" in work[c]:  # a launch that also streams HBM
                hb = roofline_entry(dict(work[c], bound="hbm"), ms / n)
                e.update(hbm_achieved=hb["achieved"], hbm_frac=hb["frac"])
        out[c] = e
    return out


def n_depth_keys(l, window, dilation):
    """Depth slots DA reads at depth l: all l + 1 without a window, else the window's
    min(window, l + 1) plus the older slots at multiples of the dilation."""
    if window <= 0:
        return l + 1
    older = l - window + 1  # slots 0..l-window lie outside the window
    n = min(window, l + 1)
    if dilation > 0 and older > 0:
        n += l // dilation - (window - 1) // dilation  # multiples in [window, l]
    return n


def roofline_entry(work, avg_ms):
    if work["bound"] == "hbm":
        ach = work["bytes"] / work["launches"] / (avg_ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None}
    if work["bound"] == "mfma":
        ach = work["flops"] / work["launches"] / (avg_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None}
    ach = work["flops"] / work["launches"] / (avg_ms * 1e-3) / 1e12
    return {"bound": "alu", "achieved": round(ach, 2), "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / PEAK_FP32_TFLOPS, 4), "traffic": None}


# Relative per-step throughput of the wirings over the serial one, as the pages report it
# for their model (another machine and model size: context, not a target).
PAGES_RELATIVE = {"serial": 0.0, "partial": 0.152, "parallel": 0.308}


def time_mixtures(D, cfg, G, x0, steps):
    """ms per forward of the three mixture wirings (independent branches on side streams:
    DA beside SA in the partial and fully parallel ones, the EA chain too in the fully
    parallel one) and their throughput relative to the serial wiring."""
    import torch
    out = {}
    x_out = torch.empty((cfg.T, cfg.h), dtype=torch.float32, device="cuda")
    for mix in ("serial", "partial", "parallel"):
        lc = layer_cfg(D, cfg, mixture=mix)
        ws = torch.empty(D.layer_ws_bytes(lc), dtype=torch.uint8, device="cuda")
        for _ in range(3):
            D.dreamer_layer_forward(lc, G, x0, x_out=x_out, ws=ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            D.dreamer_layer_forward(lc, G, x0, x_out=x_out, ws=ws)
        torch.cuda.synchronize()
        out[mix] = {"ms_per_step": round((time.perf_counter() - t0) * 1e3 / steps, 4)}
        del ws
    for mix in out:
        out[mix]["relative_throughput_vs_serial"] = round(
            out["serial"]["ms_per_step"] / out[mix]["ms_per_step"] - 1.0, 4)
        out[mix]["pages_relative_throughput"] = PAGES_RELATIVE[mix]
    out["parallel"]["side_stream"] = True
    return out


# DA key sets timed beside the full one: (window, dilation)
DEPTH_WINDOWS = [(0, 0), (4, 4), (2, 0)]


def time_depth_windows(D, cfg, G, x0, steps):
    """Windowed / dilated depth attention: ms per forward, DA kernel ms per forward and the
    algorithmic DA bytes per forward for each (window, dilation) of DEPTH_WINDOWS.  DA runs
    in its own launches here (fuse_attn off) so that its time can be taken alone."""
    import torch
    out = {}
    x_out = torch.empty((cfg.T, cfg.h), dtype=torch.float32, device="cuda")
    for w, dil in DEPTH_WINDOWS:
        c = cfg.replace(da_window=w, da_dilation=dil)
        lc = layer_cfg(D, c, fuse_attn=False)
        ws = torch.empty(D.layer_ws_bytes(lc), dtype=torch.uint8, device="cuda")
        for _ in range(3):
            D.dreamer_layer_forward(lc, G, x0, x_out=x_out, ws=ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            D.dreamer_layer_forward(lc, G, x0, x_out=x_out, ws=ws)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        D.timing_enable("depth_attn", c.L + 8)
        D.dreamer_layer_forward(lc, G, x0, x_out=x_out, ws=ws)
        _, da_ms = D.timing_read()
        D.timing_disable()
        da_bytes = algorithmic_work(c, [])["depth_attn"]["bytes"]
        out[f"window{w}_dilation{dil}"] = {
            "ms_per_step": round(ms, 4), "depth_attn_ms_per_step": round(da_ms, 4),
            "depth_attn_bytes_per_step": da_bytes,
            "depth_attn_GBps": round(da_bytes / (da_ms * 1e-3) / 1e9, 1)}
        del ws
    return out


def layer_cfg(D, cfg, cap=0, mixture="partial", fuse_attn=True):
    return D.make_layer_cfg(dtype=cfg.dtype, b=cfg.b, s=cfg.s, h=cfg.h, H=cfg.H, d=cfg.d,
                            L=cfg.L, E=cfg.E, k=cfg.k, f=cfg.f, r=cfg.r, ffn=cfg.ffn,
                            normalize=cfg.normalize, proj_experts=cfg.proj_experts,
                            decode=cfg.decode, sa_pos=cfg.sa_pos, sa_cap=cap,
                            rope_base=cfg.rope_base, rms_eps=cfg.rms_eps, rho=cfg.rho,
                            mixture=D.MIXTURES[mixture], branch_streams=True,
                            da_window=cfg.da_window, da_dilation=cfg.da_dilation,
                            fuse_attn=fuse_attn)


def usage_report(D, cfg, G, x0, lc, route, iters=20, lam=0.01):
    """Expert usage of the workload's routing (distinct experts and Gini per depth, global
    Gini over all depths), then `iters` rounds of forward -> counts over all depths ->
    b <- b + lam * sign(median(N) - N) on a copy of the bias, with the global Gini before
    and after and the time of one counts + update round."""
    import torch
    E, L = cfg.E, cfg.L
    per_depth = D.dreamer_route_counts(route[0].contiguous(), E, n_sets=L)
    st = D.dreamer_expert_usage(per_depth).cpu()
    glob = D.dreamer_expert_usage(per_depth.sum(0, keepdim=True).to(torch.int32).contiguous())
    out = {"distinct_per_depth": [int(v) for v in st[:, 0]],
           "gini_per_depth": [round(float(v), 4) for v in st[:, 2]],
           "max_over_mean_per_depth": [round(float(v), 2) for v in st[:, 1]],
           "global_gini": round(float(glob[0, 2]), 4),
           "pages_global_gini": 0.075}
    Gb = dict(G)
    Gb["bias"] = G["bias"].clone()
    x_out = torch.empty((cfg.T, cfg.h), dtype=torch.float32, device="cuda")
    ginis, t_upd = [], []
    for _ in range(iters):
        D.dreamer_layer_forward(lc, Gb, x0, x_out=x_out, route=route)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        counts = D.dreamer_route_counts(route[0].contiguous(), E)
        D.dreamer_bias_update(counts[0], Gb["bias"], lam)
        torch.cuda.synchronize()
        t_upd.append(time.perf_counter() - t0)
        ginis.append(float(D.dreamer_expert_usage(counts)[0, 2]))
    out["balancing"] = {"lambda": lam, "iterations": iters,
                        "global_gini_first": round(ginis[0], 4),
                        "global_gini_last": round(ginis[-1], 4),
                        "counts_and_update_us": round(1e6 * sorted(t_upd)[len(t_upd) // 2], 1)}
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, W_dev, min_seconds=10.0, max_reps=8):
    """The CPU oracle (libdreamer_ref: plain float64 C++17 + OpenMP, one thread per host
    core this process may run on), as it stands, timed with a steady clock around its
    layer forward on a bounded sample of the workload: the whole workload when it is small,
    else the first sequence's first 128 tokens over all L depths; forwards repeated until
    about min_seconds of CPU work.  W_dev: the workload's weights (the bench's device
    copies, brought to the host)."""
    import oracle
    from synth import make_x0
    whole = cfg.T * cfg.h * cfg.L <= 2 ** 26
    nb, s_len = (cfg.b, cfg.s) if whole else (1, min(cfg.s, 128))
    sample = cfg.replace(b=nb, s=s_len)
    W = oracle.prepare_weights({k: v.cpu() for k, v in W_dev.items()}, big_as_f32=True)
    x0 = make_x0(cfg, b0=0, nb=nb, s_len=s_len).reshape(nb * s_len, cfg.h).numpy()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.layer_forward(sample, W, x0)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    what = (f"full {cfg.name} workload (b={cfg.b}, s={cfg.s}, L={cfg.L})" if whole else
            f"{cfg.name} workload, first sequence, first {s_len} tokens, L={cfg.L}")
    return {"value": round(nb * s_len * cfg.L * reps / dt, 2), "unit": "token-depth-steps/s",
            "cores": oracle.THREADS, "kind": "oracle",
            "sample": f"{what}, {reps} forward(s) in {dt:.1f} s; C++ oracle (float64, "
                      f"OpenMP, {oracle.THREADS} threads on {_cpu_model()}) with bf16 "
                      f"storage emulation"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from depth_recurrent_layer_amd import dreamer as D
    from synth import CONFIGS, make_weights, make_x0

    cfg = CONFIGS[args.workload]
    if args.da_window is not None:
        cfg = cfg.replace(da_window=args.da_window)
    if args.da_dilation is not None:
        cfg = cfg.replace(da_dilation=args.da_dilation)
    dev = "cuda"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    reps = args.decode_tokens if cfg.decode else 1
    W = make_weights(cfg, device=dev)
    G = {k: v.contiguous() for k, v in W.items()}
    if cfg.proj_experts:
        G["w_qkv"] = D.dreamer_absorb_shared(G.pop("w_qkv_e"), G.pop("w_qkv_sh"))
        G["w_o"] = D.dreamer_absorb_shared(G.pop("w_o_e"), G.pop("w_o_sh"))
    x0 = make_x0(cfg, device=dev).reshape(cfg.T, cfg.h).contiguous()
    cap = cfg.sa_pos + reps if cfg.decode else 0
    lc = layer_cfg(D, cfg, cap=cap)
    if cfg.decode:
        # SA caches [L, b, cap, H, d]: positions 0..sa_pos-1 seeded N(0, 1) (already
        # rotated keys / values); every step appends its `reps` tokens after them
        from synth.configs import make_sa_cache
        sa = []
        for which in ("k", "v"):
            c = torch.empty((cfg.L, cfg.b, cap, cfg.H, cfg.d), dtype=cfg.torch_dtype, device=dev)
            for l0 in range(cfg.L):
                c[l0, :, :cfg.sa_pos] = make_sa_cache(cfg, which, dev, l0=l0, nl=1)[0]
            sa.append(c)
        xs = make_x0(cfg.replace(b=cfg.b * reps), device=dev).reshape(reps, cfg.b, cfg.h)
        xs = xs.float().contiguous()
        ws = torch.empty(D.decode_ws_bytes(lc, reps), dtype=torch.uint8, device=dev)
        x_out = torch.empty_like(xs)
        route = (torch.empty((reps, cfg.L, cfg.b, cfg.k), dtype=torch.int32, device=dev),
                 torch.empty((reps, cfg.L, cfg.b, cfg.k), dtype=torch.float32, device=dev))

        def step(with_route=False):
            D.dreamer_decode_tokens(lc, G, xs, tuple(sa), x_out=x_out, ws=ws,
                                    route=route if with_route else None)
    else:
        ws = torch.empty(D.layer_ws_bytes(lc), dtype=torch.uint8, device=dev)
        x_out = torch.empty((cfg.T, cfg.h), dtype=torch.float32, device=dev)
        route = (torch.empty((cfg.L, cfg.T, cfg.k), dtype=torch.int32, device=dev),
                 torch.empty((cfg.L, cfg.T, cfg.k), dtype=torch.float32, device=dev))

        def step(with_route=False):
            D.dreamer_layer_forward(lc, G, x0, x_out=x_out, ws=ws,
                                    route=route if with_route else None)

    step(with_route=True)
    torch.cuda.synchronize()
    ridx = route[0].cpu().numpy().reshape(reps, cfg.L, -1)
    counts = [np.bincount(ridx[j, l], minlength=cfg.E) for j in range(reps)
              for l in range(cfg.L)]
    work = algorithmic_work(cfg, counts, reps)
    for _ in range(args.warmup):
        step()
    # dominant kernel class: one instrumented forward per class (untimed)
    per_class = {}
    for kc in CLASSES:
        D.timing_enable(kc, 4 * cfg.L * reps + 8)
        step()
        n, ms = D.timing_read()
        D.timing_disable()
        per_class[kc] = (n, ms)
    dom = args.kernel_class or max(per_class, key=lambda c: per_class[c][1])
    if dom not in work or ("bytes" not in work[dom] and "flops" not in work[dom]):
        dom = "expert_ffn"

    # timed region: K forwards, an event pair around each, the dominant class's launches
    # bracketed by HIP events on their stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    D.timing_enable(dom, args.steps * work[dom]["launches"] + 8)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    n_launch, dom_ms = D.timing_read()
    D.timing_disable()
    ms_per_step = elapsed * 1e3 / args.steps
    ev_ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    ms_median = ev_ms[len(ev_ms) // 2] if len(ev_ms) % 2 else \
        0.5 * (ev_ms[len(ev_ms) // 2 - 1] + ev_ms[len(ev_ms) // 2])
    value = cfg.T * cfg.L * reps * args.steps / elapsed
    roof = roofline_entry(work[dom], dom_ms / max(n_launch, 1))
    roof["traffic"] = stored_traffic(dom, cfg.name)
    roof["kernel"] = dom
    roof["launches_timed"] = n_launch
    roof["avg_launch_us"] = round(dom_ms / max(n_launch, 1) * 1e3, 2)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "token-depth-steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.dtype} Dreamer layer forward b={cfg.b} s={cfg.s} "
                               f"h={cfg.h} heads={cfg.H}x{cfg.d} L={cfg.L} E={cfg.E} top-{cfg.k} "
                               f"{cfg.ffn} f={cfg.f} r={cfg.r}" +
                               (f", decode of {reps} tokens per step after {cfg.sa_pos} cached "
                                f"positions" if cfg.decode else ""),
                   "tokens": cfg.T * reps, "depths": cfg.L, "parallelism": "single GPU"},
        "roofline": roof,
        "ms_per_step_event_median": round(ms_median, 4),
        "classes": class_report(work, per_class),
    }
    if not args.no_mixtures and not cfg.decode:
        line["mixtures"] = time_mixtures(D, cfg, G, x0, args.steps)
    if not args.no_depth_windows and not cfg.decode:
        line["depth_windows"] = time_depth_windows(D, cfg, G, x0, args.steps)
    if not cfg.decode and not args.no_usage:
        line["expert_usage"] = usage_report(D, cfg, G, x0, lc, route)
    if not args.no_cpu_baseline and not cfg.decode:
        line["cpu_baseline"] = cpu_baseline(cfg, W)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
