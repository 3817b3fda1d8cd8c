"""CPU oracle of one Dreamer depth-recurrent attention-mixture layer (forward pass).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package.  The arithmetic lives in
``libdreamer_ref.so`` (plain float64 C++17 + OpenMP, ``dreamer_ref.cpp``, C ABI in
``dreamer_ref.h``), which shares no code with the GPU library; both sides only see the
seeded inputs of ``synth``.  This module only marshals numpy arrays through ctypes: it
converts inputs to contiguous float64 / int64 (weights to float64 or float32, whichever
holds them exactly), allocates the outputs, and reshapes them.

Page key used in the library's citations (all describe arXiv 2601.21582):
  [PN]    papernotes.org paper notes: "Method / overall framework", "Key design 1/2/3",
          "Loss / training", ablation table, analysis of expert usage, "Limitations and
          outlook".
  [GS-de] gist.science German technical summary, "Methodik: Dreamer-Framework".
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdreamer_ref.so")
if not os.path.exists(_LIB_PATH):
    _build.build(verbose=False)
_lib = C.CDLL(_LIB_PATH)

_P = C.c_void_p
_I = C.c_int
_L = C.c_int64
_D = C.c_double


class _Cfg(C.Structure):
    _fields_ = [("bf16", _I), ("b", _I), ("s", _I), ("h", _I), ("H", _I), ("d", _I),
                ("L", _I), ("E", _I), ("k", _I), ("f", _I), ("r", _I), ("ffn", _I),
                ("normalize", _I), ("use_da", _I), ("use_ea", _I), ("sa_rope", _I),
                ("proj_experts", _I), ("mixture", _I), ("decode", _I), ("sa_pos", _L),
                ("da_window", _I), ("da_dilation", _I), ("rope_base", _D),
                ("rms_eps", _D), ("rho", _D)]


_WKEYS = ("g", "w_qkv", "w_o", "w_qkv_e", "w_qkv_sh", "w_o_e", "w_o_sh", "w_pr", "pkeys",
          "w_r", "keys", "w1", "w3", "w2")


class _Weights(C.Structure):
    _fields_ = [("f32", _I)] + [(k, _P) for k in _WKEYS] + [("bias", _P)]


class _StepOut(C.Structure):
    _fields_ = [(k, _P) for k in ("x_next", "y", "yb", "idx", "gate", "counts", "z", "pidx",
                                  "pgate", "pz")]


def _sig(name, args, res=_I):
    f = getattr(_lib, name)
    f.argtypes, f.restype = args, res
    return f


_threads = _sig("dreamer_ref_threads", [_I])
_bf16 = _sig("dreamer_ref_bf16_round", [_P, _L, _P], None)
_rms = _sig("dreamer_ref_rmsnorm", [_P, _P, _L, _I, _D, _P])
_rope = _sig("dreamer_ref_rope", [_P, _P, _L, _I, _D, _P])
_drope = _sig("dreamer_ref_depth_rope", [_P, _L, _I, _I, _I, _D, _P])
_dkeys = _sig("dreamer_ref_depth_keys", [_I, _I, _I, _P])
_sattn = _sig("dreamer_ref_seq_attn", [_I, _I, _I, _I, _L, _P, _P, _P, _P, _P, _L, _I, _I, _D,
                                       _I, _P, _P, _P])
_dattn = _sig("dreamer_ref_depth_attn", [_L, _I, _I, _I, _I, _P, _P, _P, _P, _P, _D, _I, _I,
                                         _I, _I, _P])
_topk = _sig("dreamer_ref_topk_select", [_P, _L, _I, _I, _P])
_route = _sig("dreamer_ref_expert_route", [_L, _I, _I, _I, _I, _I, _I, _P, _P, _P, _I, _P, _D,
                                           _I, _D, _P, _P, _P, _P])
_bupd = _sig("dreamer_ref_bias_update", [_P, _P, _I, _D, _P])
_rcount = _sig("dreamer_ref_route_counts", [_P, _L, _L, _I, _P])
_usage = _sig("dreamer_ref_expert_usage", [_P, _I, _P, _P, _P, _P])
_ffn = _sig("dreamer_ref_expert_ffn", [_I, _L, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I,
                                       _P, _I, _P, _P, _P])
_step = _sig("dreamer_ref_layer_step", [_P, _P, _P, _I, _P, _P, _P, _P, _L, _I, _P, _P, _P])
_fwd = _sig("dreamer_ref_layer_forward", [_P, _P, _P, _P, _P, _P, _P, _P, _L, _I, _P, _P, _P])
_dec = _sig("dreamer_ref_decode_tokens", [_P, _P, _I, _P, _P, _P, _P, _L, _I, _P])


def set_threads(n: int) -> int:
    """OpenMP threads of the oracle (n <= 0 keeps the setting); returns the number in use."""
    return int(_threads(int(n)))


# The host cores this process may run on.
THREADS = set_threads(len(os.sched_getaffinity(0)))

# ----------------------------------------------------------------------- marshalling

_KIND = {"gelu": 0, "swiglu": 1, "linear": 2}
_MIX = {"partial": 0, "serial": 1, "parallel": 2}


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_P)


def _inplace(a, what):
    if not (isinstance(a, np.ndarray) and a.dtype in (np.float64, np.float32)
            and a.flags.c_contiguous and a.flags.writeable):
        raise TypeError(f"{what} must be a writable C-contiguous float64 or float32 array "
                        "(it is updated in place)")
    return a


def _weights_arrays(W: dict) -> tuple[dict, bool]:
    """Weight matrices as float32 when any of them is float32 (each float64 one must then
    be exact in float32), else float64; the router bias always float64."""
    arrs = {k: W[k] for k in _WKEYS if W.get(k) is not None}
    f32 = any(np.asarray(v).dtype == np.float32 for v in arrs.values())
    out = {}
    for k, v in arrs.items():
        v = np.asarray(v)
        if f32 and v.dtype != np.float32:
            v32 = v.astype(np.float32)
            if not np.array_equal(v32.astype(np.float64), v.astype(np.float64)):
                raise ValueError(f"weight {k} is not exact in float32; pass float64 weights")
            v = v32
        out[k] = np.ascontiguousarray(v if f32 else v.astype(np.float64))
    return out, f32


def _weights_struct(W: dict):
    arrs, f32 = _weights_arrays(W)
    bias = _f64(W["bias"]) if W.get("bias") is not None else None
    s = _Weights(f32=int(f32), bias=_ptr(bias))
    for k, v in arrs.items():
        setattr(s, k, _ptr(v))
    return s, (arrs, bias)


def _cfg_struct(cfg, **over):
    g = lambda k: over.get(k, getattr(cfg, k))
    return _Cfg(bf16=int(g("dtype") == "bf16"), b=g("b"), s=g("s"), h=g("h"), H=g("H"),
                d=g("d"), L=g("L"), E=g("E"), k=g("k"), f=g("f"), r=g("r"),
                ffn=_KIND[g("ffn")], normalize=int(bool(g("normalize"))),
                use_da=int(bool(g("use_da"))), use_ea=int(bool(g("use_ea"))),
                sa_rope=int(bool(g("sa_rope"))), proj_experts=int(g("proj_experts")),
                mixture=_MIX[g("mixture")], decode=int(bool(g("decode"))),
                sa_pos=int(g("sa_pos")), da_window=int(g("da_window")),
                da_dilation=int(g("da_dilation")), rope_base=float(g("rope_base")),
                rms_eps=float(g("rms_eps")), rho=float(g("rho")))


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (status {rc})")


# ---------------------------------------------------------------------------- pieces


def bf16_round(a) -> np.ndarray:
    """Nearest bfloat16 (ties to even), as float64; same shape (0-d for a scalar)."""
    x = _f64(a)
    out = np.empty_like(x)
    _bf16(_ptr(x), x.size, _ptr(out))
    return out


def rmsnorm(x, g, eps):
    x = _f64(x)
    g = _f64(g)
    out = np.empty_like(x)
    _check(_rms(_ptr(x), _ptr(g), x.size // x.shape[-1], x.shape[-1], float(eps), _ptr(out)),
           "rmsnorm")
    return out


def rope(u, pos, base):
    """Rotary embedding of u [..., D]; ``pos`` broadcasts against [..., D/2]."""
    u = _f64(u)
    D = u.shape[-1]
    p = _f64(np.broadcast_to(np.asarray(pos, np.float64), u.shape[:-1] + (D // 2,)))
    out = np.empty_like(u)
    _check(_rope(_ptr(u), _ptr(p), u.size // D, D, float(base), _ptr(out)), "rope")
    return out


def depth_rope(u, l, L, base):
    u = _f64(u)
    D = u.shape[-1]
    out = np.empty_like(u)
    _check(_drope(_ptr(u), u.size // D, D, int(l), int(L), float(base), _ptr(out)),
           "depth_rope")
    return out


def depth_keys(l, window=0, dilation=0) -> np.ndarray:
    buf = np.empty(int(l) + 1, np.int32)
    n = _dkeys(int(l), int(window), int(dilation), _ptr(buf))
    _check(0 if n >= 0 else 1, "depth_keys")
    return buf[:n].astype(np.int64)


def seq_attn(q, k_new, v_new, pos0=0, k_cache=None, v_cache=None, sa_rope=True,
             base=10000.0, bf16=False):
    """Causal SA of tokens at pos0.. over cached keys 0..pos0-1 and themselves.
    q, k_new, v_new [B, n, H, d]; caches [B, cap, H, d].  Returns (out, k_rot, v)."""
    q, k_new, v_new = _f64(q), _f64(k_new), _f64(v_new)
    B, n, H, d = q.shape
    cap, cf32 = 0, 0
    if pos0 > 0:
        if k_cache.dtype != np.float32:
            k_cache, v_cache = _f64(k_cache), _f64(v_cache)
        else:
            k_cache, v_cache = np.ascontiguousarray(k_cache), np.ascontiguousarray(v_cache)
            cf32 = 1
        cap = k_cache.shape[1]
    else:
        k_cache = v_cache = None
    out, k_rot, v_out = (np.empty_like(q) for _ in range(3))
    _check(_sattn(B, n, H, d, int(pos0), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                  _ptr(v_cache), cap, cf32, int(bool(sa_rope)), float(base), int(bool(bf16)),
                  _ptr(out), _ptr(k_rot), _ptr(v_out)), "seq_attn")
    return out, k_rot, v_out


def depth_attn(q, k_new, v_new, k_cache, v_cache, l, L, base=10000.0, bf16=False,
               use_rope=True, window=0, dilation=0):
    """DA at depth l; k_cache / v_cache [R, L, H, d] float64, slot l written in place."""
    q, k_new, v_new = _f64(q), _f64(k_new), _f64(v_new)
    for c in (k_cache, v_cache):
        if _inplace(c, "DA cache").dtype != np.float64:
            raise TypeError("DA caches must be float64")
    R, H, d = q.shape
    out = np.empty_like(q)
    _check(_dattn(R, H, d, int(l), int(L), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                  _ptr(v_cache), float(base), int(bool(bf16)), int(bool(use_rope)),
                  int(window), int(dilation), _ptr(out)), "depth_attn")
    return out


def topk_select(key, k):
    key = _f64(key)
    E = key.shape[-1]
    idx = np.empty(key.shape[:-1] + (int(k),), np.int64)
    _check(_topk(_ptr(key), key.size // E, E, int(k), _ptr(idx)), "topk_select")
    return idx


def _wpair(*ws):
    """Matrices for one call: all float32 when any is float32 (exact), else float64."""
    arrs, f32 = _weights_arrays({k: v for k, v in zip(("w_r", "keys", "w1", "w3", "w2"), ws)
                                 if v is not None})
    return arrs, f32


def _np(a):
    """A weight as a numpy array (torch tensors: float64 stays, other dtypes -> float32)."""
    if a is None:
        return None
    if hasattr(a, "detach"):
        t = a.detach().to("cpu")
        return (t if str(t.dtype) == "torch.float64" else t.float()).numpy()
    return np.asarray(a)


def expert_route(x, w_r, keys, bias, k, l, L, rho=1.0, normalize=True, base=10000.0):
    """Router at depth l.  Returns (idx [T, k] int64, gate [T, k], counts [E], z [T, E])."""
    x = _f64(x)
    arrs, f32 = _wpair(_np(w_r), _np(keys))
    bias = _f64(bias)
    T, h = x.shape
    r = arrs["w_r"].shape[0]
    E = arrs["keys"].shape[0]
    idx = np.empty((T, k), np.int64)
    gate = np.empty((T, k))
    counts = np.empty(E, np.int64)
    z = np.empty((T, E))
    _check(_route(T, h, r, E, int(k), int(l), int(L), _ptr(x), _ptr(arrs["w_r"]),
                  _ptr(arrs["keys"]), int(f32), _ptr(bias), float(rho), int(bool(normalize)),
                  float(base), _ptr(idx), _ptr(gate), _ptr(counts), _ptr(z)), "expert_route")
    return idx, gate, counts, z


def bias_update(bias, counts, lam):
    bias, counts = _f64(bias), _i64(counts)
    out = np.empty_like(bias)
    _check(_bupd(_ptr(bias), _ptr(counts), bias.size, float(lam), _ptr(out)), "bias_update")
    return out


def route_counts(idx, E):
    """Selections per expert: idx [..., n] (one depth [T, k], or [L, T, k] per leading
    index) -> counts [..., E]."""
    idx = _i64(idx)
    lead = idx.shape[:-2] if idx.ndim > 2 else ()
    n_sets = int(np.prod(lead)) if lead else 1
    out = np.empty((n_sets, int(E)), np.int64)
    _check(_rcount(_ptr(idx), n_sets, idx.size // n_sets, int(E), _ptr(out)), "route_counts")
    return out.reshape(*lead, int(E)) if lead else out[0]


def expert_usage(counts):
    """dict(distinct, max_over_mean, gini, lorenz) of counts [E]."""
    c = _i64(counts)
    E = c.size
    dist, mom, gini = C.c_int(), C.c_double(), C.c_double()
    lor = np.empty(E)
    _check(_usage(_ptr(c), E, C.byref(dist), C.byref(mom), C.byref(gini), _ptr(lor)),
           "expert_usage")
    return dict(distinct=int(dist.value), max_over_mean=float(mom.value),
                gini=float(gini.value), lorenz=lor)


def expert_ffn(kind, x, idx, gate, w1, w3=None, w2=None, residual=None, bf16=False,
               return_parts=False):
    """out[t] = residual[t] + sum_i gate[t,i] FFN_{idx[t,i]}(x[t]) (slot order).
    return_parts: also the gated stored slot outputs [T, k, h_out] and the stored hidden
    states [T, k, f] (None for "linear"): returns (out, slots, hidden)."""
    x, idx, gate = _f64(x), _i64(idx), _f64(gate)
    arrs, f32 = _wpair(None, None, _np(w1), _np(w3), _np(w2))
    T, h_in = x.shape
    k = idx.shape[1]
    w1a = arrs["w1"]
    E = w1a.shape[0]
    if kind == "linear":
        f, h_out = 0, w1a.shape[1]
    else:
        f, h_out = w1a.shape[1], arrs["w2"].shape[1]
    res = _f64(residual) if residual is not None else None
    out = np.empty((T, h_out))
    slots = np.empty((T, k, h_out)) if return_parts else None
    hidden = np.empty((T, k, f)) if return_parts and kind != "linear" else None
    _check(_ffn(_KIND[kind], T, h_in, f, h_out, E, k, _ptr(x), _ptr(idx), _ptr(gate),
                _ptr(w1a), _ptr(arrs.get("w3")), _ptr(arrs.get("w2")), int(f32), _ptr(res),
                int(bool(bf16)), _ptr(out), _ptr(slots), _ptr(hidden)), "expert_ffn")
    return (out, slots, hidden) if return_parts else out


# ----------------------------------------------------------------------------- layer


def prepare_weights(W: dict, big_as_f32: bool = False) -> dict:
    """Host copies of a synth weight dict (torch tensors or arrays): float64 matrices, or
    float32 ones with big_as_f32 (the same values: bf16 and f32 storage are exact in
    float32; the oracle still computes in float64).  The bias is float64."""
    out = {}
    for k_, v in W.items():
        if hasattr(v, "detach"):
            v = v.detach().to("cpu").float().numpy()
        keep32 = big_as_f32 and k_ != "bias"
        out[k_] = np.ascontiguousarray(np.asarray(v, np.float32 if keep32 else np.float64))
    return out


def new_da_cache(cfg):
    """DA caches [T, L, H, d] filled with NaN: a slot is always written before it is read."""
    shp = (cfg.T, cfg.L, cfg.H, cfg.d)
    return np.full(shp, np.nan), np.full(shp, np.nan)


def _sa_cache_args(sa_k, sa_v):
    if sa_k is None:
        return None, None, 0, 0
    _inplace(sa_k, "SA cache")
    _inplace(sa_v, "SA cache")
    if sa_k.dtype != sa_v.dtype:
        raise TypeError("SA caches must share a dtype")
    return sa_k, sa_v, sa_k.shape[2], int(sa_k.dtype == np.float32)


def _steps_buffers(cfg, n_steps, full):
    T, h, k, E, Ep = cfg.T, cfg.h, cfg.k, cfg.E, cfg.proj_experts
    buf = {}
    if cfg.use_ea:
        buf["idx"] = np.empty((n_steps, T, k), np.int64)
        buf["gate"] = np.empty((n_steps, T, k))
    if Ep:
        buf["pidx"] = np.empty((n_steps, T), np.int64)
        buf["pgate"] = np.empty((n_steps, T))
    if full:
        buf["x_next"] = np.empty((n_steps, T, h))
        buf["y"] = np.empty((n_steps, T, h))
        buf["yb"] = np.empty((n_steps, T, h))
        if cfg.use_ea:
            buf["counts"] = np.empty((n_steps, E), np.int64)
            buf["z"] = np.empty((n_steps, T, E))
        if Ep:
            buf["pz"] = np.empty((n_steps, T, Ep))
    s = _StepOut()
    for k_, v in buf.items():
        setattr(s, k_, _ptr(v))
    return s, buf


_STEP_KEYS = ("x_next", "y", "yb", "idx", "gate", "pidx", "pgate", "counts", "z", "pz")


def _step_dicts(buf, n):
    return [{k_: (buf[k_][i] if k_ in buf else None) for k_ in _STEP_KEYS} for i in range(n)]


def layer_step(cfg, W, x, l, da_k, da_v, sa_k=None, sa_v=None, force_idx=None,
               force_pidx=None):
    """One depth step l on x [T, h]; da_k / da_v [T, L, H, d] float64 (slot l written);
    sa_k / sa_v [L, b, cap, H, d] or None.  Returns dict(x_next, y, yb, idx, gate, pidx,
    pgate, counts, z, pz)."""
    x = _f64(x).reshape(cfg.T, cfg.h)
    for c in (da_k, da_v):
        if _inplace(c, "DA cache").dtype != np.float64:
            raise TypeError("DA caches must be float64")
    sk, sv, cap, cf32 = _sa_cache_args(sa_k, sa_v)
    ws, keep = _weights_struct(W)
    so, buf = _steps_buffers(cfg, 1, True)
    fi = _i64(force_idx) if force_idx is not None else None
    fp = _i64(force_pidx) if force_pidx is not None else None
    c = _cfg_struct(cfg)
    _check(_step(C.byref(c), C.byref(ws), _ptr(x), int(l), _ptr(da_k), _ptr(da_v), _ptr(sk),
                 _ptr(sv), cap, cf32, _ptr(fi), _ptr(fp), C.byref(so)), "layer_step")
    return _step_dicts(buf, 1)[0]


def layer_forward(cfg, W, x0, sa_k=None, sa_v=None, force_idx=None, force_pidx=None,
                  return_steps=False):
    """The unrolled layer x_0 -> x_L.  sa_k / sa_v [L, b, cap, H, d] float64 or float32
    (decode: positions 0..sa_pos-1 read, sa_pos appended; prefill: positions 0..s-1
    written), updated in place.  force_idx [L, T, k] / force_pidx [L, T]: expert choices
    to adopt.  Returns dict(x_out, da_k, da_v, idx, gate, pidx, pgate, steps)."""
    x0 = _f64(x0).reshape(cfg.T, cfg.h)
    sk, sv, cap, cf32 = _sa_cache_args(sa_k, sa_v)
    ws, keep = _weights_struct(W)
    so, buf = _steps_buffers(cfg, cfg.L, return_steps)
    da_k, da_v = new_da_cache(cfg)
    fi = _i64(force_idx) if force_idx is not None else None
    fp = _i64(force_pidx) if force_pidx is not None else None
    x_out = np.empty_like(x0)
    c = _cfg_struct(cfg)
    _check(_fwd(C.byref(c), C.byref(ws), _ptr(x0), _ptr(x_out), _ptr(da_k), _ptr(da_v),
                _ptr(sk), _ptr(sv), cap, cf32, _ptr(fi), _ptr(fp), C.byref(so)),
           "layer_forward")
    out = dict(x_out=x_out, da_k=da_k, da_v=da_v)
    if cfg.use_ea:
        out["idx"], out["gate"] = buf["idx"], buf["gate"]
    if cfg.proj_experts:
        out["pidx"], out["pgate"] = buf["pidx"], buf["pgate"]
    if return_steps:
        out["steps"] = _step_dicts(buf, cfg.L)
    return out


def decode_tokens(cfg, W, xs, sa_k, sa_v, return_steps=False):
    """n consecutive decode steps: xs [n, b, h]; token j at position cfg.sa_pos + j with a
    fresh DA cache, appended to sa_k / sa_v [L, b, cap, H, d] in place.  Returns
    dict(x_out [n, b, h], idx [n, L, b, k], gate, steps (per token, per depth))."""
    xs = _f64(xs)
    n = xs.shape[0]
    sk, sv, cap, cf32 = _sa_cache_args(sa_k, sa_v)
    ws, keep = _weights_struct(W)
    so, buf = _steps_buffers(cfg, n * cfg.L, return_steps)
    x_out = np.empty_like(xs)
    c = _cfg_struct(cfg)
    _check(_dec(C.byref(c), C.byref(ws), n, _ptr(xs), _ptr(x_out), _ptr(sk), _ptr(sv), cap,
                cf32, C.byref(so)), "decode_tokens")
    out = dict(x_out=x_out)
    if cfg.use_ea:
        out["idx"] = buf["idx"].reshape(n, cfg.L, cfg.T, cfg.k)
        out["gate"] = buf["gate"].reshape(n, cfg.L, cfg.T, cfg.k)
    if return_steps:
        d = _step_dicts(buf, n * cfg.L)
        out["steps"] = [d[j * cfg.L:(j + 1) * cfg.L] for j in range(n)]
    return out
