"""ctypes binding of libdreamer (include/dreamer.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU, allocates the outputs
and the scratch space with torch, and enqueues the library call on torch's current
stream.  All arithmetic happens in the library's HIP kernels; if the library cannot be
loaded, importing this module raises.
"""
from __future__ import annotations

import ctypes as C
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdreamer.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with python -m depth_recurrent_layer_amd.build")
lib = C.CDLL(LIB_PATH)

OK, E_INVAL, E_UNSUPPORTED, E_WORKSPACE, E_HIP = range(5)
F32, BF16 = 0, 1
FFN_GELU, FFN_SWIGLU, FFN_LINEAR = 0, 1, 2
FFN_KINDS = {"gelu": FFN_GELU, "swiglu": FFN_SWIGLU, "linear": FFN_LINEAR}
MIX_PARTIAL, MIX_SERIAL, MIX_PARALLEL = 0, 1, 2
MIXTURES = {"partial": MIX_PARTIAL, "serial": MIX_SERIAL, "parallel": MIX_PARALLEL}
KC = {"qkv_proj": 1, "seq_attn": 2, "depth_attn": 3, "route": 4, "permute": 5,
      "expert_ffn": 6, "combine": 7, "out_proj": 8, "attention": 9}

_vp, _i64, _i32, _f32, _f64, _sz = C.c_void_p, C.c_int64, C.c_int, C.c_float, C.c_double, C.c_size_t


class LayerCfg(C.Structure):
    _fields_ = [("dtype", _i32), ("b", _i32), ("s", _i32), ("h", _i32), ("H", _i32),
                ("d", _i32), ("L", _i32), ("E", _i32), ("k", _i32), ("f", _i32), ("r", _i32),
                ("ffn_kind", _i32), ("normalize_gates", _i32), ("use_da", _i32),
                ("use_ea", _i32), ("sa_rope", _i32), ("proj_experts", _i32),
                ("mixture", _i32), ("decode", _i32), ("sa_pos", _i64), ("sa_cap", _i64),
                ("rope_base", _f64), ("rms_eps", _f32), ("rho", _f32),
                ("branch_streams", _i32), ("da_window", _i32), ("da_dilation", _i32),
                ("fuse_attn", _i32)]


class LayerWeights(C.Structure):
    _fields_ = [(n, _vp) for n in ("g", "w_qkv", "w_o", "w_pr", "pkeys", "pbias", "w_r",
                                   "keys", "bias", "w1", "w3", "w2")]


def _sig(name, res, args):
    fn = getattr(lib, name)
    fn.restype = res
    fn.argtypes = args
    return fn


_sig("dreamer_last_error", C.c_char_p, [])
_sig("dreamer_version", _i32, [])
_sig("dreamer_rope_tables", _i32, [_i32, _i32, _f64, _vp, _vp, _vp])
_sig("dreamer_depth_attn", _i32, [_i32, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _vp, _f32, _vp])
_sig("dreamer_depth_attn_windowed", _i32, [_i32, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                           _vp, _vp, _vp, _vp, _vp, _f32, _i32, _i32, _vp])
_sig("dreamer_seq_attn_ws_bytes", _sz, [_i32, _i32, _i32, _i32, _i32, _i64])
_sig("dreamer_seq_attn", _i32, [_i32, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp,
                                _i64, _vp, _vp, _vp, _f32, _i32, _vp, _sz, _vp])
_sig("dreamer_seq_attn_noalloc", _i32, [_i32, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp,
                                        _vp, _i64, _vp, _vp, _vp, _f32, _i32, _vp])
_sig("dreamer_expert_route_ws_bytes", _sz, [_i64, _i32, _i32])
_sig("dreamer_expert_route", _i32, [_i32, _i64, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                    _vp, _vp, _f32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                    _vp])
_sig("dreamer_expert_ffn_ws_bytes", _sz, [_i32, _i32, _i64, _i32, _i32, _i32, _i32, _i32])
_sig("dreamer_expert_ffn", _i32, [_i32, _i32, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                  _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp])
_sig("dreamer_absorb_shared", _i32, [_i32, _i64, _i64, _vp, _vp, _vp, _vp])
_sig("dreamer_layer_ws_bytes", _sz, [C.POINTER(LayerCfg)])
_sig("dreamer_layer_forward", _i32, [C.POINTER(LayerCfg), C.POINTER(LayerWeights), _vp, _vp,
                                     _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _vp, _sz, _vp])
_sig("dreamer_route_counts", _i32, [_vp, _i64, _i64, _i32, _vp, _vp])
_sig("dreamer_bias_update", _i32, [_vp, _i32, _f32, _vp, _vp])
_sig("dreamer_expert_usage", _i32, [_vp, _i64, _i32, _vp, _vp])
_sig("dreamer_decode_ws_bytes", _sz, [C.POINTER(LayerCfg), _i32])
_sig("dreamer_decode_tokens", _i32, [C.POINTER(LayerCfg), C.POINTER(LayerWeights), _i32, _vp,
                                     _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp])
_sig("dreamer_timing_enable", _i32, [_i32, _i32])
_sig("dreamer_timing_read", _i32, [C.POINTER(_i32), C.POINTER(_f64)])
_sig("dreamer_timing_disable", _i32, [])

# every symbol the header declares (checked by the CPU tests)
EXPORTS = ["dreamer_last_error", "dreamer_version", "dreamer_rope_tables", "dreamer_depth_attn",
           "dreamer_depth_attn_windowed",
           "dreamer_seq_attn_ws_bytes", "dreamer_seq_attn", "dreamer_seq_attn_noalloc",
           "dreamer_expert_route_ws_bytes",
           "dreamer_expert_route", "dreamer_expert_ffn_ws_bytes", "dreamer_expert_ffn",
           "dreamer_absorb_shared", "dreamer_layer_ws_bytes", "dreamer_layer_forward",
           "dreamer_route_counts", "dreamer_bias_update", "dreamer_expert_usage",
           "dreamer_decode_ws_bytes", "dreamer_decode_tokens", "dreamer_timing_enable", "dreamer_timing_read", "dreamer_timing_disable"]


class DreamerError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libdreamer error {code}: {msg}")
        self.code = code


def _check(rc):
    if rc != OK:
        raise DreamerError(rc, lib.dreamer_last_error().decode())


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("libdreamer tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("libdreamer tensors must be contiguous")


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------------------ entries

def dreamer_rope_tables(D, npos, base=10000.0, device="cuda"):
    cos = torch.empty((npos, D // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    _check(lib.dreamer_rope_tables(D, npos, float(base), _p(cos), _p(sin), _stream()))
    return cos, sin


def dreamer_depth_attn(q, k_new, v_new, k_cache, v_cache, l, L, cos_d, sin_d, scale=None,
                       out=None, window=None, dilation=0):
    """q, k_new, v_new [rows, H, d]; caches [rows, L, H, d] (slot l written).  window /
    dilation (not None) call dreamer_depth_attn_windowed."""
    _dev(q, k_new, v_new, k_cache, v_cache, cos_d, sin_d)
    rows, H, d = q.shape
    out = torch.empty_like(q) if out is None else out
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    args = (_dt(q), rows, H, d, l, L, _p(q), _p(k_new), _p(v_new), _p(k_cache), _p(v_cache),
            _p(out), _p(cos_d), _p(sin_d), float(scale))
    if window is None:
        _check(lib.dreamer_depth_attn(*args, _stream()))
    else:
        _check(lib.dreamer_depth_attn_windowed(*args, int(window), int(dilation), _stream()))
    return out


def dreamer_seq_attn(q, k_new, v_new, pos0=0, k_cache=None, v_cache=None, cos_s=None,
                     sin_s=None, scale=None, sa_rope=True, out=None):
    """q, k_new, v_new [B, q_len, H, d]; caches [B, cap, H, d] or None."""
    _dev(q, k_new, v_new, k_cache, v_cache, cos_s, sin_s)
    B, n, H, d = q.shape
    dt = _dt(q)
    out = torch.empty_like(q) if out is None else out
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    cap = 0 if k_cache is None else k_cache.shape[1]
    wsb = lib.dreamer_seq_attn_ws_bytes(dt, B, n, H, d, pos0)
    ws = _ws(wsb, q.device)
    _check(lib.dreamer_seq_attn(dt, B, n, H, d, pos0, _p(q), _p(k_new), _p(v_new), _p(k_cache),
                                _p(v_cache), cap, _p(out), _p(cos_s), _p(sin_s), float(scale),
                                int(bool(sa_rope)), _p(ws), ws.numel(), _stream()))
    return out


def dreamer_seq_attn_noalloc(q, k_new, v_new, pos0=0, k_cache=None, v_cache=None, cos_s=None,
                             sin_s=None, scale=None, sa_rope=True, out=None):
    """dreamer_seq_attn on the library's fixed scratch (no workspace).  The library
    allocates nothing; `out` is allocated here only when not given."""
    _dev(q, k_new, v_new, k_cache, v_cache, cos_s, sin_s)
    B, n, H, d = q.shape
    out = torch.empty_like(q) if out is None else out
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    cap = 0 if k_cache is None else k_cache.shape[1]
    _check(lib.dreamer_seq_attn_noalloc(_dt(q), B, n, H, d, pos0, _p(q), _p(k_new), _p(v_new),
                                        _p(k_cache), _p(v_cache), cap, _p(out), _p(cos_s),
                                        _p(sin_s), float(scale), int(bool(sa_rope)),
                                        _stream()))
    return out


def dreamer_expert_route(x, w_r, keys, bias, k, l, L, cos_r, sin_r, rho=1.0, normalize=True):
    """x [T, h]; w_r [r, h]; keys [E, r]; bias [E] f32 -> (idx [T,k] i32, gate [T,k], counts [E])."""
    _dev(x, w_r, keys, bias, cos_r, sin_r)
    T, h = x.shape
    r, E = w_r.shape[0], keys.shape[0]
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    gate = torch.empty((T, k), dtype=torch.float32, device=x.device)
    counts = torch.empty((E,), dtype=torch.int32, device=x.device)
    ws = _ws(lib.dreamer_expert_route_ws_bytes(T, r, E), x.device)
    _check(lib.dreamer_expert_route(_dt(x), T, h, r, E, k, l, L, _p(x), _p(w_r), _p(keys),
                                    _p(bias), float(rho), int(bool(normalize)), _p(cos_r),
                                    _p(sin_r), _p(idx), _p(gate), _p(counts), _p(ws), ws.numel(),
                                    _stream()))
    return idx, gate, counts


def dreamer_expert_ffn(kind, x, idx, gate, w1, w3=None, w2=None, residual=None):
    """out [T, h_out] f32 = residual + sum_i gate[:, i] * FFN_idx[:, i](x)."""
    _dev(x, idx, gate, w1, w3, w2, residual)
    kind_i = FFN_KINDS[kind] if isinstance(kind, str) else int(kind)
    T, h_in = x.shape
    k = idx.shape[1]
    E = w1.shape[0]
    if kind_i == FFN_LINEAR:
        f, h_out = 0, w1.shape[1]
    else:
        f, h_out = w1.shape[1], w2.shape[1]
    dt = _dt(x)
    out = torch.empty((T, h_out), dtype=torch.float32, device=x.device)
    ws = _ws(lib.dreamer_expert_ffn_ws_bytes(dt, kind_i, T, h_in, f, h_out, E, k), x.device)
    _check(lib.dreamer_expert_ffn(dt, kind_i, T, h_in, f, h_out, E, k, _p(x), _p(idx), _p(gate),
                                  _p(w1), _p(w3), _p(w2), _p(residual), _p(out), _p(ws),
                                  ws.numel(), _stream()))
    return out


def dreamer_absorb_shared(w_e, w_shared):
    """out[e] = w_e[e] + w_shared (bf16: rounded once)."""
    _dev(w_e, w_shared)
    out = torch.empty_like(w_e)
    _check(lib.dreamer_absorb_shared(_dt(w_e), w_e.shape[0], w_shared.numel(), _p(w_e),
                                     _p(w_shared), _p(out), _stream()))
    return out


def make_layer_cfg(*, dtype, b, s, h, H, d, L, E, k, f, r, ffn="swiglu", normalize=True,
                   use_da=True, use_ea=True, sa_rope=True, proj_experts=0, decode=False,
                   sa_pos=0, sa_cap=0, rope_base=10000.0, rms_eps=1e-6, rho=1.0,
                   mixture=MIX_PARTIAL, branch_streams=False, da_window=0,
                   da_dilation=0, fuse_attn=True) -> LayerCfg:
    return LayerCfg(dtype=BF16 if dtype in ("bf16", BF16) else F32, b=b, s=s, h=h, H=H, d=d,
                    L=L, E=E, k=k, f=f, r=r, ffn_kind=FFN_KINDS[ffn] if isinstance(ffn, str) else ffn,
                    normalize_gates=int(bool(normalize)), use_da=int(bool(use_da)),
                    use_ea=int(bool(use_ea)), sa_rope=int(bool(sa_rope)),
                    proj_experts=proj_experts, mixture=mixture, decode=int(bool(decode)),
                    sa_pos=sa_pos, sa_cap=sa_cap, rope_base=rope_base, rms_eps=rms_eps, rho=rho,
                    branch_streams=int(bool(branch_streams)), da_window=da_window,
                    da_dilation=da_dilation, fuse_attn=int(bool(fuse_attn)))


def layer_ws_bytes(cfg: LayerCfg) -> int:
    return int(lib.dreamer_layer_ws_bytes(C.byref(cfg)))


def dreamer_layer_forward(cfg: LayerCfg, weights: dict, x_in, *, x_out=None, route=None,
                          proj_route=None, x_steps=None, y_steps=None, da_cache=None,
                          sa_cache=None, route_in=None, proj_route_in=None, ws=None):
    """The unrolled layer.  weights: dict of device tensors named like the struct fields
    (dense: w_qkv [6h,h], w_o [h,2h]; MoE: absorbed stacks).  Optional outputs are passed
    as preallocated tensors: route=(idx [L,T,k] i32, gate [L,T,k] f32),
    proj_route=(idx [L,T], gate [L,T]), x_steps [L,T,h] f32, y_steps [L,T,h] storage,
    da_cache=(k, v) [T,L,H,d], sa_cache=(k, v) [L,b,cap,H,d].  route_in [L,T,k] /
    proj_route_in [L,T] int32 replay given expert choices.  Returns x_out [T, h] f32."""
    W = LayerWeights(**{n: (weights[n].data_ptr() if weights.get(n) is not None else None)
                        for n, _ in LayerWeights._fields_})
    _dev(x_in, *[v for v in weights.values() if torch.is_tensor(v)])
    T = cfg.b * cfg.s
    x_out = torch.empty((T, cfg.h), dtype=torch.float32, device=x_in.device) if x_out is None else x_out
    if ws is None:
        ws = _ws(layer_ws_bytes(cfg), x_in.device)
    ri, rg = route if route is not None else (None, None)
    pi, pg = proj_route if proj_route is not None else (None, None)
    dk, dv = da_cache if da_cache is not None else (None, None)
    sk, sv = sa_cache if sa_cache is not None else (None, None)
    _dev(route_in, proj_route_in)
    for t in (route_in, proj_route_in):
        if t is not None and t.dtype != torch.int32:
            raise TypeError("route_in / proj_route_in must be int32")
    _check(lib.dreamer_layer_forward(C.byref(cfg), C.byref(W), _p(x_in), _p(x_out), _p(ri),
                                     _p(rg), _p(pi), _p(pg), _p(x_steps), _p(y_steps), _p(dk),
                                     _p(dv), _p(sk), _p(sv), _p(route_in), _p(proj_route_in),
                                     _p(ws), ws.numel(), _stream()))
    return x_out


def dreamer_route_counts(idx, E: int, n_sets: int = 1):
    """Selections per expert of int32 expert ids idx (n_sets equal sets, flattened):
    returns counts [n_sets, E] int32."""
    _dev(idx)
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise TypeError("idx must be a contiguous int32 tensor")
    counts = torch.empty((n_sets, E), dtype=torch.int32, device=idx.device)
    _check(lib.dreamer_route_counts(_p(idx), n_sets, idx.numel() // n_sets, E, _p(counts),
                                    _stream()))
    return counts


def dreamer_bias_update(counts, bias, lam: float):
    """bias += lam * sign(median(counts) - counts), in place (counts [E] int32, bias [E] f32)."""
    _dev(counts, bias)
    _check(lib.dreamer_bias_update(_p(counts), bias.numel(), float(lam), _p(bias), _stream()))
    return bias


def dreamer_expert_usage(counts):
    """counts [n_sets, E] int32 -> stats [n_sets, 3] f32 = (distinct, max/mean, Gini)."""
    _dev(counts)
    c = counts.reshape(-1, counts.shape[-1]).contiguous()
    stats = torch.empty((c.shape[0], 3), dtype=torch.float32, device=c.device)
    _check(lib.dreamer_expert_usage(_p(c), c.shape[0], c.shape[1], _p(stats), _stream()))
    return stats


def decode_ws_bytes(cfg: LayerCfg, n_tokens: int) -> int:
    return int(lib.dreamer_decode_ws_bytes(C.byref(cfg), n_tokens))


def dreamer_decode_tokens(cfg: LayerCfg, weights: dict, x_in, sa_cache, *, x_out=None,
                          route=None, da_cache=None, ws=None):
    """n decode steps: x_in [n, b, h] f32 (token j at position cfg.sa_pos + j),
    sa_cache=(k, v) [L, b, cap, H, d] appended in place, route=(idx, gate)
    [n, L, b, k], da_cache=(k, v) [b, L, H, d].  Returns x_out [n, b, h] f32."""
    W = LayerWeights(**{n: (weights[n].data_ptr() if weights.get(n) is not None else None)
                        for n, _ in LayerWeights._fields_})
    _dev(x_in, *[v for v in weights.values() if torch.is_tensor(v)])
    n = x_in.shape[0]
    x_out = torch.empty_like(x_in, dtype=torch.float32) if x_out is None else x_out
    if ws is None:
        ws = _ws(decode_ws_bytes(cfg, n), x_in.device)
    ri, rg = route if route is not None else (None, None)
    dk, dv = da_cache if da_cache is not None else (None, None)
    sk, sv = sa_cache
    _check(lib.dreamer_decode_tokens(C.byref(cfg), C.byref(W), n, _p(x_in), _p(x_out), _p(ri),
                                     _p(rg), _p(dk), _p(dv), _p(sk), _p(sv), _p(ws), ws.numel(),
                                     _stream()))
    return x_out


def timing_enable(kclass: str, max_launches: int):
    _check(lib.dreamer_timing_enable(KC[kclass], max_launches))


def timing_read():
    n = _i32(0)
    ms = _f64(0.0)
    _check(lib.dreamer_timing_read(C.byref(n), C.byref(ms)))
    return n.value, ms.value


def timing_disable():
    _check(lib.dreamer_timing_disable())
