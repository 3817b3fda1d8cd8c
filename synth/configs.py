"""The five seeded synthetic workloads and the recipe that fills their tensors.

Shapes follow the workload descriptions (tiny fp32 layer; bf16 layer; bf16 layer with
linear-MoE projections; bf16 decode step; bf16 deep recurrence).  Every tensor is drawn
from ``synth.rng`` under its own tensor id, so a slice of any tensor can be regenerated
alone.  Nothing here computes any part of the layer.

Weight layout convention (shared by the oracle and the library): every projection
matrix is stored ``[out_features, in_features]`` (row-major), i.e. ``y = x @ W.T``.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import torch

from . import rng

# tensor ids (one stream each)
TID_X0 = 1
TID_WQKV = 10
TID_WO = 11
TID_WQKV_E = 12
TID_WQKV_SH = 13
TID_WO_E = 14
TID_WO_SH = 15
TID_WPR = 16
TID_PKEYS = 17
TID_WR = 20
TID_KEYS = 21
TID_BIAS = 22
TID_BIAS_PERM = 23
TID_W1 = 30
TID_W3 = 31
TID_W2 = 32
TID_SAK = 40
TID_SAV = 41

WEIGHT_STD = 0.02


@dataclass(frozen=True)
class DreamerConfig:
    name: str
    dtype: str          # "f32" or "bf16" storage
    b: int              # batch (decode: number of sequences)
    s: int              # sequence length (decode: 1 new token)
    h: int
    H: int
    d: int
    L: int
    E: int
    k: int
    f: int
    r: int
    ffn: str            # "gelu" or "swiglu"
    normalize: bool     # normalise the top-k gates
    bias: str           # "u0.1", "u0.2", "zipf1.1"
    seed: int
    proj_experts: int = 0   # >0: top-1 linear-MoE Q/K/V/O projections with this many experts
    decode: bool = False
    sa_pos: int = 0         # decode: cached positions per sequence (new token sits here)
    use_da: bool = True
    use_ea: bool = True
    sa_rope: bool = True
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    rho: float = 1.0
    mixture: str = "partial"  # "partial" (DA+SA, then EA), "serial", "parallel"
    da_window: int = 0        # DA over the most recent depths only (0: all depths)
    da_dilation: int = 0      # with a window: also every da_dilation-th older depth

    @property
    def T(self) -> int:
        return self.b * self.s

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "DreamerConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny": DreamerConfig("tiny", "f32", b=1, s=16, h=64, H=4, d=16, L=4, E=16, k=1, f=32,
                          r=16, ffn="gelu", normalize=False, bias="u0.1", seed=0),
    "small": DreamerConfig("small", "bf16", b=8, s=512, h=512, H=8, d=64, L=8, E=256, k=4,
                           f=64, r=64, ffn="swiglu", normalize=True, bias="u0.2", seed=1),
    "linear_moe": DreamerConfig("linear_moe", "bf16", b=4, s=2048, h=1024, H=16, d=64, L=16,
                                E=1024, k=8, f=128, r=64, ffn="swiglu", normalize=True,
                                bias="u0.2", seed=2, proj_experts=16),
    "decode": DreamerConfig("decode", "bf16", b=64, s=1, h=2048, H=32, d=64, L=32, E=4096,
                            k=8, f=128, r=64, ffn="swiglu", normalize=True, bias="u0.2",
                            seed=3, decode=True, sa_pos=4096),
    "deep": DreamerConfig("deep", "bf16", b=2, s=4096, h=2048, H=32, d=64, L=64, E=2048,
                          k=8, f=128, r=64, ffn="swiglu", normalize=True, bias="zipf1.1",
                          seed=4),
}
CONFIG_ORDER = ["tiny", "small", "linear_moe", "decode", "deep"]


def make_x0(cfg: DreamerConfig, device="cpu", b0: int = 0, nb: int | None = None,
            s_len: int | None = None) -> torch.Tensor:
    """Input stream x_0 ~ N(0,1), float32, shape [nb, s_len, h] taken from the full
    [b, s, h] draw (batches b0..b0+nb-1, positions 0..s_len-1)."""
    nb = cfg.b if nb is None else nb
    s_len = cfg.s if s_len is None else s_len
    rows = []
    for bi in range(b0, b0 + nb):
        off = bi * cfg.s * cfg.h
        rows.append(rng.normal((1, s_len, cfg.h), cfg.seed, TID_X0, 1.0, torch.float32,
                               device, offset=off))
    return torch.cat(rows, 0)


def make_bias(cfg: DreamerConfig, device="cpu") -> torch.Tensor:
    """EA router bias, float32 [E]."""
    if cfg.bias.startswith("u"):
        a = float(cfg.bias[1:])
        return rng.uniform((cfg.E,), cfg.seed, TID_BIAS, -a, a, torch.float32, device)
    if cfg.bias.startswith("zipf"):
        ex = float(cfg.bias[4:])
        perm = rng.permutation(cfg.E, cfg.seed, TID_BIAS_PERM).to(torch.float64)
        b = -0.2 + 0.4 * (perm + 1.0) ** (-ex)
        return b.to(torch.float32).to(device)
    raise ValueError(cfg.bias)


def make_weights(cfg: DreamerConfig, device="cpu", experts: bool = True) -> dict:
    """All parameters in storage dtype (the bias in float32).

    Keys: g [h]; dense: w_qkv [6h, h] (rows: SA q,k,v then DA q,k,v), w_o [h, 2h]
    (columns: SA output then DA output); linear MoE: w_qkv_e [Ep, 6h, h], w_qkv_sh [6h, h],
    w_o_e [Ep, h, 2h], w_o_sh [h, 2h], w_pr [r, h], pkeys [Ep, r];
    EA: w_r [r, h], keys [E, r], bias [E], w1 [E, f, h], w3 [E, f, h] (swiglu), w2 [E, h, f].
    With experts=False the three expert stacks are left out (callers that regenerate
    single experts on demand use ``expert_weight``)."""
    dt, sd, h, dev = cfg.torch_dtype, cfg.seed, cfg.h, device
    W = {"g": torch.ones(h, dtype=dt, device=dev)}
    nrm = lambda shape, tid: rng.normal(shape, sd, tid, WEIGHT_STD, dt, dev)
    if cfg.proj_experts:
        Ep = cfg.proj_experts
        W["w_qkv_e"] = nrm((Ep, 6 * h, h), TID_WQKV_E)
        W["w_qkv_sh"] = nrm((6 * h, h), TID_WQKV_SH)
        W["w_o_e"] = nrm((Ep, h, 2 * h), TID_WO_E)
        W["w_o_sh"] = nrm((h, 2 * h), TID_WO_SH)
        W["w_pr"] = nrm((cfg.r, h), TID_WPR)
        W["pkeys"] = nrm((Ep, cfg.r), TID_PKEYS)
    else:
        W["w_qkv"] = nrm((6 * h, h), TID_WQKV)
        W["w_o"] = nrm((h, 2 * h), TID_WO)
    W["w_r"] = nrm((cfg.r, h), TID_WR)
    W["keys"] = nrm((cfg.E, cfg.r), TID_KEYS)
    W["bias"] = make_bias(cfg, dev)
    if experts:
        W["w1"] = nrm((cfg.E, cfg.f, h), TID_W1)
        if cfg.ffn == "swiglu":
            W["w3"] = nrm((cfg.E, cfg.f, h), TID_W3)
        W["w2"] = nrm((cfg.E, h, cfg.f), TID_W2)
    return W


def expert_weight(cfg: DreamerConfig, name: str, e: int, device="cpu") -> torch.Tensor:
    """Regenerate one expert's matrix (name in w1, w3, w2) without drawing the stack."""
    tid = {"w1": TID_W1, "w3": TID_W3, "w2": TID_W2}[name]
    shape = (cfg.f, cfg.h) if name != "w2" else (cfg.h, cfg.f)
    n = shape[0] * shape[1]
    return rng.normal(shape, cfg.seed, tid, WEIGHT_STD, cfg.torch_dtype, device, offset=e * n)


def make_sa_cache(cfg: DreamerConfig, which: str, device="cpu", l0: int = 0,
                  nl: int | None = None, b0: int = 0, nb: int | None = None) -> torch.Tensor:
    """Decode SA cache contents N(0,1) (already rotated keys / values), storage dtype,
    shape [nl, nb, sa_pos, H, d] for depths l0.., sequences b0.. of the full
    [L, b, sa_pos, H, d] draw."""
    tid = TID_SAK if which == "k" else TID_SAV
    nl = cfg.L if nl is None else nl
    nb = cfg.b if nb is None else nb
    P, h = cfg.sa_pos, cfg.h
    out = torch.empty((nl, nb, P, cfg.H, cfg.d), dtype=cfg.torch_dtype, device=device)
    for li in range(nl):
        for bi in range(nb):
            off = ((l0 + li) * cfg.b + (b0 + bi)) * P * h
            out[li, bi] = rng.normal((P, cfg.H, cfg.d), cfg.seed, tid, 1.0, cfg.torch_dtype,
                                     device, offset=off)
    return out
