"""CPU oracle for one Dreamer depth-recurrent attention-mixture layer (forward).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this module.  The GPU library shares no code
with it (no kernels, helpers, tables or constants); both sides only share the seeded
input generator in ``synth``.

Plain float64 numpy, written from the method description, slow and obvious on purpose.

Page key used in citations (all pages describe arXiv 2601.21582, "Depth-Recurrent
Attention Mixtures: Giving Latent Reasoning the Attention it Deserves"):
  [PN]    papernotes.org paper notes (Chinese): section "Method / overall framework"
          (the loop flowchart and the DA-cache remark), "Key design 1" (depth attention,
          depth RoPE with half the dims reversed, the parallel-residual equation),
          "Key design 2" (expert attention, the gate equation, the bias update),
          "Key design 3" (linear-MoE projections, the shared-expert identity),
          "Loss / training" (RMSNorm on the residual stream), ablation table,
          "Limitations and outlook" (windowed / dilated depth attention as future work).
  [GS-de] gist.science German technical summary, section "Methodik: Dreamer-Framework".
  [GS-nl] gist.science Dutch technical summary, section "Methodologie: Dreamer Framework".

Where the pages leave a step open, the reading taken is stated at the function
(ids R1..R20 are listed with their reasons in the design notes of the repository).

Storage emulation: with ``bf16=True`` every value that the GPU path stores in bfloat16
is rounded to bfloat16 (round-to-nearest-even) at the same named points:
x_hat as projection input (the residual keeps it unrounded), the six projections,
rotated q/k, attention outputs, the bf16 copy of y, the expert hidden state, the gated
expert outputs.  Everything else stays float64.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

# ----------------------------------------------------------------------------- rounding


def bf16_round(a) -> np.ndarray:
    """Round to the nearest bfloat16 value (ties to even), returned as float64.

    Goes through float32 first (both steps round to nearest even)."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    out = u.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isnan(f), np.nan, out)


def _store(bf16: bool):
    return bf16_round if bf16 else (lambda a: np.asarray(a, dtype=np.float64))


# ------------------------------------------------------------------------------ pieces


def rmsnorm(x, g, eps):
    """Residual-stream RMSNorm ([PN] "Loss / training"; flowchart node at the loop head).
    R3: eps added to the mean square; gain g multiplies."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, np.float64)


def rope(u, pos, base):
    """Rotary embedding, rotate-half pairing (i, i + D/2), theta_i = base^(-2i/D).

    ``pos`` broadcasts against [..., D/2]: one position per frequency pair (R4, R5)."""
    u = np.asarray(u, np.float64)
    D = u.shape[-1]
    half = D // 2
    theta = base ** (-2.0 * np.arange(half) / D)
    ang = np.asarray(pos, np.float64) * theta
    c, s = np.cos(ang), np.sin(ang)
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def depth_positions(l, L, D):
    """Per-pair positions of depth RoPE ([PN] "Key design 1"; [GS-de] DA encoding).

    R4: half of the rotary pairs are 'reversed': pairs i < D/4 sit at depth l, pairs
    i >= D/4 sit at L-1-l (distance to the maximum depth)."""
    i = np.arange(D // 2)
    return np.where(i < D // 4, float(l), float(L - 1 - l))


def depth_rope(u, l, L, base):
    return rope(u, depth_positions(l, L, u.shape[-1]), base)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, np.float64)))


def gelu(x):
    """R13: exact (erf) GELU."""
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def silu(x):
    x = np.asarray(x, np.float64)
    return x * sigmoid(x)


def softmax_lastdim(s):
    s = s - np.max(s, axis=-1, keepdims=True)
    e = np.exp(s)
    return e / np.sum(e, axis=-1, keepdims=True)


# -------------------------------------------------------------------- sequence attention


def seq_attn(q, k_new, v_new, pos0=0, k_cache=None, v_cache=None, sa_rope=True,
             base=10000.0, bf16=False):
    """Causal sequence attention SA at one depth ([PN] "Method": SA(x_l) in the
    parallel-residual equation; [GS-de] "standard self-attention" along tokens).

    q, k_new, v_new: [B, n, H, d] projections of the n new tokens at positions
    pos0..pos0+n-1.  k_cache/v_cache: [B, >=pos0, H, d] already-rotated keys and values
    of positions 0..pos0-1 (decode), or None when pos0 == 0.
    R5: plain RoPE over sequence positions on q and k; R6: scale 1/sqrt(d).
    Returns (out [B, n, H, d], k_rot [B, n, H, d], v [B, n, H, d]) where k_rot/v are the
    values appended to the cache at pos0.."""
    st = _store(bf16)
    q, k_new, v_new = (np.asarray(a, np.float64) for a in (q, k_new, v_new))
    B, n, H, d = q.shape
    if sa_rope:
        p = (pos0 + np.arange(n, dtype=np.float64))[None, :, None, None]
        q = st(rope(q, p, base))
        k_new = st(rope(k_new, p, base))
    if pos0 > 0:
        K = np.concatenate([np.asarray(k_cache[:, :pos0], np.float64), k_new], axis=1)
        V = np.concatenate([np.asarray(v_cache[:, :pos0], np.float64), v_new], axis=1)
    else:
        K, V = k_new, v_new
    # scores[b, h, i, j] = q[b, i, h] . K[b, j, h] / sqrt(d)
    qt, Kt, Vt = (a.transpose(0, 2, 1, 3) for a in (q, K, V))
    s = np.matmul(qt, Kt.transpose(0, 1, 3, 2)) / np.sqrt(d)
    qi = pos0 + np.arange(n)[:, None]
    kj = np.arange(K.shape[1])[None, :]
    s = np.where(kj <= qi, s, -np.inf)
    p_ = softmax_lastdim(s)
    out = np.matmul(p_, Vt).transpose(0, 2, 1, 3)
    return st(out), k_new, v_new


# ----------------------------------------------------------------------- depth attention


def depth_keys(l, window=0, dilation=0):
    """Depth slots read by DA at depth l (R26: the local-window plus dilated sparse depth
    attention that [PN] "Limitations and outlook" proposes as future work).  window 0: every depth 0..l.  window
    w > 0: the w most recent depths l-w+1..l, plus, when dilation D > 0, every older depth
    j with (l - j) divisible by D.  The current depth is always read."""
    if window <= 0:
        return np.arange(l + 1)
    return np.array([j for j in range(l + 1)
                     if l - j < window or (dilation > 0 and (l - j) % dilation == 0)])


def depth_attn(q, k_new, v_new, k_cache, v_cache, l, L, base=10000.0, bf16=False,
               use_rope=True, window=0, dilation=0):
    """Depth attention DA at depth l ([PN] "Key design 1"; [GS-de]/[GS-nl] DA bullets).

    Each of the R rows (tokens, b*s flattened) attends over its own keys at depths
    0..l (R1: inclusive of the current depth), with depth RoPE (half reversed, R4) on
    q and on the new key.  The rotated new key and the value are written into slot l
    of k_cache/v_cache ([R, L, H, d], modified in place), so the cache never depends on
    the sequence length; slots > l are never read.  window / dilation restrict the keys
    to depth_keys(l, window, dilation) (R26).
    Returns out [R, H, d]."""
    st = _store(bf16)
    q = np.asarray(q, np.float64)
    k_new = np.asarray(k_new, np.float64)
    d = q.shape[-1]
    if use_rope:
        q = st(depth_rope(q, l, L, base))
        k_new = st(depth_rope(k_new, l, L, base))
    k_cache[:, l] = k_new
    v_cache[:, l] = np.asarray(v_new, np.float64)
    keys = depth_keys(l, window, dilation)
    K = np.asarray(k_cache[:, keys], np.float64)   # [R, n_keys, H, d]
    V = np.asarray(v_cache[:, keys], np.float64)
    # s[r, h, j] = q[r, h] . K[r, j, h] / sqrt(d)
    s = np.matmul(q[:, :, None, :], K.transpose(0, 2, 3, 1))[:, :, 0, :] / np.sqrt(d)
    p_ = softmax_lastdim(s)
    return st(np.matmul(p_[:, :, None, :], V.transpose(0, 2, 1, 3))[:, :, 0, :])


# ------------------------------------------------------------------------------ routing


def topk_select(key, k):
    """The k largest entries of each row of ``key``, descending; ties go to the lower
    expert index (R10).  Uses a stable sort (library primitive)."""
    order = np.argsort(-key, axis=-1, kind="stable")
    return order[..., :k]


def expert_route(x, w_r, keys, bias, k, l, L, rho=1.0, normalize=True, base=10000.0):
    """Expert-attention router ([PN] "Key design 2"; [GS-de] routing bullet).

    Low-rank query u = x W_r^T, depth RoPE on u (R8: query only, keys are position-less
    parameters), scores z = rho * u . keys_e (R17: rho = 1 in the workloads).
    Gate equation sigma = norm(TopK(sigmoid(z), z + b, k)): the experts are chosen by
    z + b (R10), their values are sigmoid(z) of the unbiased score, and 'norm' divides
    by the sum of the k selected values (R11; skipped when normalize is False).
    Returns (idx [T, k] int64, gate [T, k] float64, counts [E] int64, z [T, E])."""
    x = np.asarray(x, np.float64)
    u = x @ np.asarray(w_r, np.float64).T
    u = depth_rope(u, l, L, base)
    z = rho * (u @ np.asarray(keys, np.float64).T)
    keyv = z + np.asarray(bias, np.float64)[None, :]
    idx = topk_select(keyv, k)
    gate = sigmoid(np.take_along_axis(z, idx, axis=-1))
    if normalize:
        gate = gate / np.sum(gate, axis=-1, keepdims=True)
    counts = np.bincount(idx.reshape(-1), minlength=keys.shape[0])
    return idx, gate, counts, z


def bias_update(bias, counts, lam):
    """Balancing update b <- b + lam * sign(median(N) - N) ([PN] "Key design 2")."""
    N = np.asarray(counts, np.float64)
    return np.asarray(bias, np.float64) + lam * np.sign(np.median(N) - N)


def route_counts(idx, E):
    """Selections per expert: idx [..., n] (the routing of one depth, or [L, T, k] for all
    depths with the trailing dims flattened per leading index) -> counts [..., E]."""
    idx = np.asarray(idx)
    lead = idx.shape[:-2] if idx.ndim > 2 else ()
    flat = idx.reshape(int(np.prod(lead)) if lead else 1, -1)
    out = np.stack([np.bincount(r, minlength=E) for r in flat])
    return out.reshape(*lead, E) if lead else out[0]


def expert_usage(counts):
    """Usage statistics of per-expert selection counts ([PN] analysis of expert usage:
    unique experts per depth, Lorenz curve and Gini coefficient of the load).
    counts [E] -> dict(distinct = #experts selected at least once, max_over_mean,
    gini = sum_i sum_j |N_i - N_j| / (2 E^2 mean(N)) (the mean-difference definition),
    lorenz = cumulative share of all selections held by the 1, 2, .., E least used
    experts)."""
    N = np.asarray(counts, np.float64)
    E = N.size
    mean = N.mean()
    gini = np.abs(N[:, None] - N[None, :]).sum() / (2.0 * E * E * mean)
    lorenz = np.cumsum(np.sort(N)) / N.sum()
    return dict(distinct=int((N > 0).sum()), max_over_mean=float(N.max() / mean),
                gini=float(gini), lorenz=lorenz)


# ------------------------------------------------------------------------------ experts


def expert_ffn(kind, x, idx, gate, w1, w3=None, w2=None, residual=None, bf16=False):
    """Sparse expert attention, value side ([PN] "Key design 2": every expert's FFN is
    the value transform; dropless, every selected (token, expert) pair is computed).

    out[t] = residual[t] + sum_i gate[t,i] * FFN_{idx[t,i]}(x[t]), summed in slot order i.
    kind "swiglu": FFN(x) = W2 (silu(x W1^T) * (x W3^T)); "gelu": W2 gelu(x W1^T)
    (R13); "linear": gate * x W1[e]^T (the linear-MoE projection experts, R12)."""
    st = _store(bf16)
    x = np.asarray(x, np.float64)
    T, kk = idx.shape
    n_out = w1.shape[1] if kind == "linear" else w2.shape[1]
    slots = np.zeros((T, kk, n_out))
    for e in np.unique(idx):
        rows, cols = np.nonzero(idx == e)
        xe = x[rows]
        W1 = np.asarray(w1[e], np.float64)
        if kind == "linear":
            o = xe @ W1.T
        else:
            a = xe @ W1.T
            if kind == "swiglu":
                hid = silu(a) * (xe @ np.asarray(w3[e], np.float64).T)
            elif kind == "gelu":
                hid = gelu(a)
            else:
                raise ValueError(kind)
            o = st(hid) @ np.asarray(w2[e], np.float64).T
        slots[rows, cols] = st(gate[rows, cols][:, None] * o)
    out = np.zeros((T, n_out)) if residual is None else np.asarray(residual, np.float64).copy()
    for i in range(kk):
        out = out + slots[:, i]
    return out


# --------------------------------------------------------------------------------- layer


def _f64(a):
    return None if a is None else np.asarray(a, np.float64)


def prepare_weights(W: dict, big_as_f32: bool = False) -> dict:
    """float64 copies of a synth weight dict (torch tensors or arrays).  With big_as_f32
    the expert stacks stay float32 arrays (the same values; read per expert as float64)."""
    out = {}
    for k_, v in W.items():
        if hasattr(v, "detach"):
            v = v.detach().to("cpu").float().numpy()
        keep32 = big_as_f32 and k_ in ("w1", "w3", "w2", "w_qkv_e", "w_o_e")
        out[k_] = np.asarray(v, np.float32 if keep32 else np.float64)
    return out


def _project(cfg, W, x, name, pidx, pgate, st):
    """Q/K/V (name 'qkv', x = x_hat) or output (name 'o', x = attention outputs)
    projection.  Dense, or the top-1 linear MoE of [PN] "Key design 3": per token
    sigma * x W_e + max(sigma_hat) * x W_shared with max(sigma_hat) = sigma for top-1
    (R12); this unabsorbed form is kept on purpose."""
    if not cfg.proj_experts:
        return x @ W["w_" + name].T
    We, Wsh = W["w_%s_e" % name], W["w_%s_sh" % name]
    out = np.empty((x.shape[0], We.shape[1]))
    for e in np.unique(pidx):
        rows = np.nonzero(pidx == e)[0]
        out[rows] = pgate[rows, None] * (x[rows] @ We[e].T)
    out += pgate[:, None] * (x @ Wsh.T)
    return out


def _sa_branch(cfg, W, qkv, l, sa_k, sa_v, st, bf16):
    """SA at depth l from the SA columns [q | k | v] of a projection ([PN] equation:
    SA(x_l)).  R21: q and k are rotated from the projection itself and stored once,
    rotated; v is stored as projected; rotation by sequence position (R5)."""
    T, h, H, d = cfg.T, cfg.h, cfg.H, cfg.d
    b, s, base = cfg.b, cfg.s, cfg.rope_base
    q_sa, k_sa, v_sa = [qkv[:, j * h:(j + 1) * h].reshape(T, H, d) for j in range(3)]
    pos = np.full(T, float(cfg.sa_pos)) if cfg.decode else (np.arange(T) % s).astype(float)
    if cfg.sa_rope:
        q_sa = rope(q_sa, pos[:, None, None], base)
        k_sa = rope(k_sa, pos[:, None, None], base)
    q_sa, k_sa, v_sa = st(q_sa), st(k_sa), st(v_sa)
    if cfg.decode:
        P = cfg.sa_pos
        a_sa, k_rot, v_app = seq_attn(q_sa.reshape(b, 1, H, d), k_sa.reshape(b, 1, H, d),
                                      v_sa.reshape(b, 1, H, d), P, sa_k[l], sa_v[l],
                                      False, base, bf16)
        sa_k[l][:, P] = k_rot[:, 0]
        sa_v[l][:, P] = v_app[:, 0]
    else:
        a_sa, k_rot, v_app = seq_attn(q_sa.reshape(b, s, H, d), k_sa.reshape(b, s, H, d),
                                      v_sa.reshape(b, s, H, d), 0, None, None, False,
                                      base, bf16)
        if sa_k is not None:
            sa_k[l][:, :s] = k_rot
            sa_v[l][:, :s] = v_app
    return a_sa.reshape(T, h)


def _da_branch(cfg, W, qkv, l, da_k, da_v, st, bf16):
    """DA over depths 0..l from the DA columns [q | k | v] of a projection (R1, R4, R21:
    q and k rotated by depth, stored once)."""
    T, h, H, d, L = cfg.T, cfg.h, cfg.H, cfg.d, cfg.L
    if not cfg.use_da:
        return np.zeros((T, h))
    q_da, k_da, v_da = [qkv[:, (3 + j) * h:(4 + j) * h].reshape(T, H, d) for j in range(3)]
    q_da = st(depth_rope(q_da, l, L, cfg.rope_base))
    k_da = st(depth_rope(k_da, l, L, cfg.rope_base))
    return depth_attn(q_da, k_da, st(v_da), da_k, da_v, l, L, cfg.rope_base, bf16,
                      use_rope=False, window=getattr(cfg, "da_window", 0),
                      dilation=getattr(cfg, "da_dilation", 0)).reshape(T, h)


def layer_step(cfg, W, x, l, da_k, da_v, sa_k=None, sa_v=None, force_idx=None,
               force_pidx=None):
    """One depth step l ([PN] flowchart: RMSNorm -> DA + SA -> residual -> EA).

    x: [T, h] residual stream x_l (float64).  da_k/da_v: [T, L, H, d] DA caches
    (slot l written here).  Decode (cfg.decode): sa_k/sa_v [L, b, cap, H, d] hold the
    rotated keys/values of positions 0..sa_pos-1; this token is appended at sa_pos.
    Prefill with sa_k given: positions 0..s-1 of depth l are written (prefill -> decode
    handoff).  force_idx / force_pidx adopt externally given routing (the gates still
    come from this step's own scores).

    cfg.mixture ([PN] ablation of the mixture's parallelism; R22):
      "partial"  y = x^ + DA(x^) + SA(x^),  x' = y + EA(y)           (the pages' default)
      "serial"   u = x^ + DA(x^),  v = u + SA(u),  x' = v + EA(v)     (DA -> SA -> EA)
      "parallel" x' = x^ + DA(x^) + SA(x^) + EA(x^)                   (all three at once)
    Returns dict(x_next, y, yb, idx, gate, pidx, pgate, counts, z, pz); y / yb is the
    stream EA reads from (partial, serial) or the attention sum (parallel)."""
    bf16 = cfg.dtype == "bf16"
    st = _store(bf16)
    T, h, L = cfg.T, cfg.h, cfg.L
    base = cfg.rope_base
    mix = getattr(cfg, "mixture", "partial")
    # R2: one RMSNorm per step, on the stream itself, at the loop head; x_hat is both
    # the attention input and the residual of the parallel-residual equation.  R20: the
    # residual keeps x_hat at full precision; the projections read its storage copy.
    xh = rmsnorm(x, W["g"], cfg.rms_eps)
    xhb = st(xh)
    pidx = pgate = pz = None
    if cfg.proj_experts:
        # R12: one top-1 projection router per token and depth on x_hat, shared by all
        # Q/K/V/O projection MoEs; gate = raw sigmoid; bias 0.
        pidx, pgate, _, pz = expert_route(xhb, W["w_pr"], W["pkeys"],
                                          np.zeros(cfg.proj_experts), 1, l, L, cfg.rho,
                                          normalize=False, base=base)
        if force_pidx is not None:
            pidx = np.asarray(force_pidx).reshape(T, 1)
            pgate = sigmoid(np.take_along_axis(pz, pidx, axis=-1))
        pidx, pgate = pidx[:, 0], pgate[:, 0]
    zero = np.zeros((T, h))
    if mix == "serial":
        # R22: DA first on x_hat; its residual sum u feeds SA (through u's storage copy);
        # the output projections act on one branch at a time ([a_SA | 0], [0 | a_DA]).
        a_da = _da_branch(cfg, W, _project(cfg, W, xhb, "qkv", pidx, pgate, st), l,
                          da_k, da_v, st, bf16)
        u = xh + _project(cfg, W, np.concatenate([zero, a_da], axis=1), "o", pidx, pgate, st)
        a_sa = _sa_branch(cfg, W, _project(cfg, W, st(u), "qkv", pidx, pgate, st), l,
                          sa_k, sa_v, st, bf16)
        y = u + _project(cfg, W, np.concatenate([a_sa, zero], axis=1), "o", pidx, pgate, st)
    else:
        qkv = _project(cfg, W, xhb, "qkv", pidx, pgate, st)
        a_sa = _sa_branch(cfg, W, qkv, l, sa_k, sa_v, st, bf16)
        a_da = _da_branch(cfg, W, qkv, l, da_k, da_v, st, bf16)
        # Parallel residual y = x_l + DA(x_{:l}) + SA(x_l) ([PN] "Key design 1"); the two
        # output projections act on [a_SA | a_DA] (R6: separate SA and DA projections).
        y = xh + _project(cfg, W, np.concatenate([a_sa, a_da], axis=1), "o", pidx, pgate,
                          st)
    yb = st(y)
    idx = gate = counts = z = None
    x_next = y
    if cfg.use_ea:
        # R7: EA reads y (no second norm); in the fully parallel wiring it reads x_hat.
        ea_in = xhb if mix == "parallel" else yb
        idx, gate, counts, z = expert_route(ea_in, W["w_r"], W["keys"], W["bias"], cfg.k, l,
                                            L, cfg.rho, cfg.normalize, base)
        if force_idx is not None:
            idx = np.asarray(force_idx).reshape(T, cfg.k)
            gate = sigmoid(np.take_along_axis(z, idx, axis=-1))
            if cfg.normalize:
                gate = gate / np.sum(gate, axis=-1, keepdims=True)
            counts = np.bincount(idx.reshape(-1), minlength=cfg.E)
        x_next = expert_ffn(cfg.ffn, ea_in, idx, gate, W["w1"], W.get("w3"), W["w2"],
                            residual=y, bf16=bf16)
    return dict(x_next=x_next, y=y, yb=yb, idx=idx, gate=gate, pidx=pidx, pgate=pgate,
                counts=counts, z=z, pz=pz)


def new_da_cache(cfg):
    """DA caches [T, L, H, d] filled with NaN: a slot is always written before it is read."""
    shp = (cfg.T, cfg.L, cfg.H, cfg.d)
    return np.full(shp, np.nan), np.full(shp, np.nan)


def layer_forward(cfg, W, x0, sa_k=None, sa_v=None, force_idx=None, force_pidx=None,
                  return_steps=False):
    """The unrolled layer x_0 -> x_L ([PN] flowchart: repeat until depth L; one shared
    set of parameters at every depth).  R15: no embedding or head; the output is x_L.

    force_idx / force_pidx: optional [L, T, k] / [L, T] routing to adopt per depth.
    Returns dict(x_out, idx [L,T,k], gate [L,T,k], pidx, pgate, steps (optional))."""
    x = np.asarray(x0, np.float64).reshape(cfg.T, cfg.h)
    da_k, da_v = new_da_cache(cfg)
    idxs, gates, pidxs, pgates, steps = [], [], [], [], []
    for l in range(cfg.L):
        r = layer_step(cfg, W, x, l, da_k, da_v, sa_k, sa_v,
                       None if force_idx is None else force_idx[l],
                       None if force_pidx is None else force_pidx[l])
        x = r["x_next"]
        idxs.append(r["idx"])
        gates.append(r["gate"])
        pidxs.append(r["pidx"])
        pgates.append(r["pgate"])
        if return_steps:
            steps.append(r)
    out = dict(x_out=x, da_k=da_k, da_v=da_v)
    if cfg.use_ea:
        out["idx"], out["gate"] = np.stack(idxs), np.stack(gates)
    if cfg.proj_experts:
        out["pidx"], out["pgate"] = np.stack(pidxs), np.stack(pgates)
    if return_steps:
        out["steps"] = steps
    return out


def decode_tokens(cfg, W, xs, sa_k, sa_v, return_steps=False):
    """n consecutive decode steps ([PN] inference: SA keys / values persist across tokens
    per depth, DA's cache lives only within one token's depth steps).  xs: [n, b, h]; token
    j runs at position cfg.sa_pos + j with a fresh (NaN) DA cache and appends to
    sa_k / sa_v [L, b, cap, H, d] in place.  Returns dict(x_out [n, b, h], idx [n, L, b, k],
    gate, steps (optional))."""
    xs = np.asarray(xs, np.float64)
    outs, idxs, gates, steps = [], [], [], []
    for j in range(xs.shape[0]):
        cj = cfg.replace(sa_pos=cfg.sa_pos + j)
        r = layer_forward(cj, W, xs[j], sa_k, sa_v, return_steps=return_steps)
        outs.append(r["x_out"])
        if cfg.use_ea:
            idxs.append(r["idx"])
            gates.append(r["gate"])
        if return_steps:
            steps.append(r["steps"])
    out = dict(x_out=np.stack(outs))
    if cfg.use_ea:
        out["idx"], out["gate"] = np.stack(idxs), np.stack(gates)
    if return_steps:
        out["steps"] = steps
    return out
