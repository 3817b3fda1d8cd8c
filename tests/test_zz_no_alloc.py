"""dreamer_seq_attn_noalloc (scratch in the library's fixed device array) against
dreamer_seq_attn (scratch from a caller workspace): the same kernels, so the same bits,
through the C ABI.  Two calls in a row per case, the second with a smaller input, so the
second runs on an array that still holds the first call's contents."""
import pytest
import torch

from synth import rng

pytestmark = pytest.mark.gpu


def _t(shape, seed, tid, dtype):
    return rng.normal(shape, seed, tid, 1.0, dtype).cuda()


def _pair(D, dt, B, S, H, d, P, rope, seed):
    """One case on both entry points; caches cloned so each side appends to its own."""
    q, k, v = (_t((B, S, H, d), seed, j, dt) for j in range(3))
    cos, sin = D.dreamer_rope_tables(d, P + S)
    if P > 0:     # decode: positions 0..P-1 cached (already rotated), the token appended at P
        cap = P + 1
        kc = torch.full((B, cap, H, d), float("nan"), dtype=dt, device="cuda")
        vc = torch.full_like(kc, float("nan"))
        kc[:, :P] = _t((B, P, H, d), seed, 10, dt)
        vc[:, :P] = _t((B, P, H, d), seed, 11, dt)
    else:         # prefill: the rotated keys and the values written to the caches
        kc = torch.full((B, S + 2, H, d), float("nan"), dtype=dt, device="cuda")
        vc = torch.full_like(kc, float("nan"))
    kc2, vc2 = kc.clone(), vc.clone()
    ref = D.dreamer_seq_attn(q, k, v, P, kc, vc, cos, sin, sa_rope=rope)
    got = D.dreamer_seq_attn_noalloc(q, k, v, P, kc2, vc2, cos, sin, sa_rope=rope)
    torch.cuda.synchronize()
    assert torch.isfinite(got).all()
    assert torch.equal(got, ref)
    assert torch.equal(kc2.nan_to_num(7.0), kc.nan_to_num(7.0))
    assert torch.equal(vc2.nan_to_num(7.0), vc.nan_to_num(7.0))


@pytest.mark.parametrize("name,dt,first,second", [
    # decode, split-K partials in the scratch: 64 sequences x 8 heads over 1000 positions,
    # then 3 sequences over 300
    ("decode bf16", torch.bfloat16, (64, 1, 8, 64, 1000), (3, 1, 8, 64, 300)),
    ("decode f32", torch.float32, (16, 1, 4, 16, 700), (2, 1, 4, 16, 65)),
    # bf16 prefill with RoPE: rotated q / k and transposed v staged in the scratch
    ("prefill bf16", torch.bfloat16, (4, 640, 8, 64, 0), (1, 70, 8, 64, 0)),
    # float32 prefill: rotated keys / values staged in the scratch
    ("prefill f32", torch.float32, (2, 200, 4, 16, 0), (1, 37, 4, 16, 0)),
])
def test_seq_attn_noalloc_matches_workspace_entry(gpu_lib, name, dt, first, second):
    D = gpu_lib
    for i, (B, S, H, d, P) in enumerate((first, second)):
        print(f"seq_attn_noalloc {name} call {i}: B={B} S={S} H={H} d={d} P={P}", flush=True)
        _pair(D, dt, B, S, H, d, P, True, 50 + i)


def test_seq_attn_noalloc_rejects_large_shape(gpu_lib):
    D = gpu_lib
    q = torch.zeros((4, 4096, 16, 64), dtype=torch.bfloat16, device="cuda")
    cos, sin = D.dreamer_rope_tables(64, 4096)
    with pytest.raises(D.DreamerError) as ei:
        D.dreamer_seq_attn_noalloc(q, q, q, 0, None, None, cos, sin)
    assert ei.value.code == D.E_WORKSPACE
