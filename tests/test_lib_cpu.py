"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports every function
include/dreamer.h declares, and its validation rejects bad arguments before any launch."""
import ctypes as C
import os
import re

import pytest

from depth_recurrent_layer_amd import dreamer as D

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "dreamer.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dreamer_[a-z_0-9]+)\s*\(", src)))


def test_header_symbols_exported():
    names = header_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(D.lib, n), f"{n} declared in dreamer.h but not exported"
    assert sorted(D.EXPORTS) == names


def test_version_and_no_error():
    assert D.lib.dreamer_version() >= 100


def test_depth_attn_rejects_bad_depth():
    rc = D.lib.dreamer_depth_attn(D.BF16, 4, 2, 64, 5, 5, None, None, None, None, None, None,
                                  None, None, 0.125, None)
    assert rc == D.E_INVAL
    assert b"bad sizes" in D.lib.dreamer_last_error()


def test_depth_attn_rejects_head_dim():
    p = C.c_void_p(16)  # never dereferenced: validation fails first
    rc = D.lib.dreamer_depth_attn(D.BF16, 4, 2, 24, 0, 5, p, p, p, p, p, p, p, p, 0.1, None)
    assert rc == D.E_UNSUPPORTED


def test_depth_attn_windowed_rejects_negative_window():
    p = C.c_void_p(16)
    for w, dil in ((-1, 0), (2, -3)):
        rc = D.lib.dreamer_depth_attn_windowed(D.BF16, 4, 2, 64, 1, 5, p, p, p, p, p, p, p, p,
                                               0.1, w, dil, None)
        assert rc == D.E_INVAL
        assert b"window" in D.lib.dreamer_last_error()


def test_layer_rejects_negative_depth_window():
    cfg = D.make_layer_cfg(dtype="bf16", b=8, s=512, h=512, H=8, d=64, L=8, E=256, k=4, f=64,
                           r=64, da_window=-2)
    W = D.LayerWeights()
    rc = D.lib.dreamer_layer_forward(C.byref(cfg), C.byref(W), None, None, None, None, None,
                                     None, None, None, None, None, None, None, None, None, None,
                                     0, None)
    assert rc == D.E_INVAL
    assert b"da_window" in D.lib.dreamer_last_error()


def test_route_rejects_k_above_E():
    rc = D.lib.dreamer_expert_route(D.BF16, 8, 64, 16, 4, 5, 0, 2, None, None, None, None, 1.0,
                                    1, None, None, None, None, None, None, 0, None)
    assert rc == D.E_UNSUPPORTED


def test_expert_ffn_rejects_unsupported_width():
    p = C.c_void_p(16)
    rc = D.lib.dreamer_expert_ffn(D.BF16, D.FFN_SWIGLU, 8, 512, 96, 512, 4, 2, p, p, p, p, p, p,
                                  None, p, p, 1 << 30, None)
    assert rc == D.E_UNSUPPORTED


def test_seq_attn_decode_needs_cache():
    p = C.c_void_p(16)
    rc = D.lib.dreamer_seq_attn(D.BF16, 2, 1, 4, 64, 10, p, p, p, None, None, 0, p, p, p, 0.1,
                                1, p, 1 << 30, None)
    assert rc == D.E_INVAL


def test_workspace_too_small():
    p = C.c_void_p(16)
    rc = D.lib.dreamer_expert_route(D.BF16, 8, 64, 32, 16, 2, 0, 2, p, p, p, p, 1.0, 1, p, p, p,
                                    p, None, p, 8, None)
    assert rc == D.E_WORKSPACE


def test_layer_ws_and_validation():
    cfg = D.make_layer_cfg(dtype="bf16", b=8, s=512, h=512, H=8, d=64, L=8, E=256, k=4, f=64,
                           r=64)
    assert D.layer_ws_bytes(cfg) > 8 * 512 * 512 * 2 * 6
    bad = D.make_layer_cfg(dtype="bf16", b=8, s=512, h=500, H=8, d=64, L=8, E=256, k=4, f=64,
                           r=64)
    W = D.LayerWeights()
    rc = D.lib.dreamer_layer_forward(C.byref(bad), C.byref(W), None, None, None, None, None,
                                     None, None, None, None, None, None, None, None, None, None,
                                     0, None)
    assert rc == D.E_INVAL
    dec = D.make_layer_cfg(dtype="bf16", b=8, s=2, h=512, H=8, d=64, L=8, E=256, k=4, f=64,
                           r=64, decode=True, sa_pos=5, sa_cap=6)
    rc = D.lib.dreamer_layer_forward(C.byref(dec), C.byref(W), None, None, None, None, None,
                                     None, None, None, None, None, None, None, None, None, None,
                                     0, None)
    assert rc == D.E_INVAL


def test_timing_enable_rejects_bad_class():
    assert D.lib.dreamer_timing_enable(99, 4) == D.E_INVAL


def test_load_bookkeeping_validation():
    p = C.c_void_p(16)
    assert D.lib.dreamer_route_counts(p, 1, 10, 20000, p, None) == D.E_UNSUPPORTED
    assert D.lib.dreamer_route_counts(None, 1, 10, 8, p, None) == D.E_INVAL
    assert D.lib.dreamer_bias_update(None, 8, 0.1, p, None) == D.E_INVAL
    assert D.lib.dreamer_expert_usage(p, 2, 9000, p, None) == D.E_UNSUPPORTED
    assert D.lib.dreamer_expert_usage(p, 0, 8, p, None) == D.E_INVAL


def test_decode_tokens_validation():
    cfg = D.make_layer_cfg(dtype="bf16", b=4, s=1, h=256, H=4, d=64, L=2, E=32, k=2, f=64, r=64,
                           decode=True, sa_pos=10, sa_cap=12)
    W = D.LayerWeights()
    # 3 tokens need positions 10..12: sa_cap 12 is too small
    rc = D.lib.dreamer_decode_tokens(C.byref(cfg), C.byref(W), 3, None, None, None, None, None,
                                     None, None, None, None, 0, None)
    assert rc == D.E_INVAL
    cfg.decode = 0
    rc = D.lib.dreamer_decode_tokens(C.byref(cfg), C.byref(W), 1, None, None, None, None, None,
                                     None, None, None, None, 0, None)
    assert rc == D.E_INVAL and b"decode" in D.lib.dreamer_last_error()


def test_seq_attn_noalloc_rejects_shapes_beyond_its_scratch():
    """bf16 prefill with RoPE needs 6 B q_len H d bytes of scratch: 4 x 4096 x 16 x 64 needs
    96 MiB, more than the fixed 64 MiB; rejected before anything touches the device."""
    p = C.c_void_p(16)  # never dereferenced: the size check fails first
    rc = D.lib.dreamer_seq_attn_noalloc(D.BF16, 4, 4096, 16, 64, 0, p, p, p, None, None, 0, p,
                                        p, p, 0.125, 1, None)
    assert rc == D.E_WORKSPACE
    assert b"scratch" in D.lib.dreamer_last_error()
