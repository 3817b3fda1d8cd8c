"""Host logic of the benchmark: its algorithmic byte counts follow the oracle's key sets."""
import importlib.util
import os

import oracle
from synth import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_depth_key_counts_match_oracle():
    b = _bench()
    for l in range(40):
        for w in range(0, 9):
            for dil in range(0, 7):
                assert b.n_depth_keys(l, w, dil) == len(oracle.depth_keys(l, w, dil)), (l, w, dil)


def test_depth_attn_bytes_full_and_windowed():
    b = _bench()
    cfg = CONFIGS["small"]
    T, h, L = cfg.T, cfg.h, cfg.L
    # bf16: q and the output (2 rows) plus the key and value of each of the l + 1 slots
    full = b.algorithmic_work(cfg, [])["depth_attn"]["bytes"]
    assert full == sum(T * h * 2 * (2 + 2 * (l + 1)) for l in range(L))
    one = b.algorithmic_work(cfg.replace(da_window=1), [])["depth_attn"]["bytes"]
    assert one == L * T * h * 2 * 4
    # float32: q, k, v in, the key and value stored, the output (6 rows), 2 per older slot
    tiny = CONFIGS["tiny"]
    f32 = b.algorithmic_work(tiny, [])["depth_attn"]["bytes"]
    assert f32 == sum(tiny.T * tiny.h * 4 * (6 + 2 * l) for l in range(tiny.L))
