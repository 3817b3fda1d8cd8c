"""Writes tests/golden/tiny_oracle.npz from the CPU oracle alone (regression fixture).

Run from the repository root:  python tests/golden/make_golden.py"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synth import CONFIGS, make_weights, make_x0  # noqa: E402

cfg = CONFIGS["tiny"]
W = oracle.prepare_weights(make_weights(cfg))
r = oracle.layer_forward(cfg, W, make_x0(cfg).numpy())
np.savez(os.path.join(ROOT, "tests", "golden", "tiny_oracle.npz"), x_out=r["x_out"],
         idx=r["idx"], gate=r["gate"])
print("wrote tiny_oracle.npz", r["x_out"].shape)
