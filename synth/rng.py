"""Counter-based random numbers for the seeded synthetic workloads.

This module only draws numbers: it holds none of the layer's arithmetic. Both the
CPU oracle (tests) and the GPU path (tests, bench) take their inputs from here.

Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; constants as in S. Vigna's public-domain
``splitmix64.c``).  The n-th output of stream ``(seed, tid)`` is
``mix(base + (n + 1) * GAMMA)`` with ``base = mix(seed * 2**32 + tid)``, so any
element of any tensor can be regenerated on its own (random access).

* uniform: the top 53 bits of an output, times 2**-53  -> [0, 1)
* normal:  Box-Muller on the uniform pair (2j, 2j+1); even n takes the cosine
  branch, odd n the sine branch.

All integer work is done in torch int64 (two's-complement wrap-around equals
arithmetic mod 2**64; logical right shifts are masked arithmetic shifts), so the
same numbers come out on the CPU and on a GPU device.  The float conversion goes
float64 -> float32 -> (optionally) bfloat16, each step round-to-nearest-even.
"""
from __future__ import annotations

import math

import torch

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MUL1 = 0xBF58476D1CE4E5B9
MUL2 = 0x94D049BB133111EB

_CHUNK = 1 << 24  # elements generated per pass (bounds the int64 temporaries)


def _s64(v: int) -> int:
    """Reinterpret an unsigned 64-bit constant as the signed int64 with the same bits."""
    v &= MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def _srl(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bits."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _srl(z, 30)) * _s64(MUL1)
    z = (z ^ _srl(z, 27)) * _s64(MUL2)
    return z ^ _srl(z, 31)


def mix_int(z: int) -> int:
    """Pure-Python SplitMix64 finaliser on an unsigned 64-bit int (the test pin)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * MUL1) & MASK64
    z = ((z ^ (z >> 27)) * MUL2) & MASK64
    return z ^ (z >> 31)


def stream_base(seed: int, tid: int) -> int:
    return mix_int(((seed & 0xFFFFFFFF) << 32) | (tid & 0xFFFFFFFF))


def raw_at(n: torch.Tensor, seed: int, tid: int) -> torch.Tensor:
    """The n-th 64-bit output (as int64 bits) of stream (seed, tid); n is an int64 tensor."""
    base = _s64(stream_base(seed, tid))
    return _mix(base + (n + 1) * _s64(GAMMA))


def uniform_at(n: torch.Tensor, seed: int, tid: int) -> torch.Tensor:
    """float64 uniforms in [0, 1) at counters n."""
    return _srl(raw_at(n, seed, tid), 11).to(torch.float64) * (2.0 ** -53)


def normal_at(n: torch.Tensor, seed: int, tid: int) -> torch.Tensor:
    """float64 standard normals at element indices n (Box-Muller, see module doc)."""
    j = n >> 1
    u1 = uniform_at(2 * j, seed, tid)
    u2 = uniform_at(2 * j + 1, seed, tid)
    r = torch.sqrt(-2.0 * torch.log1p(-u1))
    th = (2.0 * math.pi) * u2
    return torch.where((n & 1) == 0, r * torch.cos(th), r * torch.sin(th))


def _fill(shape, fn, dtype, device, offset: int = 0) -> torch.Tensor:
    numel = 1
    for s in shape:
        numel *= int(s)
    out = torch.empty(numel, dtype=dtype, device=device)
    for a in range(0, numel, _CHUNK):
        b = min(numel, a + _CHUNK)
        n = torch.arange(offset + a, offset + b, dtype=torch.int64, device=device)
        v = fn(n)
        out[a:b] = v.to(torch.float32).to(dtype) if dtype != torch.float64 else v
    return out.view(*shape)


def normal(shape, seed: int, tid: int, std: float = 1.0, dtype=torch.float32,
           device="cpu", offset: int = 0) -> torch.Tensor:
    """Tensor of N(0, std^2) draws; element i (row-major) uses counter offset + i."""
    return _fill(shape, lambda n: normal_at(n, seed, tid) * std, dtype, device, offset)


def uniform(shape, seed: int, tid: int, lo: float, hi: float, dtype=torch.float32,
            device="cpu") -> torch.Tensor:
    """Tensor of U(lo, hi) draws."""
    return _fill(shape, lambda n: lo + (hi - lo) * uniform_at(n, seed, tid), dtype, device)


def permutation(n: int, seed: int, tid: int) -> torch.Tensor:
    """A seeded permutation of 0..n-1 (stable argsort of uniforms), int64 on the CPU."""
    u = uniform_at(torch.arange(n, dtype=torch.int64), seed, tid)
    return torch.argsort(u, stable=True)
