"""The SplitMix64 -> Box-Muller stream of synth.rng, evaluated with torch ops.

Used to generate large inputs (KV caches, embedding tables) directly in device
memory. The integer part is exactly the 64-bit SplitMix64 sequence (int64
arithmetic wraps; right shifts are masked to be logical). The fp64 transcendentals
may differ from numpy's in the last bit, so consumers that need the values on the
host copy the generated tensor back rather than regenerating it.
"""
from __future__ import annotations

import torch

_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def _s64(x: int) -> int:
    x &= 0xFFFFFFFFFFFFFFFF
    return x - (1 << 64) if x >= (1 << 63) else x


def _lsr(z: torch.Tensor, k: int) -> torch.Tensor:
    return (z >> k) & ((1 << (64 - k)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _s64(_M1)
    z = (z ^ _lsr(z, 27)) * _s64(_M2)
    return z ^ _lsr(z, 31)


def normal(seed: int, n: int, std: float = 1.0, mean: float = 0.0, device="cuda",
           chunk: int = 1 << 26) -> torch.Tensor:
    """n samples of N(mean, std^2) as float32, identical in construction to synth.rng.normal."""
    n_pairs = (n + 1) // 2
    out = torch.empty(2 * n_pairs, dtype=torch.float32, device=device)
    for s in range(0, n_pairs, chunk):
        m = min(chunk, n_pairs - s)
        idx = torch.arange(2 * s, 2 * (s + m), dtype=torch.int64, device=device)
        z = _s64(seed) + (idx + 1) * _s64(_GAMMA)
        r = _lsr(_mix(z), 11).to(torch.float64)
        u = (r + 0.5) * (1.0 / 9007199254740992.0)
        u1, u2 = u[0::2], u[1::2]
        rad = torch.sqrt(-2.0 * torch.log(u1))
        t = 2.0 * torch.pi * u2
        v = torch.empty(2 * m, dtype=torch.float64, device=device)
        v[0::2] = rad * torch.cos(t)
        v[1::2] = rad * torch.sin(t)
        out[2 * s: 2 * (s + m)] = (v * std + mean).to(torch.float32)
    return out[:n]
