"""Counter-based normal samples: SplitMix64 -> 53-bit uniforms -> Box-Muller.

SplitMix64 is the generator of Steele, Lea and Flood, "Fast splittable
pseudorandom number generators" (OOPSLA 2014): output i of a stream with seed
s is mix(s + (i + 1) * 0x9E3779B97F4A7C15) with the 64-bit finaliser below.
Box-Muller (1958) turns two uniforms (u1, u2) into
sqrt(-2 ln u1) * cos(2 pi u2) and sqrt(-2 ln u1) * sin(2 pi u2).

bf16 values are produced by rounding fp32 to nearest-even on the upper 16
bits; the rounded values are exactly representable in fp32/fp64, which is
what the oracle consumes.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(x: int) -> int:
    """One finalised SplitMix64 step of a scalar state (used to derive stream seeds)."""
    with np.errstate(over="ignore"):
        z = np.uint64((int(x) + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF)
        return int(_mix(np.array([z], dtype=np.uint64))[0])


def stream_seed(workload: int, layer: int, tensor_id: int) -> int:
    """Seed of one tensor's stream: splitmix64(0xC0DE0000 ^ workload<<24 ^ layer<<16 ^ tensor)."""
    return splitmix64(0xC0DE0000 ^ (workload << 24) ^ (layer << 16) ^ tensor_id)


def _uniform_pairs(seed: int, start_pair: int, n_pairs: int):
    with np.errstate(over="ignore"):
        idx = np.arange(2 * start_pair, 2 * (start_pair + n_pairs), dtype=np.uint64)
        z = np.uint64(seed) + (idx + np.uint64(1)) * _GAMMA
        r = _mix(z) >> np.uint64(11)  # 53 random bits
    u = (r.astype(np.float64) + 0.5) * (1.0 / 9007199254740992.0)  # (0, 1), never 0
    return u[0::2], u[1::2]


def _normal_chunk(seed: int, start_pair: int, n_pairs: int) -> np.ndarray:
    u1, u2 = _uniform_pairs(seed, start_pair, n_pairs)
    r = np.sqrt(-2.0 * np.log(u1))
    t = 2.0 * np.pi * u2
    out = np.empty(2 * n_pairs, dtype=np.float64)
    out[0::2] = r * np.cos(t)
    out[1::2] = r * np.sin(t)
    return out


_CHUNK_PAIRS = 1 << 20


def normal(seed: int, n: int, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """n samples of N(mean, std^2) as float32 (the fp64 Box-Muller value rounded once)."""
    n_pairs = (n + 1) // 2
    out = np.empty(2 * n_pairs, dtype=np.float32)
    starts = list(range(0, n_pairs, _CHUNK_PAIRS))

    def work(s):
        m = min(_CHUNK_PAIRS, n_pairs - s)
        v = _normal_chunk(seed, s, m)
        out[2 * s: 2 * (s + m)] = (v * std + mean).astype(np.float32)

    if len(starts) <= 1:
        for s in starts:
            work(s)
    else:
        workers = min(len(starts), max(1, min(16, os.cpu_count() or 1)))
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(work, starts))
    return out[:n]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); return the 16-bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to the exactly equal fp32 values."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 value, returned as fp32."""
    return bits_to_f32(bf16_bits(x))


def normal_bf16(seed: int, n: int, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """N(mean, std^2) samples rounded to bf16; returned as uint16 bit patterns."""
    return bf16_bits(normal(seed, n, std, mean))
