"""Seeded synthetic inputs: counter-based SplitMix64 feeding Box-Muller.

This module holds no arithmetic of the quantized GEMV. It only draws the
Gaussian tensors that both the HIP path and the CPU oracle consume, so the
same (seed, element index) always yields the same fp32 value on any device.

Generator definitions (published, restated):
  * SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): state advances by the odd constant
    GAMMA = 0x9E3779B97F4A7C15 and each output is the state passed through the
    variant-13 finaliser (xor-shift 30, multiply, xor-shift 27, multiply,
    xor-shift 31).  Draw i of a stream seeded with s is mix(s + (i + 1) * GAMMA),
    which equals the i-th output of the sequential generator, so any element can
    be computed on its own.
  * Box-Muller (Box & Muller 1958): from u1 in (0, 1] and u2 in [0, 1),
    z0 = sqrt(-2 ln u1) cos(2 pi u2) and z1 = sqrt(-2 ln u1) sin(2 pi u2).
    Normal element 2j takes z0 and element 2j+1 takes z1 of the pair built from
    draws 2j (u1) and 2j+1 (u2).  Evaluated in float64, then scaled by sigma and
    cast to float32.

Seeds per tensor: seed = GAMMA * (1 + 64 * workload + tensor_id) + copy, taken
mod 2**64, so every workload, tensor and rotation copy has its own stream.
"""

from __future__ import annotations

import math

import torch

GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1


def _as_i64(v: int) -> int:
    """Two's-complement view of an unsigned 64-bit value (torch has no wrapping uint64 math)."""
    v &= _MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def tensor_seed(workload: int, tensor_id: int, copy: int = 0) -> int:
    return (GAMMA * (1 + 64 * workload + tensor_id) + copy) & _MASK64


def splitmix64_scalar(seed: int, i: int) -> int:
    """Pure-Python draw i of the stream seeded with `seed` (reference for the tensor path)."""
    z = (seed + (i + 1) * GAMMA) & _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    # logical right shift of int64 holding uint64 bits
    return (z >> s) & ((1 << (64 - s)) - 1)


def splitmix64(seed: int, idx: torch.Tensor) -> torch.Tensor:
    """Draws idx of the stream `seed`, as int64 tensors carrying the uint64 bits."""
    z = idx.to(torch.int64) + 1
    z = z * _as_i64(GAMMA) + _as_i64(seed)
    z = (z ^ _lsr(z, 30)) * _as_i64(_M1)
    z = (z ^ _lsr(z, 27)) * _as_i64(_M2)
    return z ^ _lsr(z, 31)


def _u53(z: torch.Tensor) -> torch.Tensor:
    return _lsr(z, 11).to(torch.float64) * (2.0 ** -53)


def gaussian(shape, sigma: float, seed: int, device="cpu", chunk: int = 1 << 24) -> torch.Tensor:
    """float32 tensor of N(0, sigma^2) values, element e drawn from pair e // 2 of the stream."""
    numel = 1
    for s in shape:
        numel *= int(s)
    out = torch.empty(numel, dtype=torch.float32, device=device)
    npairs = (numel + 1) // 2
    for p0 in range(0, npairs, chunk):
        p1 = min(npairs, p0 + chunk)
        pidx = torch.arange(p0, p1, dtype=torch.int64, device=device)
        u1 = 1.0 - _u53(splitmix64(seed, 2 * pidx))  # (0, 1]
        u2 = _u53(splitmix64(seed, 2 * pidx + 1))  # [0, 1)
        rad = torch.sqrt(-2.0 * torch.log(u1))
        ang = (2.0 * math.pi) * u2
        z = torch.stack((rad * torch.cos(ang), rad * torch.sin(ang)), dim=1).reshape(-1)
        e0, e1 = 2 * p0, min(numel, 2 * p1)
        out[e0:e1] = (z[: e1 - e0] * sigma).to(torch.float32)
        del pidx, u1, u2, rad, ang, z
    return out.reshape(tuple(int(s) for s in shape))


def gaussian_outliers(shape, sigma: float, seed: int, frac: float = 0.01, mult: float = 20.0,
                      device="cpu") -> torch.Tensor:
    """Gaussian tensor where a fraction `frac` of elements is replaced by +-mult*sigma.

    Which elements and which sign are drawn from a second stream (seed + 1), so the
    pattern is as reproducible as the values.  Used to give blocks uneven scales.
    """
    g = gaussian(shape, sigma, seed, device=device)
    numel = g.numel()
    idx = torch.arange(numel, dtype=torch.int64, device=device)
    r = _u53(splitmix64((seed + 1) & _MASK64, idx))
    pick = r < frac
    sign = torch.where((_lsr(splitmix64((seed + 2) & _MASK64, idx), 63) & 1) == 1, -1.0, 1.0)
    g = g.reshape(-1)
    g[pick] = (sign[pick] * (mult * sigma)).to(torch.float32)
    return g.reshape(g.shape if len(shape) == 0 else tuple(int(s) for s in shape))


# Tensor ids within a workload: weights take 0..31 in the order the workload lists
# them, activation sets take 32 + rows.
def act_tensor_id(rows: int) -> int:
    return 32 + int(rows)
