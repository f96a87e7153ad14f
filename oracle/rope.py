"""Rotary position embedding (RoPE), float64.

Follows the EliteKV page, section 2.1 (the block-diagonal rotation matrix R_m
whose 2x2 blocks act on adjacent channel pairs (2i, 2i+1), with the sine
below the diagonal) and the RoPE-KV page, section 1 (angle of pair i at
position m is m / 10000^(2i/d)).

Readings taken where the pages disagree:

* frequency: theta_i = base^(-2i/d), i = 0 .. d/2-1 (RoPE-KV page section 1 and
  its section 6.2 inv_freq code; the EliteKV code that multiplies by 10000 is
  not used);
* pairing: interleaved adjacent pairs, as in the EliteKV matrix (its
  ``apply_rope`` listing splits halves while its own comment says even/odd).
"""
from __future__ import annotations

import numpy as np


def thetas(head_dim: int, base: float = 10000.0) -> np.ndarray:
    """theta_i = base^(-2i/d) for i = 0 .. d/2 - 1 (RoPE-KV page, section 1)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / head_dim)


def rope(x: np.ndarray, positions: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """Apply R_p to every vector of ``x`` ([..., T, H, D]) at position ``positions[t]``.

    For pair i: y[2i] = x[2i] cos(p theta_i) - x[2i+1] sin(p theta_i),
                y[2i+1] = x[2i] sin(p theta_i) + x[2i+1] cos(p theta_i)
    (EliteKV page, section 2.1 matrix R_m).  The angle p*theta_i is formed in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    th = thetas(d, base)
    phi = np.asarray(positions, dtype=np.float64)[:, None] * th[None, :]  # [T, D/2]
    c = np.cos(phi)[:, None, :]  # broadcast over heads
    s = np.sin(phi)[:, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y
