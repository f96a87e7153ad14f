"""Scalar quantizers, float64.

Per-group asymmetric min-max (the pages only name "INT8/INT4" and "2-bit" KV
quantization; the RotateKV page quantizes the rotated cache to 2 bits).  The
reading taken for what the pages leave open:

* groups are G contiguous channels of the rotated vector;
* zero = the largest fp16 value <= min of the group (round down);
* scale = the smallest fp16 value >= (max - zero) / (2^b - 1) (round up), so the
  grid zero + k*scale, k = 0 .. 2^b-1, covers [min, max] and every element is
  within scale/2 of its reconstruction;
* codes use the STORED fp16 scale and zero: q = clip(rint((z - zero) / scale), 0, 2^b-1)
  with ties to even; a group whose scale is 0 (max == min == zero) gets q = 0.

Lloyd-Max scalar quantization (IsoQuant page, section 3.1, step 2): with an
ascending codebook c_0 < ... < c_{2^b-1} the decision thresholds are the
midpoints tau_k = (c_k + c_{k+1}) / 2 and q = #{k : z > tau_k} (a value exactly on
a threshold takes the lower code); decoding returns c_q.
"""
from __future__ import annotations

import numpy as np


def fp16_round_down(x: np.ndarray) -> np.ndarray:
    """Largest float16 <= x (x finite and within the float16 range)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        h = x.astype(np.float16)  # nearest
        over = h.astype(np.float64) > x
        h = np.where(over, np.nextafter(h, np.float16(-np.inf)), h)
    return h.astype(np.float16)


def fp16_round_up(x: np.ndarray) -> np.ndarray:
    """Smallest float16 >= x (x finite and within the float16 range)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        h = x.astype(np.float16)  # nearest
        under = h.astype(np.float64) < x
        h = np.where(under, np.nextafter(h, np.float16(np.inf)), h)
    return h.astype(np.float16)


def minmax_params(z: np.ndarray, bits: int, group: int):
    """Per-group (scale, zero) as float16 arrays of shape [..., D/G]."""
    z = np.asarray(z, dtype=np.float64)
    d = z.shape[-1]
    g = z.reshape(z.shape[:-1] + (d // group, group))
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    zero = fp16_round_down(mn)
    scale = fp16_round_up((mx - zero.astype(np.float64)) / (2 ** bits - 1))
    return scale, zero


def minmax_codes(z: np.ndarray, scale: np.ndarray, zero: np.ndarray, bits: int, group: int):
    """Codes with the stored fp16 scale/zero; returns (q uint8 [..., D], t float64 [..., D]).

    ``t`` is the pre-rounding value (z - zero) / scale (0 where scale == 0), used by the
    parity tests to recognise rounding ties.
    """
    z = np.asarray(z, dtype=np.float64)
    d = z.shape[-1]
    zg = z.reshape(z.shape[:-1] + (d // group, group))
    s = scale.astype(np.float64)[..., None]
    zr = zero.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(s > 0, (zg - zr) / np.where(s > 0, s, 1.0), 0.0)
    q = np.clip(np.rint(t), 0, 2 ** bits - 1).astype(np.uint8)
    return q.reshape(z.shape), t.reshape(z.shape)


def minmax_dequant(q: np.ndarray, scale: np.ndarray, zero: np.ndarray, group: int) -> np.ndarray:
    """y = zero + q * scale per group."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    qg = q.reshape(q.shape[:-1] + (d // group, group))
    y = zero.astype(np.float64)[..., None] + qg * scale.astype(np.float64)[..., None]
    return y.reshape(q.shape)


def lloyd_thresholds(codebook: np.ndarray) -> np.ndarray:
    c = np.asarray(codebook, dtype=np.float64)
    return 0.5 * (c[:-1] + c[1:])


def lloyd_codes(u: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """q = #{k : u > tau_k} (strict: a value on a threshold takes the lower code)."""
    tau = lloyd_thresholds(codebook)
    u = np.asarray(u, dtype=np.float64)
    q = np.zeros(u.shape, dtype=np.uint8)
    for t in tau:
        q += (u > t).astype(np.uint8)
    return q


def lloyd_dequant(q: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    return np.asarray(codebook, dtype=np.float64)[np.asarray(q, dtype=np.int64)]
