"""Bit-packing of b-bit codes, plain Python/numpy.

The pages do not fix a layout.  Reading taken: the codes of one vector form an
LSB-first bit stream -- bit m of code j is stream bit b*j + m, and byte n holds
stream bits 8n .. 8n+7 with the lowest stream bit in the least significant bit
of the byte.  A vector of d codes occupies d*b/8 bytes.
"""
from __future__ import annotations

import numpy as np


def pack(q: np.ndarray, bits: int) -> np.ndarray:
    """[..., D] codes (< 2^bits) -> [..., D*bits/8] uint8."""
    q = np.asarray(q, dtype=np.uint8)
    d = q.shape[-1]
    assert (d * bits) % 8 == 0
    flat = q.reshape(-1, d)
    stream = np.zeros((flat.shape[0], d * bits), dtype=np.uint8)
    for m in range(bits):
        stream[:, m::bits] = (flat >> m) & 1
    out = np.zeros((flat.shape[0], d * bits // 8), dtype=np.uint8)
    for bit in range(8):
        out |= (stream[:, bit::8] << bit).astype(np.uint8)
    return out.reshape(q.shape[:-1] + (d * bits // 8,))


def unpack(codes: np.ndarray, bits: int, d: int) -> np.ndarray:
    """Inverse of :func:`pack`."""
    codes = np.asarray(codes, dtype=np.uint8)
    flat = codes.reshape(-1, codes.shape[-1])
    stream = np.zeros((flat.shape[0], flat.shape[1] * 8), dtype=np.uint8)
    for bit in range(8):
        stream[:, bit::8] = (flat >> bit) & 1
    q = np.zeros((flat.shape[0], d), dtype=np.uint8)
    for m in range(bits):
        q |= (stream[:, m::bits][:, :d] << m).astype(np.uint8)
    return q.reshape(codes.shape[:-1] + (d,))
