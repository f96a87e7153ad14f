"""IsoQuant's dynamic codebook, float64: online channel statistics, KL-optimal boundaries and a
twice-as-large codebook for outlier channels.

IsoQuant page, section 4.2 (quantization error control): the codebook is adjusted dynamically
by (1) gathering each channel's value distribution online, (2) optimising the quantization
boundaries by KL divergence, and (3) giving outlier channels a codebook twice the size.  The
page states no formula for any step; the readings taken:

* statistics: per rotated channel j, the second moment m_j = mean z_j^2 of the rotated unit
  directions z = R(P u), u = y / (rho + eps) (the values the Lloyd-Max quantizer sees), over
  a calibration slice, sink positions left out;
* KL-optimal boundaries: the codebook of channel j is the N(0, 1) Lloyd-Max codebook scaled
  by s_j = sqrt(m_j), and its boundaries the midpoints of the scaled levels.  Among zero-mean
  Gaussians N(0, s^2), the one closest to the channel's distribution P in KL divergence
  minimises E_P[-log N(z; 0, s^2)] = log(s sqrt(2 pi)) + m_j / (2 s^2), i.e. s^2 = m_j;
* outlier channels: the D/16 channels with the largest s_j (equal scales in channel order)
  use the 2^(b+1)-level N(0, 1) Lloyd-Max codebook, scaled the same way: one more bit.

Storage: the codes plane keeps b bits per channel (the low b bits of a wide channel's
b+1-bit code); a separate ``extra`` plane [R, T, H, D/128] u8 holds, LSB first, the top bit
of each wide channel in increasing channel order.
"""
from __future__ import annotations

import numpy as np

from . import lloyd as _lloyd
from . import quant as _quant


def n_wide(d: int) -> int:
    return d // 16


def dynamic_codebook(moments: np.ndarray, bits: int):
    """(scale [D], wide bool [D], codebook [2^b], codebook_wide [2^(b+1)]) from the moments."""
    m = np.asarray(moments, dtype=np.float64)
    d = m.shape[0]
    scale = np.sqrt(m)
    order = sorted(range(d), key=lambda j: (-scale[j], j))
    wide = np.zeros(d, dtype=bool)
    wide[order[:n_wide(d)]] = True
    cb = _lloyd.fit_gaussian(bits, 1.0)
    cb_wide = _lloyd.fit_gaussian(bits + 1, 1.0)
    return scale, wide, cb, cb_wide


def dyn_codes(z: np.ndarray, scale, wide, cb, cb_wide, bits: int):
    """Codes of rotated values z [..., D]: q (b-bit part, uint8) and top (the top bit of the
    b+1-bit code of wide channels, 0 elsewhere).  Channel j: t = z_j / scale_j, code =
    #{k : t > tau_k} against the midpoints of its own codebook (a value on a threshold takes
    the lower code)."""
    z = np.asarray(z, dtype=np.float64)
    t = z / np.asarray(scale, dtype=np.float64)
    q_n = _quant.lloyd_codes(t, cb)
    q_w = _quant.lloyd_codes(t, cb_wide)
    wide = np.asarray(wide, dtype=bool)
    full = np.where(wide, q_w, q_n).astype(np.int64)
    q = (full & ((1 << bits) - 1)).astype(np.uint8)
    top = np.where(wide, full >> bits, 0).astype(np.uint8)
    return q, top, t


def dyn_dequant(q: np.ndarray, top: np.ndarray, scale, wide, cb, cb_wide, bits: int) -> np.ndarray:
    """Levels: scale_j * cb[q] on ordinary channels, scale_j * cb_wide[q + 2^b top] on wide ones."""
    q = np.asarray(q, dtype=np.int64)
    top = np.asarray(top, dtype=np.int64)
    wide = np.asarray(wide, dtype=bool)
    lev = np.where(wide, np.asarray(cb_wide)[q + (top << bits)], np.asarray(cb)[np.minimum(q, len(cb) - 1)])
    return lev * np.asarray(scale, dtype=np.float64)


def pack_extra(top: np.ndarray, wide) -> np.ndarray:
    """[..., D] top bits -> [..., D/128] bytes: bit k (LSB first) = top bit of the k-th wide channel."""
    top = np.asarray(top, dtype=np.uint8)
    idx = np.nonzero(np.asarray(wide, dtype=bool))[0]
    bits = top[..., idx]  # [..., D/16]
    return np.packbits(bits, axis=-1, bitorder="little")


def unpack_extra(extra: np.ndarray, wide) -> np.ndarray:
    extra = np.asarray(extra, dtype=np.uint8)
    wide = np.asarray(wide, dtype=bool)
    d = wide.shape[0]
    idx = np.nonzero(wide)[0]
    bits = np.unpackbits(extra, axis=-1, bitorder="little")[..., :len(idx)]
    top = np.zeros(extra.shape[:-1] + (d,), dtype=np.uint8)
    top[..., idx] = bits
    return top
