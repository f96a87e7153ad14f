"""The whole encode / decode pipeline, float64, step by step in the method's order.

Encode of one token-head vector x at position p = pos_offset + t:

1. RoPE (keys, when enabled) -- EliteKV page section 2.1, RoPE-KV page section 1.
2. Attention sinks -- RotateKV page (attention-sink-aware quantization protects
   sink tokens at higher precision).  Reading: the first ``n_sink`` positions are
   stored as fp16 of the post-RoPE vector, unrotated; their code, scale, zero and
   norm slots are written as zero and the remaining steps are skipped.
3. Norm separation (Lloyd-Max path only) -- IsoQuant page section 3.1 step 1:
   rho = |y|, u = y / (rho + eps), eps = 1e-6.
4. Channel permutation (optional) -- RotateKV page, outlier-aware rotation by
   channel reordering.  Reading: a fixed gather u'[j] = u[perm[j]].
5. Rotation -- FWHT (RotateKV page) or per-4-D-block SO(4) (IsoQuant page
   sections 2.2 and 3.2); see ``rotations``.
6. Quantization -- per-group min-max or Lloyd-Max; see ``quant``.
7. Bit-packing -- see ``pack``.

Decode is the exact inverse (IsoQuant page section 3.1 step 3: inverse rotation,
then restore the norm): unpack, dequantize, inverse rotation, inverse
permutation out[perm[j]] = v[j], multiply by the stored rho; sink positions
return their fp16 values.  There is no inverse RoPE: the cache holds post-RoPE
keys (EliteKV page, section 7.1 core implementation: the attention forward
applies RoPE to k before the cache update).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np

from . import dynamic as _dyn
from . import pack as _pack
from . import quant as _quant
from . import rotations as _rot
from .rope import rope as _rope


@dataclass
class CodecParams:
    bits: int
    group_size: int
    quant: str = "minmax"  # "minmax" | "lloyd"
    rot: str = "fwht"  # "fwht" | "so4" | "none" | "dense" | "rotor"
    rope: bool = False
    rope_base: float = 10000.0
    pos_offset: int = 0
    n_sink: int = 0
    perm: Optional[np.ndarray] = None  # [D] gather map
    quat: Optional[np.ndarray] = None  # [D/4][2][4] (qL, qR), (w, x, y, z)
    codebook: Optional[np.ndarray] = None  # [2^bits] ascending (Lloyd-Max)
    eps: float = 1e-6
    # dynamic codebook (Lloyd-Max only; see ``dynamic``): per rotated channel scale, the wide
    # channels and the 2^(bits+1)-level codebook they use; ``codebook`` is then the N(0,1) one
    chan_scale: Optional[np.ndarray] = None
    chan_wide: Optional[np.ndarray] = None
    codebook_wide: Optional[np.ndarray] = None
    # baseline rotations (see ``rotations``): "dense" z = M u with M = rot_matrix [D, D];
    # "rotor" 3-D rotors rotor_quat [D // 3][4] and the tail angle rotor_tail
    rot_matrix: Optional[np.ndarray] = None
    rotor_quat: Optional[np.ndarray] = None
    rotor_tail: float = 0.0


def widen(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of the stored input to float64 (bf16 arrives as uint16 bits)."""
    if dtype == "bf16":
        return (np.asarray(raw, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(raw).astype(np.float64)


def _rotate(u: np.ndarray, p: CodecParams) -> np.ndarray:
    if p.rot == "fwht":
        return _rot.fwht(u)
    if p.rot == "so4":
        return _rot.so4_rotate(u, p.quat)
    if p.rot == "none":
        return np.array(u, dtype=np.float64)
    if p.rot == "dense":
        return _rot.dense_rotate(u, p.rot_matrix)
    if p.rot == "rotor":
        return _rot.rotor_rotate(u, p.rotor_quat, p.rotor_tail)
    raise ValueError(p.rot)


def _unrotate(z: np.ndarray, p: CodecParams) -> np.ndarray:
    if p.rot == "fwht":
        return _rot.fwht(z)  # H / sqrt(d) is its own inverse
    if p.rot == "so4":
        return _rot.so4_inverse(z, p.quat)
    if p.rot == "none":
        return np.array(z, dtype=np.float64)
    if p.rot == "dense":
        return _rot.dense_inverse(z, p.rot_matrix)
    if p.rot == "rotor":
        return _rot.rotor_inverse(z, p.rotor_quat, p.rotor_tail)
    raise ValueError(p.rot)


def encode(x: np.ndarray, p: CodecParams) -> Dict[str, np.ndarray]:
    """Encode ``x`` ([R, T, H, D], float64).

    Returns the stored planes -- ``codes`` u8 [R,T,H,D*b/8]; ``scale``/``zero`` f16
    [R,T,H,D/G] (min-max); ``norm`` f32 [R,T,H] (Lloyd-Max); ``sink`` f16
    [R,n_sink,H,D] with ``sink_written`` bool [n_sink] -- and, for the tests, the
    unpacked codes ``q``, the rotated values ``z``, the pre-rounding values ``t``
    (min-max: (z-zero)/scale; Lloyd-Max: z) and the mask ``quantized`` [T] of non-sink tokens.
    """
    x = np.asarray(x, dtype=np.float64)
    r, t, h, d = x.shape
    b, g = p.bits, p.group_size
    pos = p.pos_offset + np.arange(t, dtype=np.int64)
    y = _rope(x, pos, p.rope_base) if p.rope else x.copy()

    out: Dict[str, np.ndarray] = {
        "codes": np.zeros((r, t, h, d * b // 8), dtype=np.uint8),
        "sink": np.zeros((r, p.n_sink, h, d), dtype=np.float16),
        "sink_written": np.zeros(p.n_sink, dtype=bool),
        "q": np.zeros((r, t, h, d), dtype=np.uint8),
        "t": np.zeros((r, t, h, d), dtype=np.float64),
        "z": np.zeros((r, t, h, d), dtype=np.float64),
    }
    if p.quant == "minmax":
        out["scale"] = np.zeros((r, t, h, d // g), dtype=np.float16)
        out["zero"] = np.zeros((r, t, h, d // g), dtype=np.float16)
    else:
        out["norm"] = np.zeros((r, t, h), dtype=np.float32)

    is_sink = pos < p.n_sink
    out["quantized"] = ~is_sink
    for ti in np.nonzero(is_sink)[0]:
        out["sink"][:, pos[ti]] = y[:, ti].astype(np.float16)
        out["sink_written"][pos[ti]] = True

    keep = ~is_sink
    z, rho = _front(y[:, keep], p)
    if p.quant == "lloyd":
        out["norm"][:, keep] = rho.astype(np.float32)
    if p.quant == "minmax":
        scale, zero = _quant.minmax_params(z, b, g)
        q, tt = _quant.minmax_codes(z, scale, zero, b, g)
        out["scale"][:, keep] = scale
        out["zero"][:, keep] = zero
    elif p.chan_scale is not None:
        q, top, tt = _dyn.dyn_codes(z, p.chan_scale, p.chan_wide, p.codebook, p.codebook_wide, b)
        out["extra"] = np.zeros((r, t, h, d // 128), dtype=np.uint8)
        out["extra"][:, keep] = _dyn.pack_extra(top, p.chan_wide)
        out["top"] = np.zeros((r, t, h, d), dtype=np.uint8)
        out["top"][:, keep] = top
    else:
        q = _quant.lloyd_codes(z, p.codebook)
        tt = z
    out["q"][:, keep] = q
    out["t"][:, keep] = tt
    out["z"][:, keep] = z
    out["codes"][:, keep] = _pack.pack(q, b)
    return out


def _front(y: np.ndarray, p: CodecParams):
    """Norm separation (Lloyd-Max), permutation and rotation of post-RoPE vectors y:
    returns (z, rho) with rho None for min-max."""
    u = y
    rho = None
    if p.quant == "lloyd":
        rho = np.sqrt(np.sum(u * u, axis=-1))
        u = u / (rho + p.eps)[..., None]
    if p.perm is not None:
        u = u[..., np.asarray(p.perm, dtype=np.int64)]
    return _rotate(u, p), rho


def rotated_moments(x: np.ndarray, p: CodecParams) -> np.ndarray:
    """Per rotated channel mean z_j^2 over the non-sink vectors of a calibration slice x: the
    online statistics of the dynamic codebook (IsoQuant page, section 4.2, step 1)."""
    x = np.asarray(x, dtype=np.float64)
    r, t, h, d = x.shape
    pos = p.pos_offset + np.arange(t, dtype=np.int64)
    y = _rope(x, pos, p.rope_base) if p.rope else x
    keep = pos >= p.n_sink
    z, _ = _front(y[:, keep], p)
    n = z.shape[0] * z.shape[1] * z.shape[2]
    return (z * z).reshape(-1, d).sum(axis=0) / n if n else np.zeros(d)


def decode(planes: Dict[str, np.ndarray], p: CodecParams, shape) -> np.ndarray:
    """Decode stored planes back to [R, T, H, D] float64 (post-RoPE, original channel order)."""
    r, t, h, d = shape
    b, g = p.bits, p.group_size
    q = _pack.unpack(planes["codes"], b, d)
    if p.quant == "minmax":
        yhat = _quant.minmax_dequant(q, planes["scale"], planes["zero"], g)
    elif p.chan_scale is not None:
        top = _dyn.unpack_extra(planes["extra"], p.chan_wide)
        yhat = _dyn.dyn_dequant(q, top, p.chan_scale, p.chan_wide, p.codebook, p.codebook_wide, b)
    else:
        yhat = _quant.lloyd_dequant(q, p.codebook)
    w = _unrotate(yhat, p)
    if p.perm is not None:
        v = np.empty_like(w)
        v[..., np.asarray(p.perm, dtype=np.int64)] = w
    else:
        v = w
    if p.quant == "lloyd":
        v = v * planes["norm"].astype(np.float64)[..., None]
    pos = p.pos_offset + np.arange(t, dtype=np.int64)
    for ti in np.nonzero(pos < p.n_sink)[0]:
        v[:, ti] = planes["sink"][:, pos[ti]].astype(np.float64)
    return v


PLANE_NAMES = ("codes", "scale", "zero", "norm", "sink", "extra")


def append(cache: Dict[str, np.ndarray], x: np.ndarray, positions: np.ndarray, p: CodecParams) -> Dict[str, np.ndarray]:
    """Decode-step append: one new token per row written into an encoded cache.

    EliteKV page, section 7.1 (core implementation): during single-token decoding the
    attention forward applies RoPE to the new key and the cache's update appends the
    token at the sequence's current length.  Reading: row r's vector ``x[r]`` ([R, H, D],
    float64) is the token at position ``positions[r]``, encoded exactly as ``encode``
    encodes a token at that position (same RoPE angle; a sink when the position is below
    ``n_sink``), and stored in slot ``positions[r] - pos_offset`` of a cache whose planes
    hold ``T`` slots per row (slot s = position pos_offset + s).  A row whose position has
    no slot is left unchanged.  Returns updated copies of the cache planes.
    """
    x = np.asarray(x, dtype=np.float64)
    out = {k: np.array(v, copy=True) for k, v in cache.items() if k in PLANE_NAMES}
    rows, slots = out["codes"].shape[:2]
    for r in range(rows):
        pos = int(positions[r])
        slot = pos - p.pos_offset
        if not 0 <= slot < slots:
            continue
        one = encode(x[r][None, None], replace(p, pos_offset=pos))
        for name in ("codes", "scale", "zero", "norm", "extra"):
            if name in out and name in one:
                out[name][r, slot] = one[name][0, 0]
        if pos < p.n_sink:
            out["sink"][r, pos] = one["sink"][0, pos]
    return out

