"""Parity rules between the GPU codec and the CPU oracle.

Where several results are correct, what is unique is compared exactly and the rest is
checked for validity:

* codes: bit-exact, except where the oracle's pre-rounding value lies within 1e-4 of a
  decision boundary (min-max: t within 1e-4 of k + 1/2, i.e. within 1e-4*scale of the
  boundary; Lloyd-Max: within 1e-4*(c_{k+1} - c_k) of a threshold); such mismatches must
  also be at most 1e-5 of all codes;
* fp16 scale/zero: bit-exact, except where the oracle's pre-rounding value lies within a
  window of an fp16 value (the rounding point of a directed rounding): the GPU's value must
  then be the directed rounding of some value in that window.  The window is
  max(1e-5 |v|, 1e-6 |z|_2), |z|_2 the vector's norm: the float32 error of a rotated
  coefficient scales with the vector's norm (7 butterfly stages and the RoPE pair rotation
  give at most about 4.4e-7 |z|_2), not with the coefficient, which can be small by
  cancellation.  The codes of such a group are then judged against t recomputed with the
  GPU's stored scale and zero;
* norm (fp32 rho): relative 1e-6;
* sinks (fp16): bit-exact, except one ulp where the float64 value lies within 1e-6
  relative of a midpoint between fp16 values;
* decode: both decoders get the same (GPU-produced) planes; fp32 outputs agree within
  1e-3 absolute, 16-bit outputs within 1e-3 plus half an ulp of the output type.
"""
from __future__ import annotations

import numpy as np

from oracle import codec
from oracle import pack as opack
from oracle import quant as oquant

CODE_TIE = 1e-4
CODE_MISMATCH_MAX = 1e-5
F16_REL = 1e-5
F16_NORM_ABS = 1e-6  # times the vector norm: absolute part of the scale/zero rounding window
SINK_REL = 1e-6
DECODE_ABS = 1e-3
NORM_REL = 1e-6


def params_for(case, perm=None, quat=None, codebook=None) -> codec.CodecParams:
    return codec.CodecParams(bits=case.bits, group_size=case.group_size, quant=case.quant, rot=case.rot,
                             rope=case.rope, rope_base=case.rope_base, pos_offset=case.pos_offset,
                             n_sink=case.n_sink, perm=perm if case.use_perm else None, quat=quat,
                             codebook=codebook)


def _f16_ulp_apart(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|a - b| == 1 ulp for float16 arrays (same sign side or across zero)."""
    ai = a.view(np.uint16).astype(np.int32)
    bi = b.view(np.uint16).astype(np.int32)
    # map to a monotone integer line
    ai = np.where(ai & 0x8000, -(ai & 0x7FFF), ai)
    bi = np.where(bi & 0x8000, -(bi & 0x7FFF), bi)
    return np.abs(ai - bi) == 1


def _near_f16_midpoint(x: np.ndarray, rel: float, mag: np.ndarray) -> np.ndarray:
    """x lies within rel*mag of a midpoint between neighbouring float16 values.

    ``mag`` is the magnitude the float32 computation of x is accurate relative to: for a
    RoPE output that is the norm of the rotated channel pair, not |x| itself (the two
    products of the rotation can cancel)."""
    x = np.asarray(x, dtype=np.float64)
    lo = x.astype(np.float16)
    lo64 = lo.astype(np.float64)
    nb = np.where(lo64 <= x, np.nextafter(lo, np.float16(np.inf)), np.nextafter(lo, np.float16(-np.inf)))
    mid = 0.5 * (lo64 + nb.astype(np.float64))
    return np.abs(x - mid) <= rel * np.maximum(np.maximum(np.abs(x), mag), 6e-8)


class ParityReport(dict):
    pass


def compare_encode(gpu: dict, ora: dict, p: codec.CodecParams, shape, label: str = "",
                   fraction: bool = True) -> ParityReport:
    """Compare numpy copies of GPU planes with the oracle's encode output (same inputs).

    ``fraction=False`` is for hand-built degenerate inputs that sit on decision boundaries
    by construction (exact zeros against a threshold at 0): mismatches must still all be
    ties, but their count is not bounded and they stay out of the session total."""
    r, t, h, d = shape
    b, g = p.bits, p.group_size
    rep = ParityReport(label=label)
    keep = ora["quantized"]  # [T]
    q_gpu = opack.unpack(gpu["codes"], b, d)
    q_ora = ora["q"]
    n_codes = int(keep.sum()) * r * h * d
    rep["n_codes"] = n_codes

    # sink vectors: zero codes / scale / zero / norm, fp16 values bit-exact up to midpoint ties
    if p.n_sink > 0 and (~keep).any():
        sk = ~keep
        assert np.all(gpu["codes"][:, sk] == 0), f"{label}: sink code slots not zero"
        if p.quant == "minmax":
            assert np.all(gpu["scale"][:, sk].view(np.uint16) == 0), f"{label}: sink scale slots not zero"
            assert np.all(gpu["zero"][:, sk].view(np.uint16) == 0), f"{label}: sink zero slots not zero"
        else:
            assert np.all(gpu["norm"][:, sk] == 0), f"{label}: sink norm slots not zero"
            if p.chan_scale is not None:
                assert np.all(gpu["extra"][:, sk] == 0), f"{label}: sink extra slots not zero"
        written = ora["sink_written"]
        gs = gpu["sink"][:, written]
        os_ = ora["sink"][:, written]
        diff = gs.view(np.uint16) != os_.view(np.uint16)
        if diff.any():
            # the float64 post-RoPE value behind the oracle's rounding is needed for the tie
            # rule; it is recomputed by the caller and passed as ora["sink_f64"]
            exact = ora.get("sink_f64")
            assert exact is not None, f"{label}: sink mismatch and no float64 sink values to judge ties"
            ex = exact[0][:, written]
            mag = exact[1][:, written]
            ok = _f16_ulp_apart(gs[diff], os_[diff]) & _near_f16_midpoint(ex[diff], SINK_REL, mag[diff])
            assert ok.all(), f"{label}: {int((~ok).sum())} sink values differ beyond a midpoint tie"
        rep["sink_mismatch"] = int(diff.sum())

    qg = q_gpu[:, keep]
    qo = q_ora[:, keep]
    tt = ora["t"][:, keep]
    zz = ora["z"][:, keep]
    if p.quant == "minmax":
        sg = gpu["scale"][:, keep]
        zg = gpu["zero"][:, keep]
        so = ora["scale"][:, keep]
        zo = ora["zero"][:, keep]
        zgrp = zz.reshape(zz.shape[:-1] + (d // g, g))
        mn = zgrp.min(-1)
        mx = zgrp.max(-1)
        # the rounding window of each group's min and max (see the module docstring)
        vnorm = np.sqrt(np.sum(zz * zz, axis=-1))[..., None]
        win_mn = np.maximum(F16_REL * np.abs(mn), F16_NORM_ABS * vnorm)
        win_mx = np.maximum(F16_REL * np.abs(mx), F16_NORM_ABS * vnorm)
        dz = zg.view(np.uint16) != zo.view(np.uint16)
        if dz.any():
            # the GPU's zero is the round-down of a value within the window of the min
            lo = oquant.fp16_round_down(mn - win_mn).astype(np.float64)
            hi = oquant.fp16_round_down(mn + win_mn).astype(np.float64)
            zgd = zg.astype(np.float64)
            ok = ((zgd >= lo) & (zgd <= hi))[dz]
            assert ok.all(), (f"{label}: {int((~ok).sum())} zero values differ beyond a rounding tie: "
                              f"gpu {zg[dz][~ok][:4]} oracle {zo[dz][~ok][:4]} min {mn[dz][~ok][:4]}")
        # where the stored zero legitimately differs, the scale follows from the GPU's zero
        levels = 2 ** b - 1
        pre_s = (mx - zg.astype(np.float64)) / levels
        so_ref = np.where(dz, oquant.fp16_round_up(pre_s), so)
        ds = sg.view(np.uint16) != so_ref.view(np.uint16)
        if ds.any():
            lo = oquant.fp16_round_up(np.maximum(pre_s - win_mx / levels, 0.0)).astype(np.float64)
            hi = oquant.fp16_round_up(pre_s + win_mx / levels).astype(np.float64)
            sgd = sg.astype(np.float64)
            ok = ((sgd >= lo) & (sgd <= hi))[ds]
            assert ok.all(), (f"{label}: {int((~ok).sum())} scale values differ beyond a rounding tie: "
                              f"gpu {sg[ds][~ok][:4]} oracle {so_ref[ds][~ok][:4]} pre {pre_s[ds][~ok][:4]}")
        rep["scale_mismatch"] = int(ds.sum())
        rep["zero_mismatch"] = int(dz.sum())
        # judge codes against t computed with the GPU's stored scale/zero
        s64 = sg.astype(np.float64)[..., None]
        z64 = zg.astype(np.float64)[..., None]
        with np.errstate(divide="ignore", invalid="ignore"):
            tg = np.where(s64 > 0, (zgrp - z64) / np.where(s64 > 0, s64, 1), 0.0).reshape(zz.shape)
        q_ref = np.clip(np.rint(tg), 0, 2 ** b - 1).astype(np.uint8)
        mism = qg != q_ref
        frac = np.abs(tg - np.floor(tg) - 0.5)
        tie = frac < CODE_TIE
    elif p.chan_scale is not None:
        # dynamic codebook: compare the full code (b bits + the wide channels' top bit) against
        # the thresholds of each channel's own codebook, in units of its level gaps
        from oracle import dynamic as odyn
        wide = np.asarray(p.chan_wide, dtype=bool)
        top_g = odyn.unpack_extra(gpu["extra"], wide)[:, keep]
        qg = qg.astype(np.int64) + (top_g.astype(np.int64) << b)
        q_ref = qo.astype(np.int64) + (ora["top"][:, keep].astype(np.int64) << b)
        mism = qg != q_ref
        tie = np.zeros(mism.shape, dtype=bool)
        for book, sel in ((np.asarray(p.codebook, np.float64), ~wide), (np.asarray(p.codebook_wide, np.float64), wide)):
            tau = 0.5 * (book[:-1] + book[1:])
            dist = np.abs(tt[..., sel, None] - tau) / np.diff(book)
            tie[..., sel] = (dist < CODE_TIE).any(-1)
        ng = gpu["norm"][:, keep].astype(np.float64)
        no = ora["norm"][:, keep].astype(np.float64)
        rel = np.abs(ng - no) / np.maximum(np.abs(no), 1e-30)
        assert np.all((rel <= NORM_REL) | (np.abs(ng - no) < 1e-30)), f"{label}: norm differs, max rel {rel.max():.3g}"
    else:
        q_ref = qo
        mism = qg != q_ref
        cb = np.asarray(p.codebook, dtype=np.float64)
        tau = 0.5 * (cb[:-1] + cb[1:])
        gap = np.diff(cb)
        dist = np.abs(zz[..., None] - tau) / gap  # distance to each threshold in gap units
        tie = (dist < CODE_TIE).any(-1)
        ng = gpu["norm"][:, keep].astype(np.float64)
        no = ora["norm"][:, keep].astype(np.float64)
        rel = np.abs(ng - no) / np.maximum(np.abs(no), 1e-30)
        assert np.all((rel <= NORM_REL) | (np.abs(ng - no) < 1e-30)), f"{label}: norm differs, max rel {rel.max():.3g}"
    bad = mism & ~tie
    assert not bad.any(), (f"{label}: {int(bad.sum())} codes differ away from a rounding tie "
                           f"(first at {np.argwhere(bad)[0].tolist()})")
    n_mism = int(mism.sum())
    rep["code_mismatch"] = n_mism
    if not fraction:
        return rep
    SESSION["codes"] += n_codes
    SESSION["tie_mismatches"] += n_mism
    # per comparison: the fraction bound, rounded up to one tie for small comparisons
    assert n_mism <= max(1, int(CODE_MISMATCH_MAX * n_codes)), \
        f"{label}: {n_mism} tie mismatches exceed {CODE_MISMATCH_MAX} of {n_codes} codes"
    return rep


def compare_decode(y_gpu: np.ndarray, y_ora: np.ndarray, out_dtype: str, label: str = "") -> float:
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y_ora)
    if out_dtype == "f32":
        tol = DECODE_ABS
    elif out_dtype == "bf16":
        tol = DECODE_ABS + np.abs(y_ora) * 2.0 ** -8
    else:
        tol = DECODE_ABS + np.abs(y_ora) * 2.0 ** -11
    bad = err > tol
    assert not bad.any(), f"{label}: decode differs by up to {err.max():.3g} ({int(bad.sum())} elements)"
    return float(err.max()) if err.size else 0.0


def sink_f64(x64: np.ndarray, p: codec.CodecParams):
    """float64 post-RoPE values at the sink slots and, per element, the norm of its RoPE
    channel pair (for the sink tie rule)."""
    from oracle.rope import rope
    r, t, h, d = x64.shape
    pos = p.pos_offset + np.arange(t)
    y = rope(x64, pos, p.rope_base) if p.rope else x64
    pair = np.sqrt(x64[..., 0::2] ** 2 + x64[..., 1::2] ** 2) if p.rope else np.abs(x64)
    if p.rope:
        pair = np.repeat(pair, 2, axis=-1)
    out = np.zeros((r, p.n_sink, h, d))
    mag = np.zeros((r, p.n_sink, h, d))
    for ti in np.nonzero(pos < p.n_sink)[0]:
        out[:, pos[ti]] = y[:, ti]
        mag[:, pos[ti]] = pair[:, ti]
    return out, mag


# Tie mismatches are counted over every comparison of a test session: the 1e-5 bound is
# on the fraction of all codes compared (a single tie in a few thousand codes is not a
# failure by itself).
SESSION = {"codes": 0, "tie_mismatches": 0}
