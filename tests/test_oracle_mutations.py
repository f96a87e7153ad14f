"""Plant a plausible mistake in the oracle (CPU only, via monkeypatch) and require that
at least one pin catches it.  This is what makes the pins evidence: a dropped term, a
wrong sign or index, a transposed operand or a wrong rounding direction anywhere in
the oracle turns at least one check red."""
import numpy as np
import pytest
from scipy.stats import norm

from oracle import codec, lloyd, pack, quant, rope, rotations
from tests import oracle_pins


def _rope_neg_sine(x, positions, base=10000.0):
    x = np.asarray(x, dtype=np.float64)
    th = rope.thetas(x.shape[-1], base)
    phi = np.asarray(positions, dtype=np.float64)[:, None] * th[None, :]
    c, s = np.cos(phi)[:, None, :], np.sin(phi)[:, None, :]
    y = np.empty_like(x)
    y[..., 0::2] = x[..., 0::2] * c + x[..., 1::2] * s
    y[..., 1::2] = -x[..., 0::2] * s + x[..., 1::2] * c
    return y


def _rope_half_split(x, positions, base=10000.0):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    th = rope.thetas(d, base)
    phi = np.asarray(positions, dtype=np.float64)[:, None] * th[None, :]
    c, s = np.cos(phi)[:, None, :], np.sin(phi)[:, None, :]
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def _thetas_wrong_exponent(head_dim, base=10000.0):
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -1.0 * i / head_dim)


def _fwht_unnormalised(u):
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    return (u.reshape(-1, d) @ rotations.hadamard(d).T).reshape(u.shape)


def _quat_mul_sign_slip(a, b):
    w1, x1, y1, z1 = [np.asarray(a, dtype=np.float64)[..., i] for i in range(4)]
    w2, x2, y2, z2 = [np.asarray(b, dtype=np.float64)[..., i] for i in range(4)]
    return np.stack([
        w1 * w2 - x1 * x2 - y1 * y2 - z1 * z2,
        w1 * x2 + x1 * w2 - y1 * z2 + z1 * y2,  # cross term with the wrong sign
        w1 * y2 - x1 * z2 + y1 * w2 + z1 * x2,
        w1 * z2 + x1 * y2 - y1 * x2 + z1 * w2,
    ], axis=-1)


def _so4_swapped(u, quat):
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    q = np.asarray(quat, dtype=np.float64)
    blocks = u.reshape(u.shape[:-1] + (d // 4, 4))
    z = rotations.quat_mul(q[:, 1, :], rotations.quat_mul(blocks, q[:, 0, :]))
    return z.reshape(u.shape)


def _round_nearest(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def _minmax_params_range_from_min(z, bits, group):
    z = np.asarray(z, dtype=np.float64)
    g = z.reshape(z.shape[:-1] + (z.shape[-1] // group, group))
    mn, mx = g.min(-1), g.max(-1)
    zero = quant.fp16_round_down(mn)
    return quant.fp16_round_up((mx - mn) / (2 ** bits - 1)), zero


def _minmax_codes_floor(z, scale, zero, bits, group):
    z = np.asarray(z, dtype=np.float64)
    zg = z.reshape(z.shape[:-1] + (z.shape[-1] // group, group))
    s = scale.astype(np.float64)[..., None]
    t = np.where(s > 0, (zg - zero.astype(np.float64)[..., None]) / np.where(s > 0, s, 1), 0.0)
    q = np.clip(np.floor(t), 0, 2 ** bits - 1).astype(np.uint8)
    return q.reshape(z.shape), t.reshape(z.shape)


def _lloyd_codes_ge(u, codebook):
    tau = quant.lloyd_thresholds(codebook)
    u = np.asarray(u, dtype=np.float64)
    q = np.zeros(u.shape, dtype=np.uint8)
    for t in tau:
        q += (u >= t).astype(np.uint8)
    return q


def _fit_wrong_mean(bits, sigma=1.0, tol=1e-13, max_iter=2000):
    n = 2 ** bits
    c = norm.ppf((np.arange(n) + 0.5) / n)
    for _ in range(max_iter):
        tau = 0.5 * (c[:-1] + c[1:])
        lo = np.concatenate(([-np.inf], tau))
        hi = np.concatenate((tau, [np.inf]))
        c = (norm.pdf(lo) - norm.pdf(hi)) / (norm.cdf(hi) - norm.cdf(lo)) * 0.5 + 0.5 * c  # damped, biased
        c = c * 1.01
    return c * sigma


def _pack_msb_first(q, bits):
    q = np.asarray(q, dtype=np.uint8)
    d = q.shape[-1]
    flat = q.reshape(-1, d)
    stream = np.zeros((flat.shape[0], d * bits), dtype=np.uint8)
    for m in range(bits):
        stream[:, m::bits] = (flat >> m) & 1
    return np.packbits(stream, axis=-1, bitorder="big").reshape(q.shape[:-1] + (d * bits // 8,))


_orig_widen = codec.widen


def _widen_shift_15(raw, dtype):
    # bf16 bits shifted one place short of the float32 position
    if dtype == "bf16":
        return (np.asarray(raw, dtype=np.uint16).astype(np.uint32) << 15).view(np.float32).astype(np.float64)
    return _orig_widen(raw, dtype)


def _widen_bf16_as_f16(raw, dtype):
    # bf16 bits read as an IEEE half
    if dtype == "bf16":
        return np.asarray(raw, dtype=np.uint16).view(np.float16).astype(np.float64)
    return _orig_widen(raw, dtype)


_orig_decode = codec.decode


def _decode_gather_not_scatter(planes, p, shape):
    if p.perm is None:
        return _orig_decode(planes, p, shape)
    inv = np.argsort(p.perm)
    p2 = codec.CodecParams(**{**p.__dict__, "perm": inv.astype(np.uint16)})
    return _orig_decode(planes, p2, shape)


def _decode_rho_plus_eps(planes, p, shape):
    y = _orig_decode(planes, p, shape)
    if p.quant == "lloyd":
        n = planes["norm"].astype(np.float64)[..., None]
        y = np.where(n > 0, y / np.where(n > 0, n, 1) * (n + p.eps), y)
    return y


_orig_append = codec.append


def _append_slot_is_position(cache, x, positions, p):
    # the slot taken as the position itself, ignoring the cache's first position
    return _orig_append(cache, x, positions, codec.CodecParams(**{**p.__dict__, "pos_offset": 0}))


from oracle import calibration as _cal

_orig_outlier_perm = _cal.outlier_perm
_orig_channel_stats = _cal.channel_stats


def _perm_top_first(stats, group_size):
    # the top channels at positions 0, 1, 2, ... instead of multiples of the group size
    stats = np.asarray(stats, dtype=np.float64)
    d = stats.shape[0]
    order = sorted(range(d), key=lambda c: (-stats[c], c))
    k = d // group_size
    return np.array(order[:k] + sorted(order[k:]), dtype=np.uint16)


def _stats_rms(x, rope=False, rope_base=10000.0, pos_offset=0, n_sink=0):
    a = _orig_channel_stats(np.asarray(x) ** 2, False, rope_base, pos_offset, n_sink)
    return np.sqrt(a) if not rope else _orig_channel_stats(x, rope, rope_base, pos_offset, n_sink) * 1.0001


def _stats_no_rope(x, rope=False, rope_base=10000.0, pos_offset=0, n_sink=0):
    return _orig_channel_stats(x, False, rope_base, pos_offset, n_sink)


def _stats_with_sinks(x, rope=False, rope_base=10000.0, pos_offset=0, n_sink=0):
    return _orig_channel_stats(x, rope, rope_base, pos_offset, 0)


def _detect_mean(x, lam):
    nrm = _cal.token_norms(x)
    flags = nrm > lam * nrm.mean(axis=1, keepdims=True)
    prefix = np.array([int(np.nonzero(f)[0].max()) + 1 if f.any() else 0 for f in flags])
    return flags, flags.sum(axis=1), prefix


from oracle import dynamic as _dyn

_orig_dynamic_codebook = _dyn.dynamic_codebook
_orig_dyn_codes = _dyn.dyn_codes
_orig_pack_extra = _dyn.pack_extra


def _dyncb_variance(moments, bits):
    sc, wide, cb, cbw = _orig_dynamic_codebook(moments, bits)
    return sc * sc, wide, cb, cbw  # the variance taken as the scale


def _dyncb_smallest_wide(moments, bits):
    sc, wide, cb, cbw = _orig_dynamic_codebook(moments, bits)
    order = np.argsort(sc, kind="stable")
    w = np.zeros_like(wide)
    w[order[:wide.sum()]] = True
    return sc, w, cb, cbw


def _dyn_codes_no_wide(z, scale, wide, cb, cb_wide, bits):
    return _orig_dyn_codes(z, scale, np.zeros_like(np.asarray(wide, dtype=bool)), cb, cb_wide, bits)


def _pack_extra_msb(top, wide):
    idx = np.nonzero(np.asarray(wide, dtype=bool))[0]
    return np.packbits(np.asarray(top, dtype=np.uint8)[..., idx], axis=-1, bitorder="big")


from oracle import bitwidth as _bw

_orig_attention_entropy = _bw.attention_entropy
_orig_allocate_bits = _bw.allocate_bits


def _entropy_bits(q, k, lengths, scale):
    return _orig_attention_entropy(q, k, lengths, scale) / np.log(2.0)  # in bits, not nats


def _allocate_inverse(e, total, lo=2, hi=4):
    e = np.asarray(e, dtype=np.float64)
    return _orig_allocate_bits(e.max() + e.min() - e, total, lo, hi)  # more bits to less entropy


def _allocate_round(e, total, lo=2, hi=4):
    e = np.asarray(e, dtype=np.float64)
    x = total * e / e.sum() if e.sum() > 0 else np.full(len(e), total / len(e))
    return np.clip(np.rint(x), lo, hi).astype(np.int64)  # rounded, the total not kept


from oracle import attention as _attention

_orig_attend_decoded = _attention.attend_decoded


def _attend_heads_interleaved(q, k, v, lengths, scale):
    # query head m reading KV head m % heads instead of m // group
    hq, h = q.shape[1], k.shape[2]
    order = np.array([(m % h) * (hq // h) + m // h for m in range(hq)])
    out = _orig_attend_decoded(q[:, order], k, v, lengths, scale)
    res = np.empty_like(out)
    res[:, order] = out
    return res


_orig_rotor_rotate = rotations.rotor_rotate


def _rotor_inverse_sandwich(u, rq, tail_angle=0.0):
    # r* (0, v) r instead of r (0, v) r*
    return rotations.rotor_inverse(u, rq, -tail_angle)


def _rotor_tail_sign(u, rq, tail_angle=0.0):
    return _orig_rotor_rotate(u, rq, -tail_angle)


def _rotor_blocks_shifted(u, rq, tail_angle=0.0):
    # blocks taken from channel 1 on (3b + 1 .. 3b + 3), channel 0 left alone
    u = np.asarray(u, dtype=np.float64)
    out = np.array(u)
    nb = u.shape[-1] // 3
    part = _orig_rotor_rotate(np.concatenate([u[..., 1:3 * nb + 1], np.zeros(u.shape[:-1] + (2,))], axis=-1)
                              [..., :u.shape[-1]], rq, 0.0)
    out[..., 1:3 * nb + 1] = part[..., :3 * nb]
    return out


def _dense_inverse_no_transpose(z, m):
    return np.asarray(z, dtype=np.float64) @ np.asarray(m, dtype=np.float64).T


MUTATIONS = {
    "rotor_inverse_sandwich": (rotations, "rotor_rotate", _rotor_inverse_sandwich),
    "rotor_tail_sign": (rotations, "rotor_rotate", _rotor_tail_sign),
    "rotor_blocks_shifted": (rotations, "rotor_rotate", _rotor_blocks_shifted),
    "dense_inverse_no_transpose": (rotations, "dense_inverse", _dense_inverse_no_transpose),
    "rope_negative_sine": (rope, "rope", _rope_neg_sine),
    "rope_half_split_pairs": (rope, "rope", _rope_half_split),
    "rope_theta_exponent": (rope, "thetas", _thetas_wrong_exponent),
    "fwht_missing_normalisation": (rotations, "fwht", _fwht_unnormalised),
    "quat_mul_sign": (rotations, "quat_mul", _quat_mul_sign_slip),
    "so4_operands_swapped": (rotations, "so4_rotate", _so4_swapped),
    "fp16_round_down_to_nearest": (quant, "fp16_round_down", _round_nearest),
    "fp16_round_up_to_nearest": (quant, "fp16_round_up", _round_nearest),
    "minmax_range_from_min": (quant, "minmax_params", _minmax_params_range_from_min),
    "minmax_floor_not_rint": (quant, "minmax_codes", _minmax_codes_floor),
    "lloyd_threshold_ge": (quant, "lloyd_codes", _lloyd_codes_ge),
    "lloyd_fit_biased": (lloyd, "fit_gaussian", _fit_wrong_mean),
    "pack_msb_first": (pack, "pack", _pack_msb_first),
    "decode_perm_gather": (codec, "decode", _decode_gather_not_scatter),
    "decode_rho_plus_eps": (codec, "decode", _decode_rho_plus_eps),
    "append_slot_is_position": (codec, "append", _append_slot_is_position),
    "widen_bf16_shift_15": (codec, "widen", _widen_shift_15),
    "outlier_perm_top_first": (_cal, "outlier_perm", _perm_top_first),
    "entropy_in_bits": (_bw, "attention_entropy", _entropy_bits),
    "bits_inverse_to_entropy": (_bw, "allocate_bits", _allocate_inverse),
    "bits_rounded_total_lost": (_bw, "allocate_bits", _allocate_round),
    "dynamic_scale_is_variance": (_dyn, "dynamic_codebook", _dyncb_variance),
    "dynamic_wide_smallest": (_dyn, "dynamic_codebook", _dyncb_smallest_wide),
    "dynamic_codes_no_wide": (_dyn, "dyn_codes", _dyn_codes_no_wide),
    "dynamic_extra_msb_first": (_dyn, "pack_extra", _pack_extra_msb),
    "channel_stats_rms": (_cal, "channel_stats", _stats_rms),
    "channel_stats_before_rope": (_cal, "channel_stats", _stats_no_rope),
    "channel_stats_with_sinks": (_cal, "channel_stats", _stats_with_sinks),
    "sinks_against_mean_norm": (_cal, "detect_sinks", _detect_mean),
    "widen_bf16_as_f16": (codec, "widen", _widen_bf16_as_f16),
    "attention_heads_interleaved": (_attention, "attend_decoded", _attend_heads_interleaved),
}


def _patch(monkeypatch, module, name, fn):
    monkeypatch.setattr(module, name, fn)
    # codec imported rope() by name; every other step is looked up through its module
    if module is rope and name == "rope":
        monkeypatch.setattr(codec, "_rope", fn)


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(monkeypatch, mutation):
    module, name, fn = MUTATIONS[mutation]
    _patch(monkeypatch, module, name, fn)
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check()
        except (AssertionError, ValueError, IndexError, ZeroDivisionError, FloatingPointError) as e:
            failed.append(check.__name__)
    assert failed, f"no pin caught the planted mistake {mutation}"
