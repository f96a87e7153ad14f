"""Pins of the CPU oracle: each check ties an oracle function to something other
than itself -- a closed form, an independent library routine, brute force, a
textbook table or a worked example -- and raises AssertionError on a mismatch.

The checks are plain functions so that ``test_oracle_pins`` can run them and
``test_oracle_mutations`` can run them again against an oracle with a planted
mistake and require that at least one check fails.
"""
from __future__ import annotations

import numpy as np
from scipy.spatial.transform import Rotation

from oracle import codec, lloyd, pack, quant, rope, rotations
from tests.conftest import read_golden

RNG_SEED = 1234


def _rng(k=0):
    return np.random.default_rng(RNG_SEED + k)


# --------------------------------------------------------------------------- #
# widening of the stored input
# --------------------------------------------------------------------------- #
# bf16 bit patterns and their values from the format's definition (1 sign bit, 8 exponent
# bits with bias 127, 7 fraction bits; exponent field 0 is subnormal: 2^-126 * f / 2^7)
BF16_PATTERNS = [
    (0x3F80, 1.0),
    (0xC049, -3.140625),                         # -(1 + 73/128) * 2^1
    (0x0001, 2.0 ** -133),                       # smallest subnormal
    (0x007F, 127 * 2.0 ** -133),                 # largest subnormal
    (0x0080, 2.0 ** -126),                       # smallest normal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),    # largest finite
    (0x4780, 65536.0),
    (0x3E80, 0.25),
    (0xBF81, -(1.0 + 2.0 ** -7)),
]
# fp16: 1 sign, 5 exponent bits with bias 15, 10 fraction bits
F16_PATTERNS = [(0x3C00, 1.0), (0x0001, 2.0 ** -24), (0x7BFF, 65504.0), (0xC200, -3.0), (0x3555, 1365 / 4096)]


def check_widen_exact():
    """bf16 and fp16 bit patterns widen to the values the formats define; -0 keeps its sign;
    random finite bf16 patterns agree with torch's own bfloat16 conversion (library)."""
    import torch
    bits = np.array([b for b, _ in BF16_PATTERNS], dtype=np.uint16)
    got = codec.widen(bits, "bf16")
    assert got.dtype == np.float64
    assert np.array_equal(got, np.array([v for _, v in BF16_PATTERNS])), got
    neg0 = codec.widen(np.array([0x8000], dtype=np.uint16), "bf16")
    assert neg0[0] == 0.0 and np.signbit(neg0[0])
    h = np.array([b for b, _ in F16_PATTERNS], dtype=np.uint16).view(np.float16)
    assert np.array_equal(codec.widen(h, "f16"), np.array([v for _, v in F16_PATTERNS]))
    f = np.array([1.5, -2.0 ** -140, 3.4e38], dtype=np.float32)
    assert np.array_equal(codec.widen(f, "f32"), f.astype(np.float64))
    raw = _rng(40).integers(0, 1 << 16, size=4096, dtype=np.uint16)
    raw = raw[(raw & 0x7F80) != 0x7F80]  # finite patterns only
    ref = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(codec.widen(raw, "bf16"), ref)


# --------------------------------------------------------------------------- #
# RoPE
# --------------------------------------------------------------------------- #
def check_rope_theta_special_values():
    """theta_0 = 1 and theta_{d/4} = base^(-1/2): 0.01 at base 10000 (closed form)."""
    for d in (8, 64, 128, 256):
        th = rope.thetas(d, 10000.0)
        assert th.shape == (d // 2,)
        assert th[0] == 1.0
        assert abs(th[d // 4] - 0.01) < 1e-15
        ratio = th[1:] / th[:-1]
        assert np.allclose(ratio, 10000.0 ** (-2.0 / d), rtol=1e-12)


def check_rope_basis_vectors():
    """R_p e_{2i} = (cos p th_i) e_{2i} + (sin p th_i) e_{2i+1}; R_p e_{2i+1} = -sin e_{2i} + cos e_{2i+1}.

    Pins the adjacent pairing and the sign of the sine (EliteKV page 2.1 matrix).
    """
    d = 16
    th = rope.thetas(d)
    for p in (1, 7, 1000):
        for i in (0, 3, 7):
            e = np.zeros((1, 1, 1, d))
            e[..., 2 * i] = 1.0
            y = rope.rope(e, np.array([p]))[0, 0, 0]
            want = np.zeros(d)
            want[2 * i] = np.cos(p * th[i])
            want[2 * i + 1] = np.sin(p * th[i])
            assert np.allclose(y, want, atol=1e-14), (p, i)
            e = np.zeros((1, 1, 1, d))
            e[..., 2 * i + 1] = 1.0
            y = rope.rope(e, np.array([p]))[0, 0, 0]
            want = np.zeros(d)
            want[2 * i] = -np.sin(p * th[i])
            want[2 * i + 1] = np.cos(p * th[i])
            assert np.allclose(y, want, atol=1e-14), (p, i)


def check_rope_composition():
    """R(a) R(b) = R(a + b) (RoPE-KV page 7.1), to 1e-12."""
    x = _rng(1).standard_normal((2, 5, 3, 32))
    pa = np.array([0, 1, 17, 300, 4095])
    pb = np.array([5, 0, 2, 1000, 28672])
    two = rope.rope(rope.rope(x, pa), pb)
    one = rope.rope(x, pa + pb)
    assert np.allclose(two, one, atol=1e-12)
    assert np.array_equal(rope.rope(x, np.zeros(5, dtype=np.int64)), x)


def check_rope_relative_position():
    """(R_m q).(R_n k) depends only on m - n, and equals the full expansion with the sine term."""
    rng = _rng(2)
    d = 64
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    th = rope.thetas(d)

    def dot(m, n):
        qm = rope.rope(q.reshape(1, 1, 1, d), np.array([m]))[0, 0, 0]
        kn = rope.rope(k.reshape(1, 1, 1, d), np.array([n]))[0, 0, 0]
        return qm @ kn

    for m, n in ((5, 3), (100, 37), (32767, 1)):
        base = dot(m, n)
        assert abs(dot(m + 11, n + 11) - base) < 1e-9
        delta = (m - n) * th
        q0, q1, k0, k1 = q[0::2], q[1::2], k[0::2], k[1::2]
        full = np.sum((q0 * k0 + q1 * k1) * np.cos(delta) + (q0 * k1 - q1 * k0) * np.sin(delta))
        assert abs(full - base) < 1e-9


def check_rope_complex_form():
    """Pair (x_2i, x_2i+1) as the complex number x_2i + i x_2i+1 multiplied by exp(i p theta_i)."""
    rng = _rng(3)
    d = 128
    x = rng.standard_normal((1, 6, 2, d))
    pos = np.array([0, 1, 2, 77, 4096, 32767])
    y = rope.rope(x, pos)
    th = rope.thetas(d)
    zc = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * pos[:, None, None] * th)[None]
    assert np.allclose(y[..., 0::2], zc.real, atol=1e-12)
    assert np.allclose(y[..., 1::2], zc.imag, atol=1e-12)


# --------------------------------------------------------------------------- #
# Walsh-Hadamard
# --------------------------------------------------------------------------- #
def check_hadamard_definition():
    """H[i, j] = (-1)^popcount(i & j) (Sylvester order) and H H^T = d I."""
    for d in (2, 4, 16, 128, 256):
        h = rotations.hadamard(d)
        i = np.arange(d)
        pc = np.array([[bin(a & b).count("1") for b in i] for a in i])
        assert np.array_equal(h, (-1.0) ** pc)
        assert np.array_equal(h @ h.T, d * np.eye(d))


def _fwht_butterflies(u):
    """Textbook in-place fast Walsh-Hadamard transform (natural order), unnormalised."""
    a = np.array(u, dtype=np.float64).copy()
    d = a.shape[-1]
    hlen = 1
    while hlen < d:
        a = a.reshape(a.shape[:-1] + (d // (2 * hlen), 2, hlen))
        top = a[..., 0, :] + a[..., 1, :]
        bot = a[..., 0, :] - a[..., 1, :]
        a = np.stack([top, bot], axis=-2).reshape(a.shape[:-3] + (d,))
        hlen *= 2
    return a


def check_fwht_transform():
    """fwht matches a butterfly FWHT / sqrt(d); e_0 -> constant 1/sqrt(d); involution; Parseval."""
    rng = _rng(4)
    for d in (128, 256):
        u = rng.standard_normal((7, d))
        z = rotations.fwht(u)
        assert np.allclose(z, _fwht_butterflies(u) / np.sqrt(d), atol=1e-12)
        e0 = np.zeros(d)
        e0[0] = 1.0
        assert np.allclose(rotations.fwht(e0), np.full(d, 1.0 / np.sqrt(d)), atol=1e-15)
        ones = np.ones(d)
        want = np.zeros(d)
        want[0] = np.sqrt(d)
        assert np.allclose(rotations.fwht(ones), want, atol=1e-12)
        assert np.allclose(rotations.fwht(z), u, atol=1e-12)
        assert np.allclose(np.sum(z * z, -1), np.sum(u * u, -1), rtol=1e-12)


# --------------------------------------------------------------------------- #
# quaternions / SO(4)
# --------------------------------------------------------------------------- #
ONE = np.array([1.0, 0, 0, 0])
QI = np.array([0, 1.0, 0, 0])
QJ = np.array([0, 0, 1.0, 0])
QK = np.array([0, 0, 0, 1.0])


def check_hamilton_rules():
    """i j = k, j k = i, k i = j, j i = -k, i^2 = j^2 = k^2 = i j k = -1."""
    m = rotations.quat_mul
    assert np.array_equal(m(QI, QJ), QK)
    assert np.array_equal(m(QJ, QK), QI)
    assert np.array_equal(m(QK, QI), QJ)
    assert np.array_equal(m(QJ, QI), -QK)
    for q in (QI, QJ, QK):
        assert np.array_equal(m(q, q), -ONE)
    assert np.array_equal(m(m(QI, QJ), QK), -ONE)
    assert np.array_equal(m(ONE, QJ), QJ) and np.array_equal(m(QJ, ONE), QJ)


def _quat_params(ql, qr, nblocks=1):
    q = np.zeros((nblocks, 2, 4))
    q[:, 0] = ql
    q[:, 1] = qr
    return q


def check_so4_product_order():
    """T(v) = qL v qR: qL = i, qR = 1 maps j -> k; qL = 1, qR = i maps j -> -k."""
    assert np.array_equal(rotations.so4_rotate(QJ, _quat_params(QI, ONE)), QK)
    assert np.array_equal(rotations.so4_rotate(QJ, _quat_params(ONE, QI)), -QK)
    assert np.array_equal(rotations.so4_rotate(QK, _quat_params(ONE, ONE)), QK)


def _unit(rng, n):
    g = rng.standard_normal((n, 4))
    return g / np.linalg.norm(g, axis=1, keepdims=True)


def check_so4_orthogonality():
    """Unit (qL, qR) give an orthogonal map with det +1; norms kept; (-qL, -qR) identical; inverse exact."""
    rng = _rng(5)
    nb = 32
    q = np.zeros((nb, 2, 4))
    q[:, 0] = _unit(rng, nb)
    q[:, 1] = _unit(rng, nb)
    u = rng.standard_normal((9, 4 * nb))
    z = rotations.so4_rotate(u, q)
    assert np.allclose(np.sum(z * z, -1), np.sum(u * u, -1), rtol=1e-12)
    assert np.allclose(rotations.so4_rotate(u, -q), z, atol=1e-13)
    assert np.allclose(rotations.so4_inverse(z, q), u, atol=1e-12)
    for b in range(4):
        qb = q[b:b + 1]
        m = np.stack([rotations.so4_rotate(e, qb) for e in np.eye(4)], axis=1)
        assert np.allclose(m.T @ m, np.eye(4), atol=1e-13)
        assert abs(np.linalg.det(m) - 1.0) < 1e-12


def check_so4_reduces_to_3d_rotation():
    """qR = qL*: v = (0, r) -> (0, R r) with R the rotation of unit quaternion qL (scipy, scalar-last)."""
    rng = _rng(6)
    for _ in range(5):
        ql = _unit(rng, 1)[0]
        r3 = rng.standard_normal(3)
        v = np.concatenate(([0.0], r3))
        out = rotations.so4_rotate(v, _quat_params(ql, ql * np.array([1, -1, -1, -1])))
        want = Rotation.from_quat([ql[1], ql[2], ql[3], ql[0]]).apply(r3)
        assert abs(out[0]) < 1e-13
        assert np.allclose(out[1:], want, atol=1e-12)


# --------------------------------------------------------------------------- #
# fp16 directed rounding and min-max quantization
# --------------------------------------------------------------------------- #
_ALL_F16 = np.arange(65536, dtype=np.uint16).view(np.float16)
_FINITE_F16 = np.unique(_ALL_F16[np.isfinite(_ALL_F16)].astype(np.float64))


def check_fp16_directed_rounding():
    """Round-down/up agree with an exhaustive search over every finite float16."""
    rng = _rng(7)
    x = np.concatenate([rng.standard_normal(300) * 3, rng.standard_normal(50) * 1e-6,
                        [0.0, -0.0, 1.0, -1.0, 65504.0, -65504.0, 5.9604645e-08, 1e-9, -1e-9]])
    x = np.concatenate([x, _FINITE_F16[rng.integers(0, len(_FINITE_F16), 50)]])
    dn = quant.fp16_round_down(x).astype(np.float64)
    up = quant.fp16_round_up(x).astype(np.float64)
    for xi, d_, u_ in zip(x, dn, up):
        want_dn = _FINITE_F16[_FINITE_F16 <= xi].max()
        want_up = _FINITE_F16[_FINITE_F16 >= xi].min()
        assert d_ == want_dn, (xi, d_, want_dn)
        assert u_ == want_up, (xi, u_, want_up)


def check_minmax_properties():
    """Grid covers [min, max]; |z - y| <= scale/2; codes in range; scale and zero are the tightest fp16."""
    rng = _rng(8)
    for bits in (2, 3, 4):
        for g in (32, 128):
            z = rng.standard_normal((40, 256)) * rng.uniform(0.1, 20, (40, 1)) + rng.uniform(-5, 5, (40, 1))
            scale, zero = quant.minmax_params(z, bits, g)
            q, t = quant.minmax_codes(z, scale, zero, bits, g)
            y = quant.minmax_dequant(q, scale, zero, g)
            levels = 2 ** bits - 1
            zg = z.reshape(40, 256 // g, g)
            s64, z64 = scale.astype(np.float64), zero.astype(np.float64)
            assert np.all(z64 <= zg.min(-1))
            assert np.all(np.nextafter(zero, np.float16(np.inf)).astype(np.float64) > zg.min(-1))
            assert np.all(z64 + levels * s64 >= zg.max(-1))
            prev = np.nextafter(scale, np.float16(-np.inf)).astype(np.float64)
            assert np.all(z64 + levels * prev < zg.max(-1))
            assert q.max() <= levels
            err = np.abs(z - y).reshape(40, 256 // g, g)
            assert np.all(err <= s64[..., None] / 2 * (1 + 1e-12))
            # brute force: nearest grid point (ties excluded)
            grid = z64[..., None] + np.arange(levels + 1) * s64[..., None]  # [40, ng, L]
            dist = np.abs(zg[..., None] - grid[:, :, None, :])
            best = np.argmin(dist, axis=-1).reshape(40, 256)
            tie = np.abs(t - np.floor(t) - 0.5) < 1e-9
            assert np.array_equal(best[~tie], q[~tie])


def check_minmax_degenerate_group():
    """A constant group that is an fp16 value: scale 0, codes 0, reconstruction exact."""
    z = np.full((1, 128), 0.375)
    scale, zero = quant.minmax_params(z, 2, 128)
    q, _ = quant.minmax_codes(z, scale, zero, 2, 128)
    assert scale[0, 0] == 0 and zero[0, 0] == np.float16(0.375)
    assert np.all(q == 0)
    assert np.all(quant.minmax_dequant(q, scale, zero, 128) == 0.375)


def check_lloyd_codes_nearest():
    """Threshold rule equals brute-force nearest centroid; a value on a threshold takes the lower code."""
    rng = _rng(9)
    cb = np.sort(rng.standard_normal(8))
    u = rng.standard_normal(5000) * 1.5
    q = quant.lloyd_codes(u, cb)
    nearest = np.argmin(np.abs(u[:, None] - cb[None, :]), axis=1)
    assert np.array_equal(q, nearest)
    tau = 0.5 * (cb[:-1] + cb[1:])
    assert np.array_equal(quant.lloyd_codes(tau, cb), np.arange(7))
    assert np.array_equal(quant.lloyd_dequant(np.arange(8), cb), cb)


# --------------------------------------------------------------------------- #
# Lloyd-Max fitting
# --------------------------------------------------------------------------- #
def check_lloyd_max_table():
    """Fitted N(0,1) quantizers match Max (1960), Table I, and the 1-bit closed form."""
    rows = read_golden("lloyd_max_gaussian.txt")
    fits = {b: lloyd.fit_gaussian(b, 1.0) for b in (1, 2, 3, 4)}
    for bits, kind, vals in rows:
        b = int(bits)
        c = fits[b]
        half = c[len(c) // 2:]
        if kind == "levels":
            want = np.array([float(v) for v in vals.split()])
            assert np.allclose(half, want, atol=6e-4), (b, half, want)
        elif kind == "thresholds":
            want = np.array([float(v) for v in vals.split()])
            tau = 0.5 * (c[:-1] + c[1:])
            assert np.allclose(tau[len(tau) // 2:], want, atol=6e-4), (b, tau, want)
        elif kind == "mse":
            assert abs(lloyd.gaussian_mse(c) - float(vals)) < 6e-4 * float(vals) + 2e-6, b
    assert abs(fits[1][1] - np.sqrt(2 / np.pi)) < 1e-12


def check_lloyd_max_fixed_point():
    """Converged: every centroid is its cell's conditional mean; symmetric; scales with sigma."""
    from scipy.integrate import quad
    from scipy.stats import norm
    sigma = 1.0 / np.sqrt(128.0)
    for b in (2, 3):
        c = lloyd.fit_gaussian(b, sigma)
        assert np.allclose(c, -c[::-1], atol=1e-15)
        tau = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
        for k in range(len(c)):
            num = quad(lambda x: x * norm.pdf(x, scale=sigma), tau[k], tau[k + 1], epsabs=1e-14)[0]
            den = quad(lambda x: norm.pdf(x, scale=sigma), tau[k], tau[k + 1], epsabs=1e-14)[0]
            assert abs(num / den - c[k]) < 1e-9 * sigma * 100, (b, k)
        assert np.allclose(c, lloyd.fit_gaussian(b, 1.0) * sigma, rtol=1e-12)


def check_lloyd_max_brute_force():
    """Brute force: 1-D Lloyd iterations on a fine weighted grid of N(0,1) reach the fitted
    centroids (to the grid's discretisation error, well under 1e-3)."""
    from scipy.stats import norm
    x = np.linspace(-8.0, 8.0, 160_001)
    w = np.exp(-0.5 * x * x)
    for b in (2, 3):
        c = norm.ppf((np.arange(2 ** b) + 0.5) / 2 ** b)
        for _ in range(150):
            tau = 0.5 * (c[:-1] + c[1:])
            idx = np.searchsorted(tau, x)
            c = np.bincount(idx, w * x, 2 ** b) / np.bincount(idx, w, 2 ** b)
        assert np.allclose(c, lloyd.fit_gaussian(b, 1.0), atol=1e-3), (b, c)


# --------------------------------------------------------------------------- #
# packing
# --------------------------------------------------------------------------- #
def check_pack_worked_examples():
    for bits, codes, hexbytes in read_golden("pack_examples.txt"):
        b = int(bits)
        q = np.array([int(v) for v in codes.split()], dtype=np.uint8)
        want = np.array([int(h, 16) for h in hexbytes.split()], dtype=np.uint8)
        got = pack.pack(q[None], b)[0]
        assert np.array_equal(got, want), (b, got, want)
        assert np.array_equal(pack.unpack(want[None], b, len(q))[0], q)


def check_pack_matches_numpy_and_bigint():
    """Agrees with np.packbits(bitorder='little') of the bit stream, and with a big-integer build."""
    rng = _rng(11)
    for b in (2, 3, 4):
        q = rng.integers(0, 2 ** b, (6, 128)).astype(np.uint8)
        got = pack.pack(q, b)
        bitsarr = ((q[..., None] >> np.arange(b)) & 1).astype(np.uint8).reshape(6, -1)
        assert np.array_equal(got, np.packbits(bitsarr, axis=-1, bitorder="little"))
        for row in range(6):
            big = sum(int(v) << (b * j) for j, v in enumerate(q[row]))
            assert bytes(got[row]) == big.to_bytes(128 * b // 8, "little")
        assert np.array_equal(pack.unpack(got, b, 128), q)


# --------------------------------------------------------------------------- #
# the whole pipeline
# --------------------------------------------------------------------------- #
def check_pipeline_error_bound():
    """Post-RoPE x vs decode(encode(x)): per-vector L2 error <= sqrt(sum_g G (scale_g/2)^2) (Parseval)."""
    rng = _rng(12)
    d, g = 128, 32
    x = rng.standard_normal((2, 9, 3, d))
    x[..., [5, 77]] *= 15
    perm = rng.permutation(d)
    for bits in (2, 4):
        p = codec.CodecParams(bits=bits, group_size=g, rope=True, perm=perm, n_sink=2, pos_offset=1)
        out = codec.encode(x, p)
        y = codec.decode(out, p, x.shape)
        xr = rope.rope(x, 1 + np.arange(9))
        err = np.sqrt(np.sum((y - xr) ** 2, axis=-1))[:, 1:]  # token 0 is a sink
        s = out["scale"].astype(np.float64)[:, 1:]
        bound = np.sqrt(np.sum(g * (s / 2) ** 2, axis=-1))
        assert np.all(err <= bound * (1 + 1e-9))
        assert out["sink_written"].tolist() == [False, True]
        assert np.array_equal(out["sink"][:, 1], xr[:, 0].astype(np.float16))
        assert np.array_equal(y[:, 0], xr[:, 0].astype(np.float16).astype(np.float64))
        assert np.all(out["codes"][:, 0] == 0) and np.all(out["scale"][:, 0] == 0)


def check_pipeline_sink_at_position_zero():
    """Position 0: RoPE is the identity, so the sink is fp16(x) bit for bit."""
    rng = _rng(13)
    x = rng.standard_normal((3, 4, 2, 128)).astype(np.float16).astype(np.float64)
    p = codec.CodecParams(bits=2, group_size=128, rope=True, n_sink=1)
    out = codec.encode(x, p)
    assert np.array_equal(out["sink"][:, 0], x[:, 0].astype(np.float16))


def check_pipeline_permutation_is_a_gather():
    """Encoding with perm equals encoding the gathered vector without it; decode scatters back."""
    rng = _rng(14)
    x = rng.standard_normal((1, 6, 2, 128))
    perm = rng.permutation(128)
    p1 = codec.CodecParams(bits=2, group_size=128, perm=perm)
    p0 = codec.CodecParams(bits=2, group_size=128)
    a = codec.encode(x, p1)
    b = codec.encode(x[..., perm], p0)
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scale"], b["scale"])
    ya = codec.decode(a, p1, x.shape)
    yb = codec.decode(b, p0, x.shape)
    assert np.allclose(ya[..., perm], yb, atol=1e-13)
    e = np.zeros((1, 1, 1, 128))
    e[..., perm[5]] = 1.0
    assert np.argmax(codec.encode(e, codec.CodecParams(bits=4, group_size=128, perm=perm, rot="none"))["q"]) == 5


def check_pipeline_norm_separation():
    """Lloyd path: stored rho = |x|; |u| = rho/(rho+eps); codes are the nearest centroids of the
    rotated direction (brute force); decoded / rho rotates onto codebook points; zero vector -> zero."""
    rng = _rng(15)
    d = 128
    nb = d // 4
    q = np.zeros((nb, 2, 4))
    q[:, 0] = _unit(rng, nb)
    q[:, 1] = _unit(rng, nb)
    cb = lloyd.fit_gaussian(3, 1.0 / np.sqrt(d))
    x = rng.standard_normal((2, 5, 1, d)) * 2.5
    x[0, 0, 0] = 0.0
    p = codec.CodecParams(bits=3, group_size=d, quant="lloyd", rot="so4", quat=q, codebook=cb)
    out = codec.encode(x, p)
    rho = np.sqrt(np.sum(x * x, axis=-1))
    assert np.allclose(out["norm"], rho, rtol=1e-7)
    un = x / (rho[..., None] + 1e-6)
    assert np.allclose(np.linalg.norm(un, axis=-1), rho / (rho + 1e-6), rtol=1e-13)
    zz = rotations.so4_rotate(un, q)
    nearest = np.argmin(np.abs(zz[..., None] - cb), axis=-1)
    assert np.array_equal(nearest, out["q"])
    y = codec.decode(out, p, x.shape)
    nz = out["norm"] > 0
    w = rotations.so4_rotate(y[nz] / out["norm"][nz].astype(np.float64)[..., None], q)
    assert np.min(np.abs(w[..., None] - cb), axis=-1).max() < 1e-12
    assert np.all(y[0, 0, 0] == 0.0)


# --------------------------------------------------------------------------- #
# decode-step append
# --------------------------------------------------------------------------- #
def check_append_matches_batch_encode():
    """Appending the tokens of a tensor one position at a time (in any order) into an empty
    cache reproduces the batch encode of the whole tensor, plane for plane; positions
    without a slot leave the cache untouched; rows are independent."""
    rng = _rng(16)
    r, t, h, d = 3, 7, 2, 128
    x = rng.standard_normal((r, t, h, d))
    x[..., [3, 90]] *= 15
    perm = rng.permutation(d)
    for quant_kind in ("minmax", "lloyd"):
        if quant_kind == "minmax":
            p = codec.CodecParams(bits=2, group_size=64, rope=True, perm=perm, n_sink=3, pos_offset=2)
        else:
            cb = lloyd.fit_gaussian(3, 1.0 / np.sqrt(d))
            p = codec.CodecParams(bits=3, group_size=d, quant="lloyd", rope=True, n_sink=3, pos_offset=2,
                                  codebook=cb)
        full = codec.encode(x, p)
        names = [n for n in ("codes", "scale", "zero", "norm", "sink") if n in full]
        cache = {n: np.zeros_like(full[n]) for n in names}
        for ti in rng.permutation(t):
            cache = codec.append(cache, x[:, ti], np.full(r, p.pos_offset + ti), p)
        for n in names:
            assert np.array_equal(cache[n], full[n]), n
        # no slot: below pos_offset, at pos_offset + t, far beyond
        for pos in (p.pos_offset - 1, p.pos_offset + t, 10 ** 6):
            again = codec.append(cache, x[:, 0] + 1.0, np.full(r, pos), p)
            for n in names:
                assert np.array_equal(again[n], cache[n]), n
        # one row at a time, each at its own position
        empty = {n: np.zeros_like(full[n]) for n in names}
        pos = np.array([p.pos_offset + 4, p.pos_offset, p.pos_offset + 6])
        xs = np.stack([x[i, pos[i] - p.pos_offset] for i in range(r)])
        one = codec.append(empty, xs, pos, p)
        for i in range(r):
            s = pos[i] - p.pos_offset
            for n in names:
                if n == "sink":
                    if pos[i] < p.n_sink:
                        assert np.array_equal(one[n][i, pos[i]], full[n][i, pos[i]])
                else:
                    assert np.array_equal(one[n][i, s], full[n][i, s]), n
                    other = np.delete(one[n][i], s, axis=0)
                    assert not np.any(other), n


# --------------------------------------------------------------------------- #
# decode-step attention over the encoded cache
# --------------------------------------------------------------------------- #
def check_attention_closed_forms():
    """One slot returns its value; identical keys (or scale 0) give the mean of the values;
    two slots weigh as a logistic of their score difference; query head m reads KV head
    m // group; slots at or past a row's length do not matter."""
    from oracle import attention
    rng = _rng(17)
    r, t, h, d, hq = 2, 6, 2, 8, 4
    k = rng.standard_normal((r, t, h, d))
    v = rng.standard_normal((r, t, h, d))
    q = rng.standard_normal((r, hq, d))
    one = attention.attend_decoded(q, k, v, np.array([1, 1]), 0.7)
    for m in range(hq):
        assert np.allclose(one[:, m], v[:, 0, m // 2], atol=1e-15)
    same = np.repeat(k[:, :1], t, axis=1)
    out = attention.attend_decoded(q, same, v, None, 0.7)
    assert np.allclose(out[:, 1], v[:, :, 0].mean(axis=1), atol=1e-13)
    assert np.allclose(out[:, 3], v[:, :, 1].mean(axis=1), atol=1e-13)
    assert np.allclose(attention.attend_decoded(q, k, v, None, 0.0)[:, 2], v[:, :, 1].mean(axis=1), atol=1e-13)
    # two slots: weights 1 / (1 + e^(s0 - s1)) on the second
    k2 = np.zeros((1, 2, 1, d))
    k2[0, 0, 0, 0], k2[0, 1, 0, 0] = 0.5, 2.0
    q2 = np.zeros((1, 1, d))
    q2[0, 0, 0] = 1.5
    v2 = rng.standard_normal((1, 2, 1, d))
    w1 = 1.0 / (1.0 + np.exp(0.3 * 1.5 * (0.5 - 2.0)))
    out2 = attention.attend_decoded(q2, k2, v2, None, 0.3)
    assert np.allclose(out2[0, 0], (1 - w1) * v2[0, 0, 0] + w1 * v2[0, 1, 0], atol=1e-14)
    # slots past the length are ignored; length 0 gives zeros
    lens = np.array([3, 0])
    a = attention.attend_decoded(q, k, v, lens, 0.7)
    k3, v3 = k.copy(), v.copy()
    k3[:, 3:] += 5.0
    v3[:, 3:] -= 7.0
    assert np.array_equal(a, attention.attend_decoded(q, k3, v3, lens, 0.7))
    assert not np.any(a[1])


def check_attention_matches_library_softmax():
    """The oracle equals the same attention written with scipy's softmax and einsum."""
    from scipy.special import softmax
    from oracle import attention
    rng = _rng(18)
    r, t, h, d, hq = 3, 11, 2, 16, 6
    k = rng.standard_normal((r, t, h, d)) * 3
    v = rng.standard_normal((r, t, h, d))
    q = rng.standard_normal((r, hq, d))
    kq = np.repeat(k, hq // h, axis=2)  # [r, t, hq, d]
    vq = np.repeat(v, hq // h, axis=2)
    w = softmax(0.25 * np.einsum("rmd,rtmd->rmt", q, kq), axis=-1)
    ref = np.einsum("rmt,rtmd->rmd", w, vq)
    assert np.allclose(attention.attend_decoded(q, k, v, None, 0.25), ref, atol=1e-12)


def check_attention_rotated_domain():
    """Attention over the encoded planes equals the rotated-domain evaluation: scores from
    the rotated query and the stored codes, scale and zero (q.k = (M P q).y with the
    orthonormal Hadamard M), values summed in the rotated domain and rotated back once,
    sink slots taken unrotated from the fp16 plane.  M comes from scipy's hadamard."""
    from scipy.linalg import hadamard
    from oracle import attention
    rng = _rng(19)
    r, t, h, d, hq, g, n_sink = 2, 9, 2, 128, 4, 64, 2
    x_k = rng.standard_normal((r, t, h, d))
    x_v = rng.standard_normal((r, t, h, d))
    perm = rng.permutation(d)
    pk = codec.CodecParams(bits=2, group_size=g, rope=True, perm=perm, n_sink=n_sink)
    pv = codec.CodecParams(bits=2, group_size=g, n_sink=n_sink)
    ek = codec.encode(x_k, pk)
    ev = codec.encode(x_v, pv)
    q = rng.standard_normal((r, hq, d))
    lens = np.array([t, 5])
    scale = d ** -0.5
    got = attention.attend(q, ek, pk, ev, pv, (r, t, h, d), lens, scale)
    mh = hadamard(d) / np.sqrt(d)
    qk = pack.unpack(ek["codes"], 2, d).astype(np.float64)
    qv = pack.unpack(ev["codes"], 2, d).astype(np.float64)
    ref = np.zeros((r, hq, d))
    for i in range(r):
        for m in range(hq):
            kv = m // (hq // h)
            qt = mh @ q[i, m][perm]  # rotated query
            s = np.empty(lens[i])
            for tt in range(lens[i]):
                if tt < n_sink:
                    s[tt] = q[i, m] @ ek["sink"][i, tt, kv].astype(np.float64)
                else:
                    sc = np.repeat(ek["scale"][i, tt, kv].astype(np.float64), g)
                    ze = np.repeat(ek["zero"][i, tt, kv].astype(np.float64), g)
                    s[tt] = qt @ (ze + qk[i, tt, kv] * sc)
            w = np.exp(scale * s - np.max(scale * s))
            w /= w.sum()
            acc = np.zeros(d)
            out = np.zeros(d)
            for tt in range(lens[i]):
                if tt < n_sink:
                    out += w[tt] * ev["sink"][i, tt, kv].astype(np.float64)
                else:
                    sc = np.repeat(ev["scale"][i, tt, kv].astype(np.float64), g)
                    ze = np.repeat(ev["zero"][i, tt, kv].astype(np.float64), g)
                    acc += w[tt] * (ze + qv[i, tt, kv] * sc)
            ref[i, m] = out + mh @ acc  # the V cache has no permutation
    assert np.allclose(got, ref, atol=1e-11)




# --------------------------------------------------------------------------- #
# calibration of the RotateKV variants (channel statistics, reordering, sinks)
# --------------------------------------------------------------------------- #
def check_channel_stats():
    """Brute-force loops (sinks left out); RoPE'd statistic of a one-channel input equals the
    mean |cos| / |sin| of its angles (library trig); position 0 alone gives mean |x|."""
    from oracle import calibration as cal
    rng = _rng(30)
    x = rng.standard_normal((2, 7, 3, 8)) * np.arange(1, 9)
    got = cal.channel_stats(x, n_sink=2)
    want = np.zeros(8)
    n = 0
    for r in range(2):
        for t in range(2, 7):
            for h in range(3):
                n += 1
                for c in range(8):
                    want[c] += abs(x[r, t, h, c])
    assert np.allclose(got, want / n, rtol=1e-14)
    d, t = 128, 300
    x1 = np.zeros((1, t, 1, d))
    i = 5
    x1[..., 2 * i] = 1.0
    th = 10000.0 ** (-2.0 * i / d)
    pos = 17 + np.arange(t)
    s = cal.channel_stats(x1, rope=True, pos_offset=17)
    assert np.isclose(s[2 * i], np.mean(np.abs(np.cos(pos * th))), rtol=1e-13)
    assert np.isclose(s[2 * i + 1], np.mean(np.abs(np.sin(pos * th))), rtol=1e-13)
    assert np.all(np.delete(s, [2 * i, 2 * i + 1]) == 0.0)
    x0 = rng.standard_normal((3, 1, 2, 128))
    assert np.allclose(cal.channel_stats(x0, rope=True), np.abs(x0).reshape(-1, 128).mean(0), rtol=1e-14)


def check_outlier_perm():
    """Worked placement; a bijection; equal statistics in channel order; and the property
    the reading rests on: a huge channel placed at a multiple of G leaves every group's
    range of the rotated vector unchanged, placed elsewhere it widens it."""
    from oracle import calibration as cal
    st = np.ones(128)
    st[[5, 77, 3, 100, 9]] = [10.0, 9.0, 8.0, 7.0, 6.0]
    p = cal.outlier_perm(st, 32)
    assert sorted(p.tolist()) == list(range(128))
    assert [int(p[j]) for j in (0, 32, 64, 96)] == [5, 77, 3, 100]
    rest = [int(p[j]) for j in range(128) if j % 32]
    assert rest == sorted(set(range(128)) - {5, 77, 3, 100})
    assert list(cal.outlier_perm(np.ones(128), 128)) == list(range(128))  # equal statistics: channel order
    p2 = cal.outlier_perm(np.ones(64), 32)
    assert [int(p2[0]), int(p2[32])] == [0, 1] and list(p2[1:32]) == list(range(2, 33)) and list(p2[33:]) == list(range(33, 64))
    rng = _rng(31)
    for g in (32, 64, 128):
        x = rng.standard_normal((5, 128))
        c = 41
        x[:, c] += 200.0
        st = cal.channel_stats(x[None, :, None, :])
        perm = cal.outlier_perm(st, g).astype(np.int64)
        assert perm[0] == c
        x0 = x.copy()
        x0[:, c] = 0.0

        def ranges(v, pm):
            z = rotations.fwht(v[:, pm]).reshape(5, 128 // g, g)
            return z.max(-1) - z.min(-1)
        assert np.allclose(ranges(x, perm), ranges(x0, perm), atol=1e-9)
        bad = perm.copy()
        bad[[0, 1]] = bad[[1, 0]]  # the outlier at position 1: signs alternate inside each group
        assert np.all(ranges(x, bad) > ranges(x0, bad) + 10.0)


def check_sink_detection():
    """Token norms: numpy's norm, unchanged by RoPE; the lower median's rank property
    (brute force); a worked row (x50 and x20 tokens among unit ones); loops on random data."""
    from oracle import calibration as cal
    rng = _rng(32)
    x = rng.standard_normal((3, 11, 2, 128))
    nrm = cal.token_norms(x)
    assert np.allclose(nrm, np.linalg.norm(x.reshape(3, 11, -1), axis=-1), rtol=1e-14)
    assert np.allclose(nrm, cal.token_norms(rope.rope(x, np.arange(11) + 1000)), rtol=1e-12)
    for n in (1, 2, 5, 8, 33):
        v = rng.standard_normal(n)
        m = cal.lower_median(v)
        k = (n - 1) // 2
        assert np.sum(v < m) <= k and np.sum(v <= m) >= k + 1 and m in v
        if n % 2:
            assert m == np.median(v)
    xs = np.ones((1, 10, 1, 4))
    xs[0, 0] *= 50.0
    xs[0, 3] *= 20.0
    xs[0, 6] *= 7.9
    f, c, pfx = cal.detect_sinks(xs, 8.0)
    assert f[0].tolist() == [True, False, False, True] + [False] * 6 and c[0] == 2 and pfx[0] == 4
    f, c, pfx = cal.detect_sinks(np.ones((2, 5, 1, 4)), 1.0)
    assert not f.any() and list(pfx) == [0, 0]
    y = rng.standard_normal((2, 9, 3, 16)) * rng.uniform(0.2, 3.0, (2, 9, 1, 1))
    f, c, pfx = cal.detect_sinks(y, 1.5)
    for r in range(2):
        nn = [np.sqrt(np.sum(y[r, t] ** 2)) for t in range(9)]
        med = sorted(nn)[4]
        want = [v > 1.5 * med for v in nn]
        assert f[r].tolist() == want and c[r] == sum(want)
        assert pfx[r] == (max(i for i, w in enumerate(want) if w) + 1 if any(want) else 0)


# --------------------------------------------------------------------------- #
# IsoQuant dynamic codebook
# --------------------------------------------------------------------------- #
def check_dynamic_kl_scale():
    """The KL-closest zero-mean Gaussian to a heavy-tailed sample (Student-t, library log
    density) has s^2 = mean z^2: the cross-entropy over a fine grid of s is smallest there."""
    from scipy.stats import norm as _norm
    from oracle import dynamic as dyn
    rng = _rng(40)
    z = rng.standard_t(3, size=20000) * 0.07
    m = np.mean(z * z)
    grid = np.sqrt(m) * np.linspace(0.8, 1.2, 401)
    ce = [-np.mean(_norm.logpdf(z, scale=sg)) for sg in grid]
    assert abs(grid[int(np.argmin(ce))] - np.sqrt(m)) <= (grid[1] - grid[0])
    mm = rng.uniform(0.1, 4.0, 128)
    mm[[7, 99, 3, 50, 51, 52, 53, 60]] = 9.0 + np.arange(8)
    sc, wide, cb, cbw = dyn.dynamic_codebook(mm, 3)
    assert np.allclose(sc, np.sqrt(mm), rtol=1e-15) and wide.sum() == 8
    assert set(np.nonzero(wide)[0].tolist()) == {7, 99, 3, 50, 51, 52, 53, 60}
    assert np.allclose(cb, lloyd.fit_gaussian(3, 1.0)) and np.allclose(cbw, lloyd.fit_gaussian(4, 1.0))


def check_dynamic_codes():
    """Codes = the nearest level of the channel's own scaled codebook (brute force), wide
    channels over 2^(b+1) levels; the extra plane's worked example and round trip."""
    from oracle import dynamic as dyn
    rng = _rng(41)
    d, b = 128, 3
    mm = rng.uniform(0.5, 2.0, d) / d
    sc, wide, cb, cbw = dyn.dynamic_codebook(mm, b)
    z = rng.standard_normal((50, d)) * sc * rng.uniform(0.5, 2.5, (50, 1))
    q, top, _ = dyn.dyn_codes(z, sc, wide, cb, cbw, b)
    full = q.astype(np.int64) + (top.astype(np.int64) << b)
    for j in range(d):
        lev = (cbw if wide[j] else cb) * sc[j]
        nearest = np.argmin(np.abs(z[:, j][:, None] - lev[None, :]), axis=1)
        assert np.array_equal(full[:, j], nearest), j
        assert np.all(top[:, j] == 0) or wide[j]
    y = dyn.dyn_dequant(q, top, sc, wide, cb, cbw, b)
    assert np.array_equal(y, np.where(wide, cbw[full], cb[np.minimum(full, 7)]) * sc)
    w = np.zeros(128, dtype=bool)
    w[[3, 10, 20, 30, 40, 50, 60, 127]] = True
    tp = np.zeros((1, 128), dtype=np.uint8)
    tp[0, [3, 20, 30, 127]] = 1
    ex = dyn.pack_extra(tp, w)
    assert ex.shape == (1, 1) and ex[0, 0] == 0b10001101
    assert np.array_equal(dyn.unpack_extra(ex, w), tp)


def check_dynamic_pipeline():
    """Moments: brute force, and Parseval (sum over channels = mean (rho/(rho+eps))^2); a round
    trip is within half a level gap of each scaled codebook; on channels of unequal spread the
    dynamic codebook's error is below the static N(0, 1/D) codebook's."""
    from oracle import dynamic as dyn
    rng = _rng(42)
    d = 128
    x = rng.standard_normal((2, 9, 2, d)) * np.concatenate([np.full(64, 0.3), np.full(64, 2.0)])
    perm = rng.permutation(d)
    p = codec.CodecParams(bits=3, group_size=d, quant="lloyd", rot="fwht", perm=perm, n_sink=2)
    m = codec.rotated_moments(x, p)
    want = np.zeros(d)
    n = 0
    for r in range(2):
        for t in range(2, 9):
            for h in range(2):
                u = x[r, t, h] / (np.linalg.norm(x[r, t, h]) + 1e-6)
                zz = rotations.hadamard(d) @ u[perm] / np.sqrt(d)
                want += zz * zz
                n += 1
    assert np.allclose(m, want / n, rtol=1e-12)
    rho = np.linalg.norm(x[:, 2:], axis=-1)
    assert np.isclose(m.sum(), np.mean((rho / (rho + 1e-6)) ** 2), rtol=1e-12)
    xr = rng.standard_normal((1, 400, 1, d)) * np.exp(rng.uniform(-1.5, 1.5, d))
    pr = codec.CodecParams(bits=3, group_size=d, quant="lloyd", rot="none")
    sc, wide, cb, cbw = dyn.dynamic_codebook(codec.rotated_moments(xr, pr), 3)
    pd = codec.CodecParams(bits=3, group_size=d, quant="lloyd", rot="none", codebook=cb, chan_scale=sc,
                           chan_wide=wide, codebook_wide=cbw)
    out = codec.encode(xr, pd)
    yd = codec.decode(out, pd, xr.shape)
    assert np.array_equal(out["extra"], dyn.pack_extra(out["top"], wide))
    lev = dyn.dyn_dequant(out["q"], out["top"], sc, wide, cb, cbw, 3)
    assert np.allclose(yd, lev * out["norm"].astype(np.float64)[..., None], rtol=1e-15, atol=0)
    ps = codec.CodecParams(bits=3, group_size=d, quant="lloyd", rot="none", codebook=lloyd.fit_gaussian(3, 1 / np.sqrt(d)))
    ys = codec.decode(codec.encode(xr, ps), ps, xr.shape)
    assert np.sum((yd - xr) ** 2) < 0.5 * np.sum((ys - xr) ** 2)


# --------------------------------------------------------------------------- #
# IsoQuant dynamic bit width by attention entropy
# --------------------------------------------------------------------------- #
def check_attention_entropy():
    """Closed forms: n equal keys give ln n; one dominant key gives ~0; two slots give the
    binary entropy of their logistic weight; scipy's entropy of scipy's softmax (library)."""
    from scipy.special import softmax
    from scipy.stats import entropy as sp_entropy
    from oracle import bitwidth as bw
    rng = _rng(50)
    d = 16
    k = np.zeros((1, 7, 1, d))
    q = rng.standard_normal((1, 2, d))
    e = bw.attention_entropy(q, k, np.array([5]), 0.3)
    assert np.allclose(e, np.log(5.0), rtol=1e-14)
    k2 = rng.standard_normal((1, 2, 1, d))
    e2 = bw.attention_entropy(q[:, :1], k2, None, 0.5)
    s = 0.5 * (k2[0, :, 0] @ q[0, 0])
    w = 1.0 / (1.0 + np.exp(-(s[0] - s[1])))
    assert np.isclose(e2[0, 0], -(w * np.log(w) + (1 - w) * np.log(1 - w)), rtol=1e-12)
    kb = rng.standard_normal((2, 30, 2, d))
    qb = rng.standard_normal((2, 4, d))
    eb = bw.attention_entropy(qb, kb, np.array([30, 11]), 0.25)
    for r, n in ((0, 30), (1, 11)):
        for m in range(4):
            p = softmax(0.25 * kb[r, :n, m // 2] @ qb[r, m])
            assert np.isclose(eb[r, m], sp_entropy(p), rtol=1e-12)
    assert bw.attention_entropy(qb, kb, np.array([0, 3]), 0.25)[0].tolist() == [0.0] * 4
    assert np.allclose(bw.head_entropy(eb, 2), [eb[:, :2].mean(), eb[:, 2:].mean()])


def check_bit_allocation():
    """Worked allocations; the sum and range always hold; equal entropies give equal widths;
    more entropy never gets fewer bits (random cases against brute force over all widths:
    the allocation minimises sum (b_h - x_h)^2 among valid ones up to ties)."""
    from itertools import product
    from oracle import bitwidth as bw
    assert bw.allocate_bits(np.array([1.0, 1.0, 2.0, 4.0]), 12).tolist() == [2, 2, 4, 4]
    assert bw.allocate_bits(np.ones(8), 24).tolist() == [3] * 8
    assert bw.allocate_bits(np.zeros(4), 10).tolist() == [3, 3, 2, 2]
    assert bw.allocate_bits(np.array([3.0, 1.0, 1.0, 1.0]), 12).tolist() == [4, 3, 3, 2]
    rng = _rng(51)
    for _ in range(40):
        h = int(rng.integers(2, 7))
        e = rng.uniform(0.0, 5.0, h)
        tot = int(rng.integers(2 * h, 4 * h + 1))
        b = bw.allocate_bits(e, tot)
        assert b.sum() == tot and b.min() >= 2 and b.max() <= 4
        x = tot * e / e.sum()
        best = min(sum((c - xi) ** 2 for c, xi in zip(cb, x)) for cb in product(range(2, 5), repeat=h) if sum(cb) == tot)
        assert np.isclose(np.sum((b - x) ** 2), best, rtol=1e-12, atol=1e-12)
        order = np.argsort(e)
        assert np.all(np.diff(b[order]) >= 0)


# --------------------------------------------------------------------------- #
# baseline rotations: TurboQuant's dense orthogonal matrix, RotorQuant's 3-D rotors
# --------------------------------------------------------------------------- #
def check_dense_rotation():
    """z = M u: with M = H/sqrt(d) it is the Walsh-Hadamard transform, with a permutation matrix
    the gather, with a 2-D rotation the textbook turn; for a Haar-random M (scipy's ortho_group)
    it keeps norms, and the inverse equals a linear solve of M u = z."""
    from scipy.stats import ortho_group
    rng = _rng(40)
    for d in (128, 256):
        u = rng.standard_normal((3, d))
        h = rotations.hadamard(d) / np.sqrt(d)
        assert np.allclose(rotations.dense_rotate(u, h), rotations.fwht(u), atol=1e-12)
        perm = rng.permutation(d)
        pm = np.zeros((d, d))
        pm[np.arange(d), perm] = 1.0
        assert np.array_equal(rotations.dense_rotate(u, pm), u[:, perm])
        m = ortho_group.rvs(d, random_state=int(rng.integers(1 << 30)))
        z = rotations.dense_rotate(u, m)
        assert np.allclose(np.linalg.norm(z, axis=-1), np.linalg.norm(u, axis=-1), rtol=1e-12)
        assert np.allclose(rotations.dense_inverse(z, m), np.linalg.solve(m, z.T).T, atol=1e-10)
        assert np.allclose(rotations.dense_inverse(z, m), u, atol=1e-10)
    t = 0.3
    rot2 = np.array([[np.cos(t), -np.sin(t)], [np.sin(t), np.cos(t)]])
    assert np.allclose(rotations.dense_rotate(np.array([1.0, 0.0]), rot2), [np.cos(t), np.sin(t)], atol=1e-15)


def check_rotor_rotation():
    """Each 3-channel block turns as scipy's Rotation of the same unit quaternion; the rotor about
    z by a maps e_x to (cos a, sin a, 0); r and -r are one rotation; rotors compose as quaternion
    products; d = 128 splits into 42 blocks and a 2-D tail turned by the tail angle, d = 256 into
    85 blocks and one channel left as it is; the inverse undoes the rotation."""
    rng = _rng(41)
    assert rotations.rotor_split(128) == (42, 2) and rotations.rotor_split(256) == (85, 1)
    for d in (128, 256):
        nb, tail = rotations.rotor_split(d)
        r = _unit(rng, nb)
        u = rng.standard_normal((4, d))
        ta = 0.7
        z = rotations.rotor_rotate(u, r, ta)
        for b in range(nb):
            want = Rotation.from_quat([r[b, 1], r[b, 2], r[b, 3], r[b, 0]]).apply(u[:, 3 * b:3 * b + 3])
            assert np.allclose(z[:, 3 * b:3 * b + 3], want, atol=1e-12)
        if tail == 2:
            a, c = u[:, -2], u[:, -1]
            assert np.allclose(z[:, -2], a * np.cos(ta) - c * np.sin(ta), atol=1e-14)
            assert np.allclose(z[:, -1], a * np.sin(ta) + c * np.cos(ta), atol=1e-14)
        else:
            assert np.array_equal(z[:, -1], u[:, -1])
        assert np.allclose(np.linalg.norm(z, axis=-1), np.linalg.norm(u, axis=-1), rtol=1e-12)
        assert np.allclose(rotations.rotor_inverse(z, r, ta), u, atol=1e-12)
        assert np.allclose(rotations.rotor_rotate(u, -r, ta), z, atol=1e-12)
        r2 = _unit(rng, nb)
        both = rotations.rotor_rotate(rotations.rotor_rotate(u, r, 0.0), r2, 0.0)
        assert np.allclose(both, rotations.rotor_rotate(u, rotations.quat_mul(r2, r), 0.0), atol=1e-12)
    a = 0.9
    rz = np.tile([np.cos(a / 2), 0.0, 0.0, np.sin(a / 2)], (42, 1))
    e = np.zeros(128)
    e[0], e[5] = 1.0, 2.0  # e_x of block 0, e_z of block 1
    z = rotations.rotor_rotate(e, rz, 0.0)
    assert np.allclose(z[:3], [np.cos(a), np.sin(a), 0.0], atol=1e-15)
    assert np.allclose(z[3:6], [0.0, 0.0, 2.0], atol=1e-15)


def check_pipeline_baseline_rotations():
    """The codec with the dense and the rotor rotation: min-max round trip within the Parseval
    bound of the group scales (any orthogonal rotation); Lloyd-Max codes are the nearest
    centroids of the rotated direction (brute force) and the decoded direction rotates back onto
    codebook points."""
    from scipy.stats import ortho_group
    rng = _rng(42)
    d, g = 128, 32
    m = ortho_group.rvs(d, random_state=7)
    rq = _unit(rng, d // 3)
    x = rng.standard_normal((2, 6, 2, d))
    x[..., [3, 90]] *= 12
    for kw in (dict(rot="dense", rot_matrix=m), dict(rot="rotor", rotor_quat=rq, rotor_tail=0.4)):
        for bits in (2, 3):
            p = codec.CodecParams(bits=bits, group_size=g, perm=rng.permutation(d), **kw)
            out = codec.encode(x, p)
            y = codec.decode(out, p, x.shape)
            err = np.sqrt(np.sum((y - x) ** 2, axis=-1))
            s = out["scale"].astype(np.float64)
            assert np.all(err <= np.sqrt(np.sum(g * (s / 2) ** 2, axis=-1)) * (1 + 1e-9))
        cb = lloyd.fit_gaussian(3, 1.0 / np.sqrt(d))
        p = codec.CodecParams(bits=3, group_size=d, quant="lloyd", codebook=cb, **kw)
        out = codec.encode(x, p)
        rho = np.sqrt(np.sum(x * x, axis=-1))
        un = x / (rho[..., None] + 1e-6)
        zz = rotations.dense_rotate(un, m) if kw["rot"] == "dense" else rotations.rotor_rotate(un, rq, 0.4)
        assert np.array_equal(np.argmin(np.abs(zz[..., None] - cb), axis=-1), out["q"])
        y = codec.decode(out, p, x.shape)
        back = y / out["norm"].astype(np.float64)[..., None]
        w = rotations.dense_rotate(back, m) if kw["rot"] == "dense" else rotations.rotor_rotate(back, rq, 0.4)
        assert np.min(np.abs(w[..., None] - cb), axis=-1).max() < 1e-12


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
