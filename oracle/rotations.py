"""Orthogonal rotations of a head vector, float64.

* Walsh-Hadamard: the RotateKV page (abstract and method section) rotates with the
  fast Walsh-Hadamard transform after channel reordering.  The pages do not
  write the transform out; the reading taken is the Sylvester-ordered Hadamard
  matrix H_d (H H^T = d I) applied as z = H u / sqrt(d), computed here as a
  brute-force matrix product (no fast algorithm).
* SO(4) isoclinic block rotation: the IsoQuant page, section 2.2 (a 4-D rotation
  is v -> qL v qR with unit quaternions; (qL, qR) and (-qL, -qR) give the same
  rotation) and section 3.2 (the Hamilton product with the real part first, and
  the order T(v) = qL (v qR)).  Channels 4b..4b+3 of a vector form block b as
  (w, x, y, z).  The inverse uses the conjugates (section 2.1: q* = a - bi - cj - dk).
* Baselines the IsoQuant page sets SO(4) against (section 1, the two approaches it compares):
  - TurboQuant: a global transform by a dense random orthogonal matrix M, z = M u, O(d^2)
    per vector; the inverse is M^T.  M is an input (drawn by the caller).
  - RotorQuant: 3-D Clifford rotors.  Reading: channels 3b, 3b+1, 3b+2 form block b
    (b < d // 3) and turn by the rotor of unit quaternion r_b, acting on the pure quaternion
    (0, v) by the sandwich product r (0, v) r* of section 2.1; the page's d = 128 example
    leaves a 2-D tail (42 blocks + 2 channels), which turns in its plane by an angle t
    (the rotor of a plane); a 1-channel tail (d = 256: 85 blocks + 1) stays as it is.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg


def hadamard(d: int) -> np.ndarray:
    """Sylvester-ordered Hadamard matrix of order d (entries +-1)."""
    return scipy.linalg.hadamard(d).astype(np.float64)


def fwht(u: np.ndarray) -> np.ndarray:
    """z = H_d u / sqrt(d) over the last axis (orthonormal, symmetric, self-inverse)."""
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    h = hadamard(d)
    return (u.reshape(-1, d) @ h.T).reshape(u.shape) / np.sqrt(d)


def quat_mul(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Hamilton product a*b of quaternions stored (w, x, y, z), real part first.

    The four components are those of the IsoQuant page, section 3.2 (``quat_mul``).
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    w1, x1, y1, z1 = a[..., 0], a[..., 1], a[..., 2], a[..., 3]
    w2, x2, y2, z2 = b[..., 0], b[..., 1], b[..., 2], b[..., 3]
    return np.stack([
        w1 * w2 - x1 * x2 - y1 * y2 - z1 * z2,
        w1 * x2 + x1 * w2 + y1 * z2 - z1 * y2,
        w1 * y2 - x1 * z2 + y1 * w2 + z1 * x2,
        w1 * z2 + x1 * y2 - y1 * x2 + z1 * w2,
    ], axis=-1)


def quat_conj(q: np.ndarray) -> np.ndarray:
    """q* = (w, -x, -y, -z) (IsoQuant page, section 2.1)."""
    q = np.asarray(q, dtype=np.float64)
    return q * np.array([1.0, -1.0, -1.0, -1.0])


def so4_rotate(u: np.ndarray, quat: np.ndarray) -> np.ndarray:
    """Per 4-D block b: z_b = qL_b * (u_b * qR_b); ``quat`` is [d/4][2][4] = (qL, qR).

    IsoQuant page, section 2.2 (T(v) = qL v qR) and section 3.2 (product order).
    """
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    q = np.asarray(quat, dtype=np.float64)
    blocks = u.reshape(u.shape[:-1] + (d // 4, 4))
    ql = q[:, 0, :]
    qr = q[:, 1, :]
    z = quat_mul(ql, quat_mul(blocks, qr))
    return z.reshape(u.shape)


def so4_inverse(z: np.ndarray, quat: np.ndarray) -> np.ndarray:
    """Per block: u_b = qL_b* * z_b * qR_b* (exact inverse for unit quaternions)."""
    z = np.asarray(z, dtype=np.float64)
    d = z.shape[-1]
    q = np.asarray(quat, dtype=np.float64)
    blocks = z.reshape(z.shape[:-1] + (d // 4, 4))
    u = quat_mul(quat_conj(q[:, 0, :]), quat_mul(blocks, quat_conj(q[:, 1, :])))
    return u.reshape(z.shape)


def dense_rotate(u: np.ndarray, m: np.ndarray) -> np.ndarray:
    """z = M u for every vector of u [..., d] (M [d, d], orthogonal)."""
    u = np.asarray(u, dtype=np.float64)
    return u @ np.asarray(m, dtype=np.float64).T


def dense_inverse(z: np.ndarray, m: np.ndarray) -> np.ndarray:
    """u = M^T z (the inverse of an orthogonal M)."""
    z = np.asarray(z, dtype=np.float64)
    return z @ np.asarray(m, dtype=np.float64)


def rotor_split(d: int):
    """(number of 3-D blocks, tail channels) of a head of d channels."""
    return d // 3, d % 3


def _rotor_apply(u: np.ndarray, rq: np.ndarray, tail_angle: float, inverse: bool) -> np.ndarray:
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    nb, tail = rotor_split(d)
    r = np.asarray(rq, dtype=np.float64)[:nb]
    out = np.array(u, dtype=np.float64)
    v = u[..., :3 * nb].reshape(u.shape[:-1] + (nb, 3))
    pure = np.concatenate([np.zeros(v.shape[:-1] + (1,)), v], axis=-1)
    left, right = (quat_conj(r), r) if inverse else (r, quat_conj(r))
    w = quat_mul(left, quat_mul(pure, right))  # r (0, v) r*, or r* (0, v) r for the inverse
    out[..., :3 * nb] = w[..., 1:].reshape(u.shape[:-1] + (3 * nb,))
    if tail == 2:
        t = -tail_angle if inverse else tail_angle
        a, b = u[..., 3 * nb], u[..., 3 * nb + 1]
        out[..., 3 * nb] = a * np.cos(t) - b * np.sin(t)
        out[..., 3 * nb + 1] = a * np.sin(t) + b * np.cos(t)
    return out


def rotor_rotate(u: np.ndarray, rq: np.ndarray, tail_angle: float = 0.0) -> np.ndarray:
    """RotorQuant's rotation: block b of 3 channels -> vector part of r_b (0, v_b) r_b*;
    a 2-channel tail turned by ``tail_angle``.  ``rq`` is [d // 3][4] unit quaternions (w, x, y, z)."""
    return _rotor_apply(u, rq, tail_angle, inverse=False)


def rotor_inverse(z: np.ndarray, rq: np.ndarray, tail_angle: float = 0.0) -> np.ndarray:
    """The inverse: r_b* (0, z_b) r_b per block, the tail turned back."""
    return _rotor_apply(z, rq, tail_angle, inverse=True)

