"""Calibration of the RotateKV variants, float64: outlier-aware channel reordering and
activation-based attention-sink detection.

RotateKV page (method summary, technical framework and key design): (i) outlier-aware
rotation reorders the cache's channels so that the Walsh-Hadamard rotation adapts to the
channel-wise outlier distribution without giving up the fast transform; (iii) attention-
sink-aware quantization uses the massive activations to identify the attention sinks and
keeps them at higher precision.  The page gives neither the statistic, the ordering rule
nor a threshold; the readings taken are stated in each function.  (ii) The pre-RoPE
grouped-head rotation is not here: the page says its implementation is unknown.
"""
from __future__ import annotations

import numpy as np

from .rope import rope as _rope


def channel_stats(x: np.ndarray, rope: bool = False, rope_base: float = 10000.0, pos_offset: int = 0,
                  n_sink: int = 0) -> np.ndarray:
    """Per-channel mean absolute value of the vectors the codec would permute.

    ``x`` is a calibration slice [R, T, H, D] (float64); keys take RoPE at their positions
    pos_offset + t first (the permutation acts on post-RoPE keys).  Reading: the statistic
    is mean |y_c| over every row, token and head of the slice, sink positions (< n_sink,
    stored unrotated in fp16) left out.  Returns [D] float64.
    """
    x = np.asarray(x, dtype=np.float64)
    r, t, h, d = x.shape
    pos = pos_offset + np.arange(t, dtype=np.int64)
    y = _rope(x, pos, rope_base) if rope else x
    keep = pos >= n_sink
    y = y[:, keep]
    n = y.shape[0] * y.shape[1] * y.shape[2]
    if n == 0:
        return np.zeros(d)
    return np.abs(y).reshape(-1, d).sum(axis=0) / n


def outlier_perm(stats: np.ndarray, group_size: int) -> np.ndarray:
    """The outlier-aware gather map u'[j] = u[perm[j]] from per-channel statistics.

    Reading (derived, the page gives no rule): after the Sylvester-ordered transform,
    coefficient i takes input position j with sign (-1)^popcount(i & j).  For j a multiple
    of the min-max group size G, i & j depends only on i's bits above the group, so the
    sign is the same for every coefficient of a group: a channel placed there shifts each
    group by one constant, which the group's zero absorbs, and leaves its range (hence its
    scale) unchanged.  So the D/G channels with the largest statistic go to positions 0, G,
    2G, ... (largest first; equal statistics in ascending channel order), and every other
    channel fills the remaining positions in ascending channel order.
    """
    stats = np.asarray(stats, dtype=np.float64)
    d = stats.shape[0]
    k = d // group_size
    order = sorted(range(d), key=lambda c: (-stats[c], c))
    top = order[:k]
    rest = sorted(c for c in range(d) if c not in top)
    perm = np.empty(d, dtype=np.int64)
    free = [j for j in range(d) if j % group_size != 0]
    for a, c in enumerate(top):
        perm[a * group_size] = c
    for j, c in zip(free, rest):
        perm[j] = c
    return perm.astype(np.uint16)


def token_norms(x: np.ndarray) -> np.ndarray:
    """L2 norm of each token over all its heads and channels: [R, T] float64.

    Reading: a token's activation magnitude is the norm of its whole K (or V) row; it is the
    same before and after RoPE (RoPE rotates channel pairs), so no position enters.
    """
    x = np.asarray(x, dtype=np.float64)
    return np.sqrt(np.sum(x * x, axis=(2, 3)))


def lower_median(v: np.ndarray) -> float:
    """The element of rank floor((n - 1) / 2) of the ascending order (n >= 1)."""
    s = np.sort(np.asarray(v, dtype=np.float64))
    return float(s[(len(s) - 1) // 2])


def detect_sinks(x: np.ndarray, lam: float):
    """Activation-based sink detection per row of a calibration slice [R, T, H, D].

    Reading (the page names massive activations but no threshold): token t of row r is a
    sink when its norm exceeds ``lam`` times the row's lower median token norm.  Returns
    (flags bool [R, T], counts int [R], prefix int [R]) where prefix is one past the last
    flagged token (0 if none): the number of leading positions the codec's fp16 sink
    path must cover to keep every detected sink.
    """
    nrm = token_norms(x)
    r, t = nrm.shape
    flags = np.zeros((r, t), dtype=bool)
    for i in range(r):
        if t == 0:
            continue
        med = lower_median(nrm[i])
        flags[i] = nrm[i] > lam * med
    counts = flags.sum(axis=1)
    prefix = np.array([int(np.nonzero(f)[0].max()) + 1 if f.any() else 0 for f in flags], dtype=np.int64)
    return flags, counts, prefix
