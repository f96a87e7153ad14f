"""IsoQuant's dynamic bit-width allocation by attention entropy, float64.

IsoQuant page, section 6.2: (1) compute each head's attention entropy, (2) allocate the
quantization bit widths in proportion to the entropy, (3) load the quantization kernel of
each width.  The page gives no formula; the readings taken:

* entropy: of the softmax attention distribution of a query head over a row's slots (the
  attention of the EliteKV page, section 7.1, over the decoded cache), in nats; a KV head's
  entropy is the mean over the rows and the query heads that read it (grouped-query
  attention: query head m reads KV head m // (q_heads / heads));
* allocation: KV head h gets b_h bits, lo <= b_h <= hi, with sum_h b_h = total: the ideal
  x_h = total * e_h / sum_g e_g (total / H each when every entropy is 0) is floored and
  clamped to [lo, hi], then single bits go one at a time to the head with the largest
  remainder x_h - b_h among those below hi (equal remainders: the lower head index) while
  the sum is short, and come off the head with the smallest remainder among those above lo
  (equal remainders: the higher index) while it is over;
* kernel: each head is then encoded by the codec at its own width.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def attention_entropy(q: np.ndarray, k: np.ndarray, lengths: Optional[np.ndarray], scale: float) -> np.ndarray:
    """q [R, HQ, D], decoded keys k [R, T, H, D] -> entropy [R, HQ] (nats); 0 for a row with
    no slot."""
    q = np.asarray(q, dtype=np.float64)
    r_, hq, _ = q.shape
    t_, h = k.shape[1], k.shape[2]
    group = hq // h
    out = np.zeros((r_, hq))
    for r in range(r_):
        n = t_ if lengths is None else int(min(max(int(lengths[r]), 0), t_))
        if n == 0:
            continue
        for m in range(hq):
            s = scale * (k[r, :n, m // group] @ q[r, m])
            p = np.exp(s - s.max())
            p /= p.sum()
            nz = p > 0
            out[r, m] = -np.sum(p[nz] * np.log(p[nz]))
    return out


def head_entropy(ent: np.ndarray, kv_heads: int) -> np.ndarray:
    """[R, HQ] -> per KV head mean over rows and its query heads."""
    r_, hq = ent.shape
    return ent.reshape(r_, kv_heads, hq // kv_heads).mean(axis=(0, 2))


def allocate_bits(e: np.ndarray, total: int, lo: int = 2, hi: int = 4) -> np.ndarray:
    e = np.asarray(e, dtype=np.float64)
    h = e.shape[0]
    if not lo * h <= total <= hi * h:
        raise ValueError("total bits outside [lo * heads, hi * heads]")
    x = np.full(h, total / h) if e.sum() <= 0 else total * e / e.sum()
    b = np.clip(np.floor(x), lo, hi).astype(np.int64)
    while b.sum() < total:
        cand = [i for i in range(h) if b[i] < hi]
        i = max(cand, key=lambda j: (x[j] - b[j], -j))
        b[i] += 1
    while b.sum() > total:
        cand = [i for i in range(h) if b[i] > lo]
        i = min(cand, key=lambda j: (x[j] - b[j], -j))
        b[i] -= 1
    return b
