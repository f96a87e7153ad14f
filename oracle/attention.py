"""Decode-step attention over an encoded KV cache, float64 -- test infrastructure.

EliteKV page, section 7.1 (core implementation): in single-token decoding the query is
scaled by head_dim^(-1/2), multiplied with every cached (post-RoPE) key, the scores are
normalised by a softmax over positions, and the output is the score-weighted sum of the
cached values.  Here the cached keys and values are the codec's decoded vectors
(``codec.decode``: no inverse RoPE, sink slots return their fp16 values).

Readings (the pages are silent):
* grouped-query attention: query head m uses KV head m // (q_heads / heads), the
  grouping of the Llama models the configurations are shaped on;
* each row attends over its first ``lengths[r]`` slots (all slots when no lengths are
  given); a row with no slot to attend over returns zeros;
* ``scale`` multiplies the scores (head_dim^(-1/2) in the page's code).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import codec


def attend_decoded(q: np.ndarray, k: np.ndarray, v: np.ndarray, lengths: Optional[np.ndarray],
                   scale: float) -> np.ndarray:
    """q [R, HQ, D]; k, v [R, T, H, D] (decoded cache) -> [R, HQ, D], float64."""
    q = np.asarray(q, dtype=np.float64)
    r_, hq, d = q.shape
    _, t_, h, _ = k.shape
    group = hq // h
    out = np.zeros((r_, hq, d))
    for r in range(r_):
        n = t_ if lengths is None else int(min(max(int(lengths[r]), 0), t_))
        if n == 0:
            continue
        for m in range(hq):
            kv = m // group
            s = scale * (k[r, :n, kv] @ q[r, m])
            w = np.exp(s - s.max())
            out[r, m] = (w @ v[r, :n, kv]) / w.sum()
    return out


def attend(q: np.ndarray, k_planes: Dict[str, np.ndarray], pk: codec.CodecParams,
           v_planes: Dict[str, np.ndarray], pv: codec.CodecParams, shape,
           lengths: Optional[np.ndarray], scale: float) -> np.ndarray:
    """Attention of q over the cache stored in the K and V planes (decoded by the oracle)."""
    k = codec.decode(k_planes, pk, shape)
    v = codec.decode(v_planes, pv, shape)
    return attend_decoded(q, k, v, lengths, scale)
