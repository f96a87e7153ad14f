"""Seeded synthetic inputs for the rotation + low-bit KV-cache codec.

This module holds shapes and random draws only.  No step of the codec's
arithmetic lives here: the CPU oracle (through the tests) and the GPU path
(through the tests and the bench) both take their inputs from these
generators, and neither side imports the other.

The five workloads mirror the KV-cache shapes the pages talk about:

* ``tiny``       one layer's K and V, fp16 [1, 256, 4, 128]; channels {7, 61} x10;
                 K: RoPE (positions 0..255) + FWHT, V: FWHT; 4-bit, group 128.
* ``llama2``     Llama-2-7B single layer, fp16 [1, 4096, 32, 128]; 4 outlier
                 channels x20, token 0 x50 (an attention sink); channel
                 permutation + FWHT on K and V; 2-bit, group 128; 4 fp16 sinks.
* ``isoquant``   8192 fp32 vectors of d=128, N(0,1); norm separation, 32 SO(4)
                 blocks with unit quaternions, 3-bit Lloyd-Max for N(0, 1/128).
* ``llama3``     Llama-3-8B full cache: 32 layers x batch 4 folded into 128 rows,
                 32768 tokens, 8 KV heads, d=128, bf16; 3 outlier channels x15;
                 K: RoPE + permutation + FWHT, V: FWHT; 2-bit, group 128; 4 sinks.
* ``widehead``   d=256, 16 layers x batch 2 = 32 rows, 16384 tokens, 16 heads,
                 bf16; 13 heavy-tailed Student-t(3) channels; FWHT-256;
                 K 2-bit, V 4-bit, group 32.

Random numbers the method itself would draw (the channel permutation, the
quaternions) are produced here and handed to both sides as inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional, Tuple

import numpy as np

SEED = 0


@dataclass(frozen=True)
class TensorCase:
    """One tensor of a workload and the codec settings applied to it."""

    name: str
    shape: Tuple[int, int, int, int]  # (rows, tokens, heads, head_dim)
    dtype: str  # "f16" | "bf16" | "f32"
    bits: int
    group_size: int
    quant: str  # "minmax" | "lloyd"
    rot: str  # "fwht" | "so4" | "none"
    rope: bool
    rope_base: float = 10000.0
    pos_offset: int = 0
    n_sink: int = 0
    use_perm: bool = False
    lloyd_sigma: Optional[float] = None  # codebook fitted for N(0, sigma^2)

    @property
    def n_vectors(self) -> int:
        r, t, h, _ = self.shape
        return r * t * h

    def with_shape(self, shape) -> "TensorCase":
        return replace(self, shape=tuple(int(s) for s in shape))


@dataclass(frozen=True)
class Workload:
    key: str
    title: str
    cases: Tuple[TensorCase, ...]
    device_generated: bool  # too large for host numpy: drawn on the GPU

    def case(self, name: str) -> TensorCase:
        for c in self.cases:
            if c.name == name:
                return c
        raise KeyError(name)


def _fwht_minmax(name, shape, dtype, bits, group, rope, n_sink, perm):
    return TensorCase(name=name, shape=shape, dtype=dtype, bits=bits, group_size=group,
                      quant="minmax", rot="fwht", rope=rope, n_sink=n_sink, use_perm=perm)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny", "Tiny one-layer K/V, fp16 [1,256,4,128], 4-bit group 128",
        (_fwht_minmax("K", (1, 256, 4, 128), "f16", 4, 128, True, 0, False),
         _fwht_minmax("V", (1, 256, 4, 128), "f16", 4, 128, False, 0, False)),
        device_generated=False),
    "llama2": Workload(
        "llama2", "Llama-2-7B layer K/V, fp16 [1,4096,32,128], perm + FWHT, 2-bit, 4 sinks",
        (_fwht_minmax("K", (1, 4096, 32, 128), "f16", 2, 128, False, 4, True),
         _fwht_minmax("V", (1, 4096, 32, 128), "f16", 2, 128, False, 4, True)),
        device_generated=False),
    "isoquant": Workload(
        "isoquant", "IsoQuant path, fp32 [1,8192,1,128], SO(4) + 3-bit Lloyd-Max",
        (TensorCase(name="X", shape=(1, 8192, 1, 128), dtype="f32", bits=3, group_size=128,
                    quant="lloyd", rot="so4", rope=False, lloyd_sigma=float(1.0 / np.sqrt(128.0))),),
        device_generated=False),
    "llama3": Workload(
        "llama3", "Llama-3-8B cache K/V, bf16 [128,32768,8,128], 2-bit group 128, 4 sinks",
        (_fwht_minmax("K", (128, 32768, 8, 128), "bf16", 2, 128, True, 4, True),
         _fwht_minmax("V", (128, 32768, 8, 128), "bf16", 2, 128, False, 4, False)),
        device_generated=True),
    "widehead": Workload(
        "widehead", "Wide-head K/V, bf16 [32,16384,16,256], FWHT-256, K 2-bit V 4-bit, group 32",
        (_fwht_minmax("K", (32, 16384, 16, 256), "bf16", 2, 32, False, 0, False),
         _fwht_minmax("V", (32, 16384, 16, 256), "bf16", 4, 32, False, 0, False)),
        device_generated=True),
}

# Outlier recipe per workload: (number of channels, kind, factor).
_OUTLIERS = {
    "tiny": ("fixed", (7, 61), 10.0),
    "llama2": ("seeded", 4, 20.0),
    "isoquant": (None, 0, 1.0),
    "llama3": ("seeded", int(round(0.02 * 128)), 15.0),
    "widehead": ("student_t", int(round(0.05 * 256)), 3.0),
}


# --------------------------------------------------------------------------- #
# dtype helpers (input representation only)
# --------------------------------------------------------------------------- #
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def cast_host(a: np.ndarray, dtype: str) -> np.ndarray:
    """float64 draw -> the input dtype.  bf16 is returned as raw uint16 bits."""
    if dtype == "f16":
        return a.astype(np.float16)
    if dtype == "f32":
        return a.astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(a.astype(np.float32))
    raise ValueError(dtype)


# --------------------------------------------------------------------------- #
# parameters drawn for the method (passed to both sides as inputs)
# --------------------------------------------------------------------------- #
def permutation(head_dim: int, seed: int = SEED) -> np.ndarray:
    """Fixed seeded channel permutation, shared by every row, head and layer."""
    return np.random.default_rng(seed).permutation(head_dim).astype(np.uint16)


def haar_orthogonal(d: int, rng: np.random.Generator) -> np.ndarray:
    """[d, d] float32 orthogonal matrix drawn from the Haar measure: the Q factor of a d x d
    standard normal matrix with the signs of R's diagonal moved into Q (a random draw the
    dense-rotation baseline takes as its input)."""
    g = rng.standard_normal((d, d))
    qm, rm = np.linalg.qr(g)
    return (qm * np.sign(np.diag(rm))[None, :]).astype(np.float32)


def rotor_quaternions(d: int, rng: np.random.Generator):
    """(rq [d // 3][4] float32 unit quaternions, tail angle) for the 3-D rotor baseline."""
    g = rng.standard_normal((d // 3, 4))
    rq = (g / np.linalg.norm(g, axis=1, keepdims=True)).astype(np.float32)
    return rq, float(rng.uniform(-np.pi, np.pi))


def unit_quaternions(n_blocks: int, rng: np.random.Generator) -> np.ndarray:
    """[n_blocks][2][4] float32: (qL, qR) per 4-D block, each (w, x, y, z) of unit norm.

    All qL are drawn first, then all qR, each as g/|g| with g ~ N(0, I4).
    """
    gl = rng.standard_normal((n_blocks, 4))
    gr = rng.standard_normal((n_blocks, 4))
    q = np.empty((n_blocks, 2, 4), dtype=np.float64)
    q[:, 0] = gl / np.linalg.norm(gl, axis=1, keepdims=True)
    q[:, 1] = gr / np.linalg.norm(gr, axis=1, keepdims=True)
    return q.astype(np.float32)


# --------------------------------------------------------------------------- #
# host generation (small workloads and test cases)
# --------------------------------------------------------------------------- #
def host_workload(key: str) -> Dict[str, object]:
    """Inputs of a host-generated workload.

    Returns ``{"inputs": {name: array}, "perm": uint16[D] | None, "quat": f32[D/4,2,4] | None}``;
    fp16/fp32 inputs are numpy arrays of that dtype, bf16 inputs are uint16 bit arrays.
    Draw order from ``default_rng(0)``: permutation (if any), then per tensor its outlier
    channels followed by its values; quaternions last.
    """
    wl = WORKLOADS[key]
    if wl.device_generated:
        raise ValueError(f"workload {key} is generated on the device; use device_workload")
    rng = np.random.default_rng(SEED)
    d = wl.cases[0].shape[-1]
    perm = rng.permutation(d).astype(np.uint16) if any(c.use_perm for c in wl.cases) else None
    kind, spec, factor = _OUTLIERS[key]
    inputs = {}
    for c in wl.cases:
        ch = None
        if kind in ("seeded", "student_t"):
            ch = rng.choice(d, int(spec), replace=False)
        x = rng.standard_normal(c.shape)
        if kind == "fixed":
            x[..., list(spec)] *= factor
        elif kind == "seeded":
            x[..., ch] *= factor
        if key == "llama2":
            x[:, 0] *= 50.0  # token 0: attention sink
        inputs[c.name] = cast_host(x, c.dtype)
    quat = None
    if any(c.rot == "so4" for c in wl.cases):
        quat = unit_quaternions(d // 4, rng)
    return {"inputs": inputs, "perm": perm, "quat": quat}


def synth_case(case: TensorCase, seed: int, outliers: Tuple[int, float] = (3, 15.0),
               sink_token_scale: float = 1.0) -> Dict[str, object]:
    """Small host case of arbitrary shape with the same value recipe (for parity tests).

    ``outliers`` = (number of seeded channels, factor); the first token of every row is
    multiplied by ``sink_token_scale``.
    """
    rng = np.random.default_rng(seed)
    d = case.shape[-1]
    perm = rng.permutation(d).astype(np.uint16) if case.use_perm else None
    n_out, factor = outliers
    x = rng.standard_normal(case.shape)
    if n_out:
        ch = rng.choice(d, n_out, replace=False)
        x[..., ch] *= factor
    if case.shape[1] > 0:
        x[:, 0] *= sink_token_scale
    quat = unit_quaternions(d // 4, rng) if case.rot == "so4" else None
    return {"input": cast_host(x, case.dtype), "perm": perm, "quat": quat}


# --------------------------------------------------------------------------- #
# device generation (the full-size workloads)
# --------------------------------------------------------------------------- #
def device_workload(key: str, device="cuda", names=None) -> Dict[str, object]:
    """Full-size inputs drawn on the GPU with ``torch.Generator(device).manual_seed(0)``.

    Values are drawn row by row in float32, outlier channels applied, then rounded to the
    tensor dtype.  Host-side parameters (permutation, outlier channels) come from
    ``numpy.random.default_rng(0)`` in the same order as ``host_workload``.
    """
    import torch

    wl = WORKLOADS[key]
    rng = np.random.default_rng(SEED)
    d = wl.cases[0].shape[-1]
    perm = rng.permutation(d).astype(np.uint16) if any(c.use_perm for c in wl.cases) else None
    kind, spec, factor = _OUTLIERS[key]
    gen = torch.Generator(device=device)
    gen.manual_seed(SEED)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
    inputs = {}
    for c in wl.cases:
        ch = rng.choice(d, int(spec), replace=False) if kind in ("seeded", "student_t") else None
        if names is not None and c.name not in names:
            continue
        r, t, h, _ = c.shape
        out = torch.empty(c.shape, dtype=tdt[c.dtype], device=device)
        ch_t = torch.as_tensor(ch, device=device, dtype=torch.long) if ch is not None else None
        for i in range(r):
            x = torch.randn((t, h, d), generator=gen, device=device, dtype=torch.float32)
            if kind == "seeded":
                x[..., ch_t] *= factor
            elif kind == "student_t":
                nu = int(factor)
                z = torch.randn((t, h, len(ch)), generator=gen, device=device, dtype=torch.float32)
                chi = torch.zeros_like(z)
                for _ in range(nu):
                    chi += torch.randn(z.shape, generator=gen, device=device, dtype=torch.float32) ** 2
                x[..., ch_t] = z / torch.sqrt(chi / nu)
            out[i] = x.to(out.dtype)
            del x
        inputs[c.name] = out
    return {"inputs": inputs, "perm": perm, "quat": None}
