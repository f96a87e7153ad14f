"""Decode-step append on the GPU vs the CPU oracle, through the C ABI (Python binding).

The cache planes start filled with a byte pattern.  Rows take positions that are
ordinary slots, sink positions and positions without a slot.  Which slots an append
writes follows the oracle's append (slot = position - pos_offset, none outside the
cache); every written slot must agree with the oracle's encode of that token at its
position under the codec's parity rules, and every other byte must keep the pattern.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import workloads
from tests import gpu_util as gu
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rotate_then_bit_amd as kvq  # noqa: E402  (fails loudly if libkvq.so is missing)

FILL = 0x5A


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _filled_planes(cfg):
    return gu.poison_planes(kvq.empty_planes(cfg), FILL)


def _check_append(case, x_np, positions, perm=None, quat=None, codebook=None, label=""):
    """x_np: [R, H, D] raw input; case.shape = (R, slots, H, D) is the cache."""
    r, slots, h, d = case.shape
    say(f"[case] append {label} cache={case.shape} dtype={case.dtype} bits={case.bits} G={case.group_size} "
        f"{case.rot}/{case.quant} rope={case.rope} sink={case.n_sink} pos0={case.pos_offset} "
        f"positions={positions.tolist()[:8]}")
    cfg = gu.make_config(case, perm, quat, codebook)
    cache = _filled_planes(cfg)
    before = gu.planes_numpy(cache)
    xt = gu.torch_input(x_np, case.dtype)
    pt = torch.from_numpy(np.asarray(positions, dtype=np.int64)).cuda()
    kvq.append(xt, pt, cache, cfg)
    torch.cuda.synchronize()
    g = gu.planes_numpy(cache)
    p = parity.params_for(case, perm, quat, codebook)
    x64 = oracle.widen(x_np, case.dtype)
    # bytes outside the written slots keep the pattern
    written = np.zeros((r, slots), dtype=bool)
    sink_written = np.zeros((r, max(case.n_sink, 1)), dtype=bool)
    for i in range(r):
        s = int(positions[i]) - case.pos_offset
        if 0 <= s < slots:
            written[i, s] = True
            if positions[i] < case.n_sink:
                sink_written[i, positions[i]] = True
    for name in ("codes", "scale", "zero", "norm"):
        if name not in g:
            continue
        assert np.array_equal(g[name][~written].view(np.uint8), before[name][~written].view(np.uint8)), \
            f"{label}: {name} bytes outside the appended slots changed"
    if "sink" in g:
        assert np.array_equal(g["sink"][~sink_written[:, :case.n_sink]].view(np.uint8),
                              before["sink"][~sink_written[:, :case.n_sink]].view(np.uint8)), \
            f"{label}: sink bytes outside the appended sinks changed"
    # each written row against the oracle's encode of that token at its position
    for i in np.nonzero(written.any(1))[0]:
        s = int(positions[i]) - case.pos_offset
        pi = parity.codec.CodecParams(**{**p.__dict__, "pos_offset": int(positions[i])})
        xi = x64[i][None, None]
        ora_i = oracle.encode(xi, pi)
        if case.n_sink:
            ora_i["sink_f64"] = parity.sink_f64(xi, pi)
        gi = {n: g[n][i:i + 1, s:s + 1] for n in ("codes", "scale", "zero", "norm") if n in g}
        if "sink" in g:
            gi["sink"] = g["sink"][i:i + 1]
            if positions[i] >= case.n_sink:
                # a non-sink row must not have written any sink slot of its row
                assert np.array_equal(g["sink"][i].view(np.uint8), before["sink"][i].view(np.uint8))
        parity.compare_encode(gi, ora_i, pi, (1, 1, h, d), f"{label} row {i} pos {int(positions[i])}",
                              fraction=False)
    return written


def _positions(rng, r, slots, pos0, n_sink):
    pos = rng.integers(pos0, pos0 + slots, size=r)
    extra = [pos0 - 1, pos0 + slots, pos0 + slots + 1000, -5] + list(range(min(n_sink, 3)))
    for k, v in enumerate(extra):
        if k + 1 < r:
            pos[k + 1] = v
    return pos.astype(np.int64)


@pytest.mark.parametrize("dtype,d,bits,rot,quant,rope,use_perm,n_sink,pos0", [
    ("bf16", 128, 2, "fwht", "minmax", True, True, 4, 0),     # Llama-3 K
    ("bf16", 128, 2, "fwht", "minmax", False, False, 4, 0),   # Llama-3 V
    ("f16", 128, 2, "fwht", "minmax", False, True, 4, 0),     # Llama-2 layer
    ("bf16", 256, 4, "fwht", "minmax", False, False, 0, 0),   # wide head, V
    ("f32", 128, 3, "so4", "lloyd", False, False, 0, 0),      # IsoQuant
    ("f16", 128, 4, "fwht", "minmax", True, False, 0, 0),     # tiny K
    ("bf16", 128, 3, "none", "minmax", True, True, 2, 5),     # offset cache, sinks outside it
    ("f32", 256, 2, "fwht", "lloyd", True, True, 3, 0),
])
def test_append_small(dtype, d, bits, rot, quant, rope, use_perm, n_sink, pos0):
    r, slots, h = 13, 21, 5
    g = d if (bits == 3 or quant == "lloyd") else 64
    case = workloads.TensorCase(name="X", shape=(r, slots, h, d), dtype=dtype, bits=bits, group_size=g,
                                quant=quant, rot=rot, rope=rope, n_sink=n_sink, use_perm=use_perm, pos_offset=pos0)
    seed = 300 + d + 7 * bits + (11 if rope else 0) + (5 if use_perm else 0) + pos0
    rng = np.random.default_rng(seed)
    data = workloads.synth_case(case.with_shape((r, 1, h, d)), seed)
    x = data["input"][:, 0]
    quat = data["quat"]
    cb = gu.codebook_for(case)
    _check_append(case, x, _positions(rng, r, slots, pos0, n_sink), data["perm"], quat, cb,
                  label=f"{dtype}/d{d}/b{bits}/{rot}/{quant}/rope{int(rope)}/perm{int(use_perm)}")


def test_append_llama3_cache_full_size():
    """The Llama-3 cache shape (128 rows, 32768 slots, 8 heads): one decode step for K and V
    at scattered positions (sinks included), checked on every appended row."""
    base = workloads.WORKLOADS["llama3"]
    rng = np.random.default_rng(77)
    for name in ("K", "V"):
        case = base.case(name)
        r, slots, h, d = case.shape
        data = workloads.synth_case(case.with_shape((r, 1, h, d)), 78, outliers=(3, 15.0))
        pos = rng.integers(0, slots, size=r).astype(np.int64)
        pos[:4] = [0, 1, 3, slots - 1]
        _check_append(case, data["input"][:, 0], pos, data["perm"], None, None, label=f"llama3.{name}")


def test_append_rejects_bad_arguments():
    case = workloads.TensorCase(name="X", shape=(2, 4, 2, 128), dtype="bf16", bits=2, group_size=128,
                                quant="minmax", rot="fwht", rope=False)
    cfg = gu.make_config(case)
    cache = kvq.empty_planes(cfg)
    x = torch.zeros((2, 2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        kvq.append(x, torch.zeros(3, dtype=torch.int64, device="cuda"), cache, cfg)
    with pytest.raises(kvq.KvqError):
        kvq.append(x[:, :, 1:], torch.zeros(2, dtype=torch.int64, device="cuda"), cache, cfg)  # misaligned x


def test_append_strided_input():
    """x given as a view with its own row and head strides (every other token of a wider tensor)."""
    r, slots, h, d = 6, 9, 3, 128
    case = workloads.TensorCase(name="K", shape=(r, slots, h, d), dtype="bf16", bits=2, group_size=128,
                                quant="minmax", rot="fwht", rope=True, n_sink=2, use_perm=True)
    data = workloads.synth_case(case.with_shape((r, 2, h, d)), 404)
    wide = gu.torch_input(data["input"], "bf16")          # [r, 2, h, d] contiguous
    x_view = wide[:, 1]                                    # row stride 2*h*d, head stride d
    cfg = gu.make_config(case, data["perm"], strides=(2 * h * d, 0, d))
    cache = _filled_planes(cfg)
    pos = torch.tensor([0, 1, 2, 8, 9, 4], dtype=torch.int64, device="cuda")
    kvq.append(x_view, pos, cache, cfg)
    # the same rows appended from a contiguous copy
    cfg_c = gu.make_config(case, data["perm"])
    cache_c = _filled_planes(cfg_c)
    kvq.append(x_view.contiguous(), pos, cache_c, cfg_c)
    torch.cuda.synchronize()
    for n in cache:
        assert torch.equal(cache[n].view(torch.uint8), cache_c[n].view(torch.uint8)), n
    _check_append(case, data["input"][:, 1], pos.cpu().numpy(), data["perm"], label="strided")
