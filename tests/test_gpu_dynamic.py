"""IsoQuant's dynamic codebook on the GPU against the CPU oracle: rotated-channel moments of
a calibration slice, the codebook the host derives from them, and the codec (encode, decode,
append) with per-channel scales and the wider codebook on the outlier channels.

Tolerances: moments are float64 sums of float32 rotated values (each within a few float32
ulps of the unit direction), 1e-4 relative; codes bit-exact except where the normalised value
lies within 1e-4 of a level gap of a threshold of its channel's codebook (the Lloyd-Max rule);
decode within 1e-3 absolute, both decoders reading the same GPU planes.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import workloads
from oracle import codec as ocodec
from tests import gpu_util as gu
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rotate_then_bit_amd as kvq  # noqa: E402

MOM_REL = 1e-4


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = [  # shape, dtype, bits, rot, rope, perm, n_sink
    ((1, 700, 1, 128), "f32", 3, "so4", False, False, 0),
    ((2, 150, 4, 128), "bf16", 2, "fwht", True, True, 3),
    ((1, 90, 3, 256), "f16", 4, "fwht", False, True, 0),
    ((2, 64, 2, 256), "f32", 3, "so4", True, False, 2),
    ((1, 80, 2, 128), "bf16", 3, "none", False, False, 0),
]


def _setup(shape, dtype, bits, rot, rope, use_perm, n_sink, seed):
    case = workloads.TensorCase(name="X", shape=shape, dtype=dtype, bits=bits, group_size=shape[-1], quant="lloyd",
                                rot=rot, rope=rope, n_sink=n_sink, use_perm=use_perm)
    data = workloads.synth_case(case, seed, outliers=(4, 6.0))
    d = shape[-1]
    # channels of unequal spread, so that the per-channel scales differ
    x = oracle.widen(data["input"], dtype) * np.exp(np.random.default_rng(seed + 1).uniform(-1.0, 1.0, d))
    raw = workloads.cast_host(x, dtype)
    cb0 = oracle.fit_gaussian(bits, 1.0).astype(np.float32)
    cfg0 = gu.make_config(case, data["perm"], data["quat"], cb0)
    return case, data, raw, cfg0


@pytest.mark.parametrize("shape,dtype,bits,rot,rope,use_perm,n_sink", CASES)
def test_dynamic_codebook_codec(shape, dtype, bits, rot, rope, use_perm, n_sink):
    seed = 3000 + shape[1] + bits
    say(f"[case] dynamic codebook {shape} {dtype} {bits}-bit {rot} rope={rope} perm={use_perm} sinks={n_sink}")
    case, data, raw, cfg0 = _setup(shape, dtype, bits, rot, rope, use_perm, n_sink, seed)
    xt = gu.torch_input(raw, dtype)
    x64 = oracle.widen(raw, dtype)
    p0 = parity.params_for(case, data["perm"], data["quat"], cfg0.codebook)
    # online statistics: moments of the rotated unit directions
    m_gpu = kvq.rotated_moments(xt, cfg0).cpu().numpy()
    m_ora = ocodec.rotated_moments(x64, p0)
    assert np.all(np.abs(m_gpu - m_ora) <= MOM_REL * m_ora), np.max(np.abs(m_gpu - m_ora) / m_ora)
    # the codebook from the GPU's moments (host), then the codec with it on both sides
    sc, wide, cb, cbw = kvq.dynamic_codebook(m_gpu, bits)
    cfg = kvq.Config(**{**cfg0.__dict__, "codebook": cb, "chan_scale": sc, "chan_wide": wide, "codebook_wide": cbw,
                        "_keep": []})
    planes = kvq.encode(xt, cfg)
    y = kvq.decode(planes, cfg, out_dtype="f32")
    torch.cuda.synchronize()
    g = gu.planes_numpy(planes)
    p = ocodec.CodecParams(**{**p0.__dict__, "codebook": cb.astype(np.float64), "chan_scale": sc.astype(np.float64),
                              "chan_wide": wide.astype(bool), "codebook_wide": cbw.astype(np.float64)})
    ora = oracle.encode(x64, p)
    ora["sink_f64"] = parity.sink_f64(x64, p)
    rep = parity.compare_encode(g, ora, p, case.shape, f"dynamic {shape}")
    dec = oracle.decode(g, p, case.shape)
    err = parity.compare_decode(y.cpu().numpy(), dec, "f32", f"dynamic decode {shape}")
    say(f"  {dict(rep)} decode err {err:.2e}; wide channels {np.nonzero(wide)[0].tolist()}")


def test_dynamic_codebook_append():
    """kvq_append with the dynamic codebook writes the same slots (codes, norm, extra, sinks)
    as the oracle's append, and leaves every other byte alone."""
    shape = (3, 20, 2, 128)
    case, data, raw, cfg0 = _setup(shape, "bf16", 3, "fwht", True, True, 4, 3100)
    xt = gu.torch_input(raw, "bf16")
    sc, wide, cb, cbw = kvq.dynamic_codebook(kvq.rotated_moments(xt, cfg0).cpu().numpy(), 3)
    cfg = kvq.Config(**{**cfg0.__dict__, "codebook": cb, "chan_scale": sc, "chan_wide": wide, "codebook_wide": cbw,
                        "_keep": []})
    cache = gu.poison_planes(kvq.empty_planes(cfg), 0x5A)
    positions = np.array([2, 11, 25], dtype=np.int64)  # a sink, an ordinary slot, no slot
    x_new = raw[:, 0]
    kvq.append(gu.torch_input(np.ascontiguousarray(x_new), "bf16"), torch.from_numpy(positions).cuda(), cache, cfg)
    torch.cuda.synchronize()
    g = gu.planes_numpy(cache)
    p = ocodec.CodecParams(**{**parity.params_for(case, data["perm"], data["quat"], cb).__dict__,
                              "codebook": cb.astype(np.float64), "chan_scale": sc.astype(np.float64),
                              "chan_wide": wide.astype(bool), "codebook_wide": cbw.astype(np.float64)})
    before = {k: np.full(v.nbytes, 0x5A, dtype=np.uint8).view(v.dtype).reshape(v.shape) for k, v in g.items()}
    want = ocodec.append(before, oracle.widen(x_new, "bf16"), positions, p)
    for k in g:
        assert np.array_equal(g[k].view(np.uint8), want[k].view(np.uint8)), k
