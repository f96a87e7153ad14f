"""Calibration of the RotateKV variants on the GPU against the CPU oracle: per-channel
statistics for the outlier-aware permutation (and the codec run with the permutation they
give), and activation-based sink detection.

Tolerances: statistics are float64 sums of float32 post-RoPE values, so they agree with the
float64 oracle within 1e-5 relative (the RoPE'd values carry a few float32 ulps of the pair
norm); token norms are float64 sums of exact squares, 1e-12 relative; a flag may differ only
where the norm is within 1e-9 relative of lambda times the median (none occur here).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import workloads
from oracle import calibration as cal
from tests import gpu_util as gu
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rotate_then_bit_amd as kvq  # noqa: E402

STATS_REL = 1e-5
NORM_REL = 1e-12


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(shape, dtype, rope, n_sink=0, pos_offset=0, g=128, bits=2):
    return workloads.TensorCase(name="K", shape=shape, dtype=dtype, bits=bits, group_size=g, quant="minmax",
                                rot="fwht", rope=rope, n_sink=n_sink, pos_offset=pos_offset, use_perm=False)


STAT_CASES = [  # shape, dtype, rope, n_sink, pos_offset
    ((2, 203, 8, 128), "bf16", True, 4, 0),
    ((3, 77, 3, 128), "f16", False, 0, 0),
    ((1, 1000, 2, 128), "f32", True, 2, 5),
    ((2, 45, 4, 256), "bf16", True, 0, 31),
    ((1, 3, 1, 256), "f32", False, 5, 0),     # every token a sink: statistics 0
    ((2, 0, 4, 128), "bf16", True, 0, 0),     # empty slice
]


@pytest.mark.parametrize("shape,dtype,rope,n_sink,pos_offset", STAT_CASES)
def test_channel_stats(shape, dtype, rope, n_sink, pos_offset):
    case = _case(shape, dtype, rope, n_sink, pos_offset)
    say(f"[case] channel_stats {shape} {dtype} rope={rope} sinks={n_sink} pos_offset={pos_offset}")
    data = workloads.synth_case(case, 2000 + shape[1], outliers=(5, 12.0))
    cfg = gu.make_config(case)
    got = kvq.channel_stats(gu.torch_input(data["input"], dtype), cfg).cpu().numpy()
    want = cal.channel_stats(oracle.widen(data["input"], dtype), rope, 10000.0, pos_offset, n_sink)
    assert np.all(np.abs(got - want) <= STATS_REL * np.abs(want) + 1e-30), np.abs(got - want).max()


def test_channel_stats_strided_head_shard():
    full = _case((2, 60, 8, 128), "bf16", True, 4)
    data = workloads.synth_case(full, 2101)
    xt = gu.torch_input(data["input"], "bf16")
    shard = xt[:, :, 3:5, :]
    case = full.with_shape((2, 60, 2, 128))
    cfg = gu.make_config(case, strides=shard.stride()[:3])
    got = kvq.channel_stats(shard, cfg).cpu().numpy()
    want = cal.channel_stats(oracle.widen(np.ascontiguousarray(data["input"][:, :, 3:5]), "bf16"), True, 10000.0, 0, 4)
    assert np.all(np.abs(got - want) <= STATS_REL * np.abs(want))


@pytest.mark.parametrize("g", [32, 128])
def test_calibrated_perm_codec_parity(g):
    """Statistics -> outlier-aware permutation (host) -> codec: the permutation equals the
    oracle's for the same statistics, and the codec with it matches the oracle's encode."""
    case = workloads.TensorCase(name="K", shape=(2, 150, 8, 128), dtype="bf16", bits=2, group_size=g,
                                quant="minmax", rot="fwht", rope=True, n_sink=4, use_perm=True)
    data = workloads.synth_case(case, 2200 + g, outliers=(4, 15.0))
    xt = gu.torch_input(data["input"], "bf16")
    stats = kvq.channel_stats(xt, gu.make_config(case.with_shape(case.shape))).cpu().numpy()
    perm = kvq.outlier_perm(stats, g)
    assert np.array_equal(perm, cal.outlier_perm(stats, g))
    x64 = oracle.widen(data["input"], "bf16")
    want = cal.channel_stats(x64, True, 10000.0, 0, 4)
    assert np.array_equal(perm, cal.outlier_perm(want, g))  # no near-tie decides the order here
    cfg = gu.make_config(case, perm)
    planes = kvq.encode(xt, cfg)
    torch.cuda.synchronize()
    p = parity.params_for(case, perm)
    ora = oracle.encode(x64, p)
    ora["sink_f64"] = parity.sink_f64(x64, p)
    say(f"  {dict(parity.compare_encode(gu.planes_numpy(planes), ora, p, case.shape, f'calibrated perm G={g}'))}")


def _check_sinks(x_raw, dtype, shape, lam, label, strides=None, xt=None):
    case = _case(shape, dtype, False)
    cfg = gu.make_config(case, strides=strides)
    if xt is None:
        xt = gu.torch_input(x_raw, dtype)
    norms, flags, counts, prefix, med = (v.cpu().numpy() for v in kvq.detect_sinks(xt, cfg, lam))
    x64 = oracle.widen(x_raw, dtype)
    want_n = cal.token_norms(x64)
    assert np.all(np.abs(norms - want_n) <= NORM_REL * want_n), f"{label}: norms"
    f_o, c_o, p_o = cal.detect_sinks(x64, lam)
    r, t = shape[:2]
    for i in range(r):
        if t == 0:
            assert counts[i] == 0 and prefix[i] == 0
            continue
        assert med[i] == np.sort(norms[i])[(t - 1) // 2], f"{label}: median is not the rank element"
        near = np.abs(want_n[i] - lam * cal.lower_median(want_n[i])) <= 1e-9 * want_n[i]
        assert np.array_equal(flags[i].astype(bool) | near, f_o[i] | near), f"{label}: flags row {i}"
        assert counts[i] == int(flags[i].sum())
        fl = np.nonzero(flags[i])[0]
        assert prefix[i] == (fl.max() + 1 if fl.size else 0)
    return flags, counts, prefix


@pytest.mark.parametrize("shape,dtype", [((3, 101, 8, 128), "bf16"), ((2, 64, 3, 256), "f16"),
                                         ((2, 1, 2, 128), "f32"), ((1, 2, 4, 128), "bf16"),
                                         ((4, 0, 8, 128), "bf16"),
                                         ((1, 40000, 1, 128), "bf16")])  # rows longer than the register-held 32768
def test_detect_sinks(shape, dtype):
    say(f"[case] detect_sinks {shape} {dtype}")
    case = _case(shape, dtype, False)
    data = workloads.synth_case(case, 2300 + shape[1], outliers=(3, 15.0))
    x = oracle.widen(data["input"], dtype)
    if shape[1] > 5:
        x[:, 0] *= 50.0  # a massive-activation token and a milder one
        x[:, 5] *= 9.0
    raw = workloads.cast_host(x, dtype)
    flags, counts, prefix = _check_sinks(raw, dtype, shape, 8.0, f"sinks {shape}")
    if shape[1] > 5:
        assert flags[:, 0].all() and flags[:, 5].all() and (prefix == 6).all()


def test_detect_sinks_strided_shard():
    full = _case((2, 90, 8, 128), "bf16", False)
    data = workloads.synth_case(full, 2400)
    x = oracle.widen(data["input"], "bf16")
    x[:, 2] *= 30.0
    raw = workloads.cast_host(x, "bf16")
    xt = gu.torch_input(raw, "bf16")
    shard = xt[:, :, 2:6, :]
    flags, _, prefix = _check_sinks(np.ascontiguousarray(raw[:, :, 2:6]), "bf16", (2, 90, 4, 128), 8.0, "shard",
                                    strides=shard.stride()[:3], xt=shard)
    assert (prefix == 3).all()


def test_calibration_full_size_rows():
    """The Llama-3 cache drawn on the GPU: statistics of rows 0-1 (post-RoPE K, sinks left
    out) and sink detection over rows 0-3, against the oracle on the same rows; the Llama-2
    layer's x50 token 0 is the only detected sink of its K (prefix 1)."""
    data = workloads.device_workload("llama3", names=("K",))
    torch.cuda.synchronize()
    k = data["inputs"]["K"]
    case = workloads.WORKLOADS["llama3"].case("K")
    sl = k[:2]
    cfg = gu.make_config(case.with_shape(sl.shape), data["perm"])
    got = kvq.channel_stats(sl, cfg).cpu().numpy()
    raw = gu.raw_numpy(sl, "bf16")
    want = cal.channel_stats(oracle.widen(raw, "bf16"), True, 10000.0, 0, 4)
    assert np.all(np.abs(got - want) <= STATS_REL * want)
    say(f"[full] llama3 K statistics rows 0-1: top channels {np.argsort(-got)[:4].tolist()}")
    sl4 = k[:4]
    _check_sinks(gu.raw_numpy(sl4, "bf16"), "bf16", tuple(sl4.shape), 8.0, "llama3 rows 0-3", xt=sl4)
    del data, k, sl, sl4
    torch.cuda.empty_cache()
    h = workloads.host_workload("llama2")
    raw2 = h["inputs"]["K"]
    flags, counts, prefix = _check_sinks(raw2, "f16", raw2.shape, 8.0, "llama2 K")
    assert prefix.tolist() == [1] and counts.tolist() == [1]
