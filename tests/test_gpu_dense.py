"""The dense-rotation codec on the GPU (fp32 matrix cores) vs the CPU oracle: the baselines the
IsoQuant page, section 1, sets SO(4) against -- a Haar-random orthogonal matrix (TurboQuant's
dense global transform) and 3-D rotors (RotorQuant), the latter given to the GPU as the
block-diagonal matrix the host builds (kvq_rotor_matrix) and to the oracle as quaternions
applied by sandwich products.  Same parity rules as the other rotations: codes bit-exact up to
rounding ties, scale/zero/norm within their windows, decode within 1e-3.
"""
from __future__ import annotations

import dataclasses
import sys
import zlib

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


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _rotation(kind, d, rng):
    """(float32 matrix for the GPU, oracle parameters) of a dense or rotor rotation."""
    if kind == "dense":
        m = workloads.haar_orthogonal(d, rng)
        return m, dict(rot="dense", rot_matrix=m.astype(np.float64))
    rq, ta = workloads.rotor_quaternions(d, rng)
    m = kvq.rotor_matrix(rq, d, ta)
    return m, dict(rot="rotor", rotor_quat=rq.astype(np.float64), rotor_tail=float(np.float32(ta)))


def run_dense(case, kind, seed, out_dtypes=("f32",), label=""):
    rng = np.random.default_rng(seed)
    d = case.shape[-1]
    data = workloads.synth_case(dataclasses.replace(case, rot="none"), seed)
    m, ora_rot = _rotation(kind, d, rng)
    cb = gu.codebook_for(case)
    say(f"[case] {label} {kind} shape={case.shape} dtype={case.dtype} bits={case.bits} G={case.group_size} "
        f"{case.quant} rope={case.rope} perm={case.use_perm} sink={case.n_sink} pos0={case.pos_offset}")
    mt = torch.from_numpy(m).cuda()
    cfg = kvq.Config(shape=case.shape, dtype=case.dtype, bits=case.bits, group_size=case.group_size,
                     quant=case.quant, rot="dense", rope=case.rope, pos_offset=case.pos_offset, n_sink=case.n_sink,
                     perm=data["perm"] if case.use_perm else None, codebook=cb, rot_matrix=mt)
    planes = kvq.encode(gu.torch_input(data["input"], case.dtype), cfg)
    torch.cuda.synchronize()
    g = gu.planes_numpy(planes)
    x64 = oracle.widen(data["input"], case.dtype)
    p = dataclasses.replace(parity.params_for(case, data["perm"], None, cb), **ora_rot)
    ora = oracle.encode(x64, p)
    if case.n_sink:
        ora["sink_f64"] = parity.sink_f64(x64, p)
    rep = parity.compare_encode(g, ora, p, case.shape, label)
    ref = oracle.decode(g, p, case.shape)
    for od in out_dtypes:
        y = kvq.decode(planes, cfg, out_dtype=od)
        torch.cuda.synchronize()
        yn = y.float().cpu().numpy() if od != "f32" else y.cpu().numpy()
        parity.compare_decode(yn, ref, od, f"{label} decode->{od}")
    return rep


# (dtype, bits, quant, group, rope, perm, n_sink, pos_offset, shape)
CASES = [
    ("f32", 3, "lloyd", 128, False, False, 0, 0, (1, 203, 1, 128)),   # the IsoQuant-style path, ragged
    ("bf16", 2, "minmax", 128, True, True, 4, 0, (2, 37, 3, 128)),    # Llama-style K: RoPE, permutation, sinks
    ("f16", 4, "minmax", 32, True, False, 2, 3, (2, 37, 3, 128)),
    ("bf16", 3, "minmax", 64, False, True, 0, 5, (3, 29, 2, 128)),
    ("f32", 2, "lloyd", 128, True, True, 3, 1, (2, 19, 4, 128)),
    ("f16", 4, "lloyd", 128, False, False, 0, 0, (1, 5, 3, 128)),     # 15 vectors: less than one item
    ("bf16", 4, "lloyd", 128, False, True, 1, 0, (3, 7, 1, 128)),     # 21 vectors: an item and a part
]


@pytest.mark.parametrize("kind", ["dense", "rotor"])
@pytest.mark.parametrize("dtype,bits,quant,g,rope,use_perm,n_sink,pos,shape", CASES)
def test_dense_small(kind, dtype, bits, quant, g, rope, use_perm, n_sink, pos, shape):
    seed = zlib.crc32(f"{kind}/{dtype}/{bits}/{quant}/{g}/{shape}".encode()) % 100000
    case = workloads.TensorCase(name="X", shape=shape, dtype=dtype, bits=bits, group_size=g, quant=quant,
                                rot=kind, rope=rope, n_sink=n_sink, use_perm=use_perm, pos_offset=pos,
                                lloyd_sigma=None)
    run_dense(case, kind, seed, out_dtypes=("f32", "bf16"), label=f"dense small")


@pytest.mark.parametrize("kind", ["dense", "rotor"])
def test_dense_isoquant_workload(kind):
    """The IsoQuant workload (8192 fp32 vectors, norm separation, 3-bit Lloyd-Max for N(0, 1/128))
    with the baseline rotations in place of SO(4): 512 items over the persistent blocks."""
    wl = workloads.WORKLOADS["isoquant"]
    case = dataclasses.replace(wl.case("X"), rot=kind)
    rep = run_dense(case, kind, 4242, out_dtypes=("f32",), label="isoquant workload")
    say(f"  {dict(rep)}")


def test_dense_many_items_per_block():
    """More items than the persistent grid holds at once (256 blocks x 8 waves): 2^17 vectors,
    every wave loops over several items; sampled against the oracle."""
    rng = np.random.default_rng(5150)
    d, r, t, h = 128, 4, 2048, 16
    case = workloads.TensorCase(name="X", shape=(r, t, h, d), dtype="bf16", bits=2, group_size=128,
                                quant="minmax", rot="dense", rope=True, n_sink=4, use_perm=True)
    m = workloads.haar_orthogonal(d, rng)
    perm = rng.permutation(d).astype(np.uint16)
    gen = torch.Generator(device="cuda").manual_seed(5151)
    x = torch.randn(case.shape, generator=gen, device="cuda").to(torch.bfloat16)
    cfg = kvq.Config(shape=case.shape, dtype="bf16", bits=2, group_size=128, rot="dense", rope=True, n_sink=4,
                     perm=perm, rot_matrix=torch.from_numpy(m).cuda())
    say(f"[case] dense many items: {case.shape}")
    planes = kvq.encode(x, cfg)
    y = kvq.decode(planes, cfg, out_dtype="f32")
    torch.cuda.synchronize()
    p = dataclasses.replace(parity.params_for(case, perm), rot_matrix=m.astype(np.float64))
    for row in (0, 3):
        for t0 in (0, 1333):
            sl = slice(t0, t0 + 64)
            xs = x[row:row + 1, sl].float().cpu().numpy().astype(np.float64)
            ps = dataclasses.replace(p, pos_offset=t0)
            ora = oracle.encode(xs, ps)
            if t0 < 4:
                ora["sink_f64"] = parity.sink_f64(xs, ps)
            g = gu.planes_numpy({k: v[row:row + 1, sl] if k != "sink" else v[row:row + 1] for k, v in planes.items()})
            parity.compare_encode(g, ora, ps, xs.shape, f"dense many row {row} t0 {t0}")
            ref = oracle.decode(g, ps, xs.shape)
            parity.compare_decode(y[row:row + 1, sl].cpu().numpy(), ref, "f32", f"dense many decode row {row} t0 {t0}")


# --------------------------------------------------------------------------- #
# RotorQuant's rotors computed as rotors (KVQ_ROT_ROTOR): the codec's vector-ALU kernels
# --------------------------------------------------------------------------- #
def run_rotor_native(case, seed, out_dtypes=("f32",), label=""):
    rng = np.random.default_rng(seed)
    d = case.shape[-1]
    data = workloads.synth_case(dataclasses.replace(case, rot="none"), seed)
    rq, ta = workloads.rotor_quaternions(d, rng)
    cb = gu.codebook_for(case)
    say(f"[case] {label} rotor shape={case.shape} dtype={case.dtype} bits={case.bits} G={case.group_size} "
        f"{case.quant} rope={case.rope} perm={case.use_perm} sink={case.n_sink} pos0={case.pos_offset}")
    cfg = kvq.Config(shape=case.shape, dtype=case.dtype, bits=case.bits, group_size=case.group_size,
                     quant=case.quant, rot="rotor", rope=case.rope, pos_offset=case.pos_offset, n_sink=case.n_sink,
                     perm=data["perm"] if case.use_perm else None, codebook=cb, rotor_quat=rq, rotor_tail=ta)
    planes = kvq.encode(gu.torch_input(data["input"], case.dtype), cfg)
    torch.cuda.synchronize()
    g = gu.planes_numpy(planes)
    x64 = oracle.widen(data["input"], case.dtype)
    p = dataclasses.replace(parity.params_for(case, data["perm"], None, cb), rot="rotor",
                            rotor_quat=rq.astype(np.float64), rotor_tail=ta)
    ora = oracle.encode(x64, p)
    if case.n_sink:
        ora["sink_f64"] = parity.sink_f64(x64, p)
    rep = parity.compare_encode(g, ora, p, case.shape, label)
    ref = oracle.decode(g, p, case.shape)
    for od in out_dtypes:
        y = kvq.decode(planes, cfg, out_dtype=od)
        torch.cuda.synchronize()
        yn = y.float().cpu().numpy() if od != "f32" else y.cpu().numpy()
        parity.compare_decode(yn, ref, od, f"{label} decode->{od}")
    return rep


ROTOR_CASES = CASES + [
    ("bf16", 2, "minmax", 32, True, True, 4, 0, (2, 37, 3, 256)),    # d = 256: 85 blocks and a 1-channel tail
    ("f32", 3, "lloyd", 256, False, False, 0, 0, (1, 61, 2, 256)),
    ("f16", 4, "minmax", 64, False, True, 2, 1, (2, 9, 5, 256)),
]


@pytest.mark.parametrize("dtype,bits,quant,g,rope,use_perm,n_sink,pos,shape", ROTOR_CASES)
def test_rotor_native_small(dtype, bits, quant, g, rope, use_perm, n_sink, pos, shape):
    seed = zlib.crc32(f"native/{dtype}/{bits}/{quant}/{g}/{shape}".encode()) % 100000
    case = workloads.TensorCase(name="X", shape=shape, dtype=dtype, bits=bits, group_size=g, quant=quant,
                                rot="rotor", rope=rope, n_sink=n_sink, use_perm=use_perm, pos_offset=pos)
    run_rotor_native(case, seed, out_dtypes=("f32", "bf16"), label="rotor native")


def test_rotor_native_isoquant_workload():
    wl = workloads.WORKLOADS["isoquant"]
    case = dataclasses.replace(wl.case("X"), rot="rotor")
    rep = run_rotor_native(case, 4343, label="rotor native isoquant workload")
    say(f"  {dict(rep)}")
