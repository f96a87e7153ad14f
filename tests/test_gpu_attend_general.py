"""Decode-step attention on the general pass vs the CPU oracle: head_dim 256, K and V of
different bit widths and groups, 3-bit codes, no rotation, 8 query heads per KV head, and
caches whose slot 0 holds a position other than 0 (sink slots then shift or vanish).

As in the matrix-core tests, both sides read the same GPU-encoded planes: the oracle decodes
them in float64 and applies plain softmax attention (EliteKV page, section 7.1), the GPU
scores and sums in the rotated domain.  Tolerance: 1e-4 of the largest decoded value a row
attends over.
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

ATT_REL = 1e-4


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _compare(out_gpu, ref, vmax, label):
    err = np.abs(out_gpu.astype(np.float64) - ref)
    tol = ATT_REL * vmax[:, None, None] + 1e-6
    bad = err > tol
    assert not bad.any(), (f"{label}: attention differs by up to {err.max():.3g} "
                           f"(tolerance {tol.min():.3g}; {int(bad.sum())} elements)")
    return float(err.max())


def _case(shape, bits, g, rope, use_perm, n_sink, pos_offset, rot, name):
    return workloads.TensorCase(name=name, shape=shape, dtype="bf16", bits=bits, group_size=g, quant="minmax",
                                rot=rot, rope=rope, pos_offset=pos_offset, n_sink=n_sink, use_perm=use_perm)


# (head_dim, K bits, V bits, K group, V group, query heads per KV head, n_sink, pos_offset, rotation)
CASES = [
    (256, 2, 4, 32, 32, 2, 4, 0, "fwht"),     # the wide-head cache: K 2-bit, V 4-bit, groups of 32
    (256, 2, 4, 32, 32, 1, 0, 0, "fwht"),
    (256, 4, 4, 256, 256, 4, 2, 0, "fwht"),
    (256, 3, 3, 64, 64, 8, 0, 0, "fwht"),
    (256, 2, 2, 128, 64, 2, 4, 2, "none"),
    (128, 3, 3, 32, 32, 2, 4, 0, "fwht"),     # 3-bit codes
    (128, 3, 2, 128, 128, 1, 0, 0, "fwht"),
    (128, 2, 3, 64, 32, 4, 3, 0, "fwht"),     # K and V groups differ
    (128, 4, 2, 128, 128, 8, 4, 0, "fwht"),   # 8 query heads per KV head
    (128, 2, 2, 128, 128, 4, 4, 2, "fwht"),   # slot 0 = position 2: two sink slots
    (128, 2, 2, 128, 128, 4, 4, 100, "fwht"),  # every sink position before the cache
    (128, 2, 2, 64, 64, 2, 0, 0, "none"),     # no rotation
    (128, 4, 4, 32, 32, 1, 4, 0, "fwht"),     # 4-bit codes with small groups
]


@pytest.mark.parametrize("d,kb,vb,kg,vg,qg,n_sink,pos,rot", CASES)
def test_attend_general_small(d, kb, vb, kg, vg, qg, n_sink, pos, rot):
    r, t, h = 5, 203, 3
    seed = 3100 + d + 10 * kb + vb + kg + 3 * vg + 17 * qg + n_sink + pos + (5 if rot == "none" else 0)
    ck = _case((r, t, h, d), kb, kg, True, True, n_sink, pos, rot, "K")
    cv = _case((r, t, h, d), vb, vg, False, pos % 2 == 0, n_sink, pos, rot, "V")
    dk = workloads.synth_case(ck, seed)
    dv = workloads.synth_case(cv, seed + 1)
    cfg_k, cfg_v = gu.make_config(ck, dk["perm"]), gu.make_config(cv, dv["perm"])
    say(f"[case] attend general d={d} K{kb}/G{kg} V{vb}/G{vg} qg={qg} sinks={n_sink} pos_offset={pos} rot={rot}")
    pk_t = kvq.encode(gu.torch_input(dk["input"], "bf16"), cfg_k)
    pv_t = kvq.encode(gu.torch_input(dv["input"], "bf16"), cfg_v)
    rng = np.random.default_rng(seed + 2)
    q = rng.standard_normal((r, h * qg, d)).astype(np.float32)
    lengths = np.array([t, 1, 0, 3, 117], dtype=np.int32)
    out = kvq.attend(torch.from_numpy(q).cuda(), pk_t, cfg_k, pv_t, cfg_v, lengths=torch.from_numpy(lengths).cuda())
    torch.cuda.synchronize()
    kdec = oracle.decode(gu.planes_numpy(pk_t), parity.params_for(ck, dk["perm"]), ck.shape)
    vdec = oracle.decode(gu.planes_numpy(pv_t), parity.params_for(cv, dv["perm"]), cv.shape)
    ref = oracle.attend_decoded(q.astype(np.float64), kdec, vdec, lengths, d ** -0.5)
    vmax = np.array([np.abs(vdec[i, :max(int(lengths[i]), 1)]).max() for i in range(r)])
    o = out.cpu().numpy()
    e = _compare(o, ref, vmax, f"attend general d={d} K{kb} V{vb}")
    assert not o[2].any()  # length 0: zeros
    say(f"  max |err| {e:.3g}")


@pytest.mark.parametrize("t,qg,n_sink,pos,lengths", [
    (3, 1, 0, 0, [7, -3, 2, 1]),      # fewer slots than one step of 4; lengths past the cache and negative
    (5, 2, 6, 0, [5, 3, 0, 9]),       # every slot a sink
    (6, 8, 4, 3, [6, 1, 2, 5]),       # one sink slot (position 3), then codes
    (4, 4, 1, 0, [4, 4, 1, 2]),       # one step exactly
])
def test_attend_general_edge_shapes(t, qg, n_sink, pos, lengths):
    """Edge shapes at head_dim 256 (4 slots per step), K 2-bit and V 4-bit."""
    r, h, d = len(lengths), 2, 256
    seed = 3900 + 11 * t + qg + n_sink + pos
    ck = _case((r, t, h, d), 2, 32, True, False, n_sink, pos, "fwht", "K")
    cv = _case((r, t, h, d), 4, 32, False, False, n_sink, pos, "fwht", "V")
    dk = workloads.synth_case(ck, seed)
    dv = workloads.synth_case(cv, seed + 1)
    cfg_k, cfg_v = gu.make_config(ck), gu.make_config(cv)
    say(f"[case] attend general edge T={t} qg={qg} sinks={n_sink} pos_offset={pos} lengths={lengths}")
    pk_t = kvq.encode(gu.torch_input(dk["input"], "bf16"), cfg_k)
    pv_t = kvq.encode(gu.torch_input(dv["input"], "bf16"), cfg_v)
    q = np.random.default_rng(seed + 2).standard_normal((r, h * qg, d)).astype(np.float32)
    ln = np.array(lengths, dtype=np.int32)
    out = kvq.attend(torch.from_numpy(q).cuda(), pk_t, cfg_k, pv_t, cfg_v, lengths=torch.from_numpy(ln).cuda(),
                     scale=0.1)
    torch.cuda.synchronize()
    kdec = oracle.decode(gu.planes_numpy(pk_t), parity.params_for(ck), ck.shape)
    vdec = oracle.decode(gu.planes_numpy(pv_t), parity.params_for(cv), cv.shape)
    ref = oracle.attend_decoded(q.astype(np.float64), kdec, vdec, ln, 0.1)
    vmax = np.array([np.abs(vdec[i]).max() for i in range(r)])
    o = out.cpu().numpy()
    _compare(o, ref, vmax, f"attend general edge T={t}")
    for i, n in enumerate(lengths):
        if n <= 0:
            assert not o[i].any()


def test_attend_general_matches_noalloc():
    """The allocation-free entry point takes the general pass too (same kernels, static workspace)."""
    r, t, h, d = 3, 150, 2, 256
    ck = _case((r, t, h, d), 2, 32, True, False, 4, 0, "fwht", "K")
    cv = _case((r, t, h, d), 4, 32, False, False, 4, 0, "fwht", "V")
    dk, dv = workloads.synth_case(ck, 4001), workloads.synth_case(cv, 4002)
    cfg_k, cfg_v = gu.make_config(ck), gu.make_config(cv)
    say("[case] attend general vs attend_noalloc, wide-head shape reduced")
    pk_t = kvq.encode(gu.torch_input(dk["input"], "bf16"), cfg_k)
    pv_t = kvq.encode(gu.torch_input(dv["input"], "bf16"), cfg_v)
    q = torch.from_numpy(np.random.default_rng(4003).standard_normal((r, 2 * h, d)).astype(np.float32)).cuda()
    a = kvq.attend(q, pk_t, cfg_k, pv_t, cfg_v)
    b = kvq.attend_noalloc(q, pk_t, cfg_k, pv_t, cfg_v)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_attend_widehead_cache_full_size():
    """The wide-head cache (32 rows x 16384 slots x 16 KV heads x 256, K 2-bit and V 4-bit in
    groups of 32), 32 query heads: every row attended at its own length on the GPU, sampled
    rows checked against the oracle."""
    base = workloads.WORKLOADS["widehead"]
    data = workloads.device_workload("widehead", device=torch.device("cuda:0"))
    torch.cuda.synchronize()
    cases = {c.name: c for c in base.cases}
    cfgs = {n: gu.make_config(c, data["perm"]) for n, c in cases.items()}
    planes = {n: kvq.encode(data["inputs"][n], cfgs[n]) for n in cases}
    del data["inputs"]
    r, t, h, d = cases["K"].shape
    qg = 2
    rng = np.random.default_rng(93)
    q = rng.standard_normal((r, qg * h, d)).astype(np.float32)
    lengths = rng.integers(1, t + 1, size=r).astype(np.int32)
    lengths[:2] = [t, 3001]
    say(f"[case] attend wide-head full size: {r} rows x {t} slots x {h} KV heads, {qg * h} query heads")
    out = kvq.attend(torch.from_numpy(q).cuda(), planes["K"], cfgs["K"], planes["V"], cfgs["V"],
                     lengths=torch.from_numpy(lengths).cuda())
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    pk = parity.params_for(cases["K"], data["perm"])
    pv = parity.params_for(cases["V"], data["perm"])
    for row in (0, 1, 29):
        one = lambda n: {k: gu.planes_numpy({k: v[row:row + 1]})[k] for k, v in planes[n].items()}
        shape1 = (1, t, h, d)
        kdec = oracle.decode(one("K"), pk, shape1)
        vdec = oracle.decode(one("V"), pv, shape1)
        ln = lengths[row:row + 1]
        ref = oracle.attend_decoded(q[row:row + 1].astype(np.float64), kdec, vdec, ln, d ** -0.5)
        vmax = np.array([np.abs(vdec[0, :int(ln[0])]).max()])
        e = _compare(out[row:row + 1], ref, vmax, f"wide-head row {row} len {int(ln[0])}")
        say(f"  row {row} len {int(ln[0])}: max |err| {e:.3g}")
