"""Decode-step attention over the encoded cache on the GPU vs the CPU oracle.

Both sides read the same GPU-encoded planes; the oracle decodes them in float64 and
applies plain softmax attention, while the GPU never decodes a key (rotated-domain
scores) and sums the values in the rotated domain.  Tolerance: 1e-4 of the largest
decoded value a row attends over (fp32 scores and sums over up to 32768 slots).
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


def _case(r, t, h, bits, g, rope, use_perm, n_sink, name):
    return workloads.TensorCase(name=name, shape=(r, t, h, 128), dtype="bf16", bits=bits, group_size=g,
                                quant="minmax", rot="fwht", rope=rope, n_sink=n_sink, use_perm=use_perm)


@pytest.mark.parametrize("qg,bits,g,n_sink,perm_v,h", [
    (4, 2, 128, 4, False, 3),   # Llama-3 shape of K and V, reduced
    (1, 2, 64, 0, True, 3),
    (2, 4, 32, 3, False, 3),
    (4, 4, 64, 0, True, 3),
    (2, 2, 32, 4, True, 3),
    (1, 2, 128, 0, True, 3),    # matrix-core partial pass with one and two query heads per KV head
    (2, 2, 128, 2, False, 3),
    (4, 2, 128, 4, False, 8),   # block-cooperative matrix-core pass (KV heads a multiple of 4)
    (1, 2, 128, 0, True, 4),
    (2, 2, 128, 2, False, 4),
    (4, 4, 128, 4, False, 4),   # 4-bit codes on the block-cooperative pass
    (2, 4, 128, 0, True, 8),
])
def test_attend_small(qg, bits, g, n_sink, perm_v, h):
    r, t = 5, 203
    seed = 500 + 10 * qg + bits + g + n_sink + (7 if perm_v else 0) + 1000 * (h - 3)
    ck = _case(r, t, h, bits, g, True, True, n_sink, "K")
    cv = _case(r, t, h, bits, g, False, perm_v, n_sink, "V")
    dk = workloads.synth_case(ck, seed)
    dv = workloads.synth_case(cv, seed + 1)
    cfg_k = gu.make_config(ck, dk["perm"])
    cfg_v = gu.make_config(cv, dv["perm"])
    say(f"[case] attend qg={qg} bits={bits} G={g} sinks={n_sink} perm_v={perm_v} cache={ck.shape}")
    pk_t = kvq.encode(gu.torch_input(dk["input"], "bf16"), cfg_k)
    pv_t = kvq.encode(gu.torch_input(dv["input"], "bf16"), cfg_v)
    rng = np.random.default_rng(seed + 2)
    q = rng.standard_normal((r, h * qg, 128)).astype(np.float32)
    lengths = np.array([t, 1, 0, min(n_sink, 2), 117], dtype=np.int32)
    out = kvq.attend(torch.from_numpy(q).cuda(), pk_t, cfg_k, pv_t, cfg_v,
                     lengths=torch.from_numpy(lengths).cuda())
    torch.cuda.synchronize()
    gk, gv = gu.planes_numpy(pk_t), gu.planes_numpy(pv_t)
    pk = parity.params_for(ck, dk["perm"])
    pv = parity.params_for(cv, dv["perm"])
    kdec = oracle.decode(gk, pk, ck.shape)
    vdec = oracle.decode(gv, pv, cv.shape)
    ref = oracle.attend_decoded(q.astype(np.float64), kdec, vdec, lengths, 128 ** -0.5)
    vmax = np.array([np.abs(vdec[i, :max(int(lengths[i]), 1)]).max() for i in range(r)])
    e = _compare(out.cpu().numpy(), ref, vmax, f"attend qg={qg} b={bits} G={g}")
    assert not out.cpu().numpy()[2].any()  # length 0: zeros
    say(f"  max |err| {e:.3g}")


def test_attend_llama3_cache_full_size():
    """The Llama-3 cache shape (128 rows x 32768 slots x 8 KV heads, 32 query heads): every
    row attended at its own length on the GPU, sampled rows checked against the oracle."""
    base = workloads.WORKLOADS["llama3"]
    data = workloads.device_workload("llama3", device=torch.device("cuda:0"))
    torch.cuda.synchronize()
    cases = {c.name: c for c in base.cases}
    cfgs = {n: kvq.Config(shape=c.shape, dtype=c.dtype, bits=c.bits, group_size=c.group_size, rope=c.rope,
                          rope_base=c.rope_base, n_sink=c.n_sink, perm=data["perm"] if c.use_perm else None)
            for n, c in cases.items()}
    planes = {n: kvq.encode(data["inputs"][n], cfgs[n]) for n in cases}
    del data["inputs"]
    r, t, h, d = cases["K"].shape
    rng = np.random.default_rng(91)
    q = rng.standard_normal((r, 4 * h, d)).astype(np.float32)
    lengths = rng.integers(1, t + 1, size=r).astype(np.int32)
    lengths[:3] = [t, 5, 4000]
    say(f"[case] attend llama3 full size: {r} rows x {t} slots x {h} KV heads, {4 * h} query heads")
    out = kvq.attend(torch.from_numpy(q).cuda(), planes["K"], cfgs["K"], planes["V"], cfgs["V"],
                     lengths=torch.from_numpy(lengths).cuda())
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    pk = parity.params_for(cases["K"], data["perm"])
    pv = parity.params_for(cases["V"], data["perm"])
    for row in (0, 1, 2, 77):
        one = lambda n: {k: gu.planes_numpy({k: v[row:row + 1]})[k] for k, v in planes[n].items()}
        shape1 = (1, t, h, d)
        kdec = oracle.decode(one("K"), pk, shape1)
        vdec = oracle.decode(one("V"), pv, shape1)
        ln = lengths[row:row + 1]
        ref = oracle.attend_decoded(q[row:row + 1].astype(np.float64), kdec, vdec, ln, d ** -0.5)
        vmax = np.array([np.abs(vdec[0, :int(ln[0])]).max()])
        e = _compare(out[row:row + 1], ref, vmax, f"llama3 row {row} len {int(ln[0])}")
        say(f"  row {row} len {int(ln[0])}: max |err| {e:.3g}")



@pytest.mark.parametrize("h,bits", [(6, 2), (8, 2), (8, 4)])
def test_attend_several_windows_per_chunk(h, bits):
    """A cache with enough rows that each chunk spans many windows of the matrix-core pass (the
    last one partial at the ragged lengths), for the per-wave pass (6 KV heads) and the
    block-cooperative one (8; 2- and 4-bit codes): inputs drawn on the GPU, sampled rows
    checked against the oracle."""
    r, t = 96, 4096
    seed = 7100 + h + 10 * bits
    ck = _case(r, t, h, bits, 128, True, True, 4, "K")
    cv = _case(r, t, h, bits, 128, False, False, 4, "V")
    perm = np.random.default_rng(seed).permutation(128).astype(np.int64)
    cfg_k, cfg_v = gu.make_config(ck, perm), gu.make_config(cv, None)
    gen = torch.Generator(device="cuda").manual_seed(seed)
    xk = torch.randn((r, t, h, 128), generator=gen, device="cuda").to(torch.bfloat16)
    xv = torch.randn((r, t, h, 128), generator=gen, device="cuda").to(torch.bfloat16)
    pk_t, pv_t = kvq.encode(xk, cfg_k), kvq.encode(xv, cfg_v)
    del xk, xv
    rng = np.random.default_rng(seed + 1)
    q = rng.standard_normal((r, 4 * h, 128)).astype(np.float32)
    lengths = rng.integers(1, t + 1, size=r).astype(np.int32)
    lengths[:2] = [t, 1000]
    say(f"[case] attend several windows per chunk: {r} x {t} x {h} heads, {bits}-bit")
    out = kvq.attend(torch.from_numpy(q).cuda(), pk_t, cfg_k, pv_t, cfg_v, lengths=torch.from_numpy(lengths).cuda())
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    pk, pv = parity.params_for(ck, perm), parity.params_for(cv, None)
    for row in (0, 1, 50):
        one = lambda pl: {k: gu.planes_numpy({k: v[row:row + 1]})[k] for k, v in pl.items()}
        kdec = oracle.decode(one(pk_t), pk, (1, t, h, 128))
        vdec = oracle.decode(one(pv_t), pv, (1, t, h, 128))
        ln = lengths[row:row + 1]
        ref = oracle.attend_decoded(q[row:row + 1].astype(np.float64), kdec, vdec, ln, 128 ** -0.5)
        vmax = np.array([np.abs(vdec[0, :int(ln[0])]).max()])
        e = _compare(out[row:row + 1], ref, vmax, f"two windows row {row} len {int(ln[0])}")
        say(f"  row {row} len {int(ln[0])}: max |err| {e:.3g}")

@pytest.mark.parametrize("t,h,qg,n_sink,lengths", [
    (5, 1, 1, 0, [7, -3, 5, 2]),      # fewer slots than one step; lengths past the cache and negative
    (5, 2, 2, 6, [5, 3, 0, 9]),       # every slot a sink
    (9, 1, 4, 1, [9, 8, 1, 2]),       # one step plus one slot
    (5, 4, 1, 0, [7, -3, 5, 2]),      # the same on the block-cooperative matrix-core pass (4 KV heads)
    (9, 4, 4, 1, [9, 8, 1, 2]),
    (5, 8, 2, 6, [5, 3, 0, 9]),
])
def test_attend_edge_shapes(t, h, qg, n_sink, lengths):
    r = len(lengths)
    seed = 900 + 13 * t + h + qg + n_sink
    ck = _case(r, t, h, 2, 128, True, True, n_sink, "K")
    cv = _case(r, t, h, 2, 128, False, False, n_sink, "V")
    dk = workloads.synth_case(ck, seed)
    dv = workloads.synth_case(cv, seed + 1)
    cfg_k, cfg_v = gu.make_config(ck, dk["perm"]), gu.make_config(cv, None)
    say(f"[case] attend edge T={t} H={h} qg={qg} sinks={n_sink} lengths={lengths}")
    pk_t = kvq.encode(gu.torch_input(dk["input"], "bf16"), cfg_k)
    pv_t = kvq.encode(gu.torch_input(dv["input"], "bf16"), cfg_v)
    q = np.random.default_rng(seed + 2).standard_normal((r, h * qg, 128)).astype(np.float32)
    ln = np.array(lengths, dtype=np.int32)
    out = kvq.attend(torch.from_numpy(q).cuda(), pk_t, cfg_k, pv_t, cfg_v, lengths=torch.from_numpy(ln).cuda(),
                     scale=0.2)
    torch.cuda.synchronize()
    kdec = oracle.decode(gu.planes_numpy(pk_t), parity.params_for(ck, dk["perm"]), ck.shape)
    vdec = oracle.decode(gu.planes_numpy(pv_t), parity.params_for(cv, None), cv.shape)
    ref = oracle.attend_decoded(q.astype(np.float64), kdec, vdec, ln, 0.2)
    vmax = np.array([np.abs(vdec[i]).max() for i in range(r)])
    _compare(out.cpu().numpy(), ref, vmax, f"attend edge T={t}")
    for i, n in enumerate(lengths):
        if n <= 0:
            assert not out.cpu().numpy()[i].any()
