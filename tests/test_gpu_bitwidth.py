"""IsoQuant's dynamic bit width on the GPU against the CPU oracle: the attention entropy of
every query head over an encoded K cache, the per-head widths the host allocates from it, and
each head encoded at its own width.

Tolerance: entropies within 1e-4 + 1e-5 H nats (float32 scores over up to 32768 slots, the
same rounded keys on both sides: the oracle decodes the GPU's planes)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import workloads
from oracle import bitwidth as bw
from tests import gpu_util as gu
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rotate_then_bit_amd as kvq  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check(ent_gpu, ent_ora, label):
    err = np.abs(ent_gpu.astype(np.float64) - ent_ora)
    tol = 1e-4 + 1e-5 * np.abs(ent_ora)
    assert np.all(err <= tol), f"{label}: entropy differs by {err.max():.3g}"
    return float(err.max())


@pytest.mark.parametrize("shape,bits,g,qg,n_sink,perm", [
    ((4, 203, 3, 128), 2, 128, 4, 4, True),
    ((3, 150, 2, 256), 4, 32, 2, 0, False),
    ((2, 97, 2, 128), 3, 64, 8, 2, True),
    ((5, 64, 4, 256), 2, 256, 1, 3, False),
])
def test_attention_entropy(shape, bits, g, qg, n_sink, perm):
    r, t, h, d = shape
    say(f"[case] entropy {shape} {bits}-bit G={g} qg={qg} sinks={n_sink} perm={perm}")
    case = workloads.TensorCase(name="K", shape=shape, dtype="bf16", bits=bits, group_size=g, quant="minmax",
                                rot="fwht", rope=True, n_sink=n_sink, use_perm=perm)
    data = workloads.synth_case(case, 4000 + t, outliers=(3, 8.0), sink_token_scale=6.0)
    cfg = gu.make_config(case, data["perm"])
    planes = kvq.encode(gu.torch_input(data["input"], "bf16"), cfg)
    rng = np.random.default_rng(4100 + t)
    q = (rng.standard_normal((r, h * qg, d)) * rng.uniform(0.2, 3.0, (r, h * qg, 1))).astype(np.float32)
    lengths = np.array([t, 0, 1, min(n_sink, 2), t - 7][:r], dtype=np.int32)
    ent = kvq.attention_entropy(torch.from_numpy(q).cuda(), planes, cfg,
                                lengths=torch.from_numpy(lengths).cuda()).cpu().numpy()
    dec = oracle.decode(gu.planes_numpy(planes), parity.params_for(case, data["perm"]), shape)
    want = bw.attention_entropy(q.astype(np.float64), dec, lengths, d ** -0.5)
    say(f"  max err {_check(ent, want, str(shape)):.2e}; entropies {np.round(want.mean(1), 3).tolist()}")


def test_bits_per_head_from_entropy():
    """Entropy per KV head -> widths (host, equal to the oracle's) -> each head encoded at its
    own width through a head shard, matching the oracle's encode of that head."""
    r, t, h, d = 2, 120, 4, 128
    case = workloads.TensorCase(name="K", shape=(r, t, h, d), dtype="bf16", bits=2, group_size=128, quant="minmax",
                                rot="fwht", rope=True, n_sink=2, use_perm=True)
    data = workloads.synth_case(case, 4200, outliers=(3, 8.0))
    x = oracle.widen(data["input"], "bf16")
    x[..., 1, :] *= 4.0  # heads of different spread: their attention is more or less peaked
    raw = workloads.cast_host(x, "bf16")
    xt = gu.torch_input(raw, "bf16")
    cfg = gu.make_config(case, data["perm"])
    planes = kvq.encode(xt, cfg)
    q = torch.from_numpy(np.random.default_rng(4201).standard_normal((r, 2 * h, d)).astype(np.float32)).cuda()
    ent = kvq.attention_entropy(q, planes, cfg).cpu().numpy()
    e_head = bw.head_entropy(ent.astype(np.float64), h)
    bits = kvq.allocate_bits(e_head, 3 * h)
    assert np.array_equal(bits, bw.allocate_bits(e_head, 3 * h)) and bits.sum() == 12
    say(f"  head entropies {np.round(e_head, 3).tolist()} -> widths {bits.tolist()}")
    per = kvq.encode_heads(xt, cfg, bits)
    torch.cuda.synchronize()
    for i, (ci, pl) in enumerate(per):
        ch = case.with_shape((r, t, 1, d))
        ch = workloads.TensorCase(**{**ch.__dict__, "bits": int(bits[i])})
        p = parity.params_for(ch, data["perm"])
        xi = np.ascontiguousarray(x[:, :, i:i + 1])
        ora = oracle.encode(xi, p)
        ora["sink_f64"] = parity.sink_f64(xi, p)
        parity.compare_encode(gu.planes_numpy(pl), ora, p, ch.shape, f"head {i} at {bits[i]} bits")


def test_attention_entropy_full_size_rows():
    """Rows 0-1 of the Llama-3 cache (32768 slots, 8 KV heads, 32 query heads)."""
    data = workloads.device_workload("llama3", names=("K",))
    torch.cuda.synchronize()
    case = workloads.WORKLOADS["llama3"].case("K")
    k = data["inputs"]["K"][:2]
    cfg = gu.make_config(case.with_shape(k.shape), data["perm"])
    planes = kvq.encode(k, cfg)
    q = torch.randn((2, 32, 128), generator=torch.Generator(device="cuda").manual_seed(7), device="cuda")
    lengths = torch.tensor([32768, 20001], dtype=torch.int32, device="cuda")
    ent = kvq.attention_entropy(q, planes, cfg, lengths=lengths).cpu().numpy()
    p = parity.params_for(case.with_shape(k.shape), data["perm"])
    dec = oracle.decode(gu.planes_numpy(planes), p, tuple(k.shape))
    want = bw.attention_entropy(q.cpu().numpy().astype(np.float64), dec, lengths.cpu().numpy(), 128 ** -0.5)
    say(f"[full] llama3 rows 0-1: max err {_check(ent, want, 'llama3'):.2e}, mean entropy {want.mean():.4f}")
