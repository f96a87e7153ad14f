"""kvq_attend_noalloc (static device workspace) against kvq_attend (caller's workspace) on
the GPU: two calls in a row, the second on a smaller cache, each bit-identical to
kvq_attend on the same inputs; a cache too large for the static workspace is refused on
the host.  Both entry points run the same kernels, so their outputs must agree exactly."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rotate_then_bit_amd as kvq  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _cache(r, t, h, bits, g, n_sink, seed):
    ck = workloads.TensorCase(name="K", shape=(r, t, h, 128), dtype="bf16", bits=bits, group_size=g,
                              quant="minmax", rot="fwht", rope=True, n_sink=n_sink, use_perm=True)
    cv = workloads.TensorCase(name="V", shape=(r, t, h, 128), dtype="bf16", bits=bits, group_size=g,
                              quant="minmax", rot="fwht", rope=False, n_sink=n_sink, use_perm=False)
    dk, dv = workloads.synth_case(ck, seed), workloads.synth_case(cv, seed + 1)
    cfg_k, cfg_v = gu.make_config(ck, dk["perm"]), gu.make_config(cv, dv["perm"])
    pk = kvq.encode(gu.torch_input(dk["input"], "bf16"), cfg_k)
    pv = kvq.encode(gu.torch_input(dv["input"], "bf16"), cfg_v)
    return cfg_k, pk, cfg_v, pv


def test_noalloc_matches_attend_twice_second_smaller():
    cases = [  # (rows, slots, KV heads, query heads per KV head, bits, group, sinks)
        (24, 4100, 8, 4, 2, 128, 4),   # block-cooperative matrix-core pass, several chunks
        (3, 203, 3, 2, 4, 64, 2),      # smaller: vector-ALU pass
    ]
    prev_need = None
    for i, (r, t, h, qg, bits, g, ns) in enumerate(cases):
        say(f"[case] noalloc call {i}: cache=({r},{t},{h},128) qg={qg} bits={bits} G={g} sinks={ns}")
        cfg_k, pk, cfg_v, pv = _cache(r, t, h, bits, g, ns, 900 + 10 * i)
        need = kvq.attend_workspace_size(cfg_k, h * qg)
        assert need <= kvq.attend_noalloc_max_workspace()
        if prev_need is not None:
            assert need < prev_need  # the second call is the smaller one
        prev_need = need
        rng = np.random.default_rng(950 + i)
        q = torch.from_numpy(rng.standard_normal((r, h * qg, 128)).astype(np.float32)).cuda()
        lengths = torch.from_numpy(rng.integers(0, t + 1, r).astype(np.int32)).cuda()
        lengths[0] = t
        ref = kvq.attend(q, pk, cfg_k, pv, cfg_v, lengths=lengths)
        out = torch.full_like(q, float("nan"))
        kvq.attend_noalloc(q, pk, cfg_k, pv, cfg_v, lengths=lengths, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"call {i}: differs by {float((out - ref).abs().max()):.3g}"
        say(f"  call {i} identical to kvq_attend ({need} workspace bytes)")


def test_noalloc_refuses_a_cache_above_its_workspace():
    r, t, h = 1024, 32768, 8
    cfg = kvq.Config(shape=(r, t, h, 128), dtype="bf16", bits=2, group_size=128, rot="fwht")
    need = kvq.attend_workspace_size(cfg, 4 * h)
    assert need > kvq.attend_noalloc_max_workspace()
    # plane pointers are checked before the workspace: give aligned non-null stand-ins that
    # the refusal below keeps from ever being used
    import ctypes
    lib = ctypes.CDLL(kvq.library_path())
    lib.kvq_attend_noalloc.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64, ctypes.c_void_p, ctypes.c_float,
                                                               ctypes.c_void_p, ctypes.c_void_p]
    pl = kvq._Planes()
    pl.codes, pl.scale, pl.zero = 4096, 8192, 12288
    c = cfg.c_struct()
    st = lib.kvq_attend_noalloc(ctypes.byref(c), ctypes.byref(pl), ctypes.byref(c), ctypes.byref(pl), 4096,
                                4 * h, None, 0.1, 4096, None)
    assert st == 2
    lib.kvq_last_error_message.restype = ctypes.c_char_p
    assert b"noalloc" in lib.kvq_last_error_message()
