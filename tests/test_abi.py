"""The C ABI on the host (no GPU): the library loads, exports every symbol the header
declares, validates configurations synchronously and returns the documented status
codes, and reports plane sizes.  Nothing here launches a kernel."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import ROOT

kvq = pytest.importorskip("rotate_then_bit_amd")

HEADER = os.path.join(ROOT, "include", "kvq.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", src)))


def test_header_declares_the_binding_symbols():
    assert header_functions() == sorted(kvq.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(kvq.library_path())
    for name in header_functions():
        assert hasattr(lib, name), name
    assert kvq.abi_version() == 1


def _cfg(**kw):
    base = dict(shape=(2, 8, 4, 128), dtype="bf16", bits=2, group_size=128)
    base.update(kw)
    return kvq.Config(**base)


BAD = [
    ("bits", dict(bits=5), 3),
    ("bits1", dict(bits=1), 3),
    ("group", dict(group_size=48), 4),
    ("group_gt_d", dict(group_size=256), 4),
    ("head_dim", dict(shape=(1, 1, 1, 64)), 8),
    ("neg", dict(shape=(1, -1, 1, 128)), 2),
    ("perm_dup", dict(perm=np.zeros(128, dtype=np.uint16)), 6),
    ("perm_range", dict(perm=np.arange(1, 129, dtype=np.uint16)), 6),
    ("quat_missing", dict(rot="so4"), 1),
    ("quat_not_unit", dict(rot="so4", quat=np.ones((32, 2, 4), dtype=np.float32)), 6),
    ("codebook_missing", dict(quant="lloyd"), 1),
    ("codebook_order", dict(quant="lloyd", codebook=np.array([0, 1, 1, 2], dtype=np.float32)), 6),
    ("codebook_nan", dict(quant="lloyd", codebook=np.array([0, 1, np.nan, 2], dtype=np.float32)), 6),
    ("rope_base", dict(rope=True, rope_base=1.0), 6),
    ("positions", dict(pos_offset=2 ** 31), 6),
    ("n_sink", dict(n_sink=-1), 6),
    ("stride_align", dict(strides=(1024, 32, 3)), 7),
    ("stride_neg", dict(strides=(-8, 8, 8)), 2),
]


@pytest.mark.parametrize("name,kw,status", BAD, ids=[b[0] for b in BAD])
def test_validation_errors(name, kw, status):
    with pytest.raises(kvq.KvqError) as e:
        kvq.validate(_cfg(**kw))
    assert e.value.status == status
    assert str(e.value)


def test_abi_version_mismatch():
    c = _cfg().c_struct()
    c.abi_version = 2
    lib = ctypes.CDLL(kvq.library_path())
    lib.kvq_validate.argtypes = [ctypes.c_void_p]
    assert lib.kvq_validate(ctypes.byref(c)) == 9
    lib.kvq_last_error_message.restype = ctypes.c_char_p
    assert b"abi" in lib.kvq_last_error_message()


def test_null_config_and_outputs():
    lib = ctypes.CDLL(kvq.library_path())
    lib.kvq_validate.argtypes = [ctypes.c_void_p]
    assert lib.kvq_validate(None) == 1
    lib.kvq_encode.argtypes = [ctypes.c_void_p] * 4
    c = _cfg().c_struct()
    assert lib.kvq_encode(ctypes.byref(c), None, None, None) == 1  # planes NULL


def test_encode_rejects_missing_buffers_before_any_launch():
    """NULL / misaligned device pointers are refused on the host (no GPU needed)."""
    lib = ctypes.CDLL(kvq.library_path())
    c = _cfg().c_struct()
    P = kvq._Planes
    planes = P()
    planes.codes = 4096
    planes.scale = 8192
    planes.zero = None
    lib.kvq_encode.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.kvq_encode(ctypes.byref(c), 4096, ctypes.byref(planes), None) == 1
    planes.zero = 12288
    assert lib.kvq_encode(ctypes.byref(c), None, ctypes.byref(planes), None) == 1
    assert lib.kvq_encode(ctypes.byref(c), 4097, ctypes.byref(planes), None) == 7
    planes.codes = 4100
    assert lib.kvq_encode(ctypes.byref(c), 4096, ctypes.byref(planes), None) == 7
    lib.kvq_decode.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    planes.codes = 4096
    assert lib.kvq_decode(ctypes.byref(c), ctypes.byref(planes), 4096, 7, None) == 5  # bad out dtype
    assert lib.kvq_decode(ctypes.byref(c), ctypes.byref(planes), None, 1, None) == 1


def test_empty_tensor_is_a_no_op():
    lib = ctypes.CDLL(kvq.library_path())
    c = _cfg(shape=(0, 5, 4, 128)).c_struct()
    planes = kvq._Planes()
    lib.kvq_encode.argtypes = [ctypes.c_void_p] * 4
    assert lib.kvq_encode(ctypes.byref(c), None, ctypes.byref(planes), None) == 0


@pytest.mark.parametrize("key", sorted(workloads.WORKLOADS))
def test_packed_sizes_match_layout(key):
    wl = workloads.WORKLOADS[key]
    for case in wl.cases:
        r, t, h, d = case.shape
        cfg = kvq.Config(shape=case.shape, dtype=case.dtype, bits=case.bits, group_size=case.group_size,
                         quant=case.quant, rot=case.rot, rope=case.rope, n_sink=case.n_sink,
                         quat=np.tile(np.array([1, 0, 0, 0], np.float32), (d // 4, 2, 1)),
                         codebook=np.linspace(-1, 1, 2 ** case.bits).astype(np.float32))
        sz = kvq.packed_sizes(cfg)
        n = r * t * h
        assert sz["codes"] == n * d * case.bits // 8
        if case.quant == "minmax":
            assert sz["scale"] == sz["zero"] == n * (d // case.group_size) * 2 and sz["norm"] == 0
        else:
            assert sz["norm"] == n * 4 and sz["scale"] == 0
        assert sz["sink"] == r * case.n_sink * h * d * 2


def test_llama3_cache_bytes():
    """2-bit group-128 codes + fp16 scale/zero = 36 bytes per 256-byte bf16 vector."""
    case = workloads.WORKLOADS["llama3"].case("K")
    sz = kvq.packed_sizes(kvq.Config(shape=case.shape, dtype="bf16", bits=2, group_size=128, n_sink=4))
    n = case.n_vectors
    assert (sz["codes"] + sz["scale"] + sz["zero"]) == 36 * n


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("sigma", [1.0, 1.0 / np.sqrt(128.0), 1.0 / 16.0])
def test_host_lloyd_max_matches_oracle(bits, sigma):
    got = kvq.lloyd_max_gaussian(bits, sigma)
    want = oracle.fit_gaussian(bits, sigma)
    assert np.allclose(got, want, rtol=2e-7, atol=0), (got, want)


def test_host_lloyd_max_rejects_bad_arguments():
    with pytest.raises(kvq.KvqError):
        kvq.lloyd_max_gaussian(5, 1.0)
    with pytest.raises(kvq.KvqError):
        kvq.lloyd_max_gaussian(2, -1.0)


def test_single_hip_runtime_when_binding_imported_first():
    """Importing the binding before torch must still leave one HIP runtime in the process
    (torch's copy, which owns the caller's memory and streams)."""
    import subprocess
    import sys
    code = ("import rotate_then_bit_amd, torch\n"
            "libs = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(libs))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout


# --------------------------------------------------------------------------- #
# append and attention: host-side refusals (nothing reaches the device)
# --------------------------------------------------------------------------- #
def _lib_new_entry_points():
    lib = ctypes.CDLL(kvq.library_path())
    lib.kvq_append.argtypes = [ctypes.c_void_p] * 5
    lib.kvq_attend.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_size_t, ctypes.c_void_p]
    lib.kvq_attend_workspace_size.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    return lib


def _planes(codes=4096, scale=8192, zero=12288, sink=None):
    p = kvq._Planes()
    p.codes, p.scale, p.zero, p.sink = codes, scale, zero, sink
    return p


def test_append_refuses_bad_arguments_on_the_host():
    lib = _lib_new_entry_points()
    c = _cfg().c_struct()
    pl = _planes()
    assert lib.kvq_append(ctypes.byref(c), 4096, None, ctypes.byref(pl), None) == 1    # positions NULL
    assert lib.kvq_append(ctypes.byref(c), None, 4096, ctypes.byref(pl), None) == 1    # x NULL
    assert lib.kvq_append(ctypes.byref(c), 4100, 4096, ctypes.byref(pl), None) == 7    # x misaligned
    assert lib.kvq_append(ctypes.byref(c), 4096, 4100, ctypes.byref(pl), None) == 7    # positions misaligned
    assert lib.kvq_append(ctypes.byref(c), 4096, 4096, None, None) == 1                # planes NULL
    cs = _cfg(n_sink=4).c_struct()
    assert lib.kvq_append(ctypes.byref(cs), 4096, 4096, ctypes.byref(pl), None) == 1   # sink plane NULL
    cb = _cfg(bits=7).c_struct()
    assert lib.kvq_append(ctypes.byref(cb), 4096, 4096, ctypes.byref(pl), None) == 3


def test_attend_workspace_size_and_refusals_on_the_host():
    lib = _lib_new_entry_points()
    c = _cfg(shape=(2, 100, 4, 128)).c_struct()
    n = ctypes.c_size_t()
    assert lib.kvq_attend_workspace_size(ctypes.byref(c), 16, ctypes.byref(n)) == 0
    assert n.value >= 2 * 16 * 128 * 4 + 2 * 16 * 130 * 4
    assert kvq.attend_workspace_size(kvq.Config(shape=(2, 100, 4, 128), dtype="bf16", bits=2, group_size=128), 16) == n.value
    assert lib.kvq_attend_workspace_size(ctypes.byref(c), 6, ctypes.byref(n)) == 2     # not a multiple of heads
    assert lib.kvq_attend_workspace_size(ctypes.byref(c), 32, ctypes.byref(n)) == 8    # 8 query heads per KV head
    for kw, status in ((dict(rot="none"), 8), (dict(bits=3), 8), (dict(group_size=32, shape=(1, 4, 2, 256)), 8),
                       (dict(quant="lloyd", codebook=np.linspace(-1, 1, 4).astype(np.float32)), 8),
                       (dict(pos_offset=3), 8), (dict(n_sink=65), 8)):
        ck = _cfg(**kw).c_struct()
        assert lib.kvq_attend_workspace_size(ctypes.byref(ck), 8, ctypes.byref(n)) == status, kw
    ck, cv = _cfg().c_struct(), _cfg(bits=4).c_struct()
    pk, pv = _planes(), _planes()
    ws = 1 << 20
    # the K and V caches must agree
    assert lib.kvq_attend(ctypes.byref(ck), ctypes.byref(pk), ctypes.byref(cv), ctypes.byref(pv), 4096, 8, None,
                          0.1, 4096, 4096, ws, None) == 2
    cv = _cfg().c_struct()
    args = lambda q=4096, out=4096, wsp=4096, wsz=ws, sc=0.1: (ctypes.byref(ck), ctypes.byref(pk), ctypes.byref(cv),
                                                               ctypes.byref(pv), q, 8, None, sc, out, wsp, wsz, None)
    assert lib.kvq_attend(*args(q=None)) == 1
    assert lib.kvq_attend(*args(q=4100)) == 7
    assert lib.kvq_attend(*args(wsz=16)) == 2        # workspace too small
    assert lib.kvq_attend(*args(sc=float("nan"))) == 6
    assert lib.kvq_attend(ctypes.byref(ck), ctypes.byref(pk), None, ctypes.byref(pv), 4096, 8, None, 0.1, 4096,
                          4096, ws, None) == 1        # cfg_v NULL
