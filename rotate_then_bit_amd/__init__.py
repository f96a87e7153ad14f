"""Python binding of the kvq C ABI (``include/kvq.h``): rotation + low-bit KV-cache codec on MI355X.

Argument marshalling only -- every step of the codec runs in the HIP kernels of
``libkvq.so``.  PyTorch supplies device memory and the current HIP stream.

    import rotate_then_bit_amd as kvq
    cfg = kvq.Config(shape=(R, T, H, 128), dtype="bf16", bits=2, group_size=128,
                     rope=True, n_sink=4, perm=perm)
    planes = kvq.encode(x, cfg)                 # dict of torch tensors
    y = kvq.decode(planes, cfg, out_dtype="bf16")

The library is required: importing this package without a built ``libkvq.so``
raises, and there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence

import numpy as np

__all__ = ["Config", "KvqError", "encode", "append", "attend", "attend_workspace_size", "decode", "packed_sizes", "validate", "lloyd_max_gaussian",
           "library_path", "abi_version", "DTYPES", "ROTATIONS", "QUANTIZERS", "EXPORTED_SYMBOLS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkvq.so")

ABI_VERSION = 1
DTYPES = {"f16": 0, "bf16": 1, "f32": 2}
ROTATIONS = {"none": 0, "fwht": 1, "so4": 2}
QUANTIZERS = {"minmax": 0, "lloyd": 1}
EXPORTED_SYMBOLS = ("kvq_abi_version", "kvq_validate", "kvq_packed_sizes", "kvq_encode", "kvq_append",
                    "kvq_attend_workspace_size", "kvq_attend", "kvq_decode", "kvq_lloyd_max_gaussian",
                    "kvq_status_string", "kvq_last_error_message")


class _Config(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("rows", ctypes.c_int64),
        ("tokens", ctypes.c_int64),
        ("heads", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("stride_r", ctypes.c_int64),
        ("stride_t", ctypes.c_int64),
        ("stride_h", ctypes.c_int64),
        ("bits", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("quant", ctypes.c_int32),
        ("rot", ctypes.c_int32),
        ("rope", ctypes.c_int32),
        ("n_sink", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("pos_offset", ctypes.c_int64),
        ("perm", ctypes.c_void_p),
        ("quat", ctypes.c_void_p),
        ("codebook", ctypes.c_void_p),
    ]


class _Planes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("codes", "scale", "zero", "norm", "sink")]


class KvqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kvq status {status}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m rotate_then_bit_amd.build`")
    # The library must run on the same HIP runtime as the memory and streams it is
    # handed.  PyTorch ships its own libamdhip64 under the system one's soname: with
    # torch loaded first the dynamic linker binds libkvq.so to that copy; loaded the
    # other way round, the process ends up with two HIP runtimes, and the library's
    # calls go to one that owns no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(_LIB_PATH)
    lib.kvq_abi_version.restype = ctypes.c_int32
    lib.kvq_validate.argtypes = [ctypes.POINTER(_Config)]
    lib.kvq_packed_sizes.argtypes = [ctypes.POINTER(_Config)] + [ctypes.POINTER(ctypes.c_size_t)] * 5
    lib.kvq_encode.argtypes = [ctypes.POINTER(_Config), ctypes.c_void_p, ctypes.POINTER(_Planes), ctypes.c_void_p]
    lib.kvq_append.argtypes = [ctypes.POINTER(_Config), ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(_Planes),
                               ctypes.c_void_p]
    lib.kvq_decode.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Planes), ctypes.c_void_p, ctypes.c_int32,
                               ctypes.c_void_p]
    lib.kvq_attend_workspace_size.argtypes = [ctypes.POINTER(_Config), ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)]
    lib.kvq_attend.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Planes), ctypes.POINTER(_Config),
                               ctypes.POINTER(_Planes), ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                               ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.kvq_lloyd_max_gaussian.argtypes = [ctypes.c_int32, ctypes.c_double, ctypes.c_void_p]
    lib.kvq_status_string.restype = ctypes.c_char_p
    lib.kvq_status_string.argtypes = [ctypes.c_int]
    lib.kvq_last_error_message.restype = ctypes.c_char_p
    for fn in ("kvq_validate", "kvq_packed_sizes", "kvq_encode", "kvq_append", "kvq_decode", "kvq_lloyd_max_gaussian",
               "kvq_attend_workspace_size", "kvq_attend"):
        getattr(lib, fn).restype = ctypes.c_int
    if lib.kvq_abi_version() != ABI_VERSION:
        raise ImportError(f"libkvq ABI {lib.kvq_abi_version()} != binding ABI {ABI_VERSION}")
    return lib


_lib = _load()


def abi_version() -> int:
    return int(_lib.kvq_abi_version())


def _check(status: int):
    if status != 0:
        raise KvqError(status, (_lib.kvq_last_error_message() or b"").decode() or
                       _lib.kvq_status_string(status).decode())


@dataclass
class Config:
    """Mirror of ``kvq_config``.  Host parameter arrays are kept alive by this object."""

    shape: Sequence[int]  # (rows, tokens, heads, head_dim)
    dtype: str = "bf16"
    bits: int = 2
    group_size: int = 128
    quant: str = "minmax"
    rot: str = "fwht"
    rope: bool = False
    rope_base: float = 10000.0
    pos_offset: int = 0
    n_sink: int = 0
    perm: Optional[np.ndarray] = None
    quat: Optional[np.ndarray] = None
    codebook: Optional[np.ndarray] = None
    strides: Optional[Sequence[int]] = None  # (stride_r, stride_t, stride_h) in elements
    _keep: list = field(default_factory=list, repr=False)

    def c_struct(self) -> _Config:
        r, t, h, d = (int(v) for v in self.shape)
        c = _Config()
        c.abi_version = ABI_VERSION
        c.dtype = DTYPES[self.dtype]
        c.rows, c.tokens, c.heads, c.head_dim = r, t, h, d
        sr, st, sh = self.strides if self.strides is not None else (0, 0, 0)
        c.stride_r, c.stride_t, c.stride_h = int(sr), int(st), int(sh)
        c.bits = int(self.bits)
        c.group_size = int(self.group_size)
        c.quant = QUANTIZERS[self.quant]
        c.rot = ROTATIONS[self.rot]
        c.rope = 1 if self.rope else 0
        c.n_sink = int(self.n_sink)
        c.rope_base = float(self.rope_base)
        c.pos_offset = int(self.pos_offset)
        self._keep = []
        for name, arr, dt in (("perm", self.perm, np.uint16), ("quat", self.quat, np.float32),
                              ("codebook", self.codebook, np.float32)):
            if arr is None:
                setattr(c, name, None)
            else:
                a = np.ascontiguousarray(np.asarray(arr, dtype=dt))
                self._keep.append(a)
                setattr(c, name, a.ctypes.data)
        return c


def validate(cfg: Config) -> None:
    c = cfg.c_struct()
    _check(_lib.kvq_validate(ctypes.byref(c)))


def packed_sizes(cfg: Config) -> Dict[str, int]:
    c = cfg.c_struct()
    out = [ctypes.c_size_t() for _ in range(5)]
    _check(_lib.kvq_packed_sizes(ctypes.byref(c), *[ctypes.byref(o) for o in out]))
    return dict(zip(("codes", "scale", "zero", "norm", "sink"), (int(o.value) for o in out)))


def _stream_handle(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None or t.numel() == 0 else int(t.data_ptr())


def empty_planes(cfg: Config, device="cuda") -> Dict[str, "object"]:
    """Allocate the packed planes for ``cfg`` with torch (uninitialised)."""
    import torch
    sz = packed_sizes(cfg)
    r, t, h, d = (int(v) for v in cfg.shape)
    out = {"codes": torch.empty((r, t, h, d * cfg.bits // 8), dtype=torch.uint8, device=device)}
    if cfg.quant == "minmax":
        ng = d // cfg.group_size
        out["scale"] = torch.empty((r, t, h, ng), dtype=torch.float16, device=device)
        out["zero"] = torch.empty((r, t, h, ng), dtype=torch.float16, device=device)
    else:
        out["norm"] = torch.empty((r, t, h), dtype=torch.float32, device=device)
    if cfg.n_sink > 0:
        out["sink"] = torch.empty((r, cfg.n_sink, h, d), dtype=torch.float16, device=device)
    assert out["codes"].numel() == sz["codes"]
    return out


def _planes_struct(planes) -> _Planes:
    p = _Planes()
    for n in ("codes", "scale", "zero", "norm", "sink"):
        setattr(p, n, _ptr(planes.get(n)))
    return p


def encode(x, cfg: Config, planes=None, stream=None):
    """Encode device tensor ``x`` ([R,T,H,D] of cfg.dtype, strided as cfg.strides) into packed planes."""
    if planes is None:
        planes = empty_planes(cfg, device=x.device)
    c = cfg.c_struct()
    p = _planes_struct(planes)
    _check(_lib.kvq_encode(ctypes.byref(c), _ptr(x), ctypes.byref(p), _stream_handle(stream)))
    return planes


def append(x, positions, cache, cfg: Config, stream=None):
    """Decode-step append: encode row r's new token ``x[r]`` ([R,H,D] of cfg.dtype, strided
    as cfg.strides' row and head strides) at position ``positions[r]`` (int64 device tensor
    [R]) into slot ``positions[r] - cfg.pos_offset`` of the ``cache`` planes, which hold
    cfg.shape = (R, slots, H, D).  Rows whose position is outside the cache's slots write
    nothing.  Returns ``cache``."""
    import torch
    r = int(cfg.shape[0])
    if positions.dtype != torch.int64 or positions.numel() != r or not positions.is_contiguous():
        raise ValueError("positions must be a contiguous int64 tensor with one entry per row")
    c = cfg.c_struct()
    p = _planes_struct(cache)
    _check(_lib.kvq_append(ctypes.byref(c), _ptr(x), _ptr(positions), ctypes.byref(p), _stream_handle(stream)))
    return cache


def attend_workspace_size(k_cfg: Config, q_heads: int) -> int:
    """Bytes of device workspace ``attend`` needs for this cache shape and query-head count."""
    c = k_cfg.c_struct()
    n = ctypes.c_size_t()
    _check(_lib.kvq_attend_workspace_size(ctypes.byref(c), int(q_heads), ctypes.byref(n)))
    return int(n.value)


def attend(q, k_planes, k_cfg: Config, v_planes, v_cfg: Config, lengths=None, scale=None, out=None,
           workspace=None, stream=None):
    """Decode-step attention of ``q`` (float32 device tensor [R, q_heads, 128]) over the encoded
    K/V cache; ``lengths`` (int32 device tensor [R]) limits each row to its first slots.
    Returns ``out`` (float32 [R, q_heads, 128])."""
    import torch
    r, q_heads = int(q.shape[0]), int(q.shape[1])
    if q.dtype != torch.float32 or not q.is_contiguous():
        raise ValueError("q must be a contiguous float32 tensor [rows, q_heads, 128]")
    if lengths is not None and (lengths.dtype != torch.int32 or lengths.numel() != r or not lengths.is_contiguous()):
        raise ValueError("lengths must be a contiguous int32 tensor with one entry per row")
    if scale is None:
        scale = float(k_cfg.shape[-1]) ** -0.5
    if out is None:
        out = torch.empty_like(q)
    need = attend_workspace_size(k_cfg, q_heads)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ck, cv = k_cfg.c_struct(), v_cfg.c_struct()
    pk, pv = _planes_struct(k_planes), _planes_struct(v_planes)
    _check(_lib.kvq_attend(ctypes.byref(ck), ctypes.byref(pk), ctypes.byref(cv), ctypes.byref(pv), _ptr(q), q_heads,
                           _ptr(lengths), float(scale), _ptr(out), int(workspace.data_ptr()),
                           int(workspace.numel() * workspace.element_size()), _stream_handle(stream)))
    return out


_TORCH_DT = {"f16": "float16", "bf16": "bfloat16", "f32": "float32"}


def decode(planes, cfg: Config, out_dtype: str = "f32", out=None, stream=None):
    """Decode packed planes into a contiguous [R,T,H,D] device tensor of ``out_dtype``."""
    import torch
    if out is None:
        out = torch.empty(tuple(int(v) for v in cfg.shape), dtype=getattr(torch, _TORCH_DT[out_dtype]),
                          device=planes["codes"].device)
    c = cfg.c_struct()
    p = _planes_struct(planes)
    _check(_lib.kvq_decode(ctypes.byref(c), ctypes.byref(p), _ptr(out), DTYPES[out_dtype], _stream_handle(stream)))
    return out


def lloyd_max_gaussian(bits: int, sigma: float) -> np.ndarray:
    """Host-side Lloyd-Max codebook for N(0, sigma^2) (float32, ascending)."""
    out = np.zeros(2 ** bits, dtype=np.float32)
    _check(_lib.kvq_lloyd_max_gaussian(int(bits), float(sigma), out.ctypes.data))
    return out
