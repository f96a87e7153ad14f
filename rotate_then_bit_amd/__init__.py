"""Python binding of the kvq C ABI (``include/kvq.h``): rotation + low-bit KV-cache codec on MI355X.

Argument marshalling only -- every step of the codec runs in the HIP kernels of
``libkvq.so``.  PyTorch supplies device memory and the current HIP stream.

    import rotate_then_bit_amd as kvq
    cfg = kvq.Config(shape=(R, T, H, 128), dtype="bf16", bits=2, group_size=128,
                     rope=True, n_sink=4, perm=perm)
    planes = kvq.encode(x, cfg)                 # dict of torch tensors
    y = kvq.decode(planes, cfg, out_dtype="bf16")

The library is required: it is loaded on the first call that needs it, and that
call raises ImportError when ``libkvq.so`` has not been built.  There is no CPU
fallback.  (Importing the package itself needs no library, so the build script
can run from a clean checkout.)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence

import numpy as np

__all__ = ["Config", "KvqError", "encode", "append", "attend", "attend_noalloc", "attend_noalloc_max_workspace",
           "channel_stats", "channel_stats_workspace_size", "outlier_perm", "detect_sinks", "rotated_moments",
           "dynamic_codebook", "attention_entropy", "allocate_bits", "encode_heads",
           "attend_workspace_size", "decode", "packed_sizes", "validate", "lloyd_max_gaussian",
           "rotor_matrix", "library_path", "abi_version", "DTYPES", "ROTATIONS", "QUANTIZERS", "EXPORTED_SYMBOLS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkvq.so")

ABI_VERSION = 4
DTYPES = {"f16": 0, "bf16": 1, "f32": 2}
ROTATIONS = {"none": 0, "fwht": 1, "so4": 2, "dense": 3, "rotor": 4}
QUANTIZERS = {"minmax": 0, "lloyd": 1}
EXPORTED_SYMBOLS = ("kvq_abi_version", "kvq_validate", "kvq_packed_sizes", "kvq_encode", "kvq_append",
                    "kvq_attend_workspace_size", "kvq_attend", "kvq_attend_noalloc", "kvq_attend_noalloc_max_workspace",
                    "kvq_decode", "kvq_lloyd_max_gaussian", "kvq_channel_stats_workspace_size", "kvq_channel_stats",
                    "kvq_outlier_perm", "kvq_detect_sinks", "kvq_rotated_moments", "kvq_dynamic_codebook",
                    "kvq_attention_entropy_workspace_size", "kvq_attention_entropy", "kvq_allocate_bits",
                    "kvq_rotor_matrix", "kvq_status_string", "kvq_last_error_message")


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
        ("chan_scale", ctypes.c_void_p),
        ("chan_wide", ctypes.c_void_p),
        ("codebook_wide", ctypes.c_void_p),
        ("rot_matrix", ctypes.c_void_p),
        ("rotor_quat", ctypes.c_void_p),
        ("rotor_tail", ctypes.c_double),
    ]


class _Planes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("codes", "scale", "zero", "norm", "sink", "extra")]


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
    lib.kvq_packed_sizes.argtypes = [ctypes.POINTER(_Config)] + [ctypes.POINTER(ctypes.c_size_t)] * 6
    lib.kvq_encode.argtypes = [ctypes.POINTER(_Config), ctypes.c_void_p, ctypes.POINTER(_Planes), ctypes.c_void_p]
    lib.kvq_append.argtypes = [ctypes.POINTER(_Config), ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(_Planes),
                               ctypes.c_void_p]
    lib.kvq_decode.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Planes), ctypes.c_void_p, ctypes.c_int32,
                               ctypes.c_void_p]
    lib.kvq_attend_workspace_size.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Config), ctypes.c_int64,
                                              ctypes.POINTER(ctypes.c_size_t)]
    lib.kvq_attend.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Planes), ctypes.POINTER(_Config),
                               ctypes.POINTER(_Planes), ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                               ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.kvq_attend_noalloc.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Planes), ctypes.POINTER(_Config),
                                       ctypes.POINTER(_Planes), ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
    lib.kvq_attend_noalloc_max_workspace.restype = ctypes.c_size_t
    lib.kvq_attend_noalloc_max_workspace.argtypes = []
    lib.kvq_channel_stats_workspace_size.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(ctypes.c_size_t)]
    lib.kvq_channel_stats.argtypes = [ctypes.POINTER(_Config), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p]
    lib.kvq_outlier_perm.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
    lib.kvq_detect_sinks.argtypes = [ctypes.POINTER(_Config), ctypes.c_void_p, ctypes.c_double] + [ctypes.c_void_p] * 6
    lib.kvq_rotated_moments.argtypes = [ctypes.POINTER(_Config), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]
    lib.kvq_dynamic_codebook.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32] + [ctypes.c_void_p] * 4
    lib.kvq_attention_entropy_workspace_size.argtypes = [ctypes.POINTER(_Config), ctypes.c_int64,
                                                         ctypes.POINTER(ctypes.c_size_t)]
    lib.kvq_attention_entropy.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Planes), ctypes.c_void_p,
                                          ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.kvq_allocate_bits.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p]
    lib.kvq_lloyd_max_gaussian.argtypes = [ctypes.c_int32, ctypes.c_double, ctypes.c_void_p]
    lib.kvq_rotor_matrix.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p]
    lib.kvq_status_string.restype = ctypes.c_char_p
    lib.kvq_status_string.argtypes = [ctypes.c_int]
    lib.kvq_last_error_message.restype = ctypes.c_char_p
    for fn in ("kvq_validate", "kvq_packed_sizes", "kvq_encode", "kvq_append", "kvq_decode", "kvq_lloyd_max_gaussian",
               "kvq_attend_workspace_size", "kvq_attend", "kvq_attend_noalloc", "kvq_channel_stats_workspace_size",
               "kvq_channel_stats", "kvq_outlier_perm", "kvq_detect_sinks", "kvq_rotated_moments",
               "kvq_dynamic_codebook", "kvq_attention_entropy_workspace_size", "kvq_attention_entropy",
               "kvq_allocate_bits", "kvq_rotor_matrix"):
        getattr(lib, fn).restype = ctypes.c_int
    if lib.kvq_abi_version() != ABI_VERSION:
        raise ImportError(f"libkvq ABI {lib.kvq_abi_version()} != binding ABI {ABI_VERSION}")
    return lib


_lib_handle = None


def _L():
    """The loaded library (loaded on first use; raises ImportError if it was never built)."""
    global _lib_handle
    if _lib_handle is None:
        _lib_handle = _load()
    return _lib_handle


def abi_version() -> int:
    return int(_L().kvq_abi_version())


def _check(status: int):
    if status != 0:
        lib = _L()
        raise KvqError(status, (lib.kvq_last_error_message() or b"").decode() or
                       lib.kvq_status_string(status).decode())


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
    chan_scale: Optional[np.ndarray] = None     # dynamic codebook: per rotated channel scale
    chan_wide: Optional[np.ndarray] = None      # dynamic codebook: 0/1, D/16 ones
    codebook_wide: Optional[np.ndarray] = None  # dynamic codebook: 2^(bits+1) levels
    rot_matrix: Optional[object] = None         # dense rotation: float32 device tensor [D, D]
    rotor_quat: Optional[np.ndarray] = None     # rotor rotation: [D // 3, 4] unit quaternions
    rotor_tail: float = 0.0                     # rotor rotation: the 2-channel tail's angle
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
                              ("codebook", self.codebook, np.float32), ("chan_scale", self.chan_scale, np.float32),
                              ("chan_wide", self.chan_wide, np.uint8), ("codebook_wide", self.codebook_wide, np.float32),
                              ("rotor_quat", self.rotor_quat, np.float32)):
            if arr is None:
                setattr(c, name, None)
            else:
                a = np.ascontiguousarray(np.asarray(arr, dtype=dt))
                self._keep.append(a)
                setattr(c, name, a.ctypes.data)
        c.rot_matrix = None if self.rot_matrix is None else int(self.rot_matrix.data_ptr())
        c.rotor_tail = float(self.rotor_tail)
        return c


def validate(cfg: Config) -> None:
    c = cfg.c_struct()
    _check(_L().kvq_validate(ctypes.byref(c)))


def packed_sizes(cfg: Config) -> Dict[str, int]:
    c = cfg.c_struct()
    out = [ctypes.c_size_t() for _ in range(6)]
    _check(_L().kvq_packed_sizes(ctypes.byref(c), *[ctypes.byref(o) for o in out]))
    return dict(zip(("codes", "scale", "zero", "norm", "sink", "extra"), (int(o.value) for o in out)))


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
    if sz["extra"]:
        out["extra"] = torch.empty((r, t, h, d // 128), dtype=torch.uint8, device=device)
    assert out["codes"].numel() == sz["codes"]
    return out


def _planes_struct(planes) -> _Planes:
    p = _Planes()
    for n in ("codes", "scale", "zero", "norm", "sink", "extra"):
        setattr(p, n, _ptr(planes.get(n)))
    return p


def encode(x, cfg: Config, planes=None, stream=None):
    """Encode device tensor ``x`` ([R,T,H,D] of cfg.dtype, strided as cfg.strides) into packed planes."""
    if planes is None:
        planes = empty_planes(cfg, device=x.device)
    c = cfg.c_struct()
    p = _planes_struct(planes)
    _check(_L().kvq_encode(ctypes.byref(c), _ptr(x), ctypes.byref(p), _stream_handle(stream)))
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
    _check(_L().kvq_append(ctypes.byref(c), _ptr(x), _ptr(positions), ctypes.byref(p), _stream_handle(stream)))
    return cache


def attend_workspace_size(k_cfg: Config, q_heads: int, v_cfg: Config = None) -> int:
    """Bytes of device workspace ``attend`` needs for these caches and query-head count
    (``v_cfg`` None: a V cache configured like K)."""
    c = k_cfg.c_struct()
    cv = v_cfg.c_struct() if v_cfg is not None else None
    n = ctypes.c_size_t()
    _check(_L().kvq_attend_workspace_size(ctypes.byref(c), ctypes.byref(cv) if cv is not None else None,
                                          int(q_heads), ctypes.byref(n)))
    return int(n.value)


def attend(q, k_planes, k_cfg: Config, v_planes, v_cfg: Config, lengths=None, scale=None, out=None,
           workspace=None, stream=None):
    """Decode-step attention of ``q`` (float32 device tensor [R, q_heads, head_dim]) over the
    encoded K/V cache; ``lengths`` (int32 device tensor [R]) limits each row to its first slots.
    Returns ``out`` (float32 [R, q_heads, head_dim])."""
    import torch
    r, q_heads = int(q.shape[0]), int(q.shape[1])
    if q.dtype != torch.float32 or not q.is_contiguous():
        raise ValueError("q must be a contiguous float32 tensor [rows, q_heads, head_dim]")
    if lengths is not None and (lengths.dtype != torch.int32 or lengths.numel() != r or not lengths.is_contiguous()):
        raise ValueError("lengths must be a contiguous int32 tensor with one entry per row")
    if scale is None:
        scale = float(k_cfg.shape[-1]) ** -0.5
    if out is None:
        out = torch.empty_like(q)
    need = attend_workspace_size(k_cfg, q_heads, v_cfg)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ck, cv = k_cfg.c_struct(), v_cfg.c_struct()
    pk, pv = _planes_struct(k_planes), _planes_struct(v_planes)
    _check(_L().kvq_attend(ctypes.byref(ck), ctypes.byref(pk), ctypes.byref(cv), ctypes.byref(pv), _ptr(q), q_heads,
                           _ptr(lengths), float(scale), _ptr(out), int(workspace.data_ptr()),
                           int(workspace.numel() * workspace.element_size()), _stream_handle(stream)))
    return out


def attend_noalloc(q, k_planes, k_cfg: Config, v_planes, v_cfg: Config, lengths=None, scale=None, out=None,
                   stream=None):
    """``attend`` through the allocation-free entry point: the workspace is the library's
    static device array (``attend_noalloc_max_workspace()`` bytes per GPU); calls on one GPU
    must not overlap.  ``out`` must be given by callers that cannot allocate."""
    import torch
    r, q_heads = int(q.shape[0]), int(q.shape[1])
    if q.dtype != torch.float32 or not q.is_contiguous():
        raise ValueError("q must be a contiguous float32 tensor [rows, q_heads, head_dim]")
    if lengths is not None and (lengths.dtype != torch.int32 or lengths.numel() != r or not lengths.is_contiguous()):
        raise ValueError("lengths must be a contiguous int32 tensor with one entry per row")
    if scale is None:
        scale = float(k_cfg.shape[-1]) ** -0.5
    if out is None:
        out = torch.empty_like(q)
    ck, cv = k_cfg.c_struct(), v_cfg.c_struct()
    pk, pv = _planes_struct(k_planes), _planes_struct(v_planes)
    _check(_L().kvq_attend_noalloc(ctypes.byref(ck), ctypes.byref(pk), ctypes.byref(cv), ctypes.byref(pv), _ptr(q),
                                   q_heads, _ptr(lengths), float(scale), _ptr(out), _stream_handle(stream)))
    return out


def attend_noalloc_max_workspace() -> int:
    return int(_L().kvq_attend_noalloc_max_workspace())


_TORCH_DT = {"f16": "float16", "bf16": "bfloat16", "f32": "float32"}


def decode(planes, cfg: Config, out_dtype: str = "f32", out=None, stream=None):
    """Decode packed planes into a contiguous [R,T,H,D] device tensor of ``out_dtype``."""
    import torch
    if out is None:
        out = torch.empty(tuple(int(v) for v in cfg.shape), dtype=getattr(torch, _TORCH_DT[out_dtype]),
                          device=planes["codes"].device)
    c = cfg.c_struct()
    p = _planes_struct(planes)
    _check(_L().kvq_decode(ctypes.byref(c), ctypes.byref(p), _ptr(out), DTYPES[out_dtype], _stream_handle(stream)))
    return out


def channel_stats_workspace_size(cfg: Config) -> int:
    """Bytes of device workspace ``channel_stats`` needs for this slice shape."""
    c = cfg.c_struct()
    n = ctypes.c_size_t()
    _check(_L().kvq_channel_stats_workspace_size(ctypes.byref(c), ctypes.byref(n)))
    return int(n.value)


def channel_stats(x, cfg: Config, workspace=None, stream=None):
    """Per-channel mean |y_c| (float64 device tensor [D]) of the calibration slice ``x``, read
    as ``encode`` reads it (post-RoPE for keys, sink positions left out)."""
    import torch
    c = cfg.c_struct()
    if workspace is None:
        workspace = torch.empty(max(channel_stats_workspace_size(cfg), 8), dtype=torch.uint8, device=x.device)
    stats = torch.empty(int(cfg.shape[-1]), dtype=torch.float64, device=x.device)
    _check(_L().kvq_channel_stats(ctypes.byref(c), _ptr(x), int(stats.data_ptr()), int(workspace.data_ptr()),
                                  int(workspace.numel() * workspace.element_size()), _stream_handle(stream)))
    return stats


def outlier_perm(stats, group_size: int) -> np.ndarray:
    """Host-side outlier-aware gather map (uint16 [D]) from per-channel statistics."""
    st = np.ascontiguousarray(np.asarray(stats, dtype=np.float64))
    perm = np.zeros(st.shape[0], dtype=np.uint16)
    _check(_L().kvq_outlier_perm(st.ctypes.data, int(st.shape[0]), int(group_size), perm.ctypes.data))
    return perm


def detect_sinks(x, cfg: Config, lam: float, stream=None):
    """Activation-based sink detection of the slice ``x``: returns device tensors
    (norms f64 [R,T], flags u8 [R,T], counts i32 [R], prefix i32 [R], medians f64 [R])."""
    import torch
    r, t = int(cfg.shape[0]), int(cfg.shape[1])
    dev = x.device
    norms = torch.empty((r, t), dtype=torch.float64, device=dev)
    flags = torch.empty((r, t), dtype=torch.uint8, device=dev)
    counts = torch.empty(r, dtype=torch.int32, device=dev)
    prefix = torch.empty(r, dtype=torch.int32, device=dev)
    medians = torch.empty(r, dtype=torch.float64, device=dev)
    c = cfg.c_struct()
    _check(_L().kvq_detect_sinks(ctypes.byref(c), _ptr(x), float(lam), _ptr(norms), _ptr(flags), _ptr(counts),
                                 _ptr(prefix), _ptr(medians), _stream_handle(stream)))
    return norms, flags, counts, prefix, medians


def rotated_moments(x, cfg: Config, workspace=None, stream=None):
    """Per rotated channel mean z_j^2 (float64 device tensor [D]) of the calibration slice
    ``x`` through the codec's front end (cfg.quant must be "lloyd")."""
    import torch
    c = cfg.c_struct()
    if workspace is None:
        workspace = torch.empty(max(channel_stats_workspace_size(cfg), 8), dtype=torch.uint8, device=x.device)
    m = torch.empty(int(cfg.shape[-1]), dtype=torch.float64, device=x.device)
    _check(_L().kvq_rotated_moments(ctypes.byref(c), _ptr(x), int(m.data_ptr()), int(workspace.data_ptr()),
                                    int(workspace.numel() * workspace.element_size()), _stream_handle(stream)))
    return m


def dynamic_codebook(moments, bits: int):
    """Host-side dynamic codebook from per-channel moments: (chan_scale f32 [D], chan_wide u8 [D],
    codebook f32 [2^bits], codebook_wide f32 [2^(bits+1)])."""
    m = np.ascontiguousarray(np.asarray(moments, dtype=np.float64))
    d = m.shape[0]
    sc = np.zeros(d, dtype=np.float32)
    wide = np.zeros(d, dtype=np.uint8)
    cb = np.zeros(2 ** bits, dtype=np.float32)
    cbw = np.zeros(2 ** (bits + 1), dtype=np.float32)
    _check(_L().kvq_dynamic_codebook(m.ctypes.data, d, int(bits), sc.ctypes.data, wide.ctypes.data, cb.ctypes.data,
                                     cbw.ctypes.data))
    return sc, wide, cb, cbw


def attention_entropy(q, k_planes, k_cfg: Config, lengths=None, scale=None, out=None, workspace=None, stream=None):
    """Entropy (nats, float32 device tensor [R, q_heads]) of each query head's softmax attention
    over the encoded K cache."""
    import torch
    r, q_heads = int(q.shape[0]), int(q.shape[1])
    if q.dtype != torch.float32 or not q.is_contiguous():
        raise ValueError("q must be a contiguous float32 tensor [rows, q_heads, head_dim]")
    if scale is None:
        scale = float(k_cfg.shape[-1]) ** -0.5
    c = k_cfg.c_struct()
    n = ctypes.c_size_t()
    _check(_L().kvq_attention_entropy_workspace_size(ctypes.byref(c), q_heads, ctypes.byref(n)))
    if workspace is None:
        workspace = torch.empty(max(int(n.value), 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((r, q_heads), dtype=torch.float32, device=q.device)
    pk = _planes_struct(k_planes)
    _check(_L().kvq_attention_entropy(ctypes.byref(c), ctypes.byref(pk), _ptr(q), q_heads, _ptr(lengths), float(scale),
                                      _ptr(out), int(workspace.data_ptr()),
                                      int(workspace.numel() * workspace.element_size()), _stream_handle(stream)))
    return out


def allocate_bits(entropy, total: int, lo: int = 2, hi: int = 4) -> np.ndarray:
    """Host-side per-head widths (int32 [heads]) in proportion to the heads' entropies."""
    e = np.ascontiguousarray(np.asarray(entropy, dtype=np.float64))
    b = np.zeros(e.shape[0], dtype=np.int32)
    _check(_L().kvq_allocate_bits(e.ctypes.data, e.shape[0], int(total), int(lo), int(hi), b.ctypes.data))
    return b


def encode_heads(x, cfg: Config, bits_per_head, stream=None):
    """Encode each KV head of ``x`` ([R,T,H,D], contiguous or strided as cfg.strides) at its own
    width: head h is a head shard (the stride arguments select it) encoded with
    bits_per_head[h].  Returns a list of (Config, planes), one per head."""
    r, t, h, d = (int(v) for v in cfg.shape)
    sr, st, sh = cfg.strides if cfg.strides is not None else tuple(int(v) for v in x.stride()[:3])
    out = []
    for i in range(h):
        ci = Config(**{**cfg.__dict__, "shape": (r, t, 1, d), "bits": int(bits_per_head[i]), "strides": (sr, st, sh),
                       "_keep": []})
        out.append((ci, encode(x[:, :, i:i + 1], ci, stream=stream)))
    return out


def lloyd_max_gaussian(bits: int, sigma: float) -> np.ndarray:
    """Host-side Lloyd-Max codebook for N(0, sigma^2) (float32, ascending)."""
    out = np.zeros(2 ** bits, dtype=np.float32)
    _check(_L().kvq_lloyd_max_gaussian(int(bits), float(sigma), out.ctypes.data))
    return out


def rotor_matrix(rq, head_dim: int, tail_angle: float = 0.0) -> np.ndarray:
    """RotorQuant's 3-D rotors as the [D, D] float32 matrix of a dense rotation (host)."""
    rq = np.ascontiguousarray(rq, dtype=np.float32)
    if rq.shape != (int(head_dim) // 3, 4):
        raise ValueError(f"rq must be [{int(head_dim) // 3}, 4]")
    out = np.zeros((int(head_dim), int(head_dim)), dtype=np.float32)
    _check(_L().kvq_rotor_matrix(rq.ctypes.data, int(head_dim), float(tail_angle), out.ctypes.data))
    return out

