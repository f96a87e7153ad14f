"""Helpers for the GPU tests: run the HIP codec on host-generated inputs and copy the
planes back as numpy arrays.  Imported only by tests marked ``gpu``."""
from __future__ import annotations

import numpy as np


def torch_input(x_np: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x_np))
    return t.to(device)


def raw_numpy(t, dtype: str) -> np.ndarray:
    """Device tensor -> numpy array in the oracle's input representation (bf16 as uint16 bits)."""
    import torch
    t = t.detach().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def planes_numpy(planes) -> dict:
    import torch
    out = {}
    for k, v in planes.items():
        v = v.detach().cpu()
        if v.dtype == torch.float16:
            out[k] = v.view(torch.int16).numpy().view(np.float16)
        else:
            out[k] = v.numpy()
    return out


def make_config(case, perm=None, quat=None, codebook=None, strides=None):
    import rotate_then_bit_amd as kvq
    return kvq.Config(shape=case.shape, dtype=case.dtype, bits=case.bits, group_size=case.group_size,
                      quant=case.quant, rot=case.rot, rope=case.rope, rope_base=case.rope_base,
                      pos_offset=case.pos_offset, n_sink=case.n_sink,
                      perm=perm if case.use_perm else None, quat=quat, codebook=codebook, strides=strides)


def codebook_for(case):
    """Lloyd-Max codebook from the oracle (the inputs both sides receive)."""
    import oracle
    if case.quant != "lloyd":
        return None
    sigma = case.lloyd_sigma if case.lloyd_sigma else 1.0 / np.sqrt(case.shape[-1])
    return oracle.fit_gaussian(case.bits, sigma).astype(np.float32)


def poison_planes(planes, byte: int):
    import torch
    for v in planes.values():
        v.view(torch.uint8).fill_(byte)
    return planes
