"""Build libkvq.so (HIP kernels + C ABI) for gfx950, in-tree.

Usage: ``python -m rotate_then_bit_amd.build`` (or ``build()`` from Python).
The kernels are compiled as several translation units in parallel, then linked
with the host-side C ABI into ``rotate_then_bit_amd/libkvq.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")

# Packed FP32 VALU ops are disabled for the device code: the compiler would
# otherwise form v_pk_{add,mul,fma}_f32 from ordinary float code.  The codec
# requires finite inputs, so NaN semantics are relaxed (min/max then need no
# operand canonicalisation).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-honor-nans"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function"]

# translation units: (source, extra defines)
KERNEL_UNITS = [("kvq_kernels.hip", [f"-DKVQ_UNIT={i}"]) for i in range(22)]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the kvq library)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    hipcc = _hipcc()
    tmp = tempfile.mkdtemp(prefix="kvq_build_")
    try:
        objs = []
        cmds = []
        for src, defs in KERNEL_UNITS:
            obj = os.path.join(tmp, f"{os.path.splitext(src)[0]}_{len(objs)}.o")
            cmds.append([hipcc, *COMMON, *DEVICE_FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        api_obj = os.path.join(tmp, "kvq_api.o")
        cmds.append([hipcc, *COMMON, "-c", os.path.join(CSRC, "kvq_api.cpp"), "-o", api_obj])
        objs.append(api_obj)
        jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1), 16)
        with cf.ThreadPoolExecutor(jobs) as ex:
            for out in ex.map(_run, cmds):
                if verbose and out.strip():
                    print(out)
        tmp_lib = LIB + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib])
        os.replace(tmp_lib, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
