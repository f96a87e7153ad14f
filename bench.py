#!/usr/bin/env python3
"""Benchmark: rotation + 2-bit KV-cache codec on the Llama-3-8B-shaped cache, one MI355X.

One step = the whole hot path over the full cache: encode K (RoPE + permutation + FWHT +
2-bit group-128 min-max + packing, 4 fp16 sinks), encode V (FWHT + 2-bit), decode K and
decode V back to bf16.  Inputs are resident in HBM before timing starts.

Prints one JSON line.  ``value`` = KV vectors encoded and decoded per second
(round trip: vectors / (encode time + decode time)), with per-kernel achieved HBM
bandwidth, the HBM roofline of the slowest codec launch (its VALU fraction beside it),
the CPU oracle timed on a bounded sample of the same workload (one core, then a process
pool over the host's cores), and, outside the timed step, per-launch times of the other
workloads (the wide-head cache at full size; the Llama-2 layer, tiny and IsoQuant
workloads flagged as cache-resident or launch-bound), the decode-step append and the
decode-step attention over the encoded cache.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KV vectors encoded+decoded/sec and achieved HBM GB/s (% peak), d=128 2-bit"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD published peak
MFMA_INT8_PEAK_TOPS = 5000.0  # MI355X dense int8 matrix-core peak, AMD published (no sparsity)
# 32-bit VALU peak in lane operations: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (one add, mul,
# fma, min, max or convert per lane per cycle; packed two-wide FP32 is not used by these
# kernels, so the published 157.3 TFLOP/s -- FMA = 2 flops, two lanes per packed op -- is
# 4x this figure in flops and 2x in operations)
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# Algorithmic operations per vector element at 2-bit, one per element per step of the
# method: encode = widen 16-bit to fp32, 7 butterfly stages (log2 128), min and max,
# affine + round to an integer, merge the code into its word (+ 2 for the RoPE pair
# rotation on K: one mul and one fma per output); decode = unpack, dequantize (fma),
# 7 butterfly stages, narrow to the output type.  The permutation is data movement.
OPS_PER_ELEMENT = {("encode", "K"): 1 + 7 + 2 + 2 + 1 + 2, ("encode", "V"): 1 + 7 + 2 + 2 + 1,
                   ("decode", "K"): 1 + 1 + 7 + 1, ("decode", "V"): 1 + 1 + 7 + 1}
WORKLOAD = "llama3"
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "llama3_cache_hbm_counters.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "rotate_then_bit_amd", "csrc", f)
                  for f in ("kvq_kernels.hip", "kvq_internal.h")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="CPU time of the oracle's single-core leg (the pool leg does about twice as much work)")
    ap.add_argument("--cpu-workers", type=int, default=16, help="at most this many processes in the oracle's pool leg")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the per-launch timings of the wide-head, Llama-2 layer, tiny and IsoQuant workloads")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain device copy of known size (for counter calibration)")
    ap.add_argument("--only-other-configs", action="store_true",
                    help="run only the other workloads' timings (wide-head cache with its attention, Llama-2 layer, "
                         "tiny, IsoQuant, dynamic codebook, baseline rotations) and print them as one JSON line; "
                         "for profiling those launches")
    ap.add_argument("--other-keys", default=",".join(OTHER_CONFIGS),
                    help="with --only-other-configs: the workloads to time (comma-separated)")
    ap.add_argument("--no-other-reports", action="store_true",
                    help="with --only-other-configs: skip the dynamic-codebook and baseline-rotation reports")
    return ap.parse_args()


def plane_bytes(planes) -> int:
    return sum(int(v.numel() * v.element_size()) for v in planes.values())


def traffic_from_profile(kernel_name: str):
    """HBM bytes per launch measured with rocprofv3 counters, if taken on this kernel source."""
    if not os.path.exists(PROFILE_COUNTERS):
        return None
    txt = open(PROFILE_COUNTERS).read()
    m = re.search(r"^source_hash\s+(\S+)", txt, re.M)
    if not m or m.group(1) != kernel_source_hash():
        return None
    m = re.search(rf"^traffic_bytes_per_launch\s+{re.escape(kernel_name)}\s+(\d+)", txt, re.M)
    return int(m.group(1)) if m else None


def _pool_init():
    """Pool worker start-up: import what the oracle blocks need (outside the timing)."""
    import oracle  # noqa: F401
    import threadpoolctl  # noqa: F401


def _oracle_run(raw, t0, bits, group, rope, n_sink, perm):
    """Encode + decode one block of tokens (uint16 bf16 bits [1, T, H, D]) with the oracle,
    float64 numpy, one BLAS thread.  Returns (vectors, seconds)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from oracle.codec import CodecParams

    p = CodecParams(bits=bits, group_size=group, rope=rope, n_sink=n_sink, pos_offset=t0, perm=perm)
    with threadpool_limits(limits=1):
        t_start = time.perf_counter()
        x64 = oracle.widen(raw, "bf16")
        planes = oracle.encode(x64, p)
        oracle.decode(planes, p, x64.shape)
        dt = time.perf_counter() - t_start
    return int(np.prod(raw.shape[:3])), dt


def _oracle_block(job):
    """A pool task: one block read from a memory-mapped host copy of the rows.  job = (file,
    shape, row, t0, t1, bits, group, rope, n_sink, perm)."""
    import numpy as np

    path, shape, row, t0, t1, bits, group, rope, n_sink, perm = job
    raw = np.array(np.memmap(path, dtype=np.uint16, mode="r", shape=shape)[row:row + 1, t0:t1])
    return _oracle_run(raw, t0, bits, group, rope, n_sink, perm)


def cpu_baseline(pool, n_workers, inputs, cases, perm, budget_s: float):
    """The oracle timed on the host's cores, on whole rows of the cache (all 32768 tokens x 8
    heads of row r of K, then of V), in blocks of 4096 tokens (each block encoded at its own
    positions; the sinks fall in the first).

    Leg 1: this process, one BLAS thread, rows 0, 1, ... until ``budget_s`` of CPU time.
    Leg 2: a pool of ``n_workers`` processes (one BLAS thread each) over the next rows, about
    2 x ``budget_s`` of CPU work in all; vectors per wall-clock second of the whole pool."""
    import shutil
    import tempfile

    import numpy as np
    from threadpoolctl import threadpool_info

    import torch

    blk = 4096
    r_all, t_all = cases[0].shape[0], cases[0].shape[1]

    def host_rows(c, r0, r1):
        return inputs[c.name][r0:r1].cpu().view(torch.int16).numpy().view(np.uint16)

    # leg 1: one core
    n1, c1, r = 0, 0.0, 0
    while r < r_all and c1 < budget_s:
        for c in cases:
            raw = host_rows(c, r, r + 1)
            for t0 in range(0, t_all, blk):
                n, dt = _oracle_run(raw[:, t0:t0 + blk], t0, c.bits, c.group_size, c.rope, c.n_sink,
                                    perm if c.use_perm else None)
                n1, c1 = n1 + n, c1 + dt
        r += 1
    rows1 = r
    # leg 2: the pool, on the next rows, about 2 * budget_s of CPU work; the rows are written
    # to memory-mapped host files first (outside the timing)
    per_row_s = c1 / max(rows1, 1)
    want = max(1, int(round(2.0 * budget_s / max(per_row_s, 1e-9))))
    r0, r1 = rows1, min(r_all, rows1 + want)
    tmp = tempfile.mkdtemp(prefix="kvq_bench_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        files = []
        for c in cases:
            host = host_rows(c, r0, r1)
            path = os.path.join(tmp, f"{c.name}.u16")
            mm = np.memmap(path, dtype=np.uint16, mode="w+", shape=host.shape)
            mm[...] = host
            mm.flush()
            files.append((path, host.shape, c))
            del mm, host
        jobs = [(path, shape, rr, t0, min(t0 + blk, t_all), c.bits, c.group_size, c.rope, c.n_sink,
                 perm if c.use_perm else None)
                for rr in range(r1 - r0) for path, shape, c in files for t0 in range(0, t_all, blk)]
        t_start = time.perf_counter()
        res = pool.map(_oracle_block, jobs, chunksize=1)
        wall = time.perf_counter() - t_start
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    n2 = sum(n for n, _ in res)
    c2 = sum(dt for _, dt in res)
    blas = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info() if i.get("user_api") == "blas"]
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(n2 / wall, 1), "unit": "vectors/s", "cores": n_workers, "kind": "oracle",
            "sample": (f"{WORKLOAD} K and V rows {r0}-{r1 - 1} ({n2} vectors; per row all 32768 tokens x 8 heads, "
                       f"in blocks of {blk} tokens), encode+decode, float64 numpy, a pool of {n_workers} processes "
                       f"with one BLAS thread each; vectors per wall-clock second"),
            "seconds_wall": round(wall, 2), "cpu_seconds": round(c2, 2),
            "single_core": {"value": round(n1 / c1, 1), "unit": "vectors/s", "cores": 1,
                            "sample": f"{WORKLOAD} K and V rows 0-{rows1 - 1} ({n1} vectors, sinks included), "
                                      f"one process, one BLAS thread",
                            "seconds": round(c1, 2)},
            "cpu_model": model, "numpy": np.__version__, "blas": blas}


# bytes per vector and what bounds a launch, for the workloads timed beside the Llama-3 step
OTHER_CONFIGS = ("widehead", "llama2", "tiny", "isoquant")
REGIME = {"widehead": "hbm", "llama2": "cache-resident (76.5 MB per direction fits the 256 MB last-level cache)",
          "tiny": "launch-bound (0.66 MB per direction)", "isoquant": "launch-bound (4.6 MB per direction)"}


def warm_up(go, stream, min_ms=30.0):
    """Launch go() for at least min_ms of GPU time before a timed run (batches of doubling size,
    at most 4095 calls): after host-side set-up the GPU clocks take some tens of milliseconds of
    load to come back up, and a first call (fresh memory, code loading) says little about the
    rest."""
    import torch
    total, k = 0.0, 1
    while total < min_ms and k < 4096:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(k):
            go()
        b.record(stream)
        stream.synchronize()
        total += a.elapsed_time(b)
        k *= 2


def time_other_configs(kvq, workloads, dev, stream, keys=None):
    """Per-launch times of the other workloads: encode, and decode to the input dtype, of each
    tensor; the wide-head cache at full size (drawn on the GPU), the others from the host."""
    import numpy as np
    import torch

    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
    res = {}
    kept = {}
    for key in (keys if keys is not None else OTHER_CONFIGS):
        wl = workloads.WORKLOADS[key]
        if wl.device_generated:
            data = workloads.device_workload(key, device=dev)
            inputs = data["inputs"]
            reps = 10
        else:
            data = workloads.host_workload(key)
            inputs = {}
            for c in wl.cases:
                a = data["inputs"][c.name]
                t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16) \
                    if c.dtype == "bf16" else torch.from_numpy(np.ascontiguousarray(a))
                inputs[c.name] = t.to(dev)
            reps = 50
        torch.cuda.synchronize()
        entry = {"workload": wl.title, "regime": REGIME[key], "launches": {}}
        for c in wl.cases:
            cb = None
            if c.quant == "lloyd":
                cb = kvq.lloyd_max_gaussian(c.bits, c.lloyd_sigma or 1.0 / np.sqrt(c.shape[-1]))
            cfg = kvq.Config(shape=c.shape, dtype=c.dtype, bits=c.bits, group_size=c.group_size, quant=c.quant,
                             rot=c.rot, rope=c.rope, rope_base=c.rope_base, n_sink=c.n_sink,
                             perm=data["perm"] if c.use_perm else None, quat=data["quat"], codebook=cb)
            x = inputs[c.name]
            planes = kvq.empty_planes(cfg, device=dev)
            y = torch.empty(c.shape, dtype=tdt[c.dtype], device=dev)
            in_b = int(x.numel() * x.element_size())
            pl_b = plane_bytes(planes)
            for kind in ("encode", "decode"):
                def go():
                    if kind == "encode":
                        kvq.encode(x, cfg, planes=planes, stream=stream)
                    else:
                        kvq.decode(planes, cfg, out_dtype=c.dtype, out=y, stream=stream)
                with torch.cuda.stream(stream):
                    warm_up(go, stream)
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    for _ in range(reps):
                        go()
                    b.record(stream)
                    stream.synchronize()
                ms = a.elapsed_time(b) / reps
                nbytes = in_b + pl_b
                entry["launches"][f"{kind}_{c.name}"] = {
                    "avg_ms": round(ms, 5), "vectors": c.n_vectors,
                    "vectors_per_s": round(c.n_vectors / (ms * 1e-3), 1), "bytes": nbytes,
                    "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                    "frac_peak": round(nbytes / (ms * 1e-3) / (HBM_PEAK_GBPS * 1e9), 4)}
            kept[c.name] = (cfg, planes)
            del y
        if key == "widehead":
            entry["attend"] = time_attend_general(kvq, kept, dev, stream)
            print(f"[bench] widehead attend: {entry['attend']['ms_per_step']:.4g} ms, "
                  f"{entry['attend']['hbm_frac']:.3f} of HBM", file=sys.stderr, flush=True)
        kept.clear()
        res[key] = entry
        del inputs, data
        torch.cuda.empty_cache()
        print(f"[bench] {key}: " + ", ".join(f"{k} {v['avg_ms']:.4g} ms" for k, v in entry["launches"].items()),
              file=sys.stderr, flush=True)
    return res


def time_attend_general(kvq, kept, dev, stream, qg=2, reps=20):
    """Decode-step attention over the wide-head cache just encoded (K 2-bit and V 4-bit in groups
    of 32, head_dim 256; 2 query heads per KV head): the general vector-ALU pass, every slot of
    every row.  Bytes: the encoded K and V planes, read once."""
    import torch
    (cfg_k, pk), (cfg_v, pv) = kept["K"], kept["V"]
    r, t, h, d = cfg_k.shape
    gen = torch.Generator(device=dev).manual_seed(5)
    q = torch.randn((r, qg * h, d), generator=gen, device=dev, dtype=torch.float32)
    out = torch.empty_like(q)
    ws = torch.empty(kvq.attend_workspace_size(cfg_k, qg * h, cfg_v), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        warm_up(lambda: kvq.attend(q, pk, cfg_k, pv, cfg_v, out=out, workspace=ws, stream=stream), stream)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            kvq.attend(q, pk, cfg_k, pv, cfg_v, out=out, workspace=ws, stream=stream)
        b.record(stream)
        stream.synchronize()
    ms = a.elapsed_time(b) / reps
    nbytes = plane_bytes(pk) + plane_bytes(pv)
    return {"ms_per_step": round(ms, 4), "rows": r, "slots": t, "kv_heads": h, "q_heads": qg * h,
            "encoded_cache_bytes": nbytes, "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / (HBM_PEAK_GBPS * 1e9), 4),
            "what": "kvq_attend general pass (vector ALUs): scores and value sums in the rotated domain over "
                    "K 2-bit and V 4-bit codes, groups of 32, head_dim 256"}


def dynamic_codebook_report(kvq, workloads, dev, stream):
    """IsoQuant's dynamic codebook against the static one, SO(4) + 3-bit Lloyd-Max: the SNR of
    the round trip (dB over the non-sink vectors) and the encode/decode times, on the IsoQuant
    workload (N(0,1), every channel alike) and on the Llama-2 layer's K (4 outlier channels x20,
    token 0 x50), calibrated on the same tensor."""
    import numpy as np
    import torch

    res = {}
    for key, name in (("isoquant", "X"), ("llama2", "K")):
        wl = workloads.WORKLOADS[key]
        c = wl.case(name)
        h = workloads.host_workload(key)
        a = h["inputs"][name]
        x = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        d = c.shape[-1]
        quat = h["quat"] if h["quat"] is not None else workloads.unit_quaternions(d // 4, np.random.default_rng(1))
        base = dict(shape=c.shape, dtype=c.dtype, bits=3, quant="lloyd", rot="so4", quat=quat, n_sink=c.n_sink)
        static = kvq.Config(**base, codebook=kvq.lloyd_max_gaussian(3, 1.0 / np.sqrt(d)))
        m = kvq.rotated_moments(x, kvq.Config(**base, codebook=kvq.lloyd_max_gaussian(3, 1.0)), stream=stream)
        torch.cuda.synchronize()
        sc, wide, cb, cbw = kvq.dynamic_codebook(m.cpu().numpy(), 3)
        dyn = kvq.Config(**base, codebook=cb, chan_scale=sc, chan_wide=wide, codebook_wide=cbw)
        xf = x.float()
        keep = slice(c.n_sink, None)
        entry = {"workload": wl.title, "rotation": "so4", "bits": 3}
        for label, cfg in (("static", static), ("dynamic", dyn)):
            pl = kvq.encode(x, cfg, stream=stream)
            y = kvq.decode(pl, cfg, out_dtype="f32", stream=stream)
            torch.cuda.synchronize()
            err = (y[:, keep] - xf[:, keep]).double().pow(2).sum().item()
            sig = xf[:, keep].double().pow(2).sum().item()
            t = {}
            for kind in ("encode", "decode"):
                with torch.cuda.stream(stream):
                    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    ev[0].record(stream)
                    for _ in range(20):
                        if kind == "encode":
                            kvq.encode(x, cfg, planes=pl, stream=stream)
                        else:
                            kvq.decode(pl, cfg, out_dtype="f32", out=y, stream=stream)
                    ev[1].record(stream)
                    stream.synchronize()
                t[kind] = round(ev[0].elapsed_time(ev[1]) / 20 * 1e3, 2)
            entry[label] = {"snr_db": round(10 * np.log10(sig / err), 3), "encode_us": t["encode"], "decode_us": t["decode"]}
        entry["snr_gain_db"] = round(entry["dynamic"]["snr_db"] - entry["static"]["snr_db"], 3)
        res[key] = entry
        print(f"[bench] dynamic codebook {key}: {entry['static']['snr_db']} -> {entry['dynamic']['snr_db']} dB",
              file=sys.stderr, flush=True)
    return res


MFMA_F32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix peak


def baseline_rotations_report(kvq, workloads, dev, stream, n_big=1 << 21):
    """The rotations the IsoQuant page (section 1) compares -- its SO(4) blocks, the Walsh-Hadamard
    transform, TurboQuant's dense random orthogonal matrix and RotorQuant's 3-D rotors -- in one
    codec: norm separation + 3-bit Lloyd-Max for N(0, 1/128), fp32 input, d = 128.  Quality: SNR
    of the round trip on the IsoQuant workload (8192 N(0,1) vectors).  Speed: encode and decode of
    that 8192-vector batch (the batch of the page's benchmark), and of 2^21 vectors drawn the same
    way, with GB/s and, for the matrix rotations (on the fp32 matrix cores), TFLOP/s of the
    2 * 128 * 128 flops per vector against the 157.3 TFLOP/s fp32 matrix peak."""
    import numpy as np
    import torch

    d = 128
    wl = workloads.WORKLOADS["isoquant"]
    c = wl.case("X")
    h = workloads.host_workload("isoquant")
    x_small = torch.from_numpy(np.ascontiguousarray(h["inputs"]["X"])).to(dev)
    gen = torch.Generator(device=dev).manual_seed(11)
    x_big = torch.randn((1, n_big, 1, d), generator=gen, device=dev, dtype=torch.float32)
    rng = np.random.default_rng(2024)
    haar = torch.from_numpy(workloads.haar_orthogonal(d, rng)).to(dev)
    rq, ta = workloads.rotor_quaternions(d, rng)
    rotor = torch.from_numpy(kvq.rotor_matrix(rq, d, ta)).to(dev)
    cb = kvq.lloyd_max_gaussian(3, 1.0 / np.sqrt(d))
    kinds = {"so4 (IsoQuant)": dict(rot="so4", quat=h["quat"]), "fwht": dict(rot="fwht"),
             "dense (TurboQuant)": dict(rot="dense", rot_matrix=haar),
             "rotor (RotorQuant)": dict(rot="rotor", rotor_quat=rq, rotor_tail=ta),
             "rotor (RotorQuant, as its block-diagonal matrix)": dict(rot="dense", rot_matrix=rotor)}
    lw = workloads.WORKLOADS["llama2"]
    lk = lw.case("K")
    lh = workloads.host_workload("llama2")
    x_out = torch.from_numpy(np.ascontiguousarray(lh["inputs"]["K"])).to(dev).float()
    res = {"workload": "norm separation + 3-bit Lloyd-Max, fp32, d = 128; SNR on " + wl.title +
                       " and on the Llama-2 layer's K (4 outlier channels x20; sink tokens left out)",
           "big_vectors": n_big, "rotations": {}}
    for label, kw in kinds.items():
        entry = {}
        for size, x in (("batch_8192", x_small), ("big", x_big)):
            cfg = kvq.Config(shape=tuple(x.shape), dtype="f32", bits=3, quant="lloyd", codebook=cb, **kw)
            pl = kvq.encode(x, cfg, stream=stream)
            y = kvq.decode(pl, cfg, out_dtype="f32", stream=stream)
            torch.cuda.synchronize()
            if size == "batch_8192":
                err = (y - x).double().pow(2).sum().item()
                entry["snr_db"] = round(10 * np.log10(x.double().pow(2).sum().item() / err), 3)
            n = int(x.numel() // d)
            reps = 50 if size == "batch_8192" else 5
            for kind in ("encode", "decode"):
                with torch.cuda.stream(stream):
                    def go():
                        if kind == "encode":
                            kvq.encode(x, cfg, planes=pl, stream=stream)
                        else:
                            kvq.decode(pl, cfg, out_dtype="f32", out=y, stream=stream)
                    warm_up(go, stream)
                    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    ev[0].record(stream)
                    for _ in range(reps):
                        go()
                    ev[1].record(stream)
                    stream.synchronize()
                ms = ev[0].elapsed_time(ev[1]) / reps
                nbytes = n * d * 4 + plane_bytes(pl)
                e = {"us": round(ms * 1e3, 2), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}
                if kw["rot"] == "dense":
                    tf = 2.0 * d * d * n / (ms * 1e-3) / 1e12
                    e["TFLOPs"] = round(tf, 2)
                    e["mfma_f32_frac"] = round(tf / MFMA_F32_PEAK_TFLOPS, 4)
                entry[f"{kind}_{size}"] = e
            del pl, y
        # quality where a few channels carry most of the energy: global mixing spreads them
        cfg = kvq.Config(shape=tuple(x_out.shape), dtype="f32", bits=3, quant="lloyd", codebook=cb,
                         n_sink=lk.n_sink, **kw)
        pl = kvq.encode(x_out, cfg, stream=stream)
        y = kvq.decode(pl, cfg, out_dtype="f32", stream=stream)
        torch.cuda.synchronize()
        keep = slice(lk.n_sink, None)
        err = (y[:, keep] - x_out[:, keep]).double().pow(2).sum().item()
        entry["snr_db_outlier_channels"] = round(10 * np.log10(x_out[:, keep].double().pow(2).sum().item() / err), 3)
        del pl, y
        res["rotations"][label] = entry
        print(f"[bench] baseline {label}: SNR {entry['snr_db']} / {entry['snr_db_outlier_channels']} dB, "
              f"encode {entry['encode_batch_8192']['us']} us "
              f"/ 8192, big {entry['encode_big']['us']} us", file=sys.stderr, flush=True)
    del x_big, x_out
    torch.cuda.empty_cache()
    return res


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the codec is independent per vector and shards with no exchange step, see the design notes.",
              file=sys.stderr)
        sys.exit(2)

    # the CPU baseline's process pool is forked here, before anything touches the GPU
    pool, n_workers = None, 0
    if not args.no_cpu_baseline:
        import multiprocessing as mp
        n_workers = max(1, min(len(os.sched_getaffinity(0)), args.cpu_workers))
        pool = mp.get_context("fork").Pool(n_workers, initializer=_pool_init)

    import numpy as np
    import torch

    import rotate_then_bit_amd as kvq
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.only_other_configs:
        stream = torch.cuda.Stream(device=dev)  # default priority
        keys = [k for k in args.other_keys.split(",") if k]
        others = time_other_configs(kvq, workloads, dev, stream, keys=keys)
        if not args.no_other_reports:
            others["dynamic_codebook"] = dynamic_codebook_report(kvq, workloads, dev, stream)
            others["baseline_rotations"] = baseline_rotations_report(kvq, workloads, dev, stream)
        if args.calib_copy:
            a = torch.empty(1 << 33, dtype=torch.uint8, device=dev)
            b = torch.empty_like(a)
            b.copy_(a)
            torch.cuda.synchronize()
            del a, b
        print(json.dumps({"other_configs": others}), flush=True)
        return
    wl = workloads.WORKLOADS[WORKLOAD]
    t0 = time.time()
    data = workloads.device_workload(WORKLOAD, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] generated {WORKLOAD} inputs in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    perm = data["perm"]
    cases = {c.name: c for c in wl.cases}
    cfgs = {n: kvq.Config(shape=c.shape, dtype=c.dtype, bits=c.bits, group_size=c.group_size, rope=c.rope,
                          rope_base=c.rope_base, n_sink=c.n_sink, perm=perm if c.use_perm else None)
            for n, c in cases.items()}
    planes = {n: kvq.empty_planes(cfgs[n], device=dev) for n in cases}
    outs = {n: torch.empty(c.shape, dtype=torch.bfloat16, device=dev) for n, c in cases.items()}
    stream = torch.cuda.Stream(device=dev)  # default priority
    names = [("encode", "K"), ("encode", "V"), ("decode", "K"), ("decode", "V")]

    def launch(kind, n):
        if kind == "encode":
            kvq.encode(data["inputs"][n], cfgs[n], planes=planes[n], stream=stream)
        else:
            kvq.decode(planes[n], cfgs[n], out_dtype="bf16", out=outs[n], stream=stream)

    # algorithmic bytes per launch: every plane read or written once
    in_bytes = {n: int(data["inputs"][n].numel() * 2) for n in cases}
    pl_bytes = {n: plane_bytes(planes[n]) for n in cases}
    sink_bytes = {n: int(planes[n]["sink"].numel() * 2) if "sink" in planes[n] else 0 for n in cases}
    algo = {}
    for kind, n in names:
        if kind == "encode":
            algo[(kind, n)] = in_bytes[n] + pl_bytes[n]
        else:
            algo[(kind, n)] = pl_bytes[n] + in_bytes[n]  # planes read, bf16 output written

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            for kind, n in names:
                launch(kind, n)
        stream.synchronize()
        if args.calib_copy:
            src = data["inputs"]["K"]
            dst = torch.empty_like(src)
            dst.copy_(src)
            stream.synchronize()
            print(f"[bench] calibration copy: {src.numel() * 2} bytes read, {src.numel() * 2} written",
                  file=sys.stderr, flush=True)
            del dst
        ev = {key: [] for key in names}
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        start_ev = torch.cuda.Event(enable_timing=True)
        end_ev = torch.cuda.Event(enable_timing=True)
        start_ev.record(stream)
        for _ in range(args.steps):
            for key in names:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                launch(*key)
                b.record(stream)
                ev[key].append((a, b))
        end_ev.record(stream)
        stream.synchronize()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
    gpu_ms = start_ev.elapsed_time(end_ev)
    ms_per_step = gpu_ms / args.steps
    kern = {}
    for key in names:
        durs = [a.elapsed_time(b) for a, b in ev[key]]
        avg = sum(durs) / len(durs)
        gbps = algo[key] / (avg * 1e-3) / 1e9
        ops = OPS_PER_ELEMENT[key] * cases[key[1]].n_vectors * cases[key[1]].shape[-1]
        tops = ops / (avg * 1e-3) / 1e12
        # the binding roofline: the resource whose peak would take longer for this launch
        alu_bound = ops / (VALU_PEAK_TOPS * 1e12) > algo[key] / (HBM_PEAK_GBPS * 1e9)
        kern[f"{key[0]}_{key[1]}"] = {"avg_ms": round(avg, 4), "GBps": round(gbps, 1),
                                      "frac_peak": round(gbps / HBM_PEAK_GBPS, 4), "bytes": algo[key],
                                      "valu_Tops": round(tops, 2), "valu_frac": round(tops / VALU_PEAK_TOPS, 4),
                                      "ops": ops, "bound": "alu" if alu_bound else "hbm"}
    n_vec = cases["K"].n_vectors  # K and V vectors each
    n_kv = 2 * n_vec
    t_enc = sum(kern[f"encode_{n}"]["avg_ms"] for n in cases)
    t_dec = sum(kern[f"decode_{n}"]["avg_ms"] for n in cases)
    value = n_kv / ((t_enc + t_dec) * 1e-3)
    step_bytes = sum(algo.values())
    dominant = max(kern, key=lambda k: kern[k]["avg_ms"])
    dk = kern[dominant]
    traffic = traffic_from_profile(dominant)

    # context, outside the timed region: a plain device-to-device copy that moves the same
    # number of bytes as one launch (half read, half written)
    half = dk["bytes"] // 2
    src = data["inputs"]["K"].view(-1).view(torch.uint8)[:half]
    dst = torch.empty(half, dtype=torch.uint8, device=dev)
    with torch.cuda.stream(stream):
        warm_up(lambda: dst.copy_(src), stream)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(3):
            dst.copy_(src)
        b.record(stream)
        stream.synchronize()
    copy_gbps = 2 * half * 3 / (a.elapsed_time(b) * 1e-3) / 1e9
    # and torch's own write-only (fill) and read-only (sum) kernels over 8 GiB: what plain
    # streaming kernels reach on this GPU, next to the 8 TB/s of the data sheet
    big = torch.empty(data["inputs"]["K"].numel(), dtype=torch.bfloat16, device=dev)  # 8 GiB of its own
    ceil = {}
    with torch.cuda.stream(stream):
        for name, fn in (("write_fill", lambda: big.fill_(0.5)), ("read_sum", lambda: big.sum(dtype=torch.float32))):
            warm_up(fn, stream)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(3):
                fn()
            b.record(stream)
            stream.synchronize()
            ceil[name + "_GBps"] = round(big.numel() * big.element_size() * 3 / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
    ceil["copy_GBps"] = round(copy_gbps, 1)
    del dst, big

    # context, outside the timed region: one decode step's cache update -- every row's new K
    # and V token (its first token's values, here) appended at a random position of the
    # cache (a few thousand vectors per launch: launch-latency bound, reported in us)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    r0, t_cap = cases["K"].shape[0], cases["K"].shape[1]
    positions = torch.randint(0, t_cap, (r0,), generator=gen, device=dev, dtype=torch.int64)
    x_new = {n: data["inputs"][n][:, 0].contiguous() for n in cases}
    with torch.cuda.stream(stream):
        for _ in range(3):
            for n in cases:
                kvq.append(x_new[n], positions, planes[n], cfgs[n], stream=stream)
        stream.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        n_rep = 50
        a.record(stream)
        for _ in range(n_rep):
            for n in cases:
                kvq.append(x_new[n], positions, planes[n], cfgs[n], stream=stream)
        b.record(stream)
        stream.synchronize()
    append_us = a.elapsed_time(b) * 1e3 / n_rep
    append_vec = sum(int(x_new[n].shape[0] * x_new[n].shape[1]) for n in cases)

    # context, outside the timed region: one decode step of attention over the whole encoded
    # cache (every row at full length; Llama-3-8B's 32 query heads over its 8 KV heads), scored
    # and summed in the rotated domain without decoding a key
    r0, t0_, h0, d0 = cases["K"].shape
    q_heads = 4 * h0
    qa = torch.randn((r0, q_heads, d0), generator=gen, device=dev, dtype=torch.float32)
    oa = torch.empty_like(qa)
    wsa = torch.empty(kvq.attend_workspace_size(cfgs["K"], q_heads), dtype=torch.uint8, device=dev)
    with torch.cuda.stream(stream):
        # after a pause the GPU needs about 20 ms of this load to reach its steady clock (measured:
        # 0.59 ms for the first call after 2 s idle, 0.47 ms from about the 40th call on)
        for _ in range(60):
            kvq.attend(qa, planes["K"], cfgs["K"], planes["V"], cfgs["V"], out=oa, workspace=wsa, stream=stream)
        stream.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        n_rep = 30
        a.record(stream)
        for _ in range(n_rep):
            kvq.attend(qa, planes["K"], cfgs["K"], planes["V"], cfgs["V"], out=oa, workspace=wsa, stream=stream)
        b.record(stream)
        stream.synchronize()
    attend_ms = a.elapsed_time(b) / n_rep
    attend_bytes = pl_bytes["K"] + pl_bytes["V"]  # the encoded cache, read once
    bf16_bytes = in_bytes["K"] + in_bytes["V"]  # what the same attention reads from a bf16 cache
    # int8 matrix-core operations as issued (2 per multiply-add), per (slot, KV head): for the
    # keys two 16x16x64 products per 16 slots, for the values eight per 64 slots
    attend_mfma_ops = r0 * t0_ * h0 * 2 * (2 * 16 * 16 * 64 // 16 + 8 * 16 * 16 * 64 // 64)

    # context, outside the timed region: the RotateKV calibration passes over a slice of the
    # cache (8 rows of K: 2^23 vectors): per-channel statistics of the post-RoPE keys for the
    # outlier-aware permutation, and activation-based sink detection (token norms, median)
    cal_rows = 8
    ksl = data["inputs"]["K"][:cal_rows]
    cal_cfg = kvq.Config(shape=tuple(ksl.shape), dtype="bf16", bits=2, group_size=128, rope=True, n_sink=4)
    ws_cal = torch.empty(max(8, kvq.channel_stats_workspace_size(cal_cfg)), dtype=torch.uint8, device=dev)
    cal_t = {}
    with torch.cuda.stream(stream):
        for name, fn in (("channel_stats", lambda: kvq.channel_stats(ksl, cal_cfg, workspace=ws_cal, stream=stream)),
                         ("detect_sinks", lambda: kvq.detect_sinks(ksl, cal_cfg, 8.0, stream=stream))):
            warm_up(fn, stream)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(10):
                fn()
            b.record(stream)
            stream.synchronize()
            cal_t[name] = a.elapsed_time(b) / 10
    # the dynamic bit width's entropy pass over the same 8 rows of the encoded K cache (32 query
    # heads): per-query-head attention entropy, averaged per KV head, and the widths for an
    # average of 3 bits
    kpl = {n: v[:cal_rows] for n, v in planes["K"].items() if n != "sink"}
    kpl["sink"] = planes["K"]["sink"][:cal_rows]
    kcfg8 = kvq.Config(**{**cfgs["K"].__dict__, "shape": (cal_rows,) + tuple(cases["K"].shape[1:]), "_keep": []})
    q8 = torch.randn((cal_rows, 32, 128), generator=gen, device=dev, dtype=torch.float32)
    with torch.cuda.stream(stream):
        ent = kvq.attention_entropy(q8, kpl, kcfg8, stream=stream)
        stream.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(5):
            kvq.attention_entropy(q8, kpl, kcfg8, out=ent, stream=stream)
        b.record(stream)
        stream.synchronize()
    cal_t["attention_entropy"] = a.elapsed_time(b) / 5
    e_head = ent.double().view(cal_rows, 8, 4).mean(dim=(0, 2)).cpu().numpy()
    widths = kvq.allocate_bits(e_head, 3 * 8)
    cal_bytes = int(ksl.numel() * 2)
    calib = {"slice": f"K rows 0-{cal_rows - 1} of the cache ({int(ksl.shape[0] * ksl.shape[1] * ksl.shape[2])} vectors, "
                      f"{cal_bytes} bytes read)",
             **{k: {"ms": round(v, 4), "GBps": round(cal_bytes / (v * 1e-3) / 1e9, 1),
                    "hbm_frac": round(cal_bytes / (v * 1e-3) / (HBM_PEAK_GBPS * 1e9), 4)}
                for k, v in cal_t.items() if k != "attention_entropy"},
             "attention_entropy": {"ms": round(cal_t["attention_entropy"], 4),
                                   "what": "entropy of 32 query heads' softmax over the 8 rows' encoded K "
                                           "(36 bytes per vector) in the rotated domain",
                                   "head_entropy_nats": [round(float(v), 4) for v in e_head],
                                   "widths_for_3_bits_average": widths.tolist()},
             "what": "calibration passes, run once, not per step: RotateKV per-channel mean |post-RoPE key| for "
                     "the outlier-aware permutation (kvq_channel_stats), sink detection by token norm against "
                     "lambda x the row median (kvq_detect_sinks); IsoQuant attention entropy for per-head "
                     "bit widths (kvq_attention_entropy, kvq_allocate_bits)"}
    del ksl, ws_cal

    cpu = None
    if pool is not None:
        cpu = cpu_baseline(pool, n_workers, data["inputs"], wl.cases, perm, args.cpu_seconds)
        pool.close()
        pool.join()
        print(f"[bench] oracle: {cpu['value']:.3g} vectors/s on {n_workers} cores, "
              f"{cpu['single_core']['value']:.3g} on one", file=sys.stderr, flush=True)

    others = None
    if not args.no_other_configs:
        del data, planes, outs, qa, oa, wsa, x_new, src
        torch.cuda.empty_cache()
        others = time_other_configs(kvq, workloads, dev, stream)
        others["dynamic_codebook"] = dynamic_codebook_report(kvq, workloads, dev, stream)
        others["baseline_rotations"] = baseline_rotations_report(kvq, workloads, dev, stream)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) bf16 with 3 outlier channels x15, generated on the GPU)",
        "config": {"workload": "llama3-8b-kv-cache: 32 layers x batch 4 = 128 rows, 32768 tokens, 8 KV heads, "
                               "d=128, bf16; K: RoPE+perm+FWHT, V: FWHT; 2-bit, group 128, fp16 scale/zero, "
                               "4 fp16 sinks",
                   "rows": 128, "tokens": 32768, "heads": 8, "head_dim": 128, "bits": 2, "group_size": 128,
                   "n_sink": 4, "io_dtype": "bf16", "vectors_per_step": n_kv},
        "hbm_GBps_step": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "encode_vectors_per_s": round(n_kv / (t_enc * 1e-3), 1),
        "decode_vectors_per_s": round(n_kv / (t_dec * 1e-3), 1),
        "compression_ratio": round(in_bytes["K"] / (pl_bytes["K"] - sink_bytes["K"]), 3),
        "kernels": kern,
        "copy_GBps_same_bytes": round(copy_gbps, 1),
        "hbm_streaming_kernels": ceil,
        "attend": {"ms_per_step": round(attend_ms, 4), "rows": r0, "slots": t0_, "kv_heads": h0, "q_heads": q_heads,
                   "encoded_cache_bytes": attend_bytes,
                   "GBps": round(attend_bytes / (attend_ms * 1e-3) / 1e9, 1),
                   "bf16_cache_bytes": bf16_bytes,
                   "bf16_cache_read_at_hbm_peak_ms": round(bf16_bytes / (HBM_PEAK_GBPS * 1e9) * 1e3, 4),
                   "hbm_frac": round(attend_bytes / (attend_ms * 1e-3) / (HBM_PEAK_GBPS * 1e9), 4),
                   "mfma_int8_ops": attend_mfma_ops,
                   "mfma_int8_frac": round(attend_mfma_ops / (attend_ms * 1e-3) / (MFMA_INT8_PEAK_TOPS * 1e12), 4),
                   "what": "decode-step attention over the encoded K/V cache in the rotated domain "
                           "(kvq_attend): exact int8 matrix-core products of the codes with 8-bit digits of "
                           "the rotated queries and of the softmax weights"},
        "calibration": calib,
        "append": {"us_per_step": round(append_us, 2), "vectors_per_step": append_vec,
                   "what": "decode-step cache update: K and V of every row appended at per-row positions "
                           "(kvq_append, K with RoPE + perm), launch-latency bound"},
        # the slowest codec launch against the HBM roofline (the 8.0 TB/s target); its VALU
        # fraction beside it (the encoders' arithmetic is above the plain-VALU ridge)
        "roofline": {"kernel": dominant, "bound": "hbm", "achieved": dk["GBps"], "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": dk["frac_peak"], "traffic": traffic,
                     "algorithmic_bytes": dk["bytes"], "avg_ms": dk["avg_ms"],
                     "valu": {"achieved": dk["valu_Tops"], "peak": round(VALU_PEAK_TOPS, 2),
                              "unit": "Tops/s (32-bit VALU lane ops)", "frac": dk["valu_frac"],
                              "algorithmic_ops": dk["ops"]}},
        "other_configs": others,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
