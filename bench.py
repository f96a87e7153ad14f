#!/usr/bin/env python3
"""Benchmark: rotation + 2-bit KV-cache codec on the Llama-3-8B-shaped cache, one MI355X.

One step = the whole hot path over the full cache: encode K (RoPE + permutation + FWHT +
2-bit group-128 min-max + packing, 4 fp16 sinks), encode V (FWHT + 2-bit), decode K and
decode V back to bf16.  Inputs are resident in HBM before timing starts.

Prints one JSON line.  ``value`` = KV vectors encoded and decoded per second
(round trip: vectors / (encode time + decode time)), with per-kernel achieved HBM
bandwidth, the roofline of the dominant kernel, and the CPU oracle timed on a bounded
sample of the same workload.

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
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU time budget of the oracle sample")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain device copy of known size (for counter calibration)")
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


def cpu_baseline(inputs, cases, perm, budget_s: float, max_rows: int):
    """Time the CPU oracle (one thread) on whole rows of the cache -- all 32768 tokens x 8
    heads of row r of K, then of V, for r = 0, 1, ... -- until ``budget_s`` of CPU time
    has been spent or ``max_rows`` rows are done.  Returns (vectors, seconds, rows)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle
    from oracle.codec import CodecParams

    n_vec = 0
    t_total = 0.0
    rows_done = 0
    with threadpool_limits(limits=1):
        for r in range(max_rows):
            for case in cases:
                raw = inputs[case.name][r:r + 1].cpu().view(torch.int16).numpy().view(np.uint16)
                p = CodecParams(bits=case.bits, group_size=case.group_size, rope=case.rope, n_sink=case.n_sink,
                                perm=perm if case.use_perm else None)
                t0 = time.perf_counter()
                x64 = oracle.widen(raw, "bf16")
                planes = oracle.encode(x64, p)
                oracle.decode(planes, p, x64.shape)
                t_total += time.perf_counter() - t0
                n_vec += int(np.prod(raw.shape[:3]))
                del x64, planes
            rows_done += 1
            if t_total >= budget_s:
                break
    return n_vec, t_total, rows_done


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the codec is independent per vector and shards with no exchange step, see the design notes.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import rotate_then_bit_amd as kvq
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
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
        dst.copy_(src)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(3):
            dst.copy_(src)
        b.record(stream)
        stream.synchronize()
    copy_gbps = 2 * half * 3 / (a.elapsed_time(b) * 1e-3) / 1e9
    del dst

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
        for _ in range(3):
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

    cpu = None
    if not args.no_cpu_baseline:
        nv, tc, nrows = cpu_baseline(data["inputs"], wl.cases, perm, args.cpu_seconds, 16)
        cpu = {"value": round(nv / tc, 1), "unit": "vectors/s", "cores": 1, "kind": "oracle",
               "sample": f"{WORKLOAD} K and V rows 0-{nrows - 1}, all 32768 tokens x 8 heads ({nv} vectors, "
                         f"sinks included), encode+decode, float64 numpy, 1 thread",
               "seconds": round(tc, 2)}

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
        "append": {"us_per_step": round(append_us, 2), "vectors_per_step": append_vec,
                   "what": "decode-step cache update: K and V of every row appended at per-row positions "
                           "(kvq_append, K with RoPE + perm), launch-latency bound"},
        "roofline": dict(
            {"kernel": dominant, "bound": dk["bound"]},
            **({"achieved": dk["valu_Tops"], "peak": round(VALU_PEAK_TOPS, 2), "unit": "Tops/s (32-bit VALU lane ops)",
                "frac": dk["valu_frac"], "algorithmic_ops": dk["ops"]}
               if dk["bound"] == "alu" else
               {"achieved": dk["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": dk["frac_peak"]}),
            **{"hbm_achieved_GBps": dk["GBps"], "hbm_frac": dk["frac_peak"],
               "traffic": (round(traffic / (dk["avg_ms"] * 1e-3) / 1e9, 1) if traffic else None),
               "algorithmic_bytes": dk["bytes"], "traffic_bytes": traffic}),
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
