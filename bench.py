#!/usr/bin/env python3
"""Benchmark of the mxq hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload grouped_nvfp4_rht|...] [--no-cpu-baseline]

A step is one call of the quantizer over one batch of seeded synthetic input that
is already resident in HBM.  The default workload is grouped NVFP4 with the
16-point RHT, row-wise + column-wise, 16384 x 4096 BF16 in 8 MoE sections (the
configuration the headline metric is quoted on).  The timed steps run back to back
and cycle over several copies of the input and outputs, together far larger than
the 256 MB Infinity Cache, so each call reads its input from HBM and pays for the
write-back of earlier calls' outputs, as a stream of calls would; ms_per_step is
the HIP-event time of the whole run on the kernels' stream divided by the steps
(two events around the K calls, nothing enqueued between them).
Secondary figures: a single call after a 1 GiB read has cleared the caches of the
input (without leaving dirty lines behind), and back-to-back calls on one input
(warm caches).  Prints ONE JSON line.
"""
import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="grouped_nvfp4_rht",
                    choices=["grouped_nvfp4_rht", "grouped_nvfp4_rht_sr", "large_moe_nvfp4_fp8",
                             "dsa_rotate_fp8", "dsa_rotate_nvfp4", "swiglu_fp8", "fp8_blockwise", "fp8_1x128"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="steady-state steps only, then one 256 MiB device copy (the counter calibration "
                         "for rocprofv3 runs); prints the JSON line without the secondary figures")
    ap.add_argument("--cpu-sample-rows", type=int, default=0,
                    help="rows of the workload the oracle baseline runs on (0: the whole workload, "
                         "capped at 16384 rows)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path. Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import nvfp4_quantization_amd as mxq
    from nvfp4_quantization_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()

    # ---------------------------------------------------------------- workload
    wl = args.workload
    grouped = wl not in ("fp8_1x128", "dsa_rotate_fp8", "dsa_rotate_nvfp4", "swiglu_fp8", "fp8_blockwise")
    if wl == "fp8_1x128":
        w = synth.plain_fp8(device=dev)
        x = w.tensors["x"]
        m, k = x.shape

        def make_call(x=x):
            xi = x.clone()
            q = torch.empty((m, k), dtype=torch.uint8, device=dev)
            s = torch.empty((m, k // 128), dtype=torch.float32, device=dev)
            return lambda: mxq.mxq_quant_fp8_1x128(xi, q=q, scales=s)
        call = make_call()
        in_bytes = m * k * 2
        alg_bytes = in_bytes + m * k + m * k // 128 * 4
        desc = f"fp8_1x128 {m}x{k} bf16"
    elif wl == "dsa_rotate_fp8":
        w = synth.dsa_rotate_fp8(device=dev)
        pe, nope = w.tensors["pe"], w.tensors["nope"]
        m = pe.shape[0]

        def make_call():
            pi, ni = pe.clone(), nope.clone()
            q = torch.empty((m, 128), dtype=torch.uint8, device=dev)
            s = torch.empty((m,), dtype=torch.float32, device=dev)
            return lambda: mxq.mxq_hadamard_quant_fp8(pi, ni, q=q, scales=s)
        call = make_call()
        in_bytes = m * 128 * 2
        alg_bytes = in_bytes + m * 128 + m * 4
        desc = f"dsa cat+WHT128+fp8_1x128, {m} rows (4096 tokens x 64 heads) bf16"
    elif wl == "fp8_blockwise":
        x = synth.grouped_nvfp4(device=dev).tensors["x"]
        m, k = x.shape

        def make_call(x=x):
            xi = x.clone()
            return lambda: mxq.mxq_quant_fp8_blockwise(xi, mxq.MXQ_FP8_UE8M0, rowwise=True, columnwise=True)
        call = make_call()
        in_bytes = m * k * 2
        alg_bytes = in_bytes + 2 * (m * k + m * (k // 128) * 4)
        desc = f"fp8 row-wise 1x128 + column-wise 128x1 (transposed), UE8M0 scales, {m}x{k} bf16"
    elif wl == "swiglu_fp8":
        w = synth.swiglu_fp8(device=dev)
        gu = w.tensors["gate_up"]
        m, n = gu.shape[0], gu.shape[1] // 2

        def make_call():
            gi = gu.clone()
            q = torch.empty((m, n), dtype=torch.uint8, device=dev)
            s = torch.empty((m, n // 128), dtype=torch.float32, device=dev)
            return lambda: mxq.mxq_swiglu_quant_fp8(gi[:, :n], gi[:, n:], q=q, scales=s)
        call = make_call()
        in_bytes = m * n * 2 * 2
        alg_bytes = in_bytes + m * n + m * (n // 128) * 4
        desc = f"swiglu -> fp8_1x128, {m} tokens x {n} (fused gate|up bf16 buffer)"
    elif wl == "dsa_rotate_nvfp4":
        w = synth.dsa_rotate_fp8(device=dev)
        pe, nope = w.tensors["pe"], w.tensors["nope"]
        m = pe.shape[0]
        dsa_ws = torch.zeros((mxq.mxq_hadamard_quant_nvfp4_workspace_size(m),), dtype=torch.uint8, device=dev)

        def make_call():
            return mxq.HadamardNVFP4(pe.clone(), nope.clone(), workspace=dsa_ws)
        call = make_call()
        in_bytes = m * 128 * 2
        alg_bytes = in_bytes + m * 64 + m * 8 + 4
        desc = f"dsa cat+WHT128+nvfp4 row-wise (one tensor scale, measured), {m} rows (4096 tokens x 64 heads) bf16"
    else:
        gen = {"grouped_nvfp4_rht": synth.grouped_nvfp4, "grouped_nvfp4_rht_sr": synth.grouped_nvfp4_sr,
               "large_moe_nvfp4_fp8": synth.large_moe}[wl]
        w = gen(device=dev)
        p = w.params
        x = w.tensors["x"]
        total, k = x.shape
        S = len(p["split_sections"])
        workspace = mxq.alloc_workspace(total, k, S, p["flags"], dev)

        def make_call():
            return mxq.GroupedNVFP4(x.clone(), p["split_sections"], p["sign_mask"], p["flags"], p["seed"],
                                    p["row_offsets"], p["col_offsets"], workspace=workspace)
        call = make_call()
        in_bytes = total * k * 2
        alg_bytes = in_bytes
        if p["flags"] & 1:
            alg_bytes += total * k // 2 + total * k // 16 + S * 4
        if p["flags"] & 2:
            alg_bytes += total * k // 2 + total * k // 16 + S * 4
        if p["flags"] & 4:
            alg_bytes += total * k + total * k // 128 * 4
        outs = {1: "row", 2: "col", 4: "fp8"}
        desc = (f"{wl} {total}x{k} bf16, {S} sections, outputs "
                f"{'+'.join(v for b, v in outs.items() if p['flags'] & b)}, "
                f"{'stochastic rounding' if p['seed'] is not None else 'RNE'}")

    # ---------------------------------------------------------------- input / output sets
    # Steady state: the timed calls cycle over enough copies of the input and the
    # outputs (together well over the 256 MB Infinity Cache) that every call reads
    # its input from HBM, and pays for the write-back of earlier calls' outputs as
    # a stream of calls would.
    set_bytes = alg_bytes
    n_sets = max(3, -(-(5 << 28) // set_bytes))
    calls = [call] + [make_call() for _ in range(n_sets - 1)]

    # ---------------------------------------------------------------- warmup
    for i in range(args.warmup):
        calls[i % n_sets]()
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed steps
    # K calls back to back between two events on the call's stream, synchronized on
    # both sides.  Nothing else is enqueued inside the timed region: an event
    # recorded between calls costs the stream 3-4 us of its own.
    K = args.steps
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for i in range(K):
        calls[i % n_sets]()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = t_start.elapsed_time(t_end) / K                    # throughput: whole run / steps

    # the spread over calls: K more, each between events of its own (so each figure
    # also holds the events' cost)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for i in range(K):
        starts[i].record(stream)
        calls[i % n_sets]()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))

    # per-kernel times of K more steady-state calls, from launch marks the library
    # records on the call's stream around each of its kernels
    kern = None
    if grouped:
        kern = kernel_times(mxq, torch, calls, n_sets, K, stream, ("k_nvfp4_amax", "k_nvfp4_quant"))
    elif wl == "fp8_blockwise":
        x = synth.grouped_nvfp4(device=dev).tensors["x"]
        m, k = x.shape

        def make_call(x=x):
            xi = x.clone()
            return lambda: mxq.mxq_quant_fp8_blockwise(xi, mxq.MXQ_FP8_UE8M0, rowwise=True, columnwise=True)
        call = make_call()
        in_bytes = m * k * 2
        alg_bytes = in_bytes + 2 * (m * k + m * (k // 128) * 4)
        desc = f"fp8 row-wise 1x128 + column-wise 128x1 (transposed), UE8M0 scales, {m}x{k} bf16"
    elif wl == "swiglu_fp8":
        w = synth.swiglu_fp8(device=dev)
        gu = w.tensors["gate_up"]
        m, n = gu.shape[0], gu.shape[1] // 2

        def make_call():
            gi = gu.clone()
            q = torch.empty((m, n), dtype=torch.uint8, device=dev)
            s = torch.empty((m, n // 128), dtype=torch.float32, device=dev)
            return lambda: mxq.mxq_swiglu_quant_fp8(gi[:, :n], gi[:, n:], q=q, scales=s)
        call = make_call()
        in_bytes = m * n * 2 * 2
        alg_bytes = in_bytes + m * n + m * (n // 128) * 4
        desc = f"swiglu -> fp8_1x128, {m} tokens x {n} (fused gate|up bf16 buffer)"
    elif wl == "dsa_rotate_nvfp4":
        kern = kernel_times(mxq, torch, calls, n_sets, K, stream,
                            ("k_dsa_nvfp4_amax", "k_dsa_nvfp4_quant"))

    if args.profile:
        del calls
        a = torch.ones(1 << 27, dtype=torch.int16, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)                                        # 256 MiB read + 256 MiB written
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": True, "workload": desc, "steps": K, "ms_per_step": round(ms, 5),
                          "kernel_avg_us_live": kern, "copy_calibration_bytes": 2 * a.numel()}), flush=True)
        return

    # secondary figures: one call after reading a 1 GiB buffer (caches hold none of
    # the input and nothing dirty), and back-to-back calls on one set (input in cache)
    flush_buf = torch.empty(1 << 27, dtype=torch.int64, device=dev)
    flush_buf.fill_(1)
    cold = []
    for _ in range(min(K, 20)):
        flush_buf.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    cold.sort()
    del flush_buf
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1) / K
    del calls

    # copy ceiling (torch's device copy of 1 GiB) for context
    a = torch.empty(1 << 29, dtype=torch.int16, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        b.copy_(a)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * a.numel() * 2 * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del a, b

    value = in_bytes / (ms * 1e-3) / 1e9
    achieved = alg_bytes / (ms * 1e-3) / 1e9              # the whole call (every kernel)
    if kern is not None:
        # the dominant kernel: the one with the longest average launch
        dom = max(kern, key=kern.get)
        dom_bytes = alg_bytes if dom.endswith("_quant") else in_bytes
        dom_gbs = dom_bytes / (kern[dom] * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl, dom),
                    "kernel": dom, "kernel_avg_us": round(kern[dom], 2), "kernel_alg_bytes": dom_bytes,
                    "call_achieved": round(achieved, 1), "call_frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    line = {
        "metric": ("input GB/s and % of HBM peak, grouped NVFP4 RHT quant (row+col), 1 MI355X"
                   if wl == "grouped_nvfp4_rht" else f"input GB/s and % of HBM peak, {wl}, 1 MI355X"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": desc, "timing": f"steady state: back-to-back calls over {n_sets} input/output sets"},
        "roofline": roofline,
        "pct_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "kernel_avg_us": kern,
        "algorithmic_bytes": alg_bytes,
        "input_bytes": in_bytes,
        "step_ms_p10_p50_p90": [round(per[int(0.1 * (K - 1))], 5), round(per[K // 2], 5), round(per[int(0.9 * (K - 1))], 5)],
        "cold_single_call_ms_p50": round(cold[len(cold) // 2], 5),
        "warm_ms_per_step": round(warm_ms, 5),
        "hbm_copy_gbs_measured": round(copy_gbs, 1),
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline and wl.startswith("grouped"):
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_rows)
        # the same oracle functions over independent (section, row-block) ranges on the
        # host's cores (a secondary figure; cpu_baseline is the single-core one)
        line["cpu_baseline_all_cores"] = cpu_baseline(w, args.cpu_sample_rows, threads=host_threads())
    print(json.dumps(line), flush=True)


# HBM bytes per call from the committed counter summaries (rocprofv3 --pmc), used
# only while the kernel sources they were taken on are unchanged.
TRAFFIC_SUMMARIES = {"grouped_nvfp4_rht": "profiles/grouped_nvfp4_rht_16384x4096_hbm_traffic.md"}
KERNEL_SOURCES = ["nvfp4_quantization_amd/csrc/mxq_nvfp4.hip", "nvfp4_quantization_amd/csrc/mxq_nvfp4_impl.hpp",
                  "nvfp4_quantization_amd/csrc/mxq_nvfp4_quant_rne.hip",
                  "nvfp4_quantization_amd/csrc/mxq_device.hpp", "nvfp4_quantization_amd/csrc/mxq_internal.hpp"]


def kernel_source_digest() -> str:
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(here, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def hip_runtime():
    """The HIP runtime this process already runs on (torch's copy), opened without
    loading another, for the event flags torch does not expose."""
    import ctypes
    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
    if path is None:
        raise RuntimeError("the HIP runtime is not loaded")
    hip = ctypes.CDLL(path, mode=os.RTLD_NOLOAD | ctypes.RTLD_GLOBAL)
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000    # hip_runtime_api.h: no cache write-back at the event


def kernel_times(mxq, torch, calls, n_sets, K, stream, names):
    """Average duration (us) of each of the two kernels (`names`) of a call over K
    steady-state calls, between HIP events the library records on the call's stream
    just before, between and after them.  The events skip the system-scope fence
    (hipEventDisableSystemFence): with it, each event writes back and invalidates
    the caches and adds 3-4 us to the interval it closes."""
    import ctypes
    hip = hip_runtime()
    ev = []
    try:
        for _ in range(3 * K):
            h = ctypes.c_void_p()
            if hip.hipEventCreateWithFlags(ctypes.byref(h), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            ev.append(h)
        torch.cuda.synchronize()
        try:
            for i in range(K):
                mxq.mxq_set_launch_marks(*(e.value for e in ev[3 * i:3 * i + 3]))
                calls[i % n_sets]()
        finally:
            mxq.mxq_set_launch_marks()
        torch.cuda.synchronize()
        t = ctypes.c_float()

        def elapsed(a, b):
            if hip.hipEventElapsedTime(ctypes.byref(t), a, b) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            return t.value
        first = sum(elapsed(ev[3 * i], ev[3 * i + 1]) for i in range(K)) / K
        second = sum(elapsed(ev[3 * i + 1], ev[3 * i + 2]) for i in range(K)) / K
    finally:
        for e in ev:
            hip.hipEventDestroy(e)
    return {names[0]: round(first * 1e3, 2), names[1]: round(second * 1e3, 2)}


def measured_traffic(wl, kernel):
    """Bytes per launch of `kernel` read + written at HBM, or None when no summary
    matches the current kernel sources."""
    name = TRAFFIC_SUMMARIES.get(wl)
    if name is None:
        return None
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            key, val = line[2:].split(":", 1)
            fields[key.strip()] = val.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_digest():
        return None
    try:
        return int(fields[f"hbm_bytes_per_launch {kernel}"])
    except (KeyError, ValueError):
        return None


def host_threads() -> int:
    """Host cores this process may use, at most 16 (a one-GPU share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(w, sample_rows, threads=1):
    """The oracle as it stands (plain C; one host core, or `threads` workers over
    independent section and row-block ranges of the same functions) on the same
    input: the whole workload's sections (or the sections that fit in the first
    `sample_rows` rows), all requested outputs, timed on this host."""
    import numpy as np
    import torch
    import oracle
    p = w.params
    total = w.tensors["x"].shape[0]
    cap = sample_rows if sample_rows > 0 else min(total, 16384)
    sections, rows = [], 0
    for m in p["split_sections"]:
        if rows + m > cap:
            break
        sections.append(m)
        rows += m
    if rows == 0:                      # first section alone is larger than the cap: take part of it
        sections, rows = [cap // 128 * 128], cap // 128 * 128
    S = len(sections)
    x = w.tensors["x"][:rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    oracle.lib()
    reps, t0 = 0, time.perf_counter()
    while True:                        # repeat to about 10 s of CPU time
        oracle.group_rht_quant_nvfp4(x, sections, p["sign_mask"], p["flags"], p["seed"] or 0,
                                     p["row_offsets"][:S] if p["row_offsets"] else None,
                                     p["col_offsets"][:S] if p["col_offsets"] else None, threads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps >= 10:
            break
    what = "the whole workload" if rows == total else f"its first {S} sections ({rows} of {total} rows)"
    where = "on one core" if threads == 1 else f"on {threads} threads"
    return {"value": round(reps * x.nbytes / dt / 1e9, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}, all requested outputs, {reps} run(s) in {dt:.1f} s {where}"}


if __name__ == "__main__":
    main()
