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
the HIP-event time of the whole run on the calls' stream divided by the steps
(two events around the K calls, nothing enqueued between them).

`roofline` is the whole call's: its algorithmic bytes (input read once, every output
written once) over the call time, against the 8 TB/s HBM peak.  A call of the
three-kernel form runs an amax pass, a per-section scales pass and a quant pass that
reads the input again; only the call
as a whole moves the method's bytes, so no single kernel's rate stands for it (the
per-kernel split is in the committed rocprofv3 summaries).  Beside it: the rate of a
hand-written streaming read and copy over the same rotating buffer sizes
(libmxq_ceiling.so; the measured ceilings: a read of the input's bytes, and the
input read plus the outputs written) and torch's 1 GiB copy.
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
                    choices=["grouped_nvfp4_rht", "grouped_nvfp4_rht_given", "grouped_nvfp4_rht_sr",
                             "large_moe_nvfp4_fp8", "dsa_rotate_fp8", "dsa_rotate_nvfp4", "swiglu_fp8",
                             "fp8_blockwise", "fp8_1x128"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="steady-state steps only, then the hand-written 256 MiB copy and 128 MiB read (twice) "
                         "(the counter calibrations for rocprofv3 runs); prints a short JSON line")
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
        gen = {"grouped_nvfp4_rht": synth.grouped_nvfp4, "grouped_nvfp4_rht_given": synth.grouped_nvfp4,
               "grouped_nvfp4_rht_sr": synth.grouped_nvfp4_sr, "large_moe_nvfp4_fp8": synth.large_moe}[wl]
        w = gen(device=dev)
        p = w.params
        x = w.tensors["x"]
        total, k = x.shape
        S = len(p["split_sections"])
        workspace = mxq.alloc_workspace(total, k, S, p["flags"], dev)
        given = None
        if wl == "grouped_nvfp4_rht_given":
            # supplied section maxima (a single pass over x), here this input's own
            # measured maxima, so the outputs equal the measured call's; the call also
            # returns the maxima it measures, as a delayed-scaling caller needs
            first = mxq.GroupedNVFP4(x, p["split_sections"], p["sign_mask"], p["flags"], workspace=workspace,
                                     amax_out=True)()
            given = (first.row_amax.clone(), first.col_amax.clone())
            del first

        def make_call():
            return mxq.GroupedNVFP4(x.clone(), p["split_sections"], p["sign_mask"], p["flags"], p["seed"],
                                    p["row_offsets"], p["col_offsets"], workspace=workspace, amax_in=given,
                                    amax_out=given is not None)
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
                f"{'stochastic rounding' if p['seed'] is not None else 'RNE'}"
                f"{', supplied section maxima, measured maxima out' if given is not None else ''}")
        if given is not None:
            alg_bytes += 2 * S * 4 + 2 * S * 4       # the maxima in and out

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

    # the same calls replayed from a HIP graph (one graph holds one call per set), so
    # that the host's launch cost per call drops out: a secondary figure, for the
    # calls whose kernels take less time than their launches
    graph_ms, graph_error = None, None
    if not args.profile:
        try:
            graph = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.graph(graph, stream=side):
                for c in calls:
                    c()
            torch.cuda.synchronize()
            reps = max(1, -(-K // n_sets))
            graph.replay()
            torch.cuda.synchronize()
            g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g0.record(stream)
            for _ in range(reps):
                graph.replay()
            g1.record(stream)
            torch.cuda.synchronize()
            graph_ms = g0.elapsed_time(g1) / (reps * n_sets)
            del graph
        except RuntimeError as e:                     # reported in the line, not fatal to it
            graph_error = str(e)[:200]

    if args.profile:
        del calls
        ceil = ceiling_lib()
        a = torch.ones(1 << 27, dtype=torch.int16, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        # the counters' calibration: a hand-written copy of 256 MiB (256 MiB read, 256
        # MiB written), then a 128 MiB streaming read, twice
        if ceil.mxq_ceiling_copy(a.data_ptr(), b.data_ptr(), 2 * a.numel(), stream.cuda_stream) != 0:
            raise RuntimeError("mxq_ceiling_copy failed")
        torch.cuda.synchronize()
        sink = torch.empty((ceil.mxq_ceiling_grid(),), dtype=torch.int32, device=dev)
        c = torch.ones(1 << 26, dtype=torch.int16, device=dev)   # 128 MiB, read twice
        for _ in range(2):
            if ceil.mxq_ceiling_read(c.data_ptr(), 2 * c.numel(), sink.data_ptr(), stream.cuda_stream) != 0:
                raise RuntimeError("mxq_ceiling_read failed")
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": True, "workload": desc, "steps": K, "ms_per_step": round(ms, 5),
                          "copy_calibration_bytes": 2 * a.numel(), "read_calibration_bytes": 2 * c.numel()}),
              flush=True)
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
    # hand-written streaming read and copy over the workload's own sizes, cycling over
    # as many buffers as the workload's sets (so they come from HBM, as its inputs do)
    read_gbs, move_gbs = ceilings(torch, dev, stream, in_bytes, alg_bytes - in_bytes, n_sets, K)

    value = in_bytes / (ms * 1e-3) / 1e9
    achieved = alg_bytes / (ms * 1e-3) / 1e9              # the whole call (every kernel)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl),
                "unit_of_work": "one whole call (every kernel it launches)", "call_us": round(ms * 1e3, 2)}
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
        "algorithmic_bytes": alg_bytes,
        "input_bytes": in_bytes,
        "step_ms_p10_p50_p90": [round(per[int(0.1 * (K - 1))], 5), round(per[K // 2], 5), round(per[int(0.9 * (K - 1))], 5)],
        "cold_single_call_ms_p50": round(cold[len(cold) // 2], 5),
        "warm_ms_per_step": round(warm_ms, 5),
        "graph_ms_per_step": round(graph_ms, 5) if graph_ms is not None else graph_error,
        "hbm_copy_gbs_measured": round(copy_gbs, 1),
        "read_ceiling_gbs": round(read_gbs, 1),
        "move_ceiling_gbs": round(move_gbs, 1),
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
# Counter summaries under profiles/ holding a line "- hbm_bytes_per_call[<workload>]: N"
# (bytes read + written at the memory side per call, every kernel of the call) and the
# digest of the kernel sources they were measured with.
TRAFFIC_SUMMARIES = {"grouped_nvfp4_rht": "profiles/grouped_nvfp4_rht_16384x4096_hbm_traffic.md"}
for _wl in ("grouped_nvfp4_rht_sr", "grouped_nvfp4_rht_given", "large_moe_nvfp4_fp8", "dsa_rotate_nvfp4",
            "dsa_rotate_fp8", "swiglu_fp8", "fp8_blockwise", "fp8_1x128"):
    TRAFFIC_SUMMARIES[_wl] = "profiles/other_workloads_hbm_traffic.md"
KERNEL_SOURCE_DIR = "nvfp4_quantization_amd/csrc"


def kernel_source_digest() -> str:
    """SHA-256 over every kernel and host source of the library, in name order (a
    change to any of them makes the stored counter figures stale)."""
    import hashlib
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), KERNEL_SOURCE_DIR)
    h = hashlib.sha256()
    for f in sorted(os.listdir(here)):
        if f.endswith((".hip", ".hpp", ".cpp")):
            h.update(f.encode())
            with open(os.path.join(here, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def measured_traffic(wl):
    """Bytes per call read + written at the memory side (every kernel of the call), or
    None when no summary matches the current kernel sources."""
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
        return int(fields[f"hbm_bytes_per_call[{wl}]"])
    except (KeyError, ValueError):
        return None


_ceiling = None


def ceiling_lib():
    """libmxq_ceiling.so: the streaming read and copy kernels of the measured ceiling."""
    global _ceiling
    if _ceiling is None:
        import ctypes
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "nvfp4_quantization_amd", "_build",
                            "libmxq_ceiling.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build the library")
        L = ctypes.CDLL(path)
        p, i64 = ctypes.c_void_p, ctypes.c_int64
        L.mxq_ceiling_grid.restype = ctypes.c_int
        L.mxq_ceiling_read.restype = ctypes.c_int
        L.mxq_ceiling_read.argtypes = [p, i64, p, p]
        L.mxq_ceiling_copy.restype = ctypes.c_int
        L.mxq_ceiling_copy.argtypes = [p, p, i64, p]
        _ceiling = L
    return _ceiling


def ceilings(torch, dev, stream, in_bytes, out_bytes, n_sets, K):
    """The measured ceilings beside a workload: GB/s of a streaming read of in_bytes,
    and of the workload's own data movement done by the plainest kernels, in_bytes read
    and out_bytes written (a copy of the smaller and a read of the rest of the input),
    counted as in + out.  Each cycles over n_sets buffers of that size with K launches
    back to back, the workload's timing method."""
    L = ceiling_lib()
    nbytes = (in_bytes + 15) // 16 * 16
    obytes = max((out_bytes + 15) // 16 * 16, 16)
    srcs = [torch.ones((nbytes // 2,), dtype=torch.int16, device=dev) for _ in range(n_sets)]
    dsts = [torch.empty((obytes,), dtype=torch.uint8, device=dev) for _ in range(n_sets)]
    sink = torch.empty((L.mxq_ceiling_grid(),), dtype=torch.int32, device=dev)
    st = stream.cuda_stream

    def run(fn):
        for i in range(3):
            fn(i % n_sets)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(K):
            fn(i % n_sets)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K * 1e-3

    def rd(i):
        if L.mxq_ceiling_read(srcs[i].data_ptr(), nbytes, sink.data_ptr(), st) != 0:
            raise RuntimeError("mxq_ceiling_read failed")

    def cp(i):
        # read the input's bytes and write the outputs' bytes: the copy covers the
        # smaller of the two, and a read of the rest completes the input
        n = min(nbytes, obytes)
        if L.mxq_ceiling_copy(srcs[i].data_ptr(), dsts[i].data_ptr(), n, st) != 0:
            raise RuntimeError("mxq_ceiling_copy failed")
        if nbytes > n and L.mxq_ceiling_read(srcs[i].data_ptr() + n, nbytes - n, sink.data_ptr(), st) != 0:
            raise RuntimeError("mxq_ceiling_read failed")

    t_read = run(rd)
    t_copy = run(cp)
    return nbytes / t_read / 1e9, (nbytes + min(nbytes, obytes)) / t_copy / 1e9   # (read, move)


def host_threads() -> int:
    """Host cores this process may use, at most 16 (a one-GPU share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, sample_rows, threads=1):
    """The oracle as it stands (plain C; one host core, or `threads` workers over
    independent section and row-block ranges of the same functions) on the same
    input: the whole workload's sections (or the sections that fit in the first
    `sample_rows` rows), all requested outputs, timed on this host: the median of
    three runs."""
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
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.group_rht_quant_nvfp4(x, sections, p["sign_mask"], p["flags"], p["seed"] or 0,
                                     p["row_offsets"][:S] if p["row_offsets"] else None,
                                     p["col_offsets"][:S] if p["col_offsets"] else None, threads=threads)
        runs.append(time.perf_counter() - t0)
    dt = sorted(runs)[1]
    what = "the whole workload" if rows == total else f"its first {S} sections ({rows} of {total} rows)"
    where = "on one core" if threads == 1 else f"on {threads} threads"
    return {"value": round(x.nbytes / dt / 1e9, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}, all requested outputs, median of 3 runs ({', '.join(f'{r:.2f}' for r in runs)} s) "
                      f"{where}", "cpu_model": cpu_model()}


if __name__ == "__main__":
    main()
