#!/usr/bin/env python3
"""Benchmark of the mxq hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload grouped_nvfp4_rht|...] [--no-cpu-baseline]

A step is one call of the quantizer over one batch of seeded synthetic input that
is already resident in HBM.  The default workload is grouped NVFP4 with the
16-point RHT, row-wise + column-wise, 16384 x 4096 BF16 in 8 MoE sections (the
configuration the headline metric is quoted on).  Before every timed step a
512 MiB buffer is overwritten so the step starts with the 256 MB Infinity Cache
and the L2s holding none of the input; each step is timed with HIP events on the
stream the kernels run on, and ms_per_step is their mean (a back-to-back "warm"
figure is reported beside it).  Prints ONE JSON line.
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
                             "dsa_rotate_fp8", "fp8_1x128"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=0,
                    help="rows of the workload the oracle baseline runs on (0: the whole workload, "
                         "capped at 16384 rows)")
    ap.add_argument("--no-flush", action="store_true", help="time back-to-back calls only")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(how the path would shard is described in DESIGN.md). Run with --gpus 1.", file=sys.stderr)
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
    if wl == "fp8_1x128":
        w = synth.plain_fp8(device=dev)
        x = w.tensors["x"]
        m, k = x.shape
        q = torch.empty((m, k), dtype=torch.uint8, device=dev)
        s = torch.empty((m, k // 128), dtype=torch.float32, device=dev)
        call = lambda: mxq.mxq_quant_fp8_1x128(x, q=q, scales=s)
        in_bytes = m * k * 2
        alg_bytes = in_bytes + m * k + m * k // 128 * 4
        desc = f"fp8_1x128 {m}x{k} bf16"
    elif wl == "dsa_rotate_fp8":
        w = synth.dsa_rotate_fp8(device=dev)
        pe, nope = w.tensors["pe"], w.tensors["nope"]
        m = pe.shape[0]
        q = torch.empty((m, 128), dtype=torch.uint8, device=dev)
        s = torch.empty((m,), dtype=torch.float32, device=dev)
        call = lambda: mxq.mxq_hadamard_quant_fp8(pe, nope, q=q, scales=s)
        in_bytes = m * 128 * 2
        alg_bytes = in_bytes + m * 128 + m * 4
        desc = f"dsa cat+WHT128+fp8_1x128, {m} rows (4096 tokens x 64 heads) bf16"
    else:
        gen = {"grouped_nvfp4_rht": synth.grouped_nvfp4, "grouped_nvfp4_rht_sr": synth.grouped_nvfp4_sr,
               "large_moe_nvfp4_fp8": synth.large_moe}[wl]
        w = gen(device=dev)
        p = w.params
        x = w.tensors["x"]
        total, k = x.shape
        S = len(p["split_sections"])
        prepared = mxq.GroupedNVFP4(x, p["split_sections"], p["sign_mask"], p["flags"], p["seed"],
                                    p["row_offsets"], p["col_offsets"])
        call = prepared
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

    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def flush():
        flush_buf.fill_(1)

    # ---------------------------------------------------------------- warmup
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed steps
    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        if not args.no_flush:
            flush()
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))
    ms = sum(per) / K

    # back-to-back (caches warm with the previous call's data)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1) / K

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
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    line = {
        "metric": "input GB/s and % of HBM peak, grouped NVFP4 RHT quant (row+col), 1 MI355X",
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
        "config": {"workload": desc, "timing": "cold Infinity Cache per step" if not args.no_flush else "back-to-back"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
        "pct_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "algorithmic_bytes": alg_bytes,
        "input_bytes": in_bytes,
        "ms_p10_p50_p90": [round(per[int(0.1 * (K - 1))], 5), round(per[K // 2], 5), round(per[int(0.9 * (K - 1))], 5)],
        "warm_ms_per_step": round(warm_ms, 5),
        "hbm_copy_gbs_measured": round(copy_gbs, 1),
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline and wl.startswith("grouped"):
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_rows)
    print(json.dumps(line), flush=True)


def cpu_baseline(w, sample_rows):
    """The oracle as it stands (plain single-threaded C, one host core) on the same
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
    t0 = time.perf_counter()
    oracle.group_rht_quant_nvfp4(x, sections, p["sign_mask"], p["flags"], p["seed"] or 0,
                                 p["row_offsets"][:S] if p["row_offsets"] else None,
                                 p["col_offsets"][:S] if p["col_offsets"] else None)
    dt = time.perf_counter() - t0
    what = "the whole workload" if rows == total else f"its first {S} sections ({rows} of {total} rows)"
    return {"value": round(x.nbytes / dt / 1e9, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{what}, all requested outputs, {dt:.1f} s on one core"}


if __name__ == "__main__":
    main()
