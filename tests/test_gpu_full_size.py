"""Parity at the five workloads' full sizes, through the same prepared calls the
benchmark times: every output byte is compared with the oracle, which runs its
plain per-section / per-row-range functions on worker threads."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import nvfp4_quantization_amd as mxq
from nvfp4_quantization_amd import synth
from tests.gpu_util import announce, assert_same, bits16, device, host

pytestmark = [pytest.mark.gpu, pytest.mark.large]
THREADS = min(16, os.cpu_count() or 1)


def test_full_plain_fp8(orc):
    dev = device()
    announce("full size: plain FP8 1x128 256x1024")
    w = synth.plain_fp8(device=dev)
    q, s = mxq.mxq_quant_fp8_1x128(w.tensors["x"])
    torch.cuda.synchronize()
    rq, rs = orc.quant_fp8_1x128(bits16(w.tensors["x"]))
    assert_same("codes", host(q), rq)
    assert_same("scales", host(s), rs)


def test_full_dsa(orc):
    dev = device()
    announce("full size: DSA rotate+FP8 4096 tokens x 64 heads")
    w = synth.dsa_rotate_fp8(device=dev)
    q, s = mxq.mxq_hadamard_quant_fp8(w.tensors["pe"], w.tensors["nope"])
    torch.cuda.synchronize()
    pe, nope = bits16(w.tensors["pe"]), bits16(w.tensors["nope"])
    m = pe.shape[0]
    step = (m + THREADS - 1) // THREADS
    with ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(lambda r0: orc.hadamard_quant_fp8(pe[r0:r0 + step], nope[r0:r0 + step]),
                            range(0, m, step)))
    assert_same("codes", host(q), np.concatenate([p[0] for p in parts]))
    assert_same("scales", host(s), np.concatenate([p[1] for p in parts]))


def test_full_fp8_blockwise(orc):
    dev = device()
    announce("full size: FP8 row-wise 1x128 + column-wise 128x1, UE8M0, 16384x4096")
    x = synth.grouped_nvfp4(device=dev).tensors["x"]
    rq, rs, cq, cs = mxq.mxq_quant_fp8_blockwise(x, mxq.MXQ_FP8_UE8M0, rowwise=True, columnwise=True)
    torch.cuda.synchronize()
    wq, ws, wcq, wcs = orc.quant_fp8_blockwise(bits16(x), orc.FP8_UE8M0)
    assert_same("row_scales", host(rs), ws)
    assert_same("row_codes", host(rq), wq)
    assert_same("col_scales", host(cs), wcs)
    assert_same("col_codes", host(cq.contiguous()), wcq)


def test_full_swiglu_fp8(orc):
    dev = device()
    announce("full size: SwiGLU -> FP8 1x128, 16384 tokens x 4096 (fused gate|up buffer)")
    w = synth.swiglu_fp8(device=dev)
    gu = w.tensors["gate_up"]
    n = gu.shape[1] // 2
    q, s = mxq.mxq_swiglu_quant_fp8(gu[:, :n], gu[:, n:])
    torch.cuda.synchronize()
    gb, ub = bits16(gu[:, :n].contiguous()), bits16(gu[:, n:].contiguous())
    m = gb.shape[0]
    step = (m + THREADS - 1) // THREADS
    with ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(lambda r0: orc.swiglu_quant_fp8(gb[r0:r0 + step], ub[r0:r0 + step]), range(0, m, step)))
    assert_same("scales", host(s), np.concatenate([p[1] for p in parts]))
    assert_same("codes", host(q), np.concatenate([p[0] for p in parts]))


def test_full_dsa_nvfp4(orc):
    dev = device()
    announce("full size: DSA rotate+NVFP4 4096 tokens x 64 heads")
    w = synth.dsa_rotate_fp8(device=dev)
    call = mxq.HadamardNVFP4(w.tensors["pe"], w.tensors["nope"], amax_out=True)
    res = call()
    torch.cuda.synchronize()
    ref = orc.hadamard_quant_nvfp4(bits16(w.tensors["pe"]), bits16(w.tensors["nope"]))
    assert_same("global_scale", host(res.global_scale), np.array([ref.global_scale], np.float32))
    assert_same("amax", host(res.amax), np.array([ref.amax], np.float32))
    assert_same("scales", host(res.scales), ref.scales)
    assert_same("codes", host(res.codes), ref.codes)


def _grouped_full(orc, w, dev):
    p = w.params
    x = w.tensors["x"]
    call = mxq.GroupedNVFP4(x, p["split_sections"], p["sign_mask"], p["flags"], p["seed"],
                            p["row_offsets"], p["col_offsets"])
    res = call()
    torch.cuda.synchronize()
    assert mxq.workspace_protocol_clear(call.workspace)
    xb = bits16(x)
    ref = orc.group_rht_quant_nvfp4(xb, p["split_sections"], p["sign_mask"], p["flags"], p["seed"] or 0,
                                    p["row_offsets"], p["col_offsets"], threads=THREADS)
    for name in ("row_global", "col_global", "row_scales", "col_scales", "row_codes", "col_codes",
                 "fp8_scales", "fp8_codes"):
        got = getattr(res, name)
        if got is not None:
            assert_same(name, host(got), getattr(ref, name))


def test_full_grouped_nvfp4_rht(orc):
    dev = device()
    announce("full size: grouped NVFP4 RHT 16384x4096, 8 sections")
    _grouped_full(orc, synth.grouped_nvfp4(device=dev), dev)


def test_full_grouped_nvfp4_sr(orc):
    dev = device()
    announce("full size: grouped NVFP4 RHT + SR 16384x4096, 32 sections")
    _grouped_full(orc, synth.grouped_nvfp4_sr(device=dev), dev)


def test_full_large_moe(orc):
    dev = device()
    announce("full size: large MoE 65536x7168, 32 sections, NVFP4 row+col + FP8")
    _grouped_full(orc, synth.large_moe(device=dev), dev)
