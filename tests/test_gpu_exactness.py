"""Exactness on the device, beyond the parity cases:

- the hardware conversions in the forms the kernels use, over their whole input
  range (test-only kernels in tests/hip/mxq_selftest.hip compare them on the device
  with integer reference encoders written from the formats' definitions): BF16,
  E4M3 and E2M1 nearest-even over all 2^32 FP32 inputs, and the stochastic E2M1
  conversion (random operand r << 24) over every non-NaN input and every r;
- SiLU's division by the hardware reciprocal and a correction step, against IEEE
  division for every BF16 numerator significand and every divisor in [1, 2^24);
- the NVFP4 scale tables a call leaves in its workspace: every divisor is
  fl(E4M3(c) * g) (times 4 column-wise), every reciprocal fl(1/d), and every
  product multiplier gives the exact division's E2M1 code for every BF16 input
  (brute force), for sections whose maxima carry the factors 3 and 7 of 2688, span
  2^-30 .. 2^40 and sit on the 1e-10 floor; with stochastic rounding every
  stochastic multiplier gives the exact quotient's grid spacing and floor(256 f),
  the part of the quotient the rounding rule reads.

onnxruntime PR #33644 (Description) is why: one-ulp differences at encoding
midpoints change codes, so every decision must be the exact one."""
import ctypes
import os

import numpy as np
import pytest
import torch

import nvfp4_quantization_amd as mxq
import oracle
from tests.gpu_util import announce, device, host

pytestmark = pytest.mark.gpu
U64 = (1 << 64) - 1


def selftest():
    path = os.path.join(os.path.dirname(mxq.LIB_PATH), "libmxq_selftest.so")
    if not os.path.exists(path):
        pytest.fail(f"{path} is missing: build the library")
    L = ctypes.CDLL(path)
    for fn in (L.mxq_selftest_conversions, L.mxq_selftest_sr, L.mxq_selftest_div_rcp):
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    return L


def sweep(fn):
    dev = device()
    out = torch.zeros(16, dtype=torch.int64, device=dev)
    out[8:] = -1                                    # all ones: no mismatch seen
    assert fn(ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    return [int(v) & U64 for v in host(out)]


def test_conversions_all_fp32_inputs():
    announce("conversion sweep: BF16 / E4M3 / E2M1 over all 2^32 FP32 inputs")
    o = sweep(selftest().mxq_selftest_conversions)
    names = ["E4M3 (finite, |v| < 464)", "E4M3 NaN -> NaN code", "BF16 (non-NaN)", "BF16 NaN -> NaN",
             "E2M1 (non-NaN)"]
    report = {n: (o[i], hex(o[8 + i]) if o[8 + i] != U64 else None) for i, n in enumerate(names)}
    assert o[5] == 1 << 32, f"inputs swept: {o[5]}"
    assert all(o[i] == 0 for i in range(5)), f"mismatches (count, first input): {report}"


def test_stochastic_e2m1_every_input_and_r():
    announce("stochastic E2M1 sweep: every non-NaN FP32 input x 256 random bytes")
    o = sweep(selftest().mxq_selftest_sr)
    assert o[2] == (0x7F800001 * 2) * 256, f"conversions checked: {o[2]}"
    first = [None if o[8 + i] == U64 else (hex(o[8 + i] >> 8), o[8 + i] & 255) for i in range(2)]
    assert o[0] == 0, f"|q| in [2^-20, 16): {o[0]} mismatches, first (q bits, r) {first[0]}"
    assert o[1] == 0, f"other q: {o[1]} mismatches, first (q bits, r) {first[1]}"


def test_reciprocal_division_every_bf16_numerator():
    """SwiGLU's SiLU divides a BF16 gate value g by t = 1 + EXP(-g) with div_rn's
    correction step on the hardware reciprocal of t (where 2^-56 <= |g| <= 2^126 and
    t < 2^24): against IEEE division for every BF16 numerator significand, both signs,
    and every FP32 divisor in [1, 2^24)."""
    announce("reciprocal division sweep: 256 numerators x 24 binades x 2^23 divisors")
    o = sweep(selftest().mxq_selftest_div_rcp)
    assert o[2] == (24 << 23) * 256, f"pairs checked: {o[2]}"
    first = None if o[8] == U64 else (hex(o[8] >> 8), o[8] & 255)
    assert o[0] == 0, f"{o[0]} mismatches, first (t bits, numerator k) {first}"


def test_scale_tables_exact_for_every_bf16_input():
    dev = device()
    announce("scale tables: divisors, reciprocals and multipliers of a call's workspace")
    # 8 sections of 128 x 256 whose maxima differ in kind: plain, factors 3 and 7,
    # tiny (floored), huge, an all-zero section
    factors = [1.0, 3.0, 3.0 * 2.0 ** -30, 2.0 ** 40, 7.0 * 2.0 ** -10, 21.0, 1e-13, 0.0]
    rng = np.random.default_rng(71)
    base = rng.standard_normal((8 * 128, 256)).astype(np.float32)
    for s, f in enumerate(factors):
        block = base[s * 128:(s + 1) * 128]
        block *= np.float32(f) / np.float32(np.abs(block).max())     # max |x| = f before the BF16 round
    x = torch.from_numpy(base).to(torch.bfloat16).to(dev)
    call = mxq.GroupedNVFP4(x, [128] * 8, 0x2D3C, 3)
    res = call()
    torch.cuda.synchronize()
    tables = host(call.workspace)[mxq.WORKSPACE_TABLES:mxq.WORKSPACE_TABLES + 8 * 2 * 128 * 16].view(np.float32)
    tables = tables.reshape(8, 2, 128, 4)
    g_all = (host(res.row_global), host(res.col_global))
    u = (np.arange(0x7F80, dtype=np.uint32) << 16).view(np.float32)   # every non-negative finite BF16
    e4m3 = np.array([oracle.e4m3_value(c) for c in range(127)], np.float32)
    checked = without = 0
    for s in range(8):
        for d_ in range(2):
            g = np.float32(g_all[d_][s])
            T = tables[s, d_]
            assert T[0, 0] == g, (s, d_)
            flagged = T[127, 0] == 1.0
            for c in range(1, 127):
                d = np.float32(e4m3[c] * g)
                if d_ == 1:
                    d = np.float32(d * np.float32(4.0))
                assert T[c, 0] == d and T[c, 1] == np.float32(np.float32(1.0) / d), (s, d_, c)
                ym = T[c, 2]
                if ym < 0:
                    without += 1
                    assert flagged, f"section {s} direction {d_}: code {c} has no multiplier, entry 127 unflagged"
                    continue
                with np.errstate(over="ignore"):                  # inf quotients saturate to 6 either way
                    want = oracle.e2m1_encode(u / d)
                    got = oracle.e2m1_encode(u * ym)
                bad = np.nonzero(got != want)[0]
                assert bad.size == 0, f"section {s} dir {d_} code {c}: u={u[bad[0]]!r} ym={ym!r} d={d!r}"
                checked += 1
    assert checked > 1500 and without > 0, (checked, without)


def sr_cell(q: np.ndarray) -> np.ndarray:
    """What the stochastic E2M1 rule reads of a quotient q: for grid spacing D (0.5 /
    1 / 2 below 2 / 4 / 6) and |q| / D = k + f, the pair (D, 256 k + floor(256 f)),
    encoded as one integer; -1 for |q| >= 6 (saturation)."""
    a = np.abs(q.astype(np.float64))
    di = np.where(a < 2.0, 0, np.where(a < 4.0, 1, 2))
    D = np.array([0.5, 1.0, 2.0])[di]
    cell = np.floor(np.minimum(a, 6.0) / D * 256.0).astype(np.int64)   # (inf saturates below)
    return np.where(a < 6.0, cell + 4096 * di, -1)


def test_stochastic_scale_tables_exact_for_every_bf16_input():
    """With stochastic rounding the tables hold stochastic multipliers: fl(u * ym)
    must give the rule the same grid spacing and floor(256 f) as the exact quotient
    fl(u / d) for every BF16 u (then every random byte gives the same code).  A table
    with a scale code that has none is flagged, and its pass divides."""
    dev = device()
    announce("stochastic scale tables: multipliers of a call's workspace")
    factors = [1.0, 3.0, 3.0 * 2.0 ** -30, 2.0 ** 40, 7.0 * 2.0 ** -10, 21.0, 1e-13, 0.0, 0.37, 5.5e3, 1.9e-6, 42.0]
    S = len(factors)
    rng = np.random.default_rng(72)
    base = rng.standard_normal((S * 128, 256)).astype(np.float32)
    for s, f in enumerate(factors):
        block = base[s * 128:(s + 1) * 128]
        block *= np.float32(f) / np.float32(np.abs(block).max())
    x = torch.from_numpy(base).to(torch.bfloat16).to(dev)
    call = mxq.GroupedNVFP4(x, [128] * S, 0x2D3C, 3, 0x5EED, list(range(S)), list(range(100, 100 + S)))
    res = call()
    torch.cuda.synchronize()
    tables = host(call.workspace)[mxq.WORKSPACE_TABLES:mxq.WORKSPACE_TABLES + S * 2 * 128 * 16].view(np.float32)
    tables = tables.reshape(S, 2, 128, 4)
    g_all = (host(res.row_global), host(res.col_global))
    u = (np.arange(0x7F80, dtype=np.uint32) << 16).view(np.float32)
    e4m3 = np.array([oracle.e4m3_value(c) for c in range(127)], np.float32)
    checked = without = complete = 0
    for s in range(S):
        for d_ in range(2):
            g = np.float32(g_all[d_][s])
            T = tables[s, d_]
            flagged = T[127, 0] == 1.0
            has_none = False
            for c in range(1, 127):
                d = np.float32(e4m3[c] * g)
                if d_ == 1:
                    d = np.float32(d * np.float32(4.0))
                assert T[c, 0] == d and T[c, 1] == np.float32(np.float32(1.0) / d), (s, d_, c)
                ym = T[c, 2]
                if ym < 0:
                    without += 1
                    has_none = True
                    continue
                with np.errstate(over="ignore"):
                    want = sr_cell(u / d)
                    got = sr_cell(u * ym)
                bad = np.nonzero(got != want)[0]
                assert bad.size == 0, f"section {s} dir {d_} code {c}: u={u[bad[0]]!r} ym={ym!r} d={d!r}"
                checked += 1
            assert flagged == has_none, (s, d_, flagged, has_none)
            complete += not has_none
    assert checked > 1500 and complete > 0, (checked, without, complete)
