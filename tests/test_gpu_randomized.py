"""Randomized GPU parity: many small seeded configurations of every entry point,
each compared byte for byte with the oracle.  Shapes, section splits (empty ones
included), sign masks, output flags, rounding modes, supplied maxima and value
mixes are drawn from one seeded generator per case; the values mix normals over a
wide exponent range with NaN, +-inf, +-0, subnormals and exact E2M1 tie values.
Every case prints its parameters first, so a failure names it."""
import numpy as np
import pytest
import torch

import nvfp4_quantization_amd as mxq
from tests.gpu_util import announce, assert_same, device, host
from tests.test_gpu_parity import bf16_dev, compare_dsa4, compare_grouped, compare_grouped_amax

pytestmark = pytest.mark.gpu

SPECIALS = np.array([0x7FC0, 0xFFC1, 0x7F81, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x807F, 0x7F7F,
                     0x3F40, 0x3FA0, 0x3FE0, 0x4060, 0x40A0], np.uint16)


def mixed_matrix(rng, m, k, p_special):
    """BF16 bit patterns: scaled normals, with a fraction p_special of the entries
    replaced by special values (NaN, inf, zeros, subnormals, BF16 max, ties)."""
    x = rng.standard_normal((m, k)).astype(np.float32) * np.exp2(rng.integers(-20, 20, (m, 1))).astype(np.float32)
    b = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    if p_special > 0 and b.size:
        hit = rng.random(b.shape) < p_special
        b[hit] = rng.choice(SPECIALS, hit.sum())
    return b


def sections_for(rng, units, n):
    cuts = np.sort(rng.integers(0, units + 1, n - 1))
    return [int(v) * 128 for v in np.diff(np.concatenate([[0], cuts, [units]]))]


@pytest.mark.parametrize("case", range(64))
def test_grouped_random(orc, case):
    dev = device()
    rng = np.random.default_rng(9000 + case)
    k = int(rng.choice([128, 256, 384, 512, 640, 1024]))
    units = int(rng.integers(1, 9))
    n_sec = int(rng.integers(1, 6))
    sections = sections_for(rng, units, n_sec)
    mask = int(rng.integers(0, 1 << 16))
    flags = int(rng.choice([1, 2, 3, 5, 6, 7]))
    p_special = float(rng.choice([0.0, 0.0, 1e-3, 2e-2]))
    sr = bool(rng.random() < 0.3)
    supplied = bool(rng.random() < 0.3)
    announce(f"grouped random case={case} k={k} sections={sections} mask={mask:#06x} flags={flags} "
             f"p_special={p_special} sr={sr} supplied={supplied}")
    b = mixed_matrix(rng, sum(sections), k, p_special)
    x = bf16_dev(b, dev)
    seed = int(rng.integers(1, 1 << 40)) if sr else None
    ro = [int(v) for v in rng.integers(0, 1 << 30, n_sec)] if sr else None
    co = [int(v) for v in rng.integers(0, 1 << 30, n_sec)] if sr else None
    if supplied:
        # a supplied maximum for each requested NVFP4 direction
        amax_in = (rng.uniform(0.01, 50, n_sec).astype(np.float32) if flags & 1 else None,
                   rng.uniform(0.01, 50, n_sec).astype(np.float32) if flags & 2 else None)
        compare_grouped_amax(orc, x, sections, mask, flags, amax_in, seed=seed, ro=ro, co=co)
    else:
        compare_grouped(orc, x, sections, mask, flags, seed=seed, ro=ro, co=co)


@pytest.mark.parametrize("case", range(24))
def test_dsa_random_mixed(orc, case):
    dev = device()
    rng = np.random.default_rng(9500 + case)
    m = int(rng.integers(1, 700))
    d_pe = int(rng.choice([0, 8, 64, 120, 128]))
    p_special = float(rng.choice([0.0, 1e-3, 1e-2]))
    options = int(rng.integers(0, 2))
    amax_in = None if rng.random() < 0.6 else float(rng.uniform(0.05, 30))
    announce(f"dsa random case={case} m={m} d_pe={d_pe} p_special={p_special} options={options} amax_in={amax_in}")
    v = mixed_matrix(rng, m, 128, p_special)
    pe_np, nope_np = v[:, :d_pe].copy(), v[:, d_pe:].copy()
    pe = bf16_dev(pe_np, dev) if d_pe > 0 else None
    nope = bf16_dev(nope_np, dev) if d_pe < 128 else None
    q, s = mxq.mxq_hadamard_quant_fp8_ex(pe, nope, options, 1)
    torch.cuda.synchronize()
    rq, rs = orc.hadamard_quant_fp8_ex(pe_np, nope_np, options, 1)
    assert_same("dsa fp8 codes", host(q), rq)
    assert_same("dsa fp8 scales", host(s), rs)
    compare_dsa4(orc, pe_np, nope_np, pe, nope, amax_in=amax_in, amax_out=True)


@pytest.mark.parametrize("case", range(24))
def test_fp8_random_mixed(orc, case):
    dev = device()
    rng = np.random.default_rng(9700 + case)
    m = int(rng.integers(1, 400))
    k = 128 * int(rng.integers(1, 9))
    p_special = float(rng.choice([0.0, 1e-3, 1e-2]))
    options = int(rng.integers(0, 2))
    announce(f"fp8 random case={case} m={m} k={k} p_special={p_special} options={options}")
    b = mixed_matrix(rng, m, k, p_special)
    x = bf16_dev(b, dev)
    q, s = mxq.mxq_quant_fp8_1x128(x)
    torch.cuda.synchronize()
    rq, rs = orc.quant_fp8_1x128(b)
    assert_same("1x128 codes", host(q), rq)
    assert_same("1x128 scales", host(s), rs)
    rq_, rs_, cq_, cs_ = mxq.mxq_quant_fp8_blockwise(x, options, rowwise=True, columnwise=True)
    torch.cuda.synchronize()
    wq, ws, wcq, wcs = orc.quant_fp8_blockwise(b, options)
    assert_same("blockwise row codes", host(rq_), wq)
    assert_same("blockwise row scales", host(rs_), ws)
    assert_same("blockwise col codes", host(cq_.contiguous()), wcq)
    assert_same("blockwise col scales", host(cs_), wcs)
    g = mixed_matrix(rng, m, k, p_special / 4)
    u = mixed_matrix(rng, m, k, p_special / 4)
    q2, s2 = mxq.mxq_swiglu_quant_fp8(bf16_dev(g, dev), bf16_dev(u, dev))
    torch.cuda.synchronize()
    wq2, ws2 = orc.swiglu_quant_fp8(g, u)
    assert_same("swiglu scales", host(s2), ws2)
    assert_same("swiglu codes", host(q2), wq2)
