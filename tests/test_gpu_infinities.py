"""GPU parity on infinite inputs and FP32 overflow: every output byte of each HIP path
equals the oracle's, which follows IEEE arithmetic as written.  A finite value over
an infinite scale is +-0, an infinite value over a finite scale is infinite (FP8:
over an infinite scale, NaN: 0x7F), and a block whose rotated values hold inf - inf
is a NaN block.  An infinite measured amax makes the tensor scale infinite; supplied
finite maxima keep the rest of such a section encoding normally."""
import numpy as np
import pytest
import torch

import nvfp4_quantization_amd as mxq
from nvfp4_quantization_amd import synth
from tests.gpu_util import announce, assert_same, bits16, device, host
from tests.test_gpu_parity import bf16_dev, compare_dsa4, compare_grouped, compare_grouped_amax

pytestmark = pytest.mark.gpu

INF, NINF = 0x7F80, 0xFF80


def bf16_matrix(m, k, seed, spread=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32) * np.exp2(rng.integers(-spread, spread + 1, (m, 1)))
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def plant(b, row0):
    """Infinities from row row0 on: single ones, a cancelling same-sign pair in one
    16-row column block, a +inf / -inf pair in one row, and a row of BF16 maxima whose
    column sums overflow FP32."""
    b[row0 + 2, 7] = INF
    b[row0 + 20, 33] = NINF
    b[row0 + 40, 9] = b[row0 + 41, 9] = INF
    b[row0 + 60, 3], b[row0 + 60, 4] = INF, NINF
    b[row0 + 80:row0 + 96, 12] = 0x7F7F              # 16 x 3.39e38: the column sums overflow
    return b


@pytest.mark.parametrize("k", [256, 512])          # one- and four-wave quant work-groups
def test_grouped_infinities(orc, k):
    dev = device()
    announce(f"grouped infinities k={k}")
    b = plant(bf16_matrix(384, k, 91), 128)            # section 0 (rows 0..127) stays finite
    x = bf16_dev(b, dev)
    for mask in (0x0000, 0xA5A5):
        compare_grouped(orc, x, [128, 256], mask, 3)
        compare_grouped(orc, x, [128, 256], mask, 7)
    compare_grouped(orc, x, [128, 256], 0x3C5A, 3, seed=17, ro=[3, 4], co=[5, 6])     # SR
    meas = orc.group_rht_quant_nvfp4(b, [128, 256], 0xA5A5, 3, threads=8)
    assert np.isinf(meas.row_amax[1]) and np.isfinite(meas.row_amax[0])
    amax_in = (np.float32([meas.row_amax[0], 9.0]), np.float32([meas.col_amax[0], 9.0]))
    compare_grouped_amax(orc, x, [128, 256], 0xA5A5, 3, amax_in)
    compare_grouped_amax(orc, x, [128, 256], 0xA5A5, 7, amax_in, seed=23, ro=[1, 2], co=[7, 8])
    compare_grouped_amax(orc, x, [128, 256], 0xA5A5, 3, None)
    # a supplied amax 2^-120 of the data's: every quotient overflows to inf
    tiny = (np.float32([1e-36, 1e-36]), np.float32([1e-36, 1e-36]))
    compare_grouped_amax(orc, x, [128, 256], 0xA5A5, 3, tiny)


def test_dsa_nvfp4_infinities(orc):
    dev = device()
    announce("dsa nvfp4 infinities")
    w = synth.dsa_rotate_fp8(tokens=40, heads=8, seed=92)
    pe_np, nope_np = bits16(w.tensors["pe"]).copy(), bits16(w.tensors["nope"]).copy()
    pe_np[5, 3] = INF                                  # one infinity: the row is all +-inf
    pe_np[9, 0], pe_np[9, 1] = INF, NINF               # half the row NaN, half infinite
    nope_np[17, 2] = nope_np[17, 3] = INF
    pe, nope = bf16_dev(pe_np, dev), bf16_dev(nope_np, dev)
    compare_dsa4(orc, pe_np, nope_np, pe, nope, amax_out=True)          # measured: A = inf
    compare_dsa4(orc, pe_np, nope_np, pe, nope, amax_in=5.0, amax_out=True)
    compare_dsa4(orc, pe_np, nope_np, pe, nope, amax_in=1e-36)


def test_fp8_paths_infinities(orc):
    dev = device()
    announce("fp8 paths infinities")
    b = plant(bf16_matrix(200, 256, 93), 0)
    x = bf16_dev(b, dev)
    q, s = mxq.mxq_quant_fp8_1x128(x)
    torch.cuda.synchronize()
    rq, rs = orc.quant_fp8_1x128(b)
    assert_same("1x128 scales", host(s), rs)
    assert_same("1x128 codes", host(q), rq)
    for options in (0, 1):
        rq_, rs_, cq_, cs_ = mxq.mxq_quant_fp8_blockwise(x, options, rowwise=True, columnwise=True)
        torch.cuda.synchronize()
        wq, ws, wcq, wcs = orc.quant_fp8_blockwise(b, options)
        assert_same("blockwise row_scales", host(rs_), ws)
        assert_same("blockwise row_codes", host(rq_), wq)
        assert_same("blockwise col_scales", host(cs_), wcs)
        assert_same("blockwise col_codes", host(cq_.contiguous()), wcq)
    d = plant(bf16_matrix(128, 128, 94), 0)
    for options in (0, 1):
        q, s = mxq.mxq_hadamard_quant_fp8_ex(bf16_dev(d[:, :64], dev), bf16_dev(d[:, 64:], dev), options, 8)
        torch.cuda.synchronize()
        rq, rs = orc.hadamard_quant_fp8_ex(d[:, :64], d[:, 64:], options, 8)
        assert_same("dsa fp8 codes", host(q), rq)
        assert_same("dsa fp8 scales", host(s), rs)


def test_swiglu_infinities(orc):
    dev = device()
    announce("swiglu infinities")
    m, n = 24, 384
    g = bf16_matrix(m, n, 95, spread=0)
    u = bf16_matrix(m, n, 96)
    g[0, 5], u[0, 5] = 0x4120, 0x7F00                  # SiLU(10) * 1.7e38 overflows
    u[3, 70] = INF                                     # inf up
    g[6, 9] = INF                                      # SiLU(inf) = inf / (1 + 0) = inf
    g[7, 10] = NINF                                    # SiLU(-inf) = -inf / inf: NaN
    q, s = mxq.mxq_swiglu_quant_fp8(bf16_dev(g, dev), bf16_dev(u, dev))
    torch.cuda.synchronize()
    rq, rs = orc.swiglu_quant_fp8(g, u)
    assert_same("scales", host(s), rs)
    assert_same("codes", host(q), rq)
