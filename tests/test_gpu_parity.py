"""GPU parity: every output byte of the HIP kernels equals the CPU oracle's on the
same seeded inputs (bit-exact; the quantized codes and FP32 scales are integer-like
results of a fixed FP32 arithmetic, so no tolerance applies).  Sizes span several
tiles with ragged tails; edge cases cover NaN, subnormal, -0, all-zero and empty
inputs.  Full-size workloads live in test_gpu_full_size.py."""
import ctypes
import os

import numpy as np
import pytest
import torch

import nvfp4_quantization_amd as mxq
from nvfp4_quantization_amd import synth
from tests.gpu_util import announce, assert_same, bits16, device, host

pytestmark = pytest.mark.gpu


def bf16_dev(a_u16, dev):
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).to(dev).view(torch.bfloat16)


# ============================================================== FP8 1x128
@pytest.mark.parametrize("m,k,pad", [(256, 1024, 0), (1, 128, 0), (33, 384, 8), (300, 2048, 64)])
def test_fp8_1x128_random(orc, m, k, pad):
    dev = device()
    announce(f"fp8_1x128 m={m} k={k} pad={pad}")
    w = synth.plain_fp8(m, k + pad, seed=100 + m)
    x = w.tensors["x"].to(dev)[:, :k]              # row stride k + pad
    q, s = mxq.mxq_quant_fp8_1x128(x)
    torch.cuda.synchronize()
    rq, rs = orc.quant_fp8_1x128(bits16(x.contiguous()))
    assert_same("codes", host(q), rq)
    assert_same("scales", host(s), rs)
    qt, st = mxq.mxq_quant_fp8_1x128(x, scale_transposed=True)
    torch.cuda.synchronize()
    assert_same("codes(T)", host(qt), rq)
    assert_same("scales(T)", host(st), rs.T)


def edge_matrix(m, k, seed):
    """BF16 bit patterns with the edge cases spread over rows."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32) * np.exp2(rng.integers(-30, 30, (m, 1)))
    b = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    if m >= 8:
        b[0, 3] = 0x7FC0                   # quiet NaN
        b[1, 200 % k] = 0x7F81             # signalling NaN
        b[2, 5] = 0xFFC1                   # negative NaN
        b[3, :] = 0                        # all-zero row
        b[4, :16] = 0x8000                 # -0 block
        b[5, :] = rng.integers(1, 0x80, k)          # BF16 subnormals
        b[6, :64] = rng.integers(0x8001, 0x8080, 64)  # negative subnormals
        b[7, :] = 0x3F80                   # all exactly 1.0 (ties and exact grid values)
    if m >= 12:
        b[8, 1::7] = 0x8000                # -0 inside blocks with nonzero values
        b[9, 2::5] = 0x0000
        b[10, :] = [0x3F40, 0x3FA0, 0x3FE0, 0x4020, 0x4060, 0x40A0, 0x3E80, 0x40C0] * (k // 8)  # E2M1 ties
        b[11, :] = b[11, :] | 0x8000       # an all-negative row
    return b


def test_fp8_1x128_edges(orc):
    dev = device()
    announce("fp8_1x128 edges")
    b = edge_matrix(64, 512, 7)
    x = bf16_dev(b, dev)
    q, s = mxq.mxq_quant_fp8_1x128(x)
    torch.cuda.synchronize()
    rq, rs = orc.quant_fp8_1x128(b)
    assert_same("codes", host(q), rq)
    assert_same("scales", host(s), rs)


def test_fp8_1x128_guard_bytes(orc):
    """Outputs sit inside 0xCD-filled buffers: nothing outside them is written."""
    dev = device()
    announce("fp8_1x128 guard bytes")
    m, k = 40, 640
    b = edge_matrix(m, k, 8)
    x = bf16_dev(b, dev)
    qbuf = torch.full((m * k + 512,), 0xCD, dtype=torch.uint8, device=dev)
    sbuf = torch.full((m * k // 128 + 128,), -7.0, dtype=torch.float32, device=dev)
    q = qbuf[256:256 + m * k].view(m, k)
    s = sbuf[64:64 + m * k // 128].view(m, k // 128)
    mxq.mxq_quant_fp8_1x128(x, q=q, scales=s)
    torch.cuda.synchronize()
    qb, sb = host(qbuf), host(sbuf)
    assert (qb[:256] == 0xCD).all() and (qb[256 + m * k:] == 0xCD).all()
    assert (sb[:64] == -7.0).all() and (sb[64 + m * k // 128:] == -7.0).all()
    rq, rs = orc.quant_fp8_1x128(b)
    assert_same("codes", qb[256:256 + m * k], rq)


def test_fp8_1x128_empty():
    dev = device()
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
    q, s = mxq.mxq_quant_fp8_1x128(x)
    assert q.shape == (0, 256)


# ============================================================== FP8 block variants
@pytest.mark.parametrize("m,k", [(256, 256), (300, 384), (1, 128), (129, 128), (1000, 512)])
@pytest.mark.parametrize("options", [0, 1])
@pytest.mark.parametrize("dirs", ["row+col", "col", "row"])
def test_fp8_blockwise(orc, m, k, options, dirs):
    dev = device()
    announce(f"fp8 blockwise m={m} k={k} options={options} {dirs}")
    rng = np.random.default_rng(m + k + options)
    x = (rng.standard_normal((m, k)).astype(np.float32) * np.exp2(rng.integers(-10, 10, (m, 1)))
         * np.exp2(rng.integers(-6, 6, (1, k))))
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    row, col = "row" in dirs, "col" in dirs
    rq, rs, cq, cs = mxq.mxq_quant_fp8_blockwise(bf16_dev(xb, dev), options, rowwise=row, columnwise=col)
    torch.cuda.synchronize()
    wq, ws, wcq, wcs = orc.quant_fp8_blockwise(xb, options, rowwise=row, columnwise=col)
    if row:
        assert_same("row_scales", host(rs), ws)
        assert_same("row_codes", host(rq), wq)
    if col:
        assert_same("col_scales", host(cs), wcs)
        assert_same("col_codes", host(cq.contiguous()), wcq)


@pytest.mark.parametrize("m", [300, 256])
def test_fp8_blockwise_strided_layouts(orc, m):
    """Both outputs of the blockwise call through the C ABI with padded code rows and
    transposed scale layouts (row-wise scale (r, g) at r + g * (m + 4); column-wise
    scale (c, b) at c + b * (k + 8)): every code and scale lands where the strides say
    and matches the oracle, and no padding byte is written."""
    dev = device()
    announce(f"fp8 blockwise strided layouts m={m}")
    k = 384
    rng = np.random.default_rng(90 + m)
    x = rng.standard_normal((m, k)).astype(np.float32) * np.exp2(rng.integers(-8, 8, (m, 1)))
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    xd = bf16_dev(xb, dev)
    nb = (m + 127) // 128
    rld, cld = k + 32, (m + 15) // 16 * 16 + 32
    rs_b, cs_b = m + 4, k + 8
    rq = torch.full((m, rld), 0xEE, dtype=torch.uint8, device=dev)
    cq = torch.full((k, cld), 0xEE, dtype=torch.uint8, device=dev)
    rs = torch.full((k // 128 * rs_b,), -7.0, dtype=torch.float32, device=dev)
    cs = torch.full((nb * cs_b,), -7.0, dtype=torch.float32, device=dev)
    ro = mxq._FP8BlockOut(rq.data_ptr(), rld, rs.data_ptr(), 1, rs_b)
    co = mxq._FP8BlockOut(cq.data_ptr(), cld, cs.data_ptr(), 1, cs_b)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert mxq.lib().mxq_quant_fp8_blockwise(ctypes.c_void_p(xd.data_ptr()), m, k, k, 0, ctypes.byref(ro),
                                             ctypes.byref(co), st) == 0
    torch.cuda.synchronize()
    wq, ws, wcq, wcs = orc.quant_fp8_blockwise(xb, 0)
    rq_h, cq_h, rs_h, cs_h = host(rq), host(cq), host(rs), host(cs)
    assert_same("row_codes", rq_h[:, :k].copy(), wq)
    assert_same("col_codes", cq_h[:, :m].copy(), wcq)
    assert (rq_h[:, k:] == 0xEE).all() and (cq_h[:, m:] == 0xEE).all(), "padding written"
    rs_t = rs_h.reshape(k // 128, rs_b)
    cs_t = cs_h.reshape(nb, cs_b)
    assert_same("row_scales", rs_t[:, :m].T.copy(), ws)
    assert_same("col_scales", cs_t[:, :k].T.copy(), wcs)
    assert (rs_t[:, m:] == -7.0).all() and (cs_t[:, k:] == -7.0).all(), "scale padding written"


def test_fp8_blockwise_edges(orc):
    """NaN (quiet, signalling, negative), zero and -0 blocks, subnormals and exact ties
    in both directions, with a ragged last row block."""
    dev = device()
    announce("fp8 blockwise edges")
    b = edge_matrix(200, 256, 31)
    b[150:, 7] = 0x7FC0                      # a NaN in column 7 of the ragged block
    for options in (0, 1):
        rq, rs, cq, cs = mxq.mxq_quant_fp8_blockwise(bf16_dev(b, dev), options, rowwise=True, columnwise=True)
        torch.cuda.synchronize()
        wq, ws, wcq, wcs = orc.quant_fp8_blockwise(b, options)
        assert_same("row_scales", host(rs), ws)
        assert_same("row_codes", host(rq), wq)
        assert_same("col_scales", host(cs), wcs)
        assert_same("col_codes", host(cq.contiguous()), wcq)


@pytest.mark.parametrize("options", [0, 1])
def test_dsa_fp8_ex_layouts(orc, options):
    """The (token, head) scale layouts: [tokens][heads] and the transposed [heads][T]
    with T padded past the tokens (the padding keeps its sentinel), with UE8M0 or not."""
    dev = device()
    announce(f"dsa fp8 ex layouts options={options}")
    tokens, heads, pad = 37, 8, 64
    w = synth.dsa_rotate_fp8(tokens=tokens, heads=heads, seed=500 + options)
    pe, nope = w.tensors["pe"].to(dev), w.tensors["nope"].to(dev)
    pn, nn = bits16(w.tensors["pe"]), bits16(w.tensors["nope"])
    q, s = mxq.mxq_hadamard_quant_fp8_ex(pe, nope, options, heads)
    torch.cuda.synchronize()
    wq, wsc = orc.hadamard_quant_fp8_ex(pn, nn, options, heads)
    assert_same("codes", host(q), wq)
    assert_same("scales", host(s), wsc)
    st = torch.full((heads * pad,), float("nan"), dtype=torch.float32, device=dev)
    q2, s2 = mxq.mxq_hadamard_quant_fp8_ex(pe, nope, options, heads, scales=st, scale_stride_token=1,
                                           scale_stride_head=pad)
    torch.cuda.synchronize()
    wq2, ws2 = orc.hadamard_quant_fp8_ex(pn, nn, options, heads, token_stride=1, head_stride=pad,
                                         scale_size=heads * pad)
    assert_same("codes", host(q2), wq2)
    assert_same("scales_transposed", host(s2), ws2)


# ============================================================== SwiGLU -> FP8 1x128
def swiglu_inputs(m, n, seed, edges=False):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((m, n)).astype(np.float32) * 3
    u = rng.standard_normal((m, n)).astype(np.float32) * np.exp2(rng.integers(-10, 10, (m, 1)))
    gb = torch.from_numpy(g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    ub = torch.from_numpy(u).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    if edges and m >= 8:
        gb[0, 5] = 0x7FC0                  # NaN gate
        ub[1, 7] = 0xFFC1                  # NaN up
        gb[2, :] = 0                       # SiLU(0) = 0: a zero row
        gb[3, :] = 0x4200                  # gate 32: SiLU(g) = g exactly
        gb[4, :] = 0xC2C0                  # gate -96: e^96 overflows, SiLU = -0
        gb[5, :64] = rng.integers(1, 0x80, 64)        # subnormal gates
        ub[6, :] = rng.integers(0x8001, 0x8080, n)    # subnormal ups
        gb[7, :] = 0xC1A0                  # gate -20 (a tiny negative SiLU)
    return gb, ub


@pytest.mark.parametrize("m,n", [(1, 128), (33, 384), (256, 2048), (7, 4096)])
def test_swiglu_fp8_random(orc, m, n):
    dev = device()
    announce(f"swiglu fp8 m={m} n={n}")
    gb, ub = swiglu_inputs(m, n, 400 + m)
    q, s = mxq.mxq_swiglu_quant_fp8(bf16_dev(gb, dev), bf16_dev(ub, dev))
    torch.cuda.synchronize()
    rq, rs = orc.swiglu_quant_fp8(gb, ub)
    assert_same("scales", host(s), rs)
    assert_same("codes", host(q), rq)


def test_swiglu_fp8_fused_layout_and_edges(orc):
    """gate / up as the two halves of one [m][2n] buffer, transposed scales, and NaN,
    zero, overflowing-exponential and subnormal rows."""
    dev = device()
    announce("swiglu fp8 fused layout + edges")
    m, n = 40, 256
    gb, ub = swiglu_inputs(m, n, 77, edges=True)
    gu = bf16_dev(np.concatenate([gb, ub], axis=1), dev)
    q, s = mxq.mxq_swiglu_quant_fp8(gu[:, :n], gu[:, n:], scale_transposed=True)
    torch.cuda.synchronize()
    rq, rs = orc.swiglu_quant_fp8(gb, ub, scale_transposed=True)
    assert_same("scales", host(s), rs)
    assert_same("codes", host(q), rq)


def test_swiglu_fp8_exp_sweep(orc):
    """The kernel's SiLU on a dense sweep of gates (every BF16 value in [-104, 104] with
    up = 1): h = SILU(g) exactly, so the codes and scales show the GPU's EXP and
    division match the stated algorithm bit for bit wherever they decide a code."""
    dev = device()
    announce("swiglu fp8 exp sweep")
    b = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    v = f32 = (b.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(f32) & (np.abs(v) <= 104.0)
    gates = b[keep]
    n = 128
    m = (gates.size + n - 1) // n
    gb = np.zeros(m * n, np.uint16)
    gb[:gates.size] = gates
    gb = gb.reshape(m, n)
    ub = np.full((m, n), 0x3F80, np.uint16)
    q, s = mxq.mxq_swiglu_quant_fp8(bf16_dev(gb, dev), bf16_dev(ub, dev))
    torch.cuda.synchronize()
    rq, rs = orc.swiglu_quant_fp8(gb, ub)
    assert_same("scales", host(s), rs)
    assert_same("codes", host(q), rq)


# ============================================================== DSA rotate + FP8
@pytest.mark.parametrize("tokens,heads,d_pe", [(64, 8, 64), (7, 9, 64), (32, 4, 0), (32, 4, 128), (16, 5, 8)])
def test_dsa_random(orc, tokens, heads, d_pe):
    dev = device()
    announce(f"dsa tokens={tokens} heads={heads} d_pe={d_pe}")
    w = synth.dsa_rotate_fp8(tokens=tokens, heads=heads, d_pe=d_pe, seed=200 + tokens)
    pe = w.tensors["pe"].to(dev) if d_pe > 0 else None
    nope = w.tensors["nope"].to(dev) if d_pe < 128 else None
    q, s = mxq.mxq_hadamard_quant_fp8(pe, nope)
    torch.cuda.synchronize()
    rq, rs = orc.hadamard_quant_fp8(bits16(w.tensors["pe"]), bits16(w.tensors["nope"]))
    assert_same("codes", host(q), rq)
    assert_same("scales", host(s), rs)


def test_dsa_strided_and_edges(orc):
    dev = device()
    announce("dsa strided + edges")
    m = 96
    b = edge_matrix(m, 128, 9)
    big = np.zeros((m, 256), np.uint16)
    big[:, :64] = b[:, :64]              # pe in a wider buffer (row stride 256)
    big[:, 128:192] = b[:, 64:]          # nope further along the same rows
    t = bf16_dev(big, dev)
    q, s = mxq.mxq_hadamard_quant_fp8(t[:, :64], t[:, 128:192])
    torch.cuda.synchronize()
    rq, rs = orc.hadamard_quant_fp8(b[:, :64], b[:, 64:])
    assert_same("codes", host(q), rq)
    assert_same("scales", host(s), rs)


def rotation_cancel_rows(m, seed, inf=True):
    """BF16 rows whose 128-point rotation has exact zeros among nonzero outputs, in every
    lane quarter: small integers (their sums cancel often), a few equal or opposite
    entries, all -0, mixed +-0, and (inf) one infinity among zeros (inf and NaN
    outputs; otherwise a row of small integers)."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-2, 3, size=(m, 128)).astype(np.float32)
    for r in range(0, m, 8):
        x[r] = 0.0
        i, j = rng.choice(128, 2, replace=False)
        x[r, i] = 1.5
        x[r, j] = 1.5 if r % 16 else -1.5
        x[r + 1] = -0.0
        x[r + 2] = np.where(rng.integers(0, 2, 128) == 1, -0.0, 0.0)
        if inf:
            x[r + 3] = 0.0
            x[r + 3, rng.integers(0, 128)] = np.inf if r % 16 else -np.inf
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("d_pe", [64, 8])
def test_dsa_rotation_exact_zeros(orc, d_pe):
    """The rotation's cross-lane stages run on negated operands in two of the four lanes
    of a row, which is exact except for the sign of an exact zero; a wave with a zero
    output recomputes its rows.  Rows with exact cancellations, -0 and infinities match
    the oracle byte for byte, through the FP8 and the NVFP4 paths."""
    dev = device()
    announce(f"dsa rotation exact zeros d_pe={d_pe}")
    b = rotation_cancel_rows(512, 61 + d_pe)
    pe, nope = bf16_dev(b[:, :d_pe].copy(), dev), bf16_dev(b[:, d_pe:].copy(), dev)
    q, s = mxq.mxq_hadamard_quant_fp8(pe, nope)
    torch.cuda.synchronize()
    rq, rs = orc.hadamard_quant_fp8(b[:, :d_pe].copy(), b[:, d_pe:].copy())
    assert_same("codes", host(q), rq)
    assert_same("scales", host(s), rs)
    # NVFP4: one tensor scale, so no infinities (they would zero every other code)
    b = rotation_cancel_rows(512, 62 + d_pe, inf=False)
    pe, nope = bf16_dev(b[:, :d_pe].copy(), dev), bf16_dev(b[:, d_pe:].copy(), dev)
    compare_dsa4(orc, b[:, :d_pe].copy(), b[:, d_pe:].copy(), pe, nope, amax_out=True)


# ============================================================== DSA rotate + NVFP4
def compare_dsa4(orc, pe_np, nope_np, pe, nope, amax_in=None, amax_out=False, call=None):
    """The DSA rotate + NVFP4 call on device tensors pe / nope against the oracle on
    their host bit patterns pe_np / nope_np, every byte."""
    if call is None:
        call = mxq.HadamardNVFP4(pe, nope, amax_in=amax_in, amax_out=amax_out)
    res = call()
    torch.cuda.synchronize()
    ref = orc.hadamard_quant_nvfp4(pe_np, nope_np, amax_in=amax_in)
    assert_same("global_scale", host(res.global_scale), np.array([ref.global_scale], np.float32))
    assert_same("scales", host(res.scales), ref.scales)
    assert_same("codes", host(res.codes), ref.codes)
    if amax_out:
        assert_same("amax", host(res.amax), np.array([ref.amax], np.float32))
    return res, ref


@pytest.mark.parametrize("tokens,heads,d_pe", [(64, 8, 64), (7, 9, 64), (32, 4, 0), (32, 4, 128), (16, 5, 8),
                                               (625, 32, 64)])
def test_dsa_nvfp4_random(orc, tokens, heads, d_pe):
    dev = device()
    announce(f"dsa nvfp4 tokens={tokens} heads={heads} d_pe={d_pe}")
    w = synth.dsa_rotate_fp8(tokens=tokens, heads=heads, d_pe=d_pe, seed=300 + tokens)
    pe = w.tensors["pe"].to(dev) if d_pe > 0 else None
    nope = w.tensors["nope"].to(dev) if d_pe < 128 else None
    compare_dsa4(orc, bits16(w.tensors["pe"]), bits16(w.tensors["nope"]), pe, nope, amax_out=True)


def test_dsa_nvfp4_strided_and_edges(orc):
    """NaN rows, zero / -0 / subnormal rows, exact ties, rows 2^-30 .. 2^30 apart (the
    small ones underflow to scale code 0 under the one tensor scale), and pe / nope
    as column slices of wider rows."""
    dev = device()
    announce("dsa nvfp4 strided + edges")
    m = 100
    b = edge_matrix(m, 128, 19)
    big = np.zeros((m, 256), np.uint16)
    big[:, :64] = b[:, :64]
    big[:, 128:192] = b[:, 64:]
    t = bf16_dev(big, dev)
    compare_dsa4(orc, b[:, :64], b[:, 64:], t[:, :64], t[:, 128:192], amax_out=True)


@pytest.mark.parametrize("scale", [1.0, 0.25, 4.0])
def test_dsa_nvfp4_supplied_amax(orc, scale):
    """A supplied amax (the measured one times `scale`): one pass, saturating blocks
    above it; the measured amax comes out as well."""
    dev = device()
    announce(f"dsa nvfp4 supplied amax x{scale}")
    w = synth.dsa_rotate_fp8(tokens=48, heads=8, seed=77)
    pe_np, nope_np = bits16(w.tensors["pe"]), bits16(w.tensors["nope"])
    A = orc.hadamard_quant_nvfp4(pe_np, nope_np).amax
    amax_in = np.float32(A * np.float32(scale))
    compare_dsa4(orc, pe_np, nope_np, w.tensors["pe"].to(dev), w.tensors["nope"].to(dev),
                 amax_in=float(amax_in), amax_out=True)


def test_dsa_nvfp4_empty(orc):
    """No rows: only the tensor scale (the floor, or the supplied amax's) and a zero
    measured amax."""
    dev = device()
    announce("dsa nvfp4 empty")
    z = np.zeros((0, 64), np.uint16)
    for amax_in in (None, 2.5):
        res = mxq.mxq_hadamard_quant_nvfp4(bf16_dev(z, dev), bf16_dev(z, dev), amax_in=amax_in, amax_out=True)
        torch.cuda.synchronize()
        ref = orc.hadamard_quant_nvfp4(z, z, amax_in=amax_in)
        assert_same("global_scale", host(res.global_scale), np.array([ref.global_scale], np.float32))
        assert_same("amax", host(res.amax), np.zeros(1, np.float32))


def test_dsa_nvfp4_reuse(orc):
    """One prepared call on a workspace of arbitrary contents (every byte 0xA5) run
    twice, then a smaller input through the same workspace (left over partials and
    table from the larger call): every run matches (the call's kernels meet in
    stream order and keep no state in the workspace)."""
    dev = device()
    announce("dsa nvfp4 reuse")
    w = synth.dsa_rotate_fp8(tokens=100, heads=8, seed=78)
    pe, nope = w.tensors["pe"].to(dev), w.tensors["nope"].to(dev)
    pe_np, nope_np = bits16(w.tensors["pe"]), bits16(w.tensors["nope"])
    need = mxq.mxq_hadamard_quant_nvfp4_workspace_size(800)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=dev)
    call = mxq.HadamardNVFP4(pe, nope, amax_out=True, workspace=ws)
    compare_dsa4(orc, pe_np, nope_np, pe, nope, amax_out=True, call=call)
    compare_dsa4(orc, pe_np, nope_np, pe, nope, amax_out=True, call=call)
    small = mxq.HadamardNVFP4(pe[:300], nope[:300], workspace=call.workspace)
    compare_dsa4(orc, pe_np[:300], nope_np[:300], pe[:300], nope[:300], call=small)


def test_dsa_nvfp4_large(orc):
    """524,352 rows (8193 tokens x 64 heads, a ragged last work-group): 8193
    amax partials folded in two rounds of the scale kernel's loads."""
    dev = device()
    announce("dsa nvfp4, 524352 rows")
    w = synth.dsa_rotate_fp8(tokens=8193, heads=64, d_pe=64, seed=80)
    pe, nope = w.tensors["pe"].to(dev), w.tensors["nope"].to(dev)
    compare_dsa4(orc, bits16(w.tensors["pe"]), bits16(w.tensors["nope"]), pe, nope, amax_out=True)


# ============================================================== grouped NVFP4
def compare_grouped(orc, x_dev, sections, mask, flags, seed=None, ro=None, co=None, out=None, threads=8,
                    workspace=None):
    call = mxq.GroupedNVFP4(x_dev, sections, mask, flags, seed, ro, co, out=out, workspace=workspace)
    res = call()
    torch.cuda.synchronize()
    assert mxq.workspace_protocol_clear(call.workspace), \
        "the single-read form's error word or a partial word was left nonzero"
    ref = orc.group_rht_quant_nvfp4(bits16(x_dev), sections, mask, flags, seed or 0, ro, co, threads=threads)
    if flags & 1:
        assert_same("row_global", host(res.row_global), ref.row_global)
        assert_same("row_scales", host(res.row_scales), ref.row_scales)
        assert_same("row_codes", host(res.row_codes), ref.row_codes)
    if flags & 2:
        assert_same("col_global", host(res.col_global), ref.col_global)
        assert_same("col_scales", host(res.col_scales), ref.col_scales)
        assert_same("col_codes", host(res.col_codes), ref.col_codes)
    if flags & 4:
        assert_same("fp8_scales", host(res.fp8_scales), ref.fp8_scales)
        assert_same("fp8_codes", host(res.fp8_codes), ref.fp8_codes)
    return res, ref


@pytest.mark.parametrize("flags", [3, 1, 2, 7, 4, 5, 6])
def test_grouped_rne_small(orc, flags):
    dev = device()
    announce(f"grouped rne small flags={flags}")
    w = synth.grouped_nvfp4(total_rows=1280, k=640, parts=4, seed=31)
    compare_grouped(orc, w.tensors["x"].to(dev), w.params["split_sections"], w.params["sign_mask"], flags)


@pytest.mark.parametrize("mask", [0x0000, 0xFFFF, 0x8001, 0x5A3C])
def test_grouped_sign_masks(orc, mask):
    dev = device()
    announce(f"grouped mask={mask:#x}")
    w = synth.grouped_nvfp4(total_rows=512, k=256, parts=3, seed=32)
    compare_grouped(orc, w.tensors["x"].to(dev), w.params["split_sections"], mask, 3)


@pytest.mark.parametrize("k", [384, 512])
def test_grouped_sr_small(orc, k):
    dev = device()
    announce(f"grouped sr small k={k}")
    w = synth.grouped_nvfp4_sr(total_rows=1024, k=k, parts=12, forced_empty=3, seed=33)
    p = w.params
    compare_grouped(orc, w.tensors["x"].to(dev), p["split_sections"], p["sign_mask"], 3, p["seed"],
                    p["row_offsets"], p["col_offsets"])
    # one direction stochastic, the other nearest-even
    compare_grouped(orc, w.tensors["x"].to(dev), p["split_sections"], p["sign_mask"], 3, p["seed"],
                    None, p["col_offsets"])
    compare_grouped(orc, w.tensors["x"].to(dev), p["split_sections"], p["sign_mask"], 7, p["seed"],
                    p["row_offsets"], None)


@pytest.mark.parametrize("k", [256, 512])
def test_grouped_sr_product_and_division_passes(orc, k):
    """Stochastic rounding over sections whose scale tables differ: a pass whose table
    has a stochastic multiplier for every scale code multiplies, the others divide.
    Both kinds occur in this call (read from the flags the tables leave in the
    workspace), and every output matches the oracle.  k = 256: the three-kernel form;
    k = 512: the single-read form (its tables built by 256-thread work-groups)."""
    dev = device()
    announce(f"grouped sr: product and division passes in one call, k={k}")
    factors = [1.0, 3.0, 2.0 ** 40, 7.0 * 2.0 ** -10, 21.0, 0.37, 5.5e3, 1.9e-6, 42.0, 0.011, 613.0, 2.5]
    S = len(factors)
    rng = np.random.default_rng(73)
    base = rng.standard_normal((S * 128, k)).astype(np.float32)
    for i, f in enumerate(factors):
        block = base[i * 128:(i + 1) * 128]
        block *= np.float32(f) / np.float32(np.abs(block).max())
    x = torch.from_numpy(base).to(torch.bfloat16).to(dev)
    ro, co = list(range(7, 7 + S)), list(range(900, 900 + S))
    call = mxq.GroupedNVFP4(x, [128] * S, 0x6C1B, 3, 0xC0FFEE, ro, co)
    compare_grouped(orc, x, [128] * S, 0x6C1B, 3, 0xC0FFEE, ro, co, workspace=call.workspace)
    tables = host(call.workspace)[mxq.WORKSPACE_TABLES:mxq.WORKSPACE_TABLES + S * 2 * 128 * 16].view(np.float32)
    flags = tables.reshape(S, 2, 128, 4)[:, :, 127, 0]
    assert (flags == 0.0).any() and (flags == 1.0).any(), flags


@pytest.mark.parametrize("flags,sr", [(3, False), (3, True), (7, False), (1, False), (2, True)])
def test_grouped_single_read_reuse(orc, flags, sr):
    """The single-read form (k a multiple of 512, every section within the resident
    grid): one workspace through three calls, the second on other sections and
    fewer rows; each matches the oracle and leaves the workspace's error word and
    partial words at zero."""
    dev = device()
    announce(f"grouped single-read reuse flags={flags} sr={sr}")
    w = synth.grouped_nvfp4_sr(total_rows=3072, k=2048, parts=9, forced_empty=2, seed=40)
    p = w.params
    x = w.tensors["x"].to(dev)
    seed, ro, co = (p["seed"], p["row_offsets"], p["col_offsets"]) if sr else (None, None, None)
    ws = mxq.alloc_workspace(3072, 2048, 9, flags, dev)
    for sections, rows in ((p["split_sections"], 3072), ([1024, 0, 512, 128, 384], 2048),
                           (p["split_sections"], 3072)):
        S = len(sections)
        xi = x[:rows].contiguous()
        call = mxq.GroupedNVFP4(xi, sections, p["sign_mask"], flags, seed, ro[:S] if ro else None,
                                co[:S] if co else None, workspace=ws)
        res = call()
        torch.cuda.synchronize()
        assert mxq.workspace_protocol_clear(ws), "workspace left nonzero"
        ref = orc.group_rht_quant_nvfp4(bits16(xi), sections, p["sign_mask"], flags, seed or 0,
                                        ro[:S] if ro else None, co[:S] if co else None, threads=8)
        for name in ("row_global", "row_scales", "row_codes", "col_global", "col_scales", "col_codes",
                     "fp8_scales", "fp8_codes"):
            got = getattr(res, name)
            if got is not None:
                assert_same(name, host(got), getattr(ref, name))


def dirty_workspace(total_rows, k, num_sections, flags, dev):
    """A workspace whose bytes are all 0xA5 except the single-read form's error word
    and partial words (the only words a call needs at zero)."""
    n = mxq.mxq_group_rht_quant_nvfp4_workspace_size(total_rows, k, num_sections, flags)
    ws = torch.full((n,), 0xA5, dtype=torch.uint8, device=dev)
    ws[mxq.WORKSPACE_STATUS:mxq.WORKSPACE_STATUS + 512] = 0
    ws[mxq.WORKSPACE_SLOTS:mxq.WORKSPACE_SLOTS + mxq.WORKSPACE_SLOTS_BYTES] = 0
    return ws


@pytest.mark.parametrize("case", ["one_wave_amax", "supplied"])
def test_grouped_any_workspace_contents(orc, case):
    """The multi-kernel form's kernels meet only through the stream order: partials
    and tables left as arbitrary bytes (0xA5) change nothing, on the amax pass with one
    tile per work-group (k / 128 odd) and with supplied maxima; the workspace is then
    used again for a smaller call."""
    dev = device()
    announce(f"grouped dirty workspace {case}")
    if case == "one_wave_amax":
        w = synth.grouped_nvfp4(total_rows=1280, k=640, parts=4, seed=55)
        x, p = w.tensors["x"].to(dev), w.params
        ws = dirty_workspace(1280, 640, 4, 3, dev)
        compare_grouped(orc, x, p["split_sections"], p["sign_mask"], 3, workspace=ws)
        compare_grouped(orc, x[:512].contiguous(), [256, 0, 256], p["sign_mask"], 3, workspace=ws)
    else:
        w = synth.grouped_nvfp4(total_rows=1280, k=640, parts=5, seed=57)
        x, p = w.tensors["x"].to(dev), w.params
        sec, mask = p["split_sections"], p["sign_mask"]
        meas = orc.group_rht_quant_nvfp4(bits16(x), sec, mask, 3, threads=8)
        ws = dirty_workspace(1280, 640, 5, 3, dev)
        compare_grouped_amax(orc, x, sec, mask, 3, (meas.row_amax * np.float32(0.5), meas.col_amax),
                             workspace=ws)
        compare_grouped_amax(orc, x, sec, mask, 3, None, workspace=ws)


def test_grouped_any_workspace_contents_four_wave_amax():
    """The amax pass with four tiles per work-group, on a group too large for the
    single-read form (1056 four-tile items, above its 1024): a workspace of 0xA5 bytes
    (but the single-read words) gives the same bytes as a zeroed one, with stochastic
    rounding and FP8 (a property of the call, compared call against call; parity of
    this shape against the oracle is the full-size tests' part)."""
    dev = device()
    announce("grouped dirty workspace: four-tile amax work-groups, 4224 x 16384")
    w = synth.grouped_nvfp4_sr(total_rows=4224, k=16384, parts=3, forced_empty=0, seed=56)
    x, p = w.tensors["x"].to(dev), w.params
    args = (x, p["split_sections"], p["sign_mask"], 7, p["seed"], p["row_offsets"], p["col_offsets"])
    clean = mxq.GroupedNVFP4(*args)()
    dirty = mxq.GroupedNVFP4(*args, workspace=dirty_workspace(4224, 16384, 3, 7, dev))()
    torch.cuda.synchronize()
    for n in ("row_global", "row_scales", "row_codes", "col_global", "col_scales", "col_codes",
              "fp8_scales", "fp8_codes"):
        assert torch.equal(getattr(clean, n), getattr(dirty, n)), n


@pytest.mark.parametrize("sr", [False, True])
def test_grouped_single_read_deferred(orc, sr):
    """The single-read form's fallback for a device short of room: in the test build
    of the library every waiting item gives up at once, marks its partial deferred and
    ends, and its section's last item reads and quantizes those tiles itself.  Every
    output byte still matches the oracle, and the workspace is left clear."""
    dev = device()
    announce(f"grouped single-read deferred sr={sr}")
    path = os.path.join(os.path.dirname(mxq.LIB_PATH), "libmxq_defer0.so")
    if not os.path.exists(path):
        pytest.fail(f"{path} is missing: build the library")
    w = synth.grouped_nvfp4_sr(total_rows=2048, k=2048, parts=7, forced_empty=2, seed=41)
    p = w.params
    seed, ro, co = (p["seed"], p["row_offsets"], p["col_offsets"]) if sr else (None, None, None)
    x = w.tensors["x"].to(dev)
    saved = mxq._lib
    try:
        mxq._lib = None
        mxq.LIB_PATH, main_path = path, mxq.LIB_PATH
        try:
            call = mxq.GroupedNVFP4(x, p["split_sections"], p["sign_mask"], 3, seed, ro, co)
            res = call()
            torch.cuda.synchronize()
        finally:
            mxq.LIB_PATH = main_path
    finally:
        mxq._lib = saved
    assert mxq.workspace_protocol_clear(call.workspace), "workspace left nonzero"
    ref = orc.group_rht_quant_nvfp4(bits16(x), p["split_sections"], p["sign_mask"], 3, seed or 0, ro, co,
                                    threads=8)
    for name in ("row_global", "row_scales", "row_codes", "col_global", "col_scales", "col_codes"):
        assert_same(name, host(getattr(res, name)), getattr(ref, name))


def test_grouped_large_moe_recipe_small(orc):
    dev = device()
    announce("grouped large-moe recipe at small size")
    w = synth.large_moe(total_rows=2048, k=896, parts=12, forced_empty=3, seed=34)
    compare_grouped(orc, w.tensors["x"].to(dev), w.params["split_sections"], w.params["sign_mask"], 7)


def tie_matrix(rows, k, sections, mask, seed):
    """Short binary values whose exact quotients often land on E2M1 rounding
    boundaries: every section's max |x| is 2688 and the max |H16 D x| / 4 of every
    section is 2688 too, so both tensor scales are exactly 1 and the divisors are
    the E4M3 values themselves; some rows hold 3 (scale 0.5) and every boundary
    times 0.5.  The kernels must then fall back from the product to the exact
    division for scale codes where no multiplier decides like the quotient."""
    rng = np.random.default_rng(seed)
    mant = np.array([1, 1.5, 1.25, 1.75, 3, 3.5, 5, 6, 7, 0.75, 0.5, 0.25])
    v = rng.choice(mant, size=(rows, k)) * 2.0 ** rng.integers(-6, 4, size=(rows, k))
    v *= rng.choice([-1.0, 1.0], size=(rows, k))
    ties = np.array([3.0, 0.125, 0.375, 0.625, 0.875, 1.25, 1.75, 2.5] * 2)
    r0 = 0
    for ms in sections:
        if ms == 0:
            continue
        v[r0 + 5, 17] = 2688.0                              # row-wise section amax
        signs = np.array([-1.0 if (mask >> t) & 1 else 1.0 for t in range(16)])
        v[r0 + 32:r0 + 48, 40] = 672.0 * signs              # H16 D x = (10752, 0, ...)
        for r in range(r0 + 64, r0 + 64 + 8):              # row blocks with exact ties everywhere
            v[r, :16] = ties * rng.choice([-1.0, 1.0], size=16)
        r0 += ms
    f32 = v.astype(np.float32)
    return (f32.view(np.uint32) >> 16).astype(np.uint16)    # exact: every value is short


@pytest.mark.parametrize("k", [256, 512])
def test_grouped_exact_ties(orc, k):
    dev = device()
    announce(f"grouped exact ties k={k}")
    sections = [256, 0, 384]
    for mask in (0x0000, 0x6C93):
        b = tie_matrix(640, k, sections, mask, 77 + mask)
        x = bf16_dev(b, dev)
        compare_grouped(orc, x, sections, mask, 3)
        compare_grouped(orc, x, sections, mask, 7)


@pytest.mark.parametrize("k", [256, 512])          # one- and four-wave quant work-groups
def test_grouped_edges(orc, k):
    dev = device()
    announce(f"grouped edges k={k}")
    b = edge_matrix(384, k, 10)
    b[100:116, 40] = 0x7FC0            # NaN in a column block
    b[200:216, :] = 0                   # a zero 16-row band
    x = bf16_dev(b, dev)
    compare_grouped(orc, x, [128, 256], 0xA5A5, 7)
    compare_grouped(orc, x, [384], 0x0F0F, 3, seed=5, ro=[11], co=[12])


@pytest.mark.parametrize("sections", [[128], [0, 0, 256, 0], [128] * 9, [0] * 40 + [256] + [0] * 30,
                                      [128, 0] * 70 + [256] * 10, [0, 0, 0]])
@pytest.mark.parametrize("k", [256, 1024])
def test_grouped_section_shapes(orc, sections, k):
    """One section, all-empty-but-one, many 128-row sections, more than one launch
    group of 32 sections (71 and 150 sections: three and five groups), and an
    all-empty call (only the floor scales are written)."""
    dev = device()
    total = sum(sections)
    announce(f"grouped sections n={len(sections)} total={total} k={k}")
    w = synth.grouped_nvfp4(total_rows=max(total, 128), k=k, parts=1, seed=35)
    x = w.tensors["x"][:total].contiguous().to(dev)
    compare_grouped(orc, x, sections, 0x1357, 7)


def test_grouped_max_sections(orc):
    dev = device()
    announce("grouped 256 sections")
    rng = np.random.default_rng(36)
    sections = [int(v) * 128 for v in rng.integers(0, 3, 256)]
    total = sum(sections)
    w = synth.grouped_nvfp4(total_rows=total, k=128, parts=1, seed=36)
    compare_grouped(orc, w.tensors["x"].to(dev), sections, 0xBEEF, 3, seed=9,
                    ro=list(range(256)), co=list(range(1000, 1256)))


@pytest.mark.parametrize("k", [384, 512])
def test_grouped_guard_bytes(orc, k):
    dev = device()
    announce(f"grouped guard bytes k={k}")
    sections, flags = [256, 0, 128], 7
    total, S = sum(sections), len(sections)
    w = synth.grouped_nvfp4(total_rows=total, k=k, parts=1, seed=37)
    x = w.tensors["x"].to(dev)
    G = 4096
    sizes = dict(row_codes=total * k // 2, row_scales=total * k // 16, col_codes=total * k // 2,
                 col_scales=total * k // 16, fp8_codes=total * k)
    bufs, out = {}, mxq.NVFP4Result()
    for name, n in sizes.items():
        bufs[name] = torch.full((n + 2 * G,), 0xCD, dtype=torch.uint8, device=dev)
        setattr(out, name, bufs[name][G:G + n])
    for name, n in dict(row_global=S, col_global=S, fp8_scales=total * k // 128).items():
        bufs[name] = torch.full((n + 2 * 64,), -3.0, dtype=torch.float32, device=dev)
        setattr(out, name, bufs[name][64:64 + n])
    out.row_codes = out.row_codes.view(total, k // 2)
    out.row_scales = out.row_scales.view(total, k // 16)
    out.fp8_codes = out.fp8_codes.view(total, k)
    out.fp8_scales = out.fp8_scales.view(total, k // 128)
    compare_grouped(orc, x, sections, 0x2222, flags, out=out)
    for name, t in bufs.items():
        h = host(t)
        pad = G if h.dtype == np.uint8 else 64
        fill = 0xCD if h.dtype == np.uint8 else -3.0
        assert (h[:pad] == fill).all() and (h[-pad:] == fill).all(), name


def test_grouped_run_twice_identical(orc):
    dev = device()
    announce("grouped determinism")
    w = synth.grouped_nvfp4_sr(total_rows=640, k=256, parts=5, forced_empty=1, seed=38)
    p = w.params
    x = w.tensors["x"].to(dev)
    call = mxq.GroupedNVFP4(x, p["split_sections"], p["sign_mask"], 7, p["seed"], p["row_offsets"],
                            p["col_offsets"])
    a = {k: host(v).copy() for k, v in vars(call()).items() if v is not None}
    torch.cuda.synchronize()
    b = {k: host(v) for k, v in vars(call()).items() if v is not None}
    for name in a:
        assert_same(name, b[name], a[name])


def test_grouped_graph_capture_replays(orc):
    """The call is stream-capturable (no allocation, no memset, no sync) and every
    replay reproduces the eager result."""
    dev = device()
    announce("grouped hipGraph capture")
    w = synth.grouped_nvfp4(total_rows=768, k=512, parts=3, seed=39)
    x = w.tensors["x"].to(dev)
    call = mxq.GroupedNVFP4(x, w.params["split_sections"], w.params["sign_mask"], 7)
    eager = {k: host(v).copy() for k, v in vars(call()).items() if v is not None}
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(stream=s)
    for rep in range(3):
        for v in vars(call.out).values():
            if v is not None:
                v.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, v in vars(call.out).items():
            if v is not None:
                assert_same(f"replay{rep}:{name}", host(v), eager[name])


def test_calls_on_a_side_stream(orc):
    """A call on another stream (a torch stream or a raw handle) is ordered after the
    current stream, where the binding allocated its outputs and workspace, and gives the
    current stream's result."""
    dev = device()
    announce("grouped and DSA NVFP4 calls on a side stream")
    w = synth.grouped_nvfp4(total_rows=768, k=512, parts=3, seed=41)
    x = w.tensors["x"].to(dev)
    args = (w.params["split_sections"], w.params["sign_mask"], 7)
    want = {k: host(v).copy() for k, v in vars(mxq.mxq_group_rht_quant_nvfp4(x, *args)).items() if v is not None}
    d = synth.dsa_rotate_fp8(tokens=125, heads=8, d_pe=64, seed=42)
    pe, nope = d.tensors["pe"].to(dev), d.tensors["nope"].to(dev)
    want_dsa = {k: host(v).copy() for k, v in vars(mxq.mxq_hadamard_quant_nvfp4(pe, nope)).items()
                if v is not None}
    s = torch.cuda.Stream()
    for handle in (s, s.cuda_stream):
        got = mxq.mxq_group_rht_quant_nvfp4(x, *args, stream=handle)
        got_dsa = mxq.mxq_hadamard_quant_nvfp4(pe, nope, stream=handle)
        torch.cuda.synchronize()
        for name, v in vars(got).items():
            if v is not None:
                assert_same(f"grouped:{name}", host(v), want[name])
        for name, v in vars(got_dsa).items():
            if v is not None:
                assert_same(f"dsa:{name}", host(v), want_dsa[name])


# ============================================================== Philox vs rocRAND
def test_philox_matches_rocrand(orc):
    """The Philox4x32-10 of the oracle (and so of the kernels, which match it
    byte for byte under stochastic rounding) against rocRAND's generator, run
    (not read) on the GPU: output word n is word n%4 of the block with counter n/4."""
    dev = device()
    announce("philox vs rocRAND")
    try:
        L = ctypes.CDLL("librocrand.so")
    except OSError:
        L = ctypes.CDLL("/opt/rocm/lib/librocrand.so")
    gen = ctypes.c_void_p()
    assert L.rocrand_create_generator(ctypes.byref(gen), 404) == 0       # ROCRAND_RNG_PSEUDO_PHILOX4_32_10
    seed = 0x0123456789ABCDEF
    L.rocrand_set_seed.argtypes = [ctypes.c_void_p, ctypes.c_ulonglong]
    assert L.rocrand_set_seed(gen, seed) == 0
    n = 4096
    out = torch.zeros(n, dtype=torch.int32, device=dev)
    L.rocrand_generate.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]
    assert L.rocrand_generate(gen, ctypes.c_void_p(out.data_ptr()), n) == 0
    torch.cuda.synchronize()
    got = host(out).view(np.uint32)
    L.rocrand_destroy_generator(gen)
    want = np.concatenate([orc.philox4x32_10([i, 0, 0, 0], [seed & 0xFFFFFFFF, seed >> 32])
                           for i in range(n // 4)])
    assert_same("philox stream", got, want)


def test_grouped_hand_case_b9(orc):
    """A section whose amax is 10.5 (tensor scale 2^-8) holding the hand-worked
    block [6, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, -.25, -.75, 5.5, bf16(.1), -0, 1,
    -6, 4.5]: every E2M1 tie, saturation and a -0 element (codes 7,0,2,2,4,4,6,6,
    8,A,7,0,8,2,F,6)."""
    dev = device()
    announce("grouped hand case B9")
    vals = [6, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, -.25, -.75, 5.5, 0.1, -0.0, 1, -6, 4.5]
    x = np.zeros((128, 128), np.float32)
    x[0, :16] = vals
    x[1, 16] = 10.5
    x[2, :16] = 6.25
    x[3, 32] = 2.0 ** -20
    b = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    res, ref = compare_grouped(orc, bf16_dev(b, dev), [128], 0, 1)
    codes = host(res.row_codes)[0, :8].tolist()
    assert codes == [0x07, 0x22, 0x44, 0x66, 0xA8, 0x07, 0x28, 0x6F]
    assert host(res.row_global)[0] == np.float32(2.0 ** -8)


# ============================================================== supplied amax (single pass)
def compare_grouped_amax(orc, x_dev, sections, mask, flags, amax_in, seed=None, ro=None, co=None,
                         workspace=None, amax_out=True):
    """The call with supplied maxima (device tensors, or None) and measured maxima out,
    against the oracle given the same maxima."""
    dev = x_dev.device
    ain = None
    if amax_in is not None:
        ain = tuple(None if a is None else torch.tensor(np.asarray(a, np.float32), device=dev) for a in amax_in)
    call = mxq.GroupedNVFP4(x_dev, sections, mask, flags, seed, ro, co, amax_in=ain, amax_out=amax_out,
                            workspace=workspace)
    res = call()
    torch.cuda.synchronize()
    ref = orc.group_rht_quant_nvfp4(bits16(x_dev), sections, mask, flags, seed or 0, ro, co, threads=8,
                                    amax_in=amax_in)
    names = []
    if flags & 1:
        names += ["row_global", "row_scales", "row_codes"] + (["row_amax"] if amax_out else [])
    if flags & 2:
        names += ["col_global", "col_scales", "col_codes"] + (["col_amax"] if amax_out else [])
    if flags & 4:
        names += ["fp8_scales", "fp8_codes"]
    for n in names:
        assert_same(n, host(getattr(res, n)), getattr(ref, n))
    return res, ref


@pytest.mark.parametrize("flags", [3, 1, 2, 7])
def test_grouped_measured_amax_out(orc, flags):
    """The plain (two-pass) call reports the maxima its tensor scales used."""
    dev = device()
    announce(f"grouped amax out flags={flags}")
    w = synth.grouped_nvfp4(total_rows=1024, k=512, parts=4, seed=51)
    compare_grouped_amax(orc, w.tensors["x"].to(dev), w.params["split_sections"], w.params["sign_mask"],
                         flags, None)


@pytest.mark.parametrize("scale", [1.0, 0.25, 3.0])
def test_grouped_supplied_amax(orc, scale):
    """Single pass with supplied maxima: the measured ones (scale 1: the outputs of
    the plain call), smaller ones (saturation) and larger ones."""
    dev = device()
    announce(f"grouped supplied amax x{scale}")
    w = synth.grouped_nvfp4(total_rows=1280, k=640, parts=5, seed=52)
    x = w.tensors["x"].to(dev)
    sec, mask = w.params["split_sections"], w.params["sign_mask"]
    meas = orc.group_rht_quant_nvfp4(bits16(x), sec, mask, 3, threads=8)
    amax_in = (meas.row_amax * np.float32(scale), meas.col_amax * np.float32(scale))
    res, _ = compare_grouped_amax(orc, x, sec, mask, 3, amax_in)
    if scale == 1.0:
        plain = mxq.mxq_group_rht_quant_nvfp4(x, sec, mask, 3)
        torch.cuda.synchronize()
        for n in ("row_codes", "row_scales", "row_global", "col_codes", "col_scales", "col_global"):
            assert torch.equal(getattr(res, n), getattr(plain, n)), n


@pytest.mark.parametrize("flags,sr", [(3, False), (7, True), (2, False)])
def test_grouped_supplied_amax_no_out(orc, flags, sr):
    """Supplied maxima with no maxima out, with stochastic rounding and FP8 too
    (empty sections included: their scales come from their supplied maxima)."""
    dev = device()
    announce(f"grouped supplied amax, none out: flags={flags} sr={sr}")
    w = synth.grouped_nvfp4_sr(total_rows=2048, k=1024, parts=7, forced_empty=2, seed=58)
    x, p = w.tensors["x"].to(dev), w.params
    sec, mask = p["split_sections"], p["sign_mask"]
    rng = np.random.default_rng(59)
    amax_in = (rng.uniform(0.5, 8, 7).astype(np.float32), rng.uniform(0.5, 8, 7).astype(np.float32))
    if not flags & 1:
        amax_in = (None, amax_in[1])
    seed, ro, co = (p["seed"], p["row_offsets"], p["col_offsets"]) if sr else (None, None, None)
    compare_grouped_amax(orc, x, sec, mask, flags, amax_in, seed=seed, ro=ro, co=co, amax_out=False)


def test_grouped_large_section_scales_kernel(orc):
    """A section of 8320 x 4096 (1040 amax partials, a fold over several rounds of
    the scales kernel's loads) beside small and empty ones; the measured maxima out
    as well."""
    dev = device()
    announce("grouped: a large section (8320 rows x 4096) beside small ones")
    w = synth.grouped_nvfp4(total_rows=8576, k=4096, parts=1, seed=60)
    x = w.tensors["x"].to(dev)
    compare_grouped_amax(orc, x, [128, 8320, 0, 128], 0x6A95, 3, None)


def test_grouped_supplied_amax_sr_fp8_edges(orc):
    """Supplied maxima with stochastic rounding, the FP8 output, empty sections and
    NaN / -0 / subnormal edge values."""
    dev = device()
    announce("grouped supplied amax: SR + FP8 + edges")
    b = edge_matrix(512, 256, 53)
    b[100:116, 40] = 0x7FC0
    x = bf16_dev(b, dev)
    sec = [128, 0, 256, 128, 0]
    rng = np.random.default_rng(54)
    amax_in = (rng.uniform(0.5, 40, 5).astype(np.float32), rng.uniform(0.5, 40, 5).astype(np.float32))
    compare_grouped_amax(orc, x, sec, 0x3C5A, 7, amax_in, seed=99, ro=[1, 2, 3, 4, 5], co=[6, 7, 8, 9, 10])
    compare_grouped_amax(orc, x, sec, 0x3C5A, 3, amax_in)
    compare_grouped_amax(orc, x, sec, 0x3C5A, 2, (None, amax_in[1]))
    compare_grouped_amax(orc, x[:0], [0, 0], 0, 3, (np.ones(2, np.float32), np.ones(2, np.float32)))
