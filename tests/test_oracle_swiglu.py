"""Pins of the oracle's SwiGLU -> FP8 1x128 quantizer.

onnxruntime PR #33644 (Description): the second dynamic quantizer runs on consecutive
K128 groups directly after the FP32 SiLU/SwiGLU, with no extra round to the input type
in between, and uses the same FP8 recipe as the first (max(amax, 1e-10) * F(1/448),
saturating nearest-even E4M3, FP32 division).  The pages do not fix how e^x is
evaluated; the oracle's EXP is a stated algorithm (Cody-Waite reduction, Taylor
polynomial), pinned here against the mathematical function."""
import numpy as np
import pytest
import torch

BF = torch.bfloat16


def bf16_bits(v):
    return torch.tensor(np.asarray(v, np.float32)).to(BF).view(torch.int16).numpy().view(np.uint16)


def f32_of_bf16(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


def ulp_err(got, ref64):
    ref32 = ref64.astype(np.float32)
    ulp = np.spacing(np.abs(ref32)).astype(np.float64)
    return np.abs(got.astype(np.float64) - ref64) / ulp


def test_exp_within_one_ulp(orc):
    """EXP is faithful (error below one ulp) over its whole finite, normal range."""
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-87.0, 88.7, 1_000_000), rng.uniform(-1, 1, 200_000),
                        rng.uniform(-1e-3, 1e-3, 100_000)]).astype(np.float32)
    err = ulp_err(orc.exp(x), np.exp(x.astype(np.float64)))
    assert err.max() < 1.0, err.max()


def test_exp_special_values(orc):
    """EXP(0) = 1 exactly, overflow to +inf above ln(FLT_MAX), subnormal and zero
    results below, NaN kept; monotone over a sorted sample."""
    e = orc.exp(np.float32([0.0, -0.0, 88.8, 100.0, 1e30, -104.0, -1e30, np.nan]))
    assert e[0] == 1.0 and e[1] == 1.0
    assert np.isinf(e[2:5]).all() and (e[2:5] > 0).all()
    assert e[5] == 0.0 and e[6] == 0.0 and np.isnan(e[7])
    sub = orc.exp(np.float32([-100.0]))[0]
    assert 0 < sub < np.finfo(np.float32).tiny and abs(float(sub) - np.exp(-100.0)) <= 2 ** -149
    x = np.sort(np.random.default_rng(6).uniform(-20, 20, 200_000).astype(np.float32))
    assert (np.diff(orc.exp(x)) >= 0).all()


def test_silu_against_its_definition(orc):
    """SILU(g) = g / (1 + e^-g): within 3 ulps of the float64 value; SILU(0) = 0; for
    g >= 17, 1 + e^-g rounds to 1 and SILU(g) = g exactly; negative g gives negative
    values (or -0 when e^-g overflows)."""
    rng = np.random.default_rng(7)
    g = np.concatenate([rng.standard_normal(500_000) * 6, rng.uniform(-80, 80, 100_000)]).astype(np.float32)
    s = orc.silu(g)
    g64 = g.astype(np.float64)
    ref = g64 / (1.0 + np.exp(-g64))
    big = np.abs(ref) > 1e-30
    assert ulp_err(s[big], ref[big]).max() < 3.0
    assert orc.silu(np.float32([0.0]))[0] == 0.0
    gg = np.float32([17.0, 20.0, 100.0, 3e38])
    np.testing.assert_array_equal(orc.silu(gg), gg)
    neg = orc.silu(np.float32([-1.0, -10.0, -50.0, -90.0, -200.0]))
    assert (np.signbit(neg)).all()
    assert neg[-1] == 0.0


def test_swiglu_quant_is_fp8_of_the_fp32_product(orc):
    """Codes and scales equal the FP8 1x128 group encode of h = fl(SILU(gate) * up)
    in FP32 (no BF16 round of h), in both scale layouts."""
    rng = np.random.default_rng(8)
    m, n = 24, 384
    g = bf16_bits(rng.standard_normal((m, n)) * 3)
    u = bf16_bits(rng.standard_normal((m, n)) * np.exp2(rng.integers(-8, 8, (m, 1))))
    q, s = orc.swiglu_quant_fp8(g, u)
    qt, st = orc.swiglu_quant_fp8(g, u, scale_transposed=True)
    np.testing.assert_array_equal(q, qt)
    np.testing.assert_array_equal(s, st.T)
    h = (orc.silu(f32_of_bf16(g)) * f32_of_bf16(u)).astype(np.float32)
    assert not np.array_equal(h, f32_of_bf16(bf16_bits(h)))      # h carries more than BF16
    for r in range(m):
        for j in range(n // 128):
            sc, codes = orc.fp8_group(h[r, 128 * j:128 * (j + 1)])
            assert s[r, j] == sc
            np.testing.assert_array_equal(q[r, 128 * j:128 * (j + 1)], codes)


def test_swiglu_quant_hand_rows(orc):
    """A zero gate gives h = 0: the floor scale F(1e-10) * F(1/448) and zero codes.  A
    gate of 32 gives h = 32 * up exactly, so the row is the FP8 encode of 32 * up: its
    amax group maps to 448 (code 0x7E)."""
    n = 128
    g = np.zeros((2, n), np.uint16)
    g[1, :] = bf16_bits(np.full(n, 32.0))
    up = bf16_bits(np.linspace(-3.0, 5.0, 2 * n).reshape(2, n))
    q, s = orc.swiglu_quant_fp8(g, up)
    assert s[0, 0] == np.float32(1e-10) * np.float32(1.0 / 448.0)
    assert not (q[0] & 0x7F).any()
    amax = np.float32(32.0) * np.abs(f32_of_bf16(up[1])).max()
    assert s[1, 0] == amax * np.float32(1.0 / 448.0)
    assert q[1, np.argmax(np.abs(f32_of_bf16(up[1])))] & 0x7F == 0x7E


def test_swiglu_overflow_to_inf(orc):
    """A product that overflows FP32 (SILU(10) * 3e38) is +inf: its group's scale is
    infinite, the finite values encode as +-0 and the infinite one as NaN (0x7F)."""
    n = 128
    g = np.ones((2, n), np.float32)
    u = np.ones((2, n), np.float32)
    u[0, 1::2] = -1.0
    g[0, 5], u[0, 5] = 10.0, 3.0e38
    q, s = orc.swiglu_quant_fp8(bf16_bits(g), bf16_bits(u))
    assert np.isinf(s[0, 0]) and np.isfinite(s[1, 0])
    want = np.where(u[0] < 0, 0x80, 0x00).astype(np.uint8)
    want[5] = 0x7F
    np.testing.assert_array_equal(q[0], want)
