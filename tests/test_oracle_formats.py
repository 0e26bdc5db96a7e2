"""Pins of the oracle's format codecs against things other than the oracle itself:
the format definitions' landmark values, torch's float8_e4m3fn and bfloat16
conversions (library routines), the closed form of E2M1 nearest-even rounding,
and enumeration for stochastic rounding.

Formats: OCP E4M3FN ("FLOAT8E4M3FN" in the onnxruntime QMoE PR, Description),
E2M1 with E4M3 block scales (the NVFP4 format of the TransformerEngine NVFP4 PRs),
bfloat16 (the activations' dtype in all pages)."""
import numpy as np
import pytest
import torch
from tests.golden_util import num, rows


def f32(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


def bits(v):
    return np.asarray(v, dtype=np.float32).view(np.uint32)


# ---------------------------------------------------------------- constants
def test_constants_through_the_recipes(orc):
    # F(1e-10)*F(1/2688) is the tensor scale of an all-zero / empty section.
    assert bits(orc.nvfp4_global_scale(0.0)) == 0x29278B6D
    # An all-zero FP8 group: s = F(1e-10)*F(1/448) = 0x2A7B5124.
    q, s = orc.quant_fp8_1x128(np.zeros((1, 128), np.uint16))
    assert bits(s[0, 0]) == 0x2A7B5124 and not q.any()
    # amax 448 -> s = fl(448 * F(1/448)) = 1.0; amax 1 -> s = F(1/448) = 0x3B124925.
    row = np.zeros((1, 128), np.uint16)
    row[0, 0] = 0x43E0  # 448.0 in bfloat16
    _, s = orc.quant_fp8_1x128(row)
    assert bits(s[0, 0]) == 0x3F800000
    row[0, 0] = 0x3F80  # 1.0
    q, s = orc.quant_fp8_1x128(row)
    assert bits(s[0, 0]) == 0x3B124925
    assert q[0, 0] == 0x7E  # 1/s = 447.99997 -> 448


# ---------------------------------------------------------------- bfloat16
def test_bf16_matches_torch_rne(orc):
    rng = np.random.default_rng(0)
    raw = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # add every tie pattern with both significand parities and the overflow edge
    hi = rng.integers(0, 2**16, size=20_000, dtype=np.uint32) << 16
    ties = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001,
                           np.array([0x7F7F8000, 0x7F7FFFFF, 0xFF7F8000, 0x00008000, 0x80018000], np.uint32)])
    b = np.concatenate([raw, ties]).astype(np.uint32)
    v = b.view(np.float32)
    v = v[~np.isnan(v)]
    ours = orc.f32_to_bf16(v)
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_nan_stays_nan(orc):
    for b in (0x7FC00000, 0x7F800001, 0xFFFFFFFF, 0x7FFF0000):
        out = orc.f32_to_bf16(f32([b]))[0]
        assert (out & 0x7F80) == 0x7F80 and (out & 0x7F) != 0


# ---------------------------------------------------------------- E4M3
def test_e4m3_decode_landmarks(orc):
    assert orc.e4m3_value(0x01) == 2.0 ** -9
    assert orc.e4m3_value(0x08) == 2.0 ** -6
    assert orc.e4m3_value(0x38) == 1.0
    assert orc.e4m3_value(0x78) == 256.0
    assert orc.e4m3_value(0x7E) == 448.0
    assert np.isnan(orc.e4m3_value(0x7F)) and np.isnan(orc.e4m3_value(0xFF))
    vals = [orc.e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))
    assert all(orc.e4m3_value(0x80 | c) == -orc.e4m3_value(c) for c in range(0x7F))


def test_e4m3_decode_matches_torch(orc):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    ours = np.array([orc.e4m3_value(c) for c in range(256)], np.float32)
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.array_equal(ours[~both_nan], ref[~both_nan]) and both_nan.sum() == 2


def _e4m3_probe_values():
    rng = np.random.default_rng(1)
    # every bfloat16 value, random float32 over the useful exponent range,
    # and +-3 ulps around every midpoint between adjacent E4M3 magnitudes
    allbf = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    rnd = (rng.standard_normal(1_000_000) * np.exp2(rng.integers(-14, 9, 1_000_000))).astype(np.float32)
    mags = np.array([0.0] + [m * 2.0 ** -9 for m in range(1, 8)] +
                    [(1 + m / 8) * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8)][:119], np.float64)
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    near = (mids.view(np.uint32)[:, None].astype(np.int64) + np.arange(-3, 4)).astype(np.uint32).view(np.float32)
    v = np.concatenate([allbf, rnd, near.ravel(), -near.ravel()])
    return v[np.isfinite(v)]


def test_e4m3_encode_matches_torch_in_range(orc):
    v = _e4m3_probe_values()
    v = v[np.abs(v) < 464.0]          # torch turns larger magnitudes into NaN
    ours = orc.e4m3_encode(v)
    ref = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates_and_nan(orc):
    v = np.array([448.0, 464.0, 470.0, 1e6, np.inf, -500.0, -np.inf], np.float32)
    assert list(orc.e4m3_encode(v)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert list(orc.e4m3_encode(f32([0x7FC00000, 0xFFC00000, 0x7F800001]))) == [0x7F] * 3
    # sign of zero kept; a negative value that rounds to zero keeps its sign
    assert list(orc.e4m3_encode(np.array([0.0, -0.0, -1e-30, 2.0 ** -10], np.float32))) == [0, 0x80, 0x80, 0]


# ---------------------------------------------------------------- E2M1
def e2m1_closed_form(v):
    """Nearest-even E2M1 written as a sum of threshold tests: strict '>' where the
    tie goes down to an even code, '>=' where it goes up to one."""
    a = np.abs(v.astype(np.float64))
    c = ((a > 0.25).astype(int) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
         + (a > 2.5) + (a >= 3.5) + (a > 5.0))
    return (c | (np.signbit(v).astype(int) << 3)).astype(np.uint8)


def test_e2m1_values(orc):
    assert [orc.e2m1_value(c) for c in range(8)] == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert [orc.e2m1_value(8 | c) for c in range(1, 8)] == [-0.5, -1, -1.5, -2, -3, -4, -6]


def test_e2m1_encode_matches_closed_form(orc):
    rng = np.random.default_rng(2)
    allbf = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    thr = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1, 1.5, 2, 3, 4], np.float32)
    near = (thr.view(np.uint32)[:, None].astype(np.int64) + np.arange(-4, 5)).astype(np.uint32).view(np.float32)
    rnd = (rng.standard_normal(2_000_000) * 3).astype(np.float32)
    v = np.concatenate([allbf, near.ravel(), -near.ravel(), rnd])
    v = v[~np.isnan(v)]
    assert np.array_equal(orc.e2m1_encode(v), e2m1_closed_form(v))


def test_e2m1_hand_cases(orc):
    # ties go to the even code; saturation at 6; sign of zero kept
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.25, -0.0, -0.25, 100.0], np.float32)
    assert list(orc.e2m1_encode(v)) == [0, 2, 2, 4, 4, 6, 6, 7, 8, 8, 7]


# ---------------------------------------------------------------- stochastic rounding
@pytest.mark.parametrize("x,F,lo,hi", [(num(a), int(b), int(c), int(d)) for a, b, c, d in rows("e2m1_sr_counts.txt")])
def test_sr_enumeration(orc, x, F, lo, hi):
    """Over all 256 random bytes the value rounds up exactly F times, F = floor(256 f)."""
    r = np.arange(256, dtype=np.uint8)
    codes = orc.e2m1_encode_sr(np.full(256, x, np.float32), r)
    assert set(codes.tolist()) <= {lo, hi}
    assert int((codes == hi).sum()) == (F if hi != lo else 256)
    assert all(codes[i] == hi for i in range(256 - F, 256)) or hi == lo
    neg = orc.e2m1_encode_sr(np.full(256, -x, np.float32), r)
    assert np.array_equal(neg, codes | 8)


def test_sr_grid_values_never_move(orc):
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, 6.25, 100], np.float32)
    r = np.arange(256, dtype=np.uint8)
    for g in grid:
        codes = orc.e2m1_encode_sr(np.full(256, g, np.float32), r)
        assert len(set(codes.tolist())) == 1
        assert codes[0] == orc.e2m1_encode(np.array([g], np.float32))[0]


def test_sr_is_unbiased_on_average(orc):
    """E[value] equals x exactly when every random byte is equally likely and
    256 f is an integer (x on a 1/256-spacing sub-grid)."""
    rng = np.random.default_rng(3)
    r = np.arange(256, dtype=np.uint8)
    for _ in range(300):
        j = int(rng.integers(0, 256)) / 256.0
        base, step = [(0.0, 0.5), (0.5, 0.5), (1.0, 0.5), (1.5, 0.5),
                      (2.0, 1.0), (3.0, 1.0), (4.0, 2.0)][int(rng.integers(0, 7))]
        x = np.float32(base + step * j)
        codes = orc.e2m1_encode_sr(np.full(256, x, np.float32), r)
        mean = np.mean([orc.e2m1_value(c) for c in codes])
        assert mean == pytest.approx(float(x), abs=1e-12)
