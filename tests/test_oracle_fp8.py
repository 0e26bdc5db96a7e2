"""Pins of the oracle's FP8 1x128 quantizer and the DSA rotate+quant composition.

Recipe (onnxruntime PR #33644, Description): consecutive K128 groups, scale
max(amax, 1e-10) * float32(1/448), normalization by FP32 division, saturating
nearest-even E4M3FN.  The page notes that the arithmetic choices matter at FP8
midpoints; the brute-force test below regenerates such cases.

DSA (TensorRT-LLM PR #15158, Summary): torch.cat([qk_pe, qk_nope]) ->
rotate_activation -> fp8_quantize_1x128."""
import numpy as np
import pytest
import torch
from tests.golden_util import num, rows


def bf16(v):
    return torch.tensor(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_of_bf16(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


def torch_reference(x_bf16):
    """The recipe re-expressed with torch library routines: float32 max/multiply/
    divide and torch's float8_e4m3fn conversion (after the saturating clamp)."""
    x = torch.from_numpy(x_bf16.view(np.int16).copy()).view(torch.bfloat16).float()
    m, k = x.shape
    g = x.view(m, k // 128, 128)
    a = torch.nan_to_num(g.abs(), nan=0.0).amax(dim=2, keepdim=True)
    s = torch.clamp(a, min=torch.tensor(1e-10, dtype=torch.float32)) * (torch.tensor(1.0) / torch.tensor(448.0))
    q = (g / s).clamp(-448.0, 448.0)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).view(m, k).numpy()
    return codes, s.view(m, k // 128).numpy()


def test_b1_unit_scale(orc):
    fix = rows("fp8_unit_scale.txt")
    vals = [num(r[0]) for r in fix]
    row = np.zeros((1, 128), np.float32)
    row[0, :len(vals)] = vals
    q, s = orc.quant_fp8_1x128(bf16(row))
    assert s[0, 0] == 1.0
    assert q[0, :len(vals)].tolist() == [num(r[1]) for r in fix]


def test_b2_b3(orc):
    row = np.zeros((1, 128), np.uint16)
    row[0, 7] = 0x3F80
    q, s = orc.quant_fp8_1x128(row)
    assert s.view(np.uint32)[0, 0] == 0x3B124925 and q[0, 7] == 0x7E
    q, s = orc.quant_fp8_1x128(np.zeros((2, 256), np.uint16))
    assert (s.view(np.uint32) == 0x2A7B5124).all() and not q.any()


def test_matches_library_reexpression(orc):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 1024)).astype(np.float32) * np.exp2(rng.integers(-6, 7, (64, 1)))
    x[3, 5] = np.nan
    x[4, :128] = 0
    xb = bf16(x)
    q, s = orc.quant_fp8_1x128(xb)
    rq, rs = torch_reference(xb)
    assert np.array_equal(s, rs)
    nan_mask = np.isnan(f32_of_bf16(xb))
    assert np.array_equal(q[~nan_mask], rq[~nan_mask])
    assert (q[nan_mask] == 0x7F).all()        # a NaN element stays NaN (0x7F)


def test_every_live_group_hits_448(orc):
    """The amax element of a group maps to |x/s| in 448 (1 +- 2^-23), code 0x7E."""
    rng = np.random.default_rng(12)
    x = bf16(rng.standard_normal((256, 1024)) * np.exp2(rng.integers(-20, 20, (256, 1))))
    q, _ = orc.quant_fp8_1x128(x)
    g = (q.reshape(256, 8, 128) & 0x7F)
    assert (g.max(axis=2) == 0x7E).all()


def test_dequant_error_bound(orc):
    rng = np.random.default_rng(13)
    xb = bf16(rng.standard_normal((128, 512)))
    q, s = orc.quant_fp8_1x128(xb)
    x = f32_of_bf16(xb).astype(np.float64).reshape(128, 4, 128)
    vals = torch.from_numpy(q).view(torch.float8_e4m3fn).float().numpy().astype(np.float64).reshape(128, 4, 128)
    deq = vals * s[:, :, None]
    y = x / s[:, :, None]
    # E4M3 relative spacing 2^-3 in the normal range, absolute 2^-9 below 2^-6
    half = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * 1.0001
    assert np.all(np.abs(deq / s[:, :, None] - y) <= half)


def test_transposed_scale_layout(orc):
    rng = np.random.default_rng(14)
    xb = bf16(rng.standard_normal((64, 512)))
    q1, s1 = orc.quant_fp8_1x128(xb)
    q2, s2 = orc.quant_fp8_1x128(xb, scale_transposed=True)
    assert np.array_equal(q1, q2) and np.array_equal(s1.T, s2)


def test_division_mode_midpoints(orc):
    """Brute force over BF16 (amax, x) pairs for quotients x/s that lie within one
    FP32 ulp of an E4M3 rounding midpoint.  The oracle must use the correctly
    rounded FP32 quotient (numpy float32 division), and the search must find pairs
    where an approximate quotient x * (1/s) lands on the other side."""
    bf = np.arange(0x3F80, 0x4400, dtype=np.uint32)           # 1.0 .. 128: group amax values
    amax = f32_of_bf16(bf)
    s = np.maximum(amax, np.float32(1e-10)) * (np.float32(1.0) / np.float32(448.0))
    xs = f32_of_bf16(np.arange(0x3A00, 0x4400, dtype=np.uint32))   # candidate elements
    found = 0
    rng = np.random.default_rng(15)
    for i in rng.choice(len(bf), 200, replace=False):
        q_exact = xs / s[i]                                   # correctly rounded float32
        q_recip = xs * (np.float32(1.0) / s[i])
        c1 = torch.from_numpy(q_exact).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        c2 = torch.from_numpy(q_recip).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        diff = np.nonzero(c1 != c2)[0]
        for j in diff[:3]:
            row = np.zeros((1, 128), np.uint16)
            row[0, 0] = bf[i]
            row[0, 1] = bf16([xs[j]])[0]
            q, sc = orc.quant_fp8_1x128(row)
            assert sc[0, 0] == s[i]
            assert q[0, 1] == c1[j] and q[0, 1] != c2[j]
            found += 1
    assert found > 0


def test_b8_dsa_hand_case(orc):
    fix = rows("dsa_wht128_fp8.txt")
    v = np.arange(1, 129, dtype=np.float32)
    pe, nope = bf16(v[None, :64]), bf16(v[None, 64:])
    q, s = orc.hadamard_quant_fp8(pe, nope)
    assert s.view(np.uint32)[0] == num(fix[0][1])
    expect = np.zeros(128, np.uint8)
    for r in fix[1:]:
        expect[int(r[1])] = num(r[2])
    assert q[0].tolist() == expect.tolist()


def test_dsa_equals_unfused_composition(orc):
    """cat -> rotate -> quantize as three separate oracle steps equals the fused
    oracle entry (the PR's fused path must equal the unfused one byte for byte)."""
    rng = np.random.default_rng(16)
    pe = bf16(rng.standard_normal((300, 64)) * 3)
    nope = bf16(rng.standard_normal((300, 64)))
    q, s = orc.hadamard_quant_fp8(pe, nope)
    cat = np.concatenate([pe, nope], axis=1)
    rot = orc.f32_to_bf16(orc.wht(f32_of_bf16(cat)))
    q2, s2 = orc.quant_fp8_1x128(rot)
    assert np.array_equal(q, q2) and np.array_equal(s, s2[:, 0])
    # swapping the halves changes the result (the concat order is observable)
    q3, _ = orc.hadamard_quant_fp8(nope, pe)
    assert not np.array_equal(q, q3)


@pytest.mark.parametrize("d_pe", [0, 8, 64, 120, 128])
def test_dsa_split_points(orc, d_pe):
    rng = np.random.default_rng(17 + d_pe)
    full = bf16(rng.standard_normal((50, 128)))
    q, s = orc.hadamard_quant_fp8(full[:, :d_pe], full[:, d_pe:])
    q0, s0 = orc.hadamard_quant_fp8(full[:, :64], full[:, 64:])
    assert np.array_equal(q, q0) and np.array_equal(s, s0)
