"""Pins of the oracle's DSA rotate + NVFP4 quantizer (the FP4 counterpart of the
rotate + FP8 1x128 path).

TensorRT-LLM PR #15158 (Summary): the DSA indexer concatenates qk_pe and qk_nope and
must rotate the result with the orthonormal Hadamard transform before quantizing; the
FP4 path lacks the rotation and needs a standalone FP4 quantize-only kernel.  The
pages fix no FP4 scale recipe for it; the reading pinned here is the row-wise NVFP4
encode of the grouped path (1x16 blocks, E4M3 block scales) with one FP32 tensor
scale over the whole rotated tensor, measured or supplied by the caller."""
import numpy as np
import pytest
import scipy.linalg
import torch

from nvfp4_quantization_amd import synth

C128 = np.float32(1.0 / np.sqrt(128.0))
E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


def bf16_bits(v):
    return torch.tensor(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_of_bf16(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


def unpack(codes_bytes):
    b = np.asarray(codes_bytes, np.uint8)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def e4m3(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(torch.float8_e4m3fn).float().numpy()


def split(v_bits, d_pe):
    return v_bits[:, :d_pe].copy(), v_bits[:, d_pe:].copy()


@pytest.mark.parametrize("d_pe", [0, 64, 120, 128])
def test_one_hot_rows_follow_hadamard_rows(orc, d_pe):
    """Row r holds s at position j_r of cat(pe, nope) and zeros elsewhere, so its
    rotation is s C128 times row j_r of the Sylvester matrix: every |y| is the tensor
    amax, every block gets the top scale 0x7E and every code is +-6, with the sign of
    H[j_r][i] (scipy's Hadamard matrix)."""
    m = 136
    js = (np.arange(m) * 37 + 5) % 128
    s = np.float32(-3.25)
    v = np.zeros((m, 128), np.float32)
    v[np.arange(m), js] = s
    pe, nope = split(bf16_bits(v), d_pe)
    out = orc.hadamard_quant_nvfp4(pe, nope)
    A = f32_of_bf16(bf16_bits(np.float32(abs(s) * C128)))
    assert out.amax == A
    assert out.global_scale == orc.nvfp4_global_scale(A)
    assert (out.scales == 0x7E).all()
    H = scipy.linalg.hadamard(128)
    neg = (H[js] * np.sign(s)) < 0
    want = np.where(neg, 0xF, 0x7).astype(np.uint8)
    np.testing.assert_array_equal(unpack(out.codes), want)


def test_codes_are_nearest_grid_points(orc):
    """For seeded DSA-shaped input with outlier channels: every block scale is the
    E4M3 value nearest fl(fl(a/6)/g) (torch's float8_e4m3fn as the reference), and
    every code is an E2M1 value nearest fl(y/d), ties to the even code, with y the
    BF16 rotated value and d = e4m3(sc) * g."""
    w = synth.dsa_rotate_fp8(tokens=64, heads=8, seed=11)
    pe = w.tensors["pe"].view(torch.int16).numpy().view(np.uint16)
    nope = w.tensors["nope"].view(torch.int16).numpy().view(np.uint16)
    m = pe.shape[0]
    out = orc.hadamard_quant_nvfp4(pe, nope)
    v = f32_of_bf16(np.concatenate([pe, nope], axis=1))
    y = np.stack([orc.wht(v[r], 0, C128) for r in range(m)]).astype(np.float32)
    assert out.amax == np.abs(y).max()
    g = out.global_scale
    a = np.abs(y).reshape(m, 8, 16).max(axis=2).astype(np.float32)
    t = (a * np.float32(1.0 / 6.0)).astype(np.float32) / g
    want_sc = torch.from_numpy(t.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(out.scales, want_sc)
    d = (e4m3(out.scales) * g).astype(np.float32)
    q = (y.reshape(m, 8, 16) / d[:, :, None]).astype(np.float32).astype(np.float64)
    codes = unpack(out.codes).reshape(m, 8, 16)
    mag = E2M1[codes & 7]
    dist = np.abs(np.abs(q)[..., None] - E2M1[None, None, None, :])
    best = dist.min(axis=-1)
    assert (np.abs(np.abs(q) - mag) == best).all()
    tie = (dist == best[..., None]).sum(axis=-1) > 1
    assert ((codes[tie] & 1) == 0).all()                  # ties go to the even code
    nz = (codes & 7) != 0
    assert (np.signbit(q[nz]) == (codes[nz] >> 3).astype(bool)).all()


def test_equals_grouped_rowwise_of_the_rotation(orc):
    """The DSA FP4 call is the grouped row-wise NVFP4 encode (one section) of the
    BF16 rotated rows."""
    w = synth.dsa_rotate_fp8(tokens=32, heads=8, seed=12)
    pe = w.tensors["pe"].view(torch.int16).numpy().view(np.uint16)
    nope = w.tensors["nope"].view(torch.int16).numpy().view(np.uint16)
    m = pe.shape[0]
    out = orc.hadamard_quant_nvfp4(pe, nope)
    v = f32_of_bf16(np.concatenate([pe, nope], axis=1))
    y = np.stack([orc.wht(v[r], 0, C128) for r in range(m)]).astype(np.float32)
    ref = orc.group_rht_quant_nvfp4(bf16_bits(y), [m], 0, orc.ROWWISE)
    np.testing.assert_array_equal(out.codes.ravel(), np.asarray(ref.row_codes).ravel())
    np.testing.assert_array_equal(out.scales.ravel(), np.asarray(ref.row_scales).ravel())
    assert out.global_scale == ref.row_global[0]


def test_supplied_amax(orc):
    """The measured A supplied back reproduces the plain call; a smaller A saturates
    (scales at most 0x7E, the largest blocks at 0x7E with codes +-6 at their maxima);
    the measured A comes out either way."""
    w = synth.dsa_rotate_fp8(tokens=16, heads=8, seed=13)
    pe = w.tensors["pe"].view(torch.int16).numpy().view(np.uint16)
    nope = w.tensors["nope"].view(torch.int16).numpy().view(np.uint16)
    plain = orc.hadamard_quant_nvfp4(pe, nope)
    again = orc.hadamard_quant_nvfp4(pe, nope, amax_in=plain.amax)
    np.testing.assert_array_equal(again.codes, plain.codes)
    np.testing.assert_array_equal(again.scales, plain.scales)
    assert again.global_scale == plain.global_scale
    small = orc.hadamard_quant_nvfp4(pe, nope, amax_in=plain.amax / 8)
    assert small.amax == plain.amax
    assert small.global_scale == orc.nvfp4_global_scale(plain.amax / 8)
    assert (small.scales <= 0x7E).all() and (small.scales == 0x7E).sum() > (plain.scales == 0x7E).sum()


def test_nan_row(orc):
    """A NaN reaches all 128 rotated values of its row: that row's eight blocks get
    scale 0x7F and zero codes, and the tensor amax ignores it."""
    w = synth.dsa_rotate_fp8(tokens=8, heads=4, seed=14)
    pe = w.tensors["pe"].view(torch.int16).numpy().view(np.uint16).copy()
    nope = w.tensors["nope"].view(torch.int16).numpy().view(np.uint16).copy()
    clean = orc.hadamard_quant_nvfp4(pe, nope)
    nope[5, 3] = 0x7FC1
    out = orc.hadamard_quant_nvfp4(pe, nope)
    assert (out.scales[5] == 0x7F).all() and not out.codes[5].any()
    keep = np.arange(pe.shape[0]) != 5
    assert out.amax <= clean.amax
    v = f32_of_bf16(np.concatenate([pe, nope], axis=1))
    want = max(np.abs(orc.wht(v[r], 0, C128)).max() for r in range(pe.shape[0]) if r != 5)
    assert out.amax == want
    if out.amax == clean.amax:
        np.testing.assert_array_equal(out.codes[keep], clean.codes[keep])


def test_zero_and_empty(orc):
    """All-zero input: the floor tensor scale and zero scales and codes; no rows: the
    floor tensor scale."""
    z = np.zeros((4, 64), np.uint16)
    out = orc.hadamard_quant_nvfp4(z, z)
    assert out.amax == 0 and out.global_scale.view(np.uint32) == 0x29278B6D
    assert not out.scales.any() and not out.codes.any()
    e = orc.hadamard_quant_nvfp4(np.zeros((0, 64), np.uint16), np.zeros((0, 64), np.uint16))
    assert e.global_scale.view(np.uint32) == 0x29278B6D and e.codes.shape == (0, 64)
