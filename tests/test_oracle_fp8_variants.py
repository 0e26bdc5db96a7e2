"""Pins of the oracle's FP8 block variants: UE8M0 (power-of-two) scales, 128x1
column-wise blocks on the transpose, and the (token, head) scale layout of the DSA
rotate + FP8 output.

TensorRT-LLM PR #15158 (review: a use_ue8m0 option of fp8_quantize_1x128_sf_transpose;
the 1-D scale tensor padded, reshaped and transposed for its consumer).  The FP8
recipe itself is onnxruntime PR #33644's (Description).  Reading of UE8M0: the FP32
scale of the recipe rounded up to the nearest power of two."""
import numpy as np
import pytest
import torch


def bf16_bits(v):
    return torch.tensor(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_of_bf16(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


def e4m3_codes(v):
    """torch's float32 -> float8_e4m3fn conversion (nearest-even) as bytes."""
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def matrix(m, k, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32) * np.exp2(rng.integers(-12, 12, (m, 1)))
    return bf16_bits(x)


def test_pow2_ceil(orc):
    """Powers of two map to themselves; anything else to the next power up."""
    for e in (-126, -40, -1, 0, 1, 20, 120):
        p = np.float32(2.0) ** e
        assert orc.lib().oracle_pow2_ceil(float(p)) == p
        assert orc.lib().oracle_pow2_ceil(float(np.nextafter(p, np.float32(np.inf)))) == p * 2
        assert orc.lib().oracle_pow2_ceil(float(p * np.float32(1.75))) == p * 2


def test_ue8m0_rowwise(orc):
    """With UE8M0 each row-wise scale is a power of two s' with s <= s' < 2s (s the
    plain recipe's scale, pinned elsewhere), and the codes are torch's E4M3 of x / s'
    (exact: s' is a power of two), none of them saturated."""
    x = matrix(48, 512, 21)
    _, s, _, _ = orc.quant_fp8_blockwise(x, 0, columnwise=False)
    q2, s2, _, _ = orc.quant_fp8_blockwise(x, orc.FP8_UE8M0, columnwise=False)
    mant = s2.view(np.uint32) & 0x7FFFFF
    assert not mant.any()
    assert (s <= s2).all() and (s2 < 2 * s).all()
    xf = f32_of_bf16(x).reshape(48, 4, 128)
    want = e4m3_codes((xf / s2[:, :, None]).astype(np.float32)).reshape(48, 512)
    np.testing.assert_array_equal(q2, want)
    assert not ((q2 & 0x7F) == 0x7E).all()


def test_columnwise_is_rowwise_of_the_transpose(orc):
    """For m a multiple of 128, the column-wise codes and scales are the row-wise ones
    of x^T (the row-wise path is pinned on its own), with and without UE8M0."""
    m, k = 256, 384
    x = matrix(m, k, 22)
    xt = np.ascontiguousarray(x.T)
    for opt in (0, orc.FP8_UE8M0):
        _, _, cq, cs = orc.quant_fp8_blockwise(x, opt, rowwise=False)
        tq, ts, _, _ = orc.quant_fp8_blockwise(xt, opt, columnwise=False)
        np.testing.assert_array_equal(cq, tq)
        np.testing.assert_array_equal(cs, ts)


def test_columnwise_ragged_last_block(orc):
    """m = 300: column blocks of 128, 128 and 44 rows; the last block's scale comes
    from its 44 rows only and its codes are torch's E4M3 of fl(x / s)."""
    m, k = 300, 128
    x = matrix(m, k, 23)
    _, _, cq, cs = orc.quant_fp8_blockwise(x, 0, rowwise=False)
    assert cq.shape == (k, m) and cs.shape == (k, 3)
    xf = f32_of_bf16(x)
    last = xf[256:, :]
    a = np.abs(last).max(axis=0).astype(np.float32)
    s = (np.maximum(a, np.float32(1e-10)) * np.float32(1.0 / 448.0)).astype(np.float32)
    np.testing.assert_array_equal(cs[:, 2], s)
    want = e4m3_codes((last / s[None, :]).astype(np.float32)).T
    np.testing.assert_array_equal(cq[:, 256:], want)


def test_dsa_scale_layout(orc):
    """The (token, head) scale layout: the default [tokens][heads] equals the plain DSA
    call's scales; the transposed, padded [heads][tokens_pad] layout holds the same
    values at their transposed places and leaves the padding untouched; UE8M0 scales
    are powers of two >= the plain ones."""
    tokens, heads = 20, 6
    rng = np.random.default_rng(24)
    v = bf16_bits(rng.standard_normal((tokens * heads, 128)) * 2)
    pe, nope = v[:, :64].copy(), v[:, 64:].copy()
    q0, s0 = orc.hadamard_quant_fp8(pe, nope)
    q1, s1 = orc.hadamard_quant_fp8_ex(pe, nope, 0, heads)
    np.testing.assert_array_equal(q0, q1)
    np.testing.assert_array_equal(s0, s1)
    pad = 32
    q2, s2 = orc.hadamard_quant_fp8_ex(pe, nope, 0, heads, token_stride=1, head_stride=pad, scale_size=heads * pad)
    s2 = s2.reshape(heads, pad)
    np.testing.assert_array_equal(s2[:, :tokens], s0.reshape(tokens, heads).T)
    assert np.isnan(s2[:, tokens:]).all()
    q3, s3 = orc.hadamard_quant_fp8_ex(pe, nope, orc.FP8_UE8M0, heads)
    assert not (s3.view(np.uint32) & 0x7FFFFF).any() and (s3 >= s0).all() and (s3 < 2 * s0).all()


def test_infinite_group(orc):
    """IEEE arithmetic as written: an infinite element makes its group's amax and
    scale infinite (UE8M0 keeps infinity); the finite elements then encode x / inf
    = +-0 (codes 0x00 / 0x80, signed zeros kept) and the infinite one inf / inf =
    NaN (0x7F).  Groups without an infinity are untouched."""
    x = np.tile(np.linspace(-3, 3, 128).astype(np.float32), (2, 1))
    x[0, 17] = np.inf
    xb = bf16_bits(x)
    for opt in (0, orc.FP8_UE8M0):
        q, s, _, _ = orc.quant_fp8_blockwise(xb, opt, columnwise=False)
        assert np.isinf(s[0, 0]) and np.isfinite(s[1, 0])
        want = np.where(np.signbit(x[0]), 0x80, 0x00).astype(np.uint8)
        want[17] = 0x7F
        np.testing.assert_array_equal(q[0], want)
        q1, s1, _, _ = orc.quant_fp8_blockwise(xb[1:], opt, columnwise=False)
        np.testing.assert_array_equal(q[1], q1[0])


def test_dsa_infinite_row(orc):
    """One infinity in a DSA row reaches all 128 rotated values as +-inf (the
    Hadamard matrix has no zero entry): the row's group scale is infinite and every
    code is inf / inf = NaN (0x7F); the other rows match the call without that row."""
    tokens, heads = 4, 2
    rng = np.random.default_rng(25)
    v = bf16_bits(rng.standard_normal((tokens * heads, 128)))
    v[3, 70] = 0x7F80
    pe, nope = v[:, :64].copy(), v[:, 64:].copy()
    q, s = orc.hadamard_quant_fp8(pe, nope)
    assert np.isinf(s[3]) and (q[3] == 0x7F).all()
    keep = np.arange(tokens * heads) != 3
    q2, s2 = orc.hadamard_quant_fp8(pe[keep], nope[keep])
    np.testing.assert_array_equal(q[keep], q2)
    np.testing.assert_array_equal(s[keep], s2)
