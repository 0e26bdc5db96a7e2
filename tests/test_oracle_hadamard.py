"""Pins of the oracle's Walsh-Hadamard transforms.

The 16-point RHT (TransformerEngine PR #2555 review, quantizer.cpp comments:
a 16x16 RHT matrix per quantizer, applied to the column-wise operand) and the
normalized 128-point rotation over cat[qk_pe, qk_nope] (TensorRT-LLM PR #15158,
Summary; the orthonormality argument (Hq).(Hk) = q.k in the discussion).

Pins: scipy's Sylvester Hadamard matrix (library) on inputs whose sums are exact,
H.H^T = n.I, norm and inner-product preservation within BF16 rounding, and hand
cases whose values follow from the definition."""
import numpy as np
import pytest
import scipy.linalg
import torch
from tests.golden_util import num, rows

C128_BITS = 0x3DB504F3


def bf16_bits_to_f32(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


def f32_bits(v):
    return np.asarray(v, np.float32).view(np.uint32)


def signs(mask, n):
    return np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(n)])


@pytest.mark.parametrize("n,mask", [(16, 0), (16, 0x8001), (16, 0xFFFF), (16, 0x9216), (128, 0)])
def test_wht_equals_sylvester_matrix_on_exact_inputs(orc, n, mask):
    """Small-integer inputs keep every partial sum exact, so the butterfly equals
    H @ D @ x computed by scipy in float64 (c = 1)."""
    rng = np.random.default_rng(n + mask)
    H = scipy.linalg.hadamard(n).astype(np.float64)
    lim = 15 if n == 16 else 2          # |sum| <= 240 resp. 256: exact in bfloat16
    x = rng.integers(-lim, lim + 1, size=(500, n)).astype(np.float32)
    ours = orc.wht(x, sign_mask=mask, c=1.0)
    ref = (H @ (signs(mask, n)[:, None] * x.T.astype(np.float64))).T
    assert np.array_equal(ours.astype(np.float64), ref)


@pytest.mark.parametrize("n", [16, 128])
def test_wht_matrix_is_orthogonal(orc, n):
    """Transforming the unit vectors gives the columns of H D: (HD)(HD)^T = n I."""
    mask = 0xA5C3 if n == 16 else 0
    cols = orc.wht(np.eye(n, dtype=np.float32), sign_mask=mask, c=1.0)  # row i = H D e_i
    M = cols.T.astype(np.float64)
    assert np.array_equal(M @ M.T, n * np.eye(n))
    assert set(np.unique(M)) == {-1.0, 1.0}


def test_c128_constant(orc):
    """The 128-point normalization is F(1/sqrt(128)): 64 ones through the
    transform give 64 * C128 = 5.65685 -> bfloat16 5.65625 (0x40B5)."""
    v = np.zeros(128, np.float32)
    v[:64] = 1
    y = orc.wht(v[None])[0]
    assert f32_bits(y[0]) >> 16 == 0x40B5 and f32_bits(y[0]) & 0xFFFF == 0
    assert f32_bits(np.float32(np.sqrt(np.float32(2.0))) / np.float32(16.0)) == C128_BITS


def test_b4_hand_cases(orc):
    x = np.arange(1, 17, dtype=np.float32)
    for r in rows("wht16_integers.txt"):
        y = orc.wht(x[None], sign_mask=num(r[0]), c=0.25)[0]
        assert y.tolist() == [num(t) for t in r[1:]]


def test_b5_constant_block(orc):
    """A constant block c transforms to (4c, 0, ..., 0) (here 4c is a BF16 value)."""
    for c in [1.0, -3.5, 0.125, 2.0 ** -100, 96.0]:
        y = orc.wht(np.full((1, 16), c, np.float32), c=0.25)[0]
        assert y[0] == np.float32(4 * c) and not y[1:].any()


def test_b6_stage_order_is_observable(orc):
    """Ascending stages give FP32 0xC37B8000 at output 6, an exact BF16 tie that
    rounds to even (0xC37C); running the stages in descending order gives
    0xC37B7FFF -> 0xC37B.  The oracle must follow the ascending order."""
    inp = [0xb9a7, 0x4320, 0x4022, 0x37f4, 0x4145, 0xbc42, 0xb993, 0xbf65,
           0xbb68, 0xb9d2, 0x448b, 0xc354, 0xc39f, 0xc1be, 0xc414, 0xbc9b]
    x = bf16_bits_to_f32(inp)
    y = orc.wht(x[None], sign_mask=0, c=0.25)[0]
    assert f32_bits(y[6]) == 0xC37C0000

    def butterfly(v, order):
        v = v.astype(np.float32).copy()
        for h in order:
            for i in range(16):
                if i & h == 0:
                    a, b = v[i], v[i + h]
                    v[i], v[i + h] = np.float32(a + b), np.float32(a - b)
        return v
    asc = butterfly(x, [1, 2, 4, 8]) * np.float32(0.25)
    desc = butterfly(x, [8, 4, 2, 1]) * np.float32(0.25)
    assert f32_bits(asc[6]) == 0xC37B8000 and f32_bits(desc[6]) == 0xC37B7FFF


def test_b7_concat_order(orc):
    pe = np.full((1, 64), 0x3F80, np.uint16)     # 1.0
    nope = np.zeros((1, 64), np.uint16)
    v = np.concatenate([bf16_bits_to_f32(pe), bf16_bits_to_f32(nope)], axis=1)
    y = orc.wht(v)[0]
    assert y[0] == 5.65625 and y[64] == 5.65625 and np.count_nonzero(y) == 2
    v = np.concatenate([bf16_bits_to_f32(nope), bf16_bits_to_f32(pe)], axis=1)
    y = orc.wht(v)[0]
    assert y[0] == 5.65625 and y[64] == -5.65625 and np.count_nonzero(y) == 2


def test_rotation_preserves_norm_and_inner_products(orc):
    """(Hq).(Hk) = q.k for the orthonormal H; the only error is the BF16 rounding
    of each output (relative 2^-9) plus FP32 sums."""
    rng = np.random.default_rng(7)
    q = rng.standard_normal((2000, 128)).astype(np.float32)
    k = rng.standard_normal((2000, 128)).astype(np.float32)
    hq, hk = orc.wht(q), orc.wht(k)
    dots = np.sum(q.astype(np.float64) * k, axis=1)
    hdots = np.sum(hq.astype(np.float64) * hk, axis=1)
    bound = 2 * 2.0 ** -8 * np.linalg.norm(q, axis=1) * np.linalg.norm(k, axis=1)
    assert np.all(np.abs(hdots - dots) <= bound)
    nq = np.linalg.norm(q.astype(np.float64), axis=1)
    assert np.allclose(np.linalg.norm(hq.astype(np.float64), axis=1), nq, rtol=2.0 ** -8)
    # RHT16 with 1/4 normalization is orthonormal too
    x = rng.standard_normal((2000, 16)).astype(np.float32)
    y = orc.wht(x, sign_mask=0x3C5A)
    assert np.allclose(np.linalg.norm(y.astype(np.float64), axis=1),
                       np.linalg.norm(x.astype(np.float64), axis=1), rtol=2.0 ** -8)


def test_involution(orc):
    """Applying the normalized 128-point transform twice returns the input up
    to the BF16 rounding of each pass."""
    rng = np.random.default_rng(8)
    x = torch.from_numpy(rng.standard_normal((500, 128)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    y = orc.wht(orc.wht(x))
    assert np.allclose(y, x, atol=4 * 2.0 ** -8 * np.abs(x).max())


def test_nan_spreads_to_its_block(orc):
    x = np.ones((1, 16), np.float32)
    x[0, 5] = np.nan
    assert np.isnan(orc.wht(x)[0]).all()


def test_subnormal_inputs_are_not_flushed(orc):
    """A BF16 subnormal input block: (2^-133) * 16 = 2^-129 stays representable
    in FP32 (subnormal), and x 0.25 gives 2^-131, which BF16 keeps as a subnormal."""
    x = np.full((1, 16), bf16_bits_to_f32([0x0001])[0], np.float32)
    y = orc.wht(x)[0]
    assert y[0] == np.float32(2.0 ** -131) and not y[1:].any()
