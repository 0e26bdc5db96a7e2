"""Pins of the oracle's grouped NVFP4 quantizer.

Format (TransformerEngine PR #2564, Greptile summary; the NVFP4 quantizer of PR
#2555): E2M1 codes in 1x16 blocks with an E4M3 block scale and an FP32 tensor
scale; the column-wise output is computed from the transposed operand after the
16-point RHT (PR #2555 review: the RHT(x^T) intermediate of the unfused path);
grouping by split_sections that are multiples of 128 (PR #2555, cast.cpp comment).

The tensor-scale recipe g = max(A, 1e-10) * F(1/2688) per section and direction is
a reading (the pages name an FP32 per-tensor scale but no formula); these tests pin
the oracle's arithmetic of that reading with hand cases and invariants."""
import numpy as np
import pytest
import scipy.linalg
import torch

from nvfp4_quantization_amd import synth
from tests.golden_util import num, rows


def bf16(v):
    return torch.tensor(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_of_bf16(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


def unpack(codes_bytes):
    b = np.asarray(codes_bytes, np.uint8)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])


def e4m3(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(torch.float8_e4m3fn).float().numpy()


# ------------------------------------------------------------------ B9 hand cases
def test_b9_block_cases(orc):
    fix = {}
    for r in rows("nvfp4_blocks.txt"):
        fix.setdefault(r[0], []).append(r[1:])
    A, g_bits = num(fix["section"][0][0]), num(fix["section"][0][1])
    g = orc.nvfp4_global_scale(A)
    assert g.view(np.uint32) == g_bits
    for a, sc_want in fix["block"]:
        blk = np.zeros(16, np.float32)
        blk[3] = num(a)
        sc, codes = orc.nvfp4_block(blk, g)
        assert sc == num(sc_want), a
        if sc == 0:
            assert not codes.any()                 # scale underflow: zero block
    for a, d in fix["block_d"]:
        blk = np.zeros(16, np.float32)
        blk[0] = num(a)
        sc, _ = orc.nvfp4_block(blk, g)
        assert e4m3([sc])[0] * g == np.float32(num(d))
    xs = [num(t) for t in fix["codes_x"][0]]
    xs[11] = f32_of_bf16(bf16([xs[11]]))[0]       # BF16(0.1)
    sc, codes = orc.nvfp4_block(np.array(xs, np.float32), g)
    assert sc == 0x78                              # a = 6: t = 256, d = 1.0
    assert codes.tolist() == [num(t) for t in fix["codes_c"][0]]
    packed = (codes[0::2] | (codes[1::2] << 4)).tolist()
    assert packed == [num(t) for t in fix["packed"][0]]
    blk = np.zeros(16, np.float32)
    blk[0] = 6.25
    sc, codes = orc.nvfp4_block(blk, g)
    assert sc == 0x78 and codes[0] == 7           # saturates at 6
    assert orc.nvfp4_global_scale(0.0).view(np.uint32) == num(fix["empty_section_g"][0][0])


def test_nan_block(orc):
    blk = np.ones(16, np.float32)
    blk[9] = np.nan
    sc, codes = orc.nvfp4_block(blk, np.float32(0.01))
    assert sc == 0x7F and not codes.any()


def test_inf_block_cases(orc):
    """IEEE arithmetic as written (O3, O16).  An infinity over a finite tensor scale
    makes t infinite: the scale saturates to 448 (0x7E) and the infinity encodes as
    +6; the other values encode against d = 448 g.  Over the infinite g of an
    infinite tensor amax, a finite block amax gives t = 0 (scale 0, zero codes) and
    an infinite one t = inf / inf = NaN: the NaN scale 0x7F with zero codes, as for a
    NaN block."""
    g = np.float32(0.01)
    blk = np.ones(16, np.float32)
    blk[4], blk[7] = np.inf, np.float32(-2.0)
    sc, codes = orc.nvfp4_block(blk, g)
    assert sc == 0x7E and codes[4] == 7
    d = np.float32(448.0) * g                      # 4.48: 1 / d = 0.22 -> 0, -2 / d = -0.45 -> -0.5
    assert codes[0] == 0 and codes[7] == 0x9
    gi = orc.nvfp4_global_scale(np.float32(np.inf))
    assert np.isinf(gi) and gi > 0
    sc, codes = orc.nvfp4_block(np.ones(16, np.float32), gi)
    assert sc == 0 and not codes.any()
    sc, codes = orc.nvfp4_block(blk, gi)
    assert sc == 0x7F and not codes.any()


def test_inf_in_column_blocks(orc):
    """One +inf in a 16-row column block: all 16 rotated values are infinite (H16 has
    no zero entry), so the column block's scale saturates (0x7E) and its codes are
    +-6 with the signs of column 5 of H16 (sign mask 0).  Two +infs at rows 2 and 3
    of a column cancel (inf - inf = NaN) in the rotated values of odd index, where
    H16's columns 2 and 3 differ: that block gets the NaN scale 0x7F and zero codes.
    The tensor amax (NaN left out) is measured as inf; finite supplied maxima keep g
    finite so that the rest of the tile encodes normally, and the measured maxima
    still come out infinite."""
    m, k = 128, 128
    x = np.zeros((m, k), np.float32)
    x[:, :] = np.random.default_rng(31).standard_normal((m, k))
    x[5, 3] = np.inf
    x[2, 10] = x[3, 10] = np.inf
    xb = bf16(x)
    amax = (np.float32([8.0]), np.float32([8.0]))
    out = orc.group_rht_quant_nvfp4(xb, [m], 0, orc.ROWWISE | orc.COLUMNWISE, amax_in=amax)
    assert np.isinf(out.row_amax[0]) and np.isinf(out.col_amax[0])
    cs = out.col_scales.reshape(k, m // 16)
    cc = unpack(out.col_codes.reshape(k, m // 2))
    H = scipy.linalg.hadamard(16)
    assert cs[3, 0] == 0x7E
    np.testing.assert_array_equal(cc[3, :16], np.where(H[:, 5] > 0, 0x7, 0xF))
    assert cs[10, 0] == 0x7F and not cc[10, :16].any()
    rs = out.row_scales.reshape(m, k // 16)
    rc = unpack(out.row_codes.reshape(m, k // 2))
    assert rs[5, 0] == 0x7E and rc[5, 3] == 7
    assert rs[2, 0] == 0x7E and rs[3, 0] == 0x7E and rc[2, 10] == 7
    # measured: g is infinite, every finite block gets scale 0 and the infinite
    # ones the NaN scale; all codes are zero
    meas = orc.group_rht_quant_nvfp4(xb, [m], 0, orc.ROWWISE | orc.COLUMNWISE)
    assert np.isinf(meas.row_global[0]) and np.isinf(meas.col_global[0])
    assert not meas.row_codes.any() and not meas.col_codes.any()
    rs = meas.row_scales.reshape(m, k // 16)
    assert set(np.unique(rs)) == {0, 0x7F} and rs[5, 0] == 0x7F and rs[4, 0] == 0


def test_zero_block(orc):
    sc, codes = orc.nvfp4_block(np.zeros(16, np.float32), np.float32(0.01))
    assert sc == 0 and not codes.any()


# ------------------------------------------------------------------ invariants
def small_case(rows=256, k=256, sections=(128, 0, 128), mask=0x9216, seed=21, scale_rows=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k)).astype(np.float32)
    if scale_rows:
        x *= np.exp2(rng.integers(-3, 4, (rows, 1)))
    return bf16(x), list(sections), mask


def test_largest_block_gets_top_scale(orc):
    """The block whose amax equals the section amax gets scale 448 (0x7E) and
    decodes to +-6 * 448 * g ~ A; every other block's scale is <= 0x7E."""
    x, sections, mask = small_case()
    out = orc.group_rht_quant_nvfp4(x, sections, mask, 3)
    k = x.shape[1]
    rs = out.row_scales.reshape(-1, k // 16)
    assert rs.max() == 0x7E
    starts = np.cumsum([0] + sections)
    for s, (a, b) in enumerate(zip(starts[:-1], starts[1:])):
        if a == b:
            continue
        assert rs[a:b].max() == 0x7E
        cs = out.col_scales[k * a // 16:k * b // 16]
        assert cs.max() == 0x7E


def test_dequant_error_bound(orc):
    x, sections, mask = small_case(sections=(256,), scale_rows=False)
    out = orc.group_rht_quant_nvfp4(x, sections, mask, 1)
    rows, k = x.shape
    g = out.row_global[0]
    sc = e4m3(out.row_scales.reshape(rows, k // 16))
    d = (sc * g).astype(np.float32)
    codes = unpack(out.row_codes.reshape(rows, k // 2))
    deq = E2M1[codes] * np.repeat(d, 16, axis=1)
    xv = f32_of_bf16(x).astype(np.float64)
    y = xv / np.repeat(d, 16, axis=1)
    spacing = np.where(np.abs(y) < 2, 0.5, np.where(np.abs(y) < 4, 1.0, 2.0))
    err = np.abs(deq - xv) / np.repeat(d, 16, axis=1)
    sat = np.abs(y) > 6
    assert np.all(err[~sat] <= spacing[~sat] / 2 * (1 + 1e-6))
    assert np.all(err[sat] <= np.abs(y[sat]) - 6 + 1e-6)


def test_empty_sections_write_floor_scale(orc):
    x, _, mask = small_case(rows=128)
    out = orc.group_rht_quant_nvfp4(x, [0, 128, 0], mask, 3)
    assert out.row_global.view(np.uint32)[0] == 0x29278B6D == out.row_global.view(np.uint32)[2]
    assert out.col_global.view(np.uint32)[2] == 0x29278B6D


def test_grouping_equals_per_section_calls(orc):
    """A grouped call equals the single-section calls concatenated (row outputs
    by rows, column outputs section after section)."""
    x, sections, mask = small_case(rows=512, sections=(128, 256, 0, 128))
    k = x.shape[1]
    full = orc.group_rht_quant_nvfp4(x, sections, mask, 7)
    r0 = 0
    for s, m in enumerate(sections):
        if m == 0:
            continue
        one = orc.group_rht_quant_nvfp4(x[r0:r0 + m], [m], mask, 7)
        assert np.array_equal(full.row_codes[r0 * k // 2:(r0 + m) * k // 2], one.row_codes)
        assert np.array_equal(full.row_scales[r0 * k // 16:(r0 + m) * k // 16], one.row_scales)
        assert np.array_equal(full.col_codes[k * r0 // 2:k * (r0 + m) // 2], one.col_codes)
        assert np.array_equal(full.col_scales[k * r0 // 16:k * (r0 + m) // 16], one.col_scales)
        assert np.array_equal(full.fp8_codes[r0 * k:(r0 + m) * k], one.fp8_codes)
        assert full.row_global[s] == one.row_global[0] and full.col_global[s] == one.col_global[0]
        r0 += m


def test_other_sections_do_not_matter(orc):
    """Section-local amax and section-local SR counters: changing the other
    sections' data and sizes leaves this section's bytes unchanged."""
    rng = np.random.default_rng(22)
    k = 128
    mine = bf16(rng.standard_normal((128, k)))
    a = bf16(rng.standard_normal((256, k)) * 50)
    b = bf16(rng.standard_normal((128, k)) * 0.01)
    o1 = orc.group_rht_quant_nvfp4(np.concatenate([a, mine]), [256, 128], 0x1234, 3, seed=99,
                                   row_offsets=[5, 7], col_offsets=[6, 8])
    o2 = orc.group_rht_quant_nvfp4(np.concatenate([b, mine]), [128, 128], 0x1234, 3, seed=99,
                                   row_offsets=[1, 7], col_offsets=[2, 8])
    assert np.array_equal(o1.row_codes[256 * k // 2:], o2.row_codes[128 * k // 2:])
    assert np.array_equal(o1.col_codes[k * 256 // 2:], o2.col_codes[k * 128 // 2:])
    assert np.array_equal(o1.col_scales[k * 256 // 16:], o2.col_scales[k * 128 // 16:])


def test_columnwise_is_rowwise_of_the_rotated_transpose(orc):
    """The unfused definition: build the BF16 [cols x rows] intermediate RHT(x^T)
    with scipy's Hadamard matrix (exact for small-integer inputs), quantize it
    row-wise as its own section, and compare with the column-wise outputs."""
    rng = np.random.default_rng(23)
    rows, k, mask = 128, 128, 0xC35A
    xi = rng.integers(-15, 16, (rows, k)).astype(np.float32)
    x = bf16(xi)
    H = scipy.linalg.hadamard(16).astype(np.float64)
    D = np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(16)])
    blocks = xi.astype(np.float64).reshape(rows // 16, 16, k)          # [b][t][c]
    rot = np.einsum("ij,bjc->bic", H * D[None, :] * 0.25, blocks)     # exact
    yt = rot.transpose(2, 0, 1).reshape(k, rows)                        # [c][16b + i]
    inter = bf16(yt)                                                    # BF16 intermediate
    assert np.array_equal(f32_of_bf16(inter), yt.astype(np.float32))
    col = orc.group_rht_quant_nvfp4(x, [rows], mask, 2)
    via = orc.group_rht_quant_nvfp4(inter, [k], 0, 1)
    # same tensor scale: the column values' amax equals the intermediate's amax
    assert col.col_global[0] == via.row_global[0]
    assert np.array_equal(col.col_codes, via.row_codes)
    assert np.array_equal(col.col_scales, via.row_scales)


def test_fp8_rowwise_output_is_the_fp8_quantizer(orc):
    x, sections, mask = small_case(rows=256, k=384, sections=(128, 128))
    out = orc.group_rht_quant_nvfp4(x, sections, mask, 4)
    q, s = orc.quant_fp8_1x128(x)
    assert np.array_equal(out.fp8_codes, q.ravel()) and np.array_equal(out.fp8_scales, s.ravel())


# ------------------------------------------------------------------ stochastic rounding
def test_sr_deterministic_and_streams_distinct(orc):
    x, sections, mask = small_case(rows=256, sections=(256,))
    a = orc.group_rht_quant_nvfp4(x, sections, mask, 3, seed=7, row_offsets=[3], col_offsets=[3])
    b = orc.group_rht_quant_nvfp4(x, sections, mask, 3, seed=7, row_offsets=[3], col_offsets=[3])
    c = orc.group_rht_quant_nvfp4(x, sections, mask, 3, seed=8, row_offsets=[3], col_offsets=[3])
    r = orc.group_rht_quant_nvfp4(x, sections, mask, 3)
    assert np.array_equal(a.row_codes, b.row_codes) and np.array_equal(a.col_codes, b.col_codes)
    assert not np.array_equal(a.row_codes, c.row_codes)
    assert not np.array_equal(a.row_codes, r.row_codes)
    # scales do not depend on the rounding mode
    assert np.array_equal(a.row_scales, r.row_scales) and np.array_equal(a.col_scales, r.col_scales)
    # SR moves each code by at most one grid step from RNE, in the direction of x
    ca, cr = unpack(a.row_codes), unpack(r.row_codes)
    assert np.all(np.abs(E2M1[ca].astype(np.float64) - E2M1[cr]) <= 2.0)


def test_sr_matches_philox_bytes(orc):
    """The SR codes of one block follow from the element-wise SR encoder with the
    block's 16 Philox bytes (counter = (lo off, hi off, lo beta, hi beta))."""
    x, sections, mask = small_case(rows=128, k=128, sections=(128,))
    seed, off = 0x0123456789ABCDEF, 0xFEDCBA9876543210
    out = orc.group_rht_quant_nvfp4(x, sections, mask, 1, seed=seed, row_offsets=[off], col_offsets=None)
    g = out.row_global[0]
    k = 128
    for (r, kb) in [(0, 0), (5, 3), (127, 7)]:
        beta = r * (k // 16) + kb
        w = orc.philox4x32_10([off & 0xFFFFFFFF, off >> 32, beta & 0xFFFFFFFF, beta >> 32],
                              [seed & 0xFFFFFFFF, seed >> 32])
        rb = np.array([(int(w[t >> 2]) >> (8 * (t & 3))) & 0xFF for t in range(16)], np.uint8)
        sc, codes = orc.nvfp4_block(f32_of_bf16(x[r, 16 * kb:16 * kb + 16]), g, rb)
        assert out.row_scales[r * (k // 16) + kb] == sc
        got = unpack(out.row_codes[r * k // 2 + 8 * kb:r * k // 2 + 8 * kb + 8])
        assert got.tolist() == codes.tolist()


def test_sr_unbiased_over_seeds(orc):
    """Averaged over many seeds, SR dequantizes to x within the sampling error."""
    rng = np.random.default_rng(24)
    x = bf16(rng.standard_normal((128, 128)))
    acc = np.zeros((128, 128))
    n = 200
    for sd in range(n):
        o = orc.group_rht_quant_nvfp4(x, [128], 0, 1, seed=sd, row_offsets=[0], col_offsets=None)
        g = o.row_global[0]
        d = e4m3(o.row_scales.reshape(128, 8)) * g
        acc += E2M1[unpack(o.row_codes.reshape(128, 64))] * np.repeat(d, 16, axis=1)
    err = np.abs(acc / n - f32_of_bf16(x))
    d_full = np.repeat(e4m3(o.row_scales.reshape(128, 8)) * g, 16, axis=1)
    xv = np.abs(f32_of_bf16(x) / d_full)
    inside = xv < 5.9
    assert np.all(err[inside] <= 4 * d_full[inside] / np.sqrt(n) + 1e-7)


def test_rejects_misaligned_sections(orc):
    with pytest.raises(ValueError):
        orc.group_rht_quant_nvfp4(np.zeros((192, 128), np.uint16), [64, 128], 0, 3)


def test_threaded_oracle_equals_single_thread(orc):
    """The work-splitting helper (independent sections / column ranges on threads)
    produces the same bytes as the plain loop."""
    x, sections, mask = small_case(rows=512, k=256, sections=(128, 0, 256, 128))
    a = orc.group_rht_quant_nvfp4(x, sections, mask, 7, seed=3, row_offsets=[1, 2, 3, 4],
                                  col_offsets=[5, 6, 7, 8])
    b = orc.group_rht_quant_nvfp4(x, sections, mask, 7, seed=3, row_offsets=[1, 2, 3, 4],
                                  col_offsets=[5, 6, 7, 8], threads=4)
    for name in ("row_codes", "row_scales", "row_global", "col_codes", "col_scales", "col_global",
                 "fp8_codes", "fp8_scales"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name


# ------------------------------------------------------------------ caller-supplied amax
def _small_group(seed=41):
    w = synth.grouped_nvfp4(total_rows=640, k=256, parts=4, seed=seed)
    x = w.tensors["x"].view(torch.int16).numpy().view(np.uint16)
    return x, w.params["split_sections"], w.params["sign_mask"]


def test_given_measured_amax_reproduces_plain_call(orc):
    """Supplying the maxima the plain call measures changes nothing."""
    x, sec, mask = _small_group()
    a = orc.group_rht_quant_nvfp4(x, sec, mask, 3)
    b = orc.group_rht_quant_nvfp4(x, sec, mask, 3, amax_in=(a.row_amax, a.col_amax))
    for n in ("row_codes", "row_scales", "row_global", "col_codes", "col_scales", "col_global"):
        assert np.array_equal(getattr(a, n), getattr(b, n)), n


def test_measured_amax_matches_closed_form(orc):
    """Row amax = max |x|; column amax = max |BF16(0.25 * H16 D x)| with H16 the
    Sylvester matrix, on small-integer inputs where every sum is exact in FP32."""
    from scipy.linalg import hadamard
    rng = np.random.default_rng(7)
    v = rng.integers(-40, 41, size=(256, 128)).astype(np.float32)
    x = (v.view(np.uint32) >> 16).astype(np.uint16)
    mask = 0x35A1
    out = orc.group_rht_quant_nvfp4(x, [128, 128], mask, 3, threads=2)
    D = np.array([-1.0 if (mask >> t) & 1 else 1.0 for t in range(16)])
    H = hadamard(16).astype(np.float64)
    for s in range(2):
        xs = v[128 * s:128 * (s + 1)].astype(np.float64)
        assert out.row_amax[s] == np.abs(xs).max()
        blocks = xs.reshape(8, 16, 128)                       # [block][t][column]
        y = 0.25 * np.einsum("it,btc->bic", H, D[None, :, None] * blocks)
        # y is exact in FP32 (integers / 4); the column values are its BF16 roundings
        want = torch.tensor(np.float32(np.abs(y).max())).to(torch.bfloat16).float().item()
        assert out.col_amax[s] == np.float32(want)


def test_small_given_amax_saturates(orc):
    """A supplied amax below the data's: blocks above it take the top scale 0x7E and
    their largest elements the top code 6 (saturation, never NaN)."""
    x, sec, mask = _small_group(43)
    a = orc.group_rht_quant_nvfp4(x, sec, mask, 1)
    b = orc.group_rht_quant_nvfp4(x, sec, mask, 1, amax_in=(a.row_amax / 4, None))
    assert (b.row_scales <= 0x7E).all() and (b.row_scales != 0x7F).all()
    assert (b.row_scales == 0x7E).sum() > (a.row_scales == 0x7E).sum()
    f = x.view(np.uint16).astype(np.uint32) << 16
    xf = f.view(np.float32).reshape(x.shape)
    r, c = np.unravel_index(np.argmax(np.abs(xf[:sec[0]])), xf[:sec[0]].shape)
    code = (b.row_codes[r * x.shape[1] // 2 + c // 2] >> (4 * (c & 1))) & 7
    assert code == 7


def test_large_given_amax_keeps_error_bound(orc):
    """A supplied amax above the data's only coarsens the scales: dequantized values
    stay within half a code step of the inputs."""
    x, sec, mask = _small_group(44)
    a = orc.group_rht_quant_nvfp4(x, sec, mask, 1)
    b = orc.group_rht_quant_nvfp4(x, sec, mask, 1, amax_in=(a.row_amax * 3, None))
    assert (b.row_global > a.row_global).all()
    # every block keeps a nonzero scale and codes that dequantize close to x
    k = x.shape[1]
    xf = ((x.astype(np.uint32) << 16).view(np.float32)).reshape(-1, k)
    R0 = 0
    for s, m in enumerate(sec):
        g = b.row_global[s]
        for r in range(R0, R0 + m, 37):
            for kb in range(0, k // 16, 5):
                sc = b.row_scales[r * (k // 16) + kb]
                d = np.float32(e4m3([sc])[0]) * g
                for t in range(16):
                    c = kb * 16 + t
                    code = (b.row_codes[r * k // 2 + c // 2] >> (4 * (c & 1))) & 0xF
                    val = [0, .5, 1, 1.5, 2, 3, 4, 6][code & 7] * (-1 if code & 8 else 1) * d
                    assert abs(val - xf[r, c]) <= 1.0 * d + 1e-30
        R0 += m
