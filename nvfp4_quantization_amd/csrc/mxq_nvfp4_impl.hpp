// mxq_nvfp4_impl.hpp -- device code of the grouped NVFP4 quantization with a
// 16-point RHT on the column-wise operand (gfx950), shared by the translation units
// that instantiate its kernels (mxq_nvfp4.hip and mxq_nvfp4_quant_*.hip).
//
// The method: TransformerEngine PR #2564 "[NVFP4][MOE] Bug Fix for NVFP4 Grouped
// Quant" (Greptile summary: grouped row-wise + column-wise RHT cast fusion, the
// workspace supplied by the caller) and the review comments of PR #2555 on
// quantizer.cpp (RHT only for the column-wise operand; the RHT(x^T) intermediate
// has the input dtype; a separate column-wise RNG).
//
// The FP32 tensor scale of a section needs the section's amax before any code is
// final, so a call runs three kernels per group of sections:
//
//   k_nvfp4_amax   one work-group per 16-row band and 1024 columns: max |x| and
//                  max |H16 D x| of the band, one partial each (ordinary stores).
//   k_nvfp4_scales one work-group per section: folds the section's partials into
//                  the two tensor scales and writes the section's scale tables.
//                  The kernels meet only through the stream order: no counters,
//                  no waits, and nothing in the workspace outlives the call.
//   k_nvfp4_quant  one wave per tile: re-reads the tile (partly from the Infinity
//                  Cache) and writes
//                  every requested output: the row pass first (a row block needs
//                  only its own row, so it starts as the rows arrive), then the
//                  column pass (all 16 rows of each column block), then FP8.
//
// Scale tables: for each direction and E4M3 scale code c the quantizer divides by
// d = fl(E4M3(c) * g).  The table holds (d, y = fl(1/d), ym): ym is a multiplier
// whose plain product fl(u * ym) picks the same E2M1 code as fl(u / d) for every
// BF16 u, or negative when there is none.  fl(u * ym) and fl(u / d) differ by a
// few FP32 ulps at most, so a BF16 u can only be decided differently when u / d
// lies within about 2^-21 (relative) of one of the seven E2M1 rounding boundaries
// 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; BF16 values are 2^-8 apart, so only the two
// BF16 neighbours of each boundary times d can, and those fourteen are checked
// against the exact division for ym = y and its nearest neighbours.  With
// stochastic rounding the rule reads more of the quotient (its grid spacing and
// floor(256 f)), and the table holds a multiplier that keeps that part of the exact
// quotient for every BF16 u (build_tables_wg).  A pass (one direction of one
// section) takes one multiply per element when every scale code of its table has a
// multiplier, else the exact division.  Codes without a nearest-even multiplier come
// from short divisors whose exact boundary ties need opposite roundings; they arise
// when the section amax carries a factor of 3 (2688 = 2^7 * 3 * 7).  Column values enter unscaled: BF16(x/4) =
// BF16(x)/4 and fl((u/4)/d) = fl(u/(4d)) whenever x/4 is a normal number, and
// where it is not, both quotients are far below the smallest E2M1 step with the
// same sign, so the column tables are built for 4d and the 1/4 costs nothing per
// element.
#pragma once

#include "mxq_device.hpp"
#include "mxq_internal.hpp"

namespace mxq {

namespace {

// Tensor scale g = fl(max(A, F(1e-10)) * F(1/2688)).
__device__ __forceinline__ float tensor_scale(float amax) {
    return (amax > k_floor() ? amax : k_floor()) * k_inv2688();
}

// E4M3 block-scale code of a 1x16 block with amax a (a BF16 value):
// E4M3(fl(fl(a * F(1/6)) / g)), yg = fl(1/g).  The quotient is clamped to 448
// before the conversion so that it saturates: with a measured tensor amax it never
// exceeds 448 by more than rounding, but a caller-supplied amax below the data's
// can push it anywhere up to infinity.  The division's special cases are IEEE's
// (div_fixup: an infinite a over a finite g gives infinity, hence 448; a finite a
// over an infinite g gives 0; infinite over infinite gives NaN).  The clamp keeps a
// NaN (IEEE minimum), and the conversion turns it into the NaN code 0x7F: a block
// whose amax is NaN gets the NaN scale with no separate test.  (a >= 0: the sign
// bit is clear.)
__device__ __forceinline__ uint32_t block_code(float a, float g, float yg) {
    const float a6 = a * k_inv6();
    const float t = div_ieee(a6, g, yg);
    return e4m3_code(__builtin_elementwise_minimum(t, 448.0f)) & 0x7Fu;
}

__device__ __forceinline__ uint32_t e2m1_one(float q) { return e2m1_pack2<0>(0u, q, q) & 0xFu; }

// The multiplier for the product path of divisor d (y = fl(1/d)): fl(1/d) or a
// neighbour one ulp away such that fl(u * ym) has the E2M1 code of fl(u / d) for
// every BF16 u; negative when neither does (exact quotients that fall on rounding
// boundaries are common, because d and the boundaries are short binary numbers).
// fl(u * ym) and fl(u / d) differ by a few ulps at most, so only the two BF16
// neighbours of each boundary times d can be decided differently: those 14 values
// are checked against the exact quotient, which is computed once for all
// candidates.  Candidates two or more ulps away never qualify where these do not
// (a survey of random tensor scales over every scale code found none).
__device__ float product_multiplier(float d, float y) {
    const float taus[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
    float us[14];
    uint32_t exact[14];
#pragma unroll
    for (int i = 0; i < 7; ++i) {
        const uint32_t lo = __builtin_bit_cast(uint32_t, taus[i] * d) & 0xFFFF0000u;
        us[2 * i] = __builtin_bit_cast(float, lo);
        us[2 * i + 1] = __builtin_bit_cast(float, lo + 0x10000u);
        exact[2 * i] = e2m1_one(div_rn(us[2 * i], d, y));
        exact[2 * i + 1] = e2m1_one(div_rn(us[2 * i + 1], d, y));
    }
    const int deltas[3] = {0, -1, 1};
    for (int c = 0; c < 3; ++c) {
        const float ym = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, y) + (uint32_t)deltas[c]);
        bool ok = true;
#pragma unroll
        for (int j = 0; j < 14; ++j) ok &= e2m1_one(us[j] * ym) == exact[j];
        if (ok) return ym;
    }
    return -y;
}

// Running max |x| over packed BF16 pairs, NaN ignored.
__device__ __forceinline__ uint32_t absmax_nonan_pairs(uint32_t acc, uint32_t w) {
    return absmax_pk_nonan(acc, w);
}

// Blocks whose random words are drawn together under stochastic rounding (1, 2 and 4
// measured: 4 is fastest).
constexpr int kSrChains = 4;

__device__ __forceinline__ u32x4 block_random(uint64_t seed, uint64_t off, uint64_t beta) {
    u32x4 c = {(uint32_t)off, (uint32_t)(off >> 32), (uint32_t)beta, (uint32_t)(beta >> 32)};
    return philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
}

// Butterfly h = 1, 2, 4, 8 over 16 values.
__device__ __forceinline__ void butterfly16(float (&v)[16]) {
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i & h) continue;
            const float x0 = v[i], x1 = v[i + h];
            v[i] = x0 + x1;
            v[i + h] = x0 - x1;
        }
    }
}

// BF16 element of a packed pair widened to FP32 with its sign flipped when
// neg = 0x80000000 (adding the top bit flips it).
__device__ __forceinline__ float lo_signed(uint32_t p, uint32_t neg) {
    return __builtin_bit_cast(float, (p << 16) + neg);
}
__device__ __forceinline__ float hi_signed(uint32_t p, uint32_t neg) {
    return __builtin_bit_cast(float, (p & 0xFFFF0000u) ^ neg);
}
__device__ __forceinline__ uint32_t sign_of_row(uint32_t mask, int t) { return ((mask >> t) & 1u) << 31; }

// FP32 value of BF16(v) (nearest-even), one conversion.
__device__ __forceinline__ float round_bf16(float v) { return __builtin_bit_cast(float, pack_bf16(0.0f, v)); }

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v = __builtin_fmaxf(v, shfl_xor_f32(v, o));
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t w = shfl_xor_u32(v, o);
        v = w > v ? w : v;
    }
    return v;
}
__device__ __forceinline__ uint32_t group8_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
        uint32_t w = shfl_xor_u32(v, o);
        v = w > v ? w : v;
    }
    return v;
}

// Section of token tile T (uniform): the last section starting at or before T
// (empty sections start where the next one does, so they are skipped).
__device__ __forceinline__ int section_of(const Nvfp4Group& G, int T) {
    int s = 0;
    for (int i = 1; i < G.num_sections; ++i) s = G.tt_start[i] <= T ? i : s;
    return s;
}

// max |v_i| over 16 values: a tree of three-input maxima (depth 3, 8 operations).
// NaNs are ignored (callers that care detect them separately).
__device__ __forceinline__ float absmax16(const float (&v)[16]) {
    auto m3 = [](float a, float b, float c) {
        return __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(a), __builtin_fabsf(b)), __builtin_fabsf(c));
    };
    const float a = m3(v[0], v[1], v[2]), b = m3(v[3], v[4], v[5]), c = m3(v[6], v[7], v[8]);
    const float d = m3(v[9], v[10], v[11]), e = m3(v[12], v[13], v[14]);
    return __builtin_fmaxf(m3(a, b, c), m3(d, e, v[15]));
}

// max |v_i| over 16 values, NaN when any of them is NaN (IEEE maximum; a block that
// holds a NaN thus gets the NaN scale from block_code).
__device__ __forceinline__ float absmax16_nan(const float (&v)[16]) {
    auto m3 = [](float a, float b, float c) {
        return __builtin_elementwise_maximum(__builtin_elementwise_maximum(__builtin_fabsf(a), __builtin_fabsf(b)),
                                             __builtin_fabsf(c));
    };
    const float a = m3(v[0], v[1], v[2]), b = m3(v[3], v[4], v[5]), c = m3(v[6], v[7], v[8]);
    const float d = m3(v[9], v[10], v[11]), e = m3(v[12], v[13], v[14]);
    return __builtin_elementwise_maximum(m3(a, b, c), m3(d, e, v[15]));
}

// E2M1 codes of 8 values u[0..7] (element 2i in the low nibble of byte i):
// nearest-even of u * y (MUL) or of fl(u / d) (DIV), or stochastic with random bytes
// r0 .. r0+7 of rnd, of fl(u / d) (SR) or of u * y (SR_MUL).  IEEE: the quotients
// with IEEE's special cases (an infinite u, or an overflowing quotient), which only a
// block whose scale saturated can meet.
enum class Enc { Mul, Div, Sr, SrMul };
template <Enc E>
struct EncTag {
    static constexpr Enc value = E;
};
template <Enc E, bool IEEE = false>
__device__ __forceinline__ uint32_t encode8(const float* u, float d, float y, const u32x4& rnd, int r0) {
    uint32_t c = 0;
    if (E == Enc::Mul || E == Enc::Div) {
        float q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = E == Enc::Mul ? u[i] * y : IEEE ? div_ieee(u[i], d, y) : div_rn(u[i], d, y);
        // each conversion writes one byte of c and keeps the others; all four are
        // written, so c starts as the bits of q[0], whose register the first
        // conversion can then overwrite in place (no zeroing instruction)
        c = e2m1_pack2<0>(__builtin_bit_cast(uint32_t, q[0]), q[0], q[1]);
        c = e2m1_pack2<1>(c, q[2], q[3]);
        c = e2m1_pack2<2>(c, q[4], q[5]);
        c = e2m1_pack2<3>(c, q[6], q[7]);
    } else {
        float q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            q[i] = E == Enc::SrMul ? u[i] * y : IEEE ? div_ieee(u[i], d, y) : div_rn(u[i], d, y);
        // random bytes r0 .. r0 + 7: word r0 / 4 and the next (r0 is 0 or 8)
        const uint32_t wa = r0 == 0 ? rnd.x : rnd.z, wb = r0 == 0 ? rnd.y : rnd.w;
        const uint32_t r[8] = {rbyte_hi<0>(wa), rbyte_hi<1>(wa), rbyte_hi<2>(wa), rbyte_hi<3>(wa),
                               rbyte_hi<0>(wb), rbyte_hi<1>(wb), rbyte_hi<2>(wb), rbyte_hi<3>(wb)};
        c = e2m1_sr8(q, r);
    }
    return c;
}

// ---------------------------------------------------------------- amax work
// A quarter tile: rows 32q .. 32q+31; lane (h, c) holds rows 16h .. 16h+15 of it
// and columns 4c .. 4c+3 (one 8-byte load per row).
__device__ __forceinline__ void load_quarter(uint2 (&v)[16], const uint16_t* base, int64_t k, int q) {
#pragma unroll
    for (int t = 0; t < 16; ++t) v[t] = *reinterpret_cast<const uint2*>(base + (int64_t)(32 * q + t) * k);
}

// Row max |x| of the lane's 64 rows x 4 columns of a tile, NaN ignored (the rare
// path: the quarters are loaded again).
__device__ uint32_t lane_absmax_nonan(const uint16_t* base, int64_t k) {
    uint32_t m = 0;
#pragma unroll 1
    for (int q = 0; q < 4; ++q) {
#pragma unroll 1
        for (int t = 0; t < 16; ++t) {
            const uint2 w = *reinterpret_cast<const uint2*>(base + (int64_t)(32 * q + t) * k);
            m = absmax_nonan_pairs(absmax_nonan_pairs(m, w.x), w.y);
        }
    }
    return m;
}

// mr: running max |x| as BF16 bits (ROW without COL: packed integer maxima,
// NaN ignored); rmax: running FP32 max |x| (ROW with COL, from the widened values
// the butterfly needs anyway; a NaN input can spoil it, which nan reports);
// mc: running max |H16 D x|.
template <bool ROW, bool COL>
__device__ __forceinline__ void amax_quarter(const uint2 (&v)[16], uint32_t sign_mask, uint32_t& mr, float& rmax,
                                             float& mc, bool& nan) {
    if (ROW && !COL) {
        uint32_t m = 0;
#pragma unroll
        for (int t = 0; t < 16; ++t) m = absmax_pk(absmax_pk(m, v[t].x), v[t].y);
        m = fold_pk(m);
        if (m > 0x7F80u) {                           // a NaN: take the maximum without it
            m = 0;
#pragma unroll
            for (int t = 0; t < 16; ++t) m = absmax_nonan_pairs(absmax_nonan_pairs(m, v[t].x), v[t].y);
        }
        mr = m > mr ? m : mr;
    }
    if (COL) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float f[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const uint32_t w = j < 2 ? v[t].x : v[t].y;
                const uint32_t neg = sign_of_row(sign_mask, t);
                f[t] = (j & 1) ? hi_signed(w, neg) : lo_signed(w, neg);
            }
            if (ROW) {
#pragma unroll
                for (int t = 0; t < 16; ++t) rmax = __builtin_fmaxf(rmax, __builtin_fabsf(f[t]));
            }
            // stages h = 1, 2, 4; the last stage is not formed: for its pair (a, b) the
            // larger of |fl(a + b)| and |fl(a - b)| is fl(|a| + |b|) (rounding is
            // monotone and symmetric)
#pragma unroll
            for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if (i & h) continue;
                    const float x0 = f[i], x1 = f[i + h];
                    f[i] = x0 + x1;
                    f[i + h] = x0 - x1;
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float m = __builtin_fabsf(f[i]) + __builtin_fabsf(f[i + 8]);
                if (i == 0) nan |= m != m;          // depends on all 16 inputs: a NaN input reaches it
                mc = __builtin_fmaxf(mc, m);        // NaN values are quiet, and max ignores them
            }
        }
    }
}

// ---------------------------------------------------------------- quant work
// Tile in registers: lane (tb, cc) holds rows 16 tb .. 16 tb + 15 and columns
// 16 cc .. 16 cc + 15 as p[t][half] (8 BF16 each).
#define P(t, i) ((i) == 0 ? p[t][0].x : (i) == 1 ? p[t][0].y : (i) == 2 ? p[t][0].z : (i) == 3 ? p[t][0].w \
               : (i) == 4 ? p[t][1].x : (i) == 5 ? p[t][1].y : (i) == 6 ? p[t][1].z : p[t][1].w)

// Packed BF16 pair i (columns 2i, 2i + 1 of the lane's 16) of row t of the lane's tile.
__device__ __forceinline__ uint32_t tile_word(const uint4 (&p)[16][2], int t, int i) { return P(t, i); }

// Hide the tile's provenance from the compiler (no instruction is emitted).
// Otherwise it reuses values computed from the tile by an earlier pass in a later
// one, keeping hundreds of them live across the passes.
__device__ __forceinline__ void launder(uint4 (&p)[16][2]) {
#pragma unroll
    for (int t = 0; t < 16; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(p[t][h].x), "+v"(p[t][h].y), "+v"(p[t][h].z), "+v"(p[t][h].w));
}

struct BlockOut {
    uint2 codes;          // 16 E2M1 codes
    uint32_t scale;       // E4M3 scale byte
    bool unsafe;          // (Enc::Mul) the scale code needs the exact division
    float amax;           // max |value| of the block without NaNs (column: before BF16 rounding)
};

// 16 codes of one block of values u with scale code sc <= 0x7F (0x7F: the block holds
// a NaN).  The table entry's fourth word keeps the codes (all ones) or clears them
// (zero: scale 0, whose blocks decode to zero, and the NaN scale 0x7F).
template <Enc E>
__device__ __forceinline__ BlockOut encode_block(const float (&u)[16], uint32_t sc, const float4* tab,
                                                 const u32x4& rnd) {
    const float4 e = tab[sc];
    const float d = e.x, y = (E == Enc::Mul || E == Enc::SrMul) ? __builtin_fabsf(e.z) : e.y;
    const uint32_t keep = __builtin_bit_cast(uint32_t, e.w);
    BlockOut o;
    // Only a saturated scale lets a value be infinite or a quotient overflow (below it
    // |u / d| stays near 6 or less, where div_rn is exact).  The division path takes
    // the IEEE quotients throughout (one more operation per element, cheaper than a
    // branch per block); stochastic rounding by division, where the division is on
    // every element, branches.  (A product needs no such case: it is 6 or more, an
    // infinity included, exactly where the quotient is, and both saturate.)
    if (E == Enc::Sr && sc == 0x7Eu) {
        o.codes = make_uint2(encode8<E, true>(u, d, y, rnd, 0) & keep, encode8<E, true>(u + 8, d, y, rnd, 8) & keep);
    } else {
        constexpr bool kIeee = E == Enc::Div;
        o.codes = make_uint2(encode8<E, kIeee>(u, d, y, rnd, 0) & keep, encode8<E, kIeee>(u + 8, d, y, rnd, 8) & keep);
    }
    o.scale = sc;
    o.unsafe = e.z < 0.0f;
    return o;
}

// Column j of the lane: rows 16 tb .. +15 after the sign flip and the butterfly,
// rounded to BF16 (unscaled; the column tables carry the 1/4).
template <Enc E>
__device__ __forceinline__ BlockOut column_block(const uint4 (&p)[16][2], int j, uint32_t sign_mask, float g_c,
                                                 float yg_c, const float4* tab_c, const u32x4& rnd) {
    float v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const uint32_t w = P(t, j >> 1);
        const uint32_t neg = sign_of_row(sign_mask, t);
        v[t] = (j & 1) ? hi_signed(w, neg) : lo_signed(w, neg);
    }
    butterfly16(v);
    // NaN when an output is: a NaN input reaches all of them, and inf - inf (from
    // infinite or overflowing inputs) some
    const float m = absmax16_nan(v);
    // block amax of the column values BF16(v/4) = BF16(max |v|) / 4
    const uint32_t sc = block_code(0.25f * round_bf16(m), g_c, yg_c);
    float m_nonan = m;                               // the block's measured amax leaves NaNs out
    if (m != m) m_nonan = absmax16(v);
#pragma unroll
    for (int t = 0; t < 16; ++t) v[t] = round_bf16(v[t]);
    BlockOut o = encode_block<E>(v, sc, tab_c, rnd);
    o.amax = m_nonan;
    return o;
}

// Row t of the lane: columns 16 cc .. +15 (one row-wise block).  The block maximum
// is IEEE's: NaN when the block holds a NaN, which block_code turns into the NaN scale
// 0x7F (whose table entry clears the codes).
template <Enc E>
__device__ __forceinline__ BlockOut row_block(const uint4 (&p)[16][2], int t, float g_r, float yg_r,
                                              const float4* tab_r, const u32x4& rnd) {
    float u[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        u[2 * i] = lo_bf16(P(t, i));
        u[2 * i + 1] = hi_bf16(P(t, i));
    }
    const float a = absmax16_nan(u);                 // one of the values: BF16 already
    const uint32_t sc = block_code(a, g_r, yg_r);
    BlockOut o = encode_block<E>(u, sc, tab_r, rnd);
    o.amax = a;
    return o;
}

// max |x| of row t of the lane without NaNs (packed integer maxima: every NaN,
// signalling or quiet, has |bits| above 0x7F80).
__device__ __forceinline__ float row_absmax_nonan(const uint4 (&p)[16][2], int t) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = absmax_pk_nonan(m, P(t, i));
    return bf16_mag(m);
}

// The row pass of a tile: 16 row blocks per lane.  The scale bytes go to LDS (rsc:
// row r of the tile at r * RSTRIDE, this lane's block at + cc), to leave later in one
// piece per row for the whole work-group.  rc_tile: the tile's first row-code byte
// (wave-uniform).  Returns the lane's max |x| without NaNs (used with supplied maxima).
template <bool SR, int RSTRIDE>
__device__ __forceinline__ float row_pass(const Nvfp4Group& G, const uint4 (&p)[16][2], int s, int64_t c0,
                                          int64_t r_local0, float g_r, float yg_r, const float4* tab_r,
                                          bool div_mode, uint8_t* rsc, uint8_t* rc_tile, int tid) {
    const int64_t k = G.k;
    const u32x4 no_rnd = {0, 0, 0, 0};
    const int lane_row = (tid & 63) >> 3 << 4, cc = tid & 7;
    // the lane's offset in the tile fits 32 bits (k <= 2^26), so that each row's
    // store is a uniform base plus this offset, with no vector address arithmetic
    const uint32_t lane_off = (uint32_t)lane_row * (uint32_t)(k >> 1) + (uint32_t)cc * 8u;
    float amax = 0.0f;                               // max |x| of the lane's rows, NaNs aside
    auto put = [&](int t, const BlockOut& o) {
        uint8_t* const row_base = rc_tile + (int64_t)t * (k >> 1);
        // non-temporal (as the column codes): streamed out now rather than written back
        // from the caches while the next call's amax kernel reads
        __builtin_nontemporal_store(((uint64_t)o.codes.y << 32) | o.codes.x,
                                    reinterpret_cast<uint64_t*>(row_base + lane_off));
        rsc[(lane_row + t) * RSTRIDE + cc] = (uint8_t)o.scale;
        float am = o.amax;
        if (am != am) am = row_absmax_nonan(p, t);  // a NaN block: its other values count
        amax = __builtin_fmaxf(amax, am);
    };
    auto rnd_of = [&](int t) {
        return block_random(G.seed, G.row_off[s], (uint64_t)((r_local0 + t) * (k >> 4) + (c0 >> 4)));
    };
    if (SR && G.sr_row) {
        // kSrChains rows at a time, their Philox chains (ten dependent rounds of
        // quarter-rate multiplies each) all drawn before the first is used, so that
        // they overlap (the dividing encode branches on a saturated scale, and no
        // chain drawn after a branch would overlap one drawn before it).  By product
        // when every scale code of the row table has a stochastic multiplier.
        auto rows = [&](auto enc) {
#pragma unroll
            for (int t0 = 0; t0 < 16; t0 += kSrChains) {
                u32x4 rnd[kSrChains];
#pragma unroll
                for (int i = 0; i < kSrChains; ++i) rnd[i] = rnd_of(t0 + i);
#pragma unroll
                for (int i = 0; i < kSrChains; ++i)
                    put(t0 + i, row_block<decltype(enc)::value>(p, t0 + i, g_r, yg_r, tab_r, rnd[i]));
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if (div_mode)
            rows(EncTag<Enc::Sr>{});
        else
            rows(EncTag<Enc::SrMul>{});
    } else if (div_mode) {
        // the section's row table has a scale code without a multiplier: exact division
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            put(t, row_block<Enc::Div>(p, t, g_r, yg_r, tab_r, no_rnd));
            if (t & 1) __builtin_amdgcn_sched_barrier(0);   // two rows at a time
        }
    } else {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            put(t, row_block<Enc::Mul>(p, t, g_r, yg_r, tab_r, no_rnd));
            if (t & 1) __builtin_amdgcn_sched_barrier(0);   // two rows at a time
        }
    }
    return amax;
}

// Scale-table entry of scale code `code` for tensor scale g: (d, fl(1/d), ym, keep)
// with d = fl(E4M3(code) * g), or (4d, fl(1/d)/4, ...) for column values that enter
// unscaled (quarter), and keep = all ones (the codes stay).  Entry 0 (scale code 0
// never divides) holds (g, fl(1/g), fl(1/g), 0) and entry 127 (the NaN scale) zeros:
// both clear their blocks' codes.  Entry 127's first word is free for a flag.
__device__ __forceinline__ float4 table_entry(int code, float g, bool quarter) {
    if (code == 0) {
        const float yg = 1.0f / g;
        return make_float4(g, yg, yg, 0.0f);
    }
    if (code == 127) return make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float d = e4m3_value((uint32_t)code) * g;
    float y = 1.0f / d;
    if (quarter) { d *= 4.0f; y *= 0.25f; }
    return make_float4(d, y, product_multiplier(d, y), k_keep_codes());
}

}  // namespace

// ---------------------------------------------------------------- the kernels
// Scale tables of section s (row-wise, then column-wise), one entry per thread
// (direction tid >> 7, scale code tid & 127; threads 256 and up take no entry),
// into the workspace and, when tab is given, into it as well.  Entry 127's first
// word flags a direction with a scale code that has no multiplier (its exact ties
// need opposite roundings): that direction's pass then divides exactly.
//
// Every nonzero E4M3 value is (1 + m/8) 2^e, so the divisors d of codes that share
// m differ by exact powers of two, and so do their critical inputs, reciprocals and
// candidate multipliers, with the same quotients and products.  Lanes 0..7 of each
// direction's first wave search the multiplier of the representative 1 + m/8
// (m = lane) once; each entry takes it scaled by 2^-e when its own d and fl(1/d)
// are the representative's scaled exactly and g < 2^100 keeps every intermediate
// value of the search normal and finite, and searches on its own otherwise.
// A direction with stochastic rounding takes stochastic multipliers instead: ym
// such that fl(u * ym) and fl(u / d) give the stochastic rule the same grid spacing
// and the same floor(256 f), hence the same code for every random byte, for every
// BF16 u.  Every grid point of the rule (the multiples of D/256 below 6, and 6) is
// a multiple of 2^(E-9) in the binade [2^E, 2^(E+1)) of the quotient it bounds, so
// two positive quotients that agree in exponent and in the top 9 mantissa bits fall
// in the same cell of every binade.  Scaling u by a power of two scales both
// quotients exactly (while they stay normal), so the 128 BF16 significands
// u = 1 + k/128 decide it for every BF16 u: a candidate (y, y - 1 ulp, y + 1 ulp)
// qualifies when for each of them fl(u * ym) and the exact fl(u / d) share their bits
// above the 14th.  Each (direction, m) representative is checked this way by the
// whole work-group (2048 pairs), and an entry takes its representative's multiplier
// scaled by 2^-e under the same condition as above, else none.
// Every thread of the work-group calls it (it holds barriers).  sh: kTableLdsWords
// words of LDS.
constexpr int kTableLdsWords = 4 + 16 + 16;
template <bool ROW, bool COL>
__device__ __forceinline__ void build_tables_wg(const Nvfp4Group& G, int s, float g_r, float g_c,
                                                float4 (*tab)[128], uint32_t* sh, int tid) {
    const int lane = tid & 63;
    const bool in = tid < 256;
    const int dir = (tid >> 7) & 1, code = tid & 127;           // dir is wave-uniform
    const bool active = in && (dir == 0 ? ROW : COL);
    const bool sr_r = ROW && G.sr_row, sr_c = COL && G.sr_col;
    const bool sr_dir = dir == 0 ? sr_r : sr_c;
    const float g = dir ? g_c : g_r;
    uint32_t* const sh_none = sh;
    uint32_t* const sh_fail = sh + 4;                            // [dir * 8 + m]: bit c, candidate c fails
    float* const sh_sr = reinterpret_cast<float*>(sh + 20);     // [dir * 8 + m]: the multiplier, or < 0
    // candidates of representative (jd, m)
    auto rep = [&](int jd, int m, float (&ym)[3]) {
        float d = (1.0f + (float)m * 0.125f) * (jd ? g_c : g_r);
        float y = 1.0f / d;
        if (jd) { d *= 4.0f; y *= 0.25f; }
        const uint32_t yb = __builtin_bit_cast(uint32_t, y);
        ym[0] = y;
        ym[1] = __builtin_bit_cast(float, yb - 1u);
        ym[2] = __builtin_bit_cast(float, yb + 1u);
        return d;
    };
    if (sr_r || sr_c) {                                          // uniform over the work-group
        if (tid < 16) sh_fail[tid] = 0u;
        __syncthreads();
        // a wave's 64 pairs share one representative (128 per representative)
        for (int idx = tid; idx < 16 * 128; idx += (int)blockDim.x) {
            const int job = idx >> 7, jd = job >> 3;
            if (!(jd == 0 ? sr_r : sr_c)) continue;
            float ym[3];
            const float d = rep(jd, job & 7, ym);
            const float u = 1.0f + (float)(idx & 127) * 0x1p-7f;
            const uint32_t want = __builtin_bit_cast(uint32_t, div_rn(u, d, ym[0])) >> 14;
            uint32_t f = 0;
#pragma unroll
            for (int c = 0; c < 3; ++c) f |= ((__builtin_bit_cast(uint32_t, u * ym[c]) >> 14) != want ? 1u : 0u) << c;
            f = (__ballot(f & 1u) ? 1u : 0u) | (__ballot(f & 2u) ? 2u : 0u) | (__ballot(f & 4u) ? 4u : 0u);
            if (lane == 0 && f) atomicOr(sh_fail + job, f);
        }
        __syncthreads();
        if (tid < 16) {
            float ym[3];
            rep(tid >> 3, tid & 7, ym);
            const uint32_t f = sh_fail[tid];
            sh_sr[tid] = !(f & 1u) ? ym[0] : !(f & 2u) ? ym[1] : !(f & 4u) ? ym[2] : -1.0f;
        }
        __syncthreads();
    }
    float rep_ym = 0.0f;
    if (active && !sr_dir && lane < 8) {
        float d = (1.0f + (float)lane * 0.125f) * g;
        float y = 1.0f / d;
        if (dir) { d *= 4.0f; y *= 0.25f; }
        rep_ym = product_multiplier(d, y);
    }
    float4 ent = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    bool none = false;
    if (active) {
        const float v = e4m3_value((uint32_t)code);
        const uint32_t vb = __builtin_bit_cast(uint32_t, v);
        const int m = (int)((vb >> 20) & 7), ex = (int)((vb >> 23) & 0xFF) - 127;
        const float cls_ym = __shfl(rep_ym, m, 64);
        if (code == 0 || code == 127) {
            ent = table_entry(code, g, dir == 1);
        } else {
            float d = v * g, y = 1.0f / d;
            float rd = (1.0f + (float)m * 0.125f) * g, ry = 1.0f / rd;
            if (dir == 1) { d *= 4.0f; y *= 0.25f; rd *= 4.0f; ry *= 0.25f; }
            const bool scaled = g < 0x1p100f && d == __builtin_ldexpf(rd, ex) && y == __builtin_ldexpf(ry, -ex);
            float ym;
            if (sr_dir)
                ym = scaled ? __builtin_ldexpf(sh_sr[dir * 8 + m], -ex) : -y;
            else
                ym = scaled ? __builtin_ldexpf(cls_ym, -ex) : product_multiplier(d, y);
            ent = make_float4(d, y, ym, k_keep_codes());
        }
        none = ent.z < 0.0f;
    }
    const bool any = __ballot(none) != 0;
    if (in && lane == 0) sh_none[tid >> 6] = any ? 1u : 0u;
    __syncthreads();
    if (active) {
        if (code == 127) ent.x = (sh_none[2 * dir] | sh_none[2 * dir + 1]) ? 1.0f : 0.0f;
        G.tables[(s * 2 + dir) * 128 + code] = ent;
        if (tab) tab[dir][code] = ent;
    }
}

// The amax pass over bands of kAmaxRows = 16 rows: a 256-thread work-group takes
// 16 rows x kAmaxCols = 1024 columns, each thread 4 adjacent columns of all 16 rows
// (16 loads of 8 bytes), so a wave's load instruction reads 512 contiguous bytes of
// one row and the 16-point RHT of a column block runs inside the lane.  About 50
// VGPRs: 8 waves per SIMD, every work-group of a 16384 x 4096 call resident in two
// rounds (with 8 columns per thread, 93 VGPRs and 5 waves per SIMD, the pass took
// 27.0 against 24.5 us, MI355X).  The work-group writes one partial, the (row,
// column) maxima of its band, with an ordinary store; nothing in this kernel reads
// them (the scales kernel that follows on the stream does), so no work-group waits
// for another and the kernel leaves no state behind.  Partial p = band * n_chunks +
// chunk: bits 16..31 the BF16 bits of max |x| (NaN-free), bits 32..63 the FP32 bits
// of max |H16 D x| (NaN-free, before the 1/4 and the BF16 rounding).  Columns at
// or past k (the last chunk when k % 1024 != 0) are not read.  The loads are
// ordinary ones, not non-temporal: this pass alone is faster with the non-temporal
// hint (22.3 against 24.7 us on the 16384 x 4096 call), but the input then does not
// stay in the Infinity Cache, and the quant pass's second read costs 8.5 us more
// (the call: 78.9 against 72.9 us).
template <bool ROW, bool COL>
__global__ __launch_bounds__(256) void k_nvfp4_amax(const Nvfp4Group G, int n_chunks) {
    __shared__ uint32_t red[2][4];
    const int tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int band = (int)blockIdx.x / n_chunks, chunk = (int)blockIdx.x - band * n_chunks;
    const int64_t c0 = (int64_t)chunk * kAmaxCols + tid * (2 * kAmaxWords);
    uint32_t mr = 0;
    float mc = 0.0f;
    if (c0 < G.k) {
        const uint16_t* base = G.x + (int64_t)band * 16 * G.k + c0;
        uint32_t v[16][kAmaxWords];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            if constexpr (kAmaxWords == 4) {
                const uint4 q = *reinterpret_cast<const uint4*>(base + (int64_t)t * G.k);
                v[t][0] = q.x; v[t][1] = q.y; v[t][2] = q.z; v[t][3] = q.w;
            } else {
                const uint2 q = *reinterpret_cast<const uint2*>(base + (int64_t)t * G.k);
                v[t][0] = q.x; v[t][1] = q.y;
            }
        }
        if (ROW) {
            uint32_t m = 0;
#pragma unroll
            for (int t = 0; t < 16; ++t)
#pragma unroll
                for (int i = 0; i < kAmaxWords; ++i) m = absmax_pk(m, v[t][i]);
            m = fold_pk(m);
            if (m > 0x7F80u) {                       // a NaN: the maximum without it
                m = 0;
#pragma unroll
                for (int t = 0; t < 16; ++t)
#pragma unroll
                    for (int i = 0; i < kAmaxWords; ++i) m = absmax_nonan_pairs(m, v[t][i]);
            }
            mr = m;
        }
        if (COL) {
#pragma unroll
            for (int j = 0; j < 2 * kAmaxWords; ++j) {
                float f[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const uint32_t wd = v[t][j >> 1];
                    const uint32_t neg = sign_of_row(G.sign_mask, t);
                    f[t] = (j & 1) ? hi_signed(wd, neg) : lo_signed(wd, neg);
                }
                // stages h = 1, 2, 4; the last stage is not formed: for its pair (a, b)
                // the larger of |fl(a + b)| and |fl(a - b)| is fl(|a| + |b|) (rounding is
                // monotone and symmetric)
#pragma unroll
                for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        if (i & h) continue;
                        const float x0 = f[i], x1 = f[i + h];
                        f[i] = x0 + x1;
                        f[i + h] = x0 - x1;
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i)      // NaN values are quiet here, and max ignores them
                    mc = __builtin_fmaxf(mc, __builtin_fabsf(f[i]) + __builtin_fabsf(f[i + 8]));
            }
        }
    }
    mr = wave_max_u32(mr);
    mc = wave_max_f32(mc);
    if (lane == 0) {
        red[0][w] = mr;
        red[1][w] = __builtin_bit_cast(uint32_t, mc);
    }
    __syncthreads();
    if (tid == 0) {
        uint32_t r = 0, c = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r = red[0][i] > r ? red[0][i] : r;
            c = red[1][i] > c ? red[1][i] : c;                    // non-negative FP32: ordered as integers
        }
        G.partials[blockIdx.x] = (uint64_t)(r << 16) | ((uint64_t)c << 32);
    }
}

// Tensor scales and tables of every section (one 1024-thread work-group per
// section), from the partials of the amax pass (ppt partials per 128-row token
// tile, in row order) or, GIVEN,
// from the caller-supplied maxima.  Measured: the maxima out are the measured
// ones (an empty section: 0).  GIVEN: they are zeroed here, and the quant kernel
// raises them.
constexpr int kScalesThreads = 1024;
template <bool ROW, bool COL, bool GIVEN>
__global__ __launch_bounds__(kScalesThreads) void k_nvfp4_scales(const Nvfp4Group G, int ppt) {
    __shared__ uint32_t red[2][kScalesThreads / 64];
    __shared__ uint32_t sh_tab[kTableLdsWords];
    const int s = blockIdx.x, tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6;
    float a_r = 0.0f, a_c = 0.0f;
    if (GIVEN) {
        a_r = ROW ? G.amax_in_row[s] : 0.0f;
        a_c = COL ? G.amax_in_col[s] : 0.0f;
    } else {
        const int first = G.tt_start[s] * ppt;
        const int n = (G.tt_start[s + 1] - G.tt_start[s]) * ppt;
        uint32_t ar = 0, ac = 0;
        // 8 loads in flight per thread per round
        for (int i0 = tid; i0 < n; i0 += kScalesThreads * 8) {
            uint64_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = i0 + kScalesThreads * u < n ? G.partials[first + i0 + kScalesThreads * u] : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                ar = (uint32_t)v[u] > ar ? (uint32_t)v[u] : ar;
                ac = (uint32_t)(v[u] >> 32) > ac ? (uint32_t)(v[u] >> 32) : ac;
            }
        }
        ar = wave_max_u32(ar);
        ac = wave_max_u32(ac);
        if (lane == 0) {
            red[0][w] = ar;
            red[1][w] = ac;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kScalesThreads / 64; ++i) {
            ar = red[0][i] > ar ? red[0][i] : ar;
            ac = red[1][i] > ac ? red[1][i] : ac;
        }
        // max |BF16(y/4)| over the section = BF16(max |y| / 4) (both roundings are
        // monotone)
        a_r = __builtin_bit_cast(float, ar);
        a_c = lo_bf16(pack_bf16(__builtin_bit_cast(float, ac) * 0.25f, 0.0f));
    }
    const float g_r = ROW ? tensor_scale(a_r) : 0.0f, g_c = COL ? tensor_scale(a_c) : 0.0f;
    if (tid == 0) {
        if (ROW) G.row_global[s] = g_r;
        if (COL) G.col_global[s] = g_c;
        if (ROW && G.amax_out_row) G.amax_out_row[s] = GIVEN ? 0.0f : a_r;
        if (COL && G.amax_out_col) G.amax_out_col[s] = GIVEN ? 0.0f : a_c;
    }
    build_tables_wg<ROW, COL>(G, s, g_r, g_c, nullptr, sh_tab, tid);
}

// LDS of one work-group's quant passes (W waves, one tile each).
template <int W>
struct QuantLds {
    float4 tab[2][128];                                 // the section's scale tables
    // Column codes / scales of a tile by (column, 16-row block): 64 + 8 bytes per
    // column, with one more slot after every 16 columns so that the 8 lane groups
    // that write columns 16 apart use both halves of the LDS banks.
    uint2 codes[W][kTileCols * 8 + 8 * 8];
    uint8_t sc[W][kTileCols * 8 + 8 * 8];
    uint8_t rsc[kTileRows * 8 * W];                      // row scales of the work-group's tiles
    uint32_t amax[2][W];                                 // AOUT: each wave's measured maxima (FP32 bits)
};

// Every output of wave w's tile (token tile T, column tile C of section s), the tile
// in p and the section's tables in L.tab: the row pass first (a row block needs only
// its own row, so it starts on the rows that have arrived), then the column pass
// (all 16 rows of each column block), then FP8.  The W waves of a work-group take
// W adjacent column tiles of the same rows, so that each row's W x 8 scale bytes
// leave as one piece: scattered 8-byte pieces cost the memory system about three
// times as much per byte.  AOUT: the section maxima are supplied, and the measured
// ones are wanted out.
// tid: threadIdx.x (a caller that loops may pass it laundered, so that no address
// derived from it is hoisted out of the loop and kept live through the passes).
template <bool ROW, bool COL, bool FP8, bool SR, bool AOUT, int W>
__device__ __forceinline__ void quant_passes(const Nvfp4Group& G, uint4 (&p)[16][2], QuantLds<W>& L, int w, int s,
                                             int T, int C, int tid) {
    const int lane = tid & 63;
    const int tb = lane >> 3, cc = lane & 7;
    const int64_t k = G.k;
    uint2* const lds_codes = L.codes[w];
    uint8_t* const lds_sc = L.sc[w];
    const int tt0 = G.tt_start[s];
    const int ms = (G.tt_start[s + 1] - tt0) * kTileRows;           // section rows
    const int T_local = T - tt0;
    const int64_t row0 = (int64_t)T * kTileRows + tb * 16;           // group-relative
    const int64_t c0 = (int64_t)C * kTileCols + cc * 16;
    const int64_t r_local0 = (int64_t)T_local * kTileRows + tb * 16;  // section-local
    const u32x4 no_rnd = {0, 0, 0, 0};
    if (ROW) {
        const float g_r = L.tab[0][0].x, yg_r = L.tab[0][0].y;
        const float4* tab_r = L.tab[0];
        uint8_t* const rc_tile = G.row_codes + (int64_t)T * kTileRows * (k >> 1) + (int64_t)C * (kTileCols / 2);
        const float ra = row_pass<SR, 8 * W>(G, p, s, c0, r_local0, g_r, yg_r, tab_r, tab_r[127].x != 0.0f,
                                             L.rsc + 8 * w, rc_tile, tid);
        if (W > 1) {
            __syncthreads();
        } else {
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
        // 128 rows x 8W bytes: W consecutive threads store one row's piece.  Pieces of 32
        // bytes (W = 4) go non-temporally like the codes (1 us faster in this kernel);
        // 8-byte pieces were much slower that way, as the column scales showed.
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int i = it * 64 * W + tid;
            const int r = i / W, part = i - r * W;
            const uint2 v = *reinterpret_cast<const uint2*>(L.rsc + r * 8 * W + part * 8);
            uint8_t* const dst = G.row_scales + ((int64_t)T * kTileRows + r) * (k >> 4) + (int64_t)(C - w) * 8 + part * 8;
            if (W >= 4)
                __builtin_nontemporal_store(u32x2v{v.x, v.y}, reinterpret_cast<u32x2v*>(dst));
            else
                *reinterpret_cast<uint2*>(dst) = v;
        }
        if (AOUT) {
            // supplied maxima: measure this call's for the caller's next step
            const float wm = wave_max_f32(ra);
            if (lane == 0) L.amax[0][w] = __builtin_bit_cast(uint32_t, wm);
        }
        launder(p);
    }

    if (COL) {
        const float g_c = L.tab[1][0].x, yg_c = L.tab[1][0].y;
        const float4* tab_c = L.tab[1];
        const uint32_t mask = G.sign_mask;
        float col_amax = 0.0f;                       // max |H16 D x| of the lane's blocks (NaNs aside)
        auto put = [&](int j, const BlockOut& o) {
            lds_codes[(cc * 17 + j) * 8 + tb] = o.codes;
            lds_sc[(cc * 17 + j) * 8 + tb] = (uint8_t)o.scale;
        };
        if (SR && G.sr_col) {
            const int64_t b_local = r_local0 >> 4;                  // section-local 16-row block
            // kSrChains columns' Philox chains drawn together, by product or by
            // division (as in the row pass)
            auto cols = [&](auto enc) {
#pragma unroll
                for (int j0 = 0; j0 < 16; j0 += kSrChains) {
                    u32x4 rnd[kSrChains];
#pragma unroll
                    for (int i = 0; i < kSrChains; ++i)
                        rnd[i] = block_random(G.seed, G.col_off[s], (uint64_t)((c0 + j0 + i) * (int64_t)(ms >> 4) + b_local));
#pragma unroll
                    for (int i = 0; i < kSrChains; ++i) {
                        const BlockOut o = column_block<decltype(enc)::value>(p, j0 + i, mask, g_c, yg_c, tab_c, rnd[i]);
                        put(j0 + i, o);
                        if (AOUT) col_amax = __builtin_fmaxf(col_amax, o.amax);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            if (tab_c[127].x != 0.0f)
                cols(EncTag<Enc::Sr>{});
            else
                cols(EncTag<Enc::SrMul>{});
        } else if (tab_c[127].x != 0.0f) {
            // the section's column table has a scale code without a multiplier:
            // exact division for the whole pass
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const BlockOut o = column_block<Enc::Div>(p, j, mask, g_c, yg_c, tab_c, no_rnd);
                put(j, o);
                if (AOUT) col_amax = __builtin_fmaxf(col_amax, o.amax);
                if (j & 1) __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // No branch in this loop, so the scheduler can overlap neighbouring columns.
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const BlockOut o = column_block<Enc::Mul>(p, j, mask, g_c, yg_c, tab_c, no_rnd);
                put(j, o);
                if (AOUT) col_amax = __builtin_fmaxf(col_amax, o.amax);
                if (j & 1) __builtin_amdgcn_sched_barrier(0);   // two columns at a time: bounds registers
            }
        }
        // the LDS region is this wave's own: order its writes before the reads below
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        uint8_t* codes_s = G.col_codes + k * (int64_t)tt0 * kTileRows / 2;
        uint8_t* scales_s = G.col_scales + k * (int64_t)tt0 * kTileRows / 16;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int idx = it * 64 + lane;
            const int col = idx >> 2, part = idx & 3;
            const uint4 v = *reinterpret_cast<const uint4*>(&lds_codes[(col + (col >> 4)) * 8 + part * 2]);
            // Non-temporal: the codes (two thirds of the output bytes) stream out during
            // this kernel instead of staying dirty in the caches, where the next call's
            // first kernel would have to write them back.  The column scales, 8-byte
            // pieces, are slower this way.
            __builtin_nontemporal_store(u32x4v{v.x, v.y, v.z, v.w},
                                        reinterpret_cast<u32x4v*>(codes_s + ((int64_t)C * kTileCols + col) * (ms >> 1) +
                                                                  T_local * 64 + part * 16));
        }
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int col = it * 64 + lane;
            const uint2 v = *reinterpret_cast<const uint2*>(&lds_sc[(col + (col >> 4)) * 8]);
            *reinterpret_cast<uint2*>(scales_s + ((int64_t)C * kTileCols + col) * (ms >> 4) + T_local * 8) = v;
        }
        if (AOUT) {
            // supplied maxima: measure this call's, max |BF16(y/4)| = BF16(max |y|) / 4
            const float wm = 0.25f * round_bf16(wave_max_f32(col_amax));
            if (lane == 0) L.amax[1][w] = __builtin_bit_cast(uint32_t, wm);
        }
        launder(p);
    }

    if (FP8) {
        // FP8 1x128 of each row: the group's max |x| without NaNs over 8 lanes
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int64_t row = row0 + t;
            float u[16];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                u[2 * i] = lo_bf16(P(t, i));
                u[2 * i + 1] = hi_bf16(P(t, i));
            }
            uint32_t acc = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc = absmax_pk(acc, P(t, i));
            uint32_t mf = fold_pk(acc);
            const bool nan = mf > 0x7F80u;
            if (nan) {
                mf = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) mf = absmax_pk_nonan(mf, P(t, i));
            }
            mf = group8_max_u32(mf);
            const float amax = bf16_mag(mf);
            const float sf = (amax > k_floor() ? amax : k_floor()) * k_inv448();
            const float yf = 1.0f / sf, sd = fp8_divisor(sf);
            const bool fix = nan || sf == __builtin_inff();     // NaN codes: NaN values, or inf / inf
            uint32_t c4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c4[j] = e4m3_pack4(div_rn(u[4 * j], sd, yf), div_rn(u[4 * j + 1], sd, yf),
                                   div_rn(u[4 * j + 2], sd, yf), div_rn(u[4 * j + 3], sd, yf));
                if (fix) {
                    // a NaN element: the conversion gives 0xFF, the format's NaN code is 0x7F
                    const uint32_t cj = c4[j];
                    const uint32_t ff = cj & (cj >> 1) & (cj >> 2) & (cj >> 3) & (cj >> 4) & (cj >> 5) &
                                        (cj >> 6) & (cj >> 7) & 0x01010101u;
                    c4[j] = cj ^ (ff * 0x80u);
                }
            }
            // non-temporal, as the NVFP4 codes
            __builtin_nontemporal_store(u32x4v{c4[0], c4[1], c4[2], c4[3]},
                                        reinterpret_cast<u32x4v*>(G.fp8_codes + row * k + c0));
            if (cc == 0) G.fp8_scales[row * (k >> 7) + C] = sf;
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    if (AOUT && (G.amax_out_row || G.amax_out_col)) {
        // one atomic maximum per direction for the work-group (non-negative FP32 orders
        // like its bits): same-address atomics are served one at a time, and one per
        // wave cost the call about as much as its arithmetic
        if (W > 1) {
            __syncthreads();
        } else {
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
        if (tid == 0) {
            uint32_t mr = 0, mc = 0;
#pragma unroll
            for (int i = 0; i < W; ++i) {
                mr = L.amax[0][i] > mr ? L.amax[0][i] : mr;
                mc = L.amax[1][i] > mc ? L.amax[1][i] : mc;
            }
            if (ROW && G.amax_out_row)
                __hip_atomic_fetch_max(reinterpret_cast<uint32_t*>(G.amax_out_row + s), mr, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            if (COL && G.amax_out_col)
                __hip_atomic_fetch_max(reinterpret_cast<uint32_t*>(G.amax_out_col + s), mc, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Lane (tb, cc) of a tile loads rows 16 tb .. 16 tb + 15, columns 16 cc .. 16 cc + 15
// (two 16-byte loads per row).  NT: non-temporal, for the input's last reader.
template <bool NT>
__device__ __forceinline__ void load_tile(uint4 (&p)[16][2], const uint16_t* base, int64_t k) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        if (NT) {
            p[t][0] = nt_load16(base + t * k);
            p[t][1] = nt_load16(base + t * k + 8);
        } else {
            p[t][0] = *reinterpret_cast<const uint4*>(base + t * k);
            p[t][1] = *reinterpret_cast<const uint4*>(base + t * k + 8);
        }
    }
}

// The quant pass of the three-kernel call: one wave per tile, W waves per work-group over W
// adjacent column tiles of the same rows (k / 128 a multiple of W).
template <bool ROW, bool COL, bool FP8, bool SR, bool AOUT, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2))) void k_nvfp4_quant(const Nvfp4Group G) {
    const int lane = threadIdx.x & 63;
    const int w = W > 1 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) : 0;   // wave-uniform
    const int b = (int)blockIdx.x * W + w;
    const int T = b / G.n_ctiles, C = b - T * G.n_ctiles;
    const int s = section_of(G, T);
    const int tb = lane >> 3, cc = lane & 7;
    const int64_t k = G.k;
    const uint16_t* base = G.x + ((int64_t)T * kTileRows + tb * 16) * k + (int64_t)C * kTileCols + cc * 16;
    // The section's scale tables are loaded before the tile: loads complete in order,
    // so waiting for the table does not wait for the tile, and the first pass can
    // start on the rows that have arrived.
    const float4* src = G.tables + s * 256;
    const float4 te0 = ROW ? src[lane] : float4{}, te1 = ROW ? src[64 + lane] : float4{};
    const float4 te2 = COL ? src[128 + lane] : float4{}, te3 = COL ? src[192 + lane] : float4{};
    __builtin_amdgcn_sched_barrier(0);
    // Non-temporal without the FP8 output: this kernel is the input's last reader
    // (quant 51.7 -> 45.6 us on 16384 x 4096, no worse at 65536 x 7168).  With the FP8
    // output's non-temporal stores as well, the hint cost 10 % on 65536 x 7168 (461 ->
    // 510 us) and nothing on 16384 x 4096: plain loads there.
    uint4 p[16][2];
    load_tile<!FP8>(p, base, k);
    __builtin_amdgcn_sched_barrier(0);

    __shared__ QuantLds<W> L;
    // every wave writes the whole table (the same values): no wave reads an entry
    // before its own write
    if (ROW) { L.tab[0][lane] = te0; L.tab[0][64 + lane] = te1; }
    if (COL) { L.tab[1][lane] = te2; L.tab[1][64 + lane] = te3; }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    quant_passes<ROW, COL, FP8, SR, AOUT, W>(G, p, L, w, s, T, C, (int)threadIdx.x);
}

#undef P

// Launch of the quant kernel for one flag combination (instantiated by the
// mxq_nvfp4_quant_*.hip units, one per (SR, AOUT) pair).
template <bool SR, bool AOUT>
hipError_t launch_quant_variant(const Nvfp4Group& g, uint32_t flags, hipStream_t stream) {
    if (g.n_ctiles % 4 == 0) {
        const dim3 grid((unsigned)(g.total_tiles / 4)), block(256);
        switch (flags & 7u) {
            case 1: hipLaunchKernelGGL((k_nvfp4_quant<true, false, false, SR, AOUT, 4>), grid, block, 0, stream, g); break;
            case 2: hipLaunchKernelGGL((k_nvfp4_quant<false, true, false, SR, AOUT, 4>), grid, block, 0, stream, g); break;
            case 3: hipLaunchKernelGGL((k_nvfp4_quant<true, true, false, SR, AOUT, 4>), grid, block, 0, stream, g); break;
            case 5: hipLaunchKernelGGL((k_nvfp4_quant<true, false, true, SR, AOUT, 4>), grid, block, 0, stream, g); break;
            case 6: hipLaunchKernelGGL((k_nvfp4_quant<false, true, true, SR, AOUT, 4>), grid, block, 0, stream, g); break;
            case 7: hipLaunchKernelGGL((k_nvfp4_quant<true, true, true, SR, AOUT, 4>), grid, block, 0, stream, g); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    const dim3 grid((unsigned)g.total_tiles), block(64);
    switch (flags & 7u) {
        case 1: hipLaunchKernelGGL((k_nvfp4_quant<true, false, false, SR, AOUT, 1>), grid, block, 0, stream, g); break;
        case 2: hipLaunchKernelGGL((k_nvfp4_quant<false, true, false, SR, AOUT, 1>), grid, block, 0, stream, g); break;
        case 3: hipLaunchKernelGGL((k_nvfp4_quant<true, true, false, SR, AOUT, 1>), grid, block, 0, stream, g); break;
        case 5: hipLaunchKernelGGL((k_nvfp4_quant<true, false, true, SR, AOUT, 1>), grid, block, 0, stream, g); break;
        case 6: hipLaunchKernelGGL((k_nvfp4_quant<false, true, true, SR, AOUT, 1>), grid, block, 0, stream, g); break;
        case 7: hipLaunchKernelGGL((k_nvfp4_quant<true, true, true, SR, AOUT, 1>), grid, block, 0, stream, g); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mxq
