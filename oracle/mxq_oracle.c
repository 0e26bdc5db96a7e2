/*
 * mxq_oracle.c -- CPU oracle (test infrastructure only; see mxq_oracle.h).
 *
 * Every function restates a definition: the OCP E4M3FN / E2M1 formats, the
 * bfloat16 format, the Walsh-Hadamard butterfly, the FP8 1x128 recipe of the
 * onnxruntime QMoE PR (Description), the NVFP4 two-level scaling with the
 * per-section reading of the tensor scale, and Philox4x32-10 from the SC'11 paper.
 * Nothing here is tuned; clarity wins over speed wherever they disagree.
 */
#include "mxq_oracle.h"

#include <math.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Constants, each the binary32 value nearest to the real number named.      */
/* ------------------------------------------------------------------------ */
/* IEEE division and square root are correctly rounded, so these are exact
 * statements of F(r).  sqrtf(2)/16 is F(sqrt 2)/16 = F(1/sqrt 128) because
 * dividing by 16 is exact. */
static float f_one_over(float d) { volatile float one = 1.0f; return one / d; }
static float F_1E_10(void)      { return 1e-10f; }
static float F_1_OVER_448(void) { return f_one_over(448.0f); }
static float F_1_OVER_2688(void){ return f_one_over(2688.0f); }
static float F_1_OVER_6(void)   { return f_one_over(6.0f); }
static float F_C128(void)       { volatile float two = 2.0f; return sqrtf(two) / 16.0f; }

static uint32_t f32_bits(float v) { uint32_t b; memcpy(&b, &v, 4); return b; }
static float    bits_f32(uint32_t b) { float v; memcpy(&v, &b, 4); return v; }

/* ------------------------------------------------------------------------ */
/* bfloat16                                                                  */
/* ------------------------------------------------------------------------ */
float oracle_bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

/* Nearest bfloat16 with ties to the even significand.  For a finite v, the two
 * candidates are v with its low 16 bits cleared (same sign, magnitude rounded
 * toward zero) and the next bfloat16 away from zero.  Comparing the dropped
 * 16 bits with one half of a bfloat16 ulp (0x8000) decides; a carry out of the
 * mantissa moves to the next binade (or to infinity), which is correct. */
uint16_t oracle_f32_to_bf16(float v)
{
    uint32_t b = f32_bits(v);
    if (isnan(v)) return (uint16_t)((b >> 16) | 0x0040u); /* stays a (quiet) NaN */
    uint32_t lo    = b & 0xFFFF0000u;
    uint32_t rest  = b & 0x0000FFFFu;
    uint32_t up    = lo + 0x00010000u;
    uint32_t pick;
    if (rest < 0x8000u)      pick = lo;
    else if (rest > 0x8000u) pick = up;
    else                     pick = ((lo >> 16) & 1u) ? up : lo; /* tie: even significand */
    return (uint16_t)(pick >> 16);
}

/* ------------------------------------------------------------------------ */
/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;  */
/* S.1111.111 is NaN; largest finite value 448.                              */
/* ------------------------------------------------------------------------ */
static double e4m3_magnitude(int c) /* c in 0..126 */
{
    int e = (c >> 3) & 15, m = c & 7;
    if (e == 0) return ldexp((double)m / 8.0, -6);
    return ldexp(1.0 + (double)m / 8.0, e - 7);
}

float oracle_e4m3_value(uint8_t code)
{
    int c = code & 0x7F;
    if (c == 0x7F) return NAN;
    double m = e4m3_magnitude(c);
    return (float)((code & 0x80) ? -m : m);
}

/* Nearest code among 0x00..0x7E (magnitudes increase with the code), ties to
 * the even code; |v| >= 448 saturates to 0x7E; NaN -> 0x7F; the sign bit of v
 * is kept, so -0 and negative values that round to zero give 0x80. */
uint8_t oracle_e4m3_encode(float v)
{
    if (isnan(v)) return 0x7F;
    uint8_t s = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(s | 0x7E);
    /* bracket: lo = largest code with magnitude <= a (binary search) */
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (e4m3_magnitude(mid) <= a) lo = mid; else hi = mid - 1;
    }
    if (e4m3_magnitude(lo) == a) return (uint8_t)(s | lo);
    int up = lo + 1;                               /* exists because a < 448 */
    double twice_a = 2.0 * a;                      /* exact in double */
    double sum = e4m3_magnitude(lo) + e4m3_magnitude(up); /* exact in double */
    int c;
    if (twice_a < sum)      c = lo;
    else if (twice_a > sum) c = up;
    else                    c = (lo % 2 == 0) ? lo : up;
    return (uint8_t)(s | c);
}

/* ------------------------------------------------------------------------ */
/* E2M1 (FP4): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7; bit 3 is */
/* the sign.                                                                 */
/* ------------------------------------------------------------------------ */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

float oracle_e2m1_value(uint8_t code)
{
    double m = E2M1_MAG[code & 7];
    return (float)((code & 8) ? -m : m);
}

/* Nearest code, ties to the even code, |v| >= 6 saturates to 7, sign kept. */
uint8_t oracle_e2m1_encode(float v)
{
    uint8_t s = signbit(v) ? 0x8 : 0x0;
    double a = fabs((double)v);
    if (!(a < 6.0)) return (uint8_t)(s | 7); /* also NaN: callers never pass one */
    int lo = 0;
    for (int c = 1; c < 8; ++c) if (E2M1_MAG[c] <= a) lo = c;
    if (E2M1_MAG[lo] == a) return (uint8_t)(s | lo);
    int up = lo + 1;
    double twice_a = 2.0 * a, sum = E2M1_MAG[lo] + E2M1_MAG[up];
    int c;
    if (twice_a < sum)      c = lo;
    else if (twice_a > sum) c = up;
    else                    c = (lo % 2 == 0) ? lo : up;
    return (uint8_t)(s | c);
}

/* Stochastic rounding on the E2M1 grid with 8 random bits r: the magnitude is
 * written a = (k + f) * D with D the local grid spacing (0.5 below 2, 1 below 4,
 * 2 above); with F = floor(256 f) the value rounds up iff F + r >= 256, so it
 * rounds up with probability F/256.  Values at or above 6 saturate. */
uint8_t oracle_e2m1_encode_sr(float v, uint8_t r)
{
    uint8_t s = signbit(v) ? 0x8 : 0x0;
    float a = fabsf(v);
    if (!(a < 6.0f)) return (uint8_t)(s | 7);
    float D = (a < 2.0f) ? 0.5f : (a < 4.0f) ? 1.0f : 2.0f;
    float u = a / D;                 /* exact: D is a power of two */
    float k = floorf(u);
    float f = u - k;                 /* exact */
    int F = (int)floorf(256.0f * f); /* exact product */
    if (F + (int)r >= 256) k += 1.0f;
    double mag = (double)k * (double)D; /* on the grid by construction */
    for (int c = 0; c < 8; ++c)
        if (E2M1_MAG[c] == mag) return (uint8_t)(s | c);
    return (uint8_t)(s | 7); /* unreachable */
}

float oracle_amax(const float* v, int64_t n)
{
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        if (isnan(v[i])) continue;
        float a = fabsf(v[i]);
        if (a > m) m = a;
    }
    return m;
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11): ten rounds of the 4x32 S-box with   */
/* multipliers 0xD2511F53 / 0xCD9E8D57; the key is bumped by the Weyl        */
/* constants 0x9E3779B9 / 0xBB67AE85 between rounds.                         */
/* ------------------------------------------------------------------------ */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* 16 random bytes for one 1x16 block: counter (lo(off), hi(off), lo(beta),
 * hi(beta)), key (lo(seed), hi(seed)); byte t of the block is byte t&3 of
 * output word t>>2. */
static void block_random_bytes(uint64_t seed, uint64_t off, uint64_t beta, uint8_t r[16])
{
    uint32_t ctr[4] = {(uint32_t)off, (uint32_t)(off >> 32), (uint32_t)beta, (uint32_t)(beta >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    oracle_philox4x32_10(ctr, key, w);
    for (int t = 0; t < 16; ++t) r[t] = (uint8_t)((w[t >> 2] >> (8 * (t & 3))) & 0xFFu);
}

/* ------------------------------------------------------------------------ */
/* Walsh-Hadamard transform, Sylvester order, stages h = 1, 2, 4, ...        */
/* ------------------------------------------------------------------------ */
void oracle_wht(const float* in, int n, uint32_t sign_mask, float c, float* out)
{
    float v[128];
    for (int i = 0; i < n; ++i) {
        int flip = (i < 32) && ((sign_mask >> i) & 1u);
        v[i] = flip ? -in[i] : in[i];
    }
    for (int h = 1; h < n; h *= 2) {
        for (int i = 0; i < n; ++i) {
            if (i & h) continue;
            float a = v[i], b = v[i + h];
            v[i] = a + b;
            v[i + h] = a - b;
        }
    }
    for (int i = 0; i < n; ++i) {
        float scaled = v[i] * c;
        out[i] = oracle_bf16_to_f32(oracle_f32_to_bf16(scaled));
    }
}

/* ------------------------------------------------------------------------ */
/* FP8 1x128                                                                 */
/* ------------------------------------------------------------------------ */
float oracle_fp8_group(const float* x, uint8_t* codes)
{
    float a = oracle_amax(x, 128);
    float floor_ = F_1E_10();
    float s = ((a > floor_) ? a : floor_) * F_1_OVER_448();
    for (int i = 0; i < 128; ++i) {
        float q = x[i] / s;
        codes[i] = oracle_e4m3_encode(q);
    }
    return s;
}

void oracle_quant_fp8_1x128(const uint16_t* x, int64_t m, int64_t k, int64_t ldx,
                            uint8_t* q, int64_t ldq, float* scales,
                            int64_t scale_stride_row, int64_t scale_stride_group)
{
    float g[128];
    for (int64_t r = 0; r < m; ++r) {
        for (int64_t gi = 0; gi < k / 128; ++gi) {
            for (int i = 0; i < 128; ++i) g[i] = oracle_bf16_to_f32(x[r * ldx + gi * 128 + i]);
            float s = oracle_fp8_group(g, q + r * ldq + gi * 128);
            scales[r * scale_stride_row + gi * scale_stride_group] = s;
        }
    }
}

void oracle_hadamard_quant_fp8(const uint16_t* pe, int64_t ld_pe, int32_t d_pe,
                               const uint16_t* nope, int64_t ld_nope, int64_t m,
                               uint8_t* q, float* scales)
{
    float v[128], y[128];
    float c = F_C128();
    for (int64_t r = 0; r < m; ++r) {
        for (int i = 0; i < d_pe; ++i)        v[i] = oracle_bf16_to_f32(pe[r * ld_pe + i]);
        for (int i = d_pe; i < 128; ++i)      v[i] = oracle_bf16_to_f32(nope[r * ld_nope + (i - d_pe)]);
        oracle_wht(v, 128, 0u, c, y);
        scales[r] = oracle_fp8_group(y, q + r * 128);
    }
}

/* ------------------------------------------------------------------------ */
/* NVFP4                                                                     */
/* ------------------------------------------------------------------------ */
float oracle_nvfp4_global_scale(float amax)
{
    float floor_ = F_1E_10();
    return ((amax > floor_) ? amax : floor_) * F_1_OVER_2688();
}

void oracle_nvfp4_block(const float* v, float g, const uint8_t* rbits,
                        uint8_t* scale_code, uint8_t* codes)
{
    for (int i = 0; i < 16; ++i) {
        if (isnan(v[i])) {              /* a NaN block has no finite encoding */
            *scale_code = 0x7F;
            for (int j = 0; j < 16; ++j) codes[j] = 0;
            return;
        }
    }
    float a  = oracle_amax(v, 16);
    float a6 = a * F_1_OVER_6();
    float t  = a6 / g;
    uint8_t sc = oracle_e4m3_encode(t);
    *scale_code = sc;
    /* Scale underflow: the block decodes to zero.  The NaN scale (t = inf / inf: an
     * infinite block amax over the infinite tensor scale of an infinite tensor
     * amax) has no finite decode: its block carries zero codes, as a NaN block does. */
    if (sc == 0x00 || sc == 0x7F) {
        for (int j = 0; j < 16; ++j) codes[j] = 0;
        return;
    }
    float d = oracle_e4m3_value(sc) * g;
    for (int i = 0; i < 16; ++i) {
        float q = v[i] / d;
        codes[i] = rbits ? oracle_e2m1_encode_sr(q, rbits[i]) : oracle_e2m1_encode(q);
    }
}

/* The 16 column-wise values of column c, 16-row block b of a section. */
static void column_block_values(const uint16_t* x, int64_t k, uint16_t sign_mask,
                                int64_t c, int64_t b, float* y)
{
    float col[16];
    for (int t = 0; t < 16; ++t) col[t] = oracle_bf16_to_f32(x[(16 * b + t) * k + c]);
    oracle_wht(col, 16, sign_mask, 0.25f, y);
}

void oracle_nvfp4_section_amax(const uint16_t* x, int64_t rows, int64_t k,
                               uint16_t sign_mask, float* amax_row, float* amax_col)
{
    float ar = 0.0f, ac = 0.0f, y[16];
    for (int64_t i = 0; i < rows * k; ++i) {
        float v = oracle_bf16_to_f32(x[i]);
        if (!isnan(v) && fabsf(v) > ar) ar = fabsf(v);
    }
    for (int64_t b = 0; b < rows / 16; ++b) {
        for (int64_t c = 0; c < k; ++c) {
            column_block_values(x, k, sign_mask, c, b, y);
            float m = oracle_amax(y, 16);
            if (m > ac) ac = m;
        }
    }
    *amax_row = ar;
    *amax_col = ac;
}

static void pack_nibbles(const uint8_t* codes16, uint8_t* out8)
{
    for (int j = 0; j < 8; ++j)
        out8[j] = (uint8_t)((codes16[2 * j] & 0xF) | ((codes16[2 * j + 1] & 0xF) << 4));
}

void oracle_nvfp4_section(const uint16_t* x, int64_t rows, int64_t k, uint16_t sign_mask,
                          uint32_t flags, float g_row, float g_col,
                          int use_sr_row, int use_sr_col, uint64_t seed,
                          uint64_t row_offset, uint64_t col_offset,
                          int64_t row_begin, int64_t row_end,
                          int64_t col_begin, int64_t col_end,
                          uint8_t* row_codes, uint8_t* row_scales,
                          uint8_t* col_codes, uint8_t* col_scales,
                          uint8_t* fp8_codes, float* fp8_scales)
{
    float v[128];
    uint8_t codes[16], rb[16], sc;
    if (flags & ORACLE_ROWWISE) {
        for (int64_t r = row_begin; r < row_end; ++r) {
            for (int64_t kb = 0; kb < k / 16; ++kb) {
                for (int t = 0; t < 16; ++t) v[t] = oracle_bf16_to_f32(x[r * k + 16 * kb + t]);
                if (use_sr_row) block_random_bytes(seed, row_offset, (uint64_t)(r * (k / 16) + kb), rb);
                oracle_nvfp4_block(v, g_row, use_sr_row ? rb : NULL, &sc, codes);
                row_scales[r * (k / 16) + kb] = sc;
                pack_nibbles(codes, row_codes + r * (k / 2) + 8 * kb);
            }
        }
    }
    if (flags & ORACLE_FP8_ROWWISE) {
        for (int64_t r = row_begin; r < row_end; ++r) {
            for (int64_t gi = 0; gi < k / 128; ++gi) {
                for (int i = 0; i < 128; ++i) v[i] = oracle_bf16_to_f32(x[r * k + 128 * gi + i]);
                fp8_scales[r * (k / 128) + gi] = oracle_fp8_group(v, fp8_codes + r * k + 128 * gi);
            }
        }
    }
    if (flags & ORACLE_COLUMNWISE) {
        for (int64_t c = col_begin; c < col_end; ++c) {
            for (int64_t b = 0; b < rows / 16; ++b) {
                column_block_values(x, k, sign_mask, c, b, v);
                if (use_sr_col) block_random_bytes(seed, col_offset, (uint64_t)(c * (rows / 16) + b), rb);
                oracle_nvfp4_block(v, g_col, use_sr_col ? rb : NULL, &sc, codes);
                col_scales[c * (rows / 16) + b] = sc;
                pack_nibbles(codes, col_codes + c * (rows / 2) + 8 * b);
            }
        }
    }
}

int oracle_group_rht_quant_nvfp4_amax(const uint16_t* x, int64_t k,
                                      const int64_t* split_sections, int64_t num_sections,
                                      uint16_t sign_mask, uint32_t flags, uint64_t seed,
                                      const uint64_t* row_offsets, const uint64_t* col_offsets,
                                      uint8_t* row_codes, uint8_t* row_scales, float* row_global,
                                      uint8_t* col_codes, uint8_t* col_scales, float* col_global,
                                      uint8_t* fp8_codes, float* fp8_scales,
                                      const float* amax_row_in, const float* amax_col_in,
                                      float* amax_row_out, float* amax_col_out)
{
    if (k <= 0 || k % 128 != 0) return 1;
    int64_t R = 0; /* first row of the current section */
    for (int64_t s = 0; s < num_sections; ++s) {
        int64_t m = split_sections[s];
        if (m < 0 || m % 128 != 0) return 2;
        const uint16_t* xs = x + R * k;
        float ar = 0.0f, ac = 0.0f;
        oracle_nvfp4_section_amax(xs, m, k, sign_mask, &ar, &ac);
        if (amax_row_out) amax_row_out[s] = ar;
        if (amax_col_out) amax_col_out[s] = ac;
        /* a caller-supplied amax replaces the measured one in the tensor scale */
        float gr = oracle_nvfp4_global_scale(amax_row_in ? amax_row_in[s] : ar);
        float gc = oracle_nvfp4_global_scale(amax_col_in ? amax_col_in[s] : ac);
        if (flags & ORACLE_ROWWISE)    row_global[s] = gr;
        if (flags & ORACLE_COLUMNWISE) col_global[s] = gc;
        oracle_nvfp4_section(xs, m, k, sign_mask, flags, gr, gc,
                             row_offsets != NULL, col_offsets != NULL, seed,
                             row_offsets ? row_offsets[s] : 0, col_offsets ? col_offsets[s] : 0,
                             0, m, 0, k,
                             (flags & ORACLE_ROWWISE) ? row_codes + R * (k / 2) : NULL,
                             (flags & ORACLE_ROWWISE) ? row_scales + R * (k / 16) : NULL,
                             (flags & ORACLE_COLUMNWISE) ? col_codes + k * R / 2 : NULL,
                             (flags & ORACLE_COLUMNWISE) ? col_scales + k * R / 16 : NULL,
                             (flags & ORACLE_FP8_ROWWISE) ? fp8_codes + R * k : NULL,
                             (flags & ORACLE_FP8_ROWWISE) ? fp8_scales + R * (k / 128) : NULL);
        R += m;
    }
    return 0;
}

int oracle_group_rht_quant_nvfp4(const uint16_t* x, int64_t k,
                                 const int64_t* split_sections, int64_t num_sections,
                                 uint16_t sign_mask, uint32_t flags, uint64_t seed,
                                 const uint64_t* row_offsets, const uint64_t* col_offsets,
                                 uint8_t* row_codes, uint8_t* row_scales, float* row_global,
                                 uint8_t* col_codes, uint8_t* col_scales, float* col_global,
                                 uint8_t* fp8_codes, float* fp8_scales)
{
    return oracle_group_rht_quant_nvfp4_amax(x, k, split_sections, num_sections, sign_mask, flags, seed,
                                             row_offsets, col_offsets, row_codes, row_scales, row_global,
                                             col_codes, col_scales, col_global, fp8_codes, fp8_scales,
                                             NULL, NULL, NULL, NULL);
}

/* ------------------------------------------------------------------------ */
/* Element-wise loops                                                        */
/* ------------------------------------------------------------------------ */
void oracle_e4m3_encode_n(const float* v, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(v[i]);
}

void oracle_e2m1_encode_n(const float* v, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e2m1_encode(v[i]);
}

void oracle_e2m1_encode_sr_n(const float* v, const uint8_t* r, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e2m1_encode_sr(v[i], r[i]);
}

void oracle_f32_to_bf16_n(const float* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(v[i]);
}

void oracle_wht_n(const float* in, int64_t count, int n, uint32_t sign_mask, float c, float* out)
{
    for (int64_t i = 0; i < count; ++i) oracle_wht(in + i * n, n, sign_mask, c, out + i * n);
}

/* ------------------------------------------------------------------------ */
/* DSA rotate + NVFP4 row-wise                                               */
/* ------------------------------------------------------------------------ */
/* The rotated values of row r: v = cat(pe[r][0:d_pe], nope[r][0:128-d_pe]),
 * y = WHT_128(v; no signs, F(1/sqrt(128))), each y_i a BF16 value. */
static void dsa_rotated_row(const uint16_t* pe, int64_t ld_pe, int32_t d_pe,
                            const uint16_t* nope, int64_t ld_nope, int64_t r, float* y)
{
    float v[128];
    for (int i = 0; i < d_pe; ++i)   v[i] = oracle_bf16_to_f32(pe[r * ld_pe + i]);
    for (int i = d_pe; i < 128; ++i) v[i] = oracle_bf16_to_f32(nope[r * ld_nope + (i - d_pe)]);
    oracle_wht(v, 128, 0u, F_C128(), y);
}

void oracle_hadamard_quant_nvfp4(const uint16_t* pe, int64_t ld_pe, int32_t d_pe,
                                 const uint16_t* nope, int64_t ld_nope, int64_t m,
                                 const float* amax_in, uint8_t* codes, uint8_t* scales,
                                 float* global_scale, float* amax_out)
{
    float y[128];
    /* pass 1: A = max |y| over every rotated value of the tensor, NaN ignored */
    float A = 0.0f;
    for (int64_t r = 0; r < m; ++r) {
        dsa_rotated_row(pe, ld_pe, d_pe, nope, ld_nope, r, y);
        float a = oracle_amax(y, 128);
        if (a > A) A = a;
    }
    if (amax_out) *amax_out = A;
    float g = oracle_nvfp4_global_scale(amax_in ? *amax_in : A);
    *global_scale = g;
    /* pass 2: each 1x16 block of each row with the tensor scale g */
    for (int64_t r = 0; r < m; ++r) {
        dsa_rotated_row(pe, ld_pe, d_pe, nope, ld_nope, r, y);
        for (int b = 0; b < 8; ++b) {
            uint8_t c16[16];
            oracle_nvfp4_block(y + 16 * b, g, NULL, &scales[r * 8 + b], c16);
            for (int i = 0; i < 8; ++i)
                codes[r * 64 + b * 8 + i] = (uint8_t)(c16[2 * i] | (c16[2 * i + 1] << 4));
        }
    }
}

/* ------------------------------------------------------------------------ */
/* SwiGLU -> FP8 1x128                                                       */
/* ------------------------------------------------------------------------ */
/* 2^j for an integer j in [-126, 127] (a normal binary32). */
static float pow2i(int j) { return bits_f32((uint32_t)(j + 127) << 23); }

float oracle_exp(float x)
{
    if (x != x) return x;
    if (x > 128.0f) x = 128.0f;            /* e^128 and e^-128 are already beyond */
    if (x < -128.0f) x = -128.0f;          /* binary32's range                    */
    const float log2e = (float)(1.0 / log(2.0));
    const float L1 = 0.693145751953125f;   /* ln 2 to 16 significant bits */
    const float L2 = (float)(log(2.0) - 0.693145751953125);
    float k = rintf(x * log2e);            /* nearest integer, ties to even */
    float r = fmaf(-k, L1, x);
    r = fmaf(-k, L2, r);
    /* e^r by its Taylor polynomial of degree 7, Horner's rule from the top */
    double fact = 1.0;
    for (int n = 2; n <= 7; ++n) fact *= n;            /* 7! */
    float p = (float)(1.0 / fact);
    for (int n = 6; n >= 0; --n) {
        fact /= (n + 1);                                 /* n! */
        p = fmaf(p, r, (float)(1.0 / fact));
    }
    int ki = (int)k;
    int k1 = (int)floorf(k * 0.5f), k2 = ki - k1;
    return (p * pow2i(k1)) * pow2i(k2);
}

float oracle_silu(float g)
{
    float e = oracle_exp(-g);
    float t = 1.0f + e;
    return g / t;
}

void oracle_swiglu_quant_fp8(const uint16_t* gate, int64_t ld_gate, const uint16_t* up, int64_t ld_up,
                             int64_t m, int64_t n, uint8_t* q, int64_t ldq, float* scales,
                             int64_t scale_stride_row, int64_t scale_stride_group)
{
    float h[128];
    for (int64_t r = 0; r < m; ++r) {
        for (int64_t g0 = 0; g0 < n; g0 += 128) {
            for (int i = 0; i < 128; ++i) {
                float gv = oracle_bf16_to_f32(gate[r * ld_gate + g0 + i]);
                float uv = oracle_bf16_to_f32(up[r * ld_up + g0 + i]);
                h[i] = oracle_silu(gv) * uv;       /* FP32, no rounding to the input type */
            }
            scales[r * scale_stride_row + (g0 / 128) * scale_stride_group] =
                oracle_fp8_group(h, q + r * ldq + g0);
        }
    }
}

void oracle_exp_n(const float* x, int64_t count, float* out)
{
    for (int64_t i = 0; i < count; ++i) out[i] = oracle_exp(x[i]);
}

void oracle_silu_n(const float* x, int64_t count, float* out)
{
    for (int64_t i = 0; i < count; ++i) out[i] = oracle_silu(x[i]);
}

/* ------------------------------------------------------------------------ */
/* FP8 block variants: UE8M0 scales, 128x1 column blocks, scale layouts      */
/* ------------------------------------------------------------------------ */
float oracle_pow2_ceil(float s)
{
    /* the smallest power of two >= s, for a positive normal s: the exponent of s,
     * plus one unless s is already a power of two.  An infinite s (an infinite
     * group amax) stays infinite. */
    if (isinf(s)) return s;
    int e;
    float f = frexpf(s, &e);                  /* s = f * 2^e, f in [0.5, 1) */
    return (f == 0.5f) ? s : ldexpf(1.0f, e);
}

float oracle_fp8_block(const float* x, int n, uint32_t options, uint8_t* codes)
{
    float a = oracle_amax(x, n);
    float floor_ = F_1E_10();
    float s = ((a > floor_) ? a : floor_) * F_1_OVER_448();
    if (options & ORACLE_FP8_UE8M0) s = oracle_pow2_ceil(s);
    for (int i = 0; i < n; ++i) codes[i] = oracle_e4m3_encode(x[i] / s);
    return s;
}

void oracle_quant_fp8_blockwise(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, uint32_t options,
                                uint8_t* row_codes, int64_t row_ld, float* row_scales,
                                int64_t row_stride_r, int64_t row_stride_g,
                                uint8_t* col_codes, int64_t col_ld, float* col_scales,
                                int64_t col_stride_c, int64_t col_stride_b)
{
    float v[128];
    uint8_t c[128];
    if (row_codes) {
        for (int64_t r = 0; r < m; ++r)
            for (int64_t g = 0; g < k / 128; ++g) {
                for (int i = 0; i < 128; ++i) v[i] = oracle_bf16_to_f32(x[r * ldx + g * 128 + i]);
                row_scales[r * row_stride_r + g * row_stride_g] =
                    oracle_fp8_block(v, 128, options, row_codes + r * row_ld + g * 128);
            }
    }
    if (col_codes) {
        /* column c, row block b: rows 128b .. min(128b + 128, m) - 1 of column c;
         * the codes go to row c of the transposed output */
        for (int64_t cc = 0; cc < k; ++cc)
            for (int64_t b = 0; 128 * b < m; ++b) {
                int n = (int)((m - 128 * b) < 128 ? (m - 128 * b) : 128);
                for (int i = 0; i < n; ++i) v[i] = oracle_bf16_to_f32(x[(128 * b + i) * ldx + cc]);
                col_scales[cc * col_stride_c + b * col_stride_b] = oracle_fp8_block(v, n, options, c);
                for (int i = 0; i < n; ++i) col_codes[cc * col_ld + 128 * b + i] = c[i];
            }
    }
}

void oracle_hadamard_quant_fp8_ex(const uint16_t* pe, int64_t ld_pe, int32_t d_pe,
                                  const uint16_t* nope, int64_t ld_nope, int64_t m, uint32_t options,
                                  int64_t heads, uint8_t* q, float* scales,
                                  int64_t scale_stride_token, int64_t scale_stride_head)
{
    float v[128], y[128];
    for (int64_t r = 0; r < m; ++r) {
        for (int i = 0; i < d_pe; ++i)   v[i] = oracle_bf16_to_f32(pe[r * ld_pe + i]);
        for (int i = d_pe; i < 128; ++i) v[i] = oracle_bf16_to_f32(nope[r * ld_nope + (i - d_pe)]);
        oracle_wht(v, 128, 0u, F_C128(), y);
        int64_t token = r / heads, head = r % heads;
        scales[token * scale_stride_token + head * scale_stride_head] = oracle_fp8_block(y, 128, options, q + r * 128);
    }
}
