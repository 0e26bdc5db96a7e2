/*
 * mxq_oracle.h -- CPU oracle for the mxq block-quantization path.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, single-threaded reference
 * that the GPU kernels are checked against, byte for byte.  Only the test suite,
 * the package smoke check and the benchmark's CPU-baseline leg may load it.  It
 * shares no code, header, table or constant with the HIP library: every step
 * below is written out from the format and algorithm definitions.
 *
 * Arithmetic: IEEE-754 binary32, round-to-nearest-even, one rounding per
 * operation, no FMA contraction, subnormals kept (compile with
 * -O2 -ffp-contract=off, never -ffast-math).
 *
 * Sources (the pages these definitions come from):
 *  - onnxruntime PR #33644 (QMoE dynamic FP8 activation quantization),
 *    Description: K128 groups, scale = max(amax, 1e-10) * float32(1/448),
 *    saturating nearest-even E4M3FN conversion, FP32 normalization by division.
 *  - TransformerEngine PR #2564 "[NVFP4][MOE] Bug Fix for NVFP4 Grouped Quant",
 *    Greptile summary: grouped NVFP4 quantization with row-wise output and a
 *    column-wise output computed after a Hadamard transform.
 *  - TransformerEngine PR #2555 review comments on quantizer.cpp: the RHT is
 *    applied to the transposed (column-wise) operand only, a 16x16 RHT matrix
 *    per quantizer, an input-dtype [cols x rows] intermediate for RHT(x^T), and a
 *    separate column-wise RNG state for stochastic rounding.
 *  - TensorRT-LLM PR #15158 "Add rotate_activation to DSA fused_cat_fp8 path",
 *    Summary and discussion: cat[qk_pe, qk_nope] -> orthonormal Hadamard
 *    rotation -> FP8 1x128 quantization; (Hq).(Hk) = q.k for orthonormal H.
 *  - Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 *    easy as 1, 2, 3", SC'11.
 *
 * Where the pages leave a step open, the reading adopted is the one listed in
 * the design notes (per-section, per-direction FP32 tensor scale
 * g = max(A,1e-10)/2688 as a multiply by float32(1/2688); BF16 rounding of
 * rotated values; even element in the low nibble; ...).
 */
#ifndef MXQ_ORACLE_H
#define MXQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- formats ----------------------------------------------------------- */
float    oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_f32_to_bf16(float v);              /* nearest, ties to even */
float    oracle_e4m3_value(uint8_t code);          /* OCP E4M3FN decode; 0x7F/0xFF -> NaN */
uint8_t  oracle_e4m3_encode(float v);              /* saturating RNE; NaN -> 0x7F */
float    oracle_e2m1_value(uint8_t code);          /* low 4 bits used */
uint8_t  oracle_e2m1_encode(float v);              /* saturating RNE (ties to even code) */
uint8_t  oracle_e2m1_encode_sr(float v, uint8_t r);/* stochastic rounding with 8 random bits */
float    oracle_amax(const float* v, int64_t n);   /* max |v|, NaN ignored, empty -> +0 */

/* ---- Philox4x32-10 -------------------------------------------------------- */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* ---- Walsh-Hadamard ----------------------------------------------------------
 * y_i = BF16(fl(v_i * c)) after sign flips (bit i of sign_mask set -> negate
 * input i) and log2(n) butterfly stages with h = 1, 2, 4, ... in that order.
 * n must be a power of two <= 128.  Output: n floats, each exactly a BF16 value. */
void oracle_wht(const float* in, int n, uint32_t sign_mask, float c, float* out);

/* ---- FP8 1x128 --------------------------------------------------------------
 * One 128-element group: s = fl(max(amax, F(1e-10)) * F(1/448));
 * code_i = E4M3(fl(x_i / s)).  Returns s. */
float oracle_fp8_group(const float* x, uint8_t* codes);

/* x: [m][ldx] BF16 bits, k % 128 == 0.  q: [m][ldq] codes.
 * scales[r*scale_stride_row + g*scale_stride_group] for group g of row r. */
void oracle_quant_fp8_1x128(const uint16_t* x, int64_t m, int64_t k, int64_t ldx,
                            uint8_t* q, int64_t ldq, float* scales,
                            int64_t scale_stride_row, int64_t scale_stride_group);

/* DSA-indexer rotate+quant: v = cat(pe[r][0:d_pe], nope[r][0:128-d_pe]);
 * y = WHT_128(v; no signs, c = F(1/sqrt(128))); FP8 1x128 of y.
 * q: [m][128], scales: [m]. */
void oracle_hadamard_quant_fp8(const uint16_t* pe, int64_t ld_pe, int32_t d_pe,
                               const uint16_t* nope, int64_t ld_nope, int64_t m,
                               uint8_t* q, float* scales);

/* DSA-indexer rotate + NVFP4 row-wise (the FP4 counterpart of the call above):
 * y = WHT_128(cat(pe[r][0:d_pe], nope[r][0:128-d_pe]); no signs, F(1/sqrt(128))),
 * rounded to BF16; one tensor scale g = fl(max(A, F(1e-10)) * F(1/2688)) with A the
 * max |y| over the whole tensor (NaN ignored), or *amax_in when amax_in is not
 * NULL; then every 1x16 block of every row encoded with g as oracle_nvfp4_block.
 * codes [m][64] (even element in the low nibble), scales [m][8] E4M3,
 * *global_scale = g, *amax_out = the measured A (when not NULL). */
void oracle_hadamard_quant_nvfp4(const uint16_t* pe, int64_t ld_pe, int32_t d_pe,
                                 const uint16_t* nope, int64_t ld_nope, int64_t m,
                                 const float* amax_in, uint8_t* codes, uint8_t* scales,
                                 float* global_scale, float* amax_out);

/* ---- FP8 block variants ----------------------------------------------------------
 * ORACLE_FP8_UE8M0: the scale s = fl(max(a, F(1e-10)) * F(1/448)) is rounded up to
 * the nearest power of two (a UE8M0-representable scale; amax / s then stays <= 448). */
#define ORACLE_FP8_UE8M0 1u
float oracle_pow2_ceil(float s);                   /* smallest power of two >= s (s > 0 normal) */
/* n <= 128 values as one block: s as above (UE8M0 with the option), codes E4M3(fl(x/s)). */
float oracle_fp8_block(const float* x, int n, uint32_t options, uint8_t* codes);
/* Row-wise 1x128 (row_codes [m][row_ld], scale of (r, g) at r*row_stride_r + g*row_stride_g)
 * and column-wise 128x1 blocks on the transpose (col_codes [k][col_ld]: row c holds column c
 * of x; column c's block b covers rows 128b .. min(128b+128, m)-1; its scale at
 * c*col_stride_c + b*col_stride_b).  Either output may be NULL.  k % 128 == 0. */
void oracle_quant_fp8_blockwise(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, uint32_t options,
                                uint8_t* row_codes, int64_t row_ld, float* row_scales,
                                int64_t row_stride_r, int64_t row_stride_g,
                                uint8_t* col_codes, int64_t col_ld, float* col_scales,
                                int64_t col_stride_c, int64_t col_stride_b);
/* The DSA rotate + FP8 with options and a (token, head) scale layout: row r is token
 * r / heads, head r % heads, and its scale goes to token*scale_stride_token +
 * head*scale_stride_head. */
void oracle_hadamard_quant_fp8_ex(const uint16_t* pe, int64_t ld_pe, int32_t d_pe,
                                  const uint16_t* nope, int64_t ld_nope, int64_t m, uint32_t options,
                                  int64_t heads, uint8_t* q, float* scales,
                                  int64_t scale_stride_token, int64_t scale_stride_head);

/* ---- SwiGLU -> FP8 1x128 ---------------------------------------------------------
 * EXP(x), e^x in binary32 by these steps (one rounding per operation):
 *   NaN -> NaN; x clamped to [-128, 128];
 *   k = rint(fl(x * F(log2 e))); r = fma(-k, L1, x); r = fma(-k, L2, r) with
 *   L1 = 0.693145751953125 (ln 2 to 16 bits) and L2 = F(ln 2 - L1);
 *   p = the degree-7 Taylor polynomial of e^r with coefficients F(1/n!) by Horner's
 *   rule (p = fma(p, r, F(1/n!)) from n = 6 down to 0, starting from F(1/7!));
 *   result = fl(fl(p * 2^k1) * 2^k2), k1 = floor(k/2), k2 = k - k1.
 * SILU(g) = fl(g / fl(1 + EXP(-g)));  the SwiGLU value h = fl(SILU(gate) * up) stays
 * FP32 and goes straight into FP8 1x128 (oracle_fp8_group). */
float oracle_exp(float x);
float oracle_silu(float g);
/* gate [m][ld_gate], up [m][ld_up] BF16; n % 128 == 0; q [m][ldq];
 * scales[r*scale_stride_row + g*scale_stride_group] for group g of row r. */
void oracle_swiglu_quant_fp8(const uint16_t* gate, int64_t ld_gate, const uint16_t* up, int64_t ld_up,
                             int64_t m, int64_t n, uint8_t* q, int64_t ldq, float* scales,
                             int64_t scale_stride_row, int64_t scale_stride_group);
/* count values through oracle_exp / oracle_silu (for sweeps) */
void oracle_exp_n(const float* x, int64_t count, float* out);
void oracle_silu_n(const float* x, int64_t count, float* out);

/* ---- NVFP4 -------------------------------------------------------------------- */
/* g = fl(max(A, F(1e-10)) * F(1/2688)) */
float oracle_nvfp4_global_scale(float amax);

/* Encode one 1x16 block of values (each already a BF16 value) with tensor scale g.
 * rbits: 16 random bytes for stochastic rounding, or NULL for RNE.
 * Writes the E4M3 block-scale code and 16 E2M1 codes (one per byte, 0..15). */
void oracle_nvfp4_block(const float* v, float g, const uint8_t* rbits,
                        uint8_t* scale_code, uint8_t* codes);

/* Per-section amax of the row-wise values (x) and of the column-wise values
 * (BF16(RHT16(x)) per 16-row block of each column).  x: [rows][k] BF16, rows % 16 == 0. */
void oracle_nvfp4_section_amax(const uint16_t* x, int64_t rows, int64_t k,
                               uint16_t sign_mask, float* amax_row, float* amax_col);

/* Flags for oracle_nvfp4_section and oracle_group_rht_quant_nvfp4. */
#define ORACLE_ROWWISE     1u
#define ORACLE_COLUMNWISE  2u
#define ORACLE_FP8_ROWWISE 4u

/* Quantize one section (rows x k, rows % 128 == 0 or 0) given its tensor scales.
 *  row_codes  [rows][k/2], row_scales [rows][k/16]          (ROWWISE)
 *  col_codes  [k][rows/2], col_scales [k][rows/16]          (COLUMNWISE)
 *  fp8_codes  [rows][k],   fp8_scales [rows][k/128]         (FP8_ROWWISE)
 * use_sr_row / use_sr_col select stochastic rounding with Philox keyed by seed,
 * counter (lo(off), hi(off), lo(beta), hi(beta)); beta = r*(k/16)+kb for rows,
 * c*(rows/16)+b for columns.  Rows [row_begin, row_end) of the row-wise outputs
 * and columns [col_begin, col_end) of the column-wise outputs are produced
 * (pass 0, rows / 0, k for everything); this lets a caller split the work. */
void oracle_nvfp4_section(const uint16_t* x, int64_t rows, int64_t k, uint16_t sign_mask,
                          uint32_t flags, float g_row, float g_col,
                          int use_sr_row, int use_sr_col, uint64_t seed,
                          uint64_t row_offset, uint64_t col_offset,
                          int64_t row_begin, int64_t row_end,
                          int64_t col_begin, int64_t col_end,
                          uint8_t* row_codes, uint8_t* row_scales,
                          uint8_t* col_codes, uint8_t* col_scales,
                          uint8_t* fp8_codes, float* fp8_scales);

/* The whole grouped call (same layouts as the library):
 *  x [total_rows][k]; sections: split_sections[num_sections] (host);
 *  row: codes [total][k/2], scales [total][k/16], global [num_sections]
 *  col: section s at codes + k*R_s/2 as [k][m_s/2], scales + k*R_s/16 as [k][m_s/16],
 *       global [num_sections]
 *  fp8: codes [total][k], scales [total][k/128].
 * row_offsets / col_offsets: NULL for RNE in that direction.  Returns 0 on success. */
int oracle_group_rht_quant_nvfp4(const uint16_t* x, int64_t k,
                                 const int64_t* split_sections, int64_t num_sections,
                                 uint16_t sign_mask, uint32_t flags, uint64_t seed,
                                 const uint64_t* row_offsets, const uint64_t* col_offsets,
                                 uint8_t* row_codes, uint8_t* row_scales, float* row_global,
                                 uint8_t* col_codes, uint8_t* col_scales, float* col_global,
                                 uint8_t* fp8_codes, float* fp8_scales);

/* The grouped call with a caller-supplied amax (next-step scaling, a single pass
 * over x in the library): amax_row_in / amax_col_in (NULL: measure) replace the
 * section maxima in the tensor scales, g = fl(max(A_in, F(1e-10)) * F(1/2688)); the
 * measured maxima (the values the plain call would use) go to amax_row_out /
 * amax_col_out when not NULL. */
int oracle_group_rht_quant_nvfp4_amax(const uint16_t* x, int64_t k,
                                      const int64_t* split_sections, int64_t num_sections,
                                      uint16_t sign_mask, uint32_t flags, uint64_t seed,
                                      const uint64_t* row_offsets, const uint64_t* col_offsets,
                                      uint8_t* row_codes, uint8_t* row_scales, float* row_global,
                                      uint8_t* col_codes, uint8_t* col_scales, float* col_global,
                                      uint8_t* fp8_codes, float* fp8_scales,
                                      const float* amax_row_in, const float* amax_col_in,
                                      float* amax_row_out, float* amax_col_out);

/* ---- element-wise loops over arrays (for exhaustive codec sweeps) ---------- */
void oracle_e4m3_encode_n(const float* v, int64_t n, uint8_t* out);
void oracle_e2m1_encode_n(const float* v, int64_t n, uint8_t* out);
void oracle_e2m1_encode_sr_n(const float* v, const uint8_t* r, int64_t n, uint8_t* out);
void oracle_f32_to_bf16_n(const float* v, int64_t n, uint16_t* out);
/* count vectors of length n, each transformed with oracle_wht */
void oracle_wht_n(const float* in, int64_t count, int n, uint32_t sign_mask, float c, float* out);

#ifdef __cplusplus
}
#endif
#endif /* MXQ_ORACLE_H */
