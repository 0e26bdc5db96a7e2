/*
 * mxq.h -- C ABI of the mxq block-quantization library for AMD Instinct MI355X
 * (gfx950).
 *
 * These entry points quantize BF16 activations on the GPU:
 *   mxq_quant_fp8_1x128        FP8 E4M3 with one FP32 scale per 1x128 group
 *   mxq_quant_fp8_blockwise    the same row-wise and/or 128x1 column-wise on the
 *                              transpose, optionally with UE8M0 (power-of-two) scales
 *   mxq_hadamard_quant_fp8_ex  the DSA rotate + FP8 with UE8M0 and scale layouts
 *   mxq_swiglu_quant_fp8       FP32 SiLU(gate) * up -> FP8 1x128 (no BF16 round)
 *   mxq_hadamard_quant_fp8     cat[qk_pe, qk_nope] -> normalized 128-point
 *                              Walsh-Hadamard rotation -> FP8 1x128
 *   mxq_hadamard_quant_nvfp4   the same rotation -> NVFP4 row-wise (1x16 blocks,
 *                              one FP32 tensor scale, measured or supplied)
 *   mxq_group_rht_quant_nvfp4  grouped (MoE split sections) NVFP4, row-wise and
 *                              column-wise after a 16-point random-sign Hadamard
 *                              transform, optionally with an FP8 1x128 row-wise
 *                              output in the same call
 *
 * Conventions shared by every entry point
 *  - Pointers named *_bf16 / codes / scales / workspace are DEVICE pointers; the
 *    caller owns every buffer.  split_sections, mxq_sr and its offset arrays are
 *    HOST memory, read during the call only (their values are baked into the
 *    kernel arguments, so under stream capture the capture-time values are used).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *    asynchronous: MXQ_OK means the work was enqueued.
 *  - The library never allocates, frees, memsets, synchronizes or reads the
 *    environment; it keeps no global state (the per-device scratch array of
 *    mxq_group_rht_quant_nvfp4_noalloc aside) and is re-entrant.  Calls in flight
 *    at the same time need distinct workspaces.
 *  - All argument checks run on the host before anything is enqueued; on an error
 *    nothing is launched and no output is touched.  A failed launch returns
 *    MXQ_ERR_HIP (outputs are then undefined).  There is no fallback path: an
 *    unsupported request is an error, never a slower substitute.
 *  - Arithmetic is IEEE binary32 with one rounding per operation in the order
 *    stated below; every output is bit-exact with respect to that definition.
 *
 * Sources of the operations (page, then section):
 *  - onnxruntime PR #33644, QMoE dynamic FP8 activation quantization,
 *    Description: K128 groups; scale = max(amax, 1e-10) * float32(1/448); FP32
 *    normalization by division; saturating nearest-even E4M3FN.
 *  - TensorRT-LLM PR #15158, "Add rotate_activation to DSA fused_cat_fp8 path",
 *    Summary: cat[qk_pe, qk_nope] -> rotate_activation -> fp8_quantize_1x128;
 *    the discussion's (Hq).(Hk) = q.k for the orthonormal rotation.
 *  - TransformerEngine PR #2564, "[NVFP4][MOE] Bug Fix for NVFP4 Grouped Quant",
 *    Greptile summary and sequence diagram: grouped row-wise + column-wise
 *    (RHT) NVFP4 cast with a caller-provided workspace, no allocation per call;
 *    review thread: a workspace-size query.
 *  - TransformerEngine PR #2555, review comments on cast.cpp and quantizer.cpp:
 *    split_section % 128 == 0; RHT on the column-wise (transposed) operand only;
 *    row-wise-only requests skip the RHT work; a separate column-wise RNG state;
 *    deterministic RNG offsets rather than sequential generator advancement.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MXQ_OK = 0,
    MXQ_ERR_INVALID_ARGUMENT = 1,    /* NULL pointer, negative size, bad flags ...   */
    MXQ_ERR_MISALIGNED = 2,          /* k or a section not a multiple of 128, or a  */
                                     /* pointer / stride not 16-byte aligned        */
    MXQ_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < the size query's value    */
    MXQ_ERR_UNSUPPORTED = 4,         /* outside the supported profile (limits)      */
    MXQ_ERR_HIP = 5                  /* a HIP launch failed                          */
} mxq_status;

/* Static string naming the status; never NULL. */
const char* mxq_status_string(mxq_status s);

/* Library version string, e.g. "mxq 0.1.0 gfx950". */
const char* mxq_version(void);

/* Limits of the supported profile. */
#define MXQ_ROW_ALIGN 128          /* rows per section and k: multiples of this   */
#define MXQ_MAX_SECTIONS 256       /* split sections per grouped call             */
/* Every array a call addresses spans fewer than MXQ_MAX_EXTENT elements: rows of
 * length n at stride ld span (rows - 1) * ld + n, and a scale array addressed as
 * r * s_r + c * s_c reaches index (rows - 1) * s_r + (cols - 1) * s_c.  Larger
 * extents give MXQ_ERR_UNSUPPORTED before anything is enqueued. */
#define MXQ_MAX_EXTENT (1LL << 40)

/* ---------------------------------------------------------------------------
 * FP8 E4M3 (OCP E4M3FN), one FP32 scale per 1x128 group along k.
 * onnxruntime PR #33644, Description: the QMoE dynamic activation quantizer's
 * K128 groups, its scale max(amax, 1e-10) * float32(1/448), the FP32 division of
 * each element by its group's scale and the saturating nearest-even E4M3FN encode;
 * the one-ulp differences at E4M3 midpoints it reports are why the division is
 * exact IEEE here, never a reciprocal multiply.
 *
 *   x_bf16   [m][ldx] BF16 bit patterns, row-major, ldx >= k
 *   q_e4m3   [m][ldq] E4M3 codes, ldq >= k
 *   scales   scales[r * scale_stride_row + g * scale_stride_group] for group g of
 *            row r; ({k/128, 1} is [m][k/128]; {1, m} is the transposed [k/128][m])
 *
 * For each group G of 128 consecutive elements of a row:
 *   a = max |x| over G (NaN ignored; 0 if none),  s = fl(max(a, F(1e-10)) * F(1/448)),
 *   q_i = E4M3(fl(x_i / s))   (IEEE division, nearest-even, saturating at 448;
 *                               a NaN element gives 0x7F).
 * Requirements: k % 128 == 0; ldx, ldq multiples of 8 and 16; x, q 16-byte
 * aligned; scales 4-byte aligned.  m == 0 is a successful no-op.
 * ------------------------------------------------------------------------- */
mxq_status mxq_quant_fp8_1x128(const uint16_t* x_bf16, int64_t m, int64_t k, int64_t ldx,
                               uint8_t* q_e4m3, int64_t ldq,
                               float* scales, int64_t scale_stride_row, int64_t scale_stride_group,
                               void* stream);

/* ---------------------------------------------------------------------------
 * FP8 block variants (consumer-facing layouts of the same recipe).
 * TensorRT-LLM PR #15158, review of the DSA scale normalization: a use_ue8m0 option
 * of fp8_quantize_1x128_sf_transpose, and the 1-D scale tensor padded, reshaped and
 * transposed for its consumer.  The recipe is mxq_quant_fp8_1x128's.
 *
 * MXQ_FP8_UE8M0: every scale s = fl(max(a, F(1e-10)) * F(1/448)) is rounded up to
 * the nearest power of two (stored as that FP32 power of two: its UE8M0 byte is the
 * FP32 exponent field, bits >> 23); the codes are E4M3(x / s), exact divisions, and
 * |x| / s stays <= 448.
 * ------------------------------------------------------------------------- */
enum { MXQ_FP8_UE8M0 = 1u };

typedef struct {
    uint8_t* codes;             /* row-wise: [m][ld];  column-wise: [k][ld], row c = column c of x */
    int64_t  ld;
    float*   scales;            /* row-wise: (row r, group g) at r * scale_stride_a + g * scale_stride_b;
                                   column-wise: (column c, row block b) at c * scale_stride_a + b * scale_stride_b */
    int64_t  scale_stride_a;
    int64_t  scale_stride_b;
} mxq_fp8_block_out;

/* Row-wise 1x128 groups and/or column-wise 128x1 blocks (rows 128b .. min(128b+128,
 * m)-1 of column c, a ragged last block when m % 128 != 0; its codes go to row c of the
 * transposed output), from one read of x.  rowwise / columnwise may be NULL (not both).
 * Requirements: k % 128 == 0; ldx % 8 == 0; ld >= k (row-wise) or >= m (column-wise),
 * a multiple of 16; x and codes 16-byte aligned, scales 4-byte aligned; options in
 * {0, MXQ_FP8_UE8M0}.  m == 0 is a successful no-op. */
mxq_status mxq_quant_fp8_blockwise(const uint16_t* x_bf16, int64_t m, int64_t k, int64_t ldx, uint32_t options,
                                   const mxq_fp8_block_out* rowwise, const mxq_fp8_block_out* columnwise,
                                   void* stream);

/* mxq_hadamard_quant_fp8 with options and a (token, head) scale layout: row r is
 * token r / heads, head r % heads (heads >= 1), and its scale goes to
 * scales[token * scale_stride_token + head * scale_stride_head]: {heads, 1} is the
 * plain [tokens][heads] order, {1, T} the transposed [heads][T] one with T >= tokens
 * (rows T past the tokens are padding the call leaves untouched). */
mxq_status mxq_hadamard_quant_fp8_ex(const uint16_t* pe, int64_t ld_pe, int32_t d_pe,
                                     const uint16_t* nope, int64_t ld_nope, int64_t m, uint32_t options,
                                     int64_t heads, uint8_t* q_e4m3, float* scales,
                                     int64_t scale_stride_token, int64_t scale_stride_head, void* stream);

/* ---------------------------------------------------------------------------
 * SwiGLU -> FP8 1x128: the second dynamic quantizer of a W8A8 MoE, directly after
 * the FP32 SiLU/SwiGLU of the gate and up projections (onnxruntime PR #33644,
 * Description: no round to the input type between SwiGLU and the quantizer; the
 * same FP8 recipe as mxq_quant_fp8_1x128).  For each element:
 *   h = fl(SILU(gate) * up),  SILU(g) = fl(g / fl(1 + EXP(-g)))   (all FP32)
 * and then, per group G of 128 consecutive h of a row, exactly as
 * mxq_quant_fp8_1x128 (a = max |h| without NaNs, s = fl(max(a, F(1e-10)) * F(1/448)),
 * q = E4M3(fl(h / s)), 0x7F for a NaN).  EXP(x) is e^x by a stated binary32
 * algorithm (the pages do not fix one): NaN kept; x clamped to [-128, 128];
 * k = rint(fl(x * F(log2 e))); r = fma(-k, 0.693145751953125, x);
 * r = fma(-k, F(ln 2 - 0.693145751953125), r); p = the degree-7 Taylor polynomial of
 * e^r with coefficients F(1/n!) by Horner's rule with fma; EXP = fl(fl(p * 2^k1) * 2^k2),
 * k1 = floor(k/2), k2 = k - k1.  Inputs whose product overflows FP32 are out of
 * contract (as are infinite inputs).
 *
 *   gate_bf16 [m][ld_gate], up_bf16 [m][ld_up] BF16 (separate buffers, or the two
 *             halves of one [m][2n] buffer with up = gate + n)
 *   q_e4m3    [m][ldq] E4M3 codes; scales as mxq_quant_fp8_1x128 (row / group strides)
 * Requirements: n % 128 == 0; ld_gate, ld_up multiples of 8, ldq of 16; gate, up,
 * q 16-byte aligned; scales 4-byte aligned.  m == 0 is a successful no-op.
 * ------------------------------------------------------------------------- */
mxq_status mxq_swiglu_quant_fp8(const uint16_t* gate_bf16, int64_t ld_gate, const uint16_t* up_bf16, int64_t ld_up,
                                int64_t m, int64_t n, uint8_t* q_e4m3, int64_t ldq,
                                float* scales, int64_t scale_stride_row, int64_t scale_stride_group, void* stream);

/* ---------------------------------------------------------------------------
 * DSA-indexer rotate + quantize.  TensorRT-LLM PR #15158, Summary: the indexer
 * concatenates qk_pe and qk_nope, applies rotate_activation (the normalized
 * 128-point Hadamard transform) and then fp8_quantize_1x128; the discussion's
 * (Hq).(Hk) = q.k is why the rotation changes no attention score.  For each row r:
 *   v = cat(pe[r][0:d_pe], nope[r][0:128-d_pe])           (qk_pe first)
 *   y = BF16(fl(WHT_128(v) * F(1/sqrt(128))))            (Sylvester order, butterfly
 *        stages h = 1, 2, 4, ..., 64; (v_i, v_i+h) <- (v_i + v_i+h, v_i - v_i+h))
 *   q[r][:], scales[r] = FP8 1x128 of y (as mxq_quant_fp8_1x128).
 *
 *   pe    [m][ld_pe]   BF16, d_pe in {0, 8, 16, ..., 128}; may be NULL if d_pe == 0
 *   nope  [m][ld_nope] BF16; may be NULL if d_pe == 128
 *   q     [m][128] E4M3 codes;  scales [m] FP32
 * Requirements: ld_pe, ld_nope multiples of 8; pointers 16-byte aligned.
 * ------------------------------------------------------------------------- */
mxq_status mxq_hadamard_quant_fp8(const uint16_t* pe, int64_t ld_pe, int32_t d_pe,
                                  const uint16_t* nope, int64_t ld_nope, int64_t m,
                                  uint8_t* q_e4m3, float* scales, void* stream);

/* ---------------------------------------------------------------------------
 * DSA-indexer rotate + NVFP4 (row-wise 1x16).  The FP4 counterpart of the call
 * above: TensorRT-LLM PR #15158 (Summary) names the FP4 path's missing rotation and
 * its need for a standalone FP4 quantize-only kernel.  For each row r:
 *   y = BF16(fl(WHT_128(cat(pe[r][0:d_pe], nope[r][0:128-d_pe])) * F(1/sqrt(128))))
 *   (as mxq_hadamard_quant_fp8), then the row-wise NVFP4 encode of
 *   mxq_group_rht_quant_nvfp4 with ONE tensor scale for the whole call:
 *   g = fl(max(A, F(1e-10)) * F(1/2688)), A = max |y| over every row (NaN ignored)
 *   or *amax_in; per 1x16 block t = fl(fl(a * F(1/6)) / g), sc = E4M3(t),
 *   d = fl(E4M3(sc) * g), codes E2M1(fl(y / d)) (nearest-even, saturating); a block
 *   of a row holding a NaN gets scale 0x7F and zero codes.
 *
 *   pe, nope, d_pe, ld_pe, ld_nope: as mxq_hadamard_quant_fp8
 *   amax_in       device float[1], or NULL: measure A (two passes over the input)
 *   amax_out      device float[1], or NULL: the measured A of this call (0 for m = 0)
 *   codes         device [m][64]: codes of y[r][2i] (low nibble) and y[r][2i+1]
 *   block_scales  device [m][8] E4M3
 *   global_scale  device float[1]: g (also written for m = 0: the floor scale, or
 *                 the scale of *amax_in)
 *   workspace     device memory of mxq_hadamard_quant_nvfp4_workspace_size(m)
 *                 bytes (2 KB of scale table and 4 bytes per 64 rows, rounded up
 *                 to 256), 256-byte aligned; any contents (the call's kernels meet
 *                 through it in stream order and keep nothing in it between
 *                 calls).  Calls that share it must be ordered.  May be NULL when
 *                 m = 0.
 * Requirements: as mxq_hadamard_quant_fp8; codes and block_scales 16-byte aligned,
 * global_scale, amax_in, amax_out 4-byte aligned; m <= 2^31 - 128.  Errors are
 * returned before anything is enqueued.
 * ------------------------------------------------------------------------- */
size_t mxq_hadamard_quant_nvfp4_workspace_size(int64_t m);

mxq_status mxq_hadamard_quant_nvfp4(const uint16_t* pe, int64_t ld_pe, int32_t d_pe,
                                    const uint16_t* nope, int64_t ld_nope, int64_t m,
                                    const float* amax_in, float* amax_out,
                                    uint8_t* codes, uint8_t* block_scales, float* global_scale,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Grouped NVFP4 quantization with a 16-point random Hadamard transform (RHT) on
 * the column-wise operand.  TransformerEngine PR #2564, Greptile summary and
 * sequence diagram: the grouped row-wise + column-wise RHT cast over MoE split
 * sections with a caller-provided workspace and no allocation per call (review
 * thread: the workspace-size query); PR #2555, review comments on cast.cpp and
 * quantizer.cpp: split sections in multiples of 128, the RHT on the column-wise
 * (transposed) operand only, its BF16 intermediate, and a separate column-wise RNG
 * with deterministic per-call offsets for stochastic rounding.
 *
 * x_bf16 is [total_rows][k] BF16 (row stride k), total_rows = sum(split_sections).
 * Section s covers rows [R_s, R_s + m_s), m_s = split_sections[s] (m_s may be 0).
 *
 * flags (any non-empty combination):
 *   MXQ_ROWWISE      NVFP4 of x along k:
 *                      codes  [total_rows][k/2]   (2 E2M1 codes per byte, even
 *                                                  element in the low nibble)
 *                      block_scales [total_rows][k/16] E4M3
 *                      global_scales[num_sections] FP32
 *   MXQ_COLUMNWISE   NVFP4 of the transposed, rotated operand: for each 16-row block
 *                    b of a section and each column c the values
 *                      Y[c][16b + t] = BF16(fl(0.25 * (H16 D x[16b + 0..15][c]))_t)
 *                    (D = diag of signs from rht_sign_mask, bit t set = negate row
 *                    16b + t; H16 Sylvester; butterfly stages h = 1, 2, 4, 8).
 *                    Section s's outputs: codes at byte offset k*R_s/2 as [k][m_s/2],
 *                    block_scales at byte offset k*R_s/16 as [k][m_s/16];
 *                    global_scales[num_sections] FP32.
 *   MXQ_FP8_ROWWISE  FP8 1x128 of x (as mxq_quant_fp8_1x128): codes [total_rows][k],
 *                    scales [total_rows][k/128].
 *
 * NVFP4 encoding of one direction of section s (values v = x or Y):
 *   A = max |v| over the section (NaN ignored);  g = fl(max(A, F(1e-10)) * F(1/2688))
 *   (stored in global_scales; an empty section stores fl(F(1e-10) * F(1/2688))).
 *   Per 1x16 block: if it holds a NaN, scale 0x7F and codes 0; else
 *   a = max |v|, t = fl(fl(a * F(1/6)) / g), sc = E4M3(t); if sc == 0, codes 0;
 *   else d = fl(E4M3value(sc) * g) and code_i = E2M1(fl(v_i / d)) (nearest-even,
 *   saturating at 6) or, with stochastic rounding, the grid neighbour above with
 *   probability floor(256 f)/256 via 8 Philox bits per element.
 *   Dequantization: E2M1value(code) * E4M3value(sc) * g.
 *
 * sr: NULL, or {seed, row_offsets, col_offsets} with host arrays of num_sections
 *   Philox4x32-10 offsets (NULL = nearest-even in that direction).  Each 1x16 block
 *   draws one Philox call with key (lo32(seed), hi32(seed)) and counter
 *   (lo32(off_s), hi32(off_s), lo32(beta), hi32(beta)); beta = r*(k/16) + kb for
 *   row r (section-local) and block kb, beta = c*(m_s/16) + b for column c and
 *   block b; element t uses byte t&3 of output word t>>2.
 *
 * workspace: device memory of at least
 *   mxq_group_rht_quant_nvfp4_workspace_size(total_rows, k, num_sections, flags)
 *   bytes (0 when only MXQ_FP8_ROWWISE is requested; otherwise 135,680 bytes plus
 *   8 bytes per 16 rows per started 1024 columns of x, rounded up to 256), 256-byte
 *   aligned,
 *   ZERO-FILLED BEFORE ITS FIRST USE.  It holds partial maxima and per-section
 *   scale tables through which the kernels of a call meet in stream order, and the
 *   single-read form's partial words and error word, which must start at zero;
 *   every call leaves them at zero again, so a workspace is zeroed once and then
 *   reused.  Calls that share a workspace must be ordered (same stream, or
 *   synchronized).
 *
 * Requirements: k % 128 == 0, every m_s % 128 == 0 (else MXQ_ERR_MISALIGNED, with
 * no unfused fallback); 1 <= num_sections <= MXQ_MAX_SECTIONS; k <= 2^26,
 * total_rows <= 2^31 - 128 and total_rows * k < 2^40 (else MXQ_ERR_UNSUPPORTED);
 * the requested outputs non-NULL and 16-byte aligned
 * (global scales 4-byte aligned); outputs of directions not requested may be NULL.
 * ------------------------------------------------------------------------- */
enum { MXQ_ROWWISE = 1u, MXQ_COLUMNWISE = 2u, MXQ_FP8_ROWWISE = 4u };

typedef struct {
    uint8_t* codes;
    uint8_t* block_scales;
    float*   global_scales;
} mxq_nvfp4_out;

typedef struct {
    uint8_t* codes;
    float*   scales;
} mxq_fp8_out;

typedef struct {
    uint64_t        seed;
    const uint64_t* row_offsets;   /* host [num_sections], or NULL: nearest-even row-wise */
    const uint64_t* col_offsets;   /* host [num_sections], or NULL: nearest-even column-wise */
} mxq_sr;

/* Bytes of workspace the grouped call needs (0 when none is needed). */
size_t mxq_group_rht_quant_nvfp4_workspace_size(int64_t total_rows, int64_t k,
                                                int64_t num_sections, uint32_t flags);

mxq_status mxq_group_rht_quant_nvfp4(const uint16_t* x_bf16, int64_t k,
                                     const int64_t* split_sections, int64_t num_sections,
                                     uint16_t rht_sign_mask, uint32_t flags, const mxq_sr* sr,
                                     const mxq_nvfp4_out* rowwise,
                                     const mxq_nvfp4_out* columnwise,
                                     const mxq_fp8_out* fp8_rowwise,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * The grouped call with caller-supplied section maxima (a single pass over x) and
 * the measured maxima out, for scaling the next step by this step's maxima.
 *
 * amax (may be NULL: as mxq_group_rht_quant_nvfp4):
 *   row_in, col_in    device float[num_sections]: the A of the tensor scales,
 *                     g = fl(max(A, F(1e-10)) * F(1/2688)), instead of the measured
 *                     maxima; given for every requested NVFP4 direction or for none
 *                     (else MXQ_ERR_INVALID_ARGUMENT).  Blocks above the supplied A
 *                     saturate (scale 0x7E, codes at +-6).
 *   row_out, col_out  device float[num_sections] or NULL: the measured maxima of this
 *                     call (max |x| without NaNs; max |BF16(H16 D x / 4)| without NaNs),
 *                     written for the requested directions; an empty section gives 0.
 * With supplied maxima the amax pass is skipped: the workspace only carries the scale
 * tables, and the maxima out are gathered with atomic maxima while quantizing.
 * Reading of TransformerEngine PR #2564 (the workspace / size-query pattern) for a
 * delayed-scaling variant of the same cast; everything else as above.
 * ------------------------------------------------------------------------- */
typedef struct {
    const float* row_in;
    const float* col_in;
    float*       row_out;
    float*       col_out;
} mxq_amax;

mxq_status mxq_group_rht_quant_nvfp4_with_amax(const uint16_t* x_bf16, int64_t k,
                                               const int64_t* split_sections, int64_t num_sections,
                                               uint16_t rht_sign_mask, uint32_t flags, const mxq_sr* sr,
                                               const mxq_nvfp4_out* rowwise,
                                               const mxq_nvfp4_out* columnwise,
                                               const mxq_fp8_out* fp8_rowwise, const mxq_amax* amax,
                                               void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * The grouped call for callers that cannot allocate: code under stream capture,
 * tight serving loops, harnesses that forbid allocation.  Arguments, outputs,
 * checks and results are those of mxq_group_rht_quant_nvfp4 without the workspace:
 * the library's own device array of MXQ_NOALLOC_SCRATCH_BYTES bytes stands in for it
 * (one per GPU, held until the process ends; its device address is looked up once
 * per device, on the first call with that device current, and the words the call
 * needs at zero are cleared then by a fill kernel on that call's stream).  A call
 * whose workspace would exceed the array (mxq_group_rht_quant_nvfp4_workspace_size
 * above MXQ_NOALLOC_SCRATCH_BYTES: more than 114,112 bands of 16 rows x 1024 columns,
 * e.g. more than 456,448 rows at k = 4096) gives
 * MXQ_ERR_UNSUPPORTED before anything is enqueued.  The call itself allocates
 * nothing (no hipMalloc, no allocating library routine).  The stream must belong to
 * the current device.  Every call on one GPU uses that GPU's array: calls that
 * overlap on one GPU (other streams, or other host threads without ordering) race.
 * ------------------------------------------------------------------------- */
#define MXQ_NOALLOC_SCRATCH_BYTES (1u << 20)

mxq_status mxq_group_rht_quant_nvfp4_noalloc(const uint16_t* x_bf16, int64_t k,
                                             const int64_t* split_sections, int64_t num_sections,
                                             uint16_t rht_sign_mask, uint32_t flags, const mxq_sr* sr,
                                             const mxq_nvfp4_out* rowwise,
                                             const mxq_nvfp4_out* columnwise,
                                             const mxq_fp8_out* fp8_rowwise, void* stream);


#ifdef __cplusplus
}
#endif
#endif /* MXQ_H */
