// mxq_api.cpp -- the C ABI of include/mxq.h: argument checks, launch planning
// and kernel launches.  Host code only; nothing here allocates, synchronizes,
// memsets or reads the environment (TransformerEngine PR #2564: the per-call
// allocation of a 4-byte scheduler workspace was the whole NVFP4 regression;
// PR #2555 review: no per-call getenv on the quantize path).
#include "mxq.h"

#include <hip/hip_runtime_api.h>

#include <cstring>

#include "mxq_internal.hpp"

namespace {

constexpr int64_t kMaxGridThreads = 0xFFFFFFFFll;    // 1-D grids only; threads per launch < 2^32
constexpr int64_t kMaxRows = (1ll << 31) - 128;
constexpr int64_t kMaxElems = 1ll << 40;
constexpr int64_t kMaxGroupK = 1ll << 26;   // the grouped kernels address a tile row with 32-bit offsets

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// a * b < lim for a, b >= 0 and lim >= 1, without forming the product.
bool product_below(int64_t a, int64_t b, int64_t lim) { return a == 0 || b <= (lim - 1) / a; }

// A [rows][ld] array whose rows hold len elements spans (rows - 1) * ld + len
// elements: below kMaxElems (rows >= 1, 0 <= len).  Bounding every array this way
// keeps the kernels' int64 index arithmetic exact.
bool extent_ok(int64_t rows, int64_t ld, int64_t len) {
    return len < kMaxElems && product_below(rows - 1, ld, kMaxElems - len);
}

// The largest index of a [rows][cols] array addressed as r * s_r + c * s_c is below
// kMaxElems (rows, cols >= 1; s_r, s_c >= 0).
bool index2_ok(int64_t rows, int64_t s_r, int64_t cols, int64_t s_c) {
    if (!product_below(rows - 1, s_r, kMaxElems) || !product_below(cols - 1, s_c, kMaxElems)) return false;
    return (rows - 1) * s_r < kMaxElems - (cols - 1) * s_c;
}

int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

}  // namespace

namespace mxq {
// The argument checks of the grouped call, everything but the workspace (which the
// call without a workspace replaces by its own array): MXQ_OK and the total row
// count, or the first error.  Nothing is enqueued.
mxq_status grouped_check(const uint16_t* x_bf16, int64_t k, const int64_t* split_sections, int64_t num_sections,
                         uint32_t flags, const mxq_nvfp4_out* rowwise, const mxq_nvfp4_out* columnwise,
                         const mxq_fp8_out* fp8_rowwise, const mxq_amax* amax, int64_t* total_rows_out) {
    if (k <= 0 || !split_sections || num_sections < 1) return MXQ_ERR_INVALID_ARGUMENT;
    if (num_sections > MXQ_MAX_SECTIONS || k > kMaxGroupK) return MXQ_ERR_UNSUPPORTED;
    if (flags == 0 || (flags & ~(uint32_t)(MXQ_ROWWISE | MXQ_COLUMNWISE | MXQ_FP8_ROWWISE)))
        return MXQ_ERR_INVALID_ARGUMENT;
    if (k % 128 != 0) return MXQ_ERR_MISALIGNED;
    int64_t total_rows = 0;
    for (int64_t s = 0; s < num_sections; ++s) {
        const int64_t ms = split_sections[s];
        if (ms < 0) return MXQ_ERR_INVALID_ARGUMENT;
        if (ms % 128 != 0) return MXQ_ERR_MISALIGNED;
        total_rows += ms;
        if (total_rows > kMaxRows) return MXQ_ERR_UNSUPPORTED;
    }
    if (total_rows * k >= kMaxElems) return MXQ_ERR_UNSUPPORTED;
    const bool row = flags & MXQ_ROWWISE, col = flags & MXQ_COLUMNWISE, fp8 = flags & MXQ_FP8_ROWWISE;
    if (row && (!rowwise || !rowwise->global_scales || (total_rows > 0 && (!rowwise->codes || !rowwise->block_scales))))
        return MXQ_ERR_INVALID_ARGUMENT;
    if (col && (!columnwise || !columnwise->global_scales ||
                (total_rows > 0 && (!columnwise->codes || !columnwise->block_scales))))
        return MXQ_ERR_INVALID_ARGUMENT;
    if (fp8 && total_rows > 0 && (!fp8_rowwise || !fp8_rowwise->codes || !fp8_rowwise->scales))
        return MXQ_ERR_INVALID_ARGUMENT;
    if (total_rows > 0 && !x_bf16) return MXQ_ERR_INVALID_ARGUMENT;
    if (x_bf16 && !aligned(x_bf16, 16)) return MXQ_ERR_MISALIGNED;
    if (row && (!aligned(rowwise->codes, 16) || !aligned(rowwise->block_scales, 16) ||
                !aligned(rowwise->global_scales, 4)))
        return MXQ_ERR_MISALIGNED;
    if (col && (!aligned(columnwise->codes, 16) || !aligned(columnwise->block_scales, 16) ||
                !aligned(columnwise->global_scales, 4)))
        return MXQ_ERR_MISALIGNED;
    if (fp8 && total_rows > 0 && (!aligned(fp8_rowwise->codes, 16) || !aligned(fp8_rowwise->scales, 4)))
        return MXQ_ERR_MISALIGNED;
    // caller-supplied maxima: all or none of the requested NVFP4 directions
    const bool given = amax && (amax->row_in || amax->col_in);
    if (given && ((row && !amax->row_in) || (col && !amax->col_in))) return MXQ_ERR_INVALID_ARGUMENT;
    if (amax && (!aligned(amax->row_in, 4) || !aligned(amax->col_in, 4) || !aligned(amax->row_out, 4) ||
                 !aligned(amax->col_out, 4)))
        return MXQ_ERR_MISALIGNED;
    const int64_t n_ct = k / 128;
    if ((total_rows / 128) * n_ct * 2 * 64 > kMaxGridThreads) return MXQ_ERR_UNSUPPORTED;
    if (!row && !col && ceil_div(total_rows * (k / 128), 32) * 256 > kMaxGridThreads) return MXQ_ERR_UNSUPPORTED;
    *total_rows_out = total_rows;
    return MXQ_OK;
}
}  // namespace mxq

extern "C" {

const char* mxq_status_string(mxq_status s) {
    switch (s) {
        case MXQ_OK: return "MXQ_OK";
        case MXQ_ERR_INVALID_ARGUMENT: return "MXQ_ERR_INVALID_ARGUMENT";
        case MXQ_ERR_MISALIGNED: return "MXQ_ERR_MISALIGNED";
        case MXQ_ERR_WORKSPACE_TOO_SMALL: return "MXQ_ERR_WORKSPACE_TOO_SMALL";
        case MXQ_ERR_UNSUPPORTED: return "MXQ_ERR_UNSUPPORTED";
        case MXQ_ERR_HIP: return "MXQ_ERR_HIP";
    }
    return "MXQ_ERR_UNKNOWN";
}

const char* mxq_version(void) { return "mxq 0.1.0 gfx950"; }

mxq_status mxq_quant_fp8_1x128(const uint16_t* x_bf16, int64_t m, int64_t k, int64_t ldx,
                               uint8_t* q_e4m3, int64_t ldq,
                               float* scales, int64_t scale_stride_row, int64_t scale_stride_group,
                               void* stream) {
    if (m < 0 || k <= 0 || ldx < k || ldq < k || scale_stride_row < 0 || scale_stride_group < 0)
        return MXQ_ERR_INVALID_ARGUMENT;
    if (k % 128 != 0 || ldx % 8 != 0 || ldq % 16 != 0) return MXQ_ERR_MISALIGNED;
    if (m == 0) return MXQ_OK;
    if (!x_bf16 || !q_e4m3 || !scales) return MXQ_ERR_INVALID_ARGUMENT;
    if (!aligned(x_bf16, 16) || !aligned(q_e4m3, 16) || !aligned(scales, 4)) return MXQ_ERR_MISALIGNED;
    if (m > kMaxRows || !extent_ok(m, ldx, k) || !extent_ok(m, ldq, k) ||
        !index2_ok(m, scale_stride_row, k / 128, scale_stride_group))
        return MXQ_ERR_UNSUPPORTED;
    const int64_t blocks = ceil_div(m * (k / 128), 32);
    if (blocks * 256 > kMaxGridThreads) return MXQ_ERR_UNSUPPORTED;
    mxq::Fp8Args a{x_bf16, q_e4m3, scales, m, k, ldx, ldq, scale_stride_row, scale_stride_group};
    return mxq::launch_quant_fp8_1x128(a, static_cast<hipStream_t>(stream)) == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

mxq_status mxq_swiglu_quant_fp8(const uint16_t* gate_bf16, int64_t ld_gate, const uint16_t* up_bf16, int64_t ld_up,
                                int64_t m, int64_t n, uint8_t* q_e4m3, int64_t ldq,
                                float* scales, int64_t scale_stride_row, int64_t scale_stride_group, void* stream) {
    if (m < 0 || n <= 0 || ld_gate < n || ld_up < n || ldq < n || scale_stride_row < 0 || scale_stride_group < 0)
        return MXQ_ERR_INVALID_ARGUMENT;
    if (n % 128 != 0 || ld_gate % 8 != 0 || ld_up % 8 != 0 || ldq % 16 != 0) return MXQ_ERR_MISALIGNED;
    if (m == 0) return MXQ_OK;
    if (!gate_bf16 || !up_bf16 || !q_e4m3 || !scales) return MXQ_ERR_INVALID_ARGUMENT;
    if (!aligned(gate_bf16, 16) || !aligned(up_bf16, 16) || !aligned(q_e4m3, 16) || !aligned(scales, 4))
        return MXQ_ERR_MISALIGNED;
    if (m > kMaxRows || !extent_ok(m, ld_gate, n) || !extent_ok(m, ld_up, n) || !extent_ok(m, ldq, n) ||
        !index2_ok(m, scale_stride_row, n / 128, scale_stride_group))
        return MXQ_ERR_UNSUPPORTED;
    if (ceil_div(m * (n / 128), 32) * 256 > kMaxGridThreads) return MXQ_ERR_UNSUPPORTED;
    mxq::SwigluFp8Args a{gate_bf16, up_bf16, q_e4m3, scales, m, n, ld_gate, ld_up, ldq, scale_stride_row,
                         scale_stride_group};
    return mxq::launch_swiglu_quant_fp8(a, static_cast<hipStream_t>(stream)) == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

mxq_status mxq_hadamard_quant_fp8(const uint16_t* pe, int64_t ld_pe, int32_t d_pe,
                                  const uint16_t* nope, int64_t ld_nope, int64_t m,
                                  uint8_t* q_e4m3, float* scales, void* stream) {
    if (m < 0 || d_pe < 0 || d_pe > 128) return MXQ_ERR_INVALID_ARGUMENT;
    if (d_pe % 8 != 0) return MXQ_ERR_MISALIGNED;
    if (d_pe > 0 && ld_pe < d_pe) return MXQ_ERR_INVALID_ARGUMENT;
    if (d_pe < 128 && ld_nope < 128 - d_pe) return MXQ_ERR_INVALID_ARGUMENT;
    if ((d_pe > 0 && ld_pe % 8 != 0) || (d_pe < 128 && ld_nope % 8 != 0)) return MXQ_ERR_MISALIGNED;
    if (m == 0) return MXQ_OK;
    if ((d_pe > 0 && !pe) || (d_pe < 128 && !nope) || !q_e4m3 || !scales) return MXQ_ERR_INVALID_ARGUMENT;
    if ((d_pe > 0 && !aligned(pe, 16)) || (d_pe < 128 && !aligned(nope, 16)) || !aligned(q_e4m3, 16) ||
        !aligned(scales, 4))
        return MXQ_ERR_MISALIGNED;
    if (m > kMaxRows || (d_pe > 0 && !extent_ok(m, ld_pe, d_pe)) || (d_pe < 128 && !extent_ok(m, ld_nope, 128 - d_pe)))
        return MXQ_ERR_UNSUPPORTED;
    if (ceil_div(m, 64) * 256 > kMaxGridThreads) return MXQ_ERR_UNSUPPORTED;
    mxq::DsaArgs a{pe, nope, q_e4m3, scales, ld_pe, ld_nope, m, d_pe, 1, 1, 0};
    return mxq::launch_hadamard_quant_fp8(a, static_cast<hipStream_t>(stream)) == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

mxq_status mxq_hadamard_quant_fp8_ex(const uint16_t* pe, int64_t ld_pe, int32_t d_pe,
                                     const uint16_t* nope, int64_t ld_nope, int64_t m, uint32_t options,
                                     int64_t heads, uint8_t* q_e4m3, float* scales,
                                     int64_t scale_stride_token, int64_t scale_stride_head, void* stream) {
    if (options & ~(uint32_t)MXQ_FP8_UE8M0) return MXQ_ERR_INVALID_ARGUMENT;
    if (heads <= 0 || scale_stride_token < 0 || scale_stride_head < 0) return MXQ_ERR_INVALID_ARGUMENT;
    if (m < 0 || d_pe < 0 || d_pe > 128) return MXQ_ERR_INVALID_ARGUMENT;
    if (d_pe % 8 != 0) return MXQ_ERR_MISALIGNED;
    if (d_pe > 0 && ld_pe < d_pe) return MXQ_ERR_INVALID_ARGUMENT;
    if (d_pe < 128 && ld_nope < 128 - d_pe) return MXQ_ERR_INVALID_ARGUMENT;
    if ((d_pe > 0 && ld_pe % 8 != 0) || (d_pe < 128 && ld_nope % 8 != 0)) return MXQ_ERR_MISALIGNED;
    if (m == 0) return MXQ_OK;
    if ((d_pe > 0 && !pe) || (d_pe < 128 && !nope) || !q_e4m3 || !scales) return MXQ_ERR_INVALID_ARGUMENT;
    if ((d_pe > 0 && !aligned(pe, 16)) || (d_pe < 128 && !aligned(nope, 16)) || !aligned(q_e4m3, 16) ||
        !aligned(scales, 4))
        return MXQ_ERR_MISALIGNED;
    if (m > kMaxRows || (d_pe > 0 && !extent_ok(m, ld_pe, d_pe)) || (d_pe < 128 && !extent_ok(m, ld_nope, 128 - d_pe)) ||
        !index2_ok(heads < m ? ceil_div(m, heads) : 1, scale_stride_token, heads < m ? heads : m, scale_stride_head))
        return MXQ_ERR_UNSUPPORTED;
    if (ceil_div(m, 64) * 256 > kMaxGridThreads) return MXQ_ERR_UNSUPPORTED;
    mxq::DsaArgs a{pe, nope, q_e4m3, scales, ld_pe, ld_nope, m, d_pe, heads, scale_stride_token, scale_stride_head};
    return mxq::launch_hadamard_quant_fp8(a, static_cast<hipStream_t>(stream), (options & MXQ_FP8_UE8M0) != 0) ==
                   hipSuccess
               ? MXQ_OK
               : MXQ_ERR_HIP;
}

mxq_status mxq_quant_fp8_blockwise(const uint16_t* x_bf16, int64_t m, int64_t k, int64_t ldx, uint32_t options,
                                   const mxq_fp8_block_out* rowwise, const mxq_fp8_block_out* columnwise,
                                   void* stream) {
    if (options & ~(uint32_t)MXQ_FP8_UE8M0) return MXQ_ERR_INVALID_ARGUMENT;
    if (!rowwise && !columnwise) return MXQ_ERR_INVALID_ARGUMENT;
    if (m < 0 || k <= 0 || ldx < k) return MXQ_ERR_INVALID_ARGUMENT;
    if (k % 128 != 0 || ldx % 8 != 0) return MXQ_ERR_MISALIGNED;
    if (rowwise) {
        if (rowwise->ld < k || rowwise->scale_stride_a < 0 || rowwise->scale_stride_b < 0)
            return MXQ_ERR_INVALID_ARGUMENT;
        if (rowwise->ld % 16 != 0) return MXQ_ERR_MISALIGNED;
    }
    if (columnwise) {
        if (columnwise->ld < m || columnwise->scale_stride_a < 0 || columnwise->scale_stride_b < 0)
            return MXQ_ERR_INVALID_ARGUMENT;
        if (columnwise->ld % 16 != 0) return MXQ_ERR_MISALIGNED;
    }
    if (m == 0) return MXQ_OK;
    if (!x_bf16 || (rowwise && (!rowwise->codes || !rowwise->scales)) ||
        (columnwise && (!columnwise->codes || !columnwise->scales)))
        return MXQ_ERR_INVALID_ARGUMENT;
    if (!aligned(x_bf16, 16) || (rowwise && (!aligned(rowwise->codes, 16) || !aligned(rowwise->scales, 4))) ||
        (columnwise && (!aligned(columnwise->codes, 16) || !aligned(columnwise->scales, 4))))
        return MXQ_ERR_MISALIGNED;
    if (m > kMaxRows || !extent_ok(m, ldx, k)) return MXQ_ERR_UNSUPPORTED;
    if (rowwise && (!extent_ok(m, rowwise->ld, k) ||
                    !index2_ok(m, rowwise->scale_stride_a, k / 128, rowwise->scale_stride_b)))
        return MXQ_ERR_UNSUPPORTED;
    if (columnwise && (!extent_ok(k, columnwise->ld, m) ||
                       !index2_ok(k, columnwise->scale_stride_a, ceil_div(m, 128), columnwise->scale_stride_b)))
        return MXQ_ERR_UNSUPPORTED;
    const bool ue8m0 = (options & MXQ_FP8_UE8M0) != 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!columnwise) {                                    // row-wise alone: the streaming kernel
        if (ceil_div(m * (k / 128), 32) * 256 > kMaxGridThreads) return MXQ_ERR_UNSUPPORTED;
        mxq::Fp8Args a{x_bf16, rowwise->codes, rowwise->scales, m, k, ldx, rowwise->ld,
                       rowwise->scale_stride_a, rowwise->scale_stride_b};
        return mxq::launch_quant_fp8_1x128(a, st, ue8m0) == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
    }
    if (ceil_div(m, 128) * (k / 128) > 0xFFFFFFFFll) return MXQ_ERR_UNSUPPORTED;
    mxq::Fp8BlockArgs a{};
    a.x = x_bf16;
    a.m = m;
    a.k = k;
    a.ldx = ldx;
    if (rowwise) {
        a.rq = rowwise->codes;
        a.rld = rowwise->ld;
        a.rs = rowwise->scales;
        a.rsr = rowwise->scale_stride_a;
        a.rsg = rowwise->scale_stride_b;
    }
    a.cq = columnwise->codes;
    a.cld = columnwise->ld;
    a.cs = columnwise->scales;
    a.csc = columnwise->scale_stride_a;
    a.csb = columnwise->scale_stride_b;
    return mxq::launch_quant_fp8_blockwise(a, ue8m0, st) == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

size_t mxq_hadamard_quant_nvfp4_workspace_size(int64_t m) {
    if (m <= 0 || m > kMaxRows) return 0;
    return (size_t)round256(mxq::kDsaPartialsOffset + 4 * ceil_div(m, 64));
}

mxq_status mxq_hadamard_quant_nvfp4(const uint16_t* pe, int64_t ld_pe, int32_t d_pe,
                                    const uint16_t* nope, int64_t ld_nope, int64_t m,
                                    const float* amax_in, float* amax_out,
                                    uint8_t* codes, uint8_t* block_scales, float* global_scale,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    if (m < 0 || d_pe < 0 || d_pe > 128) return MXQ_ERR_INVALID_ARGUMENT;
    if (d_pe % 8 != 0) return MXQ_ERR_MISALIGNED;
    if (d_pe > 0 && ld_pe < d_pe) return MXQ_ERR_INVALID_ARGUMENT;
    if (d_pe < 128 && ld_nope < 128 - d_pe) return MXQ_ERR_INVALID_ARGUMENT;
    if ((d_pe > 0 && ld_pe % 8 != 0) || (d_pe < 128 && ld_nope % 8 != 0)) return MXQ_ERR_MISALIGNED;
    if (!global_scale) return MXQ_ERR_INVALID_ARGUMENT;
    if (!aligned(global_scale, 4) || !aligned(amax_in, 4) || !aligned(amax_out, 4)) return MXQ_ERR_MISALIGNED;
    if (m > kMaxRows) return MXQ_ERR_UNSUPPORTED;
    if (m > 0 && ((d_pe > 0 && !extent_ok(m, ld_pe, d_pe)) || (d_pe < 128 && !extent_ok(m, ld_nope, 128 - d_pe))))
        return MXQ_ERR_UNSUPPORTED;
    if (m > 0) {
        if ((d_pe > 0 && !pe) || (d_pe < 128 && !nope) || !codes || !block_scales || !workspace)
            return MXQ_ERR_INVALID_ARGUMENT;
        if ((d_pe > 0 && !aligned(pe, 16)) || (d_pe < 128 && !aligned(nope, 16)) || !aligned(codes, 16) ||
            !aligned(block_scales, 16) || !aligned(workspace, 256))
            return MXQ_ERR_MISALIGNED;
        if (workspace_bytes < mxq_hadamard_quant_nvfp4_workspace_size(m)) return MXQ_ERR_WORKSPACE_TOO_SMALL;
    }
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    mxq::DsaNvfp4Args a{};
    a.pe = pe;
    a.nope = nope;
    a.ld_pe = ld_pe;
    a.ld_nope = ld_nope;
    a.m = m;
    a.d_pe = d_pe;
    a.n_wg = (int32_t)ceil_div(m, 64);
    a.codes = codes;
    a.scales = block_scales;
    a.global_scale = global_scale;
    a.amax_in = amax_in;
    a.amax_out = amax_out;
    a.table = m > 0 ? reinterpret_cast<float4*>(ws + mxq::kDsaTableOffset) : nullptr;
    a.partials = m > 0 ? reinterpret_cast<float*>(ws + mxq::kDsaPartialsOffset) : nullptr;
    return mxq::launch_hadamard_quant_nvfp4(a, static_cast<hipStream_t>(stream)) == hipSuccess ? MXQ_OK
                                                                                              : MXQ_ERR_HIP;
}

size_t mxq_group_rht_quant_nvfp4_workspace_size(int64_t total_rows, int64_t k, int64_t num_sections,
                                                uint32_t flags) {
    if (total_rows < 0 || k <= 0 || num_sections <= 0) return 0;
    if (total_rows > kMaxRows || k > kMaxGroupK) return 0;         // outside the supported profile
    if (!(flags & (MXQ_ROWWISE | MXQ_COLUMNWISE))) return 0;
    // status line, scale tables and the single-read form's partial words of one
    // launch group, then the amax pass's 8-byte partials: one per 16 rows and
    // kAmaxCols = 1024 columns (or part) of the largest group, bounded by all rows
    const int64_t partials = (total_rows / mxq::kAmaxRows) * ceil_div(k, mxq::kAmaxCols);
    return (size_t)round256(mxq::kPartialsOffset + 8 * partials);
}

mxq_status mxq_group_rht_quant_nvfp4(const uint16_t* x_bf16, int64_t k,
                                     const int64_t* split_sections, int64_t num_sections,
                                     uint16_t rht_sign_mask, uint32_t flags, const mxq_sr* sr,
                                     const mxq_nvfp4_out* rowwise, const mxq_nvfp4_out* columnwise,
                                     const mxq_fp8_out* fp8_rowwise,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    return mxq_group_rht_quant_nvfp4_with_amax(x_bf16, k, split_sections, num_sections, rht_sign_mask, flags, sr,
                                               rowwise, columnwise, fp8_rowwise, nullptr, workspace,
                                               workspace_bytes, stream);
}

mxq_status mxq_group_rht_quant_nvfp4_with_amax(const uint16_t* x_bf16, int64_t k,
                                               const int64_t* split_sections, int64_t num_sections,
                                               uint16_t rht_sign_mask, uint32_t flags, const mxq_sr* sr,
                                               const mxq_nvfp4_out* rowwise, const mxq_nvfp4_out* columnwise,
                                               const mxq_fp8_out* fp8_rowwise, const mxq_amax* amax,
                                               void* workspace, size_t workspace_bytes, void* stream) {
    // ---- checks (nothing is enqueued before all of them pass)
    int64_t total_rows = 0;
    const mxq_status c = mxq::grouped_check(x_bf16, k, split_sections, num_sections, flags, rowwise, columnwise,
                                            fp8_rowwise, amax, &total_rows);
    if (c != MXQ_OK) return c;
    const bool row = flags & MXQ_ROWWISE, col = flags & MXQ_COLUMNWISE, fp8 = flags & MXQ_FP8_ROWWISE;
    const bool given = amax && (amax->row_in || amax->col_in);
    const bool sr_row = row && sr && sr->row_offsets;
    const bool sr_col = col && sr && sr->col_offsets;
    const size_t need = mxq_group_rht_quant_nvfp4_workspace_size(total_rows, k, num_sections, flags);
    if (need > 0) {
        if (!workspace) return MXQ_ERR_INVALID_ARGUMENT;
        if (workspace_bytes < need) return MXQ_ERR_WORKSPACE_TOO_SMALL;
        if (!aligned(workspace, 256)) return MXQ_ERR_MISALIGNED;
    }
    const int64_t n_ct = k / 128;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!row && !col) {
        // the FP8 1x128 output alone needs no tensor scale: one plain FP8 launch
        if (total_rows == 0) return MXQ_OK;
        mxq::Fp8Args a{x_bf16, fp8_rowwise->codes, fp8_rowwise->scales, total_rows, k, k, k, k / 128, 1};
        return mxq::launch_quant_fp8_1x128(a, st) == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
    }

    // ---- launch groups of up to kGroupSections sections
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    int64_t row0 = 0;
    for (int64_t s0 = 0; s0 < num_sections; s0 += mxq::kGroupSections) {
        const int ns = (int)((num_sections - s0) < mxq::kGroupSections ? (num_sections - s0) : mxq::kGroupSections);
        mxq::Nvfp4Group g;
        std::memset(&g, 0, sizeof(g));
        g.x = x_bf16 ? x_bf16 + row0 * k : nullptr;
        g.k = k;
        if (row) {
            g.row_codes = rowwise->codes ? rowwise->codes + row0 * (k / 2) : nullptr;
            g.row_scales = rowwise->block_scales ? rowwise->block_scales + row0 * (k / 16) : nullptr;
            g.row_global = rowwise->global_scales + s0;
        }
        if (col) {
            g.col_codes = columnwise->codes ? columnwise->codes + row0 * k / 2 : nullptr;
            g.col_scales = columnwise->block_scales ? columnwise->block_scales + row0 * k / 16 : nullptr;
            g.col_global = columnwise->global_scales + s0;
        }
        if (fp8 && total_rows > 0) {
            g.fp8_codes = fp8_rowwise->codes + row0 * k;
            g.fp8_scales = fp8_rowwise->scales + row0 * (k / 128);
        }
        g.tables = reinterpret_cast<float4*>(ws + mxq::kTablesOffset);
        g.partials = reinterpret_cast<uint64_t*>(ws + mxq::kPartialsOffset);
        g.seed = sr ? sr->seed : 0;
        g.sign_mask = rht_sign_mask;
        g.sr_row = sr_row ? 1u : 0u;
        g.sr_col = sr_col ? 1u : 0u;
        g.num_sections = ns;
        g.n_ctiles = (int32_t)n_ct;
        int64_t tt = 0, rows_group = 0;
        for (int i = 0; i < ns; ++i) {
            const int64_t ms = split_sections[s0 + i];
            g.tt_start[i] = (int32_t)tt;
            tt += ms / 128;
            rows_group += ms;
            g.row_off[i] = sr_row ? sr->row_offsets[s0 + i] : 0;
            g.col_off[i] = sr_col ? sr->col_offsets[s0 + i] : 0;
        }
        g.tt_start[ns] = (int32_t)tt;
        if (given) {
            g.amax_in_row = row ? amax->row_in + s0 : nullptr;
            g.amax_in_col = col ? amax->col_in + s0 : nullptr;
        }
        if (amax) {
            g.amax_out_row = (row && amax->row_out) ? amax->row_out + s0 : nullptr;
            g.amax_out_col = (col && amax->col_out) ? amax->col_out + s0 : nullptr;
        }
        g.total_tiles = (int32_t)(tt * n_ct);
        uint32_t* const slots = reinterpret_cast<uint32_t*>(ws + mxq::kSlotsOffset);
        uint32_t* const status = reinterpret_cast<uint32_t*>(ws + mxq::kStatusOffset);
        if (mxq::launch_nvfp4_group(g, flags, slots, status, st) != hipSuccess) return MXQ_ERR_HIP;
        row0 += rows_group;
    }
    return MXQ_OK;
}

}  // extern "C"
