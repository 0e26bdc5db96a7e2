// mxq_fp8_block.hip -- FP8 block variants from one read of x (gfx950): row-wise
// 1x128 groups and column-wise 128x1 blocks whose codes are written transposed
// (row c of the output holds column c of x), optionally with UE8M0 (power-of-two)
// scales.
//
// FP8 recipe: onnxruntime PR #33644 (Description) -- s = max(amax, 1e-10) * F(1/448),
// E4M3(fl(x / s)) nearest-even, saturating.  Scale layouts and use_ue8m0:
// TensorRT-LLM PR #15158 (review of the scale normalization of
// fp8_quantize_1x128_sf_transpose); UE8M0 reads as the recipe's FP32 scale rounded
// up to the nearest power of two.
//
// A 256-thread work-group stages one 128 x 128 BF16 tile in LDS with rows padded to
// 65 dwords, so that both read patterns below are free of bank conflicts:
//   row-wise     thread (row t/2, half t&1) reads 32 dwords of its row;
//   column-wise  thread (column t&127, half t/128) reads 64 halfwords down its column
//                (the 64 lanes of a wave read 64 consecutive columns of one row).
#include "mxq_device.hpp"
#include "mxq_internal.hpp"

namespace mxq {

namespace {

constexpr int kRowDwords = 65;        // 128 BF16 + 2 of padding
constexpr int kCodeDwords = 36;       // a column's 128 codes + 16 bytes of padding (16-byte aligned rows)

// Bytes equal to 0xFF (the conversion's code for a NaN input) become 0x7F.
__device__ __forceinline__ uint32_t nan_to_7f(uint32_t c) {
    uint32_t ff = c & (c >> 1) & (c >> 2) & (c >> 3) & (c >> 4) & (c >> 5) & (c >> 6) & (c >> 7) & 0x01010101u;
    return c ^ (ff * 0x80u);
}

// fl(x / s): a product when s is a power of two (its reciprocal is exact), else the
// correctly rounded quotient from the reciprocal.
template <bool UE8M0>
__device__ __forceinline__ float quotient(float x, float s, float y) {
    return UE8M0 ? x * y : div_rn(x, s, y);
}

template <bool UE8M0>
__device__ __forceinline__ float block_scale(float amax) {
    const float s = (amax > k_floor() ? amax : k_floor()) * k_inv448();
    return UE8M0 ? pow2_ceil(s) : s;
}

}  // namespace

template <bool ROW, bool COL, bool UE8M0>
__global__ __launch_bounds__(256) void k_quant_fp8_blockwise(const Fp8BlockArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t tile[128 * kRowDwords];
    __shared__ uint32_t red[2][128];
    const int t = threadIdx.x;
    const int64_t n_ct = a.k >> 7;
    const int64_t rb = blockIdx.x / n_ct, ct = blockIdx.x - rb * n_ct;
    const int64_t row0 = rb * 128, c0 = ct * 128;

    // stage the tile: 2048 16-byte chunks, 8 per thread; rows past m are zeros
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int j = it * 256 + t;
        const int r = j >> 4, ch = j & 15;
        uint4 w = {0, 0, 0, 0};
        if (row0 + r < a.m) w = nt_load16(a.x + (row0 + r) * a.ldx + c0 + ch * 8);
        uint32_t* dst = tile + r * kRowDwords + ch * 4;
        dst[0] = w.x;
        dst[1] = w.y;
        dst[2] = w.z;
        dst[3] = w.w;
    }
    __syncthreads();

    // A whole row block with both outputs: the row codes, too, leave through LDS once
    // the column pass is done with it (kept in rc until then).
    const bool stage_rows = ROW && COL && row0 + 128 <= a.m;
    uint32_t rc[16];
    if (ROW) {
        const int r = t >> 1, half = t & 1;
        const uint32_t* src = tile + r * kRowDwords + half * 32;
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) m = absmax_pk(m, src[i]);
        m = fold_pk(m);
        const bool nan = m > 0x7F80u;                // a NaN in this half of the group
        if (nan) {
            m = 0;
#pragma unroll
            for (int i = 0; i < 32; ++i) m = absmax_pk_nonan(m, src[i]);
        }
        const uint32_t mo = __builtin_bit_cast(uint32_t, quad_swap<0xB1>(__builtin_bit_cast(float, m)));
        m = mo > m ? mo : m;
        const float s = block_scale<UE8M0>(bf16_mag(m));
        const float y = 1.0f / s, sd = fp8_divisor(s);
        const bool fix = nan || s == __builtin_inff();  // 0xFF codes: NaN inputs, or inf / inf
        uint32_t c[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t w0 = src[2 * j], w1 = src[2 * j + 1];
            c[j] = e4m3_pack4(quotient<UE8M0>(lo_bf16(w0), sd, y), quotient<UE8M0>(hi_bf16(w0), sd, y),
                              quotient<UE8M0>(lo_bf16(w1), sd, y), quotient<UE8M0>(hi_bf16(w1), sd, y));
            if (fix) c[j] = nan_to_7f(c[j]);
        }
        if (stage_rows) {
#pragma unroll
            for (int j = 0; j < 16; ++j) rc[j] = c[j];
            if (half == 0) a.rs[(row0 + r) * a.rsr + ct * a.rsg] = s;
        } else if (row0 + r < a.m) {
            uint4* dst = reinterpret_cast<uint4*>(a.rq + (row0 + r) * a.rld + c0 + half * 64);
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[q] = make_uint4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
            if (half == 0) a.rs[(row0 + r) * a.rsr + ct * a.rsg] = s;
        }
    }

    if (COL) {
        const int c = t & 127, half = t >> 7;
        const uint16_t* col = reinterpret_cast<const uint16_t*>(tile) + c;
        // max |x| of the half column without NaNs (|bits| above 0x7F80 are NaNs)
        uint32_t m = 0;
        bool nan = false;
#pragma unroll
        for (int i = 0; i < 64; ++i) {
            const uint32_t v = col[(half * 64 + i) * (2 * kRowDwords)] & 0x7FFFu;
            nan |= v > 0x7F80u;
            m = (v <= 0x7F80u && v > m) ? v : m;
        }
        red[half][c] = m | (nan ? 0x80000000u : 0u);
        __syncthreads();
        const uint32_t p0 = red[0][c], p1 = red[1][c];
        const uint32_t m0 = p0 & 0xFFFFu, m1 = p1 & 0xFFFFu;
        const float s = block_scale<UE8M0>(bf16_mag(m0 > m1 ? m0 : m1));
        const float y = 1.0f / s, sd = fp8_divisor(s);
        const bool fix = nan || s == __builtin_inff();
        uint32_t code[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = lo_bf16(col[(half * 64 + 4 * j + e) * (2 * kRowDwords)]);
            code[j] = e4m3_pack4(quotient<UE8M0>(v[0], sd, y), quotient<UE8M0>(v[1], sd, y),
                                 quotient<UE8M0>(v[2], sd, y), quotient<UE8M0>(v[3], sd, y));
            if (fix) code[j] = nan_to_7f(code[j]);
        }
        const int64_t r_first = row0 + half * 64;
        uint8_t* dst = a.cq + (c0 + c) * a.cld + r_first;
        if (row0 + 128 <= a.m) {
            // A whole row block (uniform over the work-group): the 128 x 128 codes go
            // through LDS (over the input tile, which both passes have read by the
            // barrier), so that 8 lanes store each column's 128 bytes as one line
            // instead of every lane storing 16-byte pieces of its own column.
            if (half == 0) a.cs[(c0 + c) * a.csc + rb * a.csb] = s;
            __syncthreads();
            uint32_t* stage = tile + c * kCodeDwords + half * 16;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint4*>(stage + 4 * q) = make_uint4(code[4 * q], code[4 * q + 1], code[4 * q + 2], code[4 * q + 3]);
            __syncthreads();
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int col = it * 32 + (t >> 3), part = t & 7;
                const uint4 v = *reinterpret_cast<const uint4*>(tile + col * kCodeDwords + part * 4);
                *reinterpret_cast<uint4*>(a.cq + (c0 + col) * a.cld + row0 + part * 16) = v;
            }
            if (stage_rows) {
                __syncthreads();                                  // the column lines are read
                uint32_t* rstage = tile + (t >> 1) * kCodeDwords + (t & 1) * 16;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<uint4*>(rstage + 4 * q) = make_uint4(rc[4 * q], rc[4 * q + 1], rc[4 * q + 2], rc[4 * q + 3]);
                __syncthreads();
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int row = it * 32 + (t >> 3), part = t & 7;
                    const uint4 v = *reinterpret_cast<const uint4*>(tile + row * kCodeDwords + part * 4);
                    *reinterpret_cast<uint4*>(a.rq + (row0 + row) * a.rld + c0 + part * 16) = v;
                }
            }
            return;
        }
        if (r_first + 64 <= a.m) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                reinterpret_cast<uint4*>(dst)[q] = make_uint4(code[4 * q], code[4 * q + 1], code[4 * q + 2], code[4 * q + 3]);
        } else {
            // the ragged last row block: only the rows that exist
#pragma unroll
            for (int i = 0; i < 64; ++i)
                if (r_first + i < a.m) dst[i] = (uint8_t)(code[i >> 2] >> (8 * (i & 3)));
        }
        if (half == 0) a.cs[(c0 + c) * a.csc + rb * a.csb] = s;
    }
}

hipError_t launch_quant_fp8_blockwise(const Fp8BlockArgs& a, bool ue8m0, hipStream_t stream) {
    const unsigned grid = (unsigned)(((a.m + 127) / 128) * (a.k / 128));
    const bool row = a.rq != nullptr, col = a.cq != nullptr;
#define MXQ_FP8B(R, C, U) hipLaunchKernelGGL((k_quant_fp8_blockwise<R, C, U>), dim3(grid), dim3(256), 0, stream, a)
    if (row && col) {
        if (ue8m0) MXQ_FP8B(true, true, true); else MXQ_FP8B(true, true, false);
    } else if (col) {
        if (ue8m0) MXQ_FP8B(false, true, true); else MXQ_FP8B(false, true, false);
    } else {
        return hipErrorInvalidValue;
    }
#undef MXQ_FP8B
    return hipGetLastError();
}

}  // namespace mxq
