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
//   column-wise  thread (wave w, lane 16 q + pl) reads the dword of columns 2p, 2p+1
//                (p = 16 w + pl) in rows 64 a + 16 q + b, once each (the four
//                quarters' rows are 16 rows = 16 banks apart).
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

// Packed max |x| of BF16 pairs per half, a half that is a NaN (|bits| > 0x7F80)
// counting as 0.
__device__ __forceinline__ uint32_t absmax_pk_nonan_halves(uint32_t acc, uint32_t p) {
    const uint32_t lo = p & 0x7FFFu, hi = (p >> 16) & 0x7FFFu;
    return absmax_pk(acc, (lo > 0x7F80u ? 0u : lo) | (hi > 0x7F80u ? 0u : hi << 16));
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
    const int t = threadIdx.x;
    const int64_t n_ct = a.k >> 7;
    // Work-groups are dealt to the 8 XCDs in turn (b % 8), each with its own L2.  When
    // the tiles split evenly, XCD x takes the contiguous tiles x N/8 .. (x+1) N/8 - 1, so
    // that the 4-byte scales of one row block (one line per row across its k/128
    // tiles) are all written through one L2 and leave as whole lines.
    const int64_t n_tiles = (int64_t)gridDim.x;
    const int64_t tile_id = n_tiles % 8 == 0 ? (int64_t)(blockIdx.x % 8) * (n_tiles / 8) + blockIdx.x / 8
                                             : (int64_t)blockIdx.x;
    const int64_t rb = tile_id / n_ct, ct = tile_id - rb * n_ct;
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
        // Thread (wave w, lane q * 16 + pl) takes columns 2p and 2p + 1, p = 16 w + pl
        // (one BF16 pair, one dword of each row), over the 32 rows 64 a + 16 q + b
        // (a = 0, 1; b = 0 .. 15).  One 32-bit read per row brings both columns, and
        // each value is read from LDS once.  For a fixed (a, b) the four quarters' rows
        // lie 16 rows apart, 16 x 65 dwords = 16 banks modulo 64, and the 16 pairs of a
        // quarter take consecutive banks: a wave's read is free of bank conflicts.  The
        // four threads of a column pair are lanes pl + 16 q of one wave, so the column
        // maxima meet over lane shuffles, with no LDS exchange and no barrier.
        const int lane = t & 63, q = lane >> 4, p = (t >> 6) * 16 + (lane & 15);
        uint32_t vv[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) vv[i] = tile[(64 * (i >> 4) + 16 * q + (i & 15)) * kRowDwords + p];
        // per-column max |x| (packed halves: column 2p low, 2p + 1 high), NaNs aside
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) m = absmax_pk(m, vv[i]);
        uint32_t nan = ((m & 0xFFFFu) > 0x7F80u ? 1u : 0u) | ((m >> 16) > 0x7F80u ? 2u : 0u);
        if (nan) {
            m = 0;
#pragma unroll
            for (int i = 0; i < 32; ++i) m = absmax_pk_nonan_halves(m, vv[i]);
        }
#pragma unroll
        for (int o = 16; o < 64; o <<= 1) {
            m = absmax_pk(m, shfl_xor_u32(m, o));
            nan |= shfl_xor_u32(nan, o);
        }
        float sc[2], yc[2], sdc[2];
        bool fixc[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            sc[h] = block_scale<UE8M0>(bf16_mag(h ? m >> 16 : m & 0xFFFFu));
            yc[h] = 1.0f / sc[h];
            sdc[h] = fp8_divisor(sc[h]);
            fixc[h] = ((nan >> h) & 1u) || sc[h] == __builtin_inff();   // 0xFF codes: NaN inputs, or inf / inf
        }
        // code[h][a][j]: column 2p + h, rows 64 a + 16 q + 4 j .. + 3
        uint32_t code[2][2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t w = vv[a2 * 16 + 4 * j + e];
                        v[e] = h ? hi_bf16(w) : lo_bf16(w);
                    }
                    uint32_t cw = e4m3_pack4(quotient<UE8M0>(v[0], sdc[h], yc[h]), quotient<UE8M0>(v[1], sdc[h], yc[h]),
                                             quotient<UE8M0>(v[2], sdc[h], yc[h]), quotient<UE8M0>(v[3], sdc[h], yc[h]));
                    if (fixc[h]) cw = nan_to_7f(cw);
                    code[h][a2][j] = cw;
                }
        if (q == 0) {
#pragma unroll
            for (int h = 0; h < 2; ++h) a.cs[(c0 + 2 * p + h) * a.csc + rb * a.csb] = sc[h];
        }
        if (row0 + 128 <= a.m) {
            // A whole row block (uniform over the work-group): the 128 x 128 codes go
            // through LDS (over the input tile, which both passes have read by the
            // barrier), so that 8 lanes store each column's 128 bytes as one line
            // instead of every lane storing 16-byte pieces of its own columns.
            __syncthreads();
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int a2 = 0; a2 < 2; ++a2)
                    *reinterpret_cast<uint4*>(tile + (2 * p + h) * kCodeDwords + 16 * a2 + 4 * q) =
                        make_uint4(code[h][a2][0], code[h][a2][1], code[h][a2][2], code[h][a2][3]);
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
                for (int qq = 0; qq < 4; ++qq)
                    *reinterpret_cast<uint4*>(rstage + 4 * qq) =
                        make_uint4(rc[4 * qq], rc[4 * qq + 1], rc[4 * qq + 2], rc[4 * qq + 3]);
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
        // the ragged last row block: 16-byte runs where all 16 rows exist, else only
        // the rows that exist
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int a2 = 0; a2 < 2; ++a2) {
                const int64_t r_first = row0 + 64 * a2 + 16 * q;
                uint8_t* dst = a.cq + (c0 + 2 * p + h) * a.cld + r_first;
                if (r_first + 16 <= a.m) {
                    *reinterpret_cast<uint4*>(dst) =
                        make_uint4(code[h][a2][0], code[h][a2][1], code[h][a2][2], code[h][a2][3]);
                } else {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (r_first + i < a.m) dst[i] = (uint8_t)(code[h][a2][i >> 2] >> (8 * (i & 3)));
                }
            }
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
