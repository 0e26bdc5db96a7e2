// mxq_nvfp4.hip -- grouped NVFP4 quantization with a 16-point RHT on the
// column-wise operand (gfx950).
//
// The method: TransformerEngine PR #2564 "[NVFP4][MOE] Bug Fix for NVFP4 Grouped
// Quant" (Greptile summary: grouped row-wise + column-wise RHT cast fusion with a
// caller-provided workspace) and the review comments of PR #2555 on quantizer.cpp
// (RHT only for the column-wise operand; the RHT(x^T) intermediate has the input
// dtype; a separate column-wise RNG).  The NVFP4 per-tensor scale needs each
// section's amax before any code is final, so a call runs two kernels:
//
//   phase A  reads x once and writes, per work-group, the max |x| of its rows and
//            the max |H16 D x| of its 16-row column blocks (2 floats of workspace);
//   phase B  reduces its section's partials to the two tensor scales, re-reads its
//            128x128 tile (usually from the Infinity Cache) and writes every output.
//
// Phase-B tile (one wave64): lane = (tb, cc), tb = lane / 8 picks 16 rows, cc =
// lane % 8 picks 16 columns, so each lane owns 16 complete row blocks (1x16 along
// k) and 16 complete column blocks (16x1 along tokens): the row encode and the
// 16-point butterfly run entirely in registers.  Column codes (8 bytes per 16
// tokens) are transposed through LDS so that each column's 128 tokens leave as one
// 64-byte run.  Work-groups map to tiles XCD by XCD: the hardware deals
// work-groups round-robin over the 8 XCDs, and each XCD gets one contiguous range
// of tiles, so the partial cache lines of neighbouring tiles meet in one L2.
#include "mxq_device.hpp"
#include "mxq_internal.hpp"

namespace mxq {

namespace {

__device__ __forceinline__ int section_of_tile(const Nvfp4Group& G, int T) {
    int s = 0;
    for (int i = 1; i < G.num_sections; ++i)
        if (G.tt_start[i] <= T) s = i;
    return s;
}

__device__ __forceinline__ int section_of_chunk(const Nvfp4Group& G, int b) {
    int s = 0;
    for (int i = 1; i < G.num_sections; ++i)
        if (G.chunk_start[i] <= b) s = i;
    return s;
}

// dword i (0..7) of row t of the lane's 16x16 sub-tile
#define P(t, i) (((i) & 3) == 0 ? p[t][(i) >> 2].x : ((i) & 3) == 1 ? p[t][(i) >> 2].y : \
                 ((i) & 3) == 2 ? p[t][(i) >> 2].z : p[t][(i) >> 2].w)

__device__ __forceinline__ void load_subtile(uint4 (&p)[16][2], const uint16_t* base, int64_t k) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const uint4* src = reinterpret_cast<const uint4*>(base + (int64_t)t * k);
        p[t][0] = src[0];
        p[t][1] = src[1];
    }
}

// Tensor scale g = fl(max(A, F(1e-10)) * F(1/2688)).
__device__ __forceinline__ float tensor_scale(float amax) {
    return (amax > k_floor() ? amax : k_floor()) * k_inv2688();
}

// Block scale of a 1x16 block with amax a (a BF16 value): sc = E4M3(fl(fl(a/6)/g)),
// d = fl(E4M3value(sc) * g), y = fl(1/d).  yg = fl(1/g).
__device__ __forceinline__ void block_scale(float a, float g, float yg, uint32_t& sc, float& d, float& y) {
    const float a6 = a * k_inv6();
    const float t = div_rn(a6, g, yg);
    sc = e4m3_code(t);
    d = e4m3_value(sc) * g;
    y = 1.0f / d;
}

// Encode 16 values held as 8 packed BF16 pairs (element 2i in the low half of
// w[i]).  Returns the 8 code bytes (even element in the low nibble) and the scale.
template <bool SR>
__device__ __forceinline__ uint2 encode_block(const uint32_t (&w)[8], float g, float yg, const u32x4& rnd,
                                              uint32_t& sc_out) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = absmax_pk(m, w[i]);
    m = fold_pk(m);
    const bool nan_block = m > 0x7F80u;
    uint32_t sc;
    float d, y;
    block_scale(bf16_mag(m), g, yg, sc, d, y);
    uint32_t lo = 0, hi = 0;
    if (!SR) {
        lo = e2m1_pack2<0>(lo, div_rn(lo_bf16(w[0]), d, y), div_rn(hi_bf16(w[0]), d, y));
        lo = e2m1_pack2<1>(lo, div_rn(lo_bf16(w[1]), d, y), div_rn(hi_bf16(w[1]), d, y));
        lo = e2m1_pack2<2>(lo, div_rn(lo_bf16(w[2]), d, y), div_rn(hi_bf16(w[2]), d, y));
        lo = e2m1_pack2<3>(lo, div_rn(lo_bf16(w[3]), d, y), div_rn(hi_bf16(w[3]), d, y));
        hi = e2m1_pack2<0>(hi, div_rn(lo_bf16(w[4]), d, y), div_rn(hi_bf16(w[4]), d, y));
        hi = e2m1_pack2<1>(hi, div_rn(lo_bf16(w[5]), d, y), div_rn(hi_bf16(w[5]), d, y));
        hi = e2m1_pack2<2>(hi, div_rn(lo_bf16(w[6]), d, y), div_rn(hi_bf16(w[6]), d, y));
        hi = e2m1_pack2<3>(hi, div_rn(lo_bf16(w[7]), d, y), div_rn(hi_bf16(w[7]), d, y));
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t c0 = e2m1_sr(div_rn(lo_bf16(w[i]), d, y), rbyte(rnd, 2 * i));
            const uint32_t c1 = e2m1_sr(div_rn(hi_bf16(w[i]), d, y), rbyte(rnd, 2 * i + 1));
            const uint32_t byte = c0 | (c1 << 4);
            if (i < 4) lo |= byte << (8 * i);
            else       hi |= byte << (8 * (i - 4));
        }
    }
    const bool zero = nan_block || sc == 0u;
    sc_out = nan_block ? 0x7Fu : sc;
    return make_uint2(zero ? 0u : lo, zero ? 0u : hi);
}

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

}  // namespace

// ---------------------------------------------------------------- phase A
// One 256-thread work-group per (section, chunk of 4 token tiles, column tile);
// wave w takes token tile 4*chunk + w of the section.
template <bool ROW, bool COL>
__global__ __launch_bounds__(256) void k_nvfp4_amax(const Nvfp4Group G) {
    const int b = blockIdx.x;
    const int s = section_of_chunk(G, b);
    const int local = b - G.chunk_start[s];
    const int chunk = local / G.n_ctiles;
    const int C = local - chunk * G.n_ctiles;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int tt_local = chunk * kChunkTiles + wave;
    const bool live = tt_local < (G.tt_start[s + 1] - G.tt_start[s]);
    const int tb = lane >> 3, cc = lane & 7;

    uint32_t mrow = 0;
    float mcol = 0.0f;
    if (live) {
        const int64_t row0 = (int64_t)(G.tt_start[s] + tt_local) * kTileRows + tb * 16;
        const int64_t c0 = (int64_t)C * kTileCols + cc * 16;
        uint4 p[16][2];
        load_subtile(p, G.x + row0 * G.k + c0, G.k);
        if (ROW) {
            uint32_t m = 0;
#pragma unroll
            for (int t = 0; t < 16; ++t)
#pragma unroll
                for (int i = 0; i < 8; ++i) m = absmax_pk(m, P(t, i));
            m = fold_pk(m);
            if (m > 0x7F80u) {
                m = 0;
#pragma unroll
                for (int t = 0; t < 16; ++t)
#pragma unroll
                    for (int i = 0; i < 8; ++i) m = absmax_pk_nonan(m, P(t, i));
            }
            mrow = m;
        }
        if (COL) {
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const uint32_t flip = ((G.sign_mask >> t) & 1u) ? 0x80008000u : 0u;
                p[t][0].x ^= flip; p[t][0].y ^= flip; p[t][0].z ^= flip; p[t][0].w ^= flip;
                p[t][1].x ^= flip; p[t][1].y ^= flip; p[t][1].z ^= flip; p[t][1].w ^= flip;
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                float v[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) v[t] = (j & 1) ? hi_bf16(P(t, j >> 1)) : lo_bf16(P(t, j >> 1));
                butterfly16(v);
#pragma unroll
                for (int t = 0; t < 16; ++t) mcol = __builtin_fmaxf(mcol, __builtin_fabsf(v[t]));
            }
        }
    }
    mrow = wave_max_u32(mrow);
    mcol = wave_max_f32(mcol);
    __shared__ float red[4][2];
    if (lane == 0) {
        red[wave][0] = bf16_mag(mrow);
        red[wave][1] = mcol;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float a = red[0][0], c = red[0][1];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            a = __builtin_fmaxf(a, red[w][0]);
            c = __builtin_fmaxf(c, red[w][1]);
        }
        G.partials[2 * b] = a;
        G.partials[2 * b + 1] = c;
    }
}

// ---------------------------------------------------------------- phase B
template <bool ROW, bool COL, bool FP8, bool SR>
__global__ __launch_bounds__(64) void k_nvfp4_quant(const Nvfp4Group G) {
    const int lane = threadIdx.x;
    const int N = G.total_tiles;
    const int b = blockIdx.x;
    if ((ROW || COL) && b == 0) {
        // empty sections still publish their (floor) tensor scales
        for (int i = lane; i < G.num_sections; i += 64) {
            if (G.tt_start[i + 1] == G.tt_start[i]) {
                const float g0 = tensor_scale(0.0f);
                if (ROW) G.row_global[i] = g0;
                if (COL) G.col_global[i] = g0;
            }
        }
    }
    if (b >= N) return;
    // XCD-contiguous tile order: XCD x = b % 8 owns one contiguous range of tiles.
    const int xcd = b & 7;
    int q = b >> 3;
    for (int y = 0; y < xcd; ++y) q += (N + 7 - y) >> 3;
    const int T = q / G.n_ctiles;
    const int C = q - T * G.n_ctiles;
    const int s = section_of_tile(G, T);
    const int tt0 = G.tt_start[s];
    const int ms = (G.tt_start[s + 1] - tt0) * kTileRows;     // section rows
    const int T_local = T - tt0;

    // Section tensor scales from the phase-A partials.
    float g_r = 0.0f, g_c = 0.0f, yg_r = 0.0f, yg_c = 0.0f;
    if (ROW || COL) {
        float ar = 0.0f, mc = 0.0f;
        for (int i = G.chunk_start[s] + lane; i < G.chunk_start[s + 1]; i += 64) {
            const float2 pr = reinterpret_cast<const float2*>(G.partials)[i];
            ar = __builtin_fmaxf(ar, pr.x);
            mc = __builtin_fmaxf(mc, pr.y);
        }
        ar = wave_max_f32(ar);
        mc = wave_max_f32(mc);
        // max |BF16(0.25 y)| over the section = BF16(0.25 * max |y|) (monotone)
        const float ac = lo_bf16(pack_bf16(mc * 0.25f, 0.0f));
        g_r = tensor_scale(ar);
        g_c = tensor_scale(ac);
        yg_r = 1.0f / g_r;
        yg_c = 1.0f / g_c;
        if (T_local == 0 && C == 0 && lane == 0) {
            if (ROW) G.row_global[s] = g_r;
            if (COL) G.col_global[s] = g_c;
        }
    }

    const int tb = lane >> 3, cc = lane & 7;
    const int64_t k = G.k;
    const int64_t row0 = (int64_t)T * kTileRows + tb * 16;       // group-relative row
    const int64_t c0 = (int64_t)C * kTileCols + cc * 16;
    uint4 p[16][2];
    load_subtile(p, G.x + row0 * k + c0, k);

    const int64_t r_local0 = (int64_t)T_local * kTileRows + tb * 16; // section-local row
    if (ROW || FP8) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const uint32_t w[8] = {p[t][0].x, p[t][0].y, p[t][0].z, p[t][0].w,
                                   p[t][1].x, p[t][1].y, p[t][1].z, p[t][1].w};
            const int64_t row = row0 + t;
            if (ROW) {
                u32x4 rnd = {0, 0, 0, 0};
                if (SR && G.sr_row)
                    rnd = block_random(G.seed, G.row_off[s], (uint64_t)((r_local0 + t) * (k >> 4) + (c0 >> 4)));
                uint32_t sc;
                const uint2 codes = (SR && G.sr_row) ? encode_block<true>(w, g_r, yg_r, rnd, sc)
                                                     : encode_block<false>(w, g_r, yg_r, rnd, sc);
                *reinterpret_cast<uint2*>(G.row_codes + row * (k >> 1) + (c0 >> 1)) = codes;
                G.row_scales[row * (k >> 4) + (c0 >> 4)] = (uint8_t)sc;
            }
            if (FP8) {
                uint32_t m = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) m = absmax_pk(m, w[i]);
                m = fold_pk(m);
                const bool has_nan = m > 0x7F80u;
                if (has_nan) {
                    m = 0;
#pragma unroll
                    for (int i = 0; i < 8; ++i) m = absmax_pk_nonan(m, w[i]);
                }
#pragma unroll
                for (int o = 1; o < 8; o <<= 1) {
                    const uint32_t other = shfl_xor_u32(m, o);
                    m = other > m ? other : m;
                }
                const float amax = bf16_mag(m);
                const float sf = (amax > k_floor() ? amax : k_floor()) * k_inv448();
                const float yf = 1.0f / sf;
                uint32_t c4[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    c4[j] = e4m3_pack4(div_rn(lo_bf16(w[2 * j]), sf, yf), div_rn(hi_bf16(w[2 * j]), sf, yf),
                                       div_rn(lo_bf16(w[2 * j + 1]), sf, yf), div_rn(hi_bf16(w[2 * j + 1]), sf, yf));
                    if (has_nan) {
                        const uint32_t cj = c4[j];
                        const uint32_t ff = cj & (cj >> 1) & (cj >> 2) & (cj >> 3) & (cj >> 4) & (cj >> 5) &
                                            (cj >> 6) & (cj >> 7) & 0x01010101u;
                        c4[j] = cj ^ (ff * 0x80u);
                    }
                }
                *reinterpret_cast<uint4*>(G.fp8_codes + row * k + c0) = make_uint4(c4[0], c4[1], c4[2], c4[3]);
                if (cc == 0) G.fp8_scales[row * (k >> 7) + C] = sf;
            }
        }
    }

    if (COL) {
        __shared__ uint2 lds_codes[kTileCols * 8];
        __shared__ uint8_t lds_sc[kTileCols * 8];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const uint32_t flip = ((G.sign_mask >> t) & 1u) ? 0x80008000u : 0u;
            p[t][0].x ^= flip; p[t][0].y ^= flip; p[t][0].z ^= flip; p[t][0].w ^= flip;
            p[t][1].x ^= flip; p[t][1].y ^= flip; p[t][1].z ^= flip; p[t][1].w ^= flip;
        }
        const int64_t b_local = r_local0 >> 4;                      // section-local 16-row block
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float v[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) v[t] = (j & 1) ? hi_bf16(P(t, j >> 1)) : lo_bf16(P(t, j >> 1));
            butterfly16(v);
            uint32_t w[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) w[i] = pack_bf16(v[2 * i] * 0.25f, v[2 * i + 1] * 0.25f);
            u32x4 rnd = {0, 0, 0, 0};
            if (SR && G.sr_col)
                rnd = block_random(G.seed, G.col_off[s], (uint64_t)((c0 + j) * (int64_t)(ms >> 4) + b_local));
            uint32_t sc;
            const uint2 codes = (SR && G.sr_col) ? encode_block<true>(w, g_c, yg_c, rnd, sc)
                                                 : encode_block<false>(w, g_c, yg_c, rnd, sc);
            const int col = cc * 16 + j;
            lds_codes[col * 8 + tb] = codes;
            lds_sc[col * 8 + tb] = (uint8_t)sc;
        }
        __syncthreads();
        uint8_t* codes_s = G.col_codes + k * (int64_t)tt0 * kTileRows / 2;
        uint8_t* scales_s = G.col_scales + k * (int64_t)tt0 * kTileRows / 16;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int idx = it * 64 + lane;
            const int col = idx >> 2, part = idx & 3;
            const uint4 v = *reinterpret_cast<const uint4*>(&lds_codes[col * 8 + part * 2]);
            *reinterpret_cast<uint4*>(codes_s + ((int64_t)C * kTileCols + col) * (ms >> 1) + T_local * 64 + part * 16) = v;
        }
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int col = it * 64 + lane;
            const uint2 v = *reinterpret_cast<const uint2*>(&lds_sc[col * 8]);
            *reinterpret_cast<uint2*>(scales_s + ((int64_t)C * kTileCols + col) * (ms >> 4) + T_local * 8) = v;
        }
    }
}

#undef P

namespace {
template <bool ROW, bool COL, bool FP8>
hipError_t launch_b(const Nvfp4Group& g, hipStream_t stream) {
    const unsigned grid = (unsigned)(g.total_tiles > 0 ? g.total_tiles : 1);
    if (g.sr_row || g.sr_col)
        hipLaunchKernelGGL((k_nvfp4_quant<ROW, COL, FP8, true>), dim3(grid), dim3(64), 0, stream, g);
    else
        hipLaunchKernelGGL((k_nvfp4_quant<ROW, COL, FP8, false>), dim3(grid), dim3(64), 0, stream, g);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_nvfp4_group(const Nvfp4Group& g, hipStream_t stream) {
    const bool row = g.flags & 1u, col = g.flags & 2u, fp8 = g.flags & 4u;
    if ((row || col) && g.total_chunks > 0) {
        if (row && col)
            hipLaunchKernelGGL((k_nvfp4_amax<true, true>), dim3(g.total_chunks), dim3(256), 0, stream, g);
        else if (row)
            hipLaunchKernelGGL((k_nvfp4_amax<true, false>), dim3(g.total_chunks), dim3(256), 0, stream, g);
        else
            hipLaunchKernelGGL((k_nvfp4_amax<false, true>), dim3(g.total_chunks), dim3(256), 0, stream, g);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (!row && !col && g.total_tiles == 0) return hipSuccess;   // FP8 only, nothing to do
    const int sel = (row ? 1 : 0) | (col ? 2 : 0) | (fp8 ? 4 : 0);
    switch (sel) {
        case 1: return launch_b<true, false, false>(g, stream);
        case 2: return launch_b<false, true, false>(g, stream);
        case 3: return launch_b<true, true, false>(g, stream);
        case 4: return launch_b<false, false, true>(g, stream);
        case 5: return launch_b<true, false, true>(g, stream);
        case 6: return launch_b<false, true, true>(g, stream);
        default: return launch_b<true, true, true>(g, stream);
    }
}

}  // namespace mxq
