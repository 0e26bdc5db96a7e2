// mxq_nvfp4.hip -- grouped NVFP4 quantization with a 16-point RHT on the
// column-wise operand (gfx950).
//
// The method: TransformerEngine PR #2564 "[NVFP4][MOE] Bug Fix for NVFP4 Grouped
// Quant" (Greptile summary: grouped row-wise + column-wise RHT cast fusion, the
// workspace supplied by the caller) and the review comments of PR #2555 on
// quantizer.cpp (RHT only for the column-wise operand; the RHT(x^T) intermediate
// has the input dtype; a separate column-wise RNG).
//
// The FP32 tensor scale of a section needs the section's amax before any code is
// final.  One fused kernel does both passes: A items reduce max|x| and max|H16 D x|
// of a 128 x 512 block to a partial; the section's last A item folds the partials
// into the two tensor scales and raises a ready flag; B items wait for the flag,
// re-read their tile (usually from the Infinity Cache) and write every output.  All
// A items precede all B items in blockIdx order, so the B items' ALU work overlaps
// the tail of the A items' HBM reads.  Cross-XCD traffic uses only agent-scope
// atomics (one counter increment per A item, flag polls by B items); a small reset
// kernel clears the control words before each launch.
//
// No deadlock: a B item only waits for A items with a smaller blockIdx, and each
// XCD dispatches its work-groups in blockIdx order, so the smallest unfinished A
// item always gets a slot.  Each wait is also bounded by a wall-clock limit that
// sets an error word instead of spinning forever.
//
// Tile work (one wave per 128 x 128 tile): lane = (tb, cc), tb = lane / 8 picks
// 16 rows and cc = lane % 8 picks 16 columns, so each lane owns 16 complete row
// blocks (1x16 along k) and 16 complete column blocks (16 tokens): the row encode
// and the 16-point butterfly run in registers.  Column codes (8 bytes per 16
// tokens) are transposed through LDS so that each column's 128 tokens leave as
// one 64-byte run.
#include "mxq_device.hpp"
#include "mxq_internal.hpp"

namespace mxq {

namespace {

constexpr uint64_t kWaitLimitTicks = 2000000ull;     // 20 ms of the 100 MHz real-time clock

__device__ __forceinline__ uint32_t ws_load(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// E4M3 block-scale code of a 1x16 block with amax a (a BF16 value):
// E4M3(fl(fl(a * F(1/6)) / g)), yg = fl(1/g).
__device__ __forceinline__ uint32_t block_code(float a, float g, float yg) {
    return e4m3_code(div_rn(a * k_inv6(), g, yg));
}

// Codes of 16 values held as 8 packed BF16 pairs (element 2i in the low half of
// w[i]) with divisor d and y = fl(1/d): 8 bytes, even element in the low nibble.
template <bool SR>
__device__ __forceinline__ uint2 encode16(const uint32_t (&w)[8], float d, float y, const u32x4& rnd) {
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
    return make_uint2(lo, hi);
}

// One 1x16 block: amax from the packed bits (m = max |bits|, > 0x7F80 means a
// NaN), scale code, then codes.  tab holds (d, 1/d) for every scale code.
template <bool SR>
__device__ __forceinline__ uint2 encode_block(const uint32_t (&w)[8], uint32_t m, float g, float yg,
                                              const float2* tab, const u32x4& rnd, uint32_t& sc_out) {
    const bool nan_block = m > 0x7F80u;
    const uint32_t sc = block_code(bf16_mag(m), g, yg);
    const float2 dy = tab[sc & 0x7Fu];
    const uint2 codes = encode16<SR>(w, dy.x, dy.y, rnd);
    const bool zero = nan_block || sc == 0u;
    sc_out = nan_block ? 0x7Fu : sc;
    return make_uint2(zero ? 0u : codes.x, zero ? 0u : codes.y);
}

__device__ __forceinline__ uint32_t packed_absmax(const uint32_t (&w)[8]) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = absmax_pk(m, w[i]);
    return fold_pk(m);
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

// Which item a work-group runs (uniform over the work-group).
struct Item {
    bool is_a;
    int s, idx, T_local, C;
};
__device__ __forceinline__ Item decode_item(const Nvfp4Group& G, int b) {
    int r = 0;
    for (int i = 1; i < G.num_rounds; ++i)
        if (G.rounds[i].start <= b) r = i;
    const Nvfp4Round R = G.rounds[r];
    const int64_t j = b - R.start;
    const int64_t n = (int64_t)R.n_a + R.n_b;
    const int64_t a0 = j * R.n_a / n, a1 = (j + 1) * R.n_a / n;
    Item it;
    it.is_a = a1 > a0;
    const int idx = (int)(it.is_a ? a0 : j - a0);
    it.s = it.is_a ? R.sec_a : R.sec_b;
    it.idx = idx;
    const int per_row = it.is_a ? G.n_agroups : G.n_ctiles;
    it.T_local = idx / per_row;
    it.C = idx - it.T_local * per_row;          // A items: column group; B items: column tile
    return it;
}

// ---------------------------------------------------------------- A work (one wave, one 128x128 tile)
template <bool ROW, bool COL>
__device__ __forceinline__ void amax_tile(const Nvfp4Group& G, uint4 (&p)[16][2], uint32_t& mrow, float& mcol) {
    mrow = 0;
    mcol = 0.0f;
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

// ---------------------------------------------------------------- B work (one wave, one 128x128 tile)
template <bool ROW, bool COL, bool FP8, bool SR>
__device__ __forceinline__ void quant_tile(const Nvfp4Group& G, uint4 (&p)[16][2], int s, int T, int C,
                                           float g_r, float yg_r, float g_c, float yg_c,
                                           const float2* tab_r, const float2* tab_c,
                                           uint2* lds_codes, uint8_t* lds_sc) {
    const int lane = threadIdx.x & 63;
    const int tb = lane >> 3, cc = lane & 7;
    const int64_t k = G.k;
    const int tt0 = G.tt_start[s];
    const int ms = (G.tt_start[s + 1] - tt0) * kTileRows;
    const int T_local = T - tt0;
    const int64_t row0 = (int64_t)T * kTileRows + tb * 16;
    const int64_t c0 = (int64_t)C * kTileCols + cc * 16;

    const int64_t r_local0 = (int64_t)T_local * kTileRows + tb * 16;
    bool lane_nan = false;
    if (ROW || FP8 || COL) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const uint32_t w[8] = {p[t][0].x, p[t][0].y, p[t][0].z, p[t][0].w,
                                   p[t][1].x, p[t][1].y, p[t][1].z, p[t][1].w};
            const int64_t row = row0 + t;
            const uint32_t m = packed_absmax(w);
            lane_nan |= m > 0x7F80u;
            if (ROW) {
                u32x4 rnd = {0, 0, 0, 0};
                if (SR && G.sr_row)
                    rnd = block_random(G.seed, G.row_off[s], (uint64_t)((r_local0 + t) * (k >> 4) + (c0 >> 4)));
                uint32_t sc;
                const uint2 codes = (SR && G.sr_row) ? encode_block<true>(w, m, g_r, yg_r, tab_r, rnd, sc)
                                                     : encode_block<false>(w, m, g_r, yg_r, tab_r, rnd, sc);
                *reinterpret_cast<uint2*>(G.row_codes + row * (k >> 1) + (c0 >> 1)) = codes;
                G.row_scales[row * (k >> 4) + (c0 >> 4)] = (uint8_t)sc;
            }
            if (FP8) {
                uint32_t mf = m;
                const bool has_nan = m > 0x7F80u;
                if (has_nan) {
                    mf = 0;
#pragma unroll
                    for (int i = 0; i < 8; ++i) mf = absmax_pk_nonan(mf, w[i]);
                }
#pragma unroll
                for (int o = 1; o < 8; o <<= 1) {
                    const uint32_t other = shfl_xor_u32(mf, o);
                    mf = other > mf ? other : mf;
                }
                const float amax = bf16_mag(mf);
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
            __builtin_amdgcn_sched_barrier(0);       // one row at a time
        }
    }

    if (COL) {
        // Column values: x * (+-1/4) per row (the sign mask and the 1/4 are both
        // exact for BF16 inputs, so scaling first equals scaling the butterfly's
        // result), the butterfly, then BF16 rounding.
        float rs[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) rs[t] = ((G.sign_mask >> t) & 1u) ? -0.25f : 0.25f;
        // Hide the sub-tile's provenance from the compiler: otherwise it reuses the
        // row pass's widened values here and keeps all 256 of them live.
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            asm volatile("" : "+v"(p[t][0].x), "+v"(p[t][0].y), "+v"(p[t][0].z), "+v"(p[t][0].w));
            asm volatile("" : "+v"(p[t][1].x), "+v"(p[t][1].y), "+v"(p[t][1].z), "+v"(p[t][1].w));
        }
        const int64_t b_local = r_local0 >> 4;                      // section-local 16-row block
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float v[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) v[t] = ((j & 1) ? hi_bf16(P(t, j >> 1)) : lo_bf16(P(t, j >> 1))) * rs[t];
            butterfly16(v);
            uint32_t w[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) w[i] = pack_bf16(v[2 * i], v[2 * i + 1]);
            uint32_t m;
            if (!lane_nan) {
                // no NaN among this lane's inputs: max |BF16(v)| = BF16(max |v|)
                float mx = 0.0f;
#pragma unroll
                for (int t = 0; t < 16; ++t) mx = __builtin_fmaxf(mx, __builtin_fabsf(v[t]));
                m = pack_bf16(mx, 0.0f) & 0xFFFFu;
            } else {
                m = packed_absmax(w);
            }
            u32x4 rnd = {0, 0, 0, 0};
            if (SR && G.sr_col)
                rnd = block_random(G.seed, G.col_off[s], (uint64_t)((c0 + j) * (int64_t)(ms >> 4) + b_local));
            uint32_t sc;
            const uint2 codes = (SR && G.sr_col) ? encode_block<true>(w, m, g_c, yg_c, tab_c, rnd, sc)
                                                 : encode_block<false>(w, m, g_c, yg_c, tab_c, rnd, sc);
            const int col = cc * 16 + j;
            lds_codes[col * 8 + tb] = codes;
            lds_sc[col * 8 + tb] = (uint8_t)sc;
            __builtin_amdgcn_sched_barrier(0);   // one column at a time: bounds register pressure
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

}  // namespace

// ---------------------------------------------------------------- the kernels
__device__ __forceinline__ uint64_t ws_load64(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Clears the control words of the group's sections (and the error word) and
// writes the floor tensor scales of empty sections.
template <bool ROW, bool COL>
__global__ __launch_bounds__(256) void k_nvfp4_reset(const Nvfp4Group G) {
    for (int i = threadIdx.x; i < G.num_sections; i += 256) {
        uint32_t* c = G.ctrl + kCtrlStride * i;
        c[0] = 0u;
        c[1] = 0u;
        if (G.tt_start[i + 1] == G.tt_start[i]) {
            const float g0 = tensor_scale(0.0f);
            if (ROW) G.row_global[i] = g0;
            if (COL) G.col_global[i] = g0;
        }
    }
    if (threadIdx.x == 0) G.ctrl[kCtrlErrorWord] = 0u;
}

// One wave per work-group.
template <bool ROW, bool COL, bool FP8, bool SR>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void k_nvfp4_grouped(const Nvfp4Group G) {
    constexpr bool AMAX = ROW || COL;
    const int lane = threadIdx.x;
    const int b = blockIdx.x;
    if (b >= G.total_items) return;
    const Item it = decode_item(G, b);
    const int s = it.s;
    const int T = G.tt_start[s] + it.T_local;
    uint32_t* ctrl = G.ctrl + kCtrlStride * s;
    const uint16_t* row_base = G.x + ((int64_t)T * kTileRows + (lane >> 3) * 16) * G.k + (lane & 7) * 16;
    uint4 p[16][2];

    if (AMAX && it.is_a) {
        uint32_t mr = 0;
        float mc = 0.0f;
#pragma unroll 1
        for (int t = 0; t < kATiles; ++t) {
            const int C = it.C * kATiles + t;
            if (C >= G.n_ctiles) break;
            load_subtile(p, row_base + (int64_t)C * kTileCols, G.k);
            uint32_t r;
            float c;
            amax_tile<ROW, COL>(G, p, r, c);
            mr = r > mr ? r : mr;
            mc = __builtin_fmaxf(mc, c);
        }
        mr = wave_max_u32(mr);
        mc = wave_max_f32(mc);
        const int n_a = (G.tt_start[s + 1] - G.tt_start[s]) * G.n_agroups;
        uint32_t last = 0;
        if (lane == 0) {
            const uint64_t part = (uint64_t)(mr << 16) | ((uint64_t)__builtin_bit_cast(uint32_t, mc) << 32);
            __hip_atomic_store(G.partials + G.a_start[s] + it.idx, part, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_s_waitcnt(0x0F70);               // vmcnt(0): the partial is stored
            last = __hip_atomic_fetch_add(ctrl + 0, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(n_a - 1);
        }
        last = (uint32_t)__shfl((int)last, 0, 64);
        if (last) {
            // every partial of the section is in: fold them into the tensor scales
            uint32_t ar = 0, ac = 0;
            for (int i = lane; i < n_a; i += 64) {
                const uint64_t v = ws_load64(G.partials + G.a_start[s] + i);
                ar = (uint32_t)v > ar ? (uint32_t)v : ar;
                ac = (uint32_t)(v >> 32) > ac ? (uint32_t)(v >> 32) : ac;
            }
            ar = wave_max_u32(ar);
            ac = wave_max_u32(ac);
            if (lane == 0) {
                // max |BF16(y/4)| over the section = BF16(max |y| / 4) (monotone)
                const float acol = lo_bf16(pack_bf16(__builtin_bit_cast(float, ac) * 0.25f, 0.0f));
                const float g_r = tensor_scale(__builtin_bit_cast(float, ar));
                const float g_c = tensor_scale(acol);
                if (ROW) G.row_global[s] = g_r;
                if (COL) G.col_global[s] = g_c;
                __hip_atomic_store(ctrl + 2, __builtin_bit_cast(uint32_t, g_r), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(ctrl + 3, __builtin_bit_cast(uint32_t, g_c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __builtin_amdgcn_s_waitcnt(0x0F70);
                __hip_atomic_store(ctrl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        return;
    }

    // ---- B item
    __shared__ float2 tab[2][128];
    __shared__ uint2 lds_codes[kTileCols * 8];
    __shared__ uint8_t lds_sc[kTileCols * 8];
    const int C = it.C;
    load_subtile(p, row_base + (int64_t)C * kTileCols, G.k);   // in flight during the wait
    float g_r = 0.f, yg_r = 0.f, g_c = 0.f, yg_c = 0.f;
    if (AMAX) {
        uint32_t rbits = 0, cbits = 0;
        if (lane == 0) {
            if (ws_load(ctrl + 1) == 0u) {
                const uint64_t t0 = wall_clock64();
                while (ws_load(ctrl + 1) == 0u) {
                    __builtin_amdgcn_s_sleep(8);
                    if (wall_clock64() - t0 > kWaitLimitTicks) {
                        __hip_atomic_fetch_or(G.ctrl + kCtrlErrorWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                }
            }
            rbits = ws_load(ctrl + 2);
            cbits = ws_load(ctrl + 3);
        }
        g_r = __builtin_bit_cast(float, (uint32_t)__shfl((int)rbits, 0, 64));
        g_c = __builtin_bit_cast(float, (uint32_t)__shfl((int)cbits, 0, 64));
        yg_r = 1.0f / g_r;
        yg_c = 1.0f / g_c;
        // (d, 1/d) for every E4M3 scale code, one table per direction
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int dir = e >> 1, code = lane + 64 * (e & 1);
            const float d = e4m3_value((uint32_t)code) * (dir ? g_c : g_r);
            tab[dir][code] = make_float2(d, 1.0f / d);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
    quant_tile<ROW, COL, FP8, SR>(G, p, s, T, C, g_r, yg_r, g_c, yg_c, tab[0], tab[1], lds_codes, lds_sc);
}

namespace {
template <bool ROW, bool COL, bool FP8>
hipError_t launch_sel(const Nvfp4Group& g, hipStream_t stream) {
    if (ROW || COL) {
        hipLaunchKernelGGL((k_nvfp4_reset<ROW, COL>), dim3(1), dim3(256), 0, stream, g);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || g.total_items == 0) return e;
    }
    const unsigned grid = (unsigned)g.total_items;
    if (g.sr_row || g.sr_col)
        hipLaunchKernelGGL((k_nvfp4_grouped<ROW, COL, FP8, true>), dim3(grid), dim3(64), 0, stream, g);
    else
        hipLaunchKernelGGL((k_nvfp4_grouped<ROW, COL, FP8, false>), dim3(grid), dim3(64), 0, stream, g);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_nvfp4_group(const Nvfp4Group& g, hipStream_t stream) {
    const bool row = g.flags & 1u, col = g.flags & 2u, fp8 = g.flags & 4u;
    if (!row && !col && g.total_items == 0) return hipSuccess;   // FP8 only, no rows
    const int sel = (row ? 1 : 0) | (col ? 2 : 0) | (fp8 ? 4 : 0);
    switch (sel) {
        case 1: return launch_sel<true, false, false>(g, stream);
        case 2: return launch_sel<false, true, false>(g, stream);
        case 3: return launch_sel<true, true, false>(g, stream);
        case 4: return launch_sel<false, false, true>(g, stream);
        case 5: return launch_sel<true, false, true>(g, stream);
        case 6: return launch_sel<false, true, true>(g, stream);
        default: return launch_sel<true, true, true>(g, stream);
    }
}

}  // namespace mxq
