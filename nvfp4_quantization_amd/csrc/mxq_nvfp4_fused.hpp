// mxq_nvfp4_fused.hpp -- the single-read form of the grouped NVFP4 call (gfx950):
// one launch that reads every tile of x once, from HBM into registers, and keeps
// it there across the wait for its section's tensor scales.
//
// TransformerEngine PR #2564 (Greptile summary, sequence diagram) fuses the grouped
// row-wise and column-wise (RHT) casts into one kernel.  The difficulty of that
// fusion is the per-section FP32 tensor scale, which needs the amax of the whole
// section before any code of it is final.  Here work-group b takes item b, four
// adjacent 128 x 128 tiles of one token tile (one per wave), and the host takes this
// form only when every item fits the resident grid at once.  Per item:
//
//   1. the waves load their tiles (each lane 16 rows x 16 columns, the layout of
//      the quantizing passes) and take max |x| and max |H16 D x| on the registers;
//   2. the item publishes both maxima in one 32-bit word of the workspace (its
//      partial; the top bit marks it present);
//   3. the section's last item waits until every partial of the section is
//      present, forms the two tensor scales, builds the scale tables and, after an
//      agent-scope release fence, clears every partial of the section;
//   4. every other item waits until its own partial reads zero, acquires, and
//      reads the tables;
//   5. every item quantizes its tiles from the registers (quant_passes).
//
// Steps 3 and 4 wait for items that may not have started, which needs the whole
// section resident at once.  Neither the dispatch order of work-groups nor the room
// other work leaves on the device is guaranteed, so step 4's wait is bounded: an
// item that waits longer than kDeferTicks marks its partial deferred (compare-and-
// swap, which fails if the partial was cleared meanwhile) and ends, freeing its
// slot.  The last item clears each partial with an atomic exchange and re-reads and
// quantizes the tiles of every deferred item of its section itself.  Only the last
// items (one per section, at most kGroupSections) wait without a fallback, and only
// for partials; every other resident work-group ends within kDeferTicks, so every
// item is eventually dispatched and publishes, and every wait ends whatever the
// dispatch order, as long as the device holds more work-groups of this kernel than
// there are sections.  (The last item's wait still gives up after kWaitTicks and
// sets the error word.)  No wait depends on residency for correctness; a starved
// call only gets slower.
//
// Workspace protocol: the partial words are zero before a call and zero after it
// (the last item clears its section's partials), so nothing carries over between
// calls.
#pragma once

#include "mxq_nvfp4_impl.hpp"


namespace mxq {

namespace {

__device__ __forceinline__ uint32_t ws_load32(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ws_store32(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 100 MHz constant clock.
__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// Maxima of the lane's part of a tile in the quant layout (rows 16 tb .. +15,
// columns 16 cc .. +15 as packed BF16 pairs): rbits = max |x| as BF16 bits and
// cmax = max |H16 D x| over the lane's 16 column blocks, both without NaNs.
// The row maximum is taken on the bit patterns (packed 16-bit maxima of |x|; every
// NaN is above 0x7F80), so that it does not depend on the column work.  The last
// butterfly stage is not formed: for its pair (a, b) the larger of |fl(a + b)| and
// |fl(a - b)| is fl(|a| + |b|) (rounding is monotone and symmetric), so 8
// additions replace 16 outputs and their maxima; FP32 maxima ignore the quiet NaNs
// that arithmetic makes of NaN inputs.
template <bool ROW, bool COL>
__device__ __forceinline__ void tile_maxima(const uint4 (&p)[16][2], uint32_t sign_mask, uint32_t& rbits,
                                            float& cmax) {
    uint32_t mr = 0;
    float mc = 0.0f;
    if (ROW) {
#pragma unroll
        for (int t = 0; t < 16; ++t)
#pragma unroll
            for (int i = 0; i < 8; ++i) mr = absmax_pk(mr, tile_word(p, t, i));
        mr = fold_pk(mr);
        if (mr > 0x7F80u) {                          // a NaN: the maximum without it
            mr = 0;
#pragma unroll
            for (int t = 0; t < 16; ++t)
#pragma unroll
                for (int i = 0; i < 8; ++i) mr = absmax_pk_nonan(mr, tile_word(p, t, i));
        }
    }
    if (COL) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float f[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const uint32_t w = tile_word(p, t, j >> 1);
                const uint32_t neg = sign_of_row(sign_mask, t);
                f[t] = (j & 1) ? hi_signed(w, neg) : lo_signed(w, neg);
            }
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
            for (int i = 0; i < 8; ++i) mc = __builtin_fmaxf(mc, __builtin_fabsf(f[i]) + __builtin_fabsf(f[i + 8]));
        }
    }
    rbits = mr;
    cmax = mc;
}

}  // namespace

// LDS of the single-read kernel.
struct FusedLds {
    QuantLds<4> q;
    uint32_t max[2][4];                               // per-wave maxima: BF16 bits of max |x|, FP32 max |H16 D x|
    uint32_t none[kTableLdsWords];
    float amax[2];
    int ok;                                           // 0: give up (error), 1: go on, 2: deferred
    uint64_t deferred[kFusedMaxItems / 64];         // the last item's list of deferred items of its section
};

// Where an item lies: its section s, processing position, and tiles T (token tile) and
// C (this wave's column tile).
struct ItemPos {
    int s, first, n, local, T, C;
};

__device__ __forceinline__ ItemPos item_pos(const Nvfp4Group& G, const Nvfp4Fused& F, int item, int w) {
    int pos = 0;
    for (int q = 1; q < F.n_order; ++q) pos = F.istart[q] <= item ? q : pos;
    ItemPos r;
    r.s = F.order[pos];
    r.first = F.istart[pos];
    r.n = F.istart[pos + 1] - r.first;
    r.local = item - r.first;
    const int T_local = r.local / F.n_cgroups;
    r.T = G.tt_start[r.s] + T_local;
    r.C = (r.local - T_local * F.n_cgroups) * 4 + w;
    return r;
}

__device__ __forceinline__ const uint16_t* tile_base(const Nvfp4Group& G, int T, int C, int lane) {
    const int tb = lane >> 3, cc = lane & 7;
    return G.x + ((int64_t)T * kTileRows + tb * 16) * G.k + (int64_t)C * kTileCols + cc * 16;
}

// The single-read grouped kernel (see the file comment).  256 threads: four waves,
// one tile each, over four adjacent column tiles of one token tile.  One work-group
// per item.
template <bool ROW, bool COL, bool FP8, bool SR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_nvfp4_fused(const Nvfp4Group G,
                                                                                            const Nvfp4Fused F) {
    __shared__ FusedLds S;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int item = (int)blockIdx.x;
    const ItemPos ip = item_pos(G, F, item, w);
    const int s = ip.s;

    uint4 p[16][2];
    load_tile<!FP8>(p, tile_base(G, ip.T, ip.C, lane), G.k);

    if (item == 0 && w == 0) {
        // empty sections: the tensor scale of an all-zero section
        for (int i = lane; i < G.num_sections; i += 64) {
            if (G.tt_start[i + 1] != G.tt_start[i]) continue;
            if (ROW) G.row_global[i] = tensor_scale(0.0f);
            if (COL) G.col_global[i] = tensor_scale(0.0f);
            if (ROW && G.amax_out_row) G.amax_out_row[i] = 0.0f;
            if (COL && G.amax_out_col) G.amax_out_col[i] = 0.0f;
        }
    }

    // ---- phase A: the item's maxima, published as its partial
    uint32_t rbits;
    float cmax;
    tile_maxima<ROW, COL>(p, G.sign_mask, rbits, cmax);
    launder(p);                                       // phase B recomputes; nothing is kept across the wait
    rbits = wave_max_u32(rbits);
    cmax = wave_max_f32(cmax);
    if (lane == 0) {
        S.max[0][w] = rbits;
        S.max[1][w] = __builtin_bit_cast(uint32_t, cmax);
    }
    __syncthreads();
    uint32_t* const slots = F.slots + ip.first;
    const int n = ip.n;
    const bool last = ip.local == n - 1;
    uint32_t mine = 0;
    if (tid == 0) {
        uint32_t r = 0, c = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r = S.max[0][i] > r ? S.max[0][i] : r;
            c = S.max[1][i] > c ? S.max[1][i] : c;    // non-negative FP32: ordered as integers
        }
        // the column maximum as BF16(max |y| / 4): max |BF16(y / 4)| over the values
        const uint32_t c16 = pack_bf16(__builtin_bit_cast(float, c) * 0.25f, 0.0f) & 0xFFFFu;
        mine = kSlotPresent | (c16 << 16) | r;
        ws_store32(slots + ip.local, mine);
    }

    if (last) {
        // ---- the section's last item: gather, scales, tables, release
        if (w == 0) {
            const uint64_t t0 = now_ticks();
            uint32_t ar, ac;
            bool ok = true;
            while (true) {
                ar = 0;
                ac = 0;
                bool all = true;
                for (int i = lane; i < n; i += 64) {
                    const uint32_t v = ws_load32(slots + i);
                    all &= (v & kSlotPresent) != 0;
                    ar = (v & 0x7FFFu) > ar ? (v & 0x7FFFu) : ar;
                    ac = ((v >> 16) & 0x7FFFu) > ac ? ((v >> 16) & 0x7FFFu) : ac;
                }
                if (__ballot(!all) == 0) break;
                if (now_ticks() - t0 > kWaitTicks) {    // cannot happen: every partial's owner has started
                    ok = false;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            ar = wave_max_u32(ar);
            ac = wave_max_u32(ac);
            if (lane == 0) {
                S.amax[0] = bf16_mag(ar);
                S.amax[1] = bf16_mag(ac);
                S.ok = ok;
                if (!ok) ws_store32(F.err, 1u);
            }
        }
        __syncthreads();
        if (!S.ok) return;
        const float a_r = S.amax[0], a_c = S.amax[1];
        const float g_r = tensor_scale(a_r), g_c = tensor_scale(a_c);
        build_tables_wg<ROW, COL>(G, s, g_r, g_c, S.q.tab, S.none, tid);
        if (tid == 0) {
            if (ROW) G.row_global[s] = g_r;
            if (COL) G.col_global[s] = g_c;
            if (ROW && G.amax_out_row) G.amax_out_row[s] = a_r;
            if (COL && G.amax_out_col) G.amax_out_col[s] = a_c;
        }
        __syncthreads();                              // every table entry is written
        if (w == 0) {
            // the tables before the cleared partials, for every waiting item; an
            // exchange, so that a partial marked deferred is seen exactly once
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            // every exchange in flight before the first result is used: one round trip
            constexpr int kChunks = kFusedMaxItems / 64;
            uint32_t old[kChunks];
#pragma unroll
            for (int c = 0; c < kChunks; ++c) {
                const int i = c * 64 + lane;
                old[c] = i < n ? __hip_atomic_exchange(slots + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
            }
#pragma unroll
            for (int c = 0; c < kChunks; ++c) {
                const uint64_t d = __ballot((old[c] & kSlotDeferred) != 0);
                if (lane == 0) S.deferred[c] = d;
            }
        }
        __syncthreads();
    } else {
        // ---- wait for the section's tables: this item's partial is cleared after them
        if (tid == 0) {
            const uint64_t t0 = now_ticks();
            int ok = 1;
            while (ws_load32(slots + ip.local) != 0u) {
                if (now_ticks() - t0 > kDeferTicks) {
                    // too long (the section is not resident): leave this item to the last one
                    uint32_t expect = mine;
                    if (__hip_atomic_compare_exchange_strong(slots + ip.local, &expect, mine | kSlotDeferred,
                                                             __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT))
                        ok = 2;
                    break;                            // deferred, or cleared meanwhile
                }
                __builtin_amdgcn_s_sleep(1);
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            S.ok = ok;
        }
        __syncthreads();
        if (S.ok != 1) return;
        const int dir = tid >> 7;
        if (dir == 0 ? ROW : COL) S.q.tab[dir][tid & 127] = G.tables[s * 256 + tid];
        __syncthreads();
    }

    // ---- phase B from the registers
    quant_passes<ROW, COL, FP8, SR, false, 4>(G, p, S.q, w, s, ip.T, ip.C, tid);

    if (last) {
        // the deferred items of the section (none unless the device was short of room):
        // read their tiles again and quantize them with the tables in LDS
        for (int c = 0; c * 64 < n; ++c) {
            uint64_t d = S.deferred[c];
            while (d != 0) {
                const int i = c * 64 + __builtin_ctzll(d);
                d &= d - 1;
                const ItemPos dp = item_pos(G, F, ip.first + i, w);
                __syncthreads();                      // the LDS staging of the previous tiles is read
                load_tile<!FP8>(p, tile_base(G, dp.T, dp.C, lane), G.k);
                quant_passes<ROW, COL, FP8, SR, false, 4>(G, p, S.q, w, s, dp.T, dp.C, tid);
            }
        }
    }
}

// Launch of the single-read kernel for one flag combination (instantiated by the
// mxq_nvfp4_fused_*.hip units, one per rounding mode): one work-group per item.
template <bool SR>
hipError_t launch_fused_variant(const Nvfp4Group& g, const Nvfp4Fused& f, uint32_t flags, hipStream_t stream) {
    const dim3 grid((unsigned)f.n_items), block(256);
    switch (flags & 7u) {
        case 1: hipLaunchKernelGGL((k_nvfp4_fused<true, false, false, SR>), grid, block, 0, stream, g, f); break;
        case 2: hipLaunchKernelGGL((k_nvfp4_fused<false, true, false, SR>), grid, block, 0, stream, g, f); break;
        case 3: hipLaunchKernelGGL((k_nvfp4_fused<true, true, false, SR>), grid, block, 0, stream, g, f); break;
        case 5: hipLaunchKernelGGL((k_nvfp4_fused<true, false, true, SR>), grid, block, 0, stream, g, f); break;
        case 6: hipLaunchKernelGGL((k_nvfp4_fused<false, true, true, SR>), grid, block, 0, stream, g, f); break;
        case 7: hipLaunchKernelGGL((k_nvfp4_fused<true, true, true, SR>), grid, block, 0, stream, g, f); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Resident 256-thread work-groups per CU of the single-read kernel variant.
template <bool SR>
hipError_t fused_occupancy(uint32_t flags, int* blocks_per_cu) {
    const void* fn;
    switch (flags & 7u) {
        case 1: fn = reinterpret_cast<const void*>(&k_nvfp4_fused<true, false, false, SR>); break;
        case 2: fn = reinterpret_cast<const void*>(&k_nvfp4_fused<false, true, false, SR>); break;
        case 3: fn = reinterpret_cast<const void*>(&k_nvfp4_fused<true, true, false, SR>); break;
        case 5: fn = reinterpret_cast<const void*>(&k_nvfp4_fused<true, false, true, SR>); break;
        case 6: fn = reinterpret_cast<const void*>(&k_nvfp4_fused<false, true, true, SR>); break;
        case 7: fn = reinterpret_cast<const void*>(&k_nvfp4_fused<true, true, true, SR>); break;
        default: return hipErrorInvalidValue;
    }
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, 256, 0);
}

}  // namespace mxq
