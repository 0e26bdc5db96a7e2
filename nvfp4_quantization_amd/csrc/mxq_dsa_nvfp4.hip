// mxq_dsa_nvfp4.hip -- DSA-indexer rotate + NVFP4 row-wise (gfx950).
//
// TensorRT-LLM PR #15158 (Summary; discussion): the indexer concatenates qk_pe and
// qk_nope, rotates the 128 values with the orthonormal Hadamard transform and then
// quantizes; its FP4 path lacks the rotation for want of a standalone FP4 quantizer.
// This is that quantizer: y = BF16(WHT_128(cat(pe, nope)) / sqrt(128)) per row, then
// the row-wise NVFP4 encode of the grouped path (TransformerEngine PR #2564 / #2555:
// 1x16 E2M1 blocks with E4M3 block scales) with one FP32 tensor scale over the whole
// rotated tensor, g = fl(max(A, F(1e-10)) * F(1/2688)), A measured or supplied.
//
// A row is held by 4 consecutive lanes, 32 values each (wht128_quarter), so every
// 1x16 block lies inside one lane: its maximum, scale code and 16 codes need no
// exchange.  The encode is the grouped path's: block_code, then one multiply per
// element by the table's multiplier (exact division where the table has none).
#include "mxq_nvfp4_impl.hpp"

namespace mxq {

namespace {

constexpr int kDsaRows = 64;          // rows per 256-thread work-group

// Maximum of a non-negative, NaN-free per-thread value over the 256-thread
// work-group (red: 4 floats of LDS), returned to every thread.
__device__ __forceinline__ float wg_max(float v, float* red) {
    v = wave_max_f32(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const float r = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    __syncthreads();
    return r;
}

// The lane's 32 butterfly outputs split into its two 1x16 blocks.
__device__ __forceinline__ void halves(const float (&v)[32], float (&h0)[16], float (&h1)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        h0[i] = v[i];
        h1[i] = v[16 + i];
    }
}

}  // namespace

// Phase A: max |y| of the work-group's 64 rows into its partial (an ordinary
// store; the scale kernel that follows on the stream folds the partials).
__global__ __launch_bounds__(256) void k_dsa_nvfp4_amax(const DsaNvfp4Args a) {
    __shared__ float red[4];
    const int quarter = threadIdx.x & 3;
    const int64_t r = (int64_t)blockIdx.x * kDsaRows + (threadIdx.x >> 2);
    const bool live = r < a.m;
    float v[32];
    wht128_quarter<true>(a.pe, a.ld_pe, a.d_pe, a.nope, a.ld_nope, r, live, quarter, v);   // |v| only
    // max |BF16(fl(v C))| = BF16(fl(max |v| C)) (both roundings are monotone), NaN
    // outputs left out (a NaN input makes all 128 of its row NaN: then m is NaN and
    // the lane gives 0; inf - inf makes some NaN and leaves the rest infinite)
    float h0[16], h1[16];
    halves(v, h0, h1);
    const float m = __builtin_fmaxf(absmax16(h0), absmax16(h1));
    const float lane = m != m ? 0.0f : round_bf16(m * k_inv_sqrt128());
    const float wg = wg_max(lane, red);
    if (threadIdx.x == 0) a.partials[blockIdx.x] = wg;
}

// The tensor scale and the scale table (one 1024-thread work-group): from the
// partials of phase A, or from the supplied amax (then the measured-amax output is
// zeroed here and raised by the quantize kernel), or from A = 0 for a tensor
// without rows.
constexpr int kDsaScaleThreads = 1024;
__global__ __launch_bounds__(kDsaScaleThreads) void k_dsa_nvfp4_scale(const DsaNvfp4Args a) {
    __shared__ uint32_t red[kDsaScaleThreads / 64];
    const int tid = (int)threadIdx.x;
    float amax = 0.0f;
    if (a.amax_in) {
        amax = *a.amax_in;
    } else if (a.m > 0) {
        // non-negative floats order like their bit patterns; 8 loads in flight per
        // thread per round
        uint32_t A = 0;
        const uint32_t* const p = reinterpret_cast<const uint32_t*>(a.partials);
        for (int i0 = tid; i0 < a.n_wg; i0 += kDsaScaleThreads * 8) {
            uint32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = i0 + kDsaScaleThreads * u < a.n_wg ? p[i0 + kDsaScaleThreads * u] : 0u;
#pragma unroll
            for (int u = 0; u < 8; ++u) A = v[u] > A ? v[u] : A;
        }
        A = wave_max_u32(A);
        if ((tid & 63) == 0) red[tid >> 6] = A;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kDsaScaleThreads / 64; ++i) A = red[i] > A ? red[i] : A;
        amax = __builtin_bit_cast(float, A);
    }
    const float g = tensor_scale(amax);
    if (a.m > 0 && tid < 128) a.table[tid] = table_entry(tid, g, false);
    if (tid == 0) {
        *a.global_scale = g;
        if (a.amax_out) *a.amax_out = a.amax_in ? 0.0f : amax;
    }
}

// Phase B: rotate again and encode.  AOUT: the amax was supplied and the measured
// one is wanted out (an atomic maximum per work-group).
template <bool AOUT>
__global__ __launch_bounds__(256) void k_dsa_nvfp4_quant(const DsaNvfp4Args a) {
    __shared__ float4 tab[128];
    __shared__ float red[4];
    if (threadIdx.x < 128) tab[threadIdx.x] = a.table[threadIdx.x];
    __syncthreads();
    const float g = tab[0].x, yg = tab[0].y;
    const int quarter = threadIdx.x & 3;
    const int64_t r = (int64_t)blockIdx.x * kDsaRows + (threadIdx.x >> 2);
    const bool live = r < a.m;
    float v[32];
    wht128_quarter(a.pe, a.ld_pe, a.d_pe, a.nope, a.ld_nope, r, live, quarter, v);
    const float c = k_inv_sqrt128();
    const u32x4 no_rnd = {0, 0, 0, 0};
    float h[2][16];
    halves(v, h[0], h[1]);
    BlockOut o[2];
    float lane_max = 0.0f;                           // (AOUT) max |y| of the lane, NaNs left out
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        // block max |y|, NaN when the block holds a NaN (its scale is then 0x7F)
        const float ab = round_bf16(absmax16_nan(h[b]) * c);
        const uint32_t sc = block_code(ab, g, yg);
#pragma unroll
        for (int i = 0; i < 16; ++i) h[b][i] = round_bf16(h[b][i] * c);
        o[b] = encode_block<Enc::Mul>(h[b], sc, tab, no_rnd);
        if (AOUT) {
            float am = ab;
            if (ab != ab) am = absmax16(h[b]);
            lane_max = __builtin_fmaxf(lane_max, am);
        }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b)
        if (o[b].unsafe) o[b] = encode_block<Enc::Div>(h[b], o[b].scale, tab, no_rnd);
    if (live) {
        // non-temporal, as on the grouped path: streamed out now, not written back from
        // the caches while the next call's amax kernel reads
        __builtin_nontemporal_store(u32x4v{o[0].codes.x, o[0].codes.y, o[1].codes.x, o[1].codes.y},
                                    reinterpret_cast<u32x4v*>(a.codes + r * 64 + quarter * 16));
        *reinterpret_cast<uint16_t*>(a.scales + r * 8 + quarter * 2) = (uint16_t)(o[0].scale | (o[1].scale << 8));
    }
    if (AOUT) {
        const float wg = wg_max(live ? lane_max : 0.0f, red);
        if (threadIdx.x == 0)
            __hip_atomic_fetch_max(reinterpret_cast<uint32_t*>(a.amax_out), __builtin_bit_cast(uint32_t, wg),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

hipError_t launch_hadamard_quant_nvfp4(const DsaNvfp4Args& a, hipStream_t stream) {
    const bool given = a.amax_in != nullptr;
    hipError_t e = hipSuccess;
    if (!given && a.m > 0) {
        hipLaunchKernelGGL(k_dsa_nvfp4_amax, dim3((unsigned)a.n_wg), dim3(256), 0, stream, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_dsa_nvfp4_scale, dim3(1), dim3(kDsaScaleThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess || a.m == 0) return e;
    if (given && a.amax_out)
        hipLaunchKernelGGL((k_dsa_nvfp4_quant<true>), dim3((unsigned)a.n_wg), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((k_dsa_nvfp4_quant<false>), dim3((unsigned)a.n_wg), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mxq
