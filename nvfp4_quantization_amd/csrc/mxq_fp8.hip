// mxq_fp8.hip -- FP8 1x128 quantization and the DSA rotate + FP8 path (gfx950).
//
// FP8 recipe: onnxruntime PR #33644 (QMoE dynamic FP8 activation quantization),
// Description -- per K128 group s = max(amax, 1e-10) * float32(1/448), x / s by
// FP32 division, saturating nearest-even E4M3FN.
// DSA: TensorRT-LLM PR #15158, Summary -- cat[qk_pe, qk_nope] -> Hadamard
// rotation -> fp8_quantize_1x128, here fused into one pass over HBM.
#include "mxq_device.hpp"
#include "mxq_internal.hpp"

namespace mxq {

// Bytes equal to 0xFF (the hardware's code for a NaN input) become 0x7F.
__device__ __forceinline__ uint32_t fix_nan_codes(uint32_t c) {
    uint32_t ff = c & (c >> 1) & (c >> 2) & (c >> 3) & (c >> 4) & (c >> 5) & (c >> 6) & (c >> 7) & 0x01010101u;
    return c ^ (ff * 0x80u);
}

// One 128-element group is held by 8 consecutive lanes, 16 elements each
// (two 16-byte loads); a 256-thread block covers 32 groups.  UE8M0: the scale is
// rounded up to a power of two.
template <bool UE8M0>
__global__ __launch_bounds__(256) void k_quant_fp8_1x128(const Fp8Args a) {
    const int64_t gpr = a.k >> 7;
    const int64_t total = a.m * gpr;
    const int64_t gi = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
    const int part = threadIdx.x & 7;
    const bool live = gi < total;
    const int64_t r = live ? gi / gpr : 0;
    const int64_t g = live ? gi - r * gpr : 0;

    uint4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
    if (live) {
        const uint4* src = reinterpret_cast<const uint4*>(a.x + r * a.ldx + g * 128 + part * 16);
        v0 = src[0];
        v1 = src[1];
    }
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
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
        uint32_t other = shfl_xor_u32(m, o);
        m = other > m ? other : m;
    }
    const float amax = bf16_mag(m);
    float s = (amax > k_floor() ? amax : k_floor()) * k_inv448();
    if (UE8M0) s = pow2_ceil(s);
    const float y = 1.0f / s, sd = fp8_divisor(s);
    const bool fix = has_nan || s == __builtin_inff();   // NaN codes: NaN elements, or inf / inf
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        c[j] = e4m3_pack4(div_rn(lo_bf16(w[2 * j]), sd, y), div_rn(hi_bf16(w[2 * j]), sd, y),
                          div_rn(lo_bf16(w[2 * j + 1]), sd, y), div_rn(hi_bf16(w[2 * j + 1]), sd, y));
        if (fix) c[j] = fix_nan_codes(c[j]);
    }
    if (live) {
        *reinterpret_cast<uint4*>(a.q + r * a.ldq + g * 128 + part * 16) = make_uint4(c[0], c[1], c[2], c[3]);
        if (part == 0) a.scales[r * a.srow + g * a.sgroup] = s;
    }
}

hipError_t launch_quant_fp8_1x128(const Fp8Args& a, hipStream_t stream, bool ue8m0) {
    const int64_t groups = a.m * (a.k / 128);
    const int64_t blocks = (groups + 31) / 32;
    if (ue8m0)
        hipLaunchKernelGGL(k_quant_fp8_1x128<true>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(k_quant_fp8_1x128<false>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// One 128-element row v = cat(pe, nope) is held by 4 lanes, 32 consecutive
// elements each.  Butterfly stages h = 1..16 run inside a lane; h = 32 and 64
// pair lanes (q ^ 1) and (q ^ 2).  A 256-thread block covers 64 rows.  UE8M0:
// the scale is rounded up to a power of two.
constexpr int kStageDwords = 36;      // a row's 128 codes + 16 bytes of padding
template <bool UE8M0>
__global__ __launch_bounds__(256) void k_hadamard_quant_fp8(const DsaArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t stage[64 * kStageDwords];
    const int quarter = threadIdx.x & 3;
    const int64_t r = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
    const bool live = r < a.m;

    float v[32];
    wht128_quarter(a.pe, a.ld_pe, a.d_pe, a.nope, a.ld_nope, r, live, quarter, v);
    uint32_t w[16];
    const float c = k_inv_sqrt128();
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = pack_bf16(v[2 * i] * c, v[2 * i + 1] * c);

    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = absmax_pk(m, w[i]);
    m = fold_pk(m);
    const bool has_nan = m > 0x7F80u;
    if (has_nan) {
        m = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) m = absmax_pk_nonan(m, w[i]);
    }
#pragma unroll
    for (int o = 1; o < 4; o <<= 1) {
        uint32_t other = shfl_xor_u32(m, o);
        m = other > m ? other : m;
    }
    const float amax = bf16_mag(m);
    float s = (amax > k_floor() ? amax : k_floor()) * k_inv448();
    if (UE8M0) s = pow2_ceil(s);
    const float y = 1.0f / s, sd = fp8_divisor(s);
    const bool fix = has_nan || s == __builtin_inff();   // NaN codes: NaN values, or inf / inf
    uint32_t cd[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        cd[j] = e4m3_pack4(div_rn(lo_bf16(w[2 * j]), sd, y), div_rn(hi_bf16(w[2 * j]), sd, y),
                           div_rn(lo_bf16(w[2 * j + 1]), sd, y), div_rn(hi_bf16(w[2 * j + 1]), sd, y));
        if (fix) cd[j] = fix_nan_codes(cd[j]);
    }
    // The work-group's 64 x 128 codes leave through LDS, so that 8 lanes store each
    // row's 128 bytes as one line (the computing lanes hold 32 bytes each).  They are
    // stored non-temporally: they stream out now instead of being written back from
    // the caches during the next call's reads (3 % faster in steady state).
    uint32_t* st = stage + (threadIdx.x >> 2) * kStageDwords + quarter * 8;
    *reinterpret_cast<uint4*>(st) = make_uint4(cd[0], cd[1], cd[2], cd[3]);
    *reinterpret_cast<uint4*>(st + 4) = make_uint4(cd[4], cd[5], cd[6], cd[7]);
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int idx = it * 256 + (int)threadIdx.x;
        const int row = idx >> 3, part = idx & 7;
        const int64_t rr = (int64_t)blockIdx.x * 64 + row;
        if (rr < a.m) {
            const uint4 v = *reinterpret_cast<const uint4*>(stage + row * kStageDwords + part * 4);
            __builtin_nontemporal_store(u32x4v{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4v*>(a.q + rr * 128 + part * 16));
        }
    }
    if (live) {
        if (quarter == 0) {
            const int64_t token = r / a.heads, head = r - token * a.heads;
            a.scales[token * a.stride_token + head * a.stride_head] = s;
        }
    }
}

hipError_t launch_hadamard_quant_fp8(const DsaArgs& a, hipStream_t stream, bool ue8m0) {
    const int64_t blocks = (a.m + 63) / 64;
    if (ue8m0)
        hipLaunchKernelGGL(k_hadamard_quant_fp8<true>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(k_hadamard_quant_fp8<false>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mxq
