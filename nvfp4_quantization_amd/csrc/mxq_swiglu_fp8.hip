// mxq_swiglu_fp8.hip -- SwiGLU -> FP8 1x128 (gfx950).
//
// onnxruntime PR #33644 (Description): in a W8A8 MoE the second dynamic quantizer
// runs on consecutive K128 groups directly after the FP32 SiLU/SwiGLU of the gate and
// up projections, with no round to the input type in between, and uses the same FP8
// recipe as the first (s = max(amax, 1e-10) * F(1/448), saturating nearest-even
// E4M3, FP32 division).  h = fl(SILU(gate) * up) with SILU(g) = fl(g / fl(1 + EXP(-g))).
//
// EXP is a stated binary32 algorithm, so that every implementation of this call
// gives the same bits: Cody and Waite's argument reduction (Software Manual for the
// Elementary Functions, 1980) with ln 2 split into a 16-bit head and a tail, the
// degree-7 Taylor polynomial of e^r by Horner's rule with fma, and the power of two
// applied in two exact halves.  It is faithful (error below one ulp).
#include "mxq_device.hpp"
#include "mxq_internal.hpp"

namespace mxq {

namespace {

__device__ __forceinline__ float f32(uint32_t b) { return __builtin_bit_cast(float, b); }
// A NaN x stays NaN through every step (the clamps keep it, and it reaches p).
__device__ __forceinline__ float exp_stated(float x) {
    x = x > 128.0f ? 128.0f : x;              // e^128 and e^-128 are beyond binary32
    x = x < -128.0f ? -128.0f : x;
    const float k = __builtin_rintf(x * f32(0x3FB8AA3Bu));          // x * F(log2 e), nearest integer
    float r = __builtin_fmaf(-k, f32(0x3F317200u), x);              // ln 2 head: 0.693145751953125
    r = __builtin_fmaf(-k, f32(0x35BFBE8Eu), r);                    // F(ln 2 - head)
    float p = f32(0x39500D01u);                                      // F(1/7!)
    p = __builtin_fmaf(p, r, f32(0x3AB60B61u));                      // F(1/6!)
    p = __builtin_fmaf(p, r, f32(0x3C088889u));                      // F(1/5!)
    p = __builtin_fmaf(p, r, f32(0x3D2AAAABu));                      // F(1/4!)
    p = __builtin_fmaf(p, r, f32(0x3E2AAAABu));                      // F(1/3!)
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    // The stated two halves, (p 2^k1) 2^k2 with k1 = floor(k / 2): for |k| <= 185 and
    // p in [0.70, 1.42] the first product is an exact normal number, so the pair
    // rounds once, to the binary32 nearest p 2^k (overflowing to infinity), which is
    // what one ldexp gives.
    return __builtin_amdgcn_ldexpf(p, (int)k);
}

// g is a BF16 value.  For 2^-56 <= |g| <= 2^126 and t < 2^24 the reciprocal form is
// the correctly rounded quotient (div_rcp_bf16); zeros, tiny, huge and non-finite g,
// and t >= 2^24 (g below about -16.6), take the IEEE division.
__device__ __forceinline__ float silu(float g) {
    const float t = 1.0f + exp_stated(-g);
    const float ag = __builtin_fabsf(g);
    if (ag >= 0x1p-56f && ag <= 0x1p126f && t < 0x1p24f) return div_rcp_bf16(g, t);
    return g / t;                               // IEEE division, correctly rounded
}

// Bytes equal to 0xFF (the conversion's code for a NaN input) become 0x7F.
__device__ __forceinline__ uint32_t nan_codes_to_7f(uint32_t c) {
    uint32_t ff = c & (c >> 1) & (c >> 2) & (c >> 3) & (c >> 4) & (c >> 5) & (c >> 6) & (c >> 7) & 0x01010101u;
    return c ^ (ff * 0x80u);
}

}  // namespace

// One 128-element group is held by 8 consecutive lanes, 16 elements each; a
// 256-thread block covers 32 groups.
__global__ __launch_bounds__(256) void k_swiglu_quant_fp8(const SwigluFp8Args a) {
    const int64_t gpr = a.n >> 7;
    const int64_t total = a.m * gpr;
    const int64_t gi = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
    const int part = threadIdx.x & 7;
    const bool live = gi < total;
    const int64_t r = live ? gi / gpr : 0;
    const int64_t g = live ? gi - r * gpr : 0;

    uint4 g0 = {0, 0, 0, 0}, g1 = {0, 0, 0, 0}, u0 = {0, 0, 0, 0}, u1 = {0, 0, 0, 0};
    if (live) {
        const uint16_t* gs = a.gate + r * a.ld_gate + g * 128 + part * 16;
        const uint16_t* us = a.up + r * a.ld_up + g * 128 + part * 16;
        g0 = nt_load16(gs);
        g1 = nt_load16(gs + 8);
        u0 = nt_load16(us);
        u1 = nt_load16(us + 8);
    }
    const uint32_t gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const uint32_t uw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    float h[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h[2 * i] = silu(lo_bf16(gw[i])) * lo_bf16(uw[i]);
        h[2 * i + 1] = silu(hi_bf16(gw[i])) * hi_bf16(uw[i]);
    }
    // group max |h| without NaNs (fmax ignores the quiet NaNs arithmetic makes)
    float m = 0.0f;
    bool has_nan = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        m = __builtin_fmaxf(m, __builtin_fabsf(h[i]));
        has_nan |= h[i] != h[i];
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) m = __builtin_fmaxf(m, shfl_xor_f32(m, o));
    const float s = (m > k_floor() ? m : k_floor()) * k_inv448();
    // (an h that overflowed to inf makes s infinite: finite h / inf = +-0, inf / inf NaN)
    const float y = 1.0f / s, sd = fp8_divisor(s);
    const bool fix = has_nan || s == __builtin_inff();
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        c[j] = e4m3_pack4(div_rn(h[4 * j], sd, y), div_rn(h[4 * j + 1], sd, y), div_rn(h[4 * j + 2], sd, y),
                          div_rn(h[4 * j + 3], sd, y));
        if (fix) c[j] = nan_codes_to_7f(c[j]);
    }
    if (live) {
        *reinterpret_cast<uint4*>(a.q + r * a.ldq + g * 128 + part * 16) = make_uint4(c[0], c[1], c[2], c[3]);
        if (part == 0) a.scales[r * a.srow + g * a.sgroup] = s;
    }
}

hipError_t launch_swiglu_quant_fp8(const SwigluFp8Args& a, hipStream_t stream) {
    const int64_t blocks = (a.m * (a.n / 128) + 31) / 32;
    hipLaunchKernelGGL(k_swiglu_quant_fp8, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mxq
