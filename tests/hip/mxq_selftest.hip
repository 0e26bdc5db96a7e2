// mxq_selftest.hip -- test-only kernels (libmxq_selftest.so, not part of the
// quantization ABI): gfx950's conversion instructions, called in exactly the forms
// the quantizers use, swept over their whole input range on the device and compared
// there with reference encoders written below from the formats' definitions in
// integer arithmetic on the FP32 bit pattern.  They report mismatch counts and the
// first mismatching input of each class.
//
//   BF16   v_cvt_pk_bf16_f32 (__builtin_convertvector to bf16x2), both halves:
//          nearest-even for every non-NaN input; a NaN gives a NaN.
//   E4M3   v_cvt_pk_fp8_f32, all four bytes of the packed word: nearest-even with
//          saturation to 448 for every finite |v| < 464 (the kernels clamp or never
//          exceed that); a NaN gives a NaN code (low 7 bits 0x7F).
//   E2M1   v_cvt_scalef32_pk_fp4_f32 with scale 1, both nibbles of bytes 0 and 3:
//          nearest-even with saturation to 6 for every non-NaN input, the sign kept.
//   E2M1 stochastic   v_cvt_scalef32_sr_pk_fp4_f32 with scale 1 as the quantizers
//          issue it (mxq::e2m1_sr8: eight conversions, the value in the pair's first
//          slot, the random operand r << 24 in both the second slot and the random
//          operand, each code written into one byte of a kept destination, then
//          packed): for grid spacing D (0.5 / 1 / 2 below 2 / 4 / 6) and
//          |q| / D = k + f, the code rounds up iff floor(256 f) + r >= 256; |q| >= 6
//          saturates; swept over every non-NaN q, both signs, every r and every
//          nibble position (in two classes: |q| in [2^-20, 16), and the rest).
//   Division by a hardware reciprocal (mxq::div_rcp_bf16, SwiGLU's SiLU): div_rn's
//          correction step on v_rcp_f32's reciprocal against IEEE division, for every
//          BF16 numerator significand, both signs, and every divisor in [1, 2^24).
//
// Every kernel is a grid-stride loop over a fixed index range whose only memory
// accesses are one atomic per wave into its result words at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_device.hpp"

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned long long u64;

// ---------------------------------------------------------------- references
__device__ uint32_t ref_bf16(uint32_t b) {                  // b not a NaN
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// E4M3FN of a finite v with |v| < 464: nearest-even, saturating to 0x7E (448).
__device__ uint32_t ref_e4m3(uint32_t b) {
    const uint32_t sign = (b >> 24) & 0x80u, a = b & 0x7FFFFFFFu;
    const uint32_t E = a >> 23;
    if (E == 0) return sign;                                 // FP32 subnormal: far below 2^-10
    const uint32_t S = (a & 0x7FFFFFu) | 0x800000u;          // 24-bit significand
    const int e = (int)E - 127;                              // a = S 2^(e-23)
    uint32_t code;
    if (e >= -6) {                                           // E4M3 normal range: 3 fraction bits
        uint32_t q = S >> 20, rem = S & 0xFFFFFu;
        if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
        int ee = e;
        if (q == 16u) { q = 8u; ++ee; }
        const int field = ee + 7;
        code = (field > 15 || (field == 15 && (q & 7u) == 7u)) ? 0x7Eu : ((uint32_t)field << 3) | (q & 7u);
    } else {                                                 // in units of 2^-9: S 2^(e-14)
        const int sh = 14 - e;                               // >= 21
        if (sh >= 32) {
            code = 0u;                                       // below 2^-10 (ties impossible: S < 2^24)
        } else {
            uint32_t q = S >> sh;
            const uint32_t rem = S & ((1u << sh) - 1u), half = 1u << (sh - 1);
            if (rem > half || (rem == half && (q & 1u))) ++q;
            code = q;                                        // 8 = 2^-6, the smallest normal
        }
    }
    return sign | code;
}

// E2M1 of a non-NaN v: nearest-even, saturating to 6; each comparison is against a
// rounding boundary, strict where the tie goes down to the even code.
__device__ uint32_t ref_e2m1(uint32_t b) {
    const uint32_t sign = (b >> 28) & 0x8u, a = b & 0x7FFFFFFFu;
    const uint32_t c = (a > 0x3E800000u) + (a >= 0x3F400000u) + (a > 0x3FA00000u) + (a >= 0x3FE00000u) +
                       (a > 0x40200000u) + (a >= 0x40600000u) + (a > 0x40A00000u);   // 0.25 .75 1.25 1.75 2.5 3.5 5
    return sign | c;
}

// Stochastic E2M1 of a non-NaN q with 8 random bits r.
__device__ uint32_t ref_e2m1_sr(uint32_t b, uint32_t r) {
    const uint32_t sign = (b >> 28) & 0x8u, a = b & 0x7FFFFFFFu;
    if (a >= 0x40C00000u) return sign | 7u;                  // |q| >= 6 (and inf)
    const int d = a < 0x40000000u ? -1 : (a < 0x40800000u ? 0 : 1);   // D = 2^d
    const uint32_t E = a >> 23;
    const uint64_t S = E ? ((a & 0x7FFFFFu) | 0x800000u) : (a & 0x7FFFFFu);
    const int e = E ? (int)E - 127 : -126;                   // |q| = S 2^(e-23)
    const int sh = 15 + d - e;                               // floor(256 |q| / D) = S >> sh; sh >= 14
    const uint64_t T = sh >= 64 ? 0 : (S >> sh);
    const uint32_t k = (uint32_t)(T >> 8), F = (uint32_t)(T & 255u);
    const uint32_t K = k + (F + r >= 256u ? 1u : 0u);
    const uint32_t code = d < 0 ? K : (d == 0 ? K + 2u : K + 4u);   // K D on the grid
    return sign | code;
}

__device__ bool is_nan(uint32_t b) { return (b & 0x7FFFFFFFu) > 0x7F800000u; }

// One atomic per wave: the wave's sum into out[i], its minimum into out[j].
__device__ void add_count(u64* out, int i, u64 v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if ((threadIdx.x & 63) == 0 && v) atomicAdd(out + i, v);
}
__device__ void min_key(u64* out, int j, u64 v) {
    for (int o = 32; o > 0; o >>= 1) {
        const u64 w = __shfl_xor(v, o, 64);
        v = w < v ? w : v;
    }
    if ((threadIdx.x & 63) == 0 && v != ~0ull) atomicMin(out + j, v);
}
__device__ __forceinline__ void keep_min(u64& m, u64 v) { m = v < m ? v : m; }

// ---------------------------------------------------------------- sweeps
// out[0] E4M3 mismatches, [1] E4M3 NaN inputs without a NaN code, [2] BF16
// mismatches, [3] BF16 NaN inputs without a NaN, [4] E2M1 mismatches, [5] inputs;
// out[8 + c]: the smallest mismatching input bits of class c (the caller fills
// out[8..15] with all-ones first).
__global__ __launch_bounds__(256) void k_sweep_conversions(u64* out) {
    u64 n[5] = {0, 0, 0, 0, 0}, first[5] = {~0ull, ~0ull, ~0ull, ~0ull, ~0ull}, seen = 0;
    const u64 stride = (u64)gridDim.x * blockDim.x;
    for (u64 i = (u64)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 32); i += stride) {
        const uint32_t b = (uint32_t)i, nb = b ^ 0x80000000u;
        const float v = __builtin_bit_cast(float, b), nv = __builtin_bit_cast(float, nb);
        ++seen;
        // E4M3: bytes 0..3 = v, -v, v, -v
        uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(v, nv, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(v, nv, (int)w, true);
        if (is_nan(b)) {
            bool bad = false;
            for (int k = 0; k < 4; ++k) bad |= ((w >> (8 * k)) & 0x7Fu) != 0x7Fu;
            if (bad) { ++n[1]; keep_min(first[1], b); }
        } else if ((b & 0x7FFFFFFFu) < 0x43E80000u) {        // |v| < 464
            const uint32_t want = ref_e4m3(b) | (ref_e4m3(nb) << 8) | (ref_e4m3(b) << 16) | (ref_e4m3(nb) << 24);
            if (w != want) { ++n[0]; keep_min(first[0], b); }
        }
        // BF16: both halves
        const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{v, nv}), bf16x2));
        if (is_nan(b)) {
            if ((h & 0x7FFFu) <= 0x7F80u || ((h >> 16) & 0x7FFFu) <= 0x7F80u) { ++n[3]; keep_min(first[3], b); }
        } else if (h != (ref_bf16(b) | (ref_bf16(nb) << 16))) {
            ++n[2]; keep_min(first[2], b);
        }
        // E2M1: nibbles of byte 0 and byte 3 = v, -v
        if (!is_nan(b)) {
            uint32_t f = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v, nv, 1.0f, 0);
            f = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(f, v, nv, 1.0f, 3);
            const uint32_t pair = ref_e2m1(b) | (ref_e2m1(nb) << 4);
            if ((f & 0xFFu) != pair || (f >> 24) != pair) { ++n[4]; keep_min(first[4], b); }
        }
    }
    for (int c = 0; c < 5; ++c) {
        add_count(out, c, n[c]);
        min_key(out, 8 + c, first[c]);
    }
    add_count(out, 5, seen);
}

// Every non-NaN magnitude m (both signs) and every r.  out[0] mismatches with |q| in
// [2^-20, 16), out[1] the others, out[2] conversions checked; out[8] / out[9] the
// smallest mismatching (q bits << 8 | r) of each class.
__global__ __launch_bounds__(256) void k_sweep_sr(u64* out) {
    u64 bad_in = 0, bad_out = 0, seen = 0, first_in = ~0ull, first_out = ~0ull;
    const u64 stride = (u64)gridDim.x * blockDim.x;
    for (u64 m = (u64)blockIdx.x * blockDim.x + threadIdx.x; m <= 0x7F800000ull; m += stride) {
        const bool in = m >= 0x35800000ull && m < 0x41800000ull;
        // nibble i holds sign s ^ (i & 1) with random byte r0 + i: over both s, every
        // (sign, r) pair is checked once
        for (uint32_t s = 0; s < 2; ++s) {
            const uint32_t b0 = (uint32_t)m | (s << 31);
            float q[8];
            for (int i = 0; i < 8; ++i) q[i] = __builtin_bit_cast(float, b0 ^ ((uint32_t)(i & 1) << 31));
            for (uint32_t r0 = 0; r0 < 256; r0 += 8) {
                uint32_t rb[8];
                for (int i = 0; i < 8; ++i) rb[i] = (r0 + i) << 24;
                const uint32_t got = mxq::e2m1_sr8(q, rb);
                for (int i = 0; i < 8; ++i) {
                    const uint32_t b = b0 ^ ((uint32_t)(i & 1) << 31), r = r0 + i;
                    if (((got >> (4 * i)) & 0xFu) != ref_e2m1_sr(b, r)) {
                        if (in) { ++bad_in; keep_min(first_in, ((u64)b << 8) | r); }
                        else { ++bad_out; keep_min(first_out, ((u64)b << 8) | r); }
                    }
                }
            }
            seen += 256;
        }
    }
    add_count(out, 0, bad_in);
    add_count(out, 1, bad_out);
    add_count(out, 2, seen);
    min_key(out, 8, first_in);
    min_key(out, 9, first_out);
}

// mxq::div_rcp_bf16 against IEEE division: every BF16 numerator significand
// (x = 1 + k/128, both signs) against every divisor t in [1, 2^24) (24 binades x 2^23
// significands).  out[0] mismatches, out[2] pairs checked, out[8] the smallest
// mismatching (t bits << 8 | k).
__global__ __launch_bounds__(256) void k_sweep_div_rcp(u64* out) {
    u64 bad = 0, seen = 0, first = ~0ull;
    const u64 stride = (u64)gridDim.x * blockDim.x;
    for (u64 i = (u64)blockIdx.x * blockDim.x + threadIdx.x; i < 24ull << 23; i += stride) {
        const uint32_t tb = ((uint32_t)(127 + (i >> 23)) << 23) | (uint32_t)(i & 0x7FFFFFu);
        const float t = __builtin_bit_cast(float, tb);
        for (uint32_t k = 0; k < 128; ++k) {
            const float x = __builtin_bit_cast(float, 0x3F800000u | (k << 16));
            const float q = mxq::div_rcp_bf16(x, t), qn = mxq::div_rcp_bf16(-x, t);
            const float want = x / t;
            if (__builtin_bit_cast(uint32_t, q) != __builtin_bit_cast(uint32_t, want) ||
                __builtin_bit_cast(uint32_t, qn) != (__builtin_bit_cast(uint32_t, want) ^ 0x80000000u)) {
                ++bad;
                keep_min(first, ((u64)tb << 8) | k);
            }
        }
        seen += 256;
    }
    add_count(out, 0, bad);
    add_count(out, 2, seen);
    min_key(out, 8, first);
}

}  // namespace

extern "C" {

// Each enqueues one sweep on the stream; out: 16 device words (out[8..15] filled
// with all-ones and out[0..7] with zero by the caller).  0 on success.
int mxq_selftest_conversions(unsigned long long* out, void* stream) {
    if (!out) return 1;
    hipLaunchKernelGGL(k_sweep_conversions, dim3(8192), dim3(256), 0, static_cast<hipStream_t>(stream), out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int mxq_selftest_div_rcp(unsigned long long* out, void* stream) {
    if (!out) return 1;
    hipLaunchKernelGGL(k_sweep_div_rcp, dim3(8192), dim3(256), 0, static_cast<hipStream_t>(stream), out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int mxq_selftest_sr(unsigned long long* out, void* stream) {
    if (!out) return 1;
    hipLaunchKernelGGL(k_sweep_sr, dim3(16384), dim3(256), 0, static_cast<hipStream_t>(stream), out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
