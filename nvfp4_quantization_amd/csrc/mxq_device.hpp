// mxq_device.hpp -- device-side building blocks shared by the mxq HIP kernels
// (gfx950 / CDNA4, wave64).
//
// Every helper is exact with respect to IEEE binary32 arithmetic with one
// rounding per operation:
//  * BF16 -> FP32 widening is a 16-bit shift (exact).
//  * div_rn(x, d, y) returns fl(x / d) given y = fl(1 / d): q0 = fl(x*y) is within
//    one ulp, the FMA residual r = x - q0*d is exact, and fl(q0 + r*y) is the
//    correctly rounded quotient (Markstein's correction step, a theorem for every
//    x and d whose values stay normal).  tests/test_exactness_cpu.py checks it
//    exhaustively for every BF16 numerator significand and every numerator
//    fl(a * F(1/6)) (a BF16) against every FP32 divisor significand, and for
//    arbitrary FP32 numerators (the SwiGLU path's) on random pairs and on pairs
//    whose quotient lies next to a rounding midpoint.
//  * The E4M3 / E2M1 / BF16 conversions use gfx950's hardware conversions.  Over
//    all 2^32 FP32 inputs they equal nearest-even with saturation for every
//    finite input below 464 (E4M3) and every non-NaN input (E2M1, BF16)
//    (tests/test_gpu_exactness.py sweeps them on the device); the kernels clamp
//    to 448 (or never exceed 464) before the E4M3 conversion.  A NaN converts to
//    a NaN code: FP8 element codes turn it into 0x7F, block scales mask it to the
//    NaN code 0x7F.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// FP32 constants, each the binary32 value nearest to the real number named.
__device__ __forceinline__ float k_floor() { return __builtin_bit_cast(float, 0x2EDBE6FFu); }      // 1e-10
__device__ __forceinline__ float k_inv448() { return __builtin_bit_cast(float, 0x3B124925u); }     // 1/448
__device__ __forceinline__ float k_inv2688() { return __builtin_bit_cast(float, 0x39C30C31u); }    // 1/2688
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));   // for vector non-temporal accesses
typedef unsigned u32x2v __attribute__((ext_vector_type(2)));

// 16 bytes loaded non-temporally, for a kernel that is the data's last reader.  Not
// a rule: it pays for wide tiles (the grouped quantize pass, the blockwise and SwiGLU
// kernels) and costs 5-25 % on the kernels that read 256-byte rows a quarter per lane
// (1x128 FP8 and the Hadamard paths), which keep plain loads.
__device__ __forceinline__ uint4 nt_load16(const void* p) {
    const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float k_inv6() { return __builtin_bit_cast(float, 0x3E2AAAABu); }       // 1/6
// all-ones bit pattern (a table word used as an AND mask, never as a number)
__device__ __forceinline__ float k_keep_codes() { return __builtin_bit_cast(float, 0xFFFFFFFFu); }
__device__ __forceinline__ float k_inv_sqrt128() { return __builtin_bit_cast(float, 0x3DB504F3u); } // 1/sqrt(128)

__device__ __forceinline__ float lo_bf16(uint32_t p) { return __builtin_bit_cast(float, p << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t p) { return __builtin_bit_cast(float, p & 0xFFFF0000u); }

// Round two floats to BF16 (nearest-even) and pack them: a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    f32x2 v = {a, b};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// Running maximum of |BF16| bit patterns over packed pairs (v_pk_max_u16).
// A result above 0x7F80 means a NaN was seen.
__device__ __forceinline__ uint32_t absmax_pk(uint32_t acc, uint32_t p) {
    u16x2 a = __builtin_bit_cast(u16x2, acc);
    u16x2 b = __builtin_bit_cast(u16x2, p & 0x7FFF7FFFu);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}
__device__ __forceinline__ uint32_t fold_pk(uint32_t acc) {
    uint32_t lo = acc & 0xFFFFu, hi = acc >> 16;
    return lo > hi ? lo : hi;
}
// |BF16| bit pattern -> FP32 value (exact).
__device__ __forceinline__ float bf16_mag(uint32_t m) { return __builtin_bit_cast(float, m << 16); }

// max |v| over the non-NaN BF16 values of packed pairs (the slow path after a
// NaN was seen).
__device__ __forceinline__ uint32_t absmax_pk_nonan(uint32_t acc, uint32_t p) {
    uint32_t lo = p & 0x7FFFu, hi = (p >> 16) & 0x7FFFu;
    if (lo <= 0x7F80u && lo > acc) acc = lo;
    if (hi <= 0x7F80u && hi > acc) acc = hi;
    return acc;
}

// fl(x / d) given y = fl(1 / d)  (see the header comment).  The residual is
// formed as q0*d - x and subtracted, so that x = -0 keeps its sign: -0 * y = -0,
// (-0)*d - (-0) = +0, and -0 - (+0)*y = -0 (the other sign order would give +0).
__device__ __forceinline__ float div_rn(float x, float d, float y) {
    float q0 = x * y;
    float rn = __builtin_fmaf(q0, d, -x);
    return __builtin_fmaf(-rn, y, q0);
}

// fl(x / t) for a BF16 numerator x (8-bit significand) and a divisor t in [1, 2^24),
// with 2^-56 <= |x| <= 2^126 (callers check the range and divide otherwise): div_rn's
// correction step on the hardware reciprocal.  tests/test_gpu_exactness.py sweeps
// every BF16 numerator significand, both signs, against every divisor in [1, 2^24) on
// the device (5.2e10 pairs, no mismatch).  Scaling x by 2^e scales every intermediate
// exactly, each rounding included, while all of them stay normal: for x in [1, 2) a
// nonzero residual fma(q0, t, -x) is a multiple of 2^-70 (q0 >= 2^-24, t >= 1), so it
// stays normal for e >= -56; q0 and the quotient stay above 2^-80, and below
// |x| <= 2^126.
__device__ __forceinline__ float div_rcp_bf16(float x, float t) {
    return div_rn(x, t, __builtin_amdgcn_rcpf(t));
}

// fl(x / d) with IEEE's special cases: div_fixup returns the quotient of infinite
// or zero operands as IEEE division gives it (inf / finite = inf, finite / inf = 0,
// inf / inf = NaN, ...) and div_rn's correctly rounded quotient otherwise (div_rn
// alone gives NaN for an infinite x or d).
__device__ __forceinline__ float div_ieee(float x, float d, float y) {
    return __builtin_amdgcn_div_fixupf(div_rn(x, d, y), d, x);
}

// The divisor that div_rn takes for an FP8 scale s (y = fl(1/s)): s, or for an
// infinite s (an infinite group amax) the largest finite value.  With y = 0 the
// quotient then comes out as IEEE's x / inf: +-0 for finite x, NaN for infinite x
// (div_rn(x, inf, 0) would give NaN for every x).
__device__ __forceinline__ float fp8_divisor(float s) { return __builtin_fminf(s, 0x1.fffffep127f); }

// E4M3 code (low byte) of a finite v with |v| < 464; nearest-even.
// (The conversion keeps the high half of its third operand, which the mask drops:
// passing v's own bits there lets it write v's register in place.)
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(v, v, __builtin_bit_cast(int, v), false) & 0xFFu;
}
__device__ __forceinline__ float e4m3_value(uint32_t code) {
    return __builtin_amdgcn_cvt_f32_fp8(code, 0);
}
// The smallest power of two >= s (s > 0 normal): a scale a UE8M0 byte can hold.
__device__ __forceinline__ float pow2_ceil(float s) {
    const uint32_t b = __builtin_bit_cast(uint32_t, s);
    return __builtin_bit_cast(float, (b & 0x7FFFFFu) ? (b & 0xFF800000u) + 0x00800000u : b);
}

// Four E4M3 codes packed into a dword, a in the lowest byte.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Two E2M1 codes (nearest-even, saturating at 6) written into byte `sel` of w:
// a in the low nibble, b in the high nibble.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t w, float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, SEL);
}

// The random byte t (0..3) of word w placed at bits 24..31 with the low 24 bits zero,
// the form the stochastic conversion takes (one byte permute).
template <int T>
__device__ __forceinline__ uint32_t rbyte_hi(uint32_t w) {
    return __builtin_amdgcn_perm(0u, w, ((uint32_t)T << 24) | 0x0C0C0Cu);
}

// Stochastic E2M1 rounding with 8 random bits r: grid spacing D = 0.5 / 1 / 2
// below 2 / 4 / 6; with u = |q| / D = k + f the value rounds up iff
// floor(256 f) + r >= 256; |q| >= 6 saturates.  gfx950's stochastic conversion does
// exactly this for the first value of a pair when the random operand is r << 24 (its
// low 24 bits zero): tests/test_gpu_exactness.py checks it against the rule for every
// non-NaN FP32 value and every r.  (The pair's second value draws on the random
// operand differently, so each value gets a conversion of its own.)
//
// Eight such codes packed (nibble i = code of q[i] with random byte rb[i], each given
// as r << 24).  The conversion writes one byte of its destination and keeps the other
// three, but the builtin's first operand does not reach the instruction (the compiler
// gives it a fresh destination whose other bytes are stale), so the eight conversions
// are written out with the destinations kept: even elements into bytes 0..3 of e, odd
// ones into o, each code in the low nibble of its byte.  A pair's second slot holds
// the random operand itself, which already sits in the register after q, so forming
// the pair costs no move; its code fills the byte's high nibble and is masked off.  A
// byte-select write needs one wait state before the next instruction reads that
// register; the order alternates e and o so no conversion reads the one just before
// (after the block the compiler inserts the wait itself).
__device__ __forceinline__ uint32_t e2m1_sr8(const float (&q)[8], const uint32_t (&rb)[8]) {
    uint32_t e, o;
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %2, %10, 1.0\n\t"
        "v_cvt_scalef32_sr_pk_fp4_f32 %1, %3, %11, 1.0\n\t"
        "v_cvt_scalef32_sr_pk_fp4_f32 %0, %4, %12, 1.0 op_sel:[0,0,1,0]\n\t"
        "v_cvt_scalef32_sr_pk_fp4_f32 %1, %5, %13, 1.0 op_sel:[0,0,1,0]\n\t"
        "v_cvt_scalef32_sr_pk_fp4_f32 %0, %6, %14, 1.0 op_sel:[0,0,0,1]\n\t"
        "v_cvt_scalef32_sr_pk_fp4_f32 %1, %7, %15, 1.0 op_sel:[0,0,0,1]\n\t"
        "v_cvt_scalef32_sr_pk_fp4_f32 %0, %8, %16, 1.0 op_sel:[0,0,1,1]\n\t"
        "v_cvt_scalef32_sr_pk_fp4_f32 %1, %9, %17, 1.0 op_sel:[0,0,1,1]"
        : "=&v"(e), "=&v"(o)
        : "v"(f32x2{q[0], __builtin_bit_cast(float, rb[0])}), "v"(f32x2{q[1], __builtin_bit_cast(float, rb[1])}),
          "v"(f32x2{q[2], __builtin_bit_cast(float, rb[2])}), "v"(f32x2{q[3], __builtin_bit_cast(float, rb[3])}),
          "v"(f32x2{q[4], __builtin_bit_cast(float, rb[4])}), "v"(f32x2{q[5], __builtin_bit_cast(float, rb[5])}),
          "v"(f32x2{q[6], __builtin_bit_cast(float, rb[6])}), "v"(f32x2{q[7], __builtin_bit_cast(float, rb[7])}),
          "v"(rb[0]), "v"(rb[1]), "v"(rb[2]), "v"(rb[3]), "v"(rb[4]), "v"(rb[5]), "v"(rb[6]), "v"(rb[7]));
    return (e & 0x0F0F0F0Fu) | ((o << 4) & 0xF0F0F0F0u);
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11).  Each round's two 32 x 32-bit
// products are formed whole (64 bits), one v_mad_u64_u32 each: the separate low and
// high multiplies would cost two quarter-rate instructions per product.  After the
// first round each three-way XOR is one v_bitop3_b32 (truth table 0x96), which the
// compiler does not form from the two XORs by itself.
struct u32x4 { uint32_t x, y, z, w; };
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.x, p1 = (uint64_t)0xCD9E8D57u * c.z;
        const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
        const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
        u32x4 n;
        if (i == 0) {                            // c.y, c.w may be uniform: let the compiler pair them
            n.x = hi1 ^ (c.y ^ k0);
            n.z = hi0 ^ (c.w ^ k1);
        } else {
            n.x = __builtin_amdgcn_bitop3_b32(hi1, c.y, k0, 0x96);
            n.z = __builtin_amdgcn_bitop3_b32(hi0, c.w, k1, 0x96);
        }
        n.y = lo1;
        n.w = lo0;
        c = n;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}


// Cross-lane helpers (wave64).
__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int m) {
    return (uint32_t)__shfl_xor((int)v, m, 64);
}
__device__ __forceinline__ float shfl_xor_f32(float v, int m) {
    return __shfl_xor(v, m, 64);
}

// The value of another lane of the same quad (4 consecutive lanes): DPP quad_perm
// control PERM (0xB1: lane ^ 1, 0x4E: lane ^ 2).
template <int PERM>
__device__ __forceinline__ float quad_swap(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), PERM, 0xF, 0xF, true));
}

// v[i] += sgn * (v[i] of the quad's lane PERM) for 32 values, one DPP v_fmac_f32 each
// (a product by +-1 is exact: one rounding).  In 16-value blocks of inline assembly
// (the compiler does not fold a DPP move into v_fmac_f32); each block starts with the
// two wait states that a DPP read of a VGPR needs after a VALU write of it.
#define MXQ_QF(n) "v_fmac_f32_dpp %" #n ", %" #n ", %16 " MXQ_QP " row_mask:0xf bank_mask:0xf\n\t"
#define MXQ_QF16 MXQ_QF(0) MXQ_QF(1) MXQ_QF(2) MXQ_QF(3) MXQ_QF(4) MXQ_QF(5) MXQ_QF(6) MXQ_QF(7) \
                 MXQ_QF(8) MXQ_QF(9) MXQ_QF(10) MXQ_QF(11) MXQ_QF(12) MXQ_QF(13) MXQ_QF(14) MXQ_QF(15)
template <int PERM>
__device__ __forceinline__ void quad_fmac16(float* v, float sgn) {
    static_assert(PERM == 0xB1 || PERM == 0x4E, "quad_perm lane ^ 1 or lane ^ 2");
    if constexpr (PERM == 0xB1) {
#define MXQ_QP "quad_perm:[1,0,3,2]"
        asm("s_nop 1\n\t" MXQ_QF16
            : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),
              "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])
            : "v"(sgn));
#undef MXQ_QP
    } else {
#define MXQ_QP "quad_perm:[2,3,0,1]"
        asm("s_nop 1\n\t" MXQ_QF16
            : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),
              "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])
            : "v"(sgn));
#undef MXQ_QP
    }
}
#undef MXQ_QF16
#undef MXQ_QF
template <int PERM>
__device__ __forceinline__ void quad_fmac32(float (&v)[32], float sgn) {
    quad_fmac16<PERM>(v, sgn);
    quad_fmac16<PERM>(v + 16, sgn);
}

// The 128-point Walsh-Hadamard butterfly of v = cat(pe[r][0:d_pe], nope[r][0:128-d_pe])
// held by 4 consecutive lanes: lane `quarter` loads elements 32q .. 32q+31 (d_pe a
// multiple of 8, so an 8-element load never straddles pe and nope) and ends with
// outputs 32q .. 32q+31 before the constant: stages h = 1..16 run inside the lane,
// h = 32 and 64 pair lanes quarter ^ 1 and quarter ^ 2.  A lane that is not live
// works on zeros (its partners' rows are its own, so it changes no live output).
//
// MAG: the caller reads only |v| (a maximum).  Each cross-lane step is then one
// v_fmac_f32 whose partner operand comes over DPP, v + sgn * other, instead of a DPP
// move and fma(v, sgn, other): the upper lane of a pair holds other - v negated, and
// after both stages every lane holds plus or minus the butterfly's value, rounded
// alike (rounding to nearest is symmetric; NaNs and infinities arise from the same
// operands).
template <bool MAG = false>
__device__ __forceinline__ void wht128_quarter(const uint16_t* pe, int64_t ld_pe, int32_t d_pe,
                                               const uint16_t* nope, int64_t ld_nope, int64_t r, bool live,
                                               int quarter, float (&v)[32]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e0 = (quarter * 4 + q) * 8;
        uint4 w = {0, 0, 0, 0};
        if (live) {
            const uint16_t* src = e0 < d_pe ? pe + r * ld_pe + e0 : nope + r * ld_nope + (e0 - d_pe);
            w = *reinterpret_cast<const uint4*>(src);
        }
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[q * 8 + 2 * i] = lo_bf16(ww[i]);
            v[q * 8 + 2 * i + 1] = hi_bf16(ww[i]);
        }
    }
#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            if (i & h) continue;
            const float x0 = v[i], x1 = v[i + h];
            v[i] = x0 + x1;
            v[i + h] = x0 - x1;
        }
    }
    if (MAG) {
        quad_fmac32<0xB1>(v, (quarter & 1) ? -1.0f : 1.0f);
        quad_fmac32<0x4E>(v, (quarter & 2) ? -1.0f : 1.0f);
        return;
    }
    // the upper lane of a pair forms other - v, the lower v + other: both are
    // fma(v, +-1, other), exact products with one rounding (signed zeros included);
    // the partner's value comes over the quad's data-parallel crossbar (DPP)
    {
        const float sgn = (quarter & 1) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf(v[i], sgn, quad_swap<0xB1>(v[i]));   // lane ^ 1
    }
    {
        const float sgn = (quarter & 2) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf(v[i], sgn, quad_swap<0x4E>(v[i]));   // lane ^ 2
    }
}

}  // namespace mxq
