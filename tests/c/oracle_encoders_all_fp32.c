/* oracle_encoders_all_fp32.c -- the oracle's format encoders against independent
 * restatements in integer arithmetic on the FP32 bit pattern, over every one of the
 * 2^32 FP32 inputs (OpenMP over the bit patterns):
 *   BF16   nearest-even of the 32-bit pattern by carry: (b + 0x7FFF + lsb) >> 16;
 *          a NaN must stay a NaN
 *   E4M3   OCP E4M3FN, nearest-even on the significand bits (3 fraction bits, the
 *          subnormal step 2^-9), saturating to 0x7E (448) at and above 448 -- also
 *          for the infinities -- with the sign kept; a NaN gives 0x7F
 *   E2M1   nearest-even over the grid 0, 0.5, 1, 1.5, 2, 3, 4, 6 by counting the
 *          rounding boundaries passed (strict where the tie goes down to the even
 *          code), saturating to 6, the sign kept (a NaN is treated as above 6, the
 *          oracle's documented handling of an input its callers never pass)
 *   E2M1 stochastic  with grid spacing D = 2^d (0.5 / 1 / 2 below 2 / 4 / 6) and
 *          |q| / D = k + f, round up iff floor(256 f) + r >= 256, floor(256 |q| / D)
 *          taken by shifting the significand; one r per input (a hash of the bits),
 *          so that every input and every r value occur
 * These pin the oracle's encoders (binary searches and comparisons in double) to
 * the formats over their whole domain.  Prints the checks and mismatches per
 * encoder; exit status 0 when there are none. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mxq_oracle.h"

static float from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static int is_nan(uint32_t b) { return (b & 0x7FFFFFFFu) > 0x7F800000u; }

static uint32_t ref_bf16(uint32_t b) { return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16; }

static uint32_t ref_e4m3(uint32_t b) {
    const uint32_t sign = (b >> 24) & 0x80u, a = b & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return 0x7Fu;                       /* NaN */
    if (a >= 0x43E00000u) return sign | 0x7Eu;               /* >= 448, infinities too */
    const uint32_t E = a >> 23;
    if (E == 0) return sign;                                 /* FP32 subnormal: far below 2^-10 */
    const uint32_t S = (a & 0x7FFFFFu) | 0x800000u;
    const int e = (int)E - 127;
    uint32_t code;
    if (e >= -6) {
        uint32_t q = S >> 20, rem = S & 0xFFFFFu;
        if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
        int ee = e;
        if (q == 16u) { q = 8u; ++ee; }
        const int field = ee + 7;
        code = (field > 15 || (field == 15 && (q & 7u) == 7u)) ? 0x7Eu : ((uint32_t)field << 3) | (q & 7u);
    } else {
        const int sh = 14 - e;
        if (sh >= 32) {
            code = 0u;
        } else {
            uint32_t q = S >> sh;
            const uint32_t rem = S & ((1u << sh) - 1u), half = 1u << (sh - 1);
            if (rem > half || (rem == half && (q & 1u))) ++q;
            code = q;
        }
    }
    return sign | code;
}

static uint32_t ref_e2m1(uint32_t b) {
    const uint32_t sign = (b >> 28) & 0x8u, a = b & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return sign | 7u;
    const uint32_t c = (a > 0x3E800000u) + (a >= 0x3F400000u) + (a > 0x3FA00000u) + (a >= 0x3FE00000u) +
                       (a > 0x40200000u) + (a >= 0x40600000u) + (a > 0x40A00000u);
    return sign | c;
}

static uint32_t ref_e2m1_sr(uint32_t b, uint32_t r) {
    const uint32_t sign = (b >> 28) & 0x8u, a = b & 0x7FFFFFFFu;
    if (a >= 0x40C00000u) return sign | 7u;                  /* >= 6, infinities and NaN too */
    const int d = a < 0x40000000u ? -1 : (a < 0x40800000u ? 0 : 1);
    const uint32_t E = a >> 23;
    const uint64_t S = E ? ((a & 0x7FFFFFu) | 0x800000u) : (a & 0x7FFFFFu);
    const int e = E ? (int)E - 127 : -126;
    const int sh = 15 + d - e;
    const uint64_t T = sh >= 64 ? 0 : (S >> sh);
    const uint32_t k = (uint32_t)(T >> 8), F = (uint32_t)(T & 255u);
    const uint32_t K = k + (F + r >= 256u ? 1u : 0u);
    return sign | (d < 0 ? K : (d == 0 ? K + 2u : K + 4u));
}

int main(void) {
    long long bad[4] = {0, 0, 0, 0};
    unsigned long long first[4] = {~0ull, ~0ull, ~0ull, ~0ull};
#pragma omp parallel
    {
        long long b0 = 0, b1 = 0, b2 = 0, b3 = 0;
        unsigned long long f0 = ~0ull, f1 = ~0ull, f2 = ~0ull, f3 = ~0ull;
#pragma omp for schedule(static)
        for (long long i = 0; i < (1ll << 32); ++i) {
            const uint32_t b = (uint32_t)i;
            const float v = from_bits(b);
            const uint32_t h = oracle_f32_to_bf16(v);
            if (is_nan(b) ? !is_nan(h << 16) : h != ref_bf16(b)) { ++b0; if (b < f0) f0 = b; }
            if (oracle_e4m3_encode(v) != ref_e4m3(b)) { ++b1; if (b < f1) f1 = b; }
            if (oracle_e2m1_encode(v) != ref_e2m1(b)) { ++b2; if (b < f2) f2 = b; }
            const uint32_t r = (b * 2654435761u) >> 24;       /* one r per input, all r occur */
            if (!is_nan(b) && oracle_e2m1_encode_sr(v, (uint8_t)r) != ref_e2m1_sr(b, r)) { ++b3; if (b < f3) f3 = b; }
        }
#pragma omp critical
        {
            bad[0] += b0; bad[1] += b1; bad[2] += b2; bad[3] += b3;
            if (f0 < first[0]) first[0] = f0;
            if (f1 < first[1]) first[1] = f1;
            if (f2 < first[2]) first[2] = f2;
            if (f3 < first[3]) first[3] = f3;
        }
    }
    const char* names[4] = {"bf16", "e4m3", "e2m1", "e2m1_sr"};
    long long total = 0;
    for (int i = 0; i < 4; ++i) {
        printf("%s: 4294967296 inputs, %lld mismatches", names[i], bad[i]);
        if (bad[i]) printf(" (first input 0x%08llx)", first[i]);
        printf("\n");
        total += bad[i];
    }
    return total ? 1 : 0;
}
