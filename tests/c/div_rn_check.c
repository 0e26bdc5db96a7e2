/* div_rn_check.c -- the exactness arguments behind the quantizers' divisions and
 * scale tables, checked on the CPU in IEEE binary32 (fmaf is a fused multiply-add
 * with one rounding, as the GPU's v_fma_f32).
 *
 * 1. Markstein's correction step.  Given y = fl(1/d):
 *        q0 = fl(x * y),  r = fma(q0, d, -x) (exact),  q = fma(-r, y, q0)
 *    and the claim is q == fl(x / d).  Division commutes with scaling by powers of
 *    two while every value stays normal, so the pairs are significands in [1, 2):
 *      bf16   every BF16 significand x against every FP32 significand d (2^30
 *             pairs): the numerators of the FP8 and NVFP4 element divisions;
 *      sixth  every x = fl(a * F(1/6)) for a BF16 significand a against every d
 *             (2^30 pairs): the NVFP4 block-scale numerators;
 *      general arbitrary FP32 numerators (the SwiGLU path divides fl(SiLU(g) * up)):
 *             N random pairs, and N pairs whose exact quotient lies next to a
 *             rounding midpoint (x = fl(m * d) and its neighbours for a midpoint m
 *             between two FP32 values), the inputs that separate a correctly
 *             rounded division from a nearly correct one.
 * 2. Product multipliers (the NVFP4 scale tables).  For a tensor scale g and each
 *    E4M3 scale code c, d = fl(E4M3(c) * g) (times 4 for the column direction, whose
 *    values enter unscaled) and y = fl(1/d); the candidates y, y - 1 ulp, y + 1 ulp are
 *    tried against the two BF16 neighbours of each E2M1 rounding boundary times d
 *    (14 values) and the first that agrees with the exact division there is taken.
 *    The claim: a multiplier so chosen gives E2M1(fl(u * ym)) == E2M1(fl(u / d)) for
 *    EVERY BF16 u -- checked here by brute force over all 32,768 non-negative finite
 *    BF16 values, for a set of tensor scales (random maxima over 2^-40 .. 2^40,
 *    maxima carrying the factors 3 and 7 of 2688, BF16 extremes, the 1e-10 floor).
 *
 * 3. Stochastic multipliers (the same tables when a direction rounds stochastically).
 *    The stochastic E2M1 rule reads, of q = fl(u / d), the grid spacing D (0.5, 1, 2
 *    below 2, 4, 6) and floor(256 |q| / D), or only that |q| >= 6.  For each
 *    representative divisor (1 + m/8) g (times 4 for columns) the first of the
 *    candidates y, y - 1 ulp, y + 1 ulp for which fl(u * ym) and fl(u / d) agree in
 *    every bit above the 14th for the 128 BF16 significands u = 1 + k/128 is taken; an
 *    entry takes its representative's scaled by 2^-e when its own d and fl(1/d) are
 *    the representative's scaled exactly and g < 2^100, else none.  The claim: for
 *    every entry with a multiplier, fl(u * ym) and fl(u / d) have the same D and
 *    floor(256 |q| / D) (or both saturate) for EVERY BF16 u, by brute force.
 *
 * Usage: div_rn_check bf16 | sixth | general N SEED | tables N SEED | srtables N SEED
 * Prints the number of checks and mismatches; exit status 0 when there are none. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t to_bits(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

static float div_markstein(float x, float d, float y) {
    volatile float q0 = x * y;                /* volatile: a rounded product, never fused */
    const float r = fmaf(q0, d, -x);
    return fmaf(-r, y, q0);
}

/* splitmix64 (Steele, Lea, Flood): test inputs only */
static uint64_t sm_next(uint64_t* s) {
    uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static long long mismatches = 0, checks = 0;

static void report_pair(float x, float d, float got, float want) {
    if (mismatches < 8)
        fprintf(stderr, "mismatch: x=%a d=%a markstein=%a ieee=%a\n", (double)x, (double)d, (double)got,
                (double)want);
}

/* every d significand against the numerator significands xs[0..nx) */
static void sweep_all_d(const float* xs, int nx) {
    long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (int64_t m = 0; m < (1 << 23); ++m) {
        const float d = from_bits(0x3F800000u | (uint32_t)m);
        const float y = 1.0f / d;
        for (int i = 0; i < nx; ++i) {
            const float got = div_markstein(xs[i], d, y), want = xs[i] / d;
            if (to_bits(got) != to_bits(want)) {
                ++bad;
#pragma omp critical
                report_pair(xs[i], d, got, want);
            }
        }
    }
    mismatches += bad;
    checks += (long long)nx << 23;
}

static void mode_general(long long n, uint64_t seed) {
    long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (long long i = 0; i < n; ++i) {
        uint64_t s = seed ^ ((uint64_t)i * 0xD1B54A32D192ED03ull);
        const uint64_t a = sm_next(&s), b = sm_next(&s);
        const float d = from_bits(0x3F800000u | (uint32_t)(b & 0x7FFFFF));
        const float y = 1.0f / d;
        /* a random numerator significand, and one next to a quotient midpoint */
        float xs[6];
        xs[0] = from_bits(0x3F800000u | (uint32_t)(a & 0x7FFFFF));
        const double q = (double)from_bits(0x3F800000u | (uint32_t)((a >> 23) & 0x7FFFFF));
        const double mid = q + ldexp(1.0, -24);                  /* between q and q + ulp (exact in double) */
        const float xm = (float)(mid * (double)d);               /* fl(mid * d): the product is exact in double */
        const uint32_t xb = to_bits(xm);
        xs[1] = xm;
        xs[2] = from_bits(xb - 1);
        xs[3] = from_bits(xb + 1);
        xs[4] = from_bits(xb - 2);
        xs[5] = from_bits(xb + 2);
        for (int j = 0; j < 6; ++j) {
            const float got = div_markstein(xs[j], d, y), want = xs[j] / d;
            if (to_bits(got) != to_bits(want)) {
                ++bad;
#pragma omp critical
                report_pair(xs[j], d, got, want);
            }
        }
    }
    mismatches += bad;
    checks += 6 * n;
}

/* ---------------------------------------------------------------- tables */
static float e4m3_value(int c) {                               /* c in 1..126 */
    const int e = (c >> 3) & 15, m = c & 7;
    return e == 0 ? ldexpf((float)m / 8.0f, -6) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
}

/* E2M1 code (magnitude index 0..7) of a non-negative, non-NaN v: nearest, ties to
 * the even code, saturating at 6. */
static int e2m1(float v) {
    static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    if (!(v < 6.0f)) return 7;
    int lo = 0;
    for (int c = 1; c < 8; ++c)
        if (mag[c] <= v) lo = c;
    if (mag[lo] == v) return lo;
    const float s = mag[lo] + mag[lo + 1], t = 2.0f * v;      /* exact */
    if (t < s) return lo;
    if (t > s) return lo + 1;
    return (lo & 1) ? lo + 1 : lo;
}

/* The multiplier search as the tables state it; -1 when no candidate agrees. */
static float find_multiplier(float d, float y) {
    static const float taus[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
    float us[14];
    int exact[14];
    for (int i = 0; i < 7; ++i) {
        const uint32_t lo = to_bits(taus[i] * d) & 0xFFFF0000u;
        us[2 * i] = from_bits(lo);
        us[2 * i + 1] = from_bits(lo + 0x10000u);
        exact[2 * i] = e2m1(us[2 * i] / d);
        exact[2 * i + 1] = e2m1(us[2 * i + 1] / d);
    }
    static const int deltas[3] = {0, -1, 1};
    for (int c = 0; c < 3; ++c) {
        const float ym = from_bits(to_bits(y) + (uint32_t)deltas[c]);
        int ok = 1;
        for (int j = 0; j < 14; ++j) ok &= e2m1(us[j] * ym) == exact[j];
        if (ok) return ym;
    }
    return -1.0f;
}

static void mode_tables(int n, uint64_t seed) {
    /* the tensor scales: g = fl(max(A, F(1e-10)) * F(1/2688)) */
    float* A = malloc(sizeof(float) * (size_t)(n + 64));
    int na = 0;
    const float fixed[] = {0.0f, 1e-10f, 1.0f, 3.0f, 7.0f, 21.0f, 2688.0f, 6.0f, 448.0f, 0.75f, 1.5f,
                           from_bits(0x7F7F0000u), from_bits(0x00800000u), 3.0f * 1024.0f, 7.0f / 1024.0f,
                           from_bits(0x40400000u | 0x10000u), 12.0f, 1e30f, 1e-30f};
    for (size_t i = 0; i < sizeof fixed / sizeof fixed[0]; ++i) A[na++] = fixed[i];
    uint64_t s = seed;
    while (na < n) {
        const uint64_t r = sm_next(&s);
        /* a BF16 maximum (the row-wise amax is a BF16 value) over 2^-40 .. 2^40 */
        const int e = (int)(r % 81) - 40;
        const uint32_t sig = (uint32_t)((r >> 8) & 0x7F) << 16;
        A[na++] = from_bits(((uint32_t)(e + 127) << 23) | sig);
    }
    const float floor_ = from_bits(0x2EDBE6FFu), inv2688 = from_bits(0x39C30C31u);
    long long bad = 0, found = 0, none = 0;
#pragma omp parallel for reduction(+ : bad, found, none) schedule(dynamic)
    for (int i = 0; i < na; ++i) {
        const float g = fmaxf(A[i], floor_) * inv2688;
        for (int dir = 0; dir < 2; ++dir) {
            for (int c = 1; c < 127; ++c) {
                float d = e4m3_value(c) * g, y = 1.0f / d;
                if (dir) { d *= 4.0f; y *= 0.25f; }
                const float ym = find_multiplier(d, y);
                if (ym < 0.0f) { ++none; continue; }
                ++found;
                for (uint32_t u16 = 0; u16 < 0x7F80u; ++u16) {
                    const float u = from_bits(u16 << 16);
                    if (e2m1(u * ym) != e2m1(u / d)) {
                        ++bad;
#pragma omp critical
                        if (bad < 8) fprintf(stderr, "table mismatch: A=%a dir=%d code=%d u=%a\n", (double)A[i],
                                             dir, c, (double)u);
                    }
                }
            }
        }
    }
    mismatches += bad;
    checks += found * 0x7F80ll;
    printf("tables: %d tensor scales, %lld entries with a multiplier, %lld without\n", na, found, none);
    free(A);
}

/* ---------------------------------------------------------------- stochastic tables */
/* What the stochastic rule reads of a non-NaN quotient q: -1 when |q| >= 6, else
 * floor(256 |q| / D) + 4096 * (index of D), computed in double from the rule's own
 * terms (|q| / D = k + f; 256 k + floor(256 f)). */
static long sr_cell(float q) {
    const double a = fabs((double)q);
    if (!(a < 6.0)) return -1;
    const int di = a < 2.0 ? 0 : (a < 4.0 ? 1 : 2);
    const double D = di == 0 ? 0.5 : (di == 1 ? 1.0 : 2.0);
    return (long)floor(a / D * 256.0) + 4096L * di;
}

/* The stochastic multiplier search as the tables state it: the first candidate for
 * which fl(u * ym) and fl(u / d) agree above bit 14 for every u = 1 + k/128; -1 when
 * none does. */
static float find_sr_multiplier(float d, float y) {
    const float ym[3] = {y, from_bits(to_bits(y) - 1u), from_bits(to_bits(y) + 1u)};
    for (int c = 0; c < 3; ++c) {
        int ok = 1;
        for (int k = 0; k < 128; ++k) {
            const float u = 1.0f + (float)k / 128.0f;
            ok &= (to_bits(u * ym[c]) >> 14) == (to_bits(u / d) >> 14);
        }
        if (ok) return ym[c];
    }
    return -1.0f;
}

static void mode_srtables(int n, uint64_t seed) {
    float* A = malloc(sizeof(float) * (size_t)(n + 64));
    int na = 0;
    const float fixed[] = {0.0f, 1e-10f, 1.0f, 3.0f, 7.0f, 21.0f, 2688.0f, 6.0f, 448.0f, 0.75f, 1.5f,
                           from_bits(0x7F7F0000u), from_bits(0x00800000u), 3.0f * 1024.0f, 7.0f / 1024.0f,
                           from_bits(0x40400000u | 0x10000u), 12.0f, 1e30f, 1e-30f};
    for (size_t i = 0; i < sizeof fixed / sizeof fixed[0]; ++i) A[na++] = fixed[i];
    uint64_t s = seed;
    while (na < n) {
        const uint64_t r = sm_next(&s);
        const int e = (int)(r % 81) - 40;
        const uint32_t sig = (uint32_t)((r >> 8) & 0x7F) << 16;
        A[na++] = from_bits(((uint32_t)(e + 127) << 23) | sig);
    }
    const float floor_ = from_bits(0x2EDBE6FFu), inv2688 = from_bits(0x39C30C31u);
    long long bad = 0, found = 0, none = 0;
#pragma omp parallel for reduction(+ : bad, found, none) schedule(dynamic)
    for (int i = 0; i < na; ++i) {
        const float g = fmaxf(A[i], floor_) * inv2688;
        for (int dir = 0; dir < 2; ++dir) {
            float cls[8];
            for (int m = 0; m < 8; ++m) {
                float d = (1.0f + (float)m * 0.125f) * g, y = 1.0f / d;
                if (dir) { d *= 4.0f; y *= 0.25f; }
                cls[m] = find_sr_multiplier(d, y);
            }
            for (int c = 1; c < 127; ++c) {
                const float v = e4m3_value(c);
                const uint32_t vb = to_bits(v);
                const int m = (int)((vb >> 20) & 7), ex = (int)((vb >> 23) & 0xFF) - 127;
                float d = v * g, y = 1.0f / d;
                float rd = (1.0f + (float)m * 0.125f) * g, ry = 1.0f / rd;
                if (dir) { d *= 4.0f; y *= 0.25f; rd *= 4.0f; ry *= 0.25f; }
                const int scaled = g < 0x1p100f && d == ldexpf(rd, ex) && y == ldexpf(ry, -ex);
                if (!scaled || cls[m] < 0.0f) { ++none; continue; }
                const float ym = ldexpf(cls[m], -ex);
                ++found;
                for (uint32_t u16 = 0; u16 < 0x7F80u; ++u16) {
                    const float u = from_bits(u16 << 16);
                    if (sr_cell(u * ym) != sr_cell(u / d)) {
                        ++bad;
#pragma omp critical
                        if (bad < 8) fprintf(stderr, "sr table mismatch: A=%a dir=%d code=%d u=%a\n", (double)A[i],
                                             dir, c, (double)u);
                    }
                }
            }
        }
    }
    mismatches += bad;
    checks += found * 0x7F80ll;
    printf("srtables: %d tensor scales, %lld entries with a multiplier, %lld without\n", na, found, none);
    free(A);
}

int main(int argc, char** argv) {
    if (argc < 2) {
        fprintf(stderr, "usage: %s bf16 | sixth | general N SEED | tables N SEED | srtables N SEED\n", argv[0]);
        return 2;
    }
    if (!strcmp(argv[1], "bf16")) {
        float xs[128];
        for (int i = 0; i < 128; ++i) xs[i] = from_bits(0x3F800000u | ((uint32_t)i << 16));
        sweep_all_d(xs, 128);
    } else if (!strcmp(argv[1], "sixth")) {
        float xs[256];
        int n = 0;
        const float inv6 = from_bits(0x3E2AAAABu);
        /* a in [1, 2) and [2, 4): fl(a / 6) lands in two binades, so both are swept */
        for (int e = 0; e < 2; ++e)
            for (int i = 0; i < 128; ++i) {
                const float a = from_bits(((uint32_t)(127 + e) << 23) | ((uint32_t)i << 16));
                const float v = a * inv6;
                /* the significand of fl(a / 6), scaled to [1, 2) */
                xs[n++] = from_bits(0x3F800000u | (to_bits(v) & 0x7FFFFFu));
            }
        sweep_all_d(xs, n);
    } else if (!strcmp(argv[1], "general") && argc >= 4) {
        mode_general(atoll(argv[2]), strtoull(argv[3], NULL, 0));
    } else if (!strcmp(argv[1], "tables") && argc >= 4) {
        mode_tables(atoi(argv[2]), strtoull(argv[3], NULL, 0));
    } else if (!strcmp(argv[1], "srtables") && argc >= 4) {
        mode_srtables(atoi(argv[2]), strtoull(argv[3], NULL, 0));
    } else {
        fprintf(stderr, "unknown mode\n");
        return 2;
    }
    printf("%s: %lld checks, %lld mismatches\n", argv[1], checks, mismatches);
    return mismatches ? 1 : 0;
}
