/*
 * CPU check of the quantising kernels' per-row division (row_div and
 * div_fast in combine_ep_plan_02_amd/csrc/ep_row_kernels.h) against IEEE
 * binary32 division, with fmaf standing in for the device's fused
 * multiply-add.
 *
 * For one row scale s the kernel takes r0 = v_rcp_f32(s), specified to 1
 * ulp: r0 is one of the two floats around 1/s (the correctly rounded one or
 * its neighbour on the other side of 1/s).  It refines r0 once,
 *     r = fma(fma(-s, r0, 1), r0, r0),
 * except for a scale whose mantissa is all ones, s = 2^k (2 - 2^-23), where
 * r is set to 2^-k-1 (1 + 2^-23).  It splits 1/s as rd + rl: rd is r or the
 * float below it, whichever is not above 1/s, and rl = fl((1 - s rd) rd).
 * For every numerator n it forms
 *     q0 = fma(n, rd, n * rl);  e = fma(s, q0, -n);  q = fma(-e, r, q0).
 * The fast path is only taken for 2^-60 <= s <= 2^60.
 *
 * Part 1 (every mantissa): for each of the 2^23 mantissas, at exponents
 * 2^-60, 2^0 and 2^59, and both floats around 1/s as r0, r equals the
 * correctly rounded 1/s.
 * Part 2 (quotients): q equals n / s bit for bit whenever |n / s| >= 2^-11;
 * below that the code is a signed zero for both E4M3FN (|v| <= 2^-10 rounds
 * to zero) and int8, so q need only stay within 2^-10 with the sign of n / s.
 * Numerators: for every rounding boundary b of the two codes (each finite
 * E4M3FN value and each midpoint between neighbours, the saturation point
 * 464; each integer and half-integer in [-128, 128]), n = fl(b * s) and its
 * neighbours within NB ulps, both signs; plus uniformly random n with
 * |n / s| <= 464, and +-0.  Scales: powers of two from 2^-60 to 2^60, every
 * all-ones mantissa at 120 exponents, the largest scale below 2^60, and
 * log-uniform draws over [2^-60, 2^60]; both floats around 1/s as r0.
 *
 * Usage: div_fast_check <n_scales> <n_random_per_scale> <seed>
 * Prints one line per part with its counts and, for the first mismatches,
 * the operands.  Exit status 0 when there is no mismatch.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define NB 3

static uint64_t rng_state;

static uint64_t next_u64(void)
{
    /* splitmix64 */
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

static double uniform01(void) { return (double)(next_u64() >> 11) * 0x1p-53; }

static float step_ulps(float x, int k)
{
    while (k > 0) { x = nextafterf(x, INFINITY); --k; }
    while (k < 0) { x = nextafterf(x, -INFINITY); ++k; }
    return x;
}

static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* The kernel's element step.  Each step is stored through a volatile, so the host compiler cannot merge
 * a negation into a neighbouring fma (GCC rewrites -fma(a, b, -c) as
 * fnma(a, b, c), which is not exact for the sign of a zero). */
struct row { float s, r, rd, rl; };

/* The kernel's per-row values: rd is r or the float below it, whichever is
 * not above 1/s, and rl = (1 - s rd) rd >= 0. */
static struct row row_split(float s, float r)
{
    struct row w = {s, r, r, 0.0f};
    volatile float ms = -s;
    volatile float e0 = fmaf(ms, r, 1.0f);
    if (e0 < 0.0f)
        w.rd = from_bits(bits(r) - 1u);
    volatile float e1 = fmaf(ms, w.rd, 1.0f);
    w.rl = e1 * w.rd;
    return w;
}

static float div_fast(float n, const struct row *w)
{
    volatile float lo = n * w->rl;
    volatile float q = fmaf(n, w->rd, lo);
    volatile float m = -n;
    volatile float e = fmaf(w->s, q, m);
    volatile float ne = -e;
    q = fmaf(ne, w->r, q);
    return q;
}


/* The two floats around 1/s: the correctly rounded rn and its neighbour on
 * the other side of 1/s (1 - s rn is exact in one fma; its sign tells the
 * side). */
static void around_recip(float s, float r0[2])
{
    const float rn = 1.0f / s;
    volatile float ms = -s;
    const float e = fmaf(ms, rn, 1.0f);
    r0[0] = rn;
    r0[1] = e > 0.0f ? nextafterf(rn, INFINITY) : nextafterf(rn, -INFINITY);
}

/* The kernel's row reciprocal from r0. */
static float row_recip(float s, float r0)
{
    volatile float ms = -s;
    volatile float d = fmaf(ms, r0, 1.0f);
    float r = fmaf(d, r0, r0);
    const uint32_t sb = bits(s);
    if ((sb & 0x7fffffu) == 0x7fffffu)
        r = from_bits(((253u - ((sb >> 23) & 0xffu)) << 23) | 1u);
    return r;
}

static long long n_pairs, n_bad;

static void check(float n, const struct row *w, float r0)
{
    const float s = w->s, r = w->r;
    const float want = n / s;
    const float got = div_fast(n, w);
    ++n_pairs;
    int ok;
    if (fabsf(want) >= 0x1p-11f)
        ok = bits(got) == bits(want);
    else
        ok = fabsf(got) <= 0x1p-10f && signbit(got) == signbit(want);
    if (!ok) {
        if (n_bad < 10)
            printf("mismatch: n %a s %a r0 %a r %a got %a want %a\n", n, s, r0, r, got, want);
        ++n_bad;
    }
}

/* Every rounding boundary of E4M3FN (values and midpoints, positive) and of
 * the int8 code (integers and half-integers); returns the count. */
static int boundaries(float *b)
{
    int m = 0;
    float vals[128];
    int nv = 0;
    for (int c = 0; c < 0x7f; ++c) { /* 0x7f is NaN */
        const int e = c >> 3, f = c & 7;
        vals[nv++] = e == 0 ? ldexpf((float)f, -9) : ldexpf(1.0f + f / 8.0f, e - 7);
    }
    for (int i = 0; i < nv; ++i) {
        b[m++] = vals[i];
        if (i + 1 < nv)
            b[m++] = 0.5f * (vals[i] + vals[i + 1]);
    }
    b[m++] = 464.0f;
    for (int k = 0; k <= 256; ++k)
        b[m++] = 0.5f * (float)k;
    return m;
}

int main(int argc, char **argv)
{
    const int n_scales = argc > 1 ? atoi(argv[1]) : 2000;
    const int n_random = argc > 2 ? atoi(argv[2]) : 1000;
    rng_state = argc > 3 ? strtoull(argv[3], NULL, 10) : 1;

    /* Part 1: the row reciprocal over every mantissa. */
    long long n_recip = 0, bad_recip = 0;
    const int exps[3] = {-60, 0, 59};
    for (int ei = 0; ei < 3; ++ei) {
        for (uint32_t m = 0; m < (1u << 23); ++m) {
            const float s = ldexpf(from_bits(0x3f800000u | m), exps[ei]);
            const float rn = 1.0f / s;
            float around[2];
            around_recip(s, around);
            for (int k = 0; k < 2; ++k) {
                const float r0 = around[k];
                const float r = row_recip(s, r0);
                ++n_recip;
                if (bits(r) != bits(rn)) {
                    if (bad_recip < 10)
                        printf("reciprocal mismatch: s %a r0 %a r %a want %a\n", s, r0, r, rn);
                    ++bad_recip;
                }
            }
        }
    }
    printf("reciprocals %lld mismatches %lld\n", n_recip, bad_recip);

    /* Part 2: quotients. */
    float bnd[1024];
    const int nb = boundaries(bnd);
    const int n_fixed = 121 + 120 + 1;
    for (int i = 0; i < n_fixed + n_scales; ++i) {
        float s;
        if (i < 121)
            s = ldexpf(1.0f, i - 60);                       /* powers of two */
        else if (i < 241)
            s = ldexpf(from_bits(0x3fffffffu), i - 121 - 60); /* all-ones mantissas */
        else if (i == 241)
            s = step_ulps(0x1p60f, -1);
        else
            s = (float)exp2(-60.0 + 120.0 * uniform01());
        if (s < 0x1p-60f || s > 0x1p60f)
            continue;
        float around[2];
        around_recip(s, around);
        for (int k = 0; k < 2; ++k) {
            const float r0 = around[k];
            const struct row w = row_split(s, row_recip(s, r0));
            for (int j = 0; j < nb; ++j) {
                const float n0 = bnd[j] * s;
                for (int u = -NB; u <= NB; ++u) {
                    const float n = step_ulps(n0, u);
                    check(n, &w, r0);
                    check(-n, &w, r0);
                }
            }
            for (int j = 0; j < n_random; ++j) {
                const float n = (float)((2.0 * uniform01() - 1.0) * 464.0) * s;
                check(n, &w, r0);
            }
            check(0.0f, &w, r0);
            check(-0.0f, &w, r0);
        }
    }
    printf("quotients %lld mismatches %lld\n", n_pairs, n_bad);
    return bad_recip == 0 && n_bad == 0 ? 0 : 1;
}
