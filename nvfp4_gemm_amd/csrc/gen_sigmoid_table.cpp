// gen_sigmoid_table.cpp -- build-time generator of the tables the SiLU
// kernels read (simolm.com PACT blog, section "Method", second bullet: the
// SiLU-multiply forward reads BF16 inputs and keeps an NVFP4 copy of gate/up
// for backward):
//   sigma32(g) = the correctly rounded binary32 value of g / (1 + exp(-g)),
//   dsilu32(g) = the correctly rounded binary32 value of the derivative
//                sigma(g) (1 + g (1 - sigma(g))),
// for the BF16 bit patterns g.
//
// sigma32: outside 2^-25 <= |g| < 2^-6 a binary64 evaluation (relative error
// about 2^-52) is far closer than any BF16 input's distance to a binary32
// rounding midpoint (at least 2^-37 there), so one final rounding gives the
// correct result.  Inside that range g/2 + g^2/4 can sit exactly on a midpoint
// while the true value differs from it by about g^4/48: the value is formed as
// the exact binary64 sum hi = g/2 + g^2/4 plus the series tail
// g^4 (-1/48 + g^2/480 - 17 g^4/80640 + 31 g^6/1451520), and an exact tie is
// broken by the sign of the tail.
//
// dsilu32: for |g| < 2^-6 the series 1/2 + g/2 - g^3/12 + g^5/80 -
// 17 g^7/10080 + 31 g^9/145152 (the derivative of the one above), with the
// exact binary64 head 1/2 + g/2 and the same tie rule; elsewhere an x87
// extended-precision evaluation (64-bit significand).  Every non-tie decision
// of either table must clear its midpoint by a margin well above the
// evaluation error, or the program fails.
//
// Only 8192 values of each need a table.  For a BF16 bit pattern b with
// biased exponent field e:
//   e <  102 (|g| < 2^-25, zeros and subnormals included): sigma32 = g * 0.5
//            (g/2 is exact in binary32 and g^2/4 is below half an ulp of it),
//            dsilu32 = 0.5;
//   e >= 134 (|g| >= 2^7), g > 0: sigma32 = g (exp(-g) < 2^-184), dsilu32 = 1;
//   e >= 134, g < 0: sigma32 = -0 (|g| e^g < 2^-149), dsilu32 = -0;
//   e == 255 (Inf, NaN): 0 (the library defines no value for them);
//   102 <= e < 134: entry ((b >> 15) << 12) | ((e - 102) << 7) | (b & 127).
// The program checks these rules against the full evaluation for every
// pattern and fails (exit status 1) on any difference.
//
// Usage: gen_sigmoid_table SIGMA.inc DSILU.inc   (8192 comma-separated uint32
// bit patterns each)
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

static float bits_to_float(uint32_t b) {
    float f;
    std::memcpy(&f, &b, 4);
    return f;
}

static uint32_t float_to_bits(float f) {
    uint32_t b;
    std::memcpy(&b, &f, 4);
    return b;
}

static float next_up(float r) {
    const uint32_t b = float_to_bits(r);
    return r >= 0.0f ? bits_to_float(b + 1u) : bits_to_float(b - 1u);
}

static float sigmoid_times_input(float gf) {
    const float ag = std::fabs(gf);
    const double g = (double)gf;
    if (ag >= 0x1p-25f && ag < 0x1p-6f) {
        const double hi = 0.5 * g + 0.25 * (g * g);
        const double g2 = g * g;
        const double corr =
            (g2 * g2) * (-1.0 / 48.0 + g2 * (1.0 / 480.0 + g2 * (-17.0 / 80640.0 + g2 * (31.0 / 1451520.0))));
        const double s = hi + corr;
        float r = (float)s;
        const double rd = (double)r;
        if (rd != s) {
            const float lo = rd < s ? r : -next_up(-r);
            const float up = rd < s ? next_up(r) : r;
            const double mid = 0.5 * ((double)lo + (double)up);
            if (s == mid) {
                const double delta = (hi - mid) + corr;
                if (delta > 0.0) r = up;
                else if (delta < 0.0) r = lo;
            }
        }
        return r;
    }
    const double e = std::exp(-g);
    return (float)(g / (1.0 + e));
}

static int g_fail = 0;

// The binary32 rounding of hi + tail (hi exact, tail the series tail): the
// two binary32 neighbours around s = hi + tail and their midpoint are found
// from s; the side is taken from (hi - mid) + tail, where hi - mid is exact
// (the two are within a factor of two), so the decision does not depend on
// s itself being on the right side of the midpoint.  The program fails when
// the decision is not clear of the tail's own evaluation error.
static float round_decided(double hi, double tail) {
    const double s = hi + tail;
    const float r = (float)s;
    if ((double)r == s) {
        // s is a binary32 value; the true value is within a few binary64 ulps
        // of it, far from the midpoints half a binary32 ulp away
        return r;
    }
    const float lo = (double)r < s ? r : -next_up(-r);
    const float up = (double)r < s ? next_up(r) : r;
    const double mid = 0.5 * ((double)lo + (double)up);
    const double delta = (hi - mid) + tail;
    if (std::fabs(delta) <= 0x1p-40 * std::fabs(tail) + 0x1p-200) g_fail = 1;
    return delta > 0.0 ? up : lo;
}

static float dsilu_value(float gf) {
    const double g = (double)gf;
    if (std::fabs(gf) < 0x1p-6f) {
        const double hi = 0.5 + 0.5 * g;  // exact for |g| >= 2^-25 (the only inputs that need it)
        const double g2 = g * g;
        const double tail = (g2 * g) * (-1.0 / 12.0 + g2 * (1.0 / 80.0 + g2 * (-17.0 / 10080.0 + g2 * (31.0 / 145152.0))));
        return round_decided(hi, tail);
    }
    const long double x = (long double)gf;
    const long double sg = 1.0L / (1.0L + expl(-x));
    const long double v = sg * (1.0L + x * (1.0L - sg));
    const float r = (float)v;
    if ((long double)r != v) {
        const float nb = ((long double)r < v) ? next_up(r) : -next_up(-r);
        const long double mid = ((long double)r + (long double)nb) / 2.0L;
        if (fabsl(v - mid) <= 0x1p-56L * fabsl(v)) g_fail = 1;
    }
    return r;
}

static uint32_t full_value(uint32_t b) {
    const float g = bits_to_float(b << 16);
    return float_to_bits(std::isfinite(g) ? sigmoid_times_input(g) : 0.0f);
}

static uint32_t full_dsilu(uint32_t b) {
    const float g = bits_to_float(b << 16);
    return float_to_bits(std::isfinite(g) ? dsilu_value(g) : 0.0f);
}

// The rules of the header comment, given the compact tables.
static uint32_t by_rule(uint32_t b, const uint32_t *compact) {
    const uint32_t e = (b >> 7) & 0xFFu;
    const float g = bits_to_float(b << 16);
    if (e < 102u) return float_to_bits(g * 0.5f);
    if (e < 134u) return compact[((b >> 15) << 12) | ((e - 102u) << 7) | (b & 127u)];
    if (e == 255u) return 0u;
    return (b & 0x8000u) ? 0x80000000u : float_to_bits(g);
}

static uint32_t by_rule_dsilu(uint32_t b, const uint32_t *compact) {
    const uint32_t e = (b >> 7) & 0xFFu;
    if (e < 102u) return float_to_bits(0.5f);
    if (e < 134u) return compact[((b >> 15) << 12) | ((e - 102u) << 7) | (b & 127u)];
    if (e == 255u) return 0u;
    return (b & 0x8000u) ? 0x80000000u : float_to_bits(1.0f);
}

static int write_table(const char *path, const uint32_t *t) {
    std::FILE *f = std::fopen(path, "w");
    if (!f) return 1;
    for (uint32_t i = 0; i < 8192u; ++i)
        std::fprintf(f, "0x%08xu,%s", t[i], (i % 8 == 7) ? "\n" : "");
    return std::fclose(f) == 0 ? 0 : 1;
}

int main(int argc, char **argv) {
    if (argc != 3) {
        std::fprintf(stderr, "usage: %s SIGMA.inc DSILU.inc\n", argv[0]);
        return 2;
    }
    static uint32_t compact[8192], compact_d[8192];
    for (uint32_t i = 0; i < 8192u; ++i) {
        const uint32_t sign = i >> 12, e = 102u + ((i >> 7) & 31u), m = i & 127u;
        compact[i] = full_value((sign << 15) | (e << 7) | m);
        compact_d[i] = full_dsilu((sign << 15) | (e << 7) | m);
    }
    for (uint32_t b = 0; b < 65536u; ++b) {
        if (by_rule(b, compact) != full_value(b)) {
            std::fprintf(stderr, "sigma32 rule differs from the full evaluation at BF16 pattern 0x%04x\n", b);
            return 1;
        }
        if (by_rule_dsilu(b, compact_d) != full_dsilu(b)) {
            std::fprintf(stderr, "dsilu32 rule differs from the full evaluation at BF16 pattern 0x%04x\n", b);
            return 1;
        }
    }
    if (g_fail) {
        std::fprintf(stderr, "an input lies too close to a binary32 rounding midpoint for the evaluation used\n");
        return 1;
    }
    return write_table(argv[1], compact) | write_table(argv[2], compact_d);
}
