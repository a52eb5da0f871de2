// gen_sigmoid_table.cpp -- build-time generator of the SiLU kernel's table of
// sigma32(g) = the correctly rounded binary32 value of g / (1 + exp(-g)), for
// all 65536 BF16 bit patterns g (simolm.com PACT blog, section "Method",
// second bullet: the SiLU-multiply forward reads BF16 inputs).
//
// Outside 2^-25 <= |g| < 2^-6 a binary64 evaluation (relative error about
// 2^-52) is far closer than any BF16 input's distance to a binary32 rounding
// midpoint (at least 2^-37 there), so one final rounding gives the correct
// result.  Inside that range g/2 + g^2/4 can sit exactly on a midpoint while
// the true value differs from it by about g^4/48: the value is formed as the
// exact binary64 sum hi = g/2 + g^2/4 plus the series tail
// g^4 (-1/48 + g^2/480 - 17 g^4/80640 + 31 g^6/1451520), and an exact tie is
// broken by the sign of the tail.
//
// Only 8192 of the 65536 values need a table.  For a BF16 bit pattern b with
// biased exponent field e:
//   e <  102 (|g| < 2^-25, zeros and subnormals included): sigma32 = g * 0.5
//            (g/2 is exact in binary32 and g^2/4 is below half an ulp of it);
//   e >= 134 (|g| >= 2^7), g > 0: sigma32 = g (exp(-g) < 2^-184);
//   e >= 134, g < 0: sigma32 = -0 (|g| e^g < 2^-149);
//   e == 255 (Inf, NaN): 0 (the library defines no value for them);
//   102 <= e < 134: entry ((b >> 15) << 12) | ((e - 102) << 7) | (b & 127).
// The program checks this rule against the full evaluation for every pattern
// and fails (exit status 1) on any difference.
//
// Usage: gen_sigmoid_table OUT.inc   (8192 comma-separated uint32 bit patterns)
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

static uint32_t full_value(uint32_t b) {
    const float g = bits_to_float(b << 16);
    return float_to_bits(std::isfinite(g) ? sigmoid_times_input(g) : 0.0f);
}

// The rule of the header comment, given the compact table.
static uint32_t by_rule(uint32_t b, const uint32_t *compact) {
    const uint32_t e = (b >> 7) & 0xFFu;
    const float g = bits_to_float(b << 16);
    if (e < 102u) return float_to_bits(g * 0.5f);
    if (e < 134u) return compact[((b >> 15) << 12) | ((e - 102u) << 7) | (b & 127u)];
    if (e == 255u) return 0u;
    return (b & 0x8000u) ? 0x80000000u : float_to_bits(g);
}

int main(int argc, char **argv) {
    if (argc != 2) {
        std::fprintf(stderr, "usage: %s OUT.inc\n", argv[0]);
        return 2;
    }
    static uint32_t compact[8192];
    for (uint32_t i = 0; i < 8192u; ++i) {
        const uint32_t sign = i >> 12, e = 102u + ((i >> 7) & 31u), m = i & 127u;
        compact[i] = full_value((sign << 15) | (e << 7) | m);
    }
    for (uint32_t b = 0; b < 65536u; ++b) {
        if (by_rule(b, compact) != full_value(b)) {
            std::fprintf(stderr, "rule differs from the full evaluation at BF16 pattern 0x%04x\n", b);
            return 1;
        }
    }
    std::FILE *f = std::fopen(argv[1], "w");
    if (!f) return 1;
    for (uint32_t i = 0; i < 8192u; ++i)
        std::fprintf(f, "0x%08xu,%s", compact[i], (i % 8 == 7) ? "\n" : "");
    return std::fclose(f) == 0 ? 0 : 1;
}
