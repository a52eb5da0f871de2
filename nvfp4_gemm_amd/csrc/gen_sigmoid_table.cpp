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
// Usage: gen_sigmoid_table OUT.inc   (65536 comma-separated uint32 bit patterns)
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

int main(int argc, char **argv) {
    if (argc != 2) {
        std::fprintf(stderr, "usage: %s OUT.inc\n", argv[0]);
        return 2;
    }
    std::FILE *f = std::fopen(argv[1], "w");
    if (!f) return 1;
    for (uint32_t b = 0; b < 65536u; ++b) {
        const float g = bits_to_float(b << 16);
        const float s = std::isfinite(g) ? sigmoid_times_input(g) : 0.0f;
        std::fprintf(f, "0x%08xu,%s", float_to_bits(s), (b % 8 == 7) ? "\n" : "");
    }
    return std::fclose(f) == 0 ? 0 : 1;
}
