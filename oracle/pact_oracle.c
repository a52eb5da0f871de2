/*
 * pact_oracle.c -- plain, slow CPU oracle (TEST INFRASTRUCTURE ONLY; see the
 * header).  Every function is written for obviousness, not speed: roundings to
 * a small value set are done by scanning that set, sums run in index order.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -fPIC -shared (no fast-math).
 */
#include "pact_oracle.h"

#include <assert.h>
#include <math.h>
#include <quadmath.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------- */
/* BF16 <-> FP32                                                              */
/* ------------------------------------------------------------------------- */
float orc_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round-to-nearest-even onto the BF16 grid: keep the top 16 bits, and round
 * up when the dropped 16 bits exceed half, or equal half with an odd kept LSB.
 * Finite inputs only (the data flow never produces Inf/NaN). */
uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
    return (uint16_t)kept;
}

/* ------------------------------------------------------------------------- */
/* E2M1 and E4M3 ([blog] FAQ: 16 E2M1 elements share one E4M3 block scale)    */
/* ------------------------------------------------------------------------- */
/* E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa; exponent 0 is
 * subnormal (0 or 0.5).  No Inf/NaN. */
float orc_e2m1_value(uint8_t code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    float mag = (e == 0) ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
    return s ? -mag : mag;
}

/* E4M3 (OCP "FN" variant): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0
 * mantissa; exponent 0 is subnormal; 0x7F/0xFF are NaN; no Inf; max 448. */
float orc_e4m3_value(uint8_t b) {
    int s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7) return NAN;
    float mag = (e == 0) ? ldexpf((float)m / 8.0f, -6) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return s ? -mag : mag;
}

/* Nearest element of an ascending value table, ties to the even index (for
 * both formats the index LSB is the mantissa LSB, so this is IEEE
 * round-to-nearest-even onto the format); values past the top saturate. */
static int nearest_even_index(double t, const double *vals, int n) {
    if (t >= vals[n - 1]) return n - 1;
    int lo = 0;
    for (int i = 0; i < n; ++i)
        if (vals[i] <= t) lo = i;
    if (vals[lo] == t) return lo;
    int hi = lo + 1;
    double dlo = t - vals[lo], dhi = vals[hi] - t; /* exact: operands are close */
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo % 2 == 0) ? lo : hi;
}

uint8_t orc_e2m1_encode_mag(float r) {
    static const double mags[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    assert(r >= 0.0f);
    return (uint8_t)nearest_even_index((double)r, mags, 8);
}

static double g_e4m3_vals[127]; /* the 127 finite non-negative E4M3 values, ascending */

__attribute__((constructor)) static void init_e4m3_vals(void) {
    for (int b = 0; b < 127; ++b) g_e4m3_vals[b] = (double)orc_e4m3_value((uint8_t)b);
}

uint8_t orc_e4m3_encode(float t) {
    assert(t >= 0.0f);
    return (uint8_t)nearest_even_index((double)t, g_e4m3_vals, 127);
}

/* ------------------------------------------------------------------------- */
/* Row quantizer Q                                                            */
/* Reading of the pages (silent on everything past "16 E2M1 + one E4M3"):     */
/*  - a second-level FP32 scale per row, d = amax_row / (6*448), so the row's */
/*    largest block takes the largest E4M3 scale;                              */
/*  - block scale = E4M3 round-to-nearest-even of amax_block / (6 d), clamped */
/*    to 448;                                                                  */
/*  - element code = E2M1 round-to-nearest-even of |x| / (scale * d), clamped */
/*    to 6, sign kept (also for zero), by a true IEEE binary32 division.       */
/* ------------------------------------------------------------------------- */
static void quantize_row(const float *x, int64_t cols, uint8_t *codes, uint8_t *scales,
                         float *d_out) {
    if (cols <= 0) {
        *d_out = 0.0f;
        return;
    }
    float amax = 0.0f;
    for (int64_t j = 0; j < cols; ++j) {
        assert(isfinite(x[j]));
        float a = fabsf(x[j]);
        if (a > amax) amax = a;
    }
    float d = amax / 2688.0f; /* 2688 = 6 * 448 */
    *d_out = d;
    memset(codes, 0, (size_t)(cols / 2));
    if (d == 0.0f) {
        for (int64_t b = 0; b < cols / 16; ++b) scales[b] = 0;
        for (int64_t j = 0; j < cols; ++j) {
            uint8_t code = (uint8_t)(signbit(x[j]) ? 8 : 0);
            codes[j / 2] |= (uint8_t)((j % 2) ? (code << 4) : code);
        }
        return;
    }
    float D = 6.0f * d;
    for (int64_t b = 0; b < cols / 16; ++b) {
        float ab = 0.0f;
        for (int64_t j = 16 * b; j < 16 * b + 16; ++j) {
            float a = fabsf(x[j]);
            if (a > ab) ab = a;
        }
        float t = ab / D;
        uint8_t sb = orc_e4m3_encode(t);
        scales[b] = sb;
        float S = orc_e4m3_value(sb) * d;
        for (int64_t j = 16 * b; j < 16 * b + 16; ++j) {
            uint8_t mag = 0;
            if (S != 0.0f) mag = orc_e2m1_encode_mag(fabsf(x[j]) / S);
            uint8_t code = (uint8_t)((signbit(x[j]) ? 8 : 0) | mag);
            codes[j / 2] |= (uint8_t)((j % 2) ? (code << 4) : code);
        }
    }
}

void orc_quantize_rows_f32(const float *x, int64_t ld, int64_t rows, int64_t cols,
                           uint8_t *codes, uint8_t *scales, float *d) {
    assert(cols % 16 == 0);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        quantize_row(x + i * ld, cols, codes + i * (cols / 2), scales + i * (cols / 16), d + i);
}

void orc_quantize_rows_bf16(const uint16_t *x, int64_t ld, int64_t rows, int64_t cols,
                            uint8_t *codes, uint8_t *scales, float *d) {
    assert(cols % 16 == 0);
#pragma omp parallel
    {
        float *row = (float *)malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < rows; ++i) {
            for (int64_t j = 0; j < cols; ++j) row[j] = orc_bf16_to_f32(x[i * ld + j]);
            quantize_row(row, cols, codes + i * (cols / 2), scales + i * (cols / 16), d + i);
        }
        free(row);
    }
}

static float operand_value(const uint8_t *codes, const uint8_t *scales, int64_t j) {
    uint8_t byte = codes[j / 2];
    uint8_t code = (uint8_t)((j % 2) ? (byte >> 4) : (byte & 15));
    return orc_e2m1_value(code) * orc_e4m3_value(scales[j / 16]); /* exact */
}

void orc_operand_values(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                        int64_t cols, float *b) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j)
            b[i * cols + j] = operand_value(codes + i * (cols / 2), scales + i * (cols / 16), j);
}

void orc_dequantize(const uint8_t *codes, const uint8_t *scales, const float *d,
                    int64_t rows, int64_t cols, float *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j)
            out[i * cols + j] =
                operand_value(codes + i * (cols / 2), scales + i * (cols / 16), j) * d[i];
}

/* ------------------------------------------------------------------------- */
/* RMSNorm ([blog] Method bullet 2: the quantized RMSNorm output is what the  */
/* backward reuses; bullet 4: quantization is fused into the norm kernel).    */
/* Reading: the quantizer sees the BF16-rounded norm output, exactly what a   */
/* separate quantize kernel would read.                                       */
/* ------------------------------------------------------------------------- */

/* Exact sum of squares: every BF16 value is M * 2^k with integer M < 256 and
 * -133 <= k <= 120, so x^2 = M^2 * 2^(2k) is an integer multiple of 2^-266.
 * Sum those integers in a 640-bit accumulator, then round once to binary64. */
#define SQ_LIMBS 10
double orc_sumsq_bf16(const uint16_t *x, int64_t n) {
    uint64_t acc[SQ_LIMBS];
    memset(acc, 0, sizeof acc);
    for (int64_t i = 0; i < n; ++i) {
        uint32_t e = (x[i] >> 7) & 0xFF, f = x[i] & 0x7F;
        assert(e != 0xFF);
        uint64_t M = (e == 0) ? f : (128u + f);
        int k = (e == 0) ? -133 : (int)e - 127 - 7;
        if (M == 0) continue;
        uint64_t sq = M * M;                  /* < 2^16 */
        int pos = 2 * k + 266;                /* bit position of the unit */
        int limb = pos / 64, sh = pos % 64;
        unsigned __int128 v = (unsigned __int128)sq << sh;
        uint64_t carry = 0;
        for (int L = limb; L < SQ_LIMBS; ++L) {
            unsigned __int128 add = (L == limb) ? (uint64_t)v : (L == limb + 1) ? (uint64_t)(v >> 64) : 0;
            unsigned __int128 s = (unsigned __int128)acc[L] + add + carry;
            acc[L] = (uint64_t)s;
            carry = (uint64_t)(s >> 64);
            if (L > limb + 1 && carry == 0) break;
        }
        assert(carry == 0);
    }
    /* locate the top set bit */
    int top = -1;
    for (int L = SQ_LIMBS - 1; L >= 0 && top < 0; --L)
        if (acc[L]) top = L * 64 + 63 - __builtin_clzll(acc[L]);
    if (top < 0) return 0.0;
#define BIT(p) ((p) < 0 ? 0u : (unsigned)((acc[(p) / 64] >> ((p) % 64)) & 1u))
    /* take 53 bits [top-52, top], then round to nearest even using the rest */
    uint64_t mant = 0;
    for (int p = top; p > top - 53; --p) mant = (mant << 1) | BIT(p);
    int lsb = top - 52;
    unsigned round_bit = BIT(lsb - 1);
    unsigned sticky = 0;
    for (int p = lsb - 2; p >= 0; --p) sticky |= BIT(p);
#undef BIT
    if (round_bit && (sticky || (mant & 1u))) mant += 1; /* may carry to 2^53: still exact */
    return ldexp((double)mant, lsb - 266);
}

void orc_rmsnorm_quant(const uint16_t *x, int64_t ld, const uint16_t *gamma, float eps,
                       int64_t rows, int64_t cols, uint16_t *y, uint8_t *codes,
                       uint8_t *scales, float *d, float *rstd) {
    assert(cols % 16 == 0);
#pragma omp parallel
    {
        float *row = (float *)malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < rows; ++i) {
            const uint16_t *xi = x + i * ld;
            double ss = orc_sumsq_bf16(xi, cols);
            double ms = ss / (double)cols;
            double v = ms + (double)eps;
            double rt = sqrt(v);
            double inv = 1.0 / rt;
            float r = (float)inv;
            if (rstd) rstd[i] = r;
            for (int64_t j = 0; j < cols; ++j) {
                float t = orc_bf16_to_f32(xi[j]) * r;
                float t2 = t * orc_bf16_to_f32(gamma[j]);
                uint16_t yb = orc_f32_to_bf16(t2);
                if (y) y[i * cols + j] = yb;
                row[j] = orc_bf16_to_f32(yb);
            }
            quantize_row(row, cols, codes + i * (cols / 2), scales + i * (cols / 16), d + i);
        }
        free(row);
    }
}

/* ------------------------------------------------------------------------- */
/* SiLU * mul ([blog] Method bullet 2: forward keeps BF16 inputs, an NVFP4   */
/* copy of gate/up is kept for backward; [abstract]).                         */
/* Reading: sigma32(g) is the correctly rounded binary32 value of            */
/* g / (1 + exp(-g)); h = bf16(sigma32(g) * u) with one binary32 multiply.    */
/* ------------------------------------------------------------------------- */
static float g_sig_table[65536];
static int g_sig_unsafe = -1; /* -1: not built; else count of undecided inputs */

/* Quad-precision (binary128, 113-bit significand) evaluation, then one
 * rounding to binary32.  The evaluation error is a few units of 2^-113
 * relative.  Small |g| puts the value within about g^3/24 (relative) of a
 * binary32 rounding midpoint (g/2 + g^2/4 can be a midpoint exactly), which is
 * still far above 2^-100 for every BF16 input that does not round to g/2; an
 * input is flagged if its quad value lies within 2^-100 of a midpoint. */
static float sigmoid_q(uint16_t gb, int *unsafe) {
    __float128 g = (__float128)orc_bf16_to_f32(gb);
    __float128 e = expq(-g);
    __float128 v = g / (1.0Q + e);
    float r = (float)v;
    *unsafe = 0;
    if (v != 0.0Q && (__float128)r != v) {
        float nb = ((__float128)r < v) ? nextafterf(r, INFINITY) : nextafterf(r, -INFINITY);
        __float128 mid = ((__float128)r + (__float128)nb) / 2.0Q; /* exact */
        __float128 dist = fabsq(v - mid), mag = fabsq(v);
        if (dist <= mag * ldexpq(1.0Q, -100)) *unsafe = 1;
    }
    return r;
}

static void build_sig_table(void) {
    int bad = 0;
    for (uint32_t b = 0; b < 65536; ++b) {
        uint32_t e = (b >> 7) & 0xFF;
        if (e == 0xFF) { g_sig_table[b] = NAN; continue; }
        int u;
        g_sig_table[b] = sigmoid_q((uint16_t)b, &u);
        bad += u;
    }
    g_sig_unsafe = bad;
}

int orc_sigmoid_check_table(void) {
    if (g_sig_unsafe < 0) build_sig_table();
    return g_sig_unsafe;
}

float orc_sigmoid_mul_g(uint16_t g_bits) {
    if (g_sig_unsafe < 0) build_sig_table();
    return g_sig_table[g_bits];
}

void orc_silu_mul_quant(const uint16_t *g, const uint16_t *u, int64_t ld, int64_t rows,
                        int64_t cols, uint16_t *h,
                        uint8_t *hc, uint8_t *hs, float *hd,
                        uint8_t *gc, uint8_t *gs, float *gd,
                        uint8_t *uc, uint8_t *us, float *ud) {
    assert(cols % 16 == 0);
    if (g_sig_unsafe < 0) build_sig_table();
    assert(g_sig_unsafe == 0);
#pragma omp parallel
    {
        float *hrow = (float *)malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < rows; ++i) {
            for (int64_t j = 0; j < cols; ++j) {
                float sg = g_sig_table[g[i * ld + j]];
                float p = sg * orc_bf16_to_f32(u[i * ld + j]);
                uint16_t hb = orc_f32_to_bf16(p);
                if (h) h[i * cols + j] = hb;
                hrow[j] = orc_bf16_to_f32(hb);
            }
            quantize_row(hrow, cols, hc + i * (cols / 2), hs + i * (cols / 16), hd + i);
        }
        free(hrow);
    }
    if (gc) orc_quantize_rows_bf16(g, ld, rows, cols, gc, gs, gd);
    if (uc) orc_quantize_rows_bf16(u, ld, rows, cols, uc, us, ud);
}

/* ------------------------------------------------------------------------- */
/* Weight layouts ([blog] Method bullet 4: forward and backward NVFP4 weight  */
/* layouts are rebuilt, transposed and re-quantized once, then cached).       */
/* Reading: the backward layout is built from the forward NVFP4 weights       */
/* reconstructed in FP32 (R = b * d, one rounding), transposed, and quantized */
/* by Q along the rows of R^T (blocks of 16 along N).                          */
/* ------------------------------------------------------------------------- */
void orc_build_weight_layouts(const uint16_t *W, int64_t N, int64_t K,
                              uint8_t *fc, uint8_t *fs, float *fd,
                              uint8_t *bc, uint8_t *bs, float *bd, int use_given_fwd) {
    assert(K % 16 == 0 && N % 16 == 0);
    if (!use_given_fwd) orc_quantize_rows_bf16(W, K, N, K, fc, fs, fd);
    float *Rt = (float *)malloc(sizeof(float) * (size_t)(N * K > 0 ? N * K : 1));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            Rt[k * N + n] = operand_value(fc + n * (K / 2), fs + n * (K / 16), k) * fd[n];
    orc_quantize_rows_f32(Rt, N, K, N, bc, bs, bd);
    free(Rt);
}

/* ------------------------------------------------------------------------- */
/* NVFP4 GEMM + BF16 LoRA term                                                */
/* [blog] Method bullet 1: frozen projections run as NVFP4 GEMMs with FP32    */
/* accumulation and BF16 output, forward and input-gradient; final note of   */
/* the Method section: adapters A, B stay BF16.  [peft] LoRA: h = W0 x + BAx. */
/* Readings: the adapters multiply the BF16 activation (not its NVFP4 copy);  */
/* the rank-r intermediate is rounded to BF16; the LoRA term is scaled by s   */
/* and added after the frozen output is scaled by both row scales; an        */
/* optional BF16 C (residual) is added last; one BF16 rounding at the end.    */
/* ------------------------------------------------------------------------- */
static void gemm_tn_rows(const uint8_t *ac, const uint8_t *as, const float *ad, int64_t Kc,
                         const uint8_t *bcodes, const uint8_t *bscales, const float *bdv,
                         int64_t Nout,
                         const uint16_t *Xl, int64_t Kl, /* LoRA input rows, length Kl */
                         const uint16_t *P, int64_t p_sj, int64_t p_sk, /* P[j,k2] strides */
                         const uint16_t *Q, int64_t q_sn, int64_t q_sj, /* Q[n,j] strides */
                         int32_t r, float s, const uint16_t *C,
                         const int64_t *row_idx, int64_t n_rows, uint16_t *out) {
    float *bvals = (float *)malloc(sizeof(float) * (size_t)(Nout * Kc > 0 ? Nout * Kc : 1));
    orc_operand_values(bcodes, bscales, Nout, Kc, bvals);
#pragma omp parallel
    {
        float *avals = (float *)malloc(sizeof(float) * (size_t)(Kc > 0 ? Kc : 1));
        float T[1024];
        assert(r <= 1024);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i) {
            int64_t m = row_idx[i];
            for (int64_t k = 0; k < Kc; ++k)
                avals[k] = operand_value(ac + m * (Kc / 2), as + m * (Kc / 16), k);
            for (int32_t j = 0; j < r; ++j) {
                float t = 0.0f;
                for (int64_t k2 = 0; k2 < Kl; ++k2) {
                    float p = orc_bf16_to_f32(Xl[m * Kl + k2]) * orc_bf16_to_f32(P[j * p_sj + k2 * p_sk]);
                    t = t + p;
                }
                T[j] = orc_bf16_to_f32(orc_f32_to_bf16(t));
            }
            for (int64_t n = 0; n < Nout; ++n) {
                const float *bn = bvals + n * Kc;
                float acc = 0.0f;
                for (int64_t k = 0; k < Kc; ++k) {
                    float p = avals[k] * bn[k];
                    acc = acc + p;
                }
                float y = acc * ad[m];
                y = y * bdv[n];
                if (r > 0) {
                    float L = 0.0f;
                    for (int32_t j = 0; j < r; ++j) {
                        float p = T[j] * orc_bf16_to_f32(Q[n * q_sn + j * q_sj]);
                        L = L + p;
                    }
                    float sl = s * L;
                    y = y + sl;
                }
                if (C) y = y + orc_bf16_to_f32(C[m * Nout + n]);
                out[i * Nout + n] = orc_f32_to_bf16(y);
            }
        }
        free(avals);
    }
    free(bvals);
}

void orc_gemm_fwd(const uint8_t *xc, const uint8_t *xs, const float *xd,
                  const uint16_t *X, int64_t M, int64_t K,
                  const uint8_t *wc, const uint8_t *ws, const float *wd, int64_t N,
                  const uint16_t *A, const uint16_t *B, int32_t r, float s,
                  const uint16_t *C, const int64_t *row_idx, int64_t n_rows, uint16_t *Y) {
    (void)M;
    assert(K % 16 == 0);
    /* T = X A^T: P[j,k] = A[j*K + k];  L = T B^T: Q[n,j] = B[n*r + j] */
    gemm_tn_rows(xc, xs, xd, K, wc, ws, wd, N, X, K, A, K, 1, B, r, 1, r, s, C, row_idx, n_rows, Y);
}

void orc_gemm_dgrad(const uint8_t *gc, const uint8_t *gs, const float *gd,
                    const uint16_t *dY, int64_t M, int64_t N,
                    const uint8_t *wc, const uint8_t *ws, const float *wd, int64_t K,
                    const uint16_t *A, const uint16_t *B, int32_t r, float s,
                    const uint16_t *C, const int64_t *row_idx, int64_t n_rows, uint16_t *dX) {
    (void)M;
    assert(N % 16 == 0);
    /* T' = dY B: P[j,n] = B[n*r + j];  L' = T' A: Q[k,j] = A[j*K + k] */
    gemm_tn_rows(gc, gs, gd, N, wc, ws, wd, K, dY, N, B, 1, r, A, 1, K, r, s, C, row_idx, n_rows, dX);
}

/* ------------------------------------------------------------------------- */
/* Nonlinear backward from the NVFP4 stash ([blog] Method bullet 2: the       */
/* quantized RMSNorm output is reused in backward instead of a separately     */
/* saved norm input; the SiLU-multiply keeps an NVFP4 copy of gate/up for     */
/* backward; [abstract]: quantized RMSNorm outputs reused, gate/up saved in   */
/* NVFP4 for backward).                                                       */
/* ------------------------------------------------------------------------- */

/* d/dg of g*sigma(g) = sigma(g) (1 + g (1 - sigma(g))), correctly rounded to
 * binary32 for a BF16 g, evaluated in binary128 like sigmoid_q (an input is
 * flagged when its quad value lies within 2^-100 of a binary32 midpoint). */
static float g_dsilu_table[65536];
static int g_dsilu_unsafe = -1;

static float dsilu_q(uint16_t gb, int *unsafe) {
    __float128 g = (__float128)orc_bf16_to_f32(gb);
    __float128 s = 1.0Q / (1.0Q + expq(-g));
    __float128 v = s * (1.0Q + g * (1.0Q - s));
    float r = (float)v;
    *unsafe = 0;
    if (v != 0.0Q && (__float128)r != v) {
        float nb = ((__float128)r < v) ? nextafterf(r, INFINITY) : nextafterf(r, -INFINITY);
        __float128 mid = ((__float128)r + (__float128)nb) / 2.0Q;
        if (fabsq(v - mid) <= fabsq(v) * ldexpq(1.0Q, -100)) *unsafe = 1;
    }
    return r;
}

static void build_dsilu_table(void) {
    int bad = 0;
    for (uint32_t b = 0; b < 65536; ++b) {
        if (((b >> 7) & 0xFF) == 0xFF) { g_dsilu_table[b] = NAN; continue; }
        int u;
        g_dsilu_table[b] = dsilu_q((uint16_t)b, &u);
        bad += u;
    }
    g_dsilu_unsafe = bad;
}

int orc_dsilu_check_table(void) {
    if (g_dsilu_unsafe < 0) build_dsilu_table();
    return g_dsilu_unsafe;
}

float orc_dsilu(uint16_t g_bits) {
    if (g_dsilu_unsafe < 0) build_dsilu_table();
    return g_dsilu_table[g_bits];
}

/* Dequantized value of element k of an NVFP4 row: fl32((code value x block
 * scale) x row scale), the product of the first two being exact. */
static float deq_elem(const uint8_t *codes, const uint8_t *scales, float d, int64_t k) {
    return operand_value(codes, scales, k) * d;
}

/* SiLU-multiply backward.  Readings: the stashed g and u are dequantized and
 * taken in BF16 (g' = bf16(deq(gq)), u' = bf16(deq(uq)); the BF16 rounding is
 * far below the NVFP4 error and makes silu and its derivative correctly
 * rounded binary32 values of BF16 inputs); du = bf16(dh * sigma32(g')),
 * dg = bf16((dh * u') * dsilu32(g')), each product one binary32 rounding;
 * dgq = Q(dg), duq = Q(du) for the gate/up input-gradient GEMMs. */
void orc_silu_mul_bwd_quant(const uint16_t *dh, int64_t ld, int64_t rows, int64_t cols,
                            const uint8_t *gc, const uint8_t *gs, const float *gd,
                            const uint8_t *uc, const uint8_t *us, const float *ud,
                            uint16_t *dg, uint16_t *du,
                            uint8_t *dgc, uint8_t *dgs, float *dgd,
                            uint8_t *duc, uint8_t *dus, float *dud) {
    assert(cols % 16 == 0);
    if (g_sig_unsafe < 0) build_sig_table();
    if (g_dsilu_unsafe < 0) build_dsilu_table();
    assert(g_sig_unsafe == 0 && g_dsilu_unsafe == 0);
#pragma omp parallel
    {
        float *grow = (float *)malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
        float *urow = (float *)malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < rows; ++i) {
            const uint8_t *gci = gc + i * (cols / 2), *gsi = gs + i * (cols / 16);
            const uint8_t *uci = uc + i * (cols / 2), *usi = us + i * (cols / 16);
            for (int64_t j = 0; j < cols; ++j) {
                uint16_t gb = orc_f32_to_bf16(deq_elem(gci, gsi, gd[i], j));
                float up = orc_bf16_to_f32(orc_f32_to_bf16(deq_elem(uci, usi, ud[i], j)));
                float d = orc_bf16_to_f32(dh[i * ld + j]);
                uint16_t dub = orc_f32_to_bf16(d * g_sig_table[gb]);
                float t = d * up;
                uint16_t dgb = orc_f32_to_bf16(t * g_dsilu_table[gb]);
                if (dg) dg[i * cols + j] = dgb;
                if (du) du[i * cols + j] = dub;
                grow[j] = orc_bf16_to_f32(dgb);
                urow[j] = orc_bf16_to_f32(dub);
            }
            if (dgc) quantize_row(grow, cols, dgc + i * (cols / 2), dgs + i * (cols / 16), dgd + i);
            if (duc) quantize_row(urow, cols, duc + i * (cols / 2), dus + i * (cols / 16), dud + i);
        }
        free(grow);
        free(urow);
    }
}

/* Exact dot product of a BF16 vector and a binary32 vector, rounded once to
 * binary64.  A BF16 value is M1 2^k1 (M1 < 2^8, -133 <= k1 <= 120), a binary32
 * value M2 2^k2 (M2 < 2^24, -149 <= k2 <= 104), so every product is an integer
 * (< 2^32) times 2^-282 with exponent below 2^225; positive and negative
 * products go to two 704-bit accumulators, subtracted at the end. */
#define DOT_LIMBS 11
static void acc_add(uint64_t *acc, uint64_t v, int pos) {
    int limb = pos / 64, sh = pos % 64;
    unsigned __int128 w = (unsigned __int128)v << sh;
    uint64_t carry = 0;
    for (int L = limb; L < DOT_LIMBS; ++L) {
        unsigned __int128 add = (L == limb) ? (uint64_t)w : (L == limb + 1) ? (uint64_t)(w >> 64) : 0;
        unsigned __int128 s = (unsigned __int128)acc[L] + add + carry;
        acc[L] = (uint64_t)s;
        carry = (uint64_t)(s >> 64);
        if (L > limb + 1 && carry == 0) break;
    }
    assert(carry == 0);
}

static int acc_cmp(const uint64_t *a, const uint64_t *b) {
    for (int L = DOT_LIMBS - 1; L >= 0; --L)
        if (a[L] != b[L]) return a[L] > b[L] ? 1 : -1;
    return 0;
}

static void acc_sub(uint64_t *a, const uint64_t *b) { /* a -= b, a >= b */
    uint64_t borrow = 0;
    for (int L = 0; L < DOT_LIMBS; ++L) {
        unsigned __int128 s = (unsigned __int128)a[L] - b[L] - borrow;
        a[L] = (uint64_t)s;
        borrow = (uint64_t)(s >> 64) ? 1 : 0;
    }
}

/* Round acc * 2^-unit_exp to nearest even binary64 (the values here stay far
 * inside the binary64 range). */
static double acc_round(const uint64_t *acc, int unit_exp) {
    int top = -1;
    for (int L = DOT_LIMBS - 1; L >= 0 && top < 0; --L)
        if (acc[L]) top = L * 64 + 63 - __builtin_clzll(acc[L]);
    if (top < 0) return 0.0;
#define BIT(p) ((p) < 0 ? 0u : (unsigned)((acc[(p) / 64] >> ((p) % 64)) & 1u))
    uint64_t mant = 0;
    for (int p = top; p > top - 53; --p) mant = (mant << 1) | BIT(p);
    int lsb = top - 52;
    unsigned round_bit = BIT(lsb - 1);
    unsigned sticky = 0;
    for (int p = lsb - 2; p >= 0; --p) sticky |= BIT(p);
#undef BIT
    if (round_bit && (sticky || (mant & 1u))) mant += 1;
    return ldexp((double)mant, lsb - unit_exp);
}

double orc_dot_bf16_f32(const uint16_t *a, const float *b, int64_t n) {
    uint64_t pos[DOT_LIMBS], neg[DOT_LIMBS];
    memset(pos, 0, sizeof pos);
    memset(neg, 0, sizeof neg);
    for (int64_t i = 0; i < n; ++i) {
        uint32_t e1 = (a[i] >> 7) & 0xFF, f1 = a[i] & 0x7F;
        assert(e1 != 0xFF);
        uint64_t M1 = (e1 == 0) ? f1 : (128u + f1);
        int k1 = (e1 == 0) ? -133 : (int)e1 - 127 - 7;
        uint32_t bb;
        memcpy(&bb, &b[i], 4);
        uint32_t e2 = (bb >> 23) & 0xFF, f2 = bb & 0x7FFFFF;
        assert(e2 != 0xFF);
        uint64_t M2 = (e2 == 0) ? f2 : ((1u << 23) + f2);
        int k2 = (e2 == 0) ? -149 : (int)e2 - 127 - 23;
        if (M1 == 0 || M2 == 0) continue;
        int neg_sign = ((a[i] >> 15) ^ (bb >> 31)) & 1;
        acc_add(neg_sign ? neg : pos, M1 * M2, k1 + k2 + 282);
    }
    if (acc_cmp(pos, neg) >= 0) {
        acc_sub(pos, neg);
        return acc_round(pos, 282);
    }
    acc_sub(neg, pos);
    return -acc_round(neg, 282);
}

/* RMSNorm backward from the stash.  With y = x rstd gamma and x^ = x rstd,
 * dx = rstd (g - x^ mean(g x^)), g = dy gamma.  Readings: x^ is recovered
 * from the NVFP4 stash as y'/gamma with y' = deq(yq) in binary32 (x^ = 0
 * where gamma = 0); since g x^ = dy y', the mean is S/H with S the exact sum
 * of dy y' rounded once to binary64, c = fl32(S / H) (binary64 division);
 * per element dx = bf16(fl32(fl32(fl32(dy gamma) - fl32(x^ c)) rstd)
 * (+ C, one more binary32 rounding before the BF16 one); optional dxq = Q(dx).
 * gamma is frozen (no gamma gradient). */
void orc_rmsnorm_bwd(const uint16_t *dy, int64_t ld, const uint8_t *yc, const uint8_t *ys,
                     const float *yd, const uint16_t *gamma, const float *rstd, const uint16_t *C,
                     int64_t ldc, int64_t rows, int64_t cols, uint16_t *dx, uint8_t *dxc,
                     uint8_t *dxs, float *dxd) {
    assert(cols % 16 == 0);
#pragma omp parallel
    {
        float *yrow = (float *)malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
        float *xrow = (float *)malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < rows; ++i) {
            const uint8_t *yci = yc + i * (cols / 2), *ysi = ys + i * (cols / 16);
            for (int64_t j = 0; j < cols; ++j) yrow[j] = deq_elem(yci, ysi, yd[i], j);
            const double S = orc_dot_bf16_f32(dy + i * ld, yrow, cols);
            const float c = (float)(S / (double)cols);
            const float r = rstd[i];
            for (int64_t j = 0; j < cols; ++j) {
                const float gm = orc_bf16_to_f32(gamma[j]);
                const float xh = gm != 0.0f ? yrow[j] / gm : 0.0f;
                const float g = orc_bf16_to_f32(dy[i * ld + j]) * gm;
                const float t = xh * c;
                const float v = (g - t) * r;
                const float w = C ? v + orc_bf16_to_f32(C[i * ldc + j]) : v;
                const uint16_t b = orc_f32_to_bf16(w);
                if (dx) dx[i * cols + j] = b;
                xrow[j] = orc_bf16_to_f32(b);
            }
            if (dxc) quantize_row(xrow, cols, dxc + i * (cols / 2), dxs + i * (cols / 16), dxd + i);
        }
        free(yrow);
        free(xrow);
    }
}

/* ------------------------------------------------------------------------- */
/* LoRA weight gradients on the NVFP4 stash ([blog] Method bullet 2 and final */
/* note: the activations kept for backward are the NVFP4 copies, the adapters */
/* are BF16; [peft] LoRA: h = W0 x + B A x, so dB = dY^T (A x)^T-side and      */
/* dA = (B^T dY)-side x^T).                                                   */
/* Readings: the LoRA input is the stash dequantized and taken in BF16,       */
/* X^ = bf16(deq(Xq)) (the BF16 X is not kept); the rank-r intermediates are   */
/* rounded to BF16 like the forward's (T^ = s bf16(X^ A^T), T' = s bf16(dY B)); */
/* dB = dY^T T^ [N, r] and dA = T'^T X^ [r, K]; the reference sums in binary64.*/
/* ------------------------------------------------------------------------- */
void orc_lora_grads(const uint8_t *xc, const uint8_t *xs, const float *xd, int64_t M, int64_t K,
                    const uint16_t *dY, int64_t ld_dy, int64_t N, const uint16_t *A, const uint16_t *B,
                    int32_t r, float s, double *dA, double *dB) {
    assert(K % 16 == 0 && r > 0);
    float *Xh = (float *)malloc(sizeof(float) * (size_t)(M * K > 0 ? M * K : 1));
    float *Th = (float *)malloc(sizeof(float) * (size_t)(M * r));
    float *Tp = (float *)malloc(sizeof(float) * (size_t)(M * r));
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k)
            Xh[m * K + k] = orc_bf16_to_f32(orc_f32_to_bf16(deq_elem(xc + m * (K / 2), xs + m * (K / 16), xd[m], k)));
        for (int32_t j = 0; j < r; ++j) {
            float t = 0.0f, u = 0.0f;
            for (int64_t k = 0; k < K; ++k) t = t + Xh[m * K + k] * orc_bf16_to_f32(A[j * K + k]);
            for (int64_t n = 0; n < N; ++n)
                u = u + orc_bf16_to_f32(dY[m * ld_dy + n]) * orc_bf16_to_f32(B[n * r + j]);
            Th[m * r + j] = s * orc_bf16_to_f32(orc_f32_to_bf16(t));
            Tp[m * r + j] = s * orc_bf16_to_f32(orc_f32_to_bf16(u));
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int32_t j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int64_t m = 0; m < M; ++m) acc += (double)orc_bf16_to_f32(dY[m * ld_dy + n]) * (double)Th[m * r + j];
            dB[n * r + j] = acc;
        }
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int32_t j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int64_t m = 0; m < M; ++m) acc += (double)Tp[m * r + j] * (double)Xh[m * K + k];
            dA[j * K + k] = acc;
        }
    free(Xh);
    free(Th);
    free(Tp);
}

/* ------------------------------------------------------------------------- */
/* AdamW step of the trainable adapters.  The hotdry.top Unsloth post         */
/* (section on paged optimizers) has Adam keep a first and a second moment    */
/* per trainable parameter in 32-bit state; the update itself is the          */
/* published AdamW rule (Loshchilov & Hutter, decoupled weight decay):        */
/*   p <- p - lr wd p;  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;    */
/*   p <- p - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).             */
/* Binary64 throughout; t >= 1 is the step number.                            */
/* ------------------------------------------------------------------------- */
/* BF16 of the binary32 master copy of binary64 values: bf16(fl32(x)). */
void orc_master_bf16(const double *x, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16((float)x[i]);
}

void orc_adamw_step(double *p, double *m, double *v, const double *g, int64_t n, double lr, double b1, double b2,
                    double eps, double wd, int64_t t) {
    assert(t >= 1);
    const double bc1 = 1.0 - pow(b1, (double)t);
    const double bc2 = 1.0 - pow(b2, (double)t);
    for (int64_t i = 0; i < n; ++i) {
        p[i] = p[i] - lr * wd * p[i];
        m[i] = b1 * m[i] + (1.0 - b1) * g[i];
        v[i] = b2 * v[i] + (1.0 - b2) * g[i] * g[i];
        const double mhat = m[i] / bc1;
        const double vhat = v[i] / bc2;
        p[i] = p[i] - lr * mhat / (sqrt(vhat) + eps);
    }
}

/* ------------------------------------------------------------------------- */
/* NVFP4-adapted GPTQ: the column sweep ([blog] Method, bullet 3: the frozen */
/* weights are calibrated offline by GPTQ adapted to the NVFP4 block scales,  */
/* with statistics from reconstructed NVFP4 activations; arXiv abstract).     */
/* GPTQ (Frantar et al.) quantizes the columns of W [N][K] in order and       */
/* spreads each column's rounding error over the columns not yet quantized,   */
/* through the upper Cholesky factor U of the inverse Hessian (H^-1 = U^T U): */
/*   err = (w_i - q_i) / U[i][i];  w_j -= err U[i][j]  (j > i).                */
/* Updates inside a block of `bs` columns are applied column by column; the   */
/* block's errors reach the later columns at the block's end, as one sum over */
/* the block's columns in increasing order (GPTQ's lazy batch update; the     */
/* same result as column by column up to the rounding order).                 */
/* NVFP4: at the first column of every 16-column block the block's E4M3 scale */
/* is chosen by the plain quantizer's rule on the current (error-updated)     */
/* weights rounded to binary32, with the row scale d of the original weights; */
/* each column's code is the plain quantizer's code of its binary32-rounded   */
/* current weight under that scale; q = code value x scale x d (exact in      */
/* binary64).  Rows are independent (OpenMP over rows).                      */
/* ------------------------------------------------------------------------- */
void orc_gptq_sweep(const double *U, double *W, const float *d, int64_t N, int64_t K, int32_t bs,
                    uint8_t *codes, uint8_t *scales) {
    assert(K % 16 == 0 && bs % 16 == 0 && bs > 0);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t n = 0; n < N; ++n) {
        double *w = W + n * K;
        uint8_t *cr = codes + n * (K / 2);
        uint8_t *sr = scales + n * (K / 16);
        const float dn = d[n];
        const float D = 6.0f * dn;
        double *err = (double *)malloc(sizeof(double) * (size_t)bs);
        float S = 0.0f;
        for (int64_t i1 = 0; i1 < K; i1 += bs) {
            const int64_t i2 = i1 + bs < K ? i1 + bs : K;
            for (int64_t i = i1; i < i2; ++i) {
                if (i % 16 == 0) {
                    /* the block's scale from its current weights */
                    float amax = 0.0f;
                    for (int64_t j = i; j < i + 16; ++j) {
                        const float a = fabsf((float)w[j]);
                        if (a > amax) amax = a;
                    }
                    uint8_t sb = 0;
                    if (dn != 0.0f) {
                        const float t = amax / D;
                        sb = orc_e4m3_encode(t);
                    }
                    sr[i / 16] = sb;
                    S = orc_e4m3_value(sb) * dn;
                }
                const float wf = (float)w[i];
                uint8_t mag = 0;
                if (S != 0.0f) mag = orc_e2m1_encode_mag(fabsf(wf) / S);
                const uint8_t code = (uint8_t)((signbit(wf) ? 8 : 0) | mag);
                if (i & 1)
                    cr[i / 2] |= (uint8_t)(code << 4);
                else
                    cr[i / 2] = code;
                const double q = (double)orc_e2m1_value(code) * (double)orc_e4m3_value(sr[i / 16]) * (double)dn;
                const double e = (w[i] - q) / U[i * K + i];
                err[i - i1] = e;
                for (int64_t j = i + 1; j < i2; ++j) w[j] -= e * U[i * K + j];
                w[i] = q;
            }
            for (int64_t j = i2; j < K; ++j) {
                double s = 0.0;
                for (int64_t i = i1; i < i2; ++i) s += err[i - i1] * U[i * K + j];
                w[j] -= s;
            }
        }
        free(err);
    }
}
