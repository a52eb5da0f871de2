// pact_device.h -- device-side building blocks shared by libpact's kernels:
// BF16 <-> FP32, the NVFP4 block encoder (per-16 E4M3 scale, E2M1 codes) and
// wavefront reductions.  gfx950 only.
//
// Format (simolm.com PACT blog, FAQ): 16 E2M1 elements share one E4M3 block
// scale; this library adds one FP32 scale per row.  Encoding rule (the pages
// leave it open; this is the reading the library implements):
//   d = fl32(amax_row / 2688), D = fl32(6 d),
//   block scale s = E4M3 round-to-nearest-even of fl32(amax_block / D), <= 448,
//   S = fl32(s d), code = sign | E2M1 round-to-nearest-even of fl32(|x| / S).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pact {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even FP32 -> BF16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two FP32 values rounded to nearest-even BF16 (the hardware's packed
// conversion), low half = a.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    typedef float f2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
    const f2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, b2_t));
}

// E4M3 value of a scale byte (0x00..0x7E), exact, via the hardware decoder.
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
    return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// E4M3 round-to-nearest-even of t >= 0, clamped to 448 (0x7E).  The hardware
// encoder rounds to nearest even but turns values above 448 into NaN, so the
// clamp happens first; t <= 448 never needs saturation after rounding.
__device__ __forceinline__ uint32_t e4m3_encode_sat(float t) {
    t = fminf(t, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t, t, 0, false) & 0xFFu;
}

// E2M1 codes (round-to-nearest-even, saturating at 6, sign kept for zero) of
// two FP32 quotients a, b (already |x|/S with the sign of x): low nibble = a.
__device__ __forceinline__ uint32_t e2m1_encode2(float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
}

// fl32(|x| / S) for x exactly representable in BF16 and S a binary32, with the
// sign of x: |x| has at most 8 significant bits, so the exact quotient is never
// within 2^-49 (relative) of a binary32 rounding midpoint; the binary64 product
// |x| * RN64(1/S) is within 2^-52 of it and therefore rounds to the same
// binary32 value.  rS = 1.0 / (double)S (correctly rounded binary64 divide).
__device__ __forceinline__ float quot_bf16(float x, double rS) {
    return (float)((double)x * rS);
}

// fl32(x / S) for any binary32 x: binary64 division rounds correctly, and
// binary64 -> binary32 rounding of it is the correctly rounded binary32
// quotient (53 >= 2*24 + 2).
__device__ __forceinline__ float quot_f32(float x, float S) {
    return (float)((double)x / (double)S);
}

// Packed FP4 dword (8 codes, element 2j in the low nibble of byte j) -> 8
// FP16 values scaled by the block scale sc: the E2M1 x E4M3 products are
// exact in FP16 (at most 6 significant bits, magnitudes in [2^-10, 2688]).
__device__ __forceinline__ half8_t decode8(uint32_t w, half2_t sc) {
    const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc;
    const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc;
    const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc;
    const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc;
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, h0);
    r.y = __builtin_bit_cast(uint32_t, h1);
    r.z = __builtin_bit_cast(uint32_t, h2);
    r.w = __builtin_bit_cast(uint32_t, h3);
    return __builtin_bit_cast(half8_t, r);
}

// Dequantized values of one NVFP4 block: R[j] = fl32(code_j x scale) x d,
// the first product exact (FP16), one binary32 rounding by the row scale d.
__device__ __forceinline__ void dequant16(uint32_t c0, uint32_t c1, uint32_t scale_byte, float d, float R[16]) {
    const half2_t sh = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)scale_byte, 1.0f, false);
    half2_t sc;
    sc[0] = sh[0];
    sc[1] = sh[0];
    const half8_t h0 = decode8(c0, sc), h1 = decode8(c1, sc);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        R[j] = (float)h0[j] * d;
        R[8 + j] = (float)h1[j] * d;
    }
}

// 8 dequantized values of one 8-code dword, rounded to BF16 (four words, low
// half first): bf16(fl32((code x scale in FP16) x d)), as dequant16.
__device__ __forceinline__ u32x4 dequant8_bf16(uint32_t w, half2_t sc, float d) {
    const half8_t h = decode8(w, sc);
    u32x4 r;
    r.x = f32x2_to_bf16x2((float)h[0] * d, (float)h[1] * d);
    r.y = f32x2_to_bf16x2((float)h[2] * d, (float)h[3] * d);
    r.z = f32x2_to_bf16x2((float)h[4] * d, (float)h[5] * d);
    r.w = f32x2_to_bf16x2((float)h[6] * d, (float)h[7] * d);
    return r;
}

// FP16 pair (both halves) of an E4M3 scale byte.
__device__ __forceinline__ half2_t e4m3_to_h2(uint32_t byte) {
    const half2_t sh = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)byte, 1.0f, false);
    half2_t sc;
    sc[0] = sh[0];
    sc[1] = sh[0];
    return sc;
}

// Per-row parameters of the quantizer.
struct RowQ {
    float d;    // row scale
    float D;    // fl32(6 d)
    double rD;  // RN64(1 / D), used by the BF16-exact encoder (0 when d == 0)
};

__device__ __forceinline__ RowQ row_params(float amax) {
    RowQ r;
    r.d = amax / 2688.0f;  // correctly rounded binary32 division (HIP default)
    r.D = 6.0f * r.d;
    r.rD = r.d == 0.0f ? 0.0 : 1.0 / (double)r.D;
    return r;
}

// row_params for an amax exactly representable in BF16 (a maximum of BF16
// magnitudes): fl32(amax / 2688) as the binary64 product with RN64(1/2688),
// equal to the correctly rounded quotient by the argument at quot_bf16.
__device__ __forceinline__ RowQ row_params_bf16(float amax) {
    RowQ r;
    r.d = quot_bf16(amax, 1.0 / 2688.0);
    r.D = 6.0f * r.d;
    r.rD = r.d == 0.0f ? 0.0 : 1.0 / (double)r.D;
    return r;
}

// Two BF16 values per 32-bit word: packed 16-bit integer helpers.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                  __builtin_bit_cast(u16x2_t, b)));
}

__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2_t, a),
                                                                  __builtin_bit_cast(u16x2_t, b)));
}

__device__ __forceinline__ uint32_t pk_sub_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2_t, a) - __builtin_bit_cast(u16x2_t, b));
}

// max |x| over 16 finite BF16 values packed two per word (low half first):
// for finite values the magnitude order is the integer order of the low 15
// bits, so the maximum is taken on the packed words and widened once.
__device__ __forceinline__ float amax16_packed(const uint32_t w[8]) {
    uint32_t m = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = pk_max_u16(m, w[j] & 0x7FFF7FFFu);
    return __uint_as_float(max(m & 0xFFFFu, m >> 16) << 16);
}

// Encode one block of 16 BF16-exact values v[0..15] (FP32 registers) given
// its block amax and the row parameters.  Returns the 8 code bytes packed in
// two dwords and the scale byte.  When d == 0 (all-zero row) every code is the
// sign bit only and the scale byte is 0.
template <bool kBF16Exact>
__device__ __forceinline__ void encode_block16(const float v[16], float bamax, RowQ rq,
                                               uint32_t &codes_lo, uint32_t &codes_hi,
                                               uint32_t &scale_byte) {
    uint32_t w[2] = {0u, 0u};
    if (rq.d == 0.0f) {
        scale_byte = 0u;
#pragma unroll
        for (int j = 0; j < 16; ++j)
            w[j >> 3] |= ((__float_as_uint(v[j]) >> 31) << 3) << (4 * (j & 7));
        codes_lo = w[0];
        codes_hi = w[1];
        return;
    }
    // fl32(bamax / D): bamax is one of the block's magnitudes, so for BF16
    // inputs the binary64 product with RN64(1/D) rounds to the same value
    // (see quot_bf16); otherwise a correctly rounded binary32 division.
    const float t = kBF16Exact ? quot_bf16(bamax, rq.rD) : bamax / rq.D;
    uint32_t sb = e4m3_encode_sat(t);
    scale_byte = sb;
    float S = e4m3_to_f32(sb) * rq.d;
    if (S == 0.0f) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
            w[j >> 3] |= ((__float_as_uint(v[j]) >> 31) << 3) << (4 * (j & 7));
    } else {
        // quotients with the sign of x, then 4 converts per dword: the byte
        // select of the converter places codes 2j, 2j+1 in byte j
        float q[16];
        if (kBF16Exact) {
            const double rS = 1.0 / (double)S;
#pragma unroll
            for (int j = 0; j < 16; ++j) q[j] = quot_bf16(v[j], rS);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) q[j] = quot_f32(v[j], S);
        }
        uint32_t a = 0u, b = 0u;
        a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, q[0], q[1], 1.0f, 0);
        a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, q[2], q[3], 1.0f, 1);
        a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, q[4], q[5], 1.0f, 2);
        a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, q[6], q[7], 1.0f, 3);
        b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, q[8], q[9], 1.0f, 0);
        b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, q[10], q[11], 1.0f, 1);
        b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, q[12], q[13], 1.0f, 2);
        b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, q[14], q[15], 1.0f, 3);
        w[0] = a;
        w[1] = b;
    }
    codes_lo = w[0];
    codes_hi = w[1];
}

// A kernel's by-value argument struct read in place from the kernel-argument
// segment: every field is a scalar load the compiler may repeat where needed,
// rather than a copy it keeps live in scalar registers (or in scratch, where
// a field's address is taken).
template <class T>
__device__ __forceinline__ const T &kernel_args() {
    return *(const T *)(const __attribute__((address_space(4))) T *)__builtin_amdgcn_kernarg_segment_ptr();
}

// ---- wavefront reductions (64 lanes) --------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// Error-free double-double accumulation: (s, c) += x.
__device__ __forceinline__ void dd_add(double &s, double &c, double x) {
    double t = s + x;
    double bp = t - s;
    double e = (s - (t - bp)) + (x - bp);
    s = t;
    c += e;
}

__device__ __forceinline__ void dd_add_dd(double &s, double &c, double s2, double c2) {
    dd_add(s, c, s2);
    c += c2;
}

__device__ __forceinline__ void wave_sum_dd(double &s, double &c) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        double s2 = __shfl_xor(s, off, 64);
        double c2 = __shfl_xor(c, off, 64);
        dd_add_dd(s, c, s2, c2);
    }
}

}  // namespace pact
