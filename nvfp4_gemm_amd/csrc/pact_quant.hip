// pact_quant.hip -- row-wise NVFP4 producers (HBM-bound):
//   pact_quantize_nvfp4        Q(x)
//   pact_rmsnorm_quant_nvfp4   y = bf16(x rstd gamma), Q(y), rstd
//   pact_silu_mul_quant_nvfp4  h = bf16(sigma32(g) u), Q(h), Q(g), Q(u)
// (simolm.com PACT blog, section "Method": quantization fused into RMSNorm and
// SiLU-multiply; the quantized RMSNorm output and NVFP4 gate/up copies are
// what backward keeps; forward nonlinear ops read BF16.)
//
// Design: one row per 64*WPR threads; each thread owns whole 16-element blocks
// (lane, lane + T, ...; moved in 64-block chunks, see load_chunk), kept in registers
// as packed BF16, so the row is read from HBM exactly once.  Block
// and row maxima are taken on the packed words (magnitude bits compare as
// integers); the row maximum (and, for RMSNorm, the sum of squares) is reduced
// across the wavefront with shuffles and across the row's wavefronts through
// LDS, in a fixed order so that every thread sees the same value.  Codes go
// out as 8-byte stores, scale bytes as one byte per block (contiguous across
// lanes).  Inputs and outputs are streamed with nontemporal accesses.  The
// SiLU kernel keeps its 32 KB sigma32 table in LDS and loops over rows.
#include "pact_device.h"
#include "pact_host.h"

namespace pact {

struct NV {
    uint8_t *codes;
    uint8_t *scales;
    float *d;
};

enum { MODE_QUANT = 0, MODE_RMS = 1, MODE_SILU = 2, MODE_SILU_BWD = 3, MODE_RMS_BWD = 4 };

struct CNV {  // NVFP4 input
    const uint8_t *codes;
    const uint8_t *scales;
    const float *d;
};

struct RowArgs {
    const uint16_t *x;  // QUANT/RMS: x, SILU: g
    int64_t ldx;
    const uint16_t *x2;  // SILU: u
    int64_t ldx2;
    const uint16_t *gamma;  // RMS
    float eps;
    uint16_t *y;  // RMS: y, SILU: h (nullable)
    int64_t ldy;
    NV q0;  // QUANT: out, RMS: yq, SILU: hq
    NV q1;  // SILU: gq (codes == nullptr: skip)
    NV q2;  // SILU: uq
    float *rstd;
    int64_t rows;
    int cols;
};

// sigma32(g): the correctly rounded binary32 value of g / (1 + exp(-g)) for a
// BF16 g.  Outside 2^-25 <= |g| < 2^7 it follows a closed rule (g/2 below,
// g or -0 above by sign, 0 for Inf/NaN); inside, it is one of 8192 entries
// generated at build time by gen_sigmoid_table.cpp, which states the method
// and checks the rule against the full evaluation for all 65536 patterns.
// Kernels copy the 32 KB table into LDS once and look entries up there.
constexpr int kSigTab = 8192;
__device__ const uint32_t kSigmoidCompact[kSigTab] = {
#include "pact_sigmoid_table.inc"
};

// dsilu32(g): the correctly rounded binary32 value of d/dg (g / (1 + exp(-g)))
// = sigma(g) (1 + g (1 - sigma(g))), same index and range as kSigmoidCompact;
// outside it 0.5 below, 1 or -0 above by sign, 0 for Inf/NaN (same generator).
__device__ const uint32_t kDsiluCompact[kSigTab] = {
#include "pact_dsilu_table.inc"
};

__device__ __forceinline__ void load_dsilu_table(uint32_t *tab, int tid, int nthreads) {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(kDsiluCompact);
    u32x4 *dst = reinterpret_cast<u32x4 *>(tab);
    for (int i = tid; i < kSigTab / 4; i += nthreads) dst[i] = src[i];
}

__device__ __forceinline__ void load_sigmoid_table(uint32_t *tab, int tid, int nthreads) {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(kSigmoidCompact);
    u32x4 *dst = reinterpret_cast<u32x4 *>(tab);
    for (int i = tid; i < kSigTab / 4; i += nthreads) dst[i] = src[i];
}

__device__ __forceinline__ uint32_t silu32_index(uint32_t b) {
    const uint32_t e = (b >> 7) & 0xFFu;
    const uint32_t ec = min(max(e, 102u), 133u) - 102u;
    return ((b >> 15) << 12) | (ec << 7) | (b & 127u);
}

// sigma32 of a BF16 pattern b given its (always in-range) table entry t.
__device__ __forceinline__ float silu32_select(uint32_t b, uint32_t t) {
    const uint32_t e = (b >> 7) & 0xFFu;
    const float g = __uint_as_float(b << 16);
    const float big = (b & 0x8000u) ? -0.0f : g;
    const float hi = e == 255u ? 0.0f : big;
    return e < 102u ? g * 0.5f : (e < 134u ? __uint_as_float(t) : hi);
}

// sigma32 of the 16 BF16 values packed in w[8] (low half first).  The table
// offset of a pattern is its magnitude bits minus 102 << 7 (one packed 16-bit
// subtraction per pair); offsets of 4096 and above (or wrapped below zero)
// mark values outside the table's range, which take the closed rule, a path
// a wavefront enters only when one of its lanes holds such a value (the
// forward's gate is a GEMM output, where exact zeros are rare).  All table
// reads are issued before any is used; the empty asm keeps the compiler from
// moving them into branches.
__device__ __forceinline__ void silu32_x16(const uint32_t w[8], const uint32_t *tab, float s[16]) {
    uint32_t t[16];
    uint32_t oor = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t r = pk_sub_u16(w[j] & 0x7FFF7FFFu, 0x33003300u);  // 0x3300 = 102 << 7
        oor = pk_max_u16(oor, r);
        const uint32_t ilo = (r & 0xFFFu) | ((w[j] >> 3) & 0x1000u);
        const uint32_t ihi = ((r >> 16) & 0xFFFu) | ((w[j] >> 19) & 0x1000u);
        t[2 * j] = tab[ilo];
        t[2 * j + 1] = tab[ihi];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) asm volatile("" : "+v"(t[j]));
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] = __uint_as_float(t[j]);
    if (max(oor & 0xFFFFu, oor >> 16) >= 0x1000u) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            s[2 * j] = silu32_select(w[j] & 0xFFFFu, t[2 * j]);
            s[2 * j + 1] = silu32_select(w[j] >> 16, t[2 * j + 1]);
        }
    }
}

// The SiLU backward reads g' = bf16 of a decoded NVFP4 value, which is exactly
// zero for every zero code.  Its LDS table is laid out by (offset, sign) and
// interleaved: entry 2k + s holds {sigma32, dsilu32} of the pattern with sign
// s and magnitude bits (102 << 7) + k, k < 4096 (exponents 102..133), and
// entries 8192 and 8193 those of +0 and -0 (+-0 and 0.5), so that zeros stay
// on the fast path.
constexpr int kSigTabZ = kSigTab + 2;

__device__ __forceinline__ int silu_tab_source(int i) { return ((i & 1) << 12) | (i >> 1); }

__device__ __forceinline__ void load_silu_dsilu_table_z(u32x2 *tab, int tid, int nthreads) {
    for (int i = tid; i < kSigTabZ; i += nthreads) {
        u32x2 e;
        e.x = i < kSigTab ? kSigmoidCompact[silu_tab_source(i)] : (i == kSigTab ? 0u : 0x80000000u);
        e.y = i < kSigTab ? kDsiluCompact[silu_tab_source(i)] : 0x3F000000u;  // 0.5f
        tab[i] = e;
    }
}

// Table entries of the two BF16 patterns packed in w (low half first), with
// one packed 16-bit subtraction and clamp for both: magnitudes outside the
// table's range map to the zero entries.  mx collects the largest magnitude,
// mn the smallest magnitude minus one (zero wraps to 0xFFFF), for silu_tab_miss.
__device__ __forceinline__ void silu_tab_entries(uint32_t w, uint32_t &ilo, uint32_t &ihi, uint32_t &mx,
                                                 uint32_t &mn) {
    const uint32_t mag = w & 0x7FFF7FFFu;
    mx = pk_max_u16(mx, mag);
    mn = pk_min_u16(mn, pk_sub_u16(mag, 0x00010001u));
    const uint32_t rc = pk_min_u16(pk_sub_u16(mag, 0x33003300u), 0x10001000u);  // 0x3300 = 102 << 7
    ilo = ((rc & 0xFFFFu) << 1) | ((w >> 15) & 1u);
    ihi = ((rc >> 16) << 1) | (w >> 31);
}

// Whether some value seen by silu_tab_entries is neither zero nor in the
// table's range (exponent below 102, or 134 and above, Inf and NaN included).
__device__ __forceinline__ bool silu_tab_miss(uint32_t mx, uint32_t mn) {
    return max(mx & 0xFFFFu, mx >> 16) >= 0x4300u || min(mn & 0xFFFFu, mn >> 16) < 0x32FFu;
}

// dsilu32 of a BF16 pattern b given its (always in-range) table entry t.
__device__ __forceinline__ float dsilu32_select(uint32_t b, uint32_t t) {
    const uint32_t e = (b >> 7) & 0xFFu;
    const float big = (b & 0x8000u) ? -0.0f : 1.0f;
    const float hi = e == 255u ? 0.0f : big;
    return e < 102u ? 0.5f : (e < 134u ? __uint_as_float(t) : hi);
}

// sigma32 and dsilu32 of the 16 BF16 values packed in w[8] from the
// interleaved table (each entry {sigma32, dsilu32}: one 8-byte LDS read serves
// both), with the fast path of silu32_x16.
__device__ __forceinline__ void silu_dsilu_x16(const uint32_t w[8], const u32x2 *tab, float s[16], float ds[16]) {
    uint32_t ts[16], td[16];
    uint32_t mx = 0u, mn = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t ilo, ihi;
        silu_tab_entries(w[j], ilo, ihi, mx, mn);
        const u32x2 lo = tab[ilo], hi = tab[ihi];
        ts[2 * j] = lo.x;
        td[2 * j] = lo.y;
        ts[2 * j + 1] = hi.x;
        td[2 * j + 1] = hi.y;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) asm volatile("" : "+v"(ts[j]), "+v"(td[j]));
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        s[j] = __uint_as_float(ts[j]);
        ds[j] = __uint_as_float(td[j]);
    }
    if (silu_tab_miss(mx, mn)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            s[2 * j] = silu32_select(w[j] & 0xFFFFu, ts[2 * j]);
            s[2 * j + 1] = silu32_select(w[j] >> 16, ts[2 * j + 1]);
            ds[2 * j] = dsilu32_select(w[j] & 0xFFFFu, td[2 * j]);
            ds[2 * j + 1] = dsilu32_select(w[j] >> 16, td[2 * j + 1]);
        }
    }
}

// Workgroup barrier ordering LDS only.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);  // every lane is active
}

// Maximum over the wavefront of two packed 16-bit unsigned values, in every
// lane: four DPP steps within 16-lane rows, then lane swaps across rows.
__device__ __forceinline__ uint32_t wave_max_pk_u16(uint32_t v) {
    v = pk_max_u16(v, dpp_mov<0xB1>(v));   // quad_perm [1, 0, 3, 2]: lane i ^ 1
    v = pk_max_u16(v, dpp_mov<0x4E>(v));   // quad_perm [2, 3, 0, 1]: lane i ^ 2
    v = pk_max_u16(v, dpp_mov<0x141>(v));  // row_half_mirror: 8-lane groups
    v = pk_max_u16(v, dpp_mov<0x140>(v));  // row_mirror: 16-lane rows
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // rows 0 and 1, 2 and 3
    v = pk_max_u16(a[0], a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // the two halves
    return pk_max_u16(b[0], b[1]);
}

// Row maxima of NV (1..3) non-negative BF16-exact values (maxima of block
// maxima), two packed per 32-bit word (BF16 patterns of non-negative values
// order as the values do), reduced across the wavefront and then across the
// row's wavefronts through LDS in a fixed order, so that every thread of the
// row sees the same values.
template <int WPR, int NV>
__device__ __forceinline__ void row_max(float &a, float &b, float &c, uint32_t (*red)[2], int wave, int lrow) {
    uint32_t w0 = (__float_as_uint(a) >> 16) | (NV > 1 ? (__float_as_uint(b) & 0xFFFF0000u) : 0u);
    uint32_t w1 = NV > 2 ? (__float_as_uint(c) >> 16) : 0u;
    w0 = wave_max_pk_u16(w0);
    if constexpr (NV > 2) w1 = wave_max_pk_u16(w1);
    if constexpr (WPR > 1) {
        if ((threadIdx.x & 63) == 0) {
            red[wave][0] = w0;
            red[wave][1] = w1;
        }
        lds_sync();
        const int f = lrow * WPR;
        w0 = red[f][0];
        w1 = red[f][1];
#pragma unroll
        for (int w = 1; w < WPR; ++w) {
            w0 = pk_max_u16(w0, red[f + w][0]);
            if constexpr (NV > 2) w1 = pk_max_u16(w1, red[f + w][1]);
        }
        lds_sync();
    }
    a = __uint_as_float(w0 << 16);
    if constexpr (NV > 1) b = __uint_as_float(w0 & 0xFFFF0000u);
    if constexpr (NV > 2) c = __uint_as_float(w1 << 16);
}

// Hides the packed words from the compiler so that the encode phase unpacks
// them again instead of keeping 16 FP32 values per block live across the row
// reduction (one VALU operation per element against up to 48 registers).
__device__ __forceinline__ void opaque8(uint32_t w[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(w[j]));
}

__device__ __forceinline__ void unpack16(const uint32_t w[8], float v[16]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_lo(w[i]);
        v[2 * i + 1] = bf16_hi(w[i]);
    }
}

// Input blocks are read with ordinary (cached) loads: inside a layer the
// producer's output is often still in the Infinity Cache, and there cached
// loads were faster (SiLU-multiply-quantize 8192 x 8192: 125-128 -> 107 us
// per call within the layer step), although nontemporal loads had been 1.6x
// faster on 8192 x 8192 inputs with the caches flushed.  Stores keep the
// nontemporal hint.
// Row blocks move between HBM and registers with fully coalesced 16-byte
// accesses.  A wavefront covers a chunk of 64 consecutive 16-element blocks
// (2 KB of BF16) with two instructions: in the first, lanes i and 32 + i read
// the two halves of block i (i < 32), in the second those of block 32 + i.
// One v_permlane32_swap per register pair (upper lanes of the first with the
// lower lanes of the second) then leaves lane l with block l of the chunk
// whole.  The alternative, each lane reading its own 32-byte block with two
// 16-byte accesses, has every instruction touch half of each cache line: on
// the MI355X a 3:5 read:write stream ran 1.7x slower that way (3.3 against
// 5.5 TB/s), a copy 1.2x.  Both helpers run in wavefront-uniform control flow
// (the swap takes all lanes); `active` (uniform) and the block bound mask the
// accesses, and masked loads yield zeros.  base: row start; cb: the chunk's
// first block (a multiple of 64).
__device__ __forceinline__ void swap_halves(u32x4 &a, u32x4 &b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const auto r = __builtin_amdgcn_permlane32_swap(a[j], b[j], false, false);
        a[j] = r[0];
        b[j] = r[1];
    }
}

__device__ __forceinline__ void load_chunk(const uint16_t *base, int cb, int nb, bool active, uint32_t w[8]) {
    const int lane = threadIdx.x & 63;
    const int i = lane & 31;
    const char *p = reinterpret_cast<const char *>(base) + 32u * (uint32_t)(cb + i) + 16u * (uint32_t)(lane >> 5);
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (active && cb + i < nb) a = *reinterpret_cast<const u32x4 *>(p);
    if (active && cb + 32 + i < nb) b = *reinterpret_cast<const u32x4 *>(p + 1024);
    swap_halves(a, b);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

__device__ __forceinline__ void store_chunk(uint16_t *base, int cb, int nb, bool active, const uint32_t w[8]) {
    const int lane = threadIdx.x & 63;
    const int i = lane & 31;
    u32x4 a, b;
    a.x = w[0]; a.y = w[1]; a.z = w[2]; a.w = w[3];
    b.x = w[4]; b.y = w[5]; b.z = w[6]; b.w = w[7];
    swap_halves(a, b);
    char *p = reinterpret_cast<char *>(base) + 32u * (uint32_t)(cb + i) + 16u * (uint32_t)(lane >> 5);
    if (active && cb + i < nb) __builtin_nontemporal_store(a, reinterpret_cast<u32x4 *>(p));
    if (active && cb + 32 + i < nb) __builtin_nontemporal_store(b, reinterpret_cast<u32x4 *>(p + 1024));
}

__device__ __forceinline__ void emit_block(const NV &q, int64_t row, int cols, int b, const float v[16],
                                           float bmax, RowQ rq) {
    uint32_t lo, hi, sb;
    encode_block16<true>(v, bmax, rq, lo, hi, sb);
    u32x2 c;
    c.x = lo;
    c.y = hi;
    uint8_t *cr = q.codes + row * (cols / 2);
    uint8_t *sr = q.scales + row * (cols / 16);
    __builtin_nontemporal_store(c, reinterpret_cast<u32x2 *>(cr + 8u * (uint32_t)b));
    __builtin_nontemporal_store((uint8_t)sb, sr + (uint32_t)b);
}

// Binade spread of the nonzero BF16 values of a set of packed words, for the
// exact-accumulation fast paths: the exponent of the largest magnitude minus
// that of the smallest nonzero one (negative for an all-zero set), or 2^20
// when a value is subnormal, infinite or NaN (such sets take the error-free
// accumulation).
struct MagRange {
    uint32_t mx = 0u, mn = 0xFFFFFFFFu;  // packed largest magnitude, smallest magnitude - 1 (zero wraps)
};

__device__ __forceinline__ void mag_range_add(MagRange &r, uint32_t w) {
    const uint32_t mag = w & 0x7FFF7FFFu;
    r.mx = pk_max_u16(r.mx, mag);
    r.mn = pk_min_u16(r.mn, pk_sub_u16(mag, 0x00010001u));
}

__device__ __forceinline__ int mag_spread(const MagRange &r) {
    const uint32_t hi = max(r.mx & 0xFFFFu, r.mx >> 16);
    const uint32_t lo = min(r.mn & 0xFFFFu, r.mn >> 16);  // 0xFFFF: no nonzero value
    if (hi >= 0x7F80u || lo < 0x7Fu) return 1 << 20;
    return (int)(hi >> 7) - (int)((lo + 1u) >> 7);
}

// Threads of a row kernel's workgroup: 256, or one row of 64 * WPR.
template <int WPR>
constexpr int row_threads() { return WPR > 4 ? 64 * WPR : 256; }

template <int WPR, int BPL, int MODE>
__global__ __launch_bounds__(row_threads<WPR>()) void row_kernel(RowArgs a_arg) {
    const RowArgs &a = kernel_args<RowArgs>();
    (void)a_arg;
    constexpr int NT = row_threads<WPR>();
    constexpr int T = 64 * WPR;
    constexpr int RPW = NT / T;
    __shared__ uint32_t red[NT / 64][2];
    __shared__ double redd[NT / 64][2];
    __shared__ uint32_t sig[MODE == MODE_SILU ? kSigTab : 1];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lrow = tid / T;
    const int lt = tid % T;
    const int c0 = lt & ~63;  // this wavefront's first chunk in the row (lane l: block c0 + l)
    const int cols = a.cols;
    const int nb = cols >> 4;
    if constexpr (MODE == MODE_SILU) {
        load_sigmoid_table(sig, tid, NT);
        lds_sync();
    }
    // SiLU workgroups loop over row groups (the table is loaded once per
    // workgroup); the other modes launch one workgroup per row group.
    const int64_t ngroups = (a.rows + RPW - 1) / RPW;
    const int rl = __builtin_amdgcn_readfirstlane(lrow);  // a row belongs to one wavefront
    for (int64_t grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
    const int64_t row = grp * RPW + rl;
    const bool active = row < a.rows;
    const uint16_t *xr = a.x + row * a.ldx;
    const uint16_t *ur = a.x2 + row * a.ldx2;
    uint16_t *yr = a.y + row * a.ldy;

    uint32_t xw[BPL][8];
    uint32_t uw[MODE == MODE_SILU ? BPL : 1][8];
    bool valid[BPL];
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
        const int cb = c0 + T * i;
        valid[i] = active && lt + T * i < nb;
        load_chunk(xr, cb, nb, active, xw[i]);
        if constexpr (MODE == MODE_SILU) load_chunk(ur, cb, nb, active, uw[i]);
    }

    if constexpr (MODE == MODE_QUANT) {
        float bmax[BPL];
        float rmax = 0.0f;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            bmax[i] = valid[i] ? amax16_packed(xw[i]) : 0.0f;
            rmax = fmaxf(rmax, bmax[i]);
        }
        float dummy1 = 0.0f, dummy2 = 0.0f;
        row_max<WPR, 1>(rmax, dummy1, dummy2, red, wave, lrow);
        const RowQ rq = row_params_bf16(rmax);
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            if (!valid[i]) continue;
            float v[16];
            opaque8(xw[i]);
            unpack16(xw[i], v);
            emit_block(a.q0, row, cols, lt + T * i, v, bmax[i], rq);
        }
        if (active && lt == 0) a.q0.d[row] = rq.d;
    } else if constexpr (MODE == MODE_RMS) {
        // Sum of squares, exact to the last place of the double-double
        // result.  Squares of BF16 values are exact in binary64 (16 bits).
        // When a lane's nonzero values span at most 15 binades, each of its
        // partial sums (at most 64 squares, masked blocks are zeros) is a
        // multiple of the smallest square's last place and below 2^53 of them
        // (2 * 15 + 14 + 2 + 6 <= 53), so plain binary64 accumulation is
        // exact; otherwise the lane accumulates error-free (double-double).
        double s = 0.0, c = 0.0;
        MagRange mr;
#pragma unroll
        for (int i = 0; i < BPL; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) mag_range_add(mr, xw[i][j]);
        if (mag_spread(mr) <= 15) {
#pragma unroll
            for (int i = 0; i < BPL; ++i) {
                float v[16];
                unpack16(xw[i], v);
#pragma unroll
                for (int j = 0; j < 16; ++j) s = __builtin_fma((double)v[j], (double)v[j], s);
            }
        } else {
#pragma unroll
            for (int i = 0; i < BPL; ++i) {
                float v[16];
                unpack16(xw[i], v);
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const double xv = (double)v[j];
                    dd_add(s, c, xv * xv);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < BPL; ++i) opaque8(xw[i]);  // unpacked again below
        wave_sum_dd(s, c);
        s = __shfl(s, 0, 64);  // every lane takes lane 0's (identical) result
        c = __shfl(c, 0, 64);
        if constexpr (WPR > 1) {
            if ((tid & 63) == 0) {
                redd[wave][0] = s;
                redd[wave][1] = c;
            }
            lds_sync();
            const int w0 = lrow * WPR;
            s = redd[w0][0];
            c = redd[w0][1];
#pragma unroll
            for (int w = 1; w < WPR; ++w) dd_add_dd(s, c, redd[w0 + w][0], redd[w0 + w][1]);
            lds_sync();
        }
        const double ss = s + c;
        const double ms = ss / (double)cols;
        const double vv = ms + (double)a.eps;
        const double rt = sqrt(vv);
        const double inv = 1.0 / rt;
        const float r = (float)inv;
        float bmax[BPL];
        float rmax = 0.0f;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            const int cb = c0 + T * i;
            uint32_t gw[8];
            load_chunk(a.gamma, cb, nb, true, gw);
            float v[16], gv[16];
            unpack16(xw[i], v);
            unpack16(gw, gv);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float t0 = v[2 * j] * r;
                const float t1 = v[2 * j + 1] * r;
                xw[i][j] = f32x2_to_bf16x2(t0 * gv[2 * j], t1 * gv[2 * j + 1]);  // y replaces x
            }
            if (a.y) store_chunk(yr, cb, nb, active, xw[i]);
            bmax[i] = valid[i] ? amax16_packed(xw[i]) : 0.0f;
            rmax = fmaxf(rmax, bmax[i]);
        }
        float dummy1 = 0.0f, dummy2 = 0.0f;
        row_max<WPR, 1>(rmax, dummy1, dummy2, red, wave, lrow);
        const RowQ rq = row_params_bf16(rmax);
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            if (!valid[i]) continue;
            float v[16];
            opaque8(xw[i]);
            unpack16(xw[i], v);
            emit_block(a.q0, row, cols, lt + T * i, v, bmax[i], rq);
        }
        if (active && lt == 0) {
            a.q0.d[row] = rq.d;
            if (a.rstd) a.rstd[row] = r;
        }
    } else {  // MODE_SILU
        float hmax[BPL], gmax[BPL], umax[BPL];
        float rh = 0.0f, rg = 0.0f, ru = 0.0f;
        uint32_t hw[BPL][8];
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            float sv[16];
            silu32_x16(xw[i], sig, sv);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                hw[i][j] = f32x2_to_bf16x2(sv[2 * j] * bf16_lo(uw[i][j]), sv[2 * j + 1] * bf16_hi(uw[i][j]));
            if (a.y) store_chunk(yr, c0 + T * i, nb, active, hw[i]);
            // masked blocks load as zeros: their maxima are 0
            hmax[i] = amax16_packed(hw[i]);
            gmax[i] = amax16_packed(xw[i]);
            umax[i] = amax16_packed(uw[i]);
            rh = fmaxf(rh, hmax[i]);
            rg = fmaxf(rg, gmax[i]);
            ru = fmaxf(ru, umax[i]);
        }
        row_max<WPR, 3>(rh, rg, ru, red, wave, lrow);
        const RowQ qh = row_params_bf16(rh), qg = row_params_bf16(rg), qu = row_params_bf16(ru);
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            if (!valid[i]) continue;
            const int b = lt + T * i;
            float v[16];
            opaque8(hw[i]);
            opaque8(xw[i]);
            opaque8(uw[i]);
            unpack16(hw[i], v);
            emit_block(a.q0, row, cols, b, v, hmax[i], qh);
            if (a.q1.codes) {
                unpack16(xw[i], v);
                emit_block(a.q1, row, cols, b, v, gmax[i], qg);
            }
            if (a.q2.codes) {
                unpack16(uw[i], v);
                emit_block(a.q2, row, cols, b, v, umax[i], qu);
            }
        }
        if (active && lt == 0) {
            a.q0.d[row] = qh.d;
            if (a.q1.codes) a.q1.d[row] = qg.d;
            if (a.q2.codes) a.q2.d[row] = qu.d;
        }
    }
    if constexpr (MODE != MODE_SILU) break;
    }  // row groups
}

// Wavefronts per row and 16-element blocks per lane of the row kernels for a
// row of nb blocks (the forward kernels and, separately, the backward ones).
static void row_shape(int mode, int64_t nb, int &wpr, int &bpl) {
    if (mode == MODE_SILU_BWD || mode == MODE_RMS_BWD) {
        if (nb <= 64) wpr = 1, bpl = 1;
        else if (nb <= 128) wpr = 1, bpl = 2;
        else if (nb <= 192) wpr = 1, bpl = 3;
        else if (nb <= 256) wpr = 4, bpl = 1;
        else if (nb <= 512) wpr = 8, bpl = 1;
        else if (nb <= 1024) wpr = 8, bpl = 2;
        else if (nb <= 1536) wpr = 8, bpl = 3;
        else wpr = 8, bpl = 4;
        return;
    }
    if (nb <= 64) wpr = 1, bpl = 1;
    else if (nb <= 128) wpr = 1, bpl = 2;
    else if (nb <= 192) wpr = 1, bpl = 3;
    else if (nb <= 256) wpr = 4, bpl = 1;
    else if (nb <= 512) wpr = 4, bpl = 2;
    else if (nb <= 768 && mode != MODE_SILU) wpr = 4, bpl = 3;
    else if (nb <= 1024) wpr = 8, bpl = 2;
    else if (nb <= 1536) wpr = 8, bpl = 3;
    else wpr = 8, bpl = 4;
}

template <int MODE>
static pact_status launch_rows(const RowArgs &a, hipStream_t st) {
    if (a.rows == 0 || a.cols == 0) return PACT_OK;
    const int nb = a.cols / 16;
    int wpr, bpl;
    row_shape(MODE, nb, wpr, bpl);
    const int threads = wpr > 4 ? 64 * wpr : 256;
    const int rpw = threads / (64 * wpr);
    const int64_t groups = (a.rows + rpw - 1) / rpw;
    // SiLU: the 32 KB table allows four resident workgroups per compute unit;
    // launch that many, each looping over row groups
    const int64_t cap = MODE == MODE_SILU ? (int64_t)device_cus() * 4 : groups;
    const dim3 grid((unsigned)(groups < cap ? groups : cap));
#define PACT_ROWS_CASE(W, B)                                                                  \
    if (wpr == W && bpl == B) {                                                               \
        hipLaunchKernelGGL((row_kernel<W, B, MODE>), grid, dim3(threads), 0, st, a);          \
        return launch_status();                                                               \
    }
    PACT_ROWS_CASE(1, 1)
    PACT_ROWS_CASE(1, 2)
    PACT_ROWS_CASE(1, 3)
    PACT_ROWS_CASE(4, 1)
    PACT_ROWS_CASE(4, 2)
    if constexpr (MODE != MODE_SILU) PACT_ROWS_CASE(4, 3)
    PACT_ROWS_CASE(8, 2)
    PACT_ROWS_CASE(8, 3)
    PACT_ROWS_CASE(8, 4)
#undef PACT_ROWS_CASE
    return PACT_ERR_UNSUPPORTED_SHAPE;
}

// ---- nonlinear backward from the NVFP4 stash --------------------------------
// (simolm.com PACT blog, section "Method", second bullet: the quantized RMSNorm
// output is reused in backward instead of a saved norm input; the SiLU-multiply
// keeps an NVFP4 copy of gate/up for backward.)
//   SILU_BWD: g' = bf16(deq(gq)), u' = bf16(deq(uq)); du = bf16(dh sigma32(g')),
//             dg = bf16((dh u') dsilu32(g')); dgq = Q(dg), duq = Q(du).
//   RMS_BWD:  y' = deq(yq); S = sum dy y' (double-double, exact to 2^-106
//             relative, rounded once); c = fl32(S / H); x^ = y'/gamma (0 where
//             gamma = 0); dx = bf16(fl32(fl32(dy gamma) - fl32(x^ c)) rstd (+ C));
//             dxq = Q(dx).
// Same layout as the forward row kernels: one row per 64 WPR threads, each
// thread owns whole 16-element blocks; NVFP4 blocks are read as 8 code bytes,
// one scale byte and the row scale.
struct BwdArgs {
    const uint16_t *dy;  // SILU_BWD: dh, RMS_BWD: dy
    int64_t lddy;
    CNV in0;  // SILU_BWD: gq, RMS_BWD: yq
    CNV in1;  // SILU_BWD: uq
    const uint16_t *gamma;  // RMS_BWD
    const float *rstd;      // RMS_BWD
    const uint16_t *C;      // RMS_BWD residual (nullable)
    int64_t ldc;
    uint16_t *o0;  // SILU_BWD: dg, RMS_BWD: dx (nullable)
    uint16_t *o1;  // SILU_BWD: du (nullable)
    int64_t ldo;
    NV q0;  // SILU_BWD: dgq, RMS_BWD: dxq (codes == nullptr: skip)
    NV q1;  // SILU_BWD: duq
    int64_t rows;
    int cols;
};

__device__ __forceinline__ void load_codes(const CNV &q, int64_t row, int cols, int b, uint32_t &c0, uint32_t &c1,
                                           uint32_t &sb) {
    const u32x2 c = *reinterpret_cast<const u32x2 *>(q.codes + row * (cols / 2) + 8 * b);
    c0 = c.x;
    c1 = c.y;
    sb = q.scales[row * (cols / 16) + b];
}

__device__ __forceinline__ void pack16(const float v[16], uint32_t w[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = f32x2_to_bf16x2(v[2 * j], v[2 * j + 1]);
}

// Occupancy floor of a backward kernel: the RMSNorm backward is held to
// 4 wavefronts per SIMD (at most 128 VGPRs) in the shapes where the compiler
// meets that without spilling (not 8 wavefronts per row x 3 blocks per lane,
// nor 4 blocks per lane).
template <int WPR, int BPL, int MODE>
constexpr int bwd_min_waves() {
    return MODE == MODE_RMS_BWD && BPL <= 3 && !(WPR == 8 && BPL == 3) ? 4 : 1;
}

template <int WPR, int BPL, int MODE>
__global__ __launch_bounds__(row_threads<WPR>()) __attribute__((amdgpu_waves_per_eu(bwd_min_waves<WPR, BPL, MODE>())))
void bwd_kernel(BwdArgs a_arg) {
    const BwdArgs &a = kernel_args<BwdArgs>();
    (void)a_arg;
    constexpr int NT = row_threads<WPR>();
    constexpr int T = 64 * WPR;
    constexpr int RPW = NT / T;
    __shared__ uint32_t red[NT / 64][2];
    __shared__ double redd[NT / 64][2];
    __shared__ u32x2 tabs[MODE == MODE_SILU_BWD ? kSigTabZ : 1];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lrow = tid / T;
    const int lt = tid % T;
    const int c0 = lt & ~63;  // this wavefront's first chunk in the row (lane l: block c0 + l)
    const int cols = a.cols;
    const int nb = cols >> 4;
    if constexpr (MODE == MODE_SILU_BWD) {
        load_silu_dsilu_table_z(tabs, tid, NT);
        lds_sync();
    }
    const int64_t ngroups = (a.rows + RPW - 1) / RPW;
    const int rl = __builtin_amdgcn_readfirstlane(lrow);
    // SiLU backward loops over row groups: the next group's operands are
    // loaded while the current one is processed (up to 3 blocks per lane; 4
    // would spill registers)
    constexpr bool PF = MODE == MODE_SILU_BWD && BPL <= 3;
    constexpr int BS = PF ? BPL : 1;
    uint32_t pdw[BS][8], pc0[BS][2], ps0[BS], pc1[BS][2], ps1[BS];
    float pd0 = 0.0f, pd1 = 0.0f;
    auto fetch = [&](int64_t g) {
        const int64_t prow = g * RPW + rl;
        const bool pact = prow < a.rows;
#pragma unroll
        for (int i = 0; i < BS; ++i) {
            const int cb = c0 + T * i;
            load_chunk(a.dy + prow * a.lddy, cb, nb, pact, pdw[i]);
            pc0[i][0] = pc0[i][1] = ps0[i] = pc1[i][0] = pc1[i][1] = ps1[i] = 0u;
            if (pact && lt + T * i < nb) {
                load_codes(a.in0, prow, cols, lt + T * i, pc0[i][0], pc0[i][1], ps0[i]);
                load_codes(a.in1, prow, cols, lt + T * i, pc1[i][0], pc1[i][1], ps1[i]);
            }
        }
        pd0 = pact ? a.in0.d[prow] : 0.0f;
        pd1 = pact ? a.in1.d[prow] : 0.0f;
    };
    if constexpr (PF) {
        if ((int64_t)blockIdx.x < ngroups) fetch(blockIdx.x);
    }
    for (int64_t grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
        const int64_t row = grp * RPW + rl;
        const bool active = row < a.rows;
        const uint16_t *dyr = a.dy + row * a.lddy;
        uint32_t dw[BPL][8];
        uint32_t k0[BPL][2], t0[BPL];
        uint32_t k1[MODE == MODE_SILU_BWD ? BPL : 1][2], t1[MODE == MODE_SILU_BWD ? BPL : 1];
        uint32_t cw[MODE == MODE_RMS_BWD ? BPL : 1][8];
        bool valid[BPL];
        float d0, d1 = 0.0f;
        if constexpr (PF) {
#pragma unroll
            for (int i = 0; i < BPL; ++i) {
                valid[i] = active && lt + T * i < nb;
#pragma unroll
                for (int j = 0; j < 8; ++j) dw[i][j] = pdw[i][j];
                k0[i][0] = pc0[i][0];
                k0[i][1] = pc0[i][1];
                t0[i] = ps0[i];
                k1[i][0] = pc1[i][0];
                k1[i][1] = pc1[i][1];
                t1[i] = ps1[i];
            }
            d0 = pd0;
            d1 = pd1;
            if (grp + gridDim.x < ngroups) fetch(grp + gridDim.x);
        } else {
#pragma unroll
            for (int i = 0; i < BPL; ++i) {
                const int cb = c0 + T * i;
                const int b = lt + T * i;
                valid[i] = active && b < nb;
                load_chunk(dyr, cb, nb, active, dw[i]);
                k0[i][0] = k0[i][1] = t0[i] = 0u;
                if constexpr (MODE == MODE_SILU_BWD) k1[i][0] = k1[i][1] = t1[i] = 0u;
                if (valid[i]) {
                    load_codes(a.in0, row, cols, b, k0[i][0], k0[i][1], t0[i]);
                    if constexpr (MODE == MODE_SILU_BWD) load_codes(a.in1, row, cols, b, k1[i][0], k1[i][1], t1[i]);
                }
            }
            d0 = active ? a.in0.d[row] : 0.0f;
            if constexpr (MODE == MODE_SILU_BWD) d1 = active ? a.in1.d[row] : 0.0f;
        }
        (void)dyr;

        if constexpr (MODE == MODE_SILU_BWD) {
            float gmax[BPL], umax[BPL];
            float rg = 0.0f, ru = 0.0f;
            uint32_t gw[BPL][8], uw[BPL][8];  // dg, du as packed BF16
#pragma unroll
            for (int i = 0; i < BPL; ++i) {
                // masked blocks hold zero codes, scales and dh: dg = du = 0
                float R[16];
                uint32_t gb[8];
                dequant16(k0[i][0], k0[i][1], t0[i], d0, R);
                pack16(R, gb);  // g' as BF16
                float U[16];
                dequant16(k1[i][0], k1[i][1], t1[i], d1, U);
                uint32_t ub[8];
                pack16(U, ub);  // u' as BF16
                float sv[16], dv[16];
                silu_dsilu_x16(gb, tabs, sv, dv);
                float vg[16], vu[16];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const float sl = sv[2 * j + h];
                        const float ds = dv[2 * j + h];
                        const float d = h ? bf16_hi(dw[i][j]) : bf16_lo(dw[i][j]);
                        const float up = h ? bf16_hi(ub[j]) : bf16_lo(ub[j]);
                        vu[2 * j + h] = d * sl;
                        const float t = d * up;
                        vg[2 * j + h] = t * ds;
                    }
                }
                pack16(vg, gw[i]);
                pack16(vu, uw[i]);
                if (a.o0) store_chunk(a.o0 + row * a.ldo, c0 + T * i, nb, active, gw[i]);
                if (a.o1) store_chunk(a.o1 + row * a.ldo, c0 + T * i, nb, active, uw[i]);
                gmax[i] = amax16_packed(gw[i]);
                umax[i] = amax16_packed(uw[i]);
                rg = fmaxf(rg, gmax[i]);
                ru = fmaxf(ru, umax[i]);
            }
            float dummy = 0.0f;
            row_max<WPR, 2>(rg, ru, dummy, red, wave, lrow);
            const RowQ qg = row_params_bf16(rg), qu = row_params_bf16(ru);
#pragma unroll
            for (int i = 0; i < BPL; ++i) {
                if (!valid[i]) continue;
                const int b = lt + T * i;
                float v[16];
                opaque8(gw[i]);
                opaque8(uw[i]);
                if (a.q0.codes) {
                    unpack16(gw[i], v);
                    emit_block(a.q0, row, cols, b, v, gmax[i], qg);
                }
                if (a.q1.codes) {
                    unpack16(uw[i], v);
                    emit_block(a.q1, row, cols, b, v, umax[i], qu);
                }
            }
            if (active && lt == 0) {
                if (a.q0.codes) a.q0.d[row] = qg.d;
                if (a.q1.codes) a.q1.d[row] = qu.d;
            }
        } else {  // MODE_RMS_BWD
            // S = sum dy y': products are exact in binary64 (8 x 24 bits)
            double s = 0.0, c = 0.0;
#pragma unroll
            for (int i = 0; i < BPL; ++i) {
                if (!valid[i]) continue;
                float R[16], v[16];
                dequant16(k0[i][0], k0[i][1], t0[i], d0, R);
                unpack16(dw[i], v);
#pragma unroll
                for (int j = 0; j < 16; ++j) dd_add(s, c, (double)v[j] * (double)R[j]);
            }
            wave_sum_dd(s, c);
            s = __shfl(s, 0, 64);
            c = __shfl(c, 0, 64);
            if constexpr (WPR > 1) {
                if ((tid & 63) == 0) {
                    redd[wave][0] = s;
                    redd[wave][1] = c;
                }
                lds_sync();
                const int w0 = lrow * WPR;
                s = redd[w0][0];
                c = redd[w0][1];
#pragma unroll
                for (int w = 1; w < WPR; ++w) dd_add_dd(s, c, redd[w0 + w][0], redd[w0 + w][1]);
                lds_sync();
            }
            const double S = s + c;
            const float cm = (float)(S / (double)cols);
            const float r = active ? a.rstd[row] : 0.0f;
            float xmax[BPL];
            float rx = 0.0f;
            uint32_t xw[BPL][8];
#pragma unroll
            for (int i = 0; i < BPL; ++i) {
                // masked blocks hold zero dy, codes, gamma and C: dx = 0
                const int cb = c0 + T * i;
                uint32_t gmw[8];
                load_chunk(a.gamma, cb, nb, true, gmw);
                float R[16], v[16], gm[16], o[16];
                dequant16(k0[i][0], k0[i][1], t0[i], d0, R);
                unpack16(dw[i], v);
                unpack16(gmw, gm);
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float xh = gm[j] != 0.0f ? R[j] / gm[j] : 0.0f;
                    const float g = v[j] * gm[j];
                    const float t = xh * cm;
                    o[j] = (g - t) * r;
                }
                if (a.C) {
                    // C is read only here, after the row sum, so that it does
                    // not hold registers through the reduction
                    load_chunk(a.C + row * a.ldc, cb, nb, active, cw[i]);
                    float cv[16];
                    unpack16(cw[i], cv);
#pragma unroll
                    for (int j = 0; j < 16; ++j) o[j] = o[j] + cv[j];
                }
                pack16(o, xw[i]);
                if (a.o0) store_chunk(a.o0 + row * a.ldo, cb, nb, active, xw[i]);
                xmax[i] = amax16_packed(xw[i]);
                rx = fmaxf(rx, xmax[i]);
            }
            if (a.q0.codes) {
                float dummy1 = 0.0f, dummy2 = 0.0f;
                row_max<WPR, 1>(rx, dummy1, dummy2, red, wave, lrow);
                const RowQ rq = row_params_bf16(rx);
#pragma unroll
                for (int i = 0; i < BPL; ++i) {
                    if (!valid[i]) continue;
                    float v[16];
                    opaque8(xw[i]);
                    unpack16(xw[i], v);
                    emit_block(a.q0, row, cols, lt + T * i, v, xmax[i], rq);
                }
                if (active && lt == 0) a.q0.d[row] = rq.d;
            }
        }
        if constexpr (MODE != MODE_SILU_BWD) break;
    }  // row groups
}

template <int MODE>
static pact_status launch_bwd(const BwdArgs &a, hipStream_t st) {
    if (a.rows == 0 || a.cols == 0) return PACT_OK;
    const int nb = a.cols / 16;
    int wpr, bpl;
    row_shape(MODE, nb, wpr, bpl);
    const int threads = wpr > 4 ? 64 * wpr : 256;
    const int rpw = threads / (64 * wpr);
    const int64_t groups = (a.rows + rpw - 1) / rpw;
    // SiLU backward: the 64 KB table allows two resident workgroups per CU,
    // which loop over row groups; RMSNorm backward: one workgroup per row group
    const int64_t cap = MODE == MODE_SILU_BWD ? (int64_t)device_cus() * 2 : groups;
    const dim3 grid((unsigned)(groups < cap ? groups : cap));
#define PACT_BWD_CASE(W, B)                                                                   \
    if (wpr == W && bpl == B) {                                                               \
        hipLaunchKernelGGL((bwd_kernel<W, B, MODE>), grid, dim3(threads), 0, st, a);          \
        return launch_status();                                                               \
    }
    PACT_BWD_CASE(1, 1)
    PACT_BWD_CASE(1, 2)
    PACT_BWD_CASE(1, 3)
    PACT_BWD_CASE(4, 1)
    PACT_BWD_CASE(8, 1)
    PACT_BWD_CASE(8, 2)
    PACT_BWD_CASE(8, 3)
    PACT_BWD_CASE(8, 4)
#undef PACT_BWD_CASE
    return PACT_ERR_UNSUPPORTED_SHAPE;
}

// Exposes dsilu32 for exhaustive verification.
__global__ __launch_bounds__(256) void dsilu_probe_kernel(const uint16_t *g, float *out, int64_t n) {
    __shared__ uint32_t tab[kSigTab];
    load_dsilu_table(tab, threadIdx.x, 256);
    lds_sync();
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = dsilu32_select(g[i], tab[silu32_index(g[i])]);
}

static CNV cnv_of(const pact_nvfp4 *q) {
    CNV n;
    n.codes = q->codes;
    n.scales = q->scales;
    n.d = q->row_scale;
    return n;
}

static NV nv_of(const pact_nvfp4 *q) {
    NV n;
    n.codes = q ? q->codes : nullptr;
    n.scales = q ? q->scales : nullptr;
    n.d = q ? q->row_scale : nullptr;
    return n;
}

static pact_status check_row_len(int64_t rows, int64_t cols) {
    if (rows < 0 || cols < 0) return PACT_ERR_INVALID_ARG;
    if (cols % 16 != 0 || cols > PACT_MAX_ROW) return PACT_ERR_UNSUPPORTED_SHAPE;
    return PACT_OK;
}

// Launch the row quantizer on an already validated BF16 matrix (also used by
// the weight-layout builder).
pact_status quantize_rows_launch(const uint16_t *x, int64_t ldx, int64_t rows, int64_t cols,
                                 const pact_nvfp4 *out, hipStream_t st) {
    RowArgs a = {};
    a.x = x;
    a.ldx = ldx;
    a.q0 = nv_of(out);
    a.rows = rows;
    a.cols = (int)cols;
    return launch_rows<MODE_QUANT>(a, st);
}

// Exposes sigma32 for exhaustive verification.
__global__ __launch_bounds__(256) void sigmoid_probe_kernel(const uint16_t *g, float *out, int64_t n) {
    __shared__ uint32_t sig[kSigTab];
    load_sigmoid_table(sig, threadIdx.x, 256);
    lds_sync();
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = silu32_select(g[i], sig[silu32_index(g[i])]);
}

}  // namespace pact

using namespace pact;

extern "C" pact_status pact_quantize_nvfp4(const uint16_t *x, int64_t ld_x, int64_t rows,
                                           int64_t cols, const pact_nvfp4 *out, void *stream) {
    PACT_TRY(check_row_len(rows, cols));
    PACT_TRY(check_bf16(x, ld_x, cols));
    PACT_TRY(check_nvfp4(out, rows, cols));
    return quantize_rows_launch(x, ld_x, rows, cols, out, as_stream(stream));
}

extern "C" pact_status pact_rmsnorm_quant_nvfp4(const uint16_t *x, int64_t ld_x,
                                                const uint16_t *gamma, float eps, int64_t rows,
                                                int64_t cols, uint16_t *y, int64_t ld_y,
                                                const pact_nvfp4 *yq, float *rstd, void *stream) {
    PACT_TRY(check_row_len(rows, cols));
    PACT_TRY(check_bf16(x, ld_x, cols));
    PACT_TRY(check_bf16(gamma, cols, cols));
    if (y) PACT_TRY(check_bf16(y, ld_y, cols));
    if (rstd && !aligned16(rstd)) return PACT_ERR_MISALIGNED;
    if (!(eps >= 0.0f)) return PACT_ERR_INVALID_ARG;
    PACT_TRY(check_nvfp4(yq, rows, cols));
    RowArgs a = {};
    a.x = x;
    a.ldx = ld_x;
    a.gamma = gamma;
    a.eps = eps;
    a.y = y;
    a.ldy = ld_y;
    a.q0 = nv_of(yq);
    a.rstd = rstd;
    a.rows = rows;
    a.cols = (int)cols;
    return launch_rows<MODE_RMS>(a, as_stream(stream));
}

extern "C" pact_status pact_silu_mul_quant_nvfp4(const uint16_t *g, int64_t ld_g,
                                                 const uint16_t *u, int64_t ld_u, int64_t rows,
                                                 int64_t cols, uint16_t *h, int64_t ld_h,
                                                 const pact_nvfp4 *hq, const pact_nvfp4 *gq,
                                                 const pact_nvfp4 *uq, void *stream) {
    PACT_TRY(check_row_len(rows, cols));
    PACT_TRY(check_bf16(g, ld_g, cols));
    PACT_TRY(check_bf16(u, ld_u, cols));
    if (h) PACT_TRY(check_bf16(h, ld_h, cols));
    PACT_TRY(check_nvfp4(hq, rows, cols));
    if (gq) PACT_TRY(check_nvfp4(gq, rows, cols));
    if (uq) PACT_TRY(check_nvfp4(uq, rows, cols));
    RowArgs a = {};
    a.x = g;
    a.ldx = ld_g;
    a.x2 = u;
    a.ldx2 = ld_u;
    a.y = h;
    a.ldy = ld_h;
    a.q0 = nv_of(hq);
    a.q1 = nv_of(gq);
    a.q2 = nv_of(uq);
    a.rows = rows;
    a.cols = (int)cols;
    return launch_rows<MODE_SILU>(a, as_stream(stream));
}

extern "C" pact_status pact_debug_sigmoid32(const uint16_t *g, float *out, int64_t n, void *stream) {
    if (n < 0 || (n > 0 && (!g || !out))) return PACT_ERR_INVALID_ARG;
    if (n == 0) return PACT_OK;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(sigmoid_probe_kernel, dim3(blocks), dim3(256), 0, as_stream(stream), g, out, n);
    return launch_status();
}

extern "C" pact_status pact_silu_mul_bwd_quant_nvfp4(const uint16_t *dh, int64_t ld_dh, const pact_nvfp4 *gq,
                                                     const pact_nvfp4 *uq, int64_t rows, int64_t cols,
                                                     uint16_t *dg, uint16_t *du, int64_t ld_out,
                                                     const pact_nvfp4 *dgq, const pact_nvfp4 *duq, void *stream) {
    PACT_TRY(check_row_len(rows, cols));
    PACT_TRY(check_bf16(dh, ld_dh, cols));
    PACT_TRY(check_nvfp4(gq, rows, cols));
    PACT_TRY(check_nvfp4(uq, rows, cols));
    if (dg) PACT_TRY(check_bf16(dg, ld_out, cols));
    if (du) PACT_TRY(check_bf16(du, ld_out, cols));
    PACT_TRY(check_nvfp4(dgq, rows, cols));
    PACT_TRY(check_nvfp4(duq, rows, cols));
    BwdArgs a = {};
    a.dy = dh;
    a.lddy = ld_dh;
    a.in0 = cnv_of(gq);
    a.in1 = cnv_of(uq);
    a.o0 = dg;
    a.o1 = du;
    a.ldo = ld_out;
    a.q0 = nv_of(dgq);
    a.q1 = nv_of(duq);
    a.rows = rows;
    a.cols = (int)cols;
    return launch_bwd<MODE_SILU_BWD>(a, as_stream(stream));
}

extern "C" pact_status pact_rmsnorm_bwd_nvfp4(const uint16_t *dy, int64_t ld_dy, const pact_nvfp4 *yq,
                                              const uint16_t *gamma, const float *rstd, const uint16_t *C,
                                              int64_t ld_c, int64_t rows, int64_t cols, uint16_t *dx,
                                              int64_t ld_dx, const pact_nvfp4 *dxq, void *stream) {
    PACT_TRY(check_row_len(rows, cols));
    PACT_TRY(check_bf16(dy, ld_dy, cols));
    PACT_TRY(check_nvfp4(yq, rows, cols));
    PACT_TRY(check_bf16(gamma, cols, cols));
    if (!rstd) return PACT_ERR_INVALID_ARG;
    if (!aligned16(rstd)) return PACT_ERR_MISALIGNED;
    if (C) PACT_TRY(check_bf16(C, ld_c, cols));
    if (dx) PACT_TRY(check_bf16(dx, ld_dx, cols));
    if (dxq) PACT_TRY(check_nvfp4(dxq, rows, cols));
    if (!dx && !dxq) return PACT_ERR_INVALID_ARG;
    BwdArgs a = {};
    a.dy = dy;
    a.lddy = ld_dy;
    a.in0 = cnv_of(yq);
    a.gamma = gamma;
    a.rstd = rstd;
    a.C = C;
    a.ldc = ld_c;
    a.o0 = dx;
    a.ldo = ld_dx;
    a.q0 = nv_of(dxq);
    a.rows = rows;
    a.cols = (int)cols;
    return launch_bwd<MODE_RMS_BWD>(a, as_stream(stream));
}

extern "C" pact_status pact_debug_dsilu32(const uint16_t *g, float *out, int64_t n, void *stream) {
    if (n < 0 || (n > 0 && (!g || !out))) return PACT_ERR_INVALID_ARG;
    if (n == 0) return PACT_OK;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(dsilu_probe_kernel, dim3(blocks), dim3(256), 0, as_stream(stream), g, out, n);
    return launch_status();
}

extern "C" pact_status pact_debug_row_plan(int32_t op, int64_t cols, int32_t *waves_per_row,
                                           int32_t *blocks_per_lane) {
    if (op < 0 || op > 4 || cols <= 0 || !waves_per_row || !blocks_per_lane) return PACT_ERR_INVALID_ARG;
    PACT_TRY(check_row_len(0, cols));
    static const int kModes[5] = {MODE_QUANT, MODE_RMS, MODE_SILU, MODE_SILU_BWD, MODE_RMS_BWD};
    int wpr, bpl;
    row_shape(kModes[op], cols / 16, wpr, bpl);
    *waves_per_row = wpr;
    *blocks_per_lane = bpl;
    return PACT_OK;
}
