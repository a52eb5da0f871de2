// pact_gemm.hip -- NVFP4 GEMM of the frozen projections on gfx950 MFMA, with
// the BF16 LoRA term in the epilogue.
//   forward: Y  = bf16(d_x d_w (Xq . W_fwd^T) + bf16(s X A^T) B^T (+ C))
//   dgrad:   dX = bf16(d_dy d_wb (dYq . W_bwd^T) + bf16(s dY B) A (+ C))
// (simolm.com PACT blog, section "Method", first bullet: NVFP4 GEMMs with FP32
// accumulation and BF16 output for the forward and the input gradient; the
// adapters stay BF16, closing paragraph of that section.)
//
// Both passes are one "TN" kernel: operand rows are K-contiguous NVFP4 rows.
// The E2M1 x E4M3 products are exact in FP16 (at most 6 significant bits,
// magnitudes in [2^-10, 2688]), so each 8-code dword is decoded with the gfx950
// FP4->FP16 converter plus one packed FP16 multiply by its block scale, and
// v_mfma_f32_32x32x16_f16 accumulates exact products in FP32.  Row scales are
// applied in the epilogue.  The summation order over K is the MFMA's own.
//
// Tiling: a workgroup of WGM x WGN wavefronts computes a BM x BN tile; each
// wavefront owns (BM/WGM) x (BN/WGN) as 32x32 fragments.  The packed NVFP4
// operands (4.5 bits per element) advance in LDS stages of 128 K-elements
// (64 code bytes + 8 scale bytes per row), brought in by direct global->LDS
// loads in which 4 lanes cover one row's 64 contiguous code bytes; two stage
// buffers alternate so a stage's loads overlap three K32 phases of MFMAs.  The
// 16-byte code pieces of a row are XOR-swizzled by row so that the decode
// reads are free of bank conflicts.  Each K32 phase is decoded once per
// workgroup (every thread one operand row) into an FP16 LDS tile laid out in
// MFMA fragment order, double-buffered: the decode of phase p+1 is interleaved
// with the MFMAs of phase p, so each wavefront reads its fragments with one
// 16-byte LDS read per fragment and K16 step.
// The LoRA-down product T = bf16(s X A^T) is a separate small kernel; the
// LoRA-up product T Q^T is accumulated by BF16 MFMAs into the row-scaled
// accumulators in the epilogue.
#include <type_traits>

#include "pact_device.h"
#include "pact_host.h"

namespace pact {

struct GemmArgs {
    const uint8_t *a_codes;
    const uint8_t *a_scales;
    const float *a_d;
    const uint8_t *b_codes;
    const uint8_t *b_scales;
    const float *b_d;
    int M, N, K;
    const uint16_t *T;  // [M][rpad] LoRA-down product (BF16, zero beyond r) or nullptr
    const uint16_t *Qs;  // LoRA-up operand: Q(n, j) = Qs[n * q_sn + j * q_sj], j < r
    int64_t q_sn, q_sj;
    int r, rpad;
    const uint16_t *C;  // nullable, leading dim ldy
    uint16_t *Y;
    int64_t ldy;
};

typedef __attribute__((address_space(3))) void lds_void_t;

// 16-byte direct global->LDS load: lane l of the wavefront writes 16 bytes at
// lds_base + 16 l (lds_base is wavefront-uniform).
__device__ __forceinline__ void load_lds16(const void *src, void *lds_base) {
    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)lds_base, 16, 0, 0);
}

// Packed FP4 dword (8 codes) -> 8 FP16 values (exact E2M1 x E4M3 products).
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

// Workgroup -> output tile.  Workgroups are dispatched round-robin over the
// 8 XCDs (each with its own L2), so consecutive tiles of the launch order are
// given to the same XCD; within an XCD's range, tiles run in groups of 4
// tile-rows x all tile-columns, so the workgroups resident together share
// A row-panels and B column-panels in that XCD's L2.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int &tm, int &tn) {
    constexpr int kXcd = 8, kGroup = 4;
    const int T = tiles_m * tiles_n;
    int t = bid;
    if (T % kXcd == 0) t = (bid % kXcd) * (T / kXcd) + bid / kXcd;
    const int per_group = kGroup * tiles_n;
    const int g = t / per_group;
    const int first_m = g * kGroup;
    const int gsize = min(tiles_m - first_m, kGroup);
    const int r = t - g * per_group;
    tm = first_m + r % gsize;
    tn = r / gsize;
}

// LDS layout (ROWS = BM + BN rows: the A tile's rows, then the B tile's):
//   P[2]  packed stages of 128 K-elements:
//         codes  [ROWS][64 B], the four 16-byte pieces of a row stored in
//                XOR-swizzled order (slot p of row r holds piece p ^ (r & 3));
//         scales [ROWS][8 B], the row's 8 E4M3 block scales of the stage;
//   F[2]  FP16 phases of 32 K-elements in MFMA fragment order: for row group
//         g (32 rows) and K16 step s, 64 lanes x 16 bytes, lane (r, h) holding
//         K [16 s + 8 h, 16 s + 8 h + 8) of row r.
// Global -> P: direct 16-byte loads, 4 lanes per row (64 contiguous bytes)
// for codes, one 4-byte load per lane for scales.  P -> F: every thread owns
// one row and decodes its 32 elements of the next phase (4 dwords: 4 FP4->FP16
// converts and 4 packed FP16 multiplies each) while the MFMAs of the current
// phase run; the wavefronts then read their fragments from F.
template <int BM, int BN, int WGM, int WGN, bool KFULL>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_kernel(GemmArgs p) {
    constexpr int NW = WGM * WGN;
    constexpr int NT = 64 * NW;
    constexpr int FM = BM / WGM / 32;  // 32x32 fragments per wave along M
    constexpr int FN = BN / WGN / 32;
    constexpr int ROWS = BM + BN;
    static_assert(ROWS == NT, "one decoded row per thread");
    static_assert(BM % 32 == 0 && BN % 32 == 0 && FM >= 1 && FN >= 1, "unsupported tile");
    constexpr int PK = 128;                   // K per packed stage
    constexpr int PCODE = ROWS * 64;
    constexpr int PSTAGE = ROWS * 72;
    constexpr int FPH = ROWS * 64;            // FP16 phase: ROWS x 32 x 2 B
    constexpr int N_CODE_I = ROWS / 16;       // direct loads per packed stage
    constexpr int N_SC_I = ROWS / 32;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * PSTAGE + 2 * FPH];
    uint8_t *const P0 = lds;
    uint8_t *const F0 = lds + 2 * PSTAGE;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = p.K;
    const int nblk = K >> 4;
    const int nst = (K + PK - 1) / PK;  // packed stages
    const int nph = 4 * nst;            // FP16 phases (K32 each)

    float16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // global row of tile row rr (rows past the end are clamped: their results
    // are never stored)
    // kernel arguments in registers (the lambdas below must not reload them)
    const uint8_t *const a_codes = p.a_codes;
    const uint8_t *const a_scales = p.a_scales;
    const uint8_t *const b_codes = p.b_codes;
    const uint8_t *const b_scales = p.b_scales;
    const int Mrows = p.M, Nrows = p.N;
    auto row_src = [=](int rr, const uint8_t *&codes, const uint8_t *&scales, int &grow) {
        if (rr < BM) {
            codes = a_codes;
            scales = a_scales;
            grow = min(m0 + rr, Mrows - 1);
        } else {
            codes = b_codes;
            scales = b_scales;
            grow = min(n0 + rr - BM, Nrows - 1);
        }
    };

    auto issue_stage = [&](int st, uint8_t *buf) {
        const int k0 = st * PK;
        for (int i = wave; i < N_CODE_I + N_SC_I; i += NW) {
            const uint8_t *codes, *scales;
            int grow;
            if (i < N_CODE_I) {
                const int rr = 16 * i + (lane >> 2);
                row_src(rr, codes, scales, grow);
                const int g = (lane & 3) ^ (rr & 3);  // global piece stored in this slot
                const uint8_t *src = codes + (int64_t)grow * (K >> 1) + (k0 >> 1) + 16 * g;
                uint8_t *dst = buf + 16 * i * 64;
                if (KFULL) {
                    load_lds16(src, dst);
                } else {
                    u32x4 v = {0u, 0u, 0u, 0u};
                    const int kk = k0 + 32 * g;
                    if (kk < K) {
                        const u32x2 lo = *reinterpret_cast<const u32x2 *>(src);
                        v.x = lo.x;
                        v.y = lo.y;
                    }
                    if (kk + 16 < K) {
                        const u32x2 hi = *reinterpret_cast<const u32x2 *>(src + 8);
                        v.z = hi.x;
                        v.w = hi.y;
                    }
                    *reinterpret_cast<u32x4 *>(dst + 16 * lane) = v;
                }
            } else {
                const int j = i - N_CODE_I;
                const int rr = 32 * j + (lane >> 1);
                row_src(rr, codes, scales, grow);
                const uint8_t *src = scales + (int64_t)grow * nblk + (k0 >> 4) + 4 * (lane & 1);
                uint8_t *dst = buf + PCODE + 32 * j * 8;
                if (KFULL) {
                    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)dst, 4, 0, 0);
                } else {
                    uint32_t w = 0u;
                    for (int b = 0; b < 4; ++b)
                        if ((k0 >> 4) + 4 * (lane & 1) + b < nblk) w |= (uint32_t)src[b] << (8 * b);
                    *reinterpret_cast<uint32_t *>(dst + 4 * lane) = w;
                }
            }
        }
    };

    // decode of phase ph: this thread's row (tid) -> F[ph & 1]
    const int drow = tid;
    const int dgrp = drow >> 5, dlr = drow & 31;
    uint8_t *const fbase_w = F0 + (((dgrp * 2) * 64 + dlr) << 4);
    u32x4 pcodes;
    uint32_t pscale;
    auto read_packed = [&](int ph) {
        const uint8_t *pb = P0 + ((ph >> 2) & 1) * PSTAGE;
        const int j = ph & 3;
        pcodes = *reinterpret_cast<const u32x4 *>(pb + drow * 64 + ((j ^ (drow & 3)) << 4));
        pscale = *reinterpret_cast<const uint16_t *>(pb + PCODE + drow * 8 + 2 * j);
    };
    auto decode_dword = [&](int ph, int d, half2_t sp) {
        const uint32_t w = d == 0 ? pcodes.x : d == 1 ? pcodes.y : d == 2 ? pcodes.z : pcodes.w;
        half2_t sc;
        sc[0] = sp[d >> 1];
        sc[1] = sp[d >> 1];
        const half8_t v = decode8(w, sc);
        // step s = d >> 1, lane half h = d & 1
        *reinterpret_cast<half8_t *>(fbase_w + (ph & 1) * FPH + (((d >> 1) * 64 + 32 * (d & 1)) << 4)) = v;
    };

    auto read_a = [&](int ph, int s, int f) {
        return *reinterpret_cast<const half8_t *>(F0 + (ph & 1) * FPH + ((((wm * FM + f) * 2 + s) * 64 + lane) << 4));
    };
    auto read_b = [&](int ph, int s, int f) {
        return *reinterpret_cast<const half8_t *>(
            F0 + (ph & 1) * FPH + ((((BM / 32 + wn * FN + f) * 2 + s) * 64 + lane) << 4));
    };

    if (nph > 0) {
        issue_stage(0, P0);
        if (nst > 1) issue_stage(1, P0 + PSTAGE);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        read_packed(0);
        const half2_t sp = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(pscale, 1.0f, false);
#pragma unroll
        for (int d = 0; d < 4; ++d) decode_dword(0, d, sp);
    }
    __syncthreads();

    // Phase loop.  The decode of phase ph+1 is unconditional (after the last
    // phase it decodes stale LDS into the unused buffer, harmlessly), so each
    // K16 step is one basic block in which scheduling groups interleave every
    // MFMA with a slice of the decode VALU and the LDS traffic.
    for (int ph = 0; ph < nph; ++ph) {
        if ((ph & 3) == 0 && ph > 0 && (ph >> 2) + 1 < nst)
            issue_stage((ph >> 2) + 1, P0 + (((ph >> 2) + 1) & 1) * PSTAGE);
        read_packed(ph + 1);
        half8_t av[FM], bv[FN];
#pragma unroll
        for (int f = 0; f < FM; ++f) av[f] = read_a(ph, 0, f);
#pragma unroll
        for (int f = 0; f < FN; ++f) bv[f] = read_b(ph, 0, f);
        const half2_t sp = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(pscale, 1.0f, false);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            half8_t an[FM], bn[FN];
            if (s == 0) {
#pragma unroll
                for (int f = 0; f < FM; ++f) an[f] = read_a(ph, 1, f);
#pragma unroll
                for (int f = 0; f < FN; ++f) bn[f] = read_b(ph, 1, f);
            }
            decode_dword(ph + 1, 2 * s, sp);
            decode_dword(ph + 1, 2 * s + 1, sp);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[fm], bv[fn], acc[fm][fn], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < FM * FN; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // 2 VALU
                if (i % 4 == 1) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // 1 LDS write
                if (s == 0 && i < FM + FN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
            }
            if (s == 0) {
#pragma unroll
                for (int f = 0; f < FM; ++f) av[f] = an[f];
#pragma unroll
                for (int f = 0; f < FN; ++f) bv[f] = bn[f];
            }
        }
        if ((ph & 3) == 2) __builtin_amdgcn_s_waitcnt(0);  // stage (ph >> 2) + 1 has landed
        __syncthreads();
    }

    // ---- epilogue: row scales, LoRA term, residual, BF16 store ----
    const int h = lane >> 5;
    // Per fragment: y = fl32(fl32(acc d_a[m]) d_b[n]) in place, then the LoRA
    // term T_s . Q^T (T_s = bf16(s . X P^T) from the down kernel) is accumulated
    // into y by one BF16 MFMA per 16 ranks, then C is added and y rounded.
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int mb = m0 + (wm * FM + fm) * 32;
        float dxv[16];
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const int m = mb + 8 * e4 + 4 * h;
            if (m + 3 < p.M) {
                const float4_t v = *reinterpret_cast<const float4_t *>(p.a_d + m);
                dxv[4 * e4] = v[0];
                dxv[4 * e4 + 1] = v[1];
                dxv[4 * e4 + 2] = v[2];
                dxv[4 * e4 + 3] = v[3];
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) dxv[4 * e4 + q] = m + q < p.M ? p.a_d[m + q] : 0.0f;
            }
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int nb = n0 + (wn * FN + fn) * 32;
            const int n = nb + (lane & 31);
            const float dw = n < p.N ? p.b_d[n] : 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float y = acc[fm][fn][e] * dxv[e];
                acc[fm][fn][e] = y * dw;
            }
            if (p.T) {
                const int mr = min(mb + (lane & 31), p.M - 1);
                const int nr = min(n, p.N - 1);
                for (int kk = 0; kk < p.rpad; kk += 16) {
                    const u32x4 va = *reinterpret_cast<const u32x4 *>(p.T + (int64_t)mr * p.rpad + kk + 8 * h);
                    u32x4 vb;
                    const int j0 = kk + 8 * h;
                    if (p.q_sj == 1 && (p.r & 7) == 0) {
                        vb = u32x4{0u, 0u, 0u, 0u};
                        if (j0 < p.r) vb = *reinterpret_cast<const u32x4 *>(p.Qs + (int64_t)nr * p.q_sn + j0);
                    } else {
                        uint32_t w[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int ja = j0 + 2 * e, jb = ja + 1;
                            const uint32_t lo = ja < p.r ? p.Qs[(int64_t)nr * p.q_sn + (int64_t)ja * p.q_sj] : 0u;
                            const uint32_t hi = jb < p.r ? p.Qs[(int64_t)nr * p.q_sn + (int64_t)jb * p.q_sj] : 0u;
                            w[e] = lo | (hi << 16);
                        }
                        vb = u32x4{w[0], w[1], w[2], w[3]};
                    }
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8_t, va), __builtin_bit_cast(bf16x8_t, vb), acc[fm][fn], 0, 0, 0);
                }
            }
            if (n >= p.N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = mb + 8 * (e >> 2) + 4 * h + (e & 3);
                if (m >= p.M) continue;
                float y = acc[fm][fn][e];
                const int64_t off = (int64_t)m * p.ldy + n;
                if (p.C) y = y + bf16_to_f32(p.C[off]);
                p.Y[off] = (uint16_t)f32_to_bf16_bits(y);
            }
        }
    }
}

// ---- LoRA down-projection --------------------------------------------------
// T [M][rpad] = bf16(s . (Xl [M][Kl] . P^T)), P(j, k) = Ps[j p_sj + k p_sk] for
// j < r, zero for r <= j < rpad; FP32 accumulation on v_mfma_f32_16x16x32_bf16.
// The LoRA scale s is applied before the BF16 rounding; for a power-of-two s
// this equals s . bf16(X P^T) exactly, i.e. the scale applied after the
// rank-r product.
// One workgroup of 16 wavefronts per 16 rows: each wavefront takes a slice of
// K, and the 16 partial tiles are summed through LDS in a fixed order.
constexpr int kDownWaves = 16;

__global__ __launch_bounds__(1024) void lora_down_kernel(const uint16_t *X, int64_t ldx, int M, int Kl,
                                                         const uint16_t *Ps, int64_t p_sj, int64_t p_sk,
                                                         int r, int rpad, float scale, uint16_t *T) {
    __shared__ float red[kDownWaves][16][17];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int m0 = blockIdx.x * 16;
    const int row = min(m0 + (lane & 15), M - 1);
    const int kg = 8 * (lane >> 4);
    const int ks = ((Kl + kDownWaves - 1) / kDownWaves + 31) / 32 * 32;
    const int kb = w * ks, ke = min(Kl, kb + ks);
    for (int f = 0; f < rpad / 16; ++f) {
        const int j = 16 * f + (lane & 15);
        float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int k0 = kb; k0 < ke; k0 += 32) {
            const int k = k0 + kg;
            u32x4 va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
            if (k < ke) {
                va = *reinterpret_cast<const u32x4 *>(X + (int64_t)row * ldx + k);
                if (j < r) {
                    if (p_sk == 1) {
                        vb = *reinterpret_cast<const u32x4 *>(Ps + (int64_t)j * p_sj + k);
                    } else {
                        uint32_t t[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            t[e] = (uint32_t)Ps[(int64_t)j * p_sj + (int64_t)(k + 2 * e) * p_sk] |
                                   ((uint32_t)Ps[(int64_t)j * p_sj + (int64_t)(k + 2 * e + 1) * p_sk] << 16);
                        vb = u32x4{t[0], t[1], t[2], t[3]};
                    }
                }
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va),
                                                          __builtin_bit_cast(bf16x8_t, vb), acc, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) red[w][4 * (lane >> 4) + e][lane & 15] = acc[e];
        __syncthreads();
        if (threadIdx.x < 256) {
            const int mi = threadIdx.x >> 4, ji = threadIdx.x & 15;
            float sum = 0.0f;
            for (int q = 0; q < kDownWaves; ++q) sum += red[q][mi][ji];
            const float ts = scale * sum;
            if (m0 + mi < M) T[(int64_t)(m0 + mi) * rpad + 16 * f + ji] = (uint16_t)f32_to_bf16_bits(ts);
        }
        __syncthreads();
    }
}

size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, int32_t r) {
    (void)N;
    (void)K;
    if (r <= 0) return 0;
    const int64_t rpad = round_up(r, 16);
    return (size_t)round_up(M * rpad * 2, 256);
}

template <int BM, int BN, int WGM, int WGN>
static void launch_gemm_cfg(const GemmArgs &a, hipStream_t st) {
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    const dim3 block(64 * WGM * WGN);
    if (a.K % 128 == 0)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WGM, WGN, true>), dim3(tiles), block, 0, st, a);
    else
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WGM, WGN, false>), dim3(tiles), block, 0, st, a);
}

static pact_status run_gemm(const GemmArgs &a, hipStream_t st) {
    auto tiles = [&](int bm, int bn) {
        return (int64_t)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
    };
    if (tiles(256, 256) >= 192) launch_gemm_cfg<256, 256, 2, 4>(a, st);
    else launch_gemm_cfg<128, 128, 2, 2>(a, st);
    return launch_status();
}

// Shared body of the forward and input-gradient entry points.
//   aq [M][Kc] NVFP4, bq [Nout][Kc] NVFP4, Xl [M][Kl] BF16 LoRA input,
//   P(j, k) = Psrc[j p_sj + k p_sk] (j < r, k < Kl), Q(n, j) = Qsrc[n q_sn + j q_sj].
static pact_status gemm_common(const pact_nvfp4 *aq, const pact_nvfp4 *bq, const uint16_t *Xl,
                               int64_t ldx, int64_t Kl, const pact_lora *lora, const uint16_t *Psrc,
                               int64_t p_sj, int64_t p_sk, const uint16_t *Qsrc, int64_t q_sn,
                               int64_t q_sj, const uint16_t *C, uint16_t *Y, int64_t ldy, void *ws,
                               size_t ws_bytes, void *stream) {
    if (!aq || !bq) return PACT_ERR_INVALID_ARG;
    const int64_t M = aq->rows, Kc = aq->cols, Nout = bq->rows;
    if (M < 0 || Kc < 0 || Nout < 0 || bq->cols != Kc) return PACT_ERR_INVALID_ARG;
    if (Kc % 16 != 0) return PACT_ERR_UNSUPPORTED_SHAPE;
    if (M > INT32_MAX || Nout > INT32_MAX || Kc > INT32_MAX) return PACT_ERR_UNSUPPORTED_SHAPE;
    PACT_TRY(check_nvfp4(aq, M, Kc));
    PACT_TRY(check_nvfp4(bq, Nout, Kc));
    PACT_TRY(check_bf16(Y, ldy, Nout));
    if (C) PACT_TRY(check_bf16(C, ldy, Nout));
    const int r = lora ? lora->r : 0;
    if (r < 0 || r > 256) return PACT_ERR_INVALID_ARG;
    if (r > 0) {
        if (!lora->A || !lora->B) return PACT_ERR_INVALID_ARG;
        if (!aligned16(lora->A) || !aligned16(lora->B)) return PACT_ERR_MISALIGNED;
        PACT_TRY(check_bf16(Xl, ldx, Kl));
    }
    if (M == 0 || Nout == 0) return PACT_OK;
    hipStream_t st = as_stream(stream);
    GemmArgs a = {};
    a.a_codes = aq->codes;
    a.a_scales = aq->scales;
    a.a_d = aq->row_scale;
    a.b_codes = bq->codes;
    a.b_scales = bq->scales;
    a.b_d = bq->row_scale;
    a.M = (int)M;
    a.N = (int)Nout;
    a.K = (int)Kc;
    a.C = C;
    a.Y = Y;
    a.ldy = ldy;
    if (r > 0) {
        const int rpad = (int)round_up(r, 16);
        const size_t need = gemm_ws_bytes(M, Nout, Kl, r);
        if (!ws || ws_bytes < need) return PACT_ERR_WORKSPACE;
        if (!aligned16(ws)) return PACT_ERR_MISALIGNED;
        uint16_t *T = static_cast<uint16_t *>(ws);
        hipLaunchKernelGGL(lora_down_kernel, dim3((unsigned)((M + 15) / 16)), dim3(64 * kDownWaves), 0, st,
                           Xl, ldx, (int)M, (int)Kl, Psrc, p_sj, p_sk, r, rpad, lora->scale, T);
        PACT_TRY(launch_status());
        a.T = T;
        a.Qs = Qsrc;
        a.q_sn = q_sn;
        a.q_sj = q_sj;
        a.r = r;
        a.rpad = rpad;
    }
    return run_gemm(a, st);
}

}  // namespace pact

using namespace pact;

extern "C" size_t pact_gemm_workspace(int64_t M, int64_t N, int64_t K, int32_t r) {
    if (M < 0 || N < 0 || K < 0) return 0;
    return gemm_ws_bytes(M, N, K, r);
}

extern "C" pact_status pact_gemm_nvfp4_fwd(const pact_nvfp4 *Xq, const uint16_t *X, int64_t ld_x,
                                           const pact_nvfp4 *W_fwd, const pact_lora *lora,
                                           const uint16_t *C, uint16_t *Y, int64_t ld_y, void *ws,
                                           size_t ws_bytes, void *stream) {
    if (!Xq || !W_fwd) return PACT_ERR_INVALID_ARG;
    const int64_t K = Xq->cols, N = W_fwd->rows;
    const int r = lora ? lora->r : 0;
    // T = X A^T: P(j, k) = A[j K + k];  L = T B^T: Q(n, j) = B[n r + j]
    return gemm_common(Xq, W_fwd, X, ld_x, K, lora, lora ? lora->A : nullptr, K, 1,
                       lora ? lora->B : nullptr, r, 1, C, Y, ld_y, ws, ws_bytes, stream);
    (void)N;
}

extern "C" pact_status pact_gemm_nvfp4_dgrad(const pact_nvfp4 *dYq, const uint16_t *dY,
                                             int64_t ld_dy, const pact_nvfp4 *W_bwd,
                                             const pact_lora *lora, const uint16_t *C, uint16_t *dX,
                                             int64_t ld_dx, void *ws, size_t ws_bytes, void *stream) {
    if (!dYq || !W_bwd) return PACT_ERR_INVALID_ARG;
    const int64_t N = dYq->cols, K = W_bwd->rows;
    const int r = lora ? lora->r : 0;
    // T' = dY B: P(j, n) = B[n r + j];  L' = T' A: Q(k, j) = A[j K + k]
    return gemm_common(dYq, W_bwd, dY, ld_dy, N, lora, lora ? lora->B : nullptr, 1, r,
                       lora ? lora->A : nullptr, 1, K, C, dX, ld_dx, ws, ws_bytes, stream);
}
