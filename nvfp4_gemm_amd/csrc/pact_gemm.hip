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
#include <algorithm>
#include <mutex>
#include <type_traits>
#include <utility>

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
    uint32_t a_bytes, b_bytes;  // code bytes of the A and B operands (below 4 GiB)
    const uint16_t *T;  // [M][rpad] LoRA-down product (BF16, zero beyond r) or nullptr
    const uint16_t *Qs;  // LoRA-up operand: Q(n, j) = Qs[n * q_sn + j * q_sj], j < r
    int64_t q_sn, q_sj;
    int r, rpad;
    int tld;  // row stride of T (rpad, or ngroups * rpad when grouped)
    // grouped (block-diagonal) LoRA, ngroups > 1: output columns [gcol[g],
    // gcol[g + 1]) use ranks [g rpad, g rpad + r) of T and Q(n, j) =
    // Qg[g][(n - gcol[g]) q_sn + j] (q_sj == 1); group boundaries are
    // multiples of 32, so every 32-column fragment lies in one group
    int ngroups;
    int gcol[kMaxGroups + 1];
    const uint16_t *Qg[kMaxGroups];
    const uint16_t *C;  // nullable, leading dim ldy
    uint16_t *Y;
    int64_t ldy;
    uint32_t y_rec;  // M * ldy * 2 when below 2^31 (Y and C then go through buffer descriptors), else 0
    int ks;       // K ranges split across workgroups (blockIdx.y); 1: no split
    float *part;  // ks > 1: FP32 partial fragments [ks][ceil(M/32)][ceil(N/32)][1024]
    DownArgs down;  // ks > 1 and down.X: the LoRA-down runs as workgroups blockIdx.y == 0
};

// The GemmArgs argument of a kernel, read in place from the kernel-argument
// segment, where it is the first (and only) explicit argument, at offset 0.
// Referring to the by-value parameter itself lets the compiler copy the
// struct into private memory when it cannot resolve every use (dynamically
// indexed members), and the values loaded back from there count as
// divergent: buffer descriptors end up in VGPRs and every buffer access
// becomes a read-first-lane loop.  Read through this reference, every field
// is a scalar load.
__device__ __forceinline__ const GemmArgs &kernel_gemm_args() {
    return *(const GemmArgs *)(const __attribute__((address_space(4))) GemmArgs *)
        __builtin_amdgcn_kernarg_segment_ptr();
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Word 3 of the buffer resource descriptors (raw buffer access).
constexpr int kRsrcWord3 = 0x00020000;

// 16-byte direct global->LDS load: lane l of the wavefront writes 16 bytes at
// lds_base + 16 l (lds_base is wavefront-uniform).
__device__ __forceinline__ void load_lds16(const void *src, void *lds_base) {
    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)lds_base, 16, 0, 0);
}

// Workgroup barrier ordering LDS only: waits for this wavefront's own LDS
// operations, not for its outstanding global loads (__syncthreads would also
// wait for those, exposing the latency of the stage loads in flight).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Waits until this wavefront's global loads, including the direct-to-LDS
// loads of a stage, have completed.
__device__ __forceinline__ void wait_global_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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

// Epilogue of 32x32 accumulator fragments whose rows start at mb and columns
// at nb: y = fl32(fl32(acc d_a[m]) d_b[n]), then the LoRA term T_s.Q^T
// (T_s = bf16(s . X P^T) from the down kernel) is accumulated into y by one
// BF16 MFMA per 16 ranks (all in the MFMA accumulator layout, lane = column).
// Then a group of horizontally adjacent fragments goes through a per-wavefront
// LDS tile to row-major order, where C is added and y is rounded to BF16, so
// that C is read and Y written in 16-byte chunks of 8 columns (8 lanes cover
// 128 contiguous bytes of a row) instead of 2-byte accesses.
// LoRA-up operands of the fragment at columns nb..nb+31: its T column offset
// and the Q row of column n (clamped to the output).
struct EpiLora {
    const uint16_t *T;   // row mr of T at the group's first rank
    const uint16_t *Q;   // Q row of the lane's column (its first rank)
};

__device__ __forceinline__ EpiLora epi_lora(const GemmArgs &p, int mb, int nb, int lane) {
    const int lr = lane & 31;
    const int mr = min(mb + lr, p.M - 1);
    const int nr = min(nb + lr, p.N - 1);
    int g = 0;
#pragma unroll
    for (int i = 1; i < kMaxGroups; ++i)
        if (i < p.ngroups && nb >= p.gcol[i]) g = i;
    EpiLora L;
    L.T = p.T + (int64_t)mr * p.tld + g * p.rpad;
    L.Q = p.ngroups > 1 ? p.Qg[g] + (int64_t)(nr - p.gcol[g]) * p.q_sn : p.Qs + (int64_t)nr * p.q_sn;
    return L;
}

struct EpiIn {
    float dw;        // d_b of the lane's column
    u32x4 t[2], q[2];  // LoRA operands, ranks [0, 32) (prefetched when rpad <= 32)
};

// d_a of the lane's 16 rows of the fragments whose rows start at mb (shared
// by the horizontally adjacent fragments of an epilogue group).
__device__ __forceinline__ void epi_load_dx(const GemmArgs &p, int mb, int lane, float (&dx)[16]) {
    const int h = lane >> 5;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
        const int m = mb + 8 * e4 + 4 * h;
        if (m + 3 < p.M) {
            const float4_t v = *reinterpret_cast<const float4_t *>(p.a_d + m);
#pragma unroll
            for (int q = 0; q < 4; ++q) dx[4 * e4 + q] = v[q];
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) dx[4 * e4 + q] = m + q < p.M ? p.a_d[m + q] : 0.0f;
        }
    }
}

__device__ __forceinline__ bool epi_lora_prefetch(const GemmArgs &p) {
    return p.T && p.rpad <= 32 && p.q_sj == 1 && (p.r & 7) == 0;
}

// The prefetched LoRA operands are read through buffer descriptors (base in
// scalar registers, 32-bit offsets, in range by construction: clamped rows).
__device__ __forceinline__ void epi_load(const GemmArgs &p, int mb, int nb, int lane, EpiIn &in) {
    const int h = lane >> 5, lr = lane & 31;
    const int n = nb + lr;
    in.dw = n < p.N ? p.b_d[n] : 0.0f;
    if (epi_lora_prefetch(p)) {
        const int mr = min(mb + lr, p.M - 1);
        const int nr = min(n, p.N - 1);
        int g = 0;
#pragma unroll
        for (int i = 1; i < kMaxGroups; ++i)
            if (i < p.ngroups && nb >= p.gcol[i]) g = i;
        const uint16_t *qb = p.ngroups > 1 ? p.Qg[g] : p.Qs;
        const int qrow = p.ngroups > 1 ? nr - p.gcol[g] : nr;
        const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc((void *)p.T, (short)0, 0x7FFFFFFF, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void *)qb, (short)0, 0x7FFFFFFF, kRsrcWord3);
        const int toff = 2 * (mr * p.tld + g * p.rpad);
        const int qoff = 2 * (qrow * (int)p.q_sn);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int j0 = 16 * i + 8 * h;
            in.t[i] = u32x4{0u, 0u, 0u, 0u};
            in.q[i] = u32x4{0u, 0u, 0u, 0u};
            if (16 * i < p.rpad) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(rt, toff + 2 * j0, 0, 0);
                in.t[i] = u32x4{v[0], v[1], v[2], v[3]};
            }
            if (j0 < p.r) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + 2 * j0, 0, 0);
                in.q[i] = u32x4{v[0], v[1], v[2], v[3]};
            }
        }
    }
}

// Row scales and LoRA term, in place, in the accumulator layout:
// y = fl32(fl32(acc d_a) d_b), then + L with L = T_s . Q^T accumulated by
// BF16 MFMAs (lane = column).  L is accumulated from zero in registers of
// its own: accumulating it into the GEMM's accumulator ties the MFMA to
// those registers and makes the compiler spill around it.
__device__ __forceinline__ void epi_finish(const GemmArgs &p, float16_t &a, int mb, int nb, int lane,
                                           const EpiIn &in, const float (&dx)[16]) {
    const int h = lane >> 5;
    float16_t lo;
#pragma unroll
    for (int e = 0; e < 16; ++e) lo[e] = 0.0f;
    if (epi_lora_prefetch(p)) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            if (16 * i < p.rpad)
                lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, in.t[i]),
                                                             __builtin_bit_cast(bf16x8_t, in.q[i]), lo, 0, 0, 0);
    } else if (p.T) {
        const EpiLora L = epi_lora(p, mb, nb, lane);
        for (int kk = 0; kk < p.rpad; kk += 16) {
            const u32x4 va = *reinterpret_cast<const u32x4 *>(L.T + kk + 8 * h);
            u32x4 vb;
            const int j0 = kk + 8 * h;
            if (p.q_sj == 1 && (p.r & 7) == 0) {
                vb = u32x4{0u, 0u, 0u, 0u};
                if (j0 < p.r) vb = *reinterpret_cast<const u32x4 *>(L.Q + j0);
            } else {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int ja = j0 + 2 * e, jb = ja + 1;
                    const uint32_t lw = ja < p.r ? L.Q[(int64_t)ja * p.q_sj] : 0u;
                    const uint32_t hw = jb < p.r ? L.Q[(int64_t)jb * p.q_sj] : 0u;
                    w[e] = lw | (hw << 16);
                }
                vb = u32x4{w[0], w[1], w[2], w[3]};
            }
            lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va),
                                                         __builtin_bit_cast(bf16x8_t, vb), lo, 0, 0, 0);
        }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const float y = a[e] * dx[e];
        a[e] = y * in.dw;
    }
    if (p.T) {
#pragma unroll
        for (int e = 0; e < 16; ++e) a[e] = a[e] + lo[e];
    }
}

// Per-wavefront LDS tile of G adjacent fragments: 32 rows of 32 G FP32 plus 4
// of padding (lanes 32-63 of an accumulator store land 16 banks away).
template <int G>
constexpr int epi_tile_stride() { return 32 * G + 4; }
template <int G>
constexpr int epi_tile_floats() { return 32 * epi_tile_stride<G>(); }

// Fragment i of the group into the tile: element e of lane (h, lr) is row
// 8 (e / 4) + 4 h + e % 4, column 32 i + lr.
template <int G>
__device__ __forceinline__ void epi_to_tile(float *tile, const float16_t &a, int i, int lane) {
    const int h = lane >> 5, lr = lane & 31;
#pragma unroll
    for (int e = 0; e < 16; ++e)
        tile[(8 * (e >> 2) + 4 * h + (e & 3)) * epi_tile_stride<G>() + 32 * i + lr] = a[e];
}

// Row-major pass over the tile (rows mb.., columns nb0 .. nb0 + 32 G): lane l
// takes columns 8 (l % 4G) .. +8 of rows l / 4G + 16/G q; C is loaded for all
// of its rows first, then y = bf16(tile + C) is stored 16 bytes at a time.
template <int G>
__device__ __forceinline__ void epi_rows(const GemmArgs &p, int lane, const float *tile, int mb, int nb0,
                                         bool have_c = false, const u32x4 *cpre = nullptr) {
    constexpr int LPR = 4 * G;      // lanes per row
    constexpr int RPI = 64 / LPR;   // rows per instruction
    constexpr int NQ = 32 / RPI;    // row steps
    const int rr = lane / LPR, c = 8 * (lane % LPR);
    const int n = nb0 + c;
    const bool full = n + 8 <= p.N;
    // y = bf16(tile + C) for the 8 columns of row `row` (tile row), C words cw
    auto finish8 = [&](int row, const u32x4 &cq, uint32_t o[4]) {
        const float4_t v0 = *reinterpret_cast<const float4_t *>(tile + row * epi_tile_stride<G>() + c);
        const float4_t v1 = *reinterpret_cast<const float4_t *>(tile + row * epi_tile_stride<G>() + c + 4);
        float y[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        if (p.C) {
            const uint32_t cw[4] = {cq.x, cq.y, cq.z, cq.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) y[j] = y[j] + ((j & 1) ? bf16_hi(cw[j >> 1]) : bf16_lo(cw[j >> 1]));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = f32_to_bf16_bits(y[2 * j]) | (f32_to_bf16_bits(y[2 * j + 1]) << 16);
    };
    u32x4 cv[NQ];
    if (full && p.y_rec) {
        // 32-bit offsets into buffer descriptors of Y and C: rows at or past M
        // lie beyond the descriptor's records, so their loads read zero and
        // their stores are dropped, with no per-row address arithmetic or test
        const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc((void *)p.Y, (short)0, (int)p.y_rec,
                                                                           kRsrcWord3);
        const uint32_t off0 = ((uint32_t)(mb + rr) * (uint32_t)p.ldy + (uint32_t)n) * 2u;
        const uint32_t step = (uint32_t)RPI * (uint32_t)p.ldy * 2u;
        if (p.C) {
            const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc((void *)p.C, (short)0,
                                                                               (int)p.y_rec, kRsrcWord3);
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                if (have_c) {
                    cv[q] = cpre[q];
                } else {
                    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(off0 + (uint32_t)q * step), 0, 0);
                    cv[q] = u32x4{v[0], v[1], v[2], v[3]};
                }
            }
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            uint32_t o[4];
            finish8(RPI * q + rr, p.C ? cv[q] : u32x4{0u, 0u, 0u, 0u}, o);
            typedef unsigned int u4_t __attribute__((ext_vector_type(4)));
            __builtin_amdgcn_raw_buffer_store_b128(u4_t{o[0], o[1], o[2], o[3]}, ry, (int)(off0 + (uint32_t)q * step),
                                                   0, 0);
        }
        return;
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int m = mb + RPI * q + rr;
        cv[q] = u32x4{0u, 0u, 0u, 0u};
        if (p.C && m < p.M) {
            const uint16_t *src = p.C + (int64_t)m * p.ldy + n;
            if (full) {
                cv[q] = *reinterpret_cast<const u32x4 *>(src);
            } else {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (n + j < p.N) w[j >> 1] |= (uint32_t)src[j] << (16 * (j & 1));
                cv[q] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int row = RPI * q + rr;
        const int m = mb + row;
        if (m >= p.M) continue;
        uint32_t o[4];
        finish8(row, cv[q], o);
        uint16_t *dst = p.Y + (int64_t)m * p.ldy + n;
        if (full) {
            *reinterpret_cast<u32x4 *>(dst) = u32x4{o[0], o[1], o[2], o[3]};
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (n + j < p.N) dst[j] = (uint16_t)(o[j >> 1] >> (16 * (j & 1)));
        }
    }
}

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1 (indices known at
// compile time, so register arrays indexed by them stay in registers).
template <typename Fn, int... I>
__device__ __forceinline__ void static_for_impl(Fn &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Epilogue of F fragments in groups of G horizontally adjacent fragments
// (mb[g + i] = mb[g], nb[g + i] = nb[g] + 32 i): the loads of a group are
// issued together, its fragments finished and written to the wavefront's LDS
// tile (epi_tile_floats<G>() floats, not shared with other wavefronts), then
// the group is stored row by row.  accf(I) returns fragment I.
// The C words epi_rows<G> reads on its buffer-descriptor path, loaded ahead
// of it; false (nothing loaded) for lanes that take the other path.
template <int G>
__device__ __forceinline__ bool epi_c_prefetch(const GemmArgs &p, int lane, int mb, int nb0, u32x4 (&cv)[2 * G]) {
    constexpr int LPR = 4 * G, RPI = 64 / LPR, NQ = 32 / RPI;
    static_assert(NQ == 2 * G, "row steps");
    const int rr = lane / LPR, n = nb0 + 8 * (lane % LPR);
    if (!p.C || !p.y_rec || n + 8 > p.N) return false;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc((void *)p.C, (short)0, (int)p.y_rec,
                                                                       kRsrcWord3);
    const uint32_t off0 = ((uint32_t)(mb + rr) * (uint32_t)p.ldy + (uint32_t)n) * 2u;
    const uint32_t step = (uint32_t)RPI * (uint32_t)p.ldy * 2u;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(off0 + (uint32_t)q * step), 0, 0);
        cv[q] = u32x4{v[0], v[1], v[2], v[3]};
    }
    return true;
}

template <int F, int G, typename AccFn>
__device__ __forceinline__ void epi_frags(const GemmArgs &p, int lane, AccFn &&accf, const int (&mb)[F],
                                          const int (&nb)[F], float *tile) {
    static_assert(F % G == 0, "whole groups");
    static_for<F / G>([&](auto gc) {
        constexpr int g = decltype(gc)::value * G;
        EpiIn in[G];
        float dx[16];
        epi_load_dx(p, mb[g], lane, dx);
        static_for<G>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            epi_load(p, mb[g + i], nb[g + i], lane, in[i]);
        });
        static_for<G>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            float16_t &a = accf(std::integral_constant<int, g + i>{});
            epi_finish(p, a, mb[g + i], nb[g + i], lane, in[i], dx);
            epi_to_tile<G>(tile, a, i, lane);
        });
        // LDS operations of one wavefront complete in order; the wait keeps
        // the compiler from treating the tile reads as independent
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        epi_rows<G>(p, lane, tile, mb[g], nb[g]);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    });
}

// ---- LoRA down-projection --------------------------------------------------
// Row of P for rank j (ok: the rank exists; the pointer is valid either way).
__device__ __forceinline__ const uint16_t *down_prow(const DownArgs &d, int j, bool &ok) {
    if (d.ngroups > 1) {
        const int g = min(j / d.grp_rpad, d.ngroups - 1), jj = j - g * d.grp_rpad;
        ok = j < d.ngroups * d.grp_rpad && jj < d.r;
        return d.Pg[g] + (int64_t)min(jj, d.r - 1) * d.p_sj;
    }
    ok = j < d.r;
    return d.Ps + (int64_t)min(j, d.r - 1) * d.p_sj;
}
// T [M][rpad] = bf16(s . (Xl [M][Kl] . P^T)), P(j, k) = Ps[j p_sj + k p_sk] for
// j < r, zero for r <= j < rpad; FP32 accumulation on v_mfma_f32_16x16x32_bf16.
// The LoRA scale s is applied before the BF16 rounding; for a power-of-two s
// this equals s . bf16(X P^T) exactly, i.e. the scale applied after the
// rank-r product.
// A group of 16 rows is computed by NW wavefronts, each taking a slice of K
// and all RG groups of 16 ranks from one pass over its slice of X (the BF16
// activations are the kernel's HBM traffic); the NW partial tiles are summed
// through LDS in a fixed order.  Ranks beyond 64 take further passes.

// K32 chunks whose loads are in flight together (fewer with more rank groups:
// a 1024-thread workgroup has 128 VGPRs per thread)
template <int RG>
constexpr int down_chunks() { return RG == 1 ? 8 : RG == 2 ? 6 : 4; }

// LDS floats of the reduction buffer
template <int RG, int NW>
constexpr int down_red_floats() { return NW * 16 * (16 * RG + 1); }

// Rows m0 .. m0+15 of T, ranks j0 .. j0 + 16 RG.  Every thread of the
// workgroup (NW wavefronts) calls it; red holds down_red_floats<RG, NW>().
template <int RG, int NW>
__device__ __forceinline__ void lora_down_rows(const DownArgs &d, int m0, float *red) {
    constexpr int RS = 16 * RG + 1;  // row stride of a partial tile
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int row = min(m0 + (lane & 15), d.M - 1);
    const int kg = 8 * (lane >> 4);
    const int ks = ((d.Kl + NW - 1) / NW + 31) / 32 * 32;
    const int kb = w * ks, ke = min(d.Kl, kb + ks);
    const uint16_t *xr = d.X + (int64_t)row * d.ldx;
    float4_t acc[RG];
#pragma unroll
    for (int f = 0; f < RG; ++f) acc[f] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // U chunks of 32 K per iteration: all their loads are issued before the
    // MFMAs, so the loop is not bound by one load latency per chunk
    constexpr int U = down_chunks<RG>();
    for (int k0 = kb; k0 < ke; k0 += 32 * U) {
        u32x4 va[U], vb[U][RG];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + 32 * u + kg;
            va[u] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int f = 0; f < RG; ++f) vb[u][f] = u32x4{0u, 0u, 0u, 0u};
            if (k < ke) {
                va[u] = *reinterpret_cast<const u32x4 *>(xr + k);
#pragma unroll
                for (int f = 0; f < RG; ++f) {
                    bool ok;
                    const uint16_t *prow = down_prow(d, d.j0 + 16 * f + (lane & 15), ok);
                    if (ok) {
                        if (d.p_sk == 1) {
                            vb[u][f] = *reinterpret_cast<const u32x4 *>(prow + k);
                        } else {
                            uint32_t t[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                t[e] = (uint32_t)prow[(int64_t)(k + 2 * e) * d.p_sk] |
                                       ((uint32_t)prow[(int64_t)(k + 2 * e + 1) * d.p_sk] << 16);
                            vb[u][f] = u32x4{t[0], t[1], t[2], t[3]};
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int f = 0; f < RG; ++f)
                acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va[u]),
                                                                 __builtin_bit_cast(bf16x8_t, vb[u][f]), acc[f], 0,
                                                                 0, 0);
    }
#pragma unroll
    for (int f = 0; f < RG; ++f)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[(w * 16 + 4 * (lane >> 4) + e) * RS + 16 * f + (lane & 15)] = acc[f][e];
    __syncthreads();
    for (int i = threadIdx.x; i < 16 * 16 * RG; i += 64 * NW) {
        const int mi = i / (16 * RG), ji = i % (16 * RG);
        float sum = 0.0f;
        for (int q = 0; q < NW; ++q) sum += red[(q * 16 + mi) * RS + ji];
        const float ts = d.scale * sum;
        if (m0 + mi < d.M) d.T[(int64_t)(m0 + mi) * d.rpad + d.j0 + ji] = (uint16_t)f32_to_bf16_bits(ts);
    }
    __syncthreads();  // red is reused by the caller's next row group
}

// The side job of d as workgroup wg of nwg (no barriers: side workgroups
// return before the launch's own work).
__device__ __forceinline__ void side_transpose(const DownArgs &d, int64_t wg, int64_t nwg) {
    const int64_t nt = (int64_t)d.side_N * d.side_r;
    for (int64_t i = wg * blockDim.x + threadIdx.x; i < nt; i += nwg * blockDim.x) {
        const int j = (int)(i / d.side_N), n = (int)(i % d.side_N);
        d.side_Bt[i] = d.side_B[(int64_t)n * d.side_r + j];
    }
}

// LoRA-down as workgroups of a split-K main kernel (which does not read T):
// row groups blockIdx.x, blockIdx.x + gridDim.x, ...; ranks up to 64.  The
// side job follows, spread over the same workgroups.
template <int NW>
__device__ __forceinline__ void lora_down_fused(const DownArgs &d, float *red) {
    const int groups = (d.M + 15) / 16;
    for (int g = blockIdx.x; g < groups; g += gridDim.x) {
        switch (d.rpad >> 4) {
            case 1: lora_down_rows<1, NW>(d, 16 * g, red); break;
            case 2: lora_down_rows<2, NW>(d, 16 * g, red); break;
            case 3: lora_down_rows<3, NW>(d, 16 * g, red); break;
            default: lora_down_rows<4, NW>(d, 16 * g, red); break;
        }
    }
    if (d.side_Bt) side_transpose(d, blockIdx.x, gridDim.x);
}

constexpr int kDownWaves = 16;

template <int RG>
__global__ __launch_bounds__(1024) void lora_down_kernel(DownArgs d) {
    __shared__ float red[down_red_floats<RG, kDownWaves>()];
    const int groups = (d.M + 15) / 16;
    if ((int)blockIdx.x >= groups) {  // side job (whole workgroups, before any barrier)
        side_transpose(d, blockIdx.x - groups, gridDim.x - groups);
        return;
    }
    lora_down_rows<RG, kDownWaves>(d, blockIdx.x * 16, red);
}

// Standalone LoRA-down for up to 64 ranks with contiguous rows of P
// (p_sk == 1).  Its cost is the number of vector memory instructions in
// flight per CU, and the rank operand P costs as many instructions as X (it is
// read from L2 by every row group).  So: a wavefront takes RPW row groups and
// uses every P fragment for all of them; NW = 4, 8 or 16 wavefronts split K
// (enough wavefronts in flight even when the row groups are few); each
// wavefront works through its K range in stages of 128 K with the loads of
// the next stage issued before the MFMAs of the current one (branch-free: out
// of range fragments read a clamped address and are zeroed).  Within a stage,
// fragment c of lane group g covers 8 K at kpos(c, g): for BF16 rows a
// row's 64 contiguous bytes per instruction; for NVFP4 rows the lane's 16
// code bytes hold its 32 K (decoded to BF16 in registers).  X is read with
// ordinary (cached) loads: the two halves of a 128-byte line come from two
// instructions, and nontemporal loads made the launch 3-10 % slower.
template <bool NV>
__device__ __forceinline__ int down_kpos(int c, int g) { return NV ? 32 * g + 8 * c : 32 * c + 8 * g; }

template <int RG, int RPW, bool NV, int NW>
__global__ __launch_bounds__(64 * NW) void lora_down_pipe_kernel(DownArgs d) {
    constexpr int RS = 16 * RG + 1;
    constexpr int ROWS = 16 * RPW;
    __shared__ float red[NW * ROWS * RS];
    const int groups = (d.M + ROWS - 1) / ROWS;
    if ((int)blockIdx.x >= groups) {  // side job (whole workgroups, before any barrier)
        side_transpose(d, blockIdx.x - groups, gridDim.x - groups);
        return;
    }
    const int m0 = blockIdx.x * ROWS;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 15, g = lane >> 4;
    const int ks = ((d.Kl + NW - 1) / NW + 127) / 128 * 128;
    const int kb = w * ks, ke = min(d.Kl, kb + ks);
    int row[RPW];
#pragma unroll
    for (int q = 0; q < RPW; ++q) row[q] = min(m0 + 16 * q + li, d.M - 1);
    const uint16_t *pr[RG];
    bool jok[RG];
#pragma unroll
    for (int f = 0; f < RG; ++f) pr[f] = down_prow(d, d.j0 + 16 * f + li, jok[f]);
    float xdm[RPW];
    if (NV) {
#pragma unroll
        for (int q = 0; q < RPW; ++q) xdm[q] = d.xd[row[q]];
    }
    const bool k32 = (d.Kl & 31) == 0;  // NVFP4 rows start 16-byte (codes) and 2-byte (scales) aligned
    float4_t acc[RPW][RG];
#pragma unroll
    for (int q = 0; q < RPW; ++q)
#pragma unroll
        for (int f = 0; f < RG; ++f) acc[q][f] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // stage buffers: X fragments (BF16) or raw NVFP4 (16 code bytes + 2 scale bytes), P fragments
    u32x4 xv[2][RPW][NV ? 1 : 4];
    uint32_t xs[2][RPW];
    u32x4 pv[2][4][RG];
    auto load = [&](int b, int kc) {
#pragma unroll
        for (int q = 0; q < RPW; ++q) {
            if (NV) {
                const int k0 = kc + 32 * g;
                const int kk = k0 < ke ? k0 : 0;
                const uint8_t *cr = d.xc + (int64_t)row[q] * (d.Kl / 2) + kk / 2;
                const uint8_t *sr = d.xs + (int64_t)row[q] * (d.Kl / 16) + kk / 16;
                uint32_t s2;
                if (k32) {
                    xv[b][q][0] = *reinterpret_cast<const u32x4 *>(cr);
                    s2 = *reinterpret_cast<const uint16_t *>(sr);
                } else {  // rows of 16 K multiples: the second block may be past the row
                    const bool two = kk + 16 < d.Kl;
                    const u32x2 lo = *reinterpret_cast<const u32x2 *>(cr);
                    const u32x2 hi = *reinterpret_cast<const u32x2 *>(two ? cr + 8 : cr);
                    xv[b][q][0] = u32x4{lo.x, lo.y, hi.x, hi.y};
                    s2 = (uint32_t)sr[0] | ((uint32_t)sr[two ? 1 : 0] << 8);
                }
                // blocks at or past the end of the K range decode to zero (scale 0)
                if (k0 >= ke) s2 = 0u;
                else if (k0 + 16 >= ke) s2 &= 0xFFu;
                xs[b][q] = s2;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int k = kc + down_kpos<NV>(c, g);
                    const u32x4 v =
                        *reinterpret_cast<const u32x4 *>(d.X + (int64_t)row[q] * d.ldx + (k < ke ? k : 0));
                    xv[b][q][c] = k < ke ? v : u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int k = kc + down_kpos<NV>(c, g);
#pragma unroll
            for (int f = 0; f < RG; ++f) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(pr[f] + (k < ke ? k : 0));
                pv[b][c][f] = (k < ke && jok[f]) ? v : u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto mma = [&](int b) {
#pragma unroll
        for (int q = 0; q < RPW; ++q) {
            half2_t sc0, sc1;
            if (NV) {
                sc0 = e4m3_to_h2(xs[b][q] & 0xFFu);
                sc1 = e4m3_to_h2(xs[b][q] >> 8);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                u32x4 xf;
                if (NV) xf = dequant8_bf16(xv[b][q][0][c], c < 2 ? sc0 : sc1, xdm[q]);
                else xf = xv[b][q][c];
#pragma unroll
                for (int f = 0; f < RG; ++f)
                    acc[q][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xf),
                                                                        __builtin_bit_cast(bf16x8_t, pv[b][c][f]),
                                                                        acc[q][f], 0, 0, 0);
            }
        }
    };
    if (kb < ke) {
        load(0, kb);
        for (int kc = kb;;) {
            if (kc + 128 >= ke) {
                mma(0);
                break;
            }
            load(1, kc + 128);
            mma(0);
            kc += 128;
            if (kc + 128 >= ke) {
                mma(1);
                break;
            }
            load(0, kc + 128);
            mma(1);
            kc += 128;
        }
    }
    // accumulator element e of lane (li, g): row 4 g + e of the group, rank 16 f + li
#pragma unroll
    for (int q = 0; q < RPW; ++q)
#pragma unroll
        for (int f = 0; f < RG; ++f)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[(w * ROWS + 16 * q + 4 * g + e) * RS + 16 * f + li] = acc[q][f][e];
    __syncthreads();
    for (int i = threadIdx.x; i < ROWS * 16 * RG; i += 64 * NW) {
        const int mi = i / (16 * RG), ji = i % (16 * RG);
        float sum = 0.0f;
#pragma unroll
        for (int q = 0; q < NW; ++q) sum += red[(q * ROWS + mi) * RS + ji];
        const float ts = d.scale * sum;
        if (m0 + mi < d.M) d.T[(int64_t)(m0 + mi) * d.rpad + d.j0 + ji] = (uint16_t)f32_to_bf16_bits(ts);
    }
}

// Wavefronts per workgroup of the pipelined LoRA-down: 16 when row groups are
// few (so that enough loads are in flight) and a wavefront's fragments fit
// 128 VGPRs (one or two rank-by-row groups); 4 for 4 rank groups of two row
// groups (its fragments take up to 256 VGPRs); 8 otherwise.  Every choice is
// free of register spills.
static int pipe_waves(int rg, int rpw, int groups) {
    if (rg * rpw <= 2 && groups <= 128) return 16;
    if (rg == 4 && rpw == 2) return 4;
    return 8;
}

template <int RG, int RPW, bool NV>
static void launch_pipe_nw(int nw, dim3 grid, dim3 block, hipStream_t st, const DownArgs &d) {
    if constexpr (RG * RPW <= 2) {
        if (nw == 16) {
            hipLaunchKernelGGL((lora_down_pipe_kernel<RG, RPW, NV, 16>), grid, block, 0, st, d);
            return;
        }
    }
    if constexpr (RG == 4 && RPW == 2)
        hipLaunchKernelGGL((lora_down_pipe_kernel<RG, RPW, NV, 4>), grid, block, 0, st, d);
    else
        hipLaunchKernelGGL((lora_down_pipe_kernel<RG, RPW, NV, 8>), grid, block, 0, st, d);
}

// One pass of the pipelined LoRA-down over ranks [j0, j0 + 16 rg): rank
// groups, row groups of 16 per wavefront, wavefronts per workgroup and
// workgroups with rows.
struct PipePass {
    int rg, rpw, nw, groups;
};

static PipePass pipe_pass(int64_t M, int rpad, int j0) {
    const int rg = (rpad - j0) / 16 < 4 ? (rpad - j0) / 16 : 4;
    const bool two = M >= 4096 && rg >= 2;  // two row groups per wavefront once rows are plentiful
    const int groups = (int)((M + (two ? 31 : 15)) / (two ? 32 : 16));
    return {rg, two ? 2 : 1, pipe_waves(rg, two ? 2 : 1, groups), groups};
}

// Ranks in passes of up to 64 (each pass reads X again); the side job rides
// on the first pass.
template <bool NV>
static pact_status launch_down_pipe(DownArgs d, hipStream_t st) {
    for (int j0 = 0; j0 < d.rpad; j0 += 64) {
        const PipePass pp = pipe_pass(d.M, d.rpad, j0);
        const int rg = pp.rg, nw = pp.nw, groups = pp.groups;
        const bool two = pp.rpw == 2;
        const dim3 grid((unsigned)(groups + (j0 == 0 ? side_blocks(d, 64 * nw) : 0))), block(64 * nw);
        d.j0 = j0;
        switch (rg * 2 + (two ? 1 : 0)) {
            case 2: launch_pipe_nw<1, 1, NV>(nw, grid, block, st, d); break;
            case 4: launch_pipe_nw<2, 1, NV>(nw, grid, block, st, d); break;
            case 5: launch_pipe_nw<2, 2, NV>(nw, grid, block, st, d); break;
            case 6: launch_pipe_nw<3, 1, NV>(nw, grid, block, st, d); break;
            case 7: launch_pipe_nw<3, 2, NV>(nw, grid, block, st, d); break;
            case 8: launch_pipe_nw<4, 1, NV>(nw, grid, block, st, d); break;
            default: launch_pipe_nw<4, 2, NV>(nw, grid, block, st, d); break;
        }
        PACT_TRY(launch_status());
    }
    return PACT_OK;
}

pact_status launch_lora_down_nvfp4(DownArgs d, hipStream_t st) {
    if (d.rpad > 64 || d.p_sk != 1 || !d.xc) return PACT_ERR_UNSUPPORTED_SHAPE;
    return launch_down_pipe<true>(d, st);
}

pact_status launch_lora_down(DownArgs d, hipStream_t st) {
    if (d.p_sk == 1) return launch_down_pipe<false>(d, st);
    const dim3 block(64 * kDownWaves);
    for (int j0 = 0; j0 < d.rpad; j0 += 64) {
        d.j0 = j0;
        const dim3 grid((unsigned)((d.M + 15) / 16 + (j0 == 0 ? side_blocks(d, 64 * kDownWaves) : 0)));
        const int rg = (d.rpad - j0) / 16 < 4 ? (d.rpad - j0) / 16 : 4;
        switch (rg) {
            case 1: hipLaunchKernelGGL(lora_down_kernel<1>, grid, block, 0, st, d); break;
            case 2: hipLaunchKernelGGL(lora_down_kernel<2>, grid, block, 0, st, d); break;
            case 3: hipLaunchKernelGGL(lora_down_kernel<3>, grid, block, 0, st, d); break;
            default: hipLaunchKernelGGL(lora_down_kernel<4>, grid, block, 0, st, d); break;
        }
        PACT_TRY(launch_status());
    }
    return PACT_OK;
}

// Split-K: a workgroup stores its FP32 partial fragments instead of running
// the epilogue; fragment (i, j) of split s is 1024 floats at
// part + ((s FM + i) FN + j) 1024, element e of lane l at (e / 4) 256 + 4 l +
// e % 4 (every store instruction writes 1 KB contiguously).  Fragments past
// the output are not stored.
template <int F, typename AccFn>
__device__ __forceinline__ void store_partials(const GemmArgs &p, int lane, AccFn &&accf, const int (&mb)[F],
                                               const int (&nb)[F], int split) {
    const int FM = (p.M + 31) >> 5, FN = (p.N + 31) >> 5;
    static_for<F>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int fi = mb[i] >> 5, fj = nb[i] >> 5;
        if (fi < FM && fj < FN) {
            float *dst = p.part + (((int64_t)split * FM + fi) * FN + fj) * 1024 + 4 * lane;
            const float16_t &a = accf(ic);
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
                *reinterpret_cast<float4_t *>(dst + 256 * e4) =
                    float4_t{a[4 * e4], a[4 * e4 + 1], a[4 * e4 + 2], a[4 * e4 + 3]};
        }
    });
}

// End of a main kernel: the epilogue, or (split K) the partial store.
template <bool SPLIT, int F, int G, typename AccFn>
__device__ __forceinline__ void finish_frags(const GemmArgs &p, int lane, AccFn &&accf, const int (&mb)[F],
                                             const int (&nb)[F], float *tile, int split) {
    if constexpr (SPLIT)
        store_partials<F>(p, lane, accf, mb, nb, split);
    else
        epi_frags<F, G>(p, lane, accf, mb, nb, tile);
}

// Main kernel.  Every wavefront owns a 128 x 128 accumulator tile (4 x 4
// fragments of 32 x 32, 256 FP32 per lane) and decodes its own MFMA operands
// from the packed NVFP4 stage in LDS: per K16 step it converts 8 fragments
// (4 of A, 4 of B; one code dword each, 8 VALU) for 16 MFMAs, 4 VALU per
// MFMA, which the MFMA pipe hides.
//
// A workgroup is 4 wavefronts arranged WM x WN x WK: the output tile is
// (128 WM) x (128 WN); the WK wavefronts at the same (i, j) split K into WK
// contiguous ranges, and their partial tiles are summed through LDS at the
// end.  The WM x WN wavefronts of one K range form a group that stages its
// packed operands together.
//
// LDS of a group: NBUF buffers of one stage of 64 K-elements each,
//   codes  [ROWS][32 B], ROWS = the tile's A rows then its B rows; the two
//          16-byte halves of a row are swapped on rows with bit 3 set, so the
//          16 rows read by 16 lanes fall on 16 distinct groups of banks;
//   scales [ROWS][4 B], the row's 4 E4M3 block scales of the stage.
// Inside a stage, K is assigned to MFMA operand slots by lane half, the same
// way in both operands: lanes 32h .. 32h+31 take elements [32h, 32h + 32) of
// the stage, 8 per K16 step, so a lane reads one 16-byte half-row and one
// 2-byte pair of scales per fragment and stage.  (Any assignment shared by
// A and B gives the same dot product; only the FP32 summation order moves.)
//
// Pipeline: stage s+1 is read into a second register set during stage s,
// stage s+3 is loaded from global memory (direct 16- and 4-byte loads into
// LDS) while stage s is consumed, and the decode of step t+1 is interleaved
// with the MFMAs of step t.  A group with several wavefronts meets at one
// barrier per stage; a single-wavefront group needs none.
constexpr int kNBuf = 4;   // LDS stage buffers per group
// Buffer descriptor word 3 for raw (untyped, unswizzled) byte access on gfx950.

constexpr int kSK = 64;    // K per stage

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int WM, int WN, int WK>
struct GemmShape {
    static constexpr int G = WM * WN;  // wavefronts per group
    static constexpr int BM = 128 * WM, BN = 128 * WN;
    static constexpr int ROWS = BM + BN;
    static constexpr int PCODE = ROWS * 32;
    static constexpr int STAGE = ROWS * 36;
    static constexpr int GROUP_BYTES = kNBuf * STAGE;
    static constexpr int N_CODE_I = ROWS / 32;  // 1 KB loads per stage: 32 rows x 32 B
    static constexpr int N_SC_I = ROWS / 64;    // 256 B loads per stage: 64 rows x 4 B
    static constexpr int LPW = (N_CODE_I + N_SC_I) / G;  // loads per wavefront per stage
    static constexpr int NQC = N_CODE_I / G;              // of which code loads
    // partial-tile exchange: 4 fragments (one column) per wavefront per round
    static constexpr int RED_BYTES = WK == 1 ? 0 : 4 * 4 * 4096;
    static constexpr int LDS_BYTES = WK * GROUP_BYTES > RED_BYTES ? WK * GROUP_BYTES : RED_BYTES;
    static_assert(G * WK == 4, "four wavefronts");
    static_assert(N_CODE_I % G == 0 && N_SC_I % G == 0, "loads split evenly");
};

template <int WM, int WN, int WK, bool KFULL, bool SPLIT>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs p_arg) {
    const GemmArgs &p = kernel_gemm_args();
    (void)p_arg;
    using SH = GemmShape<WM, WN, WK>;
    static_assert(SH::LDS_BYTES >= 4 * 4 * epi_tile_floats<4>(), "LDS holds the epilogue tiles");
    static_assert(SH::LDS_BYTES >= 4 * down_red_floats<4, 4>(), "LDS holds the fused LoRA-down buffer");
    constexpr int G = SH::G, BM = SH::BM, BN = SH::BN, ROWS = SH::ROWS;
    constexpr int PCODE = SH::PCODE, STAGE = SH::STAGE, LPW = SH::LPW, NQC = SH::NQC;
    __shared__ __attribute__((aligned(16))) uint8_t lds[SH::LDS_BYTES];

    // split K: workgroups blockIdx.y == 0 compute the LoRA-down product when
    // it is fused into this launch (the split-K epilogue reads it)
    if constexpr (SPLIT) {
        if (p.down.X && blockIdx.y == 0) {
            lora_down_fused<4>(p.down, reinterpret_cast<float *>(lds));
            return;
        }
    }
    const int split = SPLIT ? (int)blockIdx.y - (p.down.X ? 1 : 0) : 0;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int h = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave / G;  // K range
    const int wi = wave % G;   // position in the group
    const int wm = wi / WN, wn = wi % WN;
    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = p.K;
    const int nblk = K >> 4;
    // stages per group (the host makes it exact); workgroup blockIdx.y of a
    // split-K launch takes the y-th of ks equal ranges of stages
    const int S = ((K + kSK - 1) / kSK) / (WK * p.ks);
    const int gs0 = (split * WK + grp) * S;  // first global stage of this group
    uint8_t *const glds = lds + grp * SH::GROUP_BYTES;

    // ---- per-wavefront load assignment: load q of a stage ----
    // code load i (< N_CODE_I): rows 32 i + lane/2, half (lane & 1) of the
    // row's 32 bytes; scale load j: row 64 j + lane, 4 bytes.  A load
    // instruction reads rows of one operand only (32- and 64-row groups never
    // straddle the A/B boundary; which operand is known at compile time), so
    // it is a buffer load with that operand's descriptor, a 32-bit lane
    // offset and the stage offset in a scalar register.  Rows past the end
    // are clamped to the last row (their results are never stored).
    constexpr int QA_CODE = BM / (32 * G);  // code loads q < QA_CODE read A
    constexpr int QA_SC = BM / (64 * G);    // scale loads q - NQC < QA_SC read A
    static_assert(BM % (64 * G) == 0, "operand of a load is static");
    const __amdgpu_buffer_rsrc_t rs_ac =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.a_codes, (short)0, (int)(p.a_bytes), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rs_bc =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.b_codes, (short)0, (int)(p.b_bytes), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rs_as =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.a_scales, (short)0, (int)(p.a_bytes >> 3), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rs_bs =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.b_scales, (short)0, (int)(p.b_bytes >> 3), kRsrcWord3);
    // stages past the group's last one are loaded through a descriptor with
    // no records: nothing is fetched, and the main loop stays branch-free
    const __amdgpu_buffer_rsrc_t rs_none =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.a_codes, (short)0, 0, kRsrcWord3);
    const int gp = (lane & 1) ^ ((lane >> 4) & 1);  // half of its row a code-load lane carries
    uint32_t loff[LPW];  // lane's byte offset in its operand at K = 0
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
        if (q < NQC) {
            const int rr = 32 * (wi + G * q) + (lane >> 1);
            const int crow = q < QA_CODE ? min(m0 + rr, p.M - 1) : min(n0 + rr - BM, p.N - 1);
            loff[q] = (uint32_t)crow * (uint32_t)(K >> 1) + 16u * (uint32_t)gp;
        } else {
            const int rr = 64 * (wi + G * (q - NQC)) + lane;
            const int crow = q - NQC < QA_SC ? min(m0 + rr, p.M - 1) : min(n0 + rr - BM, p.N - 1);
            loff[q] = (uint32_t)crow * (uint32_t)nblk;
        }
    }
    auto ldst = [&](int q) {  // LDS offset of load q in a stage buffer (uniform)
        return q < NQC ? (wi + G * q) * 1024 : PCODE + (wi + G * (q - NQC)) * 256;
    };

    // loads of local stage s into buffer s % kNBuf
    auto issue_stage = [&](int s) {
        uint8_t *const buf = glds + (s % kNBuf) * STAGE;
        const int gstage = gs0 + s;
        const bool live = s < S;
#pragma unroll
        for (int q = 0; q < LPW; ++q) {
            lds_void_t *const dst = (lds_void_t *)(buf + ldst(q));
            if (q < NQC) {
                if (KFULL) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(!live ? rs_none : q < QA_CODE ? rs_ac : rs_bc, dst, 16, (int)loff[q],
                                                             gstage * (kSK / 2), 0, 0);
                } else {
                    // K not a multiple of the stage: 8-byte pieces (one block
                    // of 16 codes each) inside K, zeros past it
                    const uint8_t *src = (q < QA_CODE ? p.a_codes : p.b_codes) + loff[q] + gstage * (kSK / 2);
                    const int kk = gstage * kSK + 32 * gp;
                    u32x4 v = {0u, 0u, 0u, 0u};
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
                    *reinterpret_cast<u32x4 *>(buf + ldst(q) + 16 * lane) = v;
                }
            } else {
                if (KFULL) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(!live ? rs_none : q - NQC < QA_SC ? rs_as : rs_bs, dst, 4, (int)loff[q],
                                                             gstage * (kSK / 16), 0, 0);
                } else {
                    const uint8_t *src =
                        (q - NQC < QA_SC ? p.a_scales : p.b_scales) + loff[q] + gstage * (kSK / 16);
                    const int b0 = gstage * (kSK / 16);
                    uint32_t w = 0u;
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        if (b0 + b < nblk) w |= (uint32_t)src[b] << (8 * b);
                    *reinterpret_cast<uint32_t *>(buf + ldst(q) + 4 * lane) = w;
                }
            }
        }
    };

    // ---- fragment reads: this lane's row of fragment f (0..3: A, 4..7: B) ----
    const int lr = lane & 31;
    const int rd_code = lr * 32 + 16 * (h ^ ((lr >> 3) & 1));
    const int rd_sc = PCODE + lr * 4 + 2 * h;
    const int a_row0 = wm * 128, b_row0 = BM + wn * 128;
    u32x4 P[2][8];
    uint32_t SC[2][8];
    half2_t SCH[2][8];
    auto read_stage = [&](int s, u32x4 (&Pd)[8], uint32_t (&Sd)[8]) {
        const uint8_t *buf = glds + (s % kNBuf) * STAGE;
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            const int row0 = f < 4 ? a_row0 + 32 * f : b_row0 + 32 * (f - 4);
            Pd[f] = *reinterpret_cast<const u32x4 *>(buf + row0 * 32 + rd_code);
            Sd[f] = *reinterpret_cast<const uint16_t *>(buf + row0 * 4 + rd_sc);
        }
    };
    // operands of K16 step t (0..3) of a stage held in registers
    auto decode = [&](const u32x4 (&Pb)[8], const uint32_t (&Sb)[8], half2_t (&Hb)[8], int t,
                      half8_t (&out)[8]) {
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            if (t == 0) Hb[f] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(Sb[f], 1.0f, false);
            const uint32_t w = t == 0 ? Pb[f].x : t == 1 ? Pb[f].y : t == 2 ? Pb[f].z : Pb[f].w;
            half2_t sc;
            sc[0] = Hb[f][t >> 1];
            sc[1] = Hb[f][t >> 1];
            out[f] = decode8(w, sc);
        }
    };

    float16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    half8_t cur[8];
    if (S > 0) {
        // stages 0-2 in flight (those past the end fetch nothing); wait for 0
        issue_stage(0);
        if (KFULL || S > 1) issue_stage(1);
        if (KFULL || S > 2) issue_stage(2);
        if (KFULL)
            wait_vmcnt<2 * LPW>();
        else
            wait_global_loads();
        if (G > 1 || !KFULL) lds_barrier();
        read_stage(0, P[0], SC[0]);
        decode(P[0], SC[0], SCH[0], 0, cur);
    }

    // one stage; register set B holds it, set B^1 receives the next stage
    auto stage = [&](auto Bc, int s) {
        constexpr int B = decltype(Bc)::value;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t == 1) {
                // stage s+1 has landed (stages s+1 and s+2 are in flight);
                // every wavefront of the group is past stage s-1, so its
                // buffer may take stage s+3.  No branch here: a branch would
                // split the step into blocks the scheduler cannot interleave.
                if (KFULL) {
                    wait_vmcnt<LPW>();
                    if (G > 1) lds_barrier();
                    issue_stage(s + 3);
                } else {
                    wait_global_loads();
                    lds_barrier();
                    if (s + 3 < S) issue_stage(s + 3);
                }
                read_stage(s + 1, P[B ^ 1], SC[B ^ 1]);
            }
            half8_t nx[8];
            if (t < 3)
                decode(P[B], SC[B], SCH[B], t + 1, nx);
            else
                decode(P[B ^ 1], SC[B ^ 1], SCH[B ^ 1], 0, nx);
#pragma unroll
            for (int fm = 0; fm < 4; ++fm)
#pragma unroll
                for (int fn = 0; fn < 4; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur[fm], cur[4 + fn], acc[fm][fn], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // 4 VALU
                if (t == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
            }
#pragma unroll
            for (int f = 0; f < 8; ++f) cur[f] = nx[f];
        }
    };
    // pairs of stages (register sets 0, 1), then a last even stage if S is odd
    int s = 0;
    for (; s + 1 < S; s += 2) {
        stage(std::integral_constant<int, 0>(), s);
        stage(std::integral_constant<int, 1>(), s + 1);
    }
    if (s < S) stage(std::integral_constant<int, 0>(), s);

    // drain the stage loads still in flight (they write LDS)
    wait_global_loads();

    // ---- epilogue: row scales, LoRA term, residual, BF16 store ----
    const int mw = m0 + a_row0, nw = n0 + wn * 128;

    // partial fragment slot: [e4][lane][4 floats], 4 KB, conflict-free
    auto put_frag = [&](uint8_t *slot, const float16_t &a) {
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            float4_t v = {a[4 * e4], a[4 * e4 + 1], a[4 * e4 + 2], a[4 * e4 + 3]};
            *reinterpret_cast<float4_t *>(slot + e4 * 1024 + lane * 16) = v;
        }
    };
    auto get_frag = [&](const uint8_t *slot) {
        float16_t a;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const float4_t v = *reinterpret_cast<const float4_t *>(slot + e4 * 1024 + lane * 16);
            a[4 * e4] = v[0];
            a[4 * e4 + 1] = v[1];
            a[4 * e4 + 2] = v[2];
            a[4 * e4 + 3] = v[3];
        }
        return a;
    };

    if constexpr (WK == 1) {
        int mbs[16], nbs[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mbs[i] = mw + 32 * (i >> 2);
            nbs[i] = nw + 32 * (i & 3);
        }
        if constexpr (!SPLIT) lds_barrier();  // stage buffers free for the epilogue tiles
        finish_frags<SPLIT, 16, 4>(p, lane, [&](auto ic) -> float16_t & {
            constexpr int i = decltype(ic)::value;
            return acc[i >> 2][i & 3];
        }, mbs, nbs, reinterpret_cast<float *>(lds) + wave * epi_tile_floats<4>(), split);
    } else {
        // Partial tiles summed through LDS, one fragment column per round:
        // every wavefront writes its 4 fragments of the column to slot
        // (wave, fm); the owner of a fragment row then reads the WK partials
        // of it (its own included) and adds them in K-range order.  Fragment
        // row fm belongs to the wavefront of K range fm / (4 / WK) at the same
        // position in its group.
        constexpr int ROWS_PER_OWNER = 4 / WK;
        float16_t own[ROWS_PER_OWNER][4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            lds_barrier();
#pragma unroll
            for (int fm = 0; fm < 4; ++fm) put_frag(lds + (wave * 4 + fm) * 4096, acc[fm][c]);
            lds_barrier();
#pragma unroll
            for (int i = 0; i < ROWS_PER_OWNER; ++i) {
                const int fm = grp * ROWS_PER_OWNER + i;
                float16_t sum = get_frag(lds + ((0 * G + wi) * 4 + fm) * 4096);
#pragma unroll
                for (int q = 1; q < WK; ++q) {
                    const float16_t part = get_frag(lds + ((q * G + wi) * 4 + fm) * 4096);
#pragma unroll
                    for (int e = 0; e < 16; ++e) sum[e] = sum[e] + part[e];
                }
                own[i][c] = sum;
            }
        }
        constexpr int NF = 4 * ROWS_PER_OWNER;
        int mbs[NF], nbs[NF];
#pragma unroll
        for (int i = 0; i < ROWS_PER_OWNER; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                mbs[4 * i + c] = mw + 32 * (grp * ROWS_PER_OWNER + i);
                nbs[4 * i + c] = nw + 32 * c;
            }
        if constexpr (!SPLIT) lds_barrier();  // reduction slots free for the epilogue tiles
        finish_frags<SPLIT, NF, 4>(p, lane, [&](auto ic) -> float16_t & {
            constexpr int i = decltype(ic)::value;
            return own[i >> 2][i & 3];
        }, mbs, nbs, reinterpret_cast<float *>(lds) + wave * epi_tile_floats<4>(), split);
    }
}

// ---- 256 x 256 kernel with one decode per workgroup --------------------------
// For output tiles of 256 x 256 (enough of them to fill the GPU).  Eight
// wavefronts (two per SIMD) each own 128 x 64 of the tile (4 x 2 fragments).
// Each K32 phase is decoded once per workgroup: thread t converts row t of the
// tile (rows 0-255 of A, 256-511 of B) into FP16 in an LDS tile laid out in
// MFMA fragment order, so the VALU cost is 2 operations per MFMA instead of
// the 6 a per-wavefront decode of a 128 x 64 tile would take.
//
// LDS: the packed stage ring of the main kernel (4 buffers of 64 K-elements,
// rows of 32 code bytes with halves swapped on rows with bit 3 set, then the
// rows' 4 scale bytes) and two FP16 phase tiles of 32 KB:
//   F[g][s][lane] 16 bytes, g = 32-row group (0-7 A, 8-15 B), s = K16 step,
//   lane (r, h) = row r of the group, K [16 s + 8 h, 16 s + 8 h + 8).
// Phase p (one barrier, mid-phase):
//   first half:  MFMAs of step 0 (fragments read before), the decode of
//                phase p+1 into F[(p+1) & 1] from packed codes read one phase
//                earlier, the reads of this phase's step-1 fragments; on even
//                p the loads of stage p/2 + 3 are issued and each wavefront
//                waits for stage p/2 + 1;
//   barrier:     F[(p+1) & 1] complete; everyone is past phase p-1's reads;
//   second half: MFMAs of step 1, reads of phase p+1's step-0 fragments and
//                of phase p+2's packed codes.
struct Gemm8Shape {
    static constexpr int BM = 256, BN = 256, ROWS = 512;
    static constexpr int PCODE = ROWS * 32;
    static constexpr int STAGE = ROWS * 36;           // 18 KB
    static constexpr int RING = kNBuf * STAGE;        // 72 KB
    static constexpr int FPH = ROWS * 32 * 2;         // 32 KB FP16 phase tile
    static constexpr int LDS_BYTES = RING + 2 * FPH;  // 136 KB
    static constexpr int LPW = 3;                     // stage loads per wavefront: 2 code, 1 scale
};

template <int N>
__device__ __forceinline__ void wait_vmcnt_lds_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <bool SPLIT>
__global__ __launch_bounds__(512, 1) void gemm8_kernel(GemmArgs p_arg) {
    const GemmArgs &p = kernel_gemm_args();
    (void)p_arg;
    using SH = Gemm8Shape;
    static_assert(SH::LDS_BYTES >= 8 * 4 * epi_tile_floats<2>(), "LDS holds the epilogue tiles");
    static_assert(SH::LDS_BYTES >= 4 * down_red_floats<4, 8>(), "LDS holds the fused LoRA-down buffer");
    constexpr int STAGE = SH::STAGE, PCODE = SH::PCODE, FPH = SH::FPH, LPW = SH::LPW;
    __shared__ __attribute__((aligned(16))) uint8_t lds[SH::LDS_BYTES];
    uint8_t *const ring = lds;
    uint8_t *const F0 = lds + SH::RING;

    if constexpr (SPLIT) {
        if (p.down.X && blockIdx.y == 0) {  // fused LoRA-down workgroups
            lora_down_fused<8>(p.down, reinterpret_cast<float *>(lds));
            return;
        }
    }
    const int split = SPLIT ? (int)blockIdx.y - (p.down.X ? 1 : 0) : 0;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 wavefronts of 128 x 64
    const int tiles_m = (p.M + SH::BM - 1) / SH::BM;
    const int tiles_n = (p.N + SH::BN - 1) / SH::BN;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * SH::BM, n0 = tn * SH::BN;
    const int K = p.K;
    const int nblk = K >> 4;
    const int S = (K / kSK) / p.ks;  // stages (K % 64 == 0 for this kernel; the host makes it exact)
    const int s0 = split * S;  // first stage of this workgroup's K range

    // ---- stage loads: wavefront w issues code loads w (A rows 32w..) and
    // w + 8 (B rows), and scale load w (rows 64w.., A when w < 4) ----
    const __amdgpu_buffer_rsrc_t rs_ac =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.a_codes, (short)0, (int)(p.a_bytes), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rs_bc =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.b_codes, (short)0, (int)(p.b_bytes), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rs_sc = wave < 4
        ? __builtin_amdgcn_make_buffer_rsrc((void *)p.a_scales, (short)0, (int)(p.a_bytes >> 3), kRsrcWord3)
        : __builtin_amdgcn_make_buffer_rsrc((void *)p.b_scales, (short)0, (int)(p.b_bytes >> 3), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rs_none =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.a_codes, (short)0, 0, kRsrcWord3);
    const int gp = (lane & 1) ^ ((lane >> 4) & 1);
    uint32_t off_a, off_b, off_s;
    {
        const int ra = 32 * wave + (lane >> 1);                 // A tile row
        const int rb = 32 * wave + (lane >> 1);                 // B tile row (code load w + 8)
        off_a = (uint32_t)min(m0 + ra, p.M - 1) * (uint32_t)(K >> 1) + 16u * (uint32_t)gp;
        off_b = (uint32_t)min(n0 + rb, p.N - 1) * (uint32_t)(K >> 1) + 16u * (uint32_t)gp;
        const int rs = 64 * wave + lane;                        // tile row of the scale load
        const int crow = rs < SH::BM ? min(m0 + rs, p.M - 1) : min(n0 + rs - SH::BM, p.N - 1);
        off_s = (uint32_t)crow * (uint32_t)nblk;
    }
    auto issue_stage = [&](int s) {
        uint8_t *const buf = ring + (s % kNBuf) * STAGE;
        const bool live = s < S;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? rs_ac : rs_none, (lds_void_t *)(buf + wave * 1024), 16,
                                                 (int)off_a, (s0 + s) * (kSK / 2), 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? rs_bc : rs_none, (lds_void_t *)(buf + (wave + 8) * 1024),
                                                 16, (int)off_b, (s0 + s) * (kSK / 2), 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? rs_sc : rs_none, (lds_void_t *)(buf + PCODE + wave * 256), 4,
                                                 (int)off_s, (s0 + s) * (kSK / 16), 0, 0);
    };

    // ---- decode: thread t owns tile row t; phase q = half (q & 1) of stage q/2 ----
    const int drow = tid;
    const int dg = drow >> 5, dlr = drow & 31;
    const int rd_packed = drow * 32;
    const int rd_sc = PCODE + drow * 4;
    const int sw = (drow >> 3) & 1;
    uint8_t *const fwr = F0 + ((dg * 2) * 64 + dlr) * 16;  // + step * 1024 + h * 512
    u32x4 pw;        // packed codes of the next phase to decode
    uint32_t psc;    // its two block-scale bytes
    auto read_packed = [&](int q) {
        const uint8_t *buf = ring + ((q >> 1) % kNBuf) * STAGE;
        const int pc = q & 1;
        pw = *reinterpret_cast<const u32x4 *>(buf + rd_packed + 16 * (pc ^ sw));
        psc = *reinterpret_cast<const uint16_t *>(buf + rd_sc + 2 * pc);
    };
    auto decode_phase = [&](int q) {
        const half2_t sh = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(psc, 1.0f, false);
        half2_t s0, s1;
        s0[0] = sh[0];
        s0[1] = sh[0];
        s1[0] = sh[1];
        s1[1] = sh[1];
        uint8_t *const fb = fwr + (q & 1) * FPH;
        *reinterpret_cast<half8_t *>(fb) = decode8(pw.x, s0);          // step 0, h 0
        *reinterpret_cast<half8_t *>(fb + 512) = decode8(pw.y, s0);    // step 0, h 1
        *reinterpret_cast<half8_t *>(fb + 1024) = decode8(pw.z, s1);   // step 1, h 0
        *reinterpret_cast<half8_t *>(fb + 1536) = decode8(pw.w, s1);   // step 1, h 1
    };

    // ---- fragment reads: A groups 4 wm + fm, B groups 8 + 2 wn + fn ----
    auto read_frags = [&](int q, int st, half8_t (&fr)[6]) {
        const uint8_t *fb = F0 + (q & 1) * FPH + (st * 64 + lane) * 16;
#pragma unroll
        for (int f = 0; f < 4; ++f)
            fr[f] = *reinterpret_cast<const half8_t *>(fb + ((4 * wm + f) * 2) * 1024);
#pragma unroll
        for (int f = 0; f < 2; ++f)
            fr[4 + f] = *reinterpret_cast<const half8_t *>(fb + ((8 + 2 * wn + f) * 2) * 1024);
    };

    float16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    auto mfma_step = [&](const half8_t (&fr)[6]) {
#pragma unroll
        for (int fm = 0; fm < 4; ++fm)
#pragma unroll
            for (int fn = 0; fn < 2; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fr[fm], fr[4 + fn], acc[fm][fn], 0, 0, 0);
    };

    half8_t f0[6], f1[6];
    const int nph = 2 * S;
    if (S > 0) {
        issue_stage(0);
        issue_stage(1);
        issue_stage(2);
        wait_vmcnt_lds_barrier<2 * LPW>();  // stage 0 of every wavefront
        read_packed(0);
        decode_phase(0);
        read_packed(1);
        lds_barrier();
        read_frags(0, 0, f0);
    }
    // Phase q.  The barrier is a hard scheduling boundary (sched_barrier), so
    // the two halves keep their own MFMAs.
    auto phase = [&](auto Ec, int q) {
        constexpr bool EVEN = decltype(Ec)::value;
        // first half: step-0 MFMAs, step-1 fragment reads, decode of phase q+1
        if (EVEN) issue_stage((q >> 1) + 3);
        read_frags(q, 1, f1);
        decode_phase(q + 1);
        mfma_step(f0);
        // (the compiler interleaves this half itself: on the MI355X that was
        // 3-5 % faster than a fixed MFMA / VALU / LDS group pattern)
        __builtin_amdgcn_sched_barrier(0);
        // stage q/2 + 1 (read from the next phase on) has landed: stages
        // q/2 + 1 .. q/2 + 3 were in flight
        if (EVEN)
            wait_vmcnt_lds_barrier<2 * LPW>();
        else
            lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // second half: step-1 MFMAs, step-0 fragments of phase q+1, packed
        // codes of phase q+2
        read_frags(q + 1, 0, f0);
        read_packed(q + 2);
        mfma_step(f1);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int q = 0; q < nph; q += 2) {
        phase(std::integral_constant<bool, true>(), q);
        phase(std::integral_constant<bool, false>(), q + 1);
    }
    wait_global_loads();

    const int mw = m0 + 128 * wm, nw = n0 + 64 * wn;
    int mbs[8], nbs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        mbs[i] = mw + 32 * (i >> 1);
        nbs[i] = nw + 32 * (i & 1);
    }
    if constexpr (!SPLIT) lds_barrier();  // every wavefront is past its last fragment reads
    finish_frags<SPLIT, 8, 2>(p, lane, [&](auto ic) -> float16_t & {
        constexpr int i = decltype(ic)::value;
        return acc[i >> 1][i & 1];
    }, mbs, nbs, reinterpret_cast<float *>(lds) + wave * epi_tile_floats<2>(), split);
}

// Split-K epilogue: wavefront w takes the G horizontally adjacent output
// fragments (w / FNG, G (w % FNG) + i), i < G, FNG = ceil(FN / G), adds each
// one's ks partials in split order (s = 0, 1, ...; the same order on every
// run) and runs the epilogue on the sums.  A fragment past the output (FN not
// a multiple of G) reads nothing and stores nothing.
template <int G>
__global__ __launch_bounds__(256) void splitk_epi_kernel(GemmArgs p_arg) {
    const GemmArgs &p = kernel_gemm_args();
    (void)p_arg;
    __shared__ __attribute__((aligned(16))) float tiles[4][epi_tile_floats<G>()];
    const int FM = (p.M + 31) >> 5, FN = (p.N + 31) >> 5, FNG = (FN + G - 1) / G;
    const int w = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (w >= FM * FNG) return;  // whole wavefronts
    const int lane = threadIdx.x & 63;
    const int fi = w / FNG, fj = G * (w - fi * FNG);
    const int64_t fstride = (int64_t)FM * FN * 1024;
    int mbs[G], nbs[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        mbs[i] = 32 * fi;
        nbs[i] = 32 * (fj + i);
    }
    // the epilogue's operands (row and column scales, LoRA rows, C) are
    // loaded first, so their latency overlaps that of the partials
    EpiIn in[G];
    float dx[16];
    epi_load_dx(p, mbs[0], lane, dx);
#pragma unroll
    for (int i = 0; i < G; ++i) epi_load(p, mbs[i], nbs[i], lane, in[i]);
    u32x4 cv[2 * G];
    const bool cpre = epi_c_prefetch<G>(p, lane, mbs[0], nbs[0], cv);
    float16_t acc[G];
#pragma unroll
    for (int f = 0; f < G; ++f) {
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[f][e] = 0.0f;
        if (fj + f >= FN) continue;
        const float *src = p.part + ((int64_t)fi * FN + fj + f) * 1024 + 4 * lane;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const float4_t v = *reinterpret_cast<const float4_t *>(src + 256 * e4);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[f][4 * e4 + q] = v[q];
        }
        for (int s = 1; s < p.ks; ++s) {
            const float *ps = src + s * fstride;
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const float4_t v = *reinterpret_cast<const float4_t *>(ps + 256 * e4);
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[f][4 * e4 + q] = acc[f][4 * e4 + q] + v[q];
            }
        }
    }
    float *tile = tiles[threadIdx.x >> 6];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        epi_finish(p, acc[i], mbs[i], nbs[i], lane, in[i], dx);
        epi_to_tile<G>(tile, acc[i], i, lane);
    }
    // LDS operations of one wavefront complete in order; the wait keeps the
    // compiler from treating the tile reads as independent
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    epi_rows<G>(p, lane, tile, mbs[0], nbs[0], cpre, cv);
}

// ---- launch plan ------------------------------------------------------------
// Kernel: 0 = the 256 x 256 kernel (K % 64 == 0), 1..4 = the main kernel with
// wavefronts (WM, WN, WK) = (2,2,1), (2,1,2), (1,2,2), (1,1,4).  ks: K ranges
// split across workgroups, summed by the split-K epilogue kernel.
// Column split (n1 > 0, ks == 1): output columns [0, n1) run as one launch of
// `kernel`, chosen so that its 256 x 256 tiles fill whole rounds of the CUs,
// and columns [n1, N) as a second launch of `kernel2` with smaller tiles, so
// the last, partly filled round of one launch becomes a full round of smaller
// tiles.
struct GemmPlan {
    int kernel;
    int ks;
    bool fuse;    // the LoRA-down runs as a row of workgroups of the split-K launch
    int n1 = 0;   // column split: columns of the first launch (multiple of 256), 0: none
    int kernel2 = 0;
};

struct KernelShape {
    int bm, bn, wk;
    // cost model fitted to measured launches (MI355X, 256 CUs): per-workgroup
    // rate with the whole chip busy and with it nearly idle (TFLOP/s per CU),
    // fixed cost per round of workgroups (pipeline fill, epilogue; us)
    double rate_full, rate_idle, fixed_us;
};
static constexpr KernelShape kKernels[5] = {{256, 256, 1, 5.11, 7.21, 10.3},
                                            {256, 256, 1, 5.22, 7.25, 15.5},
                                            {256, 128, 2, 4.55, 6.12, 10.9},
                                            {128, 256, 2, 4.59, 6.49, 11.0},
                                            {128, 128, 4, 4.04, 5.65, 8.1}};
static constexpr double kSecondLaunchUs = 3.5;  // the second launch of a column split
static constexpr double kPartialTBs = 12.6;  // partials out and back (MALL-resident)
static constexpr double kSplitEpiUs = 0.5;   // the extra epilogue launch

static size_t partial_bytes(int64_t M, int64_t N, int ks) {
    if (ks <= 1) return 0;
    return (size_t)ks * (size_t)((M + 31) / 32) * (size_t)((N + 31) / 32) * 4096u;
}

// Estimated duration (microseconds), round by round: each round of at most
// one workgroup per CU costs a fixed amount plus one workgroup's FLOPs at a
// per-CU rate that rises as fewer CUs are busy (clock headroom, memory
// bandwidth per CU); a K split adds the partials' round trip and the
// epilogue launch.  Fitted to unsplit launches of every kernel on the layer
// shapes and to column-split pairs (MI355X, 4 % rms error).
static double plan_cost(int64_t M, int64_t N, int64_t K, int kernel, int ks, int cus) {
    const KernelShape &k = kKernels[kernel];
    const int64_t wgs = ((M + k.bm - 1) / k.bm) * ((N + k.bn - 1) / k.bn) * ks;
    const double wg_flop = 2.0 * k.bm * k.bn * (double)K / ks;
    double t = 0.0;
    for (int64_t left = wgs; left > 0; left -= cus) {
        const double fill = (double)(left < cus ? left : cus) / cus;
        const double rate = k.rate_full + (k.rate_idle - k.rate_full) * (1.0 - fill);
        t += k.fixed_us + wg_flop / (rate * 1e6);
    }
    if (ks > 1) t += 2.0 * (double)partial_bytes(M, N, ks) / (kPartialTBs * 1e6) + kSplitEpiUs;
    return t;
}

// The LoRA-down product [M][Kl] x [Kl][rpad] of a GEMM: as a launch of its
// own before the GEMM, bound by reading X (BF16) from HBM; or fused into a
// split-K launch as one workgroup per output tile taking ceil(row groups /
// tiles) groups of 16 rows each (measured: about 1 us plus 1.9 us per 1024
// of Kl per group, 30% more with strided rank-operand rows).  A fused row
// occupies its CUs that long: the GEMM workgroups are list-scheduled onto
// the CUs after the busy down workgroups and the delay of the last one over
// the down-free schedule is the fused plan's extra cost.
struct DownPlan {
    int64_t kl;    // LoRA input width (0: no LoRA)
    bool strided;  // rank-operand rows strided (the input gradient's B)
    int rpad;      // ranks, rounded up to 16
};

// A launch of its own: one workgroup per 16 (32 from 4096) rows walks all of
// Kl (measured at 1024 rows: 3 us plus 2.0 us per 1024 of Kl with the
// pipelined kernel, 2.75 us with the 16-wavefront kernel that reads strided
// rank-operand rows below 4096 rows; from 4096 rows strided rows are first
// transposed, a launch of about 3 us), or the BF16 read of X at 3 TB/s when
// that is longer.
static double down_alone_us(int64_t M, const DownPlan &dp) {
    const double kk = (double)dp.kl / 1024.0, ranks = 1.0 + 0.25 * (dp.rpad / 16 - 1);
    const bool wide = M >= 4096, slow = dp.strided && !wide;
    const double rounds = (double)((M + (wide ? 32 : 16) * 256 - 1) / ((wide ? 32 : 16) * 256));
    const double lat = 3.0 + rounds * kk * (slow ? 2.75 : 2.0) * (wide ? 1.5 : 1.0) * ranks;
    const double bw = 3.0 + (double)M * (double)dp.kl * 2.0 / 3.0e6;
    return (lat > bw ? lat : bw) + (dp.strided && wide ? 3.0 : 0.0);
}

static double down_fused_extra_us(int64_t M, int64_t N, int kernel, int ks, int cus, double t_main,
                                  const DownPlan &dp) {
    const KernelShape &k = kKernels[kernel];
    const int64_t tiles = ((M + k.bm - 1) / k.bm) * ((N + k.bn - 1) / k.bn), wgs = tiles * ks;
    const int64_t groups = (M + 15) / 16;
    const int64_t busy = std::min<int64_t>(std::min(groups, tiles), cus);  // down workgroups with rows
    const int64_t per = (groups + tiles - 1) / tiles;                      // row groups each
    const double t_down = (double)per * (1.0 + 1.9 * (double)dp.kl / 1024.0) * (dp.strided ? 1.3 : 1.0) *
                          (1.0 + 0.25 * (dp.rpad / 16 - 1));
    const int64_t rounds = (wgs + cus - 1) / cus;
    const double t_wg = t_main / (double)rounds;
    // cus - busy CUs complete a GEMM workgroup at every multiple of t_wg, the
    // busy ones at t_down + multiples of t_wg; the launch ends at the first
    // such time by which all wgs can have completed
    const int64_t F = cus - busy, B = busy;
    auto done_by = [&](double T) {
        const int64_t a = (int64_t)(T / t_wg + 1e-9);
        const int64_t b = T > t_down ? (int64_t)((T - t_down) / t_wg + 1e-9) : 0;
        return F * a + B * b;
    };
    double end = 1e300;
    if (F > 0)
        for (int64_t a = 1; a <= wgs / F + 1; ++a)
            if (done_by(a * t_wg) >= wgs) {
                end = a * t_wg;
                break;
            }
    if (B > 0)
        for (int64_t b = 1; b <= wgs / B + 1; ++b)
            if (t_down + b * t_wg < end && done_by(t_down + b * t_wg) >= wgs) {
                end = t_down + b * t_wg;
                break;
            }
    if (end > 1e299) end = t_down + (double)rounds * t_wg;
    if (end < t_down) end = t_down;  // the down workgroups themselves
    const double base = (double)rounds * t_wg;
    return end > base ? end - base : 0.0;
}

static GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int cus, const DownPlan &dp = {0, false, 16}) {
    const int64_t ns = (K + kSK - 1) / kSK;
    GemmPlan best = {1, 1, false};
    double best_cost = 1e300;
    for (int kernel = 0; kernel < 5; ++kernel) {
        if (kernel == 0 && K % kSK != 0) continue;
        const int wk = kKernels[kernel].wk;
        for (int ks : {1, 2, 3, 4, 6, 8, 12, 16}) {
            if (ks > 1 && K % kSK != 0) break;       // ragged K: no split
            if (ns % ((int64_t)wk * ks) != 0) continue;
            if (ks > 1 && ns / ((int64_t)wk * ks) < 2) continue;  // at least two stages per wavefront
            const double c = plan_cost(M, N, K, kernel, ks, cus);
            double total = c;
            bool fuse = false;
            if (dp.kl > 0) {
                total = c + down_alone_us(M, dp);
                // strided rank-operand rows: fused only at one row group per
                // workgroup (longer ones contend with the GEMM's loads)
                const KernelShape &kk = kKernels[kernel];
                const int64_t tiles = ((M + kk.bm - 1) / kk.bm) * ((N + kk.bn - 1) / kk.bn);
                if (ks > 1 && dp.rpad <= 64 && (!dp.strided || (M + 15) / 16 <= tiles)) {
                    const double t_main = c - (2.0 * (double)partial_bytes(M, N, ks) / (kPartialTBs * 1e6) + kSplitEpiUs);
                    const double fused = c + down_fused_extra_us(M, N, kernel, ks, cus, t_main, dp);
                    if (fused <= total) {
                        total = fused;
                        fuse = true;
                    }
                }
            }
            if (total < best_cost) {
                best_cost = total;
                best = {kernel, ks, fuse};
            }
        }
    }
    // column split: the 256 x 256 kernel on whole rounds of tiles, smaller
    // tiles for the rest of the columns (no K split, no partial sums)
    const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256;
    if (K % kSK == 0 && tm * tn > cus && (tm * tn) % cus != 0) {
        const double down = dp.kl > 0 ? down_alone_us(M, dp) : 0.0;
        for (int64_t rounds = 1; rounds * cus < tm * tn; ++rounds) {
            const int64_t c = rounds * cus / tm;  // whole tile columns in these rounds
            if (c <= 0 || c >= tn) continue;
            const int64_t n1 = 256 * c;
            const double c0 = plan_cost(M, n1, K, 0, 1, cus);
            for (int k2 = 2; k2 < 5; ++k2) {
                if (ns % kKernels[k2].wk != 0) continue;
                const double total = c0 + plan_cost(M, N - n1, K, k2, 1, cus) + kSecondLaunchUs + down;
                if (total < best_cost) {
                    best_cost = total;
                    best = {0, 1, false, (int)n1, k2};
                }
            }
        }
    }
    return best;
}

static size_t lora_ws_bytes(int64_t M, int32_t r) {
    if (r <= 0) return 0;
    return (size_t)round_up(M * round_up(r, 16) * 2, 256);
}

// B^T [r][N] for the input gradient's LoRA-down (so its rank operand has
// contiguous rows).
static size_t bt_bytes(int64_t N, int32_t r) { return r > 0 ? (size_t)round_up((int64_t)r * N * 2, 256) : 0; }

// Workspace of one projection: the LoRA-down product, the split-K partials of
// either direction (forward [M][N] over K, input gradient [M][K] over N), B^T
// [r][N] and A^T [K][r] (the input gradient's rank operands with contiguous
// rows).
size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, int32_t r) {
    const int cus = device_cus();
    const int rp = (int)round_up(r > 0 ? r : 16, 16);
    const GemmPlan f = plan_gemm(M, N, K, cus, DownPlan{r > 0 ? K : 0, false, rp}),
                   b = plan_gemm(M, K, N, cus, DownPlan{r > 0 ? N : 0, true, rp});
    const size_t pf = partial_bytes(M, N, f.ks), pb = partial_bytes(M, K, b.ks);
    return lora_ws_bytes(M, r) + (pf > pb ? pf : pb) + bt_bytes(N, r) + bt_bytes(K, r);
}

// Pt [r][Kl] = P^T for P [Kl][r] row-major (the input gradient's B) in
// workgroups [0, ceil(Kl r / 256)), the side job of d in the rest.
__global__ __launch_bounds__(256) void lora_transpose_kernel(const uint16_t *P, int Kl, int r, uint16_t *Pt,
                                                             DownArgs d) {
    const int64_t own = ((int64_t)Kl * r + 255) / 256;
    if ((int64_t)blockIdx.x >= own) {
        side_transpose(d, (int64_t)blockIdx.x - own, (int64_t)gridDim.x - own);
        return;
    }
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)Kl * r) return;
    const int j = (int)(i / Kl), k = (int)(i % Kl);
    Pt[i] = P[(int64_t)k * r + j];
}

template <int WM, int WN, int WK>
static void launch_gemm_cfg(const GemmArgs &a, hipStream_t st) {
    using SH = GemmShape<WM, WN, WK>;
    const int tiles = ((a.M + SH::BM - 1) / SH::BM) * ((a.N + SH::BN - 1) / SH::BN);
    const dim3 grid((unsigned)tiles, (unsigned)(a.ks + (a.ks > 1 && a.down.X ? 1 : 0)));
    if (a.ks > 1)  // the plan splits K only when K % 64 == 0
        hipLaunchKernelGGL((gemm_kernel<WM, WN, WK, true, true>), grid, dim3(256), 0, st, a);
    else if (a.K % kSK == 0)
        hipLaunchKernelGGL((gemm_kernel<WM, WN, WK, true, false>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((gemm_kernel<WM, WN, WK, false, false>), grid, dim3(256), 0, st, a);
}

static pact_status launch_plan(const GemmArgs &a, int kernel, hipStream_t st) {
    switch (kernel) {
        case 0: {
            const int tiles = ((a.M + 255) / 256) * ((a.N + 255) / 256);
            const dim3 grid((unsigned)tiles, (unsigned)(a.ks + (a.ks > 1 && a.down.X ? 1 : 0)));
            if (a.ks > 1)
                hipLaunchKernelGGL(gemm8_kernel<true>, grid, dim3(512), 0, st, a);
            else
                hipLaunchKernelGGL(gemm8_kernel<false>, grid, dim3(512), 0, st, a);
            break;
        }
        case 1: launch_gemm_cfg<2, 2, 1>(a, st); break;
        case 2: launch_gemm_cfg<2, 1, 2>(a, st); break;
        case 3: launch_gemm_cfg<1, 2, 2>(a, st); break;
        default: launch_gemm_cfg<1, 1, 4>(a, st); break;
    }
    PACT_TRY(launch_status());
    if (a.ks > 1) {
        // one fragment per wavefront: more wavefronts, more loads in flight
        const int64_t frags = ((int64_t)(a.M + 31) / 32) * ((a.N + 31) / 32);
        hipLaunchKernelGGL(splitk_epi_kernel<1>, dim3((unsigned)((frags + 3) / 4)), dim3(256), 0, st, a);
        PACT_TRY(launch_status());
    }
    return PACT_OK;
}

// Projections of a grouped forward GEMM: output columns [col[g], col[g + 1])
// with LoRA A = P[g] [r][K], B = Q[g] [col[g + 1] - col[g]][r].
struct LoraGroups {
    int n;
    int col[kMaxGroups + 1];
    const uint16_t *P[kMaxGroups];
    const uint16_t *Q[kMaxGroups];
};

// Shared body of the forward and input-gradient entry points.
//   aq [M][Kc] NVFP4, bq [Nout][Kc] NVFP4, Xl [M][Kl] BF16 LoRA input,
//   P(j, k) = Psrc[j p_sj + k p_sk] (j < r, k < Kl), Q(n, j) = Qsrc[n q_sn + j q_sj];
//   or, with groups, the block-diagonal LoRA of groups->n projections (rank r each).
static pact_status gemm_common(const pact_nvfp4 *aq, const pact_nvfp4 *bq, const uint16_t *Xl,
                               int64_t ldx, int64_t Kl, const pact_lora *lora, const uint16_t *Psrc,
                               int64_t p_sj, int64_t p_sk, const uint16_t *Qsrc, int64_t q_sn,
                               int64_t q_sj, const uint16_t *C, uint16_t *Y, int64_t ldy, void *ws,
                               size_t ws_bytes, void *stream, const LoraGroups *groups = nullptr) {
    if (!aq || !bq) return PACT_ERR_INVALID_ARG;
    const int64_t M = aq->rows, Kc = aq->cols, Nout = bq->rows;
    if (M < 0 || Kc < 0 || Nout < 0 || bq->cols != Kc) return PACT_ERR_INVALID_ARG;
    if (Kc % 16 != 0) return PACT_ERR_UNSUPPORTED_SHAPE;
    if (M > INT32_MAX || Nout > INT32_MAX || Kc > INT32_MAX) return PACT_ERR_UNSUPPORTED_SHAPE;
    // operand codes are addressed with 32-bit offsets
    if (M * (Kc / 2) > (int64_t)UINT32_MAX || Nout * (Kc / 2) > (int64_t)UINT32_MAX)
        return PACT_ERR_UNSUPPORTED_SHAPE;
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
    a.a_bytes = (uint32_t)(M * (Kc / 2));
    a.b_bytes = (uint32_t)(Nout * (Kc / 2));
    a.C = C;
    a.Y = Y;
    a.ldy = ldy;
    a.y_rec = M * ldy * 2 < ((int64_t)1 << 31) ? (uint32_t)(M * ldy * 2) : 0u;
    const int ng = groups && r > 0 ? groups->n : 1;
    const size_t t_bytes = lora_ws_bytes(M, ng * (int)round_up(r, 16));
    if (r > 0) {
        if (!ws || ws_bytes < t_bytes) return PACT_ERR_WORKSPACE;
        if (!aligned16(ws)) return PACT_ERR_MISALIGNED;
    }
    // K split across workgroups when the plan asks for it and the workspace
    // holds the partials (after the LoRA-down product); otherwise one pass
    GemmPlan plan = plan_gemm(M, Nout, Kc, device_cus(),
                              DownPlan{r > 0 ? Kl : 0, p_sk != 1, ng * (int)round_up(r > 0 ? r : 16, 16)});
    const size_t p_bytes = partial_bytes(M, Nout, plan.ks);
    if (plan.ks > 1 && (!ws || !aligned16(ws) || ws_bytes < t_bytes + p_bytes)) {
        plan.ks = 1;
        plan.fuse = false;
    }
    a.ks = plan.ks;
    a.part = plan.ks > 1 ? reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + t_bytes) : nullptr;
    if (r > 0) {
        const int rpad = (int)round_up(r, 16);
        uint16_t *T = static_cast<uint16_t *>(ws);
        DownArgs d = {Xl, ldx, (int)M, (int)Kl, Psrc, p_sj, p_sk, r, ng * rpad, 0, lora->scale, T};
        a.ngroups = ng;
        if (ng > 1) {
            d.ngroups = ng;
            d.grp_rpad = rpad;
            for (int g = 0; g < ng; ++g) {
                d.Pg[g] = groups->P[g];
                a.Qg[g] = groups->Q[g];
            }
            for (int g = 0; g <= ng; ++g) a.gcol[g] = groups->col[g];
        }
        const size_t bt_off = t_bytes + (plan.ks > 1 ? p_bytes : 0), at_off = bt_off + bt_bytes(Kl, r);
        // LoRA-up operand with strided rows (the input gradient's A [r][Nout]):
        // A^T [Nout][r] in the workspace, written by side workgroups of the
        // launch before the epilogue, so the epilogue reads a rank row of 16
        // bytes per instruction
        if (q_sn == 1 && q_sj == Nout && ng == 1 && (r & 7) == 0 && ws_bytes >= at_off + bt_bytes(Nout, r)) {
            uint16_t *At = reinterpret_cast<uint16_t *>(static_cast<uint8_t *>(ws) + at_off);
            d.side_B = Qsrc;
            d.side_Bt = At;
            d.side_N = r;
            d.side_r = (int)Nout;
            Qsrc = At;
            q_sn = r;
            q_sj = 1;
        }
        if (plan.fuse && plan.ks > 1 && ng * rpad <= 64) {
            a.down = d;  // computed by workgroups of the split-K main kernel
        } else if (d.p_sk == (int64_t)r && d.p_sj == 1 && M >= 4096 &&
                   ws_bytes >= bt_off + bt_bytes(Kl, r)) {
            // rank operand with strided rows (the input gradient's B [N][r]):
            // transpose it once so the pipelined LoRA-down reads contiguous rows
            uint16_t *Pt = reinterpret_cast<uint16_t *>(static_cast<uint8_t *>(ws) + bt_off);
            const int own = (int)((Kl * r + 255) / 256);
            hipLaunchKernelGGL(lora_transpose_kernel, dim3((unsigned)(own + side_blocks(d, 256))), dim3(256), 0, st,
                               Psrc, (int)Kl, r, Pt, d);
            PACT_TRY(launch_status());
            d.Ps = Pt;
            d.p_sj = Kl;
            d.p_sk = 1;
            d.side_Bt = nullptr;  // done
            PACT_TRY(launch_lora_down(d, st));
        } else {
            PACT_TRY(launch_lora_down(d, st));
        }
        a.T = T;
        a.Qs = Qsrc;
        a.q_sn = q_sn;
        a.q_sj = q_sj;
        a.r = r;
        a.rpad = rpad;
        a.tld = ng * rpad;
    }
    if (plan.n1 > 0 && plan.n1 < a.N) {
        // column split: columns [0, n1) with plan.kernel, [n1, N) with
        // plan.kernel2 (the same operands, shifted by n1 output columns;
        // group boundaries of a grouped LoRA shift with them)
        GemmArgs b = a;
        a.N = plan.n1;
        a.b_bytes = (uint32_t)((int64_t)plan.n1 * (Kc / 2));
        PACT_TRY(launch_plan(a, plan.kernel, st));
        const int64_t n1 = plan.n1;
        b.N = (int)(Nout - n1);
        b.b_codes += n1 * (Kc / 2);
        b.b_scales += n1 * (Kc / 16);
        b.b_d += n1;
        b.b_bytes = (uint32_t)((Nout - n1) * (Kc / 2));
        b.Y += n1;
        if (b.C) b.C += n1;
        if (b.T) {
            if (b.ngroups > 1) {
                for (int g = 0; g <= b.ngroups; ++g) b.gcol[g] -= (int)n1;
            } else {
                b.Qs += n1 * b.q_sn;
            }
        }
        return launch_plan(b, plan.kernel2, st);
    }
    return launch_plan(a, plan.kernel, st);
}

}  // namespace pact

using namespace pact;

extern "C" pact_status pact_debug_gemm_plan(int64_t M, int64_t N, int64_t K, int32_t r, int32_t dgrad,
                                            int32_t *kernel, int32_t *ks, int32_t *fused) {
    if (M < 0 || N < 0 || K < 0 || r < 0 || r > 256 || !kernel || !ks) return PACT_ERR_INVALID_ARG;
    const GemmPlan plan =
        plan_gemm(M, N, K, device_cus(), DownPlan{r > 0 ? K : 0, dgrad != 0, (int)round_up(r > 0 ? r : 16, 16)});
    *kernel = plan.kernel;
    *ks = plan.ks;
    if (fused) *fused = plan.fuse ? 1 : 0;
    return PACT_OK;
}

extern "C" pact_status pact_debug_gemm_plan_columns(int64_t M, int64_t N, int64_t K, int32_t r, int32_t dgrad,
                                                    int32_t *n1, int32_t *kernel2) {
    if (M < 0 || N < 0 || K < 0 || r < 0 || r > 256 || !n1 || !kernel2) return PACT_ERR_INVALID_ARG;
    const GemmPlan plan =
        plan_gemm(M, N, K, device_cus(), DownPlan{r > 0 ? K : 0, dgrad != 0, (int)round_up(r > 0 ? r : 16, 16)});
    *n1 = plan.n1;
    *kernel2 = plan.kernel2;
    return PACT_OK;
}

extern "C" pact_status pact_debug_lora_down_plan(int64_t M, int64_t N, int64_t K, int32_t r, int32_t ngroups,
                                                 int32_t dgrad, int32_t *route, int32_t *npass, int32_t *rg,
                                                 int32_t *rows_per_wave, int32_t *waves) {
    if (M < 0 || N < 0 || K < 0 || r < 1 || ngroups < 1 || ngroups > kMaxGroups || (dgrad && ngroups != 1) ||
        ngroups * round_up(r, 16) > 256 || !route || !npass || !rg || !rows_per_wave || !waves)
        return PACT_ERR_INVALID_ARG;
    const int rpad = ngroups * (int)round_up(r, 16);
    const GemmPlan plan = plan_gemm(M, N, K, device_cus(), DownPlan{K, dgrad != 0, rpad});
    *npass = 0;
    if (plan.fuse && plan.ks > 1 && rpad <= 64) {
        *route = 1;
        return PACT_OK;
    }
    // the input gradient's rank operand B [N][r] has strided rank rows (unless r == 1)
    const bool strided = dgrad && r > 1;
    *route = dgrad && M >= 4096 ? 3 : (strided ? 4 : 2);
    for (int j0 = 0; j0 < rpad; j0 += 64) {
        const int i = (*npass)++;
        if (*route == 4) {
            rg[i] = (rpad - j0) / 16 < 4 ? (rpad - j0) / 16 : 4;
            rows_per_wave[i] = 1;
            waves[i] = kDownWaves;
        } else {
            const PipePass pp = pipe_pass(M, rpad, j0);
            rg[i] = pp.rg;
            rows_per_wave[i] = pp.rpw;
            waves[i] = pp.nw;
        }
    }
    return PACT_OK;
}

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

extern "C" pact_status pact_gemm_nvfp4_fwd_grouped(const pact_nvfp4 *Xq, const uint16_t *X, int64_t ld_x,
                                                   const pact_nvfp4 *W_fwd, int32_t ngroups,
                                                   const int64_t *group_rows, const pact_lora *loras,
                                                   uint16_t *Y, int64_t ld_y, void *ws, size_t ws_bytes,
                                                   void *stream) {
    if (!Xq || !W_fwd || !group_rows || ngroups < 1 || ngroups > kMaxGroups) return PACT_ERR_INVALID_ARG;
    const int64_t K = Xq->cols;
    LoraGroups gr = {};
    gr.n = ngroups;
    int64_t col = 0;
    for (int g = 0; g < ngroups; ++g) {
        if (group_rows[g] < 0) return PACT_ERR_INVALID_ARG;
        if (group_rows[g] % 32 != 0) return PACT_ERR_UNSUPPORTED_SHAPE;
        gr.col[g] = (int)col;
        col += group_rows[g];
        if (col > INT32_MAX) return PACT_ERR_UNSUPPORTED_SHAPE;
    }
    gr.col[ngroups] = (int)col;
    if (col != W_fwd->rows) return PACT_ERR_INVALID_ARG;
    int r = 0;
    float scale = 0.0f;
    if (loras) {
        r = loras[0].r;
        scale = loras[0].scale;
        for (int g = 0; g < ngroups; ++g) {
            if (loras[g].r != r || loras[g].scale != scale) return PACT_ERR_INVALID_ARG;
            if (r > 0 && (!loras[g].A || !loras[g].B)) return PACT_ERR_INVALID_ARG;
            if (r > 0 && (!aligned16(loras[g].A) || !aligned16(loras[g].B))) return PACT_ERR_MISALIGNED;
            gr.P[g] = loras[g].A;
            gr.Q[g] = loras[g].B;
        }
        if (r < 0 || ngroups * round_up(r, 16) > 256) return PACT_ERR_INVALID_ARG;
    }
    const pact_lora lo = {gr.P[0], gr.Q[0], r, scale};
    // T = X [A_0; A_1; ...]^T (ranks of group g at g round_up(r, 16)), block-diagonal LoRA-up
    return gemm_common(Xq, W_fwd, X, ld_x, K, r > 0 ? &lo : nullptr, gr.P[0], K, 1, gr.Q[0], r, 1, nullptr, Y,
                       ld_y, ws, ws_bytes, stream, r > 0 ? &gr : nullptr);
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

// ---- forward GEMM with a library-owned workspace (no allocation) ----------
// For callers that cannot allocate device memory (code under stream capture,
// tight serving loops, harnesses that forbid allocation): the workspace of
// pact_gemm_nvfp4_fwd lives in this file-scope device array, one copy per
// GPU, held until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: its device address is looked up once per
// device and only that address is handed to kernels.
namespace {

constexpr size_t kScratchBytes = PACT_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on that device, with the device current).
pact_status scratch_on_current_device(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PACT_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return PACT_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PACT_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return PACT_OK;
}

}  // namespace

extern "C" size_t pact_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" pact_status pact_gemm_nvfp4_fwd_noalloc(const pact_nvfp4 *Xq, const uint16_t *X, int64_t ld_x,
                                                   const pact_nvfp4 *W_fwd, const pact_lora *lora,
                                                   const uint16_t *C, uint16_t *Y, int64_t ld_y, void *stream) {
    if (!Xq || !W_fwd) return PACT_ERR_INVALID_ARG;
    const int r = lora ? lora->r : 0;
    // the LoRA-down product must fit; split-K partials and rank-operand
    // copies that do not fit are left out (one pass over K instead)
    if (r > 0 && (r > 256 || Xq->rows < 0 || lora_ws_bytes(Xq->rows, r) > kScratchBytes)) return PACT_ERR_WORKSPACE;
    void *ws = nullptr;
    PACT_TRY(scratch_on_current_device(&ws));
    const int64_t K = Xq->cols;
    return gemm_common(Xq, W_fwd, X, ld_x, K, lora, lora ? lora->A : nullptr, K, 1, lora ? lora->B : nullptr, r, 1,
                       C, Y, ld_y, ws, kScratchBytes, stream);
}
