// pact_gemm.hip -- NVFP4 GEMM of the frozen projections on gfx950 MFMA, with
// the BF16 LoRA term in the epilogue.
//   forward: Y  = bf16(d_x d_w (Xq . W_fwd^T) + s (bf16(X A^T)) B^T (+ C))
//   dgrad:   dX = bf16(d_dy d_wb (dYq . W_bwd^T) + s (bf16(dY B)) A (+ C))
// (simolm.com PACT blog, section "Method", first bullet: NVFP4 GEMMs with FP32
// accumulation and BF16 output for the forward and the input gradient; the
// adapters stay BF16, closing paragraph of that section.)
//
// Both passes are one "TN" kernel: operand rows are K-contiguous NVFP4 rows.
// The E2M1 x E4M3 products are exact in FP16 (at most 6 significant bits,
// magnitudes in [2^-10, 2688]), so the kernel decodes each 8-code dword with
// the gfx950 FP4->FP16 converter plus one packed FP16 multiply by the block
// scale and feeds v_mfma_f32_32x32x16_f16; the FP32 accumulators then hold the
// sum of exact products.  Row scales are applied in the epilogue.  The
// summation order over K is the MFMA's own (any order is admitted).
//
// Tiling: a workgroup of 4 wavefronts computes a BM x BN tile (2 x 2 waves,
// each (BM/2) x (BN/2) as 32x32 fragments).  Each K stage is 128 elements:
// the packed codes (64 B per row) and 8 scale bytes per row are staged in LDS
// (double-buffered; the next stage's global loads are in flight while the
// current one is consumed).  Codes are laid out in LDS in fragment order so
// that one ds_read_b128 per lane fetches 32 codes of its row: lane (r, h) of a
// 32-row group holds K elements [32h, 32h + 32) of each 64-element half-stage,
// and MFMA step i consumes dword i, i.e. K [8i, 8i+8) from lanes h = 0 and
// [32 + 8i, 32 + 8i + 8) from lanes h = 1 -- the same K permutation for both
// operands, so every product pairs matching K indices.
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
    const uint16_t *T;  // [M][rpad] LoRA-down product (BF16) or nullptr
    const uint16_t *Q;  // [N][rpad] LoRA-up operand (BF16)
    int rpad;
    float s;
    const uint16_t *C;  // nullable, leading dim ldy
    uint16_t *Y;
    int64_t ldy;
};

constexpr int kBK = 128;  // K elements per stage

__device__ __forceinline__ half8_t decode8(uint32_t w, half2_t sc) {
    half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc;
    half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc;
    half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc;
    half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc;
    half8_t r;
    r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
    r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
    return r;
}

__device__ __forceinline__ half2_t scale_h2(uint32_t byte) {
    const _Float16 h = (_Float16)e4m3_to_f32(byte);  // exact: E4M3 is a subset of FP16
    half2_t r;
    r[0] = h;
    r[1] = h;
    return r;
}

template <int ROWS, bool K32>
__device__ __forceinline__ void load_codes(const uint8_t *codes, int row0, int nrows, int K, int k0,
                                           u32x4 (&reg)[ROWS * 4 / 256 > 0 ? ROWS * 4 / 256 : 1]) {
    constexpr int PER = ROWS * 4 / 256;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int c = tid + 256 * i;
        const int r = c >> 2, q = c & 3;
        const int kk = k0 + 32 * q;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row0 + r < nrows) {
            const uint8_t *p = codes + (int64_t)(row0 + r) * (K / 2) + kk / 2;
            if (K32) {
                if (kk < K) v = *reinterpret_cast<const u32x4 *>(p);
            } else {
                if (kk < K) {
                    const u32x2 lo = *reinterpret_cast<const u32x2 *>(p);
                    v.x = lo.x;
                    v.y = lo.y;
                }
                if (kk + 16 < K) {
                    const u32x2 hi = *reinterpret_cast<const u32x2 *>(p + 8);
                    v.z = hi.x;
                    v.w = hi.y;
                }
            }
        }
        reg[i] = v;
    }
}

template <int ROWS>
__device__ __forceinline__ void store_codes_lds(uint8_t *lds, const u32x4 (&reg)[ROWS * 4 / 256 > 0 ? ROWS * 4 / 256 : 1]) {
    constexpr int PER = ROWS * 4 / 256;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int c = tid + 256 * i;
        const int r = c >> 2, q = c & 3;
        const int g = r >> 5, j = q >> 1, h = q & 1;
        const int lane = (r & 31) + 32 * h;
        *reinterpret_cast<u32x4 *>(lds + (((g * 2 + j) * 64 + lane) << 4)) = reg[i];
    }
}

__device__ __forceinline__ u32x2 load_scales(const uint8_t *scales, int row, int nrows, int K, int k0) {
    u32x2 v = {0u, 0u};
    if (row < nrows) {
        const int nblk = K / 16;
        const uint8_t *p = scales + (int64_t)row * nblk + k0 / 16;
        if ((nblk & 7) == 0 && k0 + kBK <= K) {
            v = *reinterpret_cast<const u32x2 *>(p);
        } else {
            uint32_t w[2] = {0u, 0u};
            for (int i = 0; i < 8; ++i)
                if (k0 / 16 + i < nblk) w[i >> 2] |= (uint32_t)p[i] << (8 * (i & 3));
            v.x = w[0];
            v.y = w[1];
        }
    }
    return v;
}

template <int BM, int BN, bool K32>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs p) {
    constexpr int FM = BM / 64;  // 32x32 fragments per wave along M
    constexpr int FN = BN / 64;
    constexpr int A_CODES = 0;
    constexpr int B_CODES = BM * 64;
    constexpr int A_SC = (BM + BN) * 64;
    constexpr int B_SC = A_SC + BM * 8;
    constexpr int STAGE = (BM + BN) * 72;
    constexpr int PA = BM * 4 / 256 > 0 ? BM * 4 / 256 : 1;
    constexpr int PB = BN * 4 / 256 > 0 ? BN * 4 / 256 : 1;
    static_assert(BM * 4 >= 256 && BN * 4 >= 256, "tile too small for the staging map");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_m = (p.M + BM - 1) / BM;
    const int bid = blockIdx.x;
    const int tm = bid % tiles_m, tn = bid / tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = p.K;
    const int nk = (K + kBK - 1) / kBK;

    float16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    u32x4 ra[PA], rb[PB];
    u32x2 sa = {0u, 0u}, sb = {0u, 0u};
    if (nk > 0) {
        load_codes<BM, K32>(p.a_codes, m0, p.M, K, 0, ra);
        load_codes<BN, K32>(p.b_codes, n0, p.N, K, 0, rb);
        if (tid < BM) sa = load_scales(p.a_scales, m0 + tid, p.M, K, 0);
        if (tid < BN) sb = load_scales(p.b_scales, n0 + tid, p.N, K, 0);
        store_codes_lds<BM>(lds + A_CODES, ra);
        store_codes_lds<BN>(lds + B_CODES, rb);
        if (tid < BM) *reinterpret_cast<u32x2 *>(lds + A_SC + tid * 8) = sa;
        if (tid < BN) *reinterpret_cast<u32x2 *>(lds + B_SC + tid * 8) = sb;
    }
    __syncthreads();

    const int h = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        uint8_t *base = lds + cur * STAGE;
        const bool more = kt + 1 < nk;
        if (more) {
            const int k0 = (kt + 1) * kBK;
            load_codes<BM, K32>(p.a_codes, m0, p.M, K, k0, ra);
            load_codes<BN, K32>(p.b_codes, n0, p.N, K, k0, rb);
            if (tid < BM) sa = load_scales(p.a_scales, m0 + tid, p.M, K, k0);
            if (tid < BN) sb = load_scales(p.b_scales, n0 + tid, p.N, K, k0);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            u32x4 ca[FM], cb[FN];
            uint32_t sca[FM], scb[FN];
#pragma unroll
            for (int f = 0; f < FM; ++f) {
                const int g = wm * FM + f;
                ca[f] = *reinterpret_cast<const u32x4 *>(base + A_CODES + (((g * 2 + j) * 64 + lane) << 4));
                const u32x2 s8 = *reinterpret_cast<const u32x2 *>(base + A_SC + (g * 32 + (lane & 31)) * 8);
                // scale bytes of blocks 4j + 2h and 4j + 2h + 1 of this stage
                const uint32_t word = j ? s8.y : s8.x;
                sca[f] = (word >> (16 * h)) & 0xFFFFu;
            }
#pragma unroll
            for (int f = 0; f < FN; ++f) {
                const int g = wn * FN + f;
                cb[f] = *reinterpret_cast<const u32x4 *>(base + B_CODES + (((g * 2 + j) * 64 + lane) << 4));
                const u32x2 s8 = *reinterpret_cast<const u32x2 *>(base + B_SC + (g * 32 + (lane & 31)) * 8);
                const uint32_t word = j ? s8.y : s8.x;
                scb[f] = (word >> (16 * h)) & 0xFFFFu;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                half8_t av[FM], bv[FN];
#pragma unroll
                for (int f = 0; f < FM; ++f)
                    av[f] = decode8(ca[f][i], scale_h2((sca[f] >> (8 * (i >> 1))) & 0xFFu));
#pragma unroll
                for (int f = 0; f < FN; ++f)
                    bv[f] = decode8(cb[f][i], scale_h2((scb[f] >> (8 * (i >> 1))) & 0xFFu));
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[fm], bv[fn], acc[fm][fn], 0, 0, 0);
            }
        }
        if (more) {
            uint8_t *nxt = lds + (cur ^ 1) * STAGE;
            store_codes_lds<BM>(nxt + A_CODES, ra);
            store_codes_lds<BN>(nxt + B_CODES, rb);
            if (tid < BM) *reinterpret_cast<u32x2 *>(nxt + A_SC + tid * 8) = sa;
            if (tid < BN) *reinterpret_cast<u32x2 *>(nxt + B_SC + tid * 8) = sb;
        }
        __syncthreads();
    }

    // ---- epilogue: row scales, LoRA term, residual, BF16 store ----
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int mb = m0 + (wm * FM + fm) * 32;
            const int nb = n0 + (wn * FN + fn) * 32;
            float16_t L;
#pragma unroll
            for (int e = 0; e < 16; ++e) L[e] = 0.0f;
            if (p.T) {
                const int mr = mb + (lane & 31);
                const int nr = nb + (lane & 31);
                for (int kk = 0; kk < p.rpad; kk += 16) {
                    bf16x8_t a, b;
                    u32x4 va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
                    if (mr < p.M) va = *reinterpret_cast<const u32x4 *>(p.T + (int64_t)mr * p.rpad + kk + 8 * h);
                    if (nr < p.N) vb = *reinterpret_cast<const u32x4 *>(p.Q + (int64_t)nr * p.rpad + kk + 8 * h);
                    a = __builtin_bit_cast(bf16x8_t, va);
                    b = __builtin_bit_cast(bf16x8_t, vb);
                    L = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, L, 0, 0, 0);
                }
            }
            const int n = nb + (lane & 31);
            if (n >= p.N) continue;
            const float dw = p.b_d[n];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = mb + 8 * (e >> 2) + 4 * h + (e & 3);
                if (m >= p.M) continue;
                float y = acc[fm][fn][e] * p.a_d[m];
                y = y * dw;
                if (p.T) {
                    const float sl = p.s * L[e];
                    y = y + sl;
                }
                const int64_t off = (int64_t)m * p.ldy + n;
                if (p.C) y = y + bf16_to_f32(p.C[off]);
                p.Y[off] = (uint16_t)f32_to_bf16_bits(y);
            }
        }
    }
}

// ---- LoRA helpers ----------------------------------------------------------
// Padded copies of the adapters: P [rpad][Kl] and Q [Nout][rpad], zero beyond r.
__global__ void prep_adapters_kernel(const uint16_t *P, int64_t p_sj, int64_t p_sk, int Kl,
                                     const uint16_t *Qs, int64_t q_sn, int64_t q_sj, int Nout, int r,
                                     int rpad, uint16_t *Pp, uint16_t *Qp) {
    const int64_t nP = (int64_t)rpad * Kl, nQ = (int64_t)Nout * rpad;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nP + nQ;
         i += (int64_t)gridDim.x * blockDim.x) {
        if (i < nP) {
            const int j = (int)(i / Kl);
            const int64_t k = i % Kl;
            Pp[i] = j < r ? P[j * p_sj + k * p_sk] : (uint16_t)0;
        } else {
            const int64_t t = i - nP;
            const int64_t n = t / rpad;
            const int j = (int)(t % rpad);
            Qp[t] = j < r ? Qs[n * q_sn + j * q_sj] : (uint16_t)0;
        }
    }
}

// T [M][rpad] = bf16(Xl [M][Kl] . Pp^T) with FP32 accumulation
// (v_mfma_f32_16x16x32_bf16: one wavefront per 16 rows).
__global__ __launch_bounds__(256) void lora_down_kernel(const uint16_t *X, int64_t ldx, int M, int Kl,
                                                        const uint16_t *Pp, int rpad, uint16_t *T) {
    const int lane = threadIdx.x & 63;
    const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int m0 = wv * 16;
    if (m0 >= M) return;
    const int row = m0 + (lane & 15);
    const int kg = 8 * (lane >> 4);
    const int nf = rpad / 16;
    for (int f = 0; f < nf; ++f) {
        float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        const uint16_t *prow = Pp + (int64_t)(16 * f + (lane & 15)) * Kl;
        for (int k0 = 0; k0 < Kl; k0 += 32) {
            const int k = k0 + kg;
            u32x4 va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
            if (k < Kl) {
                if (row < M) va = *reinterpret_cast<const u32x4 *>(X + (int64_t)row * ldx + k);
                vb = *reinterpret_cast<const u32x4 *>(prow + k);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va),
                                                          __builtin_bit_cast(bf16x8_t, vb), acc, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = m0 + 4 * (lane >> 4) + e;
            if (m < M) T[(int64_t)m * rpad + 16 * f + (lane & 15)] = (uint16_t)f32_to_bf16_bits(acc[e]);
        }
    }
}

struct LoraWs {
    uint16_t *T, *Pp, *Qp;
    size_t bytes;
};

static LoraWs lora_ws_layout(void *ws, int64_t M, int64_t Kl, int64_t Nout, int rpad) {
    LoraWs w;
    const int64_t t_b = round_up(M * rpad * 2, 256);
    const int64_t p_b = round_up((int64_t)rpad * Kl * 2, 256);
    const int64_t q_b = round_up(Nout * rpad * 2, 256);
    uint8_t *b = static_cast<uint8_t *>(ws);
    w.T = reinterpret_cast<uint16_t *>(b);
    w.Pp = reinterpret_cast<uint16_t *>(b + t_b);
    w.Qp = reinterpret_cast<uint16_t *>(b + t_b + p_b);
    w.bytes = (size_t)(t_b + p_b + q_b);
    return w;
}

size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, int32_t r) {
    if (r <= 0) return 0;
    const int rpad = (int)round_up(r, 16);
    const int64_t big = N > K ? N : K;
    return lora_ws_layout(nullptr, M, big, big, rpad).bytes;
}

template <int BM, int BN>
static void launch_gemm_cfg(const GemmArgs &a, hipStream_t st) {
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (a.K % 32 == 0)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, true>), dim3(tiles), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((gemm_kernel<BM, BN, false>), dim3(tiles), dim3(256), 0, st, a);
}

static pact_status run_gemm(const GemmArgs &a, hipStream_t st) {
    auto tiles = [&](int bm, int bn) {
        return (int64_t)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
    };
    if (tiles(256, 256) >= 192) launch_gemm_cfg<256, 256>(a, st);
    else if (tiles(256, 128) >= 192) launch_gemm_cfg<256, 128>(a, st);
    else if (tiles(128, 128) >= 128) launch_gemm_cfg<128, 128>(a, st);
    else launch_gemm_cfg<64, 64>(a, st);
    return launch_status();
}

// Shared body of the forward and input-gradient entry points.
//   aq [M][Kc] NVFP4, bq [Nout][Kc] NVFP4, Xl [M][Kl] BF16 LoRA input,
//   P(j, k) = Psrc[j p_sj + k p_sk] (j < r, k < Kl), Qs(n, j) = Qsrc[n q_sn + j q_sj].
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
        LoraWs w = lora_ws_layout(ws, M, Kl, Nout, rpad);
        const int64_t tot = (int64_t)rpad * Kl + Nout * rpad;
        const unsigned pb = (unsigned)((tot + 255) / 256 < 4096 ? (tot + 255) / 256 : 4096);
        hipLaunchKernelGGL(prep_adapters_kernel, dim3(pb), dim3(256), 0, st, Psrc, p_sj, p_sk, (int)Kl,
                           Qsrc, q_sn, q_sj, (int)Nout, r, rpad, w.Pp, w.Qp);
        PACT_TRY(launch_status());
        hipLaunchKernelGGL(lora_down_kernel, dim3((unsigned)((M + 63) / 64)), dim3(256), 0, st, Xl, ldx,
                           (int)M, (int)Kl, w.Pp, rpad, w.T);
        PACT_TRY(launch_status());
        a.T = w.T;
        a.Q = w.Qp;
        a.rpad = rpad;
        a.s = lora->scale;
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
