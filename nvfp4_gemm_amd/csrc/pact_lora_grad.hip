// pact_lora_grad.hip -- LoRA weight gradients on the NVFP4 stash:
//   X^ = bf16(deq(Xq)), T^ = bf16(s . X^ A^T), T' = bf16(s . dY B),
//   dB = dY^T T^  [N][r],   dA = T'^T X^  [r][K],   FP32 sums, FP32 outputs.
// (simolm.com PACT blog, section "Method", second bullet and closing
// paragraph: the activations kept for backward are NVFP4 copies and the
// adapters stay BF16; kongchang.com PEFT explainer: the LoRA update B A x.)
//
// X^ is never materialized: the LoRA-down of T^ and the contraction for dA
// decode the NVFP4 rows in registers.  Five launches: T^ (LoRA-down of the
// NVFP4 rows, whose extra workgroups also write B^T), T' (LoRA-down of dY),
// the token contraction for dB, the one for dA (whose extra workgroups sum
// dB's token splits in order), and the in-order sum of dA's splits.
#include "pact_device.h"
#include "pact_host.h"

namespace pact {

constexpr int kMaxSplits = 32;

// out[c * osc + j * osj] = sum over splits s = 0, 1, ... of part[s][c][j]
// (j < r, part rows of jw floats): the reduction of a token-split contraction.
struct RedArgs {
    const float *part;
    int ms, C, r, jw;
    float *out;
    int64_t osc, osj;
    int wgs;  // workgroups doing it
};

// One output per thread; all of its partials are loaded before the in-order sum.
__device__ __forceinline__ void reduce_splits(const RedArgs &a, int64_t i) {
    if (i >= (int64_t)a.C * a.r) return;
    const int cc = (int)(i / a.r), j = (int)(i % a.r);
    const float *src = a.part + (int64_t)cc * a.jw + j;
    const int64_t step = (int64_t)a.C * a.jw;
    float v[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) v[s] = s < a.ms ? src[s * step] : 0.0f;
    float sum = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s)
        if (s < a.ms) sum += v[s];
    a.out[cc * a.osc + j * a.osj] = sum;
}

__global__ __launch_bounds__(256) void lora_grad_reduce_kernel(RedArgs a) {
    reduce_splits(a, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

struct GradArgs {
    const uint16_t *V;  // BF16 V [M][C] (ldv), or
    int64_t ldv;
    const uint8_t *vc, *vs;  // NVFP4 V: codes [M][C/2], scales [M][C/16], row scales [M]
    const float *vd;
    const uint16_t *T;  // [M][ldt], ranks j < r (zero for r <= j < ldt)
    int64_t ldt;
    int M, C, r;
    int mchunk;   // tokens per workgroup (a multiple of kGradMT)
    int cblocks;  // column blocks; workgroup b < cblocks * msplit: block b % cblocks, split b / cblocks
    float *part;  // [msplit][C][32 JT] FP32 partials
    RedArgs side;  // workgroups past the contraction's reduce an earlier contraction's partials
};

constexpr int kGradMT = 64;  // tokens per LDS stage

// Both gradients contract over the tokens: out[c][j] = sum_m V[m][c] T[m][j].
// A workgroup of 4 wavefronts owns CB columns (each wavefront CB / 4, as
// 32-column MFMA tiles, v_mfma_f32_32x32x16_bf16 with D = out) and a token
// range in stages of 64 tokens: V [64][CB] and T [64][32 JT] are loaded with
// 16-byte row-contiguous loads (NVFP4 V: 16 code bytes, two scale bytes and
// the row scale per 32 columns, decoded to BF16), stored in LDS and read back
// as MFMA operands (lane (h, l) takes 8 consecutive tokens 8h.. of column or
// rank l).  The next stage's loads are issued before the current stage's
// MFMAs.  The token ranges (splits) of a column block give FP32 partials that
// a reduction sums in split order, so every run adds in the same order.  Loads
// past M or C read a clamped address and are zeroed.
template <int CB, int JT, bool NV>
__global__ __launch_bounds__(256) void lora_grad_kernel(GradArgs g) {
    constexpr int MT = kGradMT;
    constexpr int VS = CB + 8;  // LDS row strides (BF16 elements)
    constexpr int TW = 32 * JT;
    constexpr int TS = TW + 8;
    constexpr int CT = CB / 128;  // 32-column tiles per wavefront
    constexpr int VP = NV ? MT * CB / 32 / 256 : MT * CB / 8 / 256;  // per thread: 32-column parts or 16-byte pieces
    static_assert(VP >= 1 && MT * TW / 8 == 256 * JT, "staging covers the tiles");
    __shared__ uint16_t Vs[MT * VS];
    __shared__ uint16_t Ts[MT * TS];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nwg = g.cblocks * ((g.M + g.mchunk - 1) / g.mchunk);
    if ((int)blockIdx.x >= nwg) {  // side workgroup (uniform, before any barrier)
        reduce_splits(g.side, (int64_t)(blockIdx.x - nwg) * 256 + tid);
        return;
    }
    const int split = (int)blockIdx.x / g.cblocks;
    const int h = lane >> 5, l = lane & 31;
    const int c0 = ((int)blockIdx.x % g.cblocks) * CB;
    const int mb = split * g.mchunk, me = min(g.M, mb + g.mchunk);
    const bool c32 = (g.C & 31) == 0;
    u32x4 rv[VP];
    uint32_t rs[NV ? VP : 1];
    float rd[NV ? VP : 1];
    u32x4 rt[JT];
    auto gload = [&](int m0) {
#pragma unroll
        for (int i = 0; i < VP; ++i) {
            const int p = tid + 256 * i;
            if (NV) {
                const int row = p / (CB / 32), col = c0 + 32 * (p % (CB / 32));
                const int m = min(m0 + row, g.M - 1);
                const bool ok = m0 + row < me && col < g.C;
                const int cl = ok ? col : 0;
                const uint8_t *cr = g.vc + (int64_t)m * (g.C / 2) + cl / 2;
                const uint8_t *sr = g.vs + (int64_t)m * (g.C / 16) + cl / 16;
                uint32_t s2;
                if (c32) {
                    rv[i] = *reinterpret_cast<const u32x4 *>(cr);
                    s2 = *reinterpret_cast<const uint16_t *>(sr);
                } else {
                    const bool two = cl + 16 < g.C;
                    const u32x2 lo = *reinterpret_cast<const u32x2 *>(cr);
                    const u32x2 hi = *reinterpret_cast<const u32x2 *>(two ? cr + 8 : cr);
                    rv[i] = u32x4{lo.x, lo.y, hi.x, hi.y};
                    s2 = (uint32_t)sr[0] | ((uint32_t)sr[two ? 1 : 0] << 8);
                }
                if (!ok) s2 = 0u;
                else if (col + 16 >= g.C) s2 &= 0xFFu;
                rs[i] = s2;
                rd[i] = g.vd[m];
            } else {
                const int row = p / (CB / 8), col = c0 + 8 * (p % (CB / 8));
                const int m = min(m0 + row, g.M - 1);
                const bool ok = m0 + row < me && col < g.C;
                const u32x4 v = *reinterpret_cast<const u32x4 *>(g.V + (int64_t)m * g.ldv + (ok ? col : 0));
                rv[i] = ok ? v : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < JT; ++i) {
            const int p = tid + 256 * i;
            const int row = p / (TW / 8), col = 8 * (p % (TW / 8));
            const int m = min(m0 + row, g.M - 1);
            const bool ok = m0 + row < me && col < g.ldt;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(g.T + (int64_t)m * g.ldt + (ok ? col : 0));
            rt[i] = ok ? v : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < VP; ++i) {
            const int p = tid + 256 * i;
            if (NV) {
                const int row = p / (CB / 32), cc = 32 * (p % (CB / 32));
                const half2_t s0 = e4m3_to_h2(rs[i] & 0xFFu), s1 = e4m3_to_h2(rs[i] >> 8);
                u32x4 *dst = reinterpret_cast<u32x4 *>(&Vs[row * VS + cc]);
                dst[0] = dequant8_bf16(rv[i].x, s0, rd[i]);
                dst[1] = dequant8_bf16(rv[i].y, s0, rd[i]);
                dst[2] = dequant8_bf16(rv[i].z, s1, rd[i]);
                dst[3] = dequant8_bf16(rv[i].w, s1, rd[i]);
            } else {
                const int row = p / (CB / 8), cc = 8 * (p % (CB / 8));
                *reinterpret_cast<u32x4 *>(&Vs[row * VS + cc]) = rv[i];
            }
        }
#pragma unroll
        for (int i = 0; i < JT; ++i) {
            const int p = tid + 256 * i;
            const int row = p / (TW / 8), col = 8 * (p % (TW / 8));
            *reinterpret_cast<u32x4 *>(&Ts[row * TS + col]) = rt[i];
        }
    };
    // 8 BF16 values at LDS rows r0 + 8h .. r0 + 8h + 7 of column col (stride S)
    auto col8 = [&](const uint16_t *base, int S, int r0, int col) {
        uint32_t wv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            wv[q] = (uint32_t)base[(r0 + 8 * h + 2 * q) * S + col] |
                    ((uint32_t)base[(r0 + 8 * h + 2 * q + 1) * S + col] << 16);
        return __builtin_bit_cast(bf16x8_t, u32x4{wv[0], wv[1], wv[2], wv[3]});
    };
    float16_t acc[CT][JT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int t = 0; t < JT; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[ct][t][e] = 0.0f;
    if (mb < me) {
        gload(mb);
        for (int m0 = mb; m0 < me; m0 += MT) {
            __syncthreads();  // the previous stage's LDS reads are done
            lstore();
            if (m0 + MT < me) gload(m0 + MT);
            __syncthreads();
#pragma unroll
            for (int s = 0; s < MT / 16; ++s) {
                bf16x8_t b[JT];
#pragma unroll
                for (int t = 0; t < JT; ++t) b[t] = col8(Ts, TS, 16 * s, 32 * t + l);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const bf16x8_t a = col8(Vs, VS, 16 * s, (CB / 4) * w + 32 * ct + l);
#pragma unroll
                    for (int t = 0; t < JT; ++t)
                        acc[ct][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[t], acc[ct][t], 0, 0, 0);
                }
            }
        }
    }
    // accumulator element e of lane (h, l): column 8 (e / 4) + 4 h + e % 4 of the tile, rank 32 t + l
    float *dst = g.part + (int64_t)split * g.C * TW;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int t = 0; t < JT; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int cc = c0 + (CB / 4) * w + 32 * ct + 8 * (e >> 2) + 4 * h + (e & 3);
                if (cc < g.C) dst[(int64_t)cc * TW + 32 * t + l] = acc[ct][t][e];
            }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

struct GradPlan {
    int cb, msplit, mchunk;
};

// CB = 256 columns for wide BF16 outputs with many tokens (the rank operand
// is re-read once per column block), 128 otherwise; token splits for about 512
// workgroups, down to one stage per workgroup and at most kMaxSplits (swept
// on an MI355X over the layer shapes: at M = 1024 the extra splits take a
// contraction from 13-19 to 9-15 us).
static GradPlan grad_plan(int64_t M, int64_t C, bool nv) {
    const int cb = (!nv && C >= 4096 && M >= 4096) ? 256 : 128;
    const int64_t cblocks = (C + cb - 1) / cb;
    const int64_t target = (nv && M >= 4096) ? 1024 : 512;
    int64_t ms = (target + cblocks - 1) / cblocks;
    int64_t max_ms = (M + kGradMT - 1) / kGradMT;
    if (max_ms > kMaxSplits) max_ms = kMaxSplits;
    if (ms > max_ms) ms = max_ms;
    if (ms < 1) ms = 1;
    int64_t mchunk = (M + ms - 1) / ms;
    mchunk = (mchunk + kGradMT - 1) / kGradMT * kGradMT;
    ms = (M + mchunk - 1) / mchunk;
    return {cb, (int)(ms > 0 ? ms : 1), (int)mchunk};
}

static size_t grad_part_bytes(int64_t M, int64_t C, int r, bool nv) {
    const GradPlan p = grad_plan(M, C, nv);
    const int jt = (r + 31) / 32;
    return (size_t)round_up((int64_t)p.msplit * C * 32 * jt * 4, 256);
}

// Workspace: T^ and T' [M][rpad] BF16, B^T [r][N] BF16, the FP32 partials of
// both contractions (dB's are reduced during dA's contraction).
static size_t lora_grads_ws(int64_t M, int64_t N, int64_t K, int r) {
    const int64_t rpad = round_up(r, 16);
    const size_t t = (size_t)round_up(M * rpad * 2, 256);
    const size_t bt = (size_t)round_up((int64_t)r * N * 2, 256);
    return 2 * t + bt + grad_part_bytes(M, N, r, false) + grad_part_bytes(M, K, r, true);
}

template <bool NV>
static void launch_grad_kernel(const GradArgs &g, const GradPlan &p, int jt, hipStream_t st) {
    const dim3 grid((unsigned)(g.cblocks * p.msplit + g.side.wgs));
    if constexpr (!NV) {  // 256-column blocks only for BF16 operands (grad_plan)
        if (p.cb == 256) {
            if (jt == 1) hipLaunchKernelGGL((lora_grad_kernel<256, 1, NV>), grid, dim3(256), 0, st, g);
            else hipLaunchKernelGGL((lora_grad_kernel<256, 2, NV>), grid, dim3(256), 0, st, g);
            return;
        }
    }
    {
        if (jt == 1) hipLaunchKernelGGL((lora_grad_kernel<128, 1, NV>), grid, dim3(256), 0, st, g);
        else hipLaunchKernelGGL((lora_grad_kernel<128, 2, NV>), grid, dim3(256), 0, st, g);
    }
}

// Partials of V^T T over the tokens (V BF16 when g.vc is null, else NVFP4),
// plus g.side's reduction in extra workgroups; returns the reduction of this
// contraction's partials into out[c * osc + j * osj].
static RedArgs launch_grad(GradArgs g, float *out, int64_t osc, int64_t osj, hipStream_t st, pact_status *status) {
    const GradPlan p = grad_plan(g.M, g.C, g.vc != nullptr);
    const int jt = (g.r + 31) / 32;
    g.mchunk = p.mchunk;
    g.cblocks = (g.C + p.cb - 1) / p.cb;
    if (g.vc) launch_grad_kernel<true>(g, p, jt, st);
    else launch_grad_kernel<false>(g, p, jt, st);
    *status = launch_status();
    RedArgs red{g.part, p.msplit, g.C, g.r, 32 * jt, out, osc, osj, 0};
    red.wgs = (int)(((int64_t)g.C * g.r + 255) / 256);
    return red;
}

}  // namespace pact

using namespace pact;

extern "C" size_t pact_lora_grads_workspace(int64_t M, int64_t N, int64_t K, int32_t r) {
    if (M < 0 || N < 0 || K < 0 || r <= 0) return 0;
    return lora_grads_ws(M, N, K, r);
}

extern "C" pact_status pact_lora_grads_nvfp4(const pact_nvfp4 *Xq, const uint16_t *dY, int64_t ld_dy, int64_t N,
                                             const pact_lora *lora, const uint16_t *T_dy, float *dA, float *dB,
                                             void *ws, size_t ws_bytes, void *stream) {
    if (!Xq || !lora || !lora->A || !lora->B || !dA || !dB) return PACT_ERR_INVALID_ARG;
    const int64_t M = Xq->rows, K = Xq->cols;
    const int r = lora->r;
    if (M < 0 || K < 0 || N < 0 || r <= 0) return PACT_ERR_INVALID_ARG;
    if (K % 16 != 0 || N % 16 != 0 || r > 64) return PACT_ERR_UNSUPPORTED_SHAPE;
    if (M > INT32_MAX || K > INT32_MAX || N > INT32_MAX || M * K > INT32_MAX * 64LL) return PACT_ERR_UNSUPPORTED_SHAPE;
    PACT_TRY(check_nvfp4(Xq, M, K));
    PACT_TRY(check_bf16(dY, ld_dy, N));
    if (!aligned16(lora->A) || !aligned16(lora->B) || !aligned16(dA) || !aligned16(dB)) return PACT_ERR_MISALIGNED;
    if (T_dy && !aligned16(T_dy)) return PACT_ERR_MISALIGNED;
    hipStream_t st = as_stream(stream);
    if (M == 0 || K == 0 || N == 0) {  // empty sums: zero gradients
        if (K * r > 0)
            hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((K * r + 255) / 256)), dim3(256), 0, st, dA, K * r);
        if (N * r > 0)
            hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((N * r + 255) / 256)), dim3(256), 0, st, dB, N * r);
        return launch_status();
    }
    const size_t need = lora_grads_ws(M, N, K, r);
    if (!ws || ws_bytes < need) return PACT_ERR_WORKSPACE;
    if (!aligned16(ws)) return PACT_ERR_MISALIGNED;
    const int rpad = (int)round_up(r, 16);
    uint8_t *base = static_cast<uint8_t *>(ws);
    uint16_t *Th = reinterpret_cast<uint16_t *>(base);
    base += round_up(M * rpad * 2, 256);
    uint16_t *Tp = reinterpret_cast<uint16_t *>(base);
    base += round_up(M * rpad * 2, 256);
    uint16_t *Bt = reinterpret_cast<uint16_t *>(base);
    base += round_up((int64_t)r * N * 2, 256);
    float *partB = reinterpret_cast<float *>(base);
    float *partA = reinterpret_cast<float *>(base + grad_part_bytes(M, N, r, false));
    // T^ = bf16(s X^ A^T) straight from the NVFP4 rows (P(j, k) = A[j K + k]);
    // unless T' is given, its side workgroups write B^T for T'
    DownArgs dh{};
    dh.ldx = K;
    dh.M = (int)M;
    dh.Kl = (int)K;
    dh.Ps = lora->A;
    dh.p_sj = K;
    dh.p_sk = 1;
    dh.r = r;
    dh.rpad = rpad;
    dh.scale = lora->scale;
    dh.T = Th;
    dh.xc = Xq->codes;
    dh.xs = Xq->scales;
    dh.xd = Xq->row_scale;
    if (!T_dy) {
        dh.side_B = lora->B;
        dh.side_Bt = Bt;
        dh.side_N = (int)N;
        dh.side_r = r;
    }
    PACT_TRY(launch_lora_down_nvfp4(dh, st));
    // T' = bf16(s dY B): P(j, n) = B^T[j N + n]
    if (!T_dy)
        PACT_TRY(launch_lora_down(DownArgs{dY, ld_dy, (int)M, (int)N, Bt, N, 1, r, rpad, 0, lora->scale, Tp}, st));
    // dB[n][j] = sum_m dY[m][n] T^[m][j];  dA[j][k] = sum_m T'[m][j] X^[m][k];
    // dB's split reduction runs beside dA's contraction, dA's on its own
    pact_status stt = PACT_OK;
    GradArgs gb{};
    gb.V = dY;
    gb.ldv = ld_dy;
    gb.T = Th;
    gb.ldt = rpad;
    gb.M = (int)M;
    gb.C = (int)N;
    gb.r = r;
    gb.part = partB;
    const RedArgs redB = launch_grad(gb, dB, r, 1, st, &stt);
    PACT_TRY(stt);
    GradArgs ga{};
    ga.vc = Xq->codes;
    ga.vs = Xq->scales;
    ga.vd = Xq->row_scale;
    ga.T = T_dy ? T_dy : Tp;
    ga.ldt = rpad;
    ga.M = (int)M;
    ga.C = (int)K;
    ga.r = r;
    ga.part = partA;
    ga.side = redB;
    const RedArgs redA = launch_grad(ga, dA, 1, K, st, &stt);
    PACT_TRY(stt);
    hipLaunchKernelGGL(lora_grad_reduce_kernel, dim3((unsigned)redA.wgs), dim3(256), 0, st, redA);
    return launch_status();
}
