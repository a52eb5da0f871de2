// pact_lora_grad.hip -- LoRA weight gradients on the NVFP4 stash:
//   X^ = bf16(deq(Xq)), T^ = bf16(s . X^ A^T), T' = bf16(s . dY B),
//   dB = dY^T T^  [N][r],   dA = T'^T X^  [r][K],   FP32 sums, FP32 outputs.
// (simolm.com PACT blog, section "Method", second bullet and closing
// paragraph: the activations kept for backward are NVFP4 copies and the
// adapters stay BF16; kongchang.com PEFT explainer: the LoRA update B A x.)
//
// Both gradients are contractions over the tokens m of row-major [M][C]
// matrices with the rank-r intermediate [M][rpad]: out[c][j] = sum_m V[m][c]
// T[m][j].  They run on v_mfma_f32_32x32x16_bf16 with D = out (32 columns c x
// 32 ranks j per tile): lane (h, l) of the A operand holds V[m0 + 8h + e][c0 + l]
// for e < 8 and of the B operand T[m0 + 8h + e][32 t + l] (the same token
// assignment in both, so the dot products are unchanged); those are 2-byte
// loads, coalesced across the 32 lanes of a row.  The tokens of a column
// block are split across the 4 wavefronts of a workgroup (summed through LDS
// in wavefront order) and across msplit workgroups (FP32 partials summed in
// split order by a second kernel), so every run adds in the same order.
#include "pact_device.h"
#include "pact_host.h"

namespace pact {

// X^ = bf16(deq(Xq)): one thread per 16-element block.
__global__ __launch_bounds__(256) void dequant_bf16_kernel(const uint8_t *codes, const uint8_t *scales,
                                                           const float *d, int64_t rows, int cols, uint16_t *out) {
    const int nb = cols >> 4;
    const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (blk >= rows * nb) return;
    const int64_t row = blk / nb;
    const int b = (int)(blk - row * nb);
    const u32x2 c = *reinterpret_cast<const u32x2 *>(codes + row * (cols / 2) + 8 * b);
    float R[16];
    dequant16(c.x, c.y, scales[row * (cols / 16) + b], d[row], R);
    u32x4 lo, hi;
    lo.x = f32x2_to_bf16x2(R[0], R[1]);
    lo.y = f32x2_to_bf16x2(R[2], R[3]);
    lo.z = f32x2_to_bf16x2(R[4], R[5]);
    lo.w = f32x2_to_bf16x2(R[6], R[7]);
    hi.x = f32x2_to_bf16x2(R[8], R[9]);
    hi.y = f32x2_to_bf16x2(R[10], R[11]);
    hi.z = f32x2_to_bf16x2(R[12], R[13]);
    hi.w = f32x2_to_bf16x2(R[14], R[15]);
    u32x4 *dst = reinterpret_cast<u32x4 *>(out + row * cols + 16 * b);
    dst[0] = lo;
    dst[1] = hi;
}

struct GradArgs {
    const uint16_t *V;  // [M][C] (ldv)
    int64_t ldv;
    const uint16_t *T;  // [M][ldt], ranks j < r
    int64_t ldt;
    int M, C, r;
    int mchunk;   // tokens per workgroup (a multiple of 64)
    float *part;  // [msplit][C][32 JT]
};

constexpr int kGradWaves = 4;
constexpr int kGradU = 4;  // K16 steps whose loads are in flight together

// 8 BF16 values at p, p + ld, ..., p + 7 ld (rows at or past mlim read as 0).
__device__ __forceinline__ bf16x8_t gather8(const uint16_t *p, int64_t ld, int m, int mlim, bool ok) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t lo = (ok && m + 2 * q < mlim) ? p[(int64_t)(2 * q) * ld] : 0u;
        const uint32_t hi = (ok && m + 2 * q + 1 < mlim) ? p[(int64_t)(2 * q + 1) * ld] : 0u;
        w[q] = lo | (hi << 16);
    }
    return __builtin_bit_cast(bf16x8_t, u32x4{w[0], w[1], w[2], w[3]});
}

template <int JT>
__global__ __launch_bounds__(256) void lora_grad_kernel(GradArgs g) {
    __shared__ float red[kGradWaves][JT][16][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int h = lane >> 5, l = lane & 31;
    const int c0 = blockIdx.x * 32;
    const int c = c0 + l;
    const bool cok = c < g.C;
    const int wchunk = g.mchunk / kGradWaves;  // a multiple of 16
    const int mb = blockIdx.y * g.mchunk + w * wchunk;
    const int me = min(g.M, mb + wchunk);
    float16_t acc[JT];
#pragma unroll
    for (int t = 0; t < JT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
    for (int m0 = mb; m0 < me; m0 += 16 * kGradU) {
        bf16x8_t va[kGradU], vb[kGradU][JT];
#pragma unroll
        for (int u = 0; u < kGradU; ++u) {
            const int m = m0 + 16 * u + 8 * h;
            va[u] = gather8(g.V + (int64_t)m * g.ldv + c, g.ldv, m, me, cok);
#pragma unroll
            for (int t = 0; t < JT; ++t) {
                const int j = 32 * t + l;
                vb[u][t] = gather8(g.T + (int64_t)m * g.ldt + j, g.ldt, m, me, j < g.r);
            }
        }
#pragma unroll
        for (int u = 0; u < kGradU; ++u)
#pragma unroll
            for (int t = 0; t < JT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[u], vb[u][t], acc[t], 0, 0, 0);
    }
    // accumulator element e of lane (h, l): column c0 + 8 (e / 4) + 4 h + e % 4, rank 32 t + l
#pragma unroll
    for (int t = 0; t < JT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) red[w][t][e][lane] = acc[t][e];
    __syncthreads();
    float *dst = g.part + (int64_t)blockIdx.y * g.C * (32 * JT);
    for (int i = threadIdx.x; i < JT * 16 * 64; i += 256) {
        const int t = i / (16 * 64), e = (i / 64) % 16, ln = i % 64;
        float sum = red[0][t][e][ln];
#pragma unroll
        for (int q = 1; q < kGradWaves; ++q) sum += red[q][t][e][ln];
        const int cc = c0 + 8 * (e >> 2) + 4 * (ln >> 5) + (e & 3);
        const int j = 32 * t + (ln & 31);
        if (cc < g.C) dst[(int64_t)cc * (32 * JT) + j] = sum;
    }
}

// out[c * osc + j * osj] = sum over splits s (in order) of part[s][c][j], j < r.
__global__ __launch_bounds__(256) void lora_grad_reduce_kernel(const float *part, int msplit, int C, int r, int jw,
                                                               float *out, int64_t osc, int64_t osj) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)C * r) return;
    const int cc = (int)(i / r), j = (int)(i % r);
    float sum = 0.0f;
    for (int s = 0; s < msplit; ++s) sum += part[((int64_t)s * C + cc) * jw + j];
    out[cc * osc + j * osj] = sum;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

struct GradPlan {
    int msplit, mchunk;
};

static GradPlan grad_plan(int64_t M, int64_t C) {
    const int64_t cblocks = (C + 31) / 32;
    int64_t ms = (1024 + cblocks - 1) / cblocks;  // about 1024 workgroups
    const int64_t max_ms = (M + 255) / 256;          // at least 64 tokens per wavefront
    if (ms > max_ms) ms = max_ms;
    if (ms < 1) ms = 1;
    int64_t mchunk = (M + ms - 1) / ms;
    mchunk = (mchunk + 63) / 64 * 64;
    ms = (M + mchunk - 1) / mchunk;
    return {(int)(ms > 0 ? ms : 1), (int)mchunk};
}

static size_t grad_part_bytes(int64_t M, int64_t C, int r) {
    const GradPlan p = grad_plan(M, C);
    const int jt = (r + 31) / 32;
    return (size_t)round_up((int64_t)p.msplit * C * 32 * jt * 4, 256);
}

static size_t lora_grads_ws(int64_t M, int64_t N, int64_t K, int r) {
    const int64_t rpad = round_up(r, 16);
    const size_t xh = (size_t)round_up(M * K * 2, 256);
    const size_t t = (size_t)round_up(M * rpad * 2, 256);
    const size_t pn = grad_part_bytes(M, N, r), pk = grad_part_bytes(M, K, r);
    return xh + 2 * t + (pn > pk ? pn : pk);
}

static pact_status launch_grad(const uint16_t *V, int64_t ldv, const uint16_t *T, int64_t ldt, int M, int C, int r,
                               float *part, float *out, int64_t osc, int64_t osj, hipStream_t st) {
    const GradPlan p = grad_plan(M, C);
    const int jt = (r + 31) / 32;
    GradArgs g = {V, ldv, T, ldt, M, C, r, p.mchunk, part};
    const dim3 grid((unsigned)((C + 31) / 32), (unsigned)p.msplit);
    if (jt == 1)
        hipLaunchKernelGGL(lora_grad_kernel<1>, grid, dim3(256), 0, st, g);
    else
        hipLaunchKernelGGL(lora_grad_kernel<2>, grid, dim3(256), 0, st, g);
    PACT_TRY(launch_status());
    const int64_t n = (int64_t)C * r;
    hipLaunchKernelGGL(lora_grad_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, p.msplit,
                       C, r, 32 * jt, out, osc, osj);
    return launch_status();
}

}  // namespace pact

using namespace pact;

extern "C" size_t pact_lora_grads_workspace(int64_t M, int64_t N, int64_t K, int32_t r) {
    if (M < 0 || N < 0 || K < 0 || r <= 0) return 0;
    return lora_grads_ws(M, N, K, r);
}

extern "C" pact_status pact_lora_grads_nvfp4(const pact_nvfp4 *Xq, const uint16_t *dY, int64_t ld_dy, int64_t N,
                                             const pact_lora *lora, float *dA, float *dB, void *ws,
                                             size_t ws_bytes, void *stream) {
    if (!Xq || !lora || !lora->A || !lora->B || !dA || !dB) return PACT_ERR_INVALID_ARG;
    const int64_t M = Xq->rows, K = Xq->cols;
    const int r = lora->r;
    if (M < 0 || K < 0 || N < 0 || r <= 0) return PACT_ERR_INVALID_ARG;
    if (K % 16 != 0 || N % 16 != 0 || r > 64) return PACT_ERR_UNSUPPORTED_SHAPE;
    if (M > INT32_MAX || K > INT32_MAX || N > INT32_MAX || M * K > INT32_MAX * 64LL) return PACT_ERR_UNSUPPORTED_SHAPE;
    PACT_TRY(check_nvfp4(Xq, M, K));
    PACT_TRY(check_bf16(dY, ld_dy, N));
    if (!aligned16(lora->A) || !aligned16(lora->B) || !aligned16(dA) || !aligned16(dB)) return PACT_ERR_MISALIGNED;
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
    uint16_t *Xh = reinterpret_cast<uint16_t *>(base);
    base += round_up(M * K * 2, 256);
    uint16_t *Th = reinterpret_cast<uint16_t *>(base);
    base += round_up(M * rpad * 2, 256);
    uint16_t *Tp = reinterpret_cast<uint16_t *>(base);
    base += round_up(M * rpad * 2, 256);
    float *part = reinterpret_cast<float *>(base);
    // X^ = bf16(deq(Xq))
    const int64_t blocks = M * (K / 16);
    hipLaunchKernelGGL(dequant_bf16_kernel, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, st, Xq->codes,
                       Xq->scales, Xq->row_scale, M, (int)K, Xh);
    PACT_TRY(launch_status());
    // T^ = bf16(s X^ A^T): P(j, k) = A[j K + k];  T' = bf16(s dY B): P(j, n) = B[n r + j]
    PACT_TRY(launch_lora_down(DownArgs{Xh, K, (int)M, (int)K, lora->A, K, 1, r, rpad, 0, lora->scale, Th}, st));
    PACT_TRY(launch_lora_down(DownArgs{dY, ld_dy, (int)M, (int)N, lora->B, 1, r, r, rpad, 0, lora->scale, Tp}, st));
    // dB[n][j] = sum_m dY[m][n] T^[m][j];  dA[j][k] = sum_m T'[m][j] X^[m][k]
    PACT_TRY(launch_grad(dY, ld_dy, Th, rpad, (int)M, (int)N, r, part, dB, r, 1, st));
    return launch_grad(Xh, K, Tp, rpad, (int)M, (int)K, r, part, dA, 1, K, st);
}
