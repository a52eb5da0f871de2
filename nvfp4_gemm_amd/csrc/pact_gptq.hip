// pact_gptq.hip -- NVFP4-adapted GPTQ calibration of a frozen weight.
//
// simolm.com PACT blog, section "Method", third bullet, and the arXiv
// abstract of "PACT: NVFP4 Data-Flow LoRA Fine-Tuning on Consumer GPUs": the
// frozen weights are calibrated offline by GPTQ adapted to the NVFP4 block
// scales, with statistics taken from reconstructed NVFP4 activations.  GPTQ
// itself is Frantar et al.: the columns of W [N][K] are quantized in order,
// and each column's rounding error is spread over the columns not yet
// quantized through the upper Cholesky factor U of the inverse Hessian of the
// layer's output error (H^-1 = U^T U).
//
// Steps, all in binary64 on the GPU:
//   1. H = scale X^T X (+ H) over the dequantized NVFP4 calibration rows X
//      (pact_gptq_hessian_nvfp4);
//   2. dead inputs (zero diagonal): diagonal set to 1, their weights to 0;
//      1 % (percdamp) of the mean diagonal added to the diagonal;
//   3. H = R R^T with R upper triangular, blocked from the bottom-right
//      corner (64 x 64 diagonal blocks factored in one workgroup, panels and
//      trailing updates as binary64 products), then U = R^-1 by blocked back
//      substitution: U is upper triangular and H^-1 = R^-T R^-1 = U^T U, so
//      U is the upper Cholesky factor of H^-1 (positive diagonal, unique);
//   4. the column sweep in lazy batches of bs columns: inside a batch, column
//      by column in one wavefront per 64 rows (rows are independent); at the
//      batch's end, the remaining columns take W -= Err U[batch, rest].
// NVFP4 rule: the row scale d is the plain quantizer's (max of the original
// row / 2688, binary32); at the first column of each 16-column block the
// block's E4M3 scale comes from the plain quantizer's rule applied to the
// block's current (error-updated) weights rounded to binary32, and each
// column's code is the plain quantizer's code of its binary32-rounded current
// weight under that scale.
#include <algorithm>

#include "pact_device.h"
#include "pact_host.h"

namespace pact {

// ---- binary64 product C = alpha A B + beta C ------------------------------
// A(i, k) = A[i sai + k sak], B(k, j) = B[k sbk + j sbj], C(i, j) = C[i ldc +
// j] for i < M, j < N, k < K; 64 x 64 output tiles, 256 threads of 4 x 4.
struct Dgemm {
    const double *A;
    int64_t sai, sak;
    const double *B;
    int64_t sbk, sbj;
    double *C;
    int64_t ldc;
    int M, N, K;
    double alpha, beta;
};

constexpr int kDT = 64, kDK = 16;

__global__ __launch_bounds__(256) void dgemm_kernel(Dgemm g) {
    __shared__ double As[kDK][kDT + 1];  // [k][i]
    __shared__ double Bs[kDK][kDT + 1];  // [k][j]
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int i0 = blockIdx.y * kDT, j0 = blockIdx.x * kDT;
    double acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = 0.0;
    // element e of a tile load: contiguous along the operand's unit stride
    const bool a_rows = g.sak == 1, b_cols = g.sbj == 1;
    for (int k0 = 0; k0 < g.K; k0 += kDK) {
        for (int e = threadIdx.x; e < kDT * kDK; e += 256) {
            const int ii = a_rows ? e / kDK : e % kDT, kk = a_rows ? e % kDK : e / kDT;
            const int i = i0 + ii, k = k0 + kk;
            As[kk][ii] = (i < g.M && k < g.K) ? g.A[(int64_t)i * g.sai + (int64_t)k * g.sak] : 0.0;
            const int jj = b_cols ? e % kDT : e / kDK, kb = b_cols ? e / kDT : e % kDK;
            const int j = j0 + jj, k2 = k0 + kb;
            Bs[kb][jj] = (j < g.N && k2 < g.K) ? g.B[(int64_t)k2 * g.sbk + (int64_t)j * g.sbj] : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kDK; ++kk) {
            double a[4], b[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] = As[kk][ty + 16 * r];
#pragma unroll
            for (int c = 0; c < 4; ++c) b[c] = Bs[kk][tx + 16 * c];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[r][c] = __fma_rn(a[r], b[c], acc[r][c]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int i = i0 + ty + 16 * r, j = j0 + tx + 16 * c;
            if (i < g.M && j < g.N) {
                double *dst = g.C + (int64_t)i * g.ldc + j;
                *dst = g.beta == 0.0 ? g.alpha * acc[r][c] : g.alpha * acc[r][c] + g.beta * *dst;
            }
        }
}

static pact_status dgemm(const Dgemm &g, hipStream_t st) {
    if (g.M <= 0 || g.N <= 0) return PACT_OK;
    const dim3 grid((unsigned)((g.N + kDT - 1) / kDT), (unsigned)((g.M + kDT - 1) / kDT));
    hipLaunchKernelGGL(dgemm_kernel, grid, dim3(256), 0, st, g);
    return launch_status();
}

// ---- Hessian over the dequantized NVFP4 rows --------------------------------
// X(t, i) = fl32((code x block scale) x d_t) widened to binary64; H(i, j) =
// beta H(i, j) + scale sum_t X(t, i) X(t, j), the products exact in binary64.
struct HessArgs {
    const uint8_t *codes, *scales;
    const float *d;
    int64_t n, K;
    double scale, beta;
    double *H;
};

// E2M1 magnitude of a 3-bit code: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_to_f32(uint32_t mag) {
    const uint32_t e = mag >> 1, m = mag & 1u;
    return e == 0 ? 0.5f * (float)m : (1.0f + 0.5f * (float)m) * (float)(1u << (e - 1));
}

__device__ __forceinline__ double nvfp4_value(const HessArgs &a, int64_t t, int64_t i) {
    const uint32_t byte = a.codes[t * (a.K / 2) + i / 2];
    const uint32_t code = (byte >> (4 * (i & 1))) & 15u;
    const float mag = e2m1_to_f32(code & 7u);
    const float b = mag * e4m3_to_f32(a.scales[t * (a.K / 16) + i / 16]);  // exact
    const float v = b * a.d[t];
    return (double)((code & 8u) ? -v : v);
}

__global__ __launch_bounds__(256) void hessian_kernel(HessArgs a) {
    __shared__ double Xi[kDK][kDT + 1];
    __shared__ double Xj[kDK][kDT + 1];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int64_t i0 = (int64_t)blockIdx.y * kDT, j0 = (int64_t)blockIdx.x * kDT;
    double acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = 0.0;
    for (int64_t t0 = 0; t0 < a.n; t0 += kDK) {
        for (int e = threadIdx.x; e < kDT * kDK; e += 256) {
            const int kk = e / kDT, ii = e % kDT;
            const int64_t t = t0 + kk;
            Xi[kk][ii] = (t < a.n && i0 + ii < a.K) ? nvfp4_value(a, t, i0 + ii) : 0.0;
            Xj[kk][ii] = (t < a.n && j0 + ii < a.K) ? nvfp4_value(a, t, j0 + ii) : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kDK; ++kk) {
            double x[4], y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = Xi[kk][ty + 16 * r];
#pragma unroll
            for (int c = 0; c < 4; ++c) y[c] = Xj[kk][tx + 16 * c];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[r][c] = __fma_rn(x[r], y[c], acc[r][c]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int64_t i = i0 + ty + 16 * r, j = j0 + tx + 16 * c;
            if (i < a.K && j < a.K) {
                double *dst = a.H + i * a.K + j;
                *dst = a.beta == 0.0 ? a.scale * acc[r][c] : a.scale * acc[r][c] + a.beta * *dst;
            }
        }
}

// ---- preparation: dead inputs and dampening (one workgroup) ----------------
__global__ __launch_bounds__(1024) void gptq_prep_kernel(double *H, int64_t K, double percdamp, uint8_t *dead) {
    __shared__ double part[1024];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < K; i += blockDim.x) {
        double h = H[i * K + i];
        const bool z = h == 0.0;
        dead[i] = z ? 1 : 0;
        if (z) {
            h = 1.0;
            H[i * K + i] = 1.0;
        }
        s += h;
    }
    part[threadIdx.x] = s;
    __syncthreads();
    for (int w = blockDim.x / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    const double damp = percdamp * (part[0] / (double)K);
    for (int64_t i = threadIdx.x; i < K; i += blockDim.x) H[i * K + i] += damp;
}

// ---- a 64 x 64 diagonal block: reverse Cholesky and its inverse -------------
// A = H[c0.., c0..] (already updated by the blocks below-right) = Rd Rd^T with
// Rd upper triangular; Rd goes to R, Rd^-1 to U (both at [c0][c0]); lower
// parts of both blocks are written as zeros.  A pivot that is not positive
// (H not numerically positive definite) is replaced by 1: the results are
// then unspecified, but finite.
constexpr int kCB = 64;

__global__ __launch_bounds__(256) void chol_diag_kernel(const double *H, int64_t K, int64_t c0, double *R,
                                                        double *U) {
    __shared__ double A[kCB][kCB + 1];
    __shared__ double V[kCB][kCB + 1];
    for (int e = threadIdx.x; e < kCB * kCB; e += 256) {
        const int r = e / kCB, c = e % kCB;
        A[r][c] = H[(c0 + r) * K + c0 + c];
    }
    __syncthreads();
    for (int c = kCB - 1; c >= 0; --c) {
        double piv = A[c][c];
        if (!(piv > 0.0)) piv = 1.0;
        piv = sqrt(piv);
        __syncthreads();  // everyone has read A[c][c]
        if ((int)threadIdx.x < c) A[threadIdx.x][c] = A[threadIdx.x][c] / piv;
        if (threadIdx.x == 0) A[c][c] = piv;
        __syncthreads();
        for (int e = threadIdx.x; e < c * c; e += 256) {
            const int r = e / c, s = e % c;
            A[r][s] -= A[r][c] * A[s][c];
        }
        __syncthreads();
    }
    // Rd = upper triangle of A; V = Rd^-1 (column j by back substitution)
    if ((int)threadIdx.x < kCB) {
        const int j = threadIdx.x;
        for (int i = 0; i < kCB; ++i) V[i][j] = 0.0;
        V[j][j] = 1.0 / A[j][j];
        for (int i = j - 1; i >= 0; --i) {
            double s = 0.0;
            for (int k = i + 1; k <= j; ++k) s += A[i][k] * V[k][j];
            V[i][j] = -s / A[i][i];
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kCB * kCB; e += 256) {
        const int r = e / kCB, c = e % kCB;
        R[(c0 + r) * K + c0 + c] = c >= r ? A[r][c] : 0.0;
        U[(c0 + r) * K + c0 + c] = c >= r ? V[r][c] : 0.0;
    }
}

__global__ __launch_bounds__(256) void dfill_kernel(double *p, int64_t n, double v) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

// ---- weights into binary64, row scales ------------------------------------
// One workgroup per row: Wd[n][k] = w (0 for dead inputs); d[n] = fl32(max|w|
// / 2688) over the original row, as the plain quantizer.
__global__ __launch_bounds__(256) void gptq_init_kernel(const uint16_t *W, int64_t ld_w, int64_t K,
                                                        const uint8_t *dead, double *Wd, float *d) {
    __shared__ float red[256];
    const int64_t n = blockIdx.x;
    float amax = 0.0f;
    for (int64_t k = threadIdx.x; k < K; k += 256) {
        const float v = __uint_as_float((uint32_t)W[n * ld_w + k] << 16);
        amax = fmaxf(amax, fabsf(v));
        Wd[n * K + k] = dead[k] ? 0.0 : (double)v;
    }
    red[threadIdx.x] = amax;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
        __syncthreads();
    }
    if (threadIdx.x == 0) d[n] = red[0] / 2688.0f;
}

// ---- the column sweep inside one lazy batch [i1, i2) ----------------------
// One wavefront per 64 rows, lane = row; the batch's weights sit in LDS
// column-major ([column][lane]); U rows are read from memory (the same
// address in every lane).  Writes the codes of the batch's columns, the block
// scales of its 16-column blocks, and Err[n][i - i1] = (w - q) / U[i][i].
constexpr int kSweepMaxBatch = 128;

struct SweepArgs {
    const double *U;
    const double *Wd;
    const float *d;
    int64_t N, K;
    int i1, i2;
    double *Err;  // [N][bs]
    int bs;
    uint8_t *codes, *scales;
};

__global__ __launch_bounds__(64) void gptq_sweep_kernel(SweepArgs a) {
    __shared__ double w[kSweepMaxBatch][64];
    const int lane = threadIdx.x;
    const int64_t n = (int64_t)blockIdx.x * 64 + lane;
    const bool live = n < a.N;
    const int nb = a.i2 - a.i1;
    for (int c = 0; c < nb; ++c) w[c][lane] = live ? a.Wd[n * a.K + a.i1 + c] : 0.0;
    const float dn = live ? a.d[n] : 0.0f;
    const float D = 6.0f * dn;
    uint32_t sb = 0u;
    float S = 0.0f;
    uint32_t lo = 0u;
    for (int c = 0; c < nb; ++c) {
        const int64_t i = a.i1 + c;
        if ((i & 15) == 0) {
            float amax = 0.0f;
            for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf((float)w[c + j][lane]));
            sb = dn == 0.0f ? 0u : e4m3_encode_sat(amax / D);
            S = e4m3_to_f32(sb) * dn;
            if (live) a.scales[n * (a.K / 16) + i / 16] = (uint8_t)sb;
        }
        const double wi = w[c][lane];
        const float wf = (float)wi;
        const uint32_t code = S == 0.0f ? ((__float_as_uint(wf) >> 31) << 3) : e2m1_encode2(quot_f32(wf, S), 0.0f) & 15u;
        if (i & 1) {
            if (live) a.codes[n * (a.K / 2) + i / 2] = (uint8_t)(lo | (code << 4));
        } else {
            lo = code;
        }
        const float qv = e2m1_to_f32(code & 7u) * e4m3_to_f32(sb);  // exact
        const double q = (double)((code & 8u) ? -qv : qv) * (double)dn;
        const double *Ui = a.U + i * a.K + a.i1;
        const double e = (wi - q) / Ui[c];
        if (live) a.Err[n * a.bs + c] = e;
        for (int j = c + 1; j < nb; ++j) w[j][lane] = w[j][lane] - e * Ui[j];
    }
}

}  // namespace pact

using namespace pact;

extern "C" pact_status pact_gptq_hessian_nvfp4(const pact_nvfp4 *Xq, double scale, int32_t accumulate, double *H,
                                               void *stream) {
    if (!Xq || !H) return PACT_ERR_INVALID_ARG;
    const int64_t n = Xq->rows, K = Xq->cols;
    if (n < 0 || K < 0) return PACT_ERR_INVALID_ARG;
    if (K % 16 != 0) return PACT_ERR_UNSUPPORTED_SHAPE;
    PACT_TRY(check_nvfp4(Xq, n, K));
    if (!aligned16(H)) return PACT_ERR_MISALIGNED;
    if (K == 0) return PACT_OK;
    HessArgs a = {Xq->codes, Xq->scales, Xq->row_scale, n, K, scale, accumulate ? 1.0 : 0.0, H};
    const unsigned t = (unsigned)((K + kDT - 1) / kDT);
    hipLaunchKernelGGL(hessian_kernel, dim3(t, t), dim3(256), 0, as_stream(stream), a);
    return launch_status();
}

static size_t gptq_ws_parts(int64_t N, int64_t K, size_t off[5]) {
    size_t o = 0;
    auto take = [&](int i, size_t bytes) {
        off[i] = o;
        o += (size_t)round_up((int64_t)bytes, 256);
    };
    take(0, (size_t)K * K * 8);                // R
    take(1, (size_t)K * K * 8);                // U
    take(2, (size_t)kCB * K * 8);              // block row of R U products
    take(3, (size_t)N * K * 8);                // weights in binary64
    take(4, (size_t)N * kSweepMaxBatch * 8 + (size_t)K);  // batch errors, dead-input flags
    return o;
}

extern "C" size_t pact_gptq_workspace(int64_t N, int64_t K) {
    if (N < 0 || K < 0) return 0;
    size_t off[5];
    return gptq_ws_parts(N, K, off);
}

extern "C" pact_status pact_gptq_nvfp4(const uint16_t *W, int64_t ld_w, int64_t N, int64_t K, double *H,
                                       double percdamp, int32_t blocksize, const pact_nvfp4 *W_fwd, void *ws,
                                       size_t ws_bytes, void *stream) {
    if (!H || !W_fwd) return PACT_ERR_INVALID_ARG;
    if (N < 0 || K < 0 || !(percdamp >= 0.0) || blocksize < 16 || blocksize > kSweepMaxBatch) return PACT_ERR_INVALID_ARG;
    if (K % kCB != 0 || blocksize % 16 != 0 || N > INT32_MAX || K > INT32_MAX) return PACT_ERR_UNSUPPORTED_SHAPE;
    PACT_TRY(check_nvfp4(W_fwd, N, K));
    if (N > 0) PACT_TRY(check_bf16(W, ld_w, K));
    if (!aligned16(H)) return PACT_ERR_MISALIGNED;
    size_t off[5];
    const size_t need = gptq_ws_parts(N, K, off);
    if (!ws || ws_bytes < need) return PACT_ERR_WORKSPACE;
    if (!aligned16(ws)) return PACT_ERR_MISALIGNED;
    if (N == 0 || K == 0) return PACT_OK;
    hipStream_t st = as_stream(stream);
    uint8_t *base = static_cast<uint8_t *>(ws);
    double *R = reinterpret_cast<double *>(base + off[0]);
    double *U = reinterpret_cast<double *>(base + off[1]);
    double *T = reinterpret_cast<double *>(base + off[2]);
    double *Wd = reinterpret_cast<double *>(base + off[3]);
    double *Err = reinterpret_cast<double *>(base + off[4]);
    uint8_t *dead = base + off[4] + (size_t)N * kSweepMaxBatch * 8;

    // 2. dead inputs, dampening; U starts at zero (its lower triangle stays so)
    hipLaunchKernelGGL(gptq_prep_kernel, dim3(1), dim3(1024), 0, st, H, K, percdamp, dead);
    PACT_TRY(launch_status());
    hipLaunchKernelGGL(dfill_kernel, dim3(1024), dim3(256), 0, st, U, K * K, 0.0);
    PACT_TRY(launch_status());
    // 3. H = R R^T, blocked from the bottom-right corner
    const int nb = (int)(K / kCB);
    for (int J = nb - 1; J >= 0; --J) {
        const int64_t c0 = (int64_t)J * kCB;
        hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(256), 0, st, H, K, c0, R, U);
        PACT_TRY(launch_status());
        if (c0 == 0) break;
        // panel R[0:c0, c0:c0+64] = H[0:c0, c0:c0+64] (Rd^-1)^T
        PACT_TRY(dgemm(Dgemm{H + c0, K, 1, U + c0 * K + c0, 1, K, R + c0, K, (int)c0, kCB, kCB, 1.0, 0.0}, st));
        // trailing update H[0:c0, 0:c0] -= P P^T
        PACT_TRY(dgemm(Dgemm{R + c0, K, 1, R + c0, 1, K, H, K, (int)c0, (int)c0, kCB, -1.0, 1.0}, st));
    }
    //    U = R^-1: block row I (bottom-up) from the rows below it:
    //    U[I, c1:] = -Ud_I (R[I, c1:] U[c1:, c1:]), c1 = (I + 1) 64
    for (int I = nb - 2; I >= 0; --I) {
        const int64_t r0 = (int64_t)I * kCB, c1 = r0 + kCB, L = K - c1;
        PACT_TRY(dgemm(Dgemm{R + r0 * K + c1, K, 1, U + c1 * K + c1, K, 1, T, L, kCB, (int)L, (int)L, 1.0, 0.0}, st));
        PACT_TRY(dgemm(Dgemm{U + r0 * K + r0, K, 1, T, L, 1, U + r0 * K + c1, K, kCB, (int)L, kCB, -1.0, 0.0}, st));
    }
    // 4. weights and row scales, then the sweep in lazy batches
    hipLaunchKernelGGL(gptq_init_kernel, dim3((unsigned)N), dim3(256), 0, st, W, ld_w, K, dead, Wd,
                       W_fwd->row_scale);
    PACT_TRY(launch_status());
    const unsigned rows_wg = (unsigned)((N + 63) / 64);
    for (int64_t i1 = 0; i1 < K; i1 += blocksize) {
        const int64_t i2 = std::min<int64_t>(i1 + blocksize, K);
        SweepArgs sa = {U, Wd, W_fwd->row_scale, N, K, (int)i1, (int)i2, Err, blocksize, W_fwd->codes,
                        W_fwd->scales};
        hipLaunchKernelGGL(gptq_sweep_kernel, dim3(rows_wg), dim3(64), 0, st, sa);
        PACT_TRY(launch_status());
        if (i2 < K) {
            // W[:, i2:] -= Err U[i1:i2, i2:]
            PACT_TRY(dgemm(Dgemm{Err, blocksize, 1, U + i1 * K + i2, K, 1, Wd + i2, K, (int)N, (int)(K - i2),
                                 (int)(i2 - i1), -1.0, 1.0},
                           st));
        }
    }
    return PACT_OK;
}
