// pact_layout.hip -- cached forward / backward NVFP4 weight layouts
// (simolm.com PACT blog, section "Method", fourth bullet: the forward and the
// backward weight layouts are rebuilt, transposed and re-quantized once and
// then reused).
//
// W_fwd = Q over the rows of W [N][K] (blocks of 16 along K).
// R[n][k] = fl32(b_fwd[n][k] * d_fwd[n]) (b = exact E2M1 x E4M3 value).
// W_bwd = Q over the rows of R^T [K][N] (blocks of 16 along N).
//
// Three launches: (1) the row quantizer for W_fwd (or a copy of a given
// forward layout), (2) per-column partial maxima of |R| over slices of N into
// the workspace, (3) a tiled transpose: each workgroup decodes a 64(n) x 64(k)
// tile of R into LDS, reduces the column maxima to the row scales of R^T, and
// encodes 4 blocks of 16 n-values for each of its 64 k-rows.
#include "pact_device.h"
#include "pact_host.h"

namespace pact {

pact_status quantize_rows_launch(const uint16_t *x, int64_t ldx, int64_t rows, int64_t cols,
                                 const pact_nvfp4 *out, hipStream_t st);

constexpr int kColSplit = 32;  // slices of N for the column maxima

__device__ __forceinline__ float e2m1_value(uint32_t code) {
    // magnitudes of the 8 E2M1 codes, sign from bit 3
    const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    const float m = mag[code & 7u];
    return (code & 8u) ? -m : m;
}

// R value of element k of forward row n (codes/scales row pointers given).
__device__ __forceinline__ float r_value(const uint8_t *crow, const uint8_t *srow, float d, int k) {
    const uint32_t byte = crow[k >> 1];
    const uint32_t code = (k & 1) ? (byte >> 4) : (byte & 15u);
    const float b = e2m1_value(code) * e4m3_to_f32(srow[k >> 4]);  // exact
    return b * d;
}

__global__ __launch_bounds__(256) void colmax_kernel(const uint8_t *codes, const uint8_t *scales,
                                                     const float *d, int N, int K, float *part) {
    const int kp = blockIdx.x * 256 + threadIdx.x;  // pair of columns 2kp, 2kp+1
    const int slice = blockIdx.y;
    if (2 * kp >= K) return;
    const int chunk = (N + kColSplit - 1) / kColSplit;
    const int n0 = slice * chunk;
    const int n1 = min(N, n0 + chunk);
    float m0 = 0.0f, m1 = 0.0f;
    for (int n = n0; n < n1; ++n) {
        const uint8_t *crow = codes + (int64_t)n * (K / 2);
        const uint8_t *srow = scales + (int64_t)n * (K / 16);
        const float dn = d[n];
        m0 = fmaxf(m0, fabsf(r_value(crow, srow, dn, 2 * kp)));
        m1 = fmaxf(m1, fabsf(r_value(crow, srow, dn, 2 * kp + 1)));
    }
    part[(int64_t)slice * K + 2 * kp] = m0;
    part[(int64_t)slice * K + 2 * kp + 1] = m1;
}

__global__ __launch_bounds__(256) void transpose_quant_kernel(const uint8_t *codes,
                                                              const uint8_t *scales,
                                                              const float *d, int N, int K,
                                                              const float *part, uint8_t *bcodes,
                                                              uint8_t *bscales, float *bd) {
    __shared__ float tile[64][65];
    __shared__ float rowd[64];
    __shared__ float rowD[64];
    const int n0 = blockIdx.x * 64;
    const int k0 = blockIdx.y * 64;
    const int t = threadIdx.x;
    if (t < 64) {
        const int k = k0 + t;
        float amax = 0.0f;
        if (k < K)
            for (int s = 0; s < kColSplit; ++s) amax = fmaxf(amax, part[(int64_t)s * K + k]);
        const RowQ rq = row_params(amax);
        rowd[t] = rq.d;
        rowD[t] = rq.D;
        if (k < K && blockIdx.x == 0) bd[k] = rq.d;
    }
    {
        const int nl = t >> 2;           // 0..63
        const int kq = (t & 3) * 16;     // 0, 16, 32, 48
        const int n = n0 + nl;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int k = k0 + kq + i;
            float v = 0.0f;
            if (n < N && k < K)
                v = r_value(codes + (int64_t)n * (K / 2), scales + (int64_t)n * (K / 16), d[n], k);
            tile[nl][kq + i] = v;
        }
    }
    __syncthreads();
    const int kl = t & 63;
    const int j = t >> 6;  // block of 16 n within the tile
    const int k = k0 + kl;
    const int nb0 = n0 + 16 * j;
    if (k >= K || nb0 >= N) return;
    float v[16];
    float bmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        v[i] = tile[16 * j + i][kl];
        bmax = fmaxf(bmax, fabsf(v[i]));
    }
    RowQ rq;
    rq.d = rowd[kl];
    rq.D = rowD[kl];
    rq.rD = 0.0;  // unused by the binary32 encoder
    uint32_t lo, hi, sb;
    encode_block16<false>(v, bmax, rq, lo, hi, sb);
    u32x2 c;
    c.x = lo;
    c.y = hi;
    *reinterpret_cast<u32x2 *>(bcodes + (int64_t)k * (N / 2) + nb0 / 2) = c;
    bscales[(int64_t)k * (N / 16) + nb0 / 16] = (uint8_t)sb;
}

static size_t layout_ws_bytes(int64_t K) { return (size_t)kColSplit * (size_t)K * sizeof(float); }

}  // namespace pact

using namespace pact;

extern "C" size_t pact_build_weight_layouts_workspace(int64_t N, int64_t K) {
    (void)N;
    if (K <= 0) return 0;
    return layout_ws_bytes(K);
}

extern "C" pact_status pact_build_weight_layouts(const uint16_t *W, const pact_nvfp4 *W_fwd_in,
                                                 int64_t N, int64_t K, const pact_nvfp4 *W_fwd,
                                                 const pact_nvfp4 *W_bwd, void *ws,
                                                 size_t ws_bytes, void *stream) {
    if (N < 0 || K < 0) return PACT_ERR_INVALID_ARG;
    if (N % 16 != 0 || K % 16 != 0 || N > PACT_MAX_ROW || K > PACT_MAX_ROW)
        return PACT_ERR_UNSUPPORTED_SHAPE;
    if ((W == nullptr) == (W_fwd_in == nullptr)) return PACT_ERR_INVALID_ARG;
    if (W) PACT_TRY(check_bf16(W, K, K));
    if (W_fwd_in) PACT_TRY(check_nvfp4(W_fwd_in, N, K));
    PACT_TRY(check_nvfp4(W_fwd, N, K));
    PACT_TRY(check_nvfp4(W_bwd, K, N));
    if (N == 0 || K == 0) return PACT_OK;
    if (!ws || ws_bytes < layout_ws_bytes(K)) return PACT_ERR_WORKSPACE;
    if (!aligned16(ws)) return PACT_ERR_MISALIGNED;
    hipStream_t st = as_stream(stream);
    if (W) {
        PACT_TRY(quantize_rows_launch(W, K, N, K, W_fwd, st));
    } else {
        if (W_fwd_in->codes != W_fwd->codes &&
            hipMemcpyAsync(W_fwd->codes, W_fwd_in->codes, (size_t)(N * K / 2),
                           hipMemcpyDeviceToDevice, st) != hipSuccess)
            return PACT_ERR_HIP;
        if (W_fwd_in->scales != W_fwd->scales &&
            hipMemcpyAsync(W_fwd->scales, W_fwd_in->scales, (size_t)(N * K / 16),
                           hipMemcpyDeviceToDevice, st) != hipSuccess)
            return PACT_ERR_HIP;
        if (W_fwd_in->row_scale != W_fwd->row_scale &&
            hipMemcpyAsync(W_fwd->row_scale, W_fwd_in->row_scale, (size_t)N * sizeof(float),
                           hipMemcpyDeviceToDevice, st) != hipSuccess)
            return PACT_ERR_HIP;
    }
    float *part = static_cast<float *>(ws);
    const dim3 g1((unsigned)((K / 2 + 255) / 256), kColSplit);
    hipLaunchKernelGGL(colmax_kernel, g1, dim3(256), 0, st, W_fwd->codes, W_fwd->scales,
                       W_fwd->row_scale, (int)N, (int)K, part);
    PACT_TRY(launch_status());
    const dim3 g2((unsigned)((N + 63) / 64), (unsigned)((K + 63) / 64));
    hipLaunchKernelGGL(transpose_quant_kernel, g2, dim3(256), 0, st, W_fwd->codes, W_fwd->scales,
                       W_fwd->row_scale, (int)N, (int)K, part, W_bwd->codes, W_bwd->scales,
                       W_bwd->row_scale);
    return launch_status();
}
