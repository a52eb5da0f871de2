// pact_quant.hip -- row-wise NVFP4 producers (HBM-bound):
//   pact_quantize_nvfp4        Q(x)
//   pact_rmsnorm_quant_nvfp4   y = bf16(x rstd gamma), Q(y), rstd
//   pact_silu_mul_quant_nvfp4  h = bf16(sigma32(g) u), Q(h), Q(g), Q(u)
// (simolm.com PACT blog, section "Method": quantization fused into RMSNorm and
// SiLU-multiply; the quantized RMSNorm output and NVFP4 gate/up copies are
// what backward keeps; forward nonlinear ops read BF16.)
//
// Design: one row per 64*WPR threads; each thread owns whole 16-element blocks
// (blocks lane, lane + T, ...), loaded with two 16-byte loads and kept in
// registers, so the row is read from HBM exactly once.  The row amax (and, for
// RMSNorm, the sum of squares) is reduced across the wavefront with shuffles
// and across the row's wavefronts through LDS, in a fixed order so that every
// thread sees the same value.  Codes go out as 8-byte stores, scale bytes as
// one byte per block (contiguous across lanes).
#include "pact_device.h"
#include "pact_host.h"

namespace pact {

struct NV {
    uint8_t *codes;
    uint8_t *scales;
    float *d;
};

enum { MODE_QUANT = 0, MODE_RMS = 1, MODE_SILU = 2 };

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
// BF16 g, looked up in a table of all 65536 BF16 bit patterns (256 KB,
// generated at build time by gen_sigmoid_table.cpp, which states the method).
// The table is constant data of the code object; the library keeps no state.
__device__ const uint32_t kSigmoidBits[65536] = {
#include "pact_sigmoid_table.inc"
};

__device__ __forceinline__ float sigmoid32_bits(uint32_t gbits) { return __uint_as_float(kSigmoidBits[gbits]); }

// Workgroup barrier ordering LDS only.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int WPR>
__device__ __forceinline__ void row_max3(float &a, float &b, float &c, float (*red)[4], int wave,
                                         int lrow) {
    a = wave_max(a);
    b = wave_max(b);
    c = wave_max(c);
    if constexpr (WPR > 1) {
        if ((threadIdx.x & 63) == 0) {
            red[wave][0] = a;
            red[wave][1] = b;
            red[wave][2] = c;
        }
        lds_sync();
        const int w0 = lrow * WPR;
        a = red[w0][0];
        b = red[w0][1];
        c = red[w0][2];
#pragma unroll
        for (int w = 1; w < WPR; ++w) {
            a = fmaxf(a, red[w0 + w][0]);
            b = fmaxf(b, red[w0 + w][1]);
            c = fmaxf(c, red[w0 + w][2]);
        }
        lds_sync();
    }
}

__device__ __forceinline__ void unpack16(const uint32_t w[8], float v[16]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_lo(w[i]);
        v[2 * i + 1] = bf16_hi(w[i]);
    }
}

__device__ __forceinline__ float amax16(const float v[16]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
    return m;
}

__device__ __forceinline__ void load_block(const uint16_t *p, uint32_t w[8]) {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(p);
    const u32x4 b = *reinterpret_cast<const u32x4 *>(p + 8);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

__device__ __forceinline__ void store_block(uint16_t *p, const uint32_t w[8]) {
    u32x4 a, b;
    a.x = w[0]; a.y = w[1]; a.z = w[2]; a.w = w[3];
    b.x = w[4]; b.y = w[5]; b.z = w[6]; b.w = w[7];
    *reinterpret_cast<u32x4 *>(p) = a;
    *reinterpret_cast<u32x4 *>(p + 8) = b;
}

__device__ __forceinline__ void emit_block(const NV &q, int64_t row, int cols, int b, const float v[16],
                                           float bmax, RowQ rq) {
    uint32_t lo, hi, sb;
    encode_block16<true>(v, bmax, rq, lo, hi, sb);
    u32x2 c;
    c.x = lo;
    c.y = hi;
    *reinterpret_cast<u32x2 *>(q.codes + row * (cols / 2) + 8 * b) = c;
    q.scales[row * (cols / 16) + b] = (uint8_t)sb;
}

template <int WPR, int BPL, int MODE>
__global__ __launch_bounds__(256) void row_kernel(RowArgs a) {
    constexpr int T = 64 * WPR;
    constexpr int RPW = 256 / T;
    __shared__ float red[4][4];
    __shared__ double redd[4][2];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lrow = tid / T;
    const int lt = tid % T;
    const int64_t row = (int64_t)blockIdx.x * RPW + lrow;
    const bool active = row < a.rows;
    const int cols = a.cols;
    const int nb = cols >> 4;

    uint32_t xw[BPL][8];
    uint32_t uw[MODE == MODE_SILU ? BPL : 1][8];
    bool valid[BPL];
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
        const int b = lt + T * i;
        valid[i] = active && b < nb;
        if (valid[i]) {
            load_block(a.x + row * a.ldx + 16 * b, xw[i]);
            if constexpr (MODE == MODE_SILU) load_block(a.x2 + row * a.ldx2 + 16 * b, uw[i]);
        }
    }

    if constexpr (MODE == MODE_QUANT) {
        float bmax[BPL];
        float rmax = 0.0f;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            float v[16];
            unpack16(xw[i], v);
            bmax[i] = valid[i] ? amax16(v) : 0.0f;
            rmax = fmaxf(rmax, bmax[i]);
        }
        float dummy1 = 0.0f, dummy2 = 0.0f;
        row_max3<WPR>(rmax, dummy1, dummy2, red, wave, lrow);
        const RowQ rq = row_params(rmax);
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            if (!valid[i]) continue;
            float v[16];
            unpack16(xw[i], v);
            emit_block(a.q0, row, cols, lt + T * i, v, bmax[i], rq);
        }
        if (active && lt == 0) a.q0.d[row] = rq.d;
    } else if constexpr (MODE == MODE_RMS) {
        // sum of squares: squares are exact in binary64; accumulate error-free
        double s = 0.0, c = 0.0;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            if (!valid[i]) continue;
            float v[16];
            unpack16(xw[i], v);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const double xv = (double)v[j];
                dd_add(s, c, xv * xv);
            }
        }
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
            bmax[i] = 0.0f;
            if (!valid[i]) continue;
            const int b = lt + T * i;
            uint32_t gw[8];
            load_block(a.gamma + 16 * b, gw);
            float v[16], gv[16];
            unpack16(xw[i], v);
            unpack16(gw, gv);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float t0 = v[2 * j] * r;
                const float t1 = v[2 * j + 1] * r;
                xw[i][j] = f32x2_to_bf16x2(t0 * gv[2 * j], t1 * gv[2 * j + 1]);  // y replaces x
            }
            if (a.y) store_block(a.y + row * a.ldy + 16 * b, xw[i]);
            unpack16(xw[i], v);
            bmax[i] = amax16(v);
            rmax = fmaxf(rmax, bmax[i]);
        }
        float dummy1 = 0.0f, dummy2 = 0.0f;
        row_max3<WPR>(rmax, dummy1, dummy2, red, wave, lrow);
        const RowQ rq = row_params(rmax);
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            if (!valid[i]) continue;
            float v[16];
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
            hmax[i] = gmax[i] = umax[i] = 0.0f;
            if (!valid[i]) continue;
            float gv[16], uv[16];
            unpack16(xw[i], gv);
            unpack16(uw[i], uv);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float p0 = sigmoid32_bits(xw[i][j] & 0xFFFFu) * uv[2 * j];
                const float p1 = sigmoid32_bits(xw[i][j] >> 16) * uv[2 * j + 1];
                hw[i][j] = f32x2_to_bf16x2(p0, p1);
            }
            const int b = lt + T * i;
            if (a.y) store_block(a.y + row * a.ldy + 16 * b, hw[i]);
            float hv[16];
            unpack16(hw[i], hv);
            hmax[i] = amax16(hv);
            gmax[i] = amax16(gv);
            umax[i] = amax16(uv);
            rh = fmaxf(rh, hmax[i]);
            rg = fmaxf(rg, gmax[i]);
            ru = fmaxf(ru, umax[i]);
        }
        row_max3<WPR>(rh, rg, ru, red, wave, lrow);
        const RowQ qh = row_params(rh), qg = row_params(rg), qu = row_params(ru);
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            if (!valid[i]) continue;
            const int b = lt + T * i;
            float v[16];
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
}

template <int MODE>
static pact_status launch_rows(const RowArgs &a, hipStream_t st) {
    if (a.rows == 0 || a.cols == 0) return PACT_OK;
    const int nb = a.cols / 16;
    int wpr, bpl;
    if (nb <= 64) wpr = 1, bpl = 1;
    else if (nb <= 128) wpr = 1, bpl = 2;
    else if (nb <= 192) wpr = 1, bpl = 3;
    else if (nb <= 256) wpr = 1, bpl = 4;
    else if (nb <= 384) wpr = 2, bpl = 3;
    else if (nb <= 512) wpr = 2, bpl = 4;
    else if (nb <= 768) wpr = 4, bpl = 3;
    else if (nb <= 1024) wpr = 4, bpl = 4;
    else if (nb <= 1536) wpr = 4, bpl = 6;
    else wpr = 4, bpl = 8;
    const int rpw = 4 / wpr;
    const dim3 grid((unsigned)((a.rows + rpw - 1) / rpw));
#define PACT_ROWS_CASE(W, B)                                                           \
    if (wpr == W && bpl == B) {                                                        \
        hipLaunchKernelGGL((row_kernel<W, B, MODE>), grid, dim3(256), 0, st, a);        \
        return launch_status();                                                        \
    }
    PACT_ROWS_CASE(1, 1)
    PACT_ROWS_CASE(1, 2)
    PACT_ROWS_CASE(1, 3)
    PACT_ROWS_CASE(1, 4)
    PACT_ROWS_CASE(2, 3)
    PACT_ROWS_CASE(2, 4)
    PACT_ROWS_CASE(4, 3)
    PACT_ROWS_CASE(4, 4)
    PACT_ROWS_CASE(4, 6)
    PACT_ROWS_CASE(4, 8)
#undef PACT_ROWS_CASE
    return PACT_ERR_UNSUPPORTED_SHAPE;
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
__global__ void sigmoid_probe_kernel(const uint16_t *g, float *out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = sigmoid32_bits(g[i]);
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
