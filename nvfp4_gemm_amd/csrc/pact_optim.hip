// pact_optim.hip -- fused AdamW step of the trainable adapters over one flat
// FP32 buffer, writing the BF16 copy that the GEMMs read.  The hotdry.top
// Unsloth post (section on paged optimizers) has Adam keep a first and a
// second moment per trainable parameter in 32-bit state; the rule is the
// published AdamW (Loshchilov & Hutter, decoupled weight decay).  Per element,
// binary32 with this operation order (no contraction):
//   p1 = p c_decay                                c_decay = fl32(1 - lr wd)
//   m' = b1 m + c1 g                              c1 = fl32(1 - b1)
//   v' = b2 v + (c2 g) g                          c2 = fl32(1 - b2)
//   p' = p1 - ss (m' / (sqrt(v') rs2 + eps))      ss = fl32(lr / (1 - b1^t)),
//                                                 rs2 = fl32(1 / sqrt(1 - b2^t))
//   w  = bf16(p')
// The update is HBM-bound (16 bytes read, 12 + 2 written per element): every
// element is read and written once with nontemporal accesses, 4 per thread.
#include <math.h>

#include "pact_device.h"
#include "pact_host.h"

namespace pact {

struct AdamArgs {
    float *p, *m, *v;
    const float *g;
    uint16_t *w;  // nullable
    int64_t n;
    float decay, b1, c1, b2, c2, ss, rs2, eps;
};

__device__ __forceinline__ void adam1(const AdamArgs &a, float &p, float &m, float &v, float g) {
    const float p1 = __fmul_rn(p, a.decay);
    m = __fadd_rn(__fmul_rn(a.b1, m), __fmul_rn(a.c1, g));
    v = __fadd_rn(__fmul_rn(a.b2, v), __fmul_rn(__fmul_rn(a.c2, g), g));
    const float den = __fadd_rn(__fmul_rn(__fsqrt_rn(v), a.rs2), a.eps);
    p = __fsub_rn(p1, __fmul_rn(a.ss, __fdiv_rn(m, den)));
}

__global__ __launch_bounds__(256) void adamw_kernel(AdamArgs a) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const int64_t n4 = a.n >> 2;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        f4 p = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(a.p) + i);
        f4 m = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(a.m) + i);
        f4 v = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(a.v) + i);
        const f4 g = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(a.g) + i);
        float pe[4] = {p.x, p.y, p.z, p.w}, me[4] = {m.x, m.y, m.z, m.w}, ve[4] = {v.x, v.y, v.z, v.w};
        const float ge[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) adam1(a, pe[e], me[e], ve[e], ge[e]);
        __builtin_nontemporal_store(f4{pe[0], pe[1], pe[2], pe[3]}, reinterpret_cast<f4 *>(a.p) + i);
        __builtin_nontemporal_store(f4{me[0], me[1], me[2], me[3]}, reinterpret_cast<f4 *>(a.m) + i);
        __builtin_nontemporal_store(f4{ve[0], ve[1], ve[2], ve[3]}, reinterpret_cast<f4 *>(a.v) + i);
        if (a.w)
            __builtin_nontemporal_store(u32x2{f32x2_to_bf16x2(pe[0], pe[1]), f32x2_to_bf16x2(pe[2], pe[3])},
                                        reinterpret_cast<u32x2 *>(a.w) + i);
    }
    // the last n % 4 elements
    const int64_t i = 4 * n4 + threadIdx.x;
    if (blockIdx.x == 0 && i < a.n) {
        float p = a.p[i], m = a.m[i], v = a.v[i];
        adam1(a, p, m, v, a.g[i]);
        a.p[i] = p;
        a.m[i] = m;
        a.v[i] = v;
        if (a.w) a.w[i] = (uint16_t)f32_to_bf16_bits(p);
    }
}

}  // namespace pact

using namespace pact;

extern "C" pact_status pact_adamw_step(float *p, float *m, float *v, const float *g, uint16_t *w, int64_t n,
                                       float lr, float beta1, float beta2, float eps, float weight_decay,
                                       int64_t step, void *stream) {
    if (n < 0 || step < 1) return PACT_ERR_INVALID_ARG;
    if (!(beta1 >= 0.0f && beta1 < 1.0f && beta2 >= 0.0f && beta2 < 1.0f) || !(lr >= 0.0f) || !(eps >= 0.0f) ||
        !(weight_decay >= 0.0f) || !isfinite(lr) || !isfinite(eps) || !isfinite(weight_decay))
        return PACT_ERR_INVALID_ARG;
    if (n == 0) return PACT_OK;
    if (!p || !m || !v || !g) return PACT_ERR_INVALID_ARG;
    if (!aligned16(p) || !aligned16(m) || !aligned16(v) || !aligned16(g) || (w && !aligned16(w)))
        return PACT_ERR_MISALIGNED;
    AdamArgs a;
    a.p = p;
    a.m = m;
    a.v = v;
    a.g = g;
    a.w = w;
    a.n = n;
    // host constants: binary64, rounded once to binary32
    a.decay = (float)(1.0 - (double)lr * (double)weight_decay);
    a.b1 = beta1;
    a.c1 = (float)(1.0 - (double)beta1);
    a.b2 = beta2;
    a.c2 = (float)(1.0 - (double)beta2);
    a.ss = (float)((double)lr / (1.0 - pow((double)beta1, (double)step)));
    a.rs2 = (float)(1.0 / sqrt(1.0 - pow((double)beta2, (double)step)));
    a.eps = eps;
    const int64_t n4 = n / 4;
    int64_t blocks = (n4 + 255) / 256;
    const int64_t cap = (int64_t)device_cus() * 8;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream), a);
    return launch_status();
}
