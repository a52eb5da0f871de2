// pact_host.h -- host-side helpers shared by libpact's entry points:
// argument validation and launch-error mapping.  Validation never touches the
// device, so every error path can be exercised without a GPU.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pact.h"

namespace pact {

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// Validate an NVFP4 descriptor of shape [rows][cols] (cols % 16 == 0).
inline pact_status check_nvfp4(const pact_nvfp4 *q, int64_t rows, int64_t cols) {
    if (!q || !q->codes || !q->scales || !q->row_scale) return PACT_ERR_INVALID_ARG;
    if (q->rows != rows || q->cols != cols) return PACT_ERR_INVALID_ARG;
    if (!aligned16(q->codes) || !aligned16(q->scales) || !aligned16(q->row_scale))
        return PACT_ERR_MISALIGNED;
    return PACT_OK;
}

// Validate a BF16 matrix pointer with leading dimension ld (elements).
inline pact_status check_bf16(const void *p, int64_t ld, int64_t cols) {
    if (!p) return PACT_ERR_INVALID_ARG;
    if (ld < cols) return PACT_ERR_INVALID_ARG;
    if (!aligned16(p) || (ld % 8) != 0) return PACT_ERR_MISALIGNED;
    return PACT_OK;
}

inline pact_status launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? PACT_OK : PACT_ERR_HIP;
}

#define PACT_TRY(expr)                      \
    do {                                    \
        pact_status _s = (expr);            \
        if (_s != PACT_OK) return _s;       \
    } while (0)

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

constexpr int kMaxGroups = 4;  // projections of one grouped GEMM

// LoRA-down product T [M][rpad] = bf16(s . (X [M][Kl] . P^T)) over ranks
// j0 .. j0 + 64 (P(j, k) = Ps[j p_sj + k p_sk], zero for j >= r); launched by
// launch_lora_down (all ranks) and fused into split-K GEMM launches.  X is
// BF16 rows, or (launch_lora_down_nvfp4) the BF16 values of NVFP4 rows:
// X(m, k) = bf16(fl32((code x block scale) x d_m)).
struct DownArgs {
    const uint16_t *X;  // nullptr: no fused LoRA-down
    int64_t ldx;
    int M, Kl;
    const uint16_t *Ps;
    int64_t p_sj, p_sk;
    int r, rpad, j0;
    float scale;
    uint16_t *T;
    const uint8_t *xc, *xs;  // NVFP4 source: codes [M][Kl/2], scales [M][Kl/16]
    const float *xd;         // and row scales [M]
    // grouped LoRA (ngroups > 1, p_sk == 1): ranks come in ngroups blocks of
    // grp_rpad, rank j of block g = j / grp_rpad is row j % grp_rpad (< r) of Pg[g]
    int ngroups, grp_rpad;
    const uint16_t *Pg[4];
    // side job (side_Bt != nullptr), run by extra workgroups of the launch
    // (side_blocks of them): Bt [side_r][side_N] = B^T for B [side_N][side_r]
    const uint16_t *side_B;
    uint16_t *side_Bt;
    int side_N, side_r;
};

// Workgroups of `threads` threads that the side job of d takes (0: none).
inline int side_blocks(const DownArgs &d, int threads) {
    return d.side_Bt ? (int)(((int64_t)d.side_N * d.side_r + threads - 1) / threads) : 0;
}
pact_status launch_lora_down(DownArgs d, hipStream_t st);
pact_status launch_lora_down_nvfp4(DownArgs d, hipStream_t st);

// Compute units of the current device (a host-side property query; 256 when
// the query fails).
inline int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
}

}  // namespace pact
