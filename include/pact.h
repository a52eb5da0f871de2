/*
 * pact.h -- libpact: the NVFP4 data flow through the frozen projections of a
 * LoRA decoder layer (PACT), for AMD Instinct MI355X (gfx950).
 *
 * What the library computes, and where the pages define it:
 *  - NVFP4: every 16 E2M1 elements share one E4M3 block scale, about 4.5 bits
 *    per element (simolm.com PACT blog post, section "FAQ", the question on
 *    what NVFP4 is).  This library adds one FP32 scale per row (a second-level
 *    scale the pages leave open).
 *  - The seven frozen projections (q/k/v/o/gate/up/down) run as NVFP4 GEMMs
 *    with FP32 accumulation and BF16 output, both in the forward pass and for
 *    the input gradient (blog, section "Method", first bullet; arXiv abstract
 *    of "PACT: NVFP4 Data-Flow LoRA Fine-Tuning on Consumer GPUs").
 *  - Quantization is fused into the RMSNorm and SiLU-multiply kernels; the
 *    quantized RMSNorm output is what the backward reuses; the SiLU-multiply
 *    forward reads BF16 and also keeps NVFP4 copies of gate/up for backward
 *    (blog "Method", second and fourth bullets; abstract).
 *  - Forward and backward NVFP4 weight layouts are rebuilt, transposed and
 *    re-quantized once, then cached (blog "Method", fourth bullet; abstract).
 *  - LoRA adapters A, B stay BF16 and are never quantized (blog "Method",
 *    closing paragraph); the LoRA update is h = W0 x + B A x (kongchang.com
 *    PEFT explainer, LoRA low-rank math).
 *
 * Numerics (one result is admitted for every quantized output):
 *  Row quantizer Q over a row x[0..L), L % 16 == 0:
 *    A = max|x|; d = fl32(A / 2688); if d == 0 every code is a signed zero and
 *    every scale 0; D = fl32(6 d); per block b: t = fl32(max|x_b| / D),
 *    s_b = E4M3 round-to-nearest-even of t, clamped to 448; S = fl32(s_b d);
 *    code = sign | E2M1 round-to-nearest-even of fl32(|x| / S), clamped to 6
 *    (magnitude 0 when S == 0).  fl32 is one IEEE binary32 rounding.
 *  GEMM: out = bf16( fl32(fl32(acc d_a[m]) d_b[n]) + L (+ C) ),
 *    acc = FP32 sum of exact products of decoded operands (E2M1 x E4M3, exact
 *    in FP16), L = sum_j T[m,j] Q[n,j] with T = bf16(s P) and P the FP32
 *    LoRA-down product; for a power-of-two s this is exactly s times the
 *    same sum taken with T = bf16(P).  The
 *    summation order is the kernel's own: GEMM outputs match a sequential
 *    reference within |err| <= 2 BF16 ulp + 1e-3 max_row|ref| and a relative
 *    Frobenius error <= 4e-3.  All quantized outputs are bit-exact.
 *
 * Layout of an NVFP4 tensor [rows, cols] (canonical, row-major, dense):
 *    codes  [rows][cols/2] bytes, element 2j in the low nibble of byte j,
 *           E2M1 code = sign(bit 3) | exponent(bits 2..1) | mantissa(bit 0);
 *    scales [rows][cols/16] E4M3 (OCP "FN", bias 7) bytes, values 0x00..0x7E;
 *    row_scale [rows] FP32.
 * BF16 tensors are passed as raw uint16_t bit patterns, row-major with the
 * given leading dimension (elements).
 *
 * Conventions for every entry point:
 *  - Ownership: every pointer is caller-owned DEVICE memory (except the
 *    pact_nvfp4 / pact_lora descriptor structs themselves, which are host
 *    structs read during the call).  The library allocates and frees nothing
 *    and never synchronizes; it keeps no mutable state.
 *  - Ordering: all device work is enqueued on `stream` (a hipStream_t passed
 *    as void*, NULL = default stream); calls return before it completes.
 *  - Errors: arguments are validated first; on any failure the call returns
 *    the status and enqueues nothing.  A launch failure reported by the HIP
 *    runtime returns PACT_ERR_HIP.  Nothing is printed or thrown.
 *  - Alignment: every device pointer must be 16-byte aligned, and leading
 *    dimensions of BF16 tensors multiples of 8 elements (PACT_ERR_MISALIGNED).
 *  - Inputs must be finite; non-finite inputs give unspecified outputs.
 */
#ifndef PACT_H
#define PACT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PACT_VERSION 1
/* Longest row the fused quantizers accept (columns). */
#define PACT_MAX_ROW 32768

typedef enum {
    PACT_OK = 0,
    PACT_ERR_INVALID_ARG = 1,       /* null required pointer, negative size, bad rank */
    PACT_ERR_UNSUPPORTED_SHAPE = 2, /* contraction/row length not a multiple of 16, too long */
    PACT_ERR_MISALIGNED = 3,        /* pointer not 16-byte aligned or ld not a multiple of 8 */
    PACT_ERR_WORKSPACE = 4,         /* workspace missing or smaller than required */
    PACT_ERR_HIP = 5                /* the HIP runtime reported an error */
} pact_status;

/* An NVFP4 tensor in device memory (layout above).  rows, cols give its shape;
 * cols % 16 == 0. */
typedef struct {
    uint8_t *codes;
    uint8_t *scales;
    float *row_scale;
    int64_t rows;
    int64_t cols;
} pact_nvfp4;

/* BF16 LoRA adapters of one projection with weight W [N][K]:
 * A [r][K] and B [N][r] row-major BF16 bits in device memory; r = 0 (or a NULL
 * descriptor) means frozen path only; scale multiplies the LoRA term. */
typedef struct {
    const uint16_t *A;
    const uint16_t *B;
    int32_t r;
    float scale;
} pact_lora;

/* Version of this ABI (PACT_VERSION). */
int pact_version(void);

/* Human-readable name of a status code (static string). */
const char *pact_status_string(pact_status s);

/* Row quantizer Q (blog "Method": NVFP4 operands for the frozen GEMMs; used
 * for GEMM inputs that have no fused producer, e.g. incoming gradients).
 * x [rows][cols] BF16 with leading dimension ld_x -> *out (out->rows == rows,
 * out->cols == cols).  cols % 16 == 0, cols <= PACT_MAX_ROW. */
pact_status pact_quantize_nvfp4(const uint16_t *x, int64_t ld_x, int64_t rows, int64_t cols,
                                const pact_nvfp4 *out, void *stream);

/* Fused RMSNorm -> quantize (blog "Method", second and fourth bullets):
 * ss = sum x^2 (binary64), rstd = fl32(1 / sqrt(ss / cols + eps)) (binary64
 * ops), y = bf16(fl32(fl32(x rstd) gamma)), yq = Q(y).
 * x [rows][cols] (ld_x), gamma [cols], y [rows][cols] (ld_y; may be NULL),
 * yq (required), rstd [rows] FP32 (may be NULL). */
pact_status pact_rmsnorm_quant_nvfp4(const uint16_t *x, int64_t ld_x, const uint16_t *gamma,
                                     float eps, int64_t rows, int64_t cols,
                                     uint16_t *y, int64_t ld_y, const pact_nvfp4 *yq,
                                     float *rstd, void *stream);

/* Fused SiLU*mul -> quantize (blog "Method", second bullet; abstract):
 * h = bf16(fl32(sigma32(g) u)) with sigma32(g) the correctly rounded binary32
 * value of g / (1 + exp(-g)); hq = Q(h); gq = Q(g) and uq = Q(u) are the
 * NVFP4 copies kept for backward.  g, u [rows][cols] (ld_g, ld_u), h (ld_h;
 * may be NULL), hq required, gq and uq may each be NULL. */
pact_status pact_silu_mul_quant_nvfp4(const uint16_t *g, int64_t ld_g, const uint16_t *u,
                                      int64_t ld_u, int64_t rows, int64_t cols,
                                      uint16_t *h, int64_t ld_h, const pact_nvfp4 *hq,
                                      const pact_nvfp4 *gq, const pact_nvfp4 *uq,
                                      void *stream);

/* Workspace bytes pact_build_weight_layouts needs for a weight [N][K]. */
size_t pact_build_weight_layouts_workspace(int64_t N, int64_t K);

/* Cached weight layouts (blog "Method", fourth bullet): W_fwd = Q over the
 * rows of W [N][K] (blocks along K); R = fl32(decode(W_fwd) * row_scale);
 * W_bwd = Q over the rows of R^T [K][N] (blocks along N).  Pass W (BF16) to
 * quantize it, or W = NULL and W_fwd_in = an already-quantized forward layout
 * (e.g. calibrated offline), which is copied to W_fwd when the two differ.
 * N % 16 == 0, K % 16 == 0, N <= PACT_MAX_ROW. */
pact_status pact_build_weight_layouts(const uint16_t *W, const pact_nvfp4 *W_fwd_in,
                                      int64_t N, int64_t K, const pact_nvfp4 *W_fwd,
                                      const pact_nvfp4 *W_bwd, void *ws, size_t ws_bytes,
                                      void *stream);

/* Workspace bytes the GEMMs of one projection need (forward: output [M][N]
 * over K; input gradient: [M][K] over N) with LoRA rank r: the LoRA-down
 * product [M][r rounded up to 16] BF16, then room for FP32 partial sums when
 * the launch plan splits K across workgroups (small outputs with long K), then
 * B^T [r][N] (the input gradient's LoRA-down reads it when M >= 4096) and
 * A^T [K][r] (the input gradient's LoRA-up reads it when r % 8 == 0).
 * A GEMM given less than this but at least the LoRA-down product runs
 * without the K split; results are within the same tolerance either way and
 * bit-identical across runs with the same workspace size. */
size_t pact_gemm_workspace(int64_t M, int64_t N, int64_t K, int32_t r);

/* Forward NVFP4 GEMM of one frozen projection plus its BF16 LoRA term
 * (blog "Method", first bullet and closing paragraph; PEFT explainer):
 *   Y = bf16( d_x[m] d_w[n] (Xq . W_fwd^T)[m,n] + (bf16(s X A^T) B^T)[m,n] (+ C[m,n]) )
 * Xq [M][K] NVFP4, X [M][K] BF16 (ld_x; only read when lora->r > 0),
 * W_fwd [N][K] NVFP4, C [M][N] BF16 with leading dimension ld_y (may be NULL,
 * may alias Y), Y [M][N] (ld_y).  K % 16 == 0. */
pact_status pact_gemm_nvfp4_fwd(const pact_nvfp4 *Xq, const uint16_t *X, int64_t ld_x,
                                const pact_nvfp4 *W_fwd, const pact_lora *lora,
                                const uint16_t *C, uint16_t *Y, int64_t ld_y,
                                void *ws, size_t ws_bytes, void *stream);

/* Grouped forward of ngroups (1..4) projections that share their input, such
 * as q, k, v or gate, up (blog "Method", first bullet and closing
 * paragraph: the same frozen NVFP4 GEMM and BF16 LoRA term per projection), as one GEMM
 * over the concatenation of their weight rows:
 *   Y[:, cols of g] = bf16( d_x d_w (Xq . W_g^T) + (bf16(s X A_g^T) B_g^T) ),
 * the LoRA term block-diagonal (one LoRA-down over the concatenated ranks).
 * W_fwd [sum N_g][K] NVFP4 holds W_0, W_1, ... row after row (e.g. each built
 * by pact_build_weight_layouts into its slice); group_rows[g] = N_g (host
 * array, multiples of 32); loras (host array of ngroups, or NULL: frozen only)
 * with equal r and scale, A_g [r][K], B_g [N_g][r]; Y [M][sum N_g] (ld_y), no
 * residual.  Workspace: pact_gemm_workspace(M, sum N_g, K, ngroups *
 * round_up(r, 16)).  Each group's columns equal pact_gemm_nvfp4_fwd of that
 * projection within the GEMM tolerance (the K-split plan may differ). */
pact_status pact_gemm_nvfp4_fwd_grouped(const pact_nvfp4 *Xq, const uint16_t *X, int64_t ld_x,
                                        const pact_nvfp4 *W_fwd, int32_t ngroups, const int64_t *group_rows,
                                        const pact_lora *loras, uint16_t *Y, int64_t ld_y, void *ws,
                                        size_t ws_bytes, void *stream);

/* Input-gradient NVFP4 GEMM on the cached transposed layout (blog "Method",
 * first and fourth bullets):
 *   dX = bf16( d_dy[m] d_wb[k] (dYq . W_bwd^T)[m,k] + (bf16(s dY B) A)[m,k] (+ C[m,k]) )
 * dYq [M][N] NVFP4, dY [M][N] BF16 (ld_dy; only read when lora->r > 0),
 * W_bwd [K][N] NVFP4 (from pact_build_weight_layouts), C [M][K] (ld_dx; may be
 * NULL, may alias dX), dX [M][K] (ld_dx).  N % 16 == 0. */
pact_status pact_gemm_nvfp4_dgrad(const pact_nvfp4 *dYq, const uint16_t *dY, int64_t ld_dy,
                                  const pact_nvfp4 *W_bwd, const pact_lora *lora,
                                  const uint16_t *C, uint16_t *dX, int64_t ld_dx,
                                  void *ws, size_t ws_bytes, void *stream);

/* SiLU*mul backward from the NVFP4 gate/up stash (blog "Method", second
 * bullet, and the abstract of "PACT: NVFP4 Data-Flow LoRA Fine-Tuning on
 * Consumer GPUs": the gate and up activations are kept in NVFP4 for the
 * backward pass):
 *   g' = bf16(deq(gq)), u' = bf16(deq(uq))   (deq: code x block scale x row scale),
 *   du = bf16(fl32(dh sigma32(g'))),  dg = bf16(fl32(fl32(dh u') dsilu32(g'))),
 *   dgq = Q(dg), duq = Q(du)   (the operands of the gate/up input-gradient GEMMs),
 * with sigma32 as in the forward and dsilu32(g) the correctly rounded binary32
 * value of sigma(g) (1 + g (1 - sigma(g))).  dh [rows][cols] BF16 (ld_dh); gq,
 * uq the forward's stash; dg, du [rows][cols] BF16 with leading dimension
 * ld_out (each may be NULL); dgq, duq required.  cols % 16 == 0. */
pact_status pact_silu_mul_bwd_quant_nvfp4(const uint16_t *dh, int64_t ld_dh, const pact_nvfp4 *gq,
                                          const pact_nvfp4 *uq, int64_t rows, int64_t cols,
                                          uint16_t *dg, uint16_t *du, int64_t ld_out,
                                          const pact_nvfp4 *dgq, const pact_nvfp4 *duq, void *stream);

/* RMSNorm backward from the NVFP4 norm output (blog "Method", second bullet:
 * the quantized RMSNorm output is reused in backward, the norm input is not
 * saved).  With x^ = y'/gamma, y' = deq(yq) (x^ = 0 where gamma = 0), and
 * S = sum_j dy_j y'_j summed exactly (to 2^-106 relative) and rounded once,
 * c = fl32(S / cols):
 *   dx = bf16( fl32( fl32(dy gamma) - fl32(x^ c) ) rstd  (+ C) ),  dxq = Q(dx),
 * the input gradient of y = x rstd gamma (gamma is frozen: no gamma gradient).
 * dy [rows][cols] BF16 (ld_dy); yq and rstd [rows] from
 * pact_rmsnorm_quant_nvfp4; gamma [cols]; C [rows][cols] (ld_c; the residual
 * gradient, may be NULL); dx [rows][cols] (ld_dx; may be NULL) and dxq (may be
 * NULL), not both NULL.  cols % 16 == 0. */
pact_status pact_rmsnorm_bwd_nvfp4(const uint16_t *dy, int64_t ld_dy, const pact_nvfp4 *yq,
                                   const uint16_t *gamma, const float *rstd, const uint16_t *C,
                                   int64_t ld_c, int64_t rows, int64_t cols, uint16_t *dx,
                                   int64_t ld_dx, const pact_nvfp4 *dxq, void *stream);

/* Workspace bytes of pact_lora_grads_nvfp4 for M tokens, output width N,
 * input width K and LoRA rank r (0 when r <= 0). */
size_t pact_lora_grads_workspace(int64_t M, int64_t N, int64_t K, int32_t r);

/* LoRA weight gradients of one projection on the NVFP4 stash (blog "Method",
 * second bullet and closing paragraph: activations kept for backward are the
 * NVFP4 copies, adapters stay BF16; PEFT explainer: the update B A x):
 *   X^ = bf16(deq(Xq)) [M][K],  T^ = bf16(s X^ A^T),  T' = bf16(s dY B)  [M][r],
 *   dB = dY^T T^  [N][r],   dA = T'^T X^  [r][K],
 * FP32 sums over the tokens (fixed order for a given shape), FP32 outputs.
 * Xq: the projection's input as stashed by the forward (NVFP4 [M][K]); dY
 * [M][N] BF16 (ld_dy): the gradient of the projection's output; lora: A [r][K],
 * B [N][r], scale s; dA [r][K] and dB [N][r] FP32, row-major.  K % 16 == 0,
 * N % 16 == 0, 1 <= r <= 64.  Empty M gives zero gradients.  The workspace
 * (pact_lora_grads_workspace bytes) holds T^, T', B^T and partial sums; X^ is
 * decoded in registers, never stored.  T_dy (may be NULL; 16-byte aligned):
 * T' [M][round_up(r, 16)] BF16 already computed, such as the first bytes of
 * the workspace of a pact_gemm_nvfp4_dgrad call with the same dY and lora
 * (its LoRA-down product, stream-ordered before this call and not yet
 * overwritten); the entry point then does not compute T'. */
pact_status pact_lora_grads_nvfp4(const pact_nvfp4 *Xq, const uint16_t *dY, int64_t ld_dy, int64_t N,
                                  const pact_lora *lora, const uint16_t *T_dy, float *dA, float *dB, void *ws,
                                  size_t ws_bytes, void *stream);

/* One AdamW step of the trainable adapters over a flat buffer of n FP32
 * parameters (hotdry.top Unsloth post, section on paged optimizers: Adam keeps
 * a first and a second moment per trainable parameter, in 32-bit state; the
 * rule is AdamW with decoupled weight decay, Loshchilov & Hutter).  In place:
 *   p <- p (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;
 *   p <- p - lr/(1 - b1^step) . m / (sqrt(v)/sqrt(1 - b2^step) + eps);
 *   w <- bf16(p)   (the BF16 copy the GEMMs read; w may be NULL),
 * in binary32 per element (the coefficients computed on the host in binary64
 * and rounded once).  p, m, v, g, w: device buffers of n elements, 16-byte
 * aligned; g is typically the gradients written by pact_lora_grads_nvfp4 into
 * views of one flat buffer.  step >= 1, 0 <= beta < 1, lr, eps, wd >= 0 and
 * finite, else PACT_ERR_INVALID_ARG.  n == 0 does nothing. */
pact_status pact_adamw_step(float *p, float *m, float *v, const float *g, uint16_t *w, int64_t n, float lr,
                            float beta1, float beta2, float eps, float weight_decay, int64_t step, void *stream);

/* NVFP4-adapted GPTQ, offline calibration of a frozen weight (blog "Method",
 * third bullet, and the arXiv abstract: GPTQ adapted to the NVFP4 block
 * scales, with statistics from reconstructed NVFP4 activations; GPTQ is
 * Frantar et al.).  Two calls:
 *
 * pact_gptq_hessian_nvfp4: H = scale X^T X (+ H when accumulate != 0) in
 * binary64, X [n][K] the dequantized values of the NVFP4 calibration rows Xq
 * (fl32(code x block scale x row scale)); GPTQ's Hessian is scale = 2/n.
 * H: device, [K][K] row-major binary64, 16-byte aligned.  Xq->cols % 16 == 0.
 *
 * pact_gptq_nvfp4: the forward NVFP4 layout W_fwd [N][K] of the BF16 weight
 * W [N][K] (leading dimension ld_w) calibrated with H [K][K]: columns whose
 * diagonal is 0 are dead (weights set to 0); percdamp times the mean diagonal
 * is added to the diagonal; U, the upper Cholesky factor of H^-1, spreads
 * each column's rounding error over the later columns, in lazy batches of
 * `blocksize` columns (16..128, a multiple of 16).  Row scales are the plain
 * quantizer's (max|w| of the original row / 2688); at the first column of
 * every 16-column block the block's E4M3 scale is the plain quantizer's rule
 * on the block's current weights rounded to binary32; each code is the plain
 * quantizer's code of the current weight rounded to binary32.  H is used as
 * scratch (overwritten).  K % 64 == 0 (else PACT_ERR_UNSUPPORTED_SHAPE);
 * workspace of pact_gptq_workspace(N, K) bytes (2 K^2 + N K + 64 K binary64
 * values and change; PACT_ERR_WORKSPACE when smaller).  The result feeds
 * pact_build_weight_layouts(W = NULL, W_fwd_in = W_fwd) for the transposed
 * layout.  If H (after dampening) is not numerically positive definite the
 * output is unspecified. */
pact_status pact_gptq_hessian_nvfp4(const pact_nvfp4 *Xq, double scale, int32_t accumulate, double *H,
                                    void *stream);
size_t pact_gptq_workspace(int64_t N, int64_t K);
pact_status pact_gptq_nvfp4(const uint16_t *W, int64_t ld_w, int64_t N, int64_t K, double *H, double percdamp,
                            int32_t blocksize, const pact_nvfp4 *W_fwd, void *ws, size_t ws_bytes, void *stream);

/* Forward GEMM for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, harnesses that forbid allocation):
 * pact_gemm_nvfp4_fwd with the same arguments and results, but its workspace
 * is a library-owned device array of PACT_NOALLOC_SCRATCH_BYTES bytes, one
 * per GPU, held until the process ends; the call itself allocates nothing.
 * The LoRA-down product [M][round_up(r, 16)] BF16 must fit in that array
 * (else PACT_ERR_WORKSPACE, nothing launched); when the K-split partials do
 * not fit as well, the GEMM runs in one pass over K (same tolerance).  Every
 * call on one GPU shares that GPU's array: calls that overlap in time on one
 * GPU (different streams or threads without ordering between them) race and
 * give undefined results.  Nothing in the array needs clearing between calls:
 * every byte a call reads was written earlier in the same call.  The first
 * call on each device looks the array's address up with that device current;
 * PACT_ERR_HIP when the lookup fails. */
#define PACT_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
size_t pact_noalloc_scratch_bytes(void);
pact_status pact_gemm_nvfp4_fwd_noalloc(const pact_nvfp4 *Xq, const uint16_t *X, int64_t ld_x,
                                        const pact_nvfp4 *W_fwd, const pact_lora *lora, const uint16_t *C,
                                        uint16_t *Y, int64_t ld_y, void *stream);

/* Diagnostic: out[i] = sigma32(g[i]) (the binary32 sigmoid-times-input the
 * SiLU kernel uses) for n BF16 inputs g, so that it can be checked against a
 * reference over all 65536 BF16 values.  Device pointers; stream-ordered. */
pact_status pact_debug_sigmoid32(const uint16_t *g, float *out, int64_t n, void *stream);

/* Diagnostic: out[i] = dsilu32(g[i]) (the binary32 SiLU derivative the SiLU
 * backward uses) for n BF16 inputs g.  Device pointers; stream-ordered. */
pact_status pact_debug_dsilu32(const uint16_t *g, float *out, int64_t n, void *stream);

/* Diagnostic, not part of the data flow: the HBM ceiling of a read/write mix.
 * Reads read_bytes from src and writes write_bytes to dst with the row
 * kernels' access pattern (consecutive lanes on consecutive 16-byte chunks,
 * cached loads, nontemporal stores) and no other work, so its duration is
 * what the memory system delivers for that mix and size.  Chunk c (16 bytes)
 * of dst, c < write_bytes / 16, receives the bitwise xor of the chunks of src
 * that the same thread read up to and including chunk c (zero when none);
 * with write_bytes == 0, dst needs 16 bytes and is left unchanged for a
 * zero-filled source.  Device pointers; stream-ordered.  Errors:
 * PACT_ERR_INVALID_ARG for negative sizes, a null dst, or a null src with
 * read_bytes > 0; PACT_ERR_MISALIGNED for sizes or pointers not multiples
 * of 16. */
pact_status pact_debug_stream(const void *src, int64_t read_bytes, void *dst, int64_t write_bytes, void *stream);

/* Diagnostic: the launch plan of a GEMM with output [M][N] contracted over K
 * with LoRA rank r (0: none) on the current device, as pact_gemm_nvfp4_fwd
 * (dgrad == 0) or pact_gemm_nvfp4_dgrad (dgrad != 0) chooses it given the
 * full workspace (host only, no GPU work): *kernel = 0 for the 256 x 256
 * single-decode kernel, 1-4 for the main kernel with wavefronts (2,2,1),
 * (2,1,2), (1,2,2), (1,1,4); *ks = number of K ranges split across
 * workgroups (1: no split); *fused (may be NULL) = 1 when the LoRA-down runs
 * as workgroups of the split-K launch, 0 when it runs as a launch of its
 * own.  PACT_ERR_INVALID_ARG for negative sizes, r outside 0..256 or null
 * kernel / ks. */
pact_status pact_debug_gemm_plan(int64_t M, int64_t N, int64_t K, int32_t r, int32_t dgrad, int32_t *kernel,
                                 int32_t *ks, int32_t *fused);

/* Diagnostic: the column split of the same launch plan (host only): when
 * *n1 > 0, output columns [0, *n1) run as one launch of the kernel that
 * pact_debug_gemm_plan reports and columns [*n1, N) as a second launch of
 * kernel *kernel2 (numbered as there), so that whole rounds of workgroups
 * fill the CUs; *n1 == 0: one launch.  PACT_ERR_INVALID_ARG as for
 * pact_debug_gemm_plan. */
pact_status pact_debug_gemm_plan_columns(int64_t M, int64_t N, int64_t K, int32_t r, int32_t dgrad, int32_t *n1,
                                         int32_t *kernel2);

/* Diagnostic: how the LoRA-down product T of the same GEMM call is computed
 * (host only, no GPU work), given the full workspace.  Arguments as for
 * pact_debug_gemm_plan, plus ngroups >= 1 projections of rank r each (a
 * grouped forward; 1 for the plain entry points, and dgrad requires 1).
 * *route: 1 = workgroups of the split-K main launch; 2 = the pipelined
 * kernel on contiguous rank rows; 3 = a transpose of the input gradient's
 * strided rank operand, then the pipelined kernel; 4 = the kernel that
 * gathers strided rank rows.  Unless *route == 1, *npass passes over the
 * ranks (64 per pass) are written to rg[i] (16-rank groups of the pass),
 * rows_per_wave[i] (16-row groups per wavefront) and waves[i] (wavefronts
 * per workgroup); each array must hold 4 entries.  PACT_ERR_INVALID_ARG for
 * negative sizes, r < 1, ngroups outside 1..4, more than 256 padded ranks,
 * or a null pointer. */
pact_status pact_debug_lora_down_plan(int64_t M, int64_t N, int64_t K, int32_t r, int32_t ngroups, int32_t dgrad,
                                      int32_t *route, int32_t *npass, int32_t *rg, int32_t *rows_per_wave,
                                      int32_t *waves);

/* Diagnostic: the launch shape of a row kernel for rows of `cols` elements
 * (host only, no GPU work).  op: 0 pact_quantize_nvfp4, 1
 * pact_rmsnorm_quant_nvfp4, 2 pact_silu_mul_quant_nvfp4, 3
 * pact_silu_mul_bwd_quant_nvfp4, 4 pact_rmsnorm_bwd_nvfp4.  Writes the
 * wavefronts that share one row and the 16-element blocks each lane holds.
 * PACT_ERR_INVALID_ARG for an unknown op, cols <= 0 or a null output;
 * PACT_ERR_UNSUPPORTED_SHAPE for cols not a multiple of 16 or above
 * PACT_MAX_ROW (as the entry points themselves). */
pact_status pact_debug_row_plan(int32_t op, int64_t cols, int32_t *waves_per_row, int32_t *blocks_per_lane);

#ifdef __cplusplus
}
#endif
#endif /* PACT_H */
