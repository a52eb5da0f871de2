/*
 * pact_oracle.h -- plain, slow CPU oracle for the NVFP4 frozen-projection
 * data flow of PACT (LoRA fine-tuning with an NVFP4 data flow).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this code: only the tests, the smoke check and the benchmark's
 * cpu_baseline leg use it.  It shares no source with the HIP library.
 *
 * Sources (web pages on PACT):
 *   [blog]     simolm.com post on PACT, sections "Problem", "Method", "FAQ"
 *   [abstract] arXiv abstract page "PACT: NVFP4 Data-Flow LoRA Fine-Tuning on
 *              Consumer GPUs", the abstract paragraph
 *   [peft]     kongchang.com PEFT explainer, subsection on LoRA's low-rank math
 *
 * Where the pages leave a step open the oracle takes one plain reading; each
 * such reading is stated beside the function that takes it.  Floating point
 * follows the stated op sequence with one IEEE binary32 (or binary64 where
 * said) rounding per op, compiled with -ffp-contract=off and no fast-math.
 *
 * BF16 is passed as raw uint16_t bit patterns everywhere.
 */
#ifndef PACT_ORACLE_H
#define PACT_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- element formats ([blog] FAQ: 16 E2M1 values share one E4M3 scale) ---- */
float    orc_e2m1_value(uint8_t code);          /* code 0..15 -> value          */
float    orc_e4m3_value(uint8_t byte);          /* byte 0..255 -> value (NaN for 0x7F/0xFF) */
uint8_t  orc_e2m1_encode_mag(float r);          /* r >= 0 -> magnitude code 0..7, RNE, sat 6 */
uint8_t  orc_e4m3_encode(float t);              /* t >= 0 -> byte 0x00..0x7E, RNE, sat 448   */
float    orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16(float f);              /* round to nearest even                      */

/* ---- row quantizer Q: per-row FP32 scale d, per-16 E4M3 scale, E2M1 codes ----
 * x: rows x cols FP32 values with row stride ld (elements); cols % 16 == 0.
 * codes: rows x cols/2 bytes (element 2j in the low nibble of byte j),
 * scales: rows x cols/16 bytes, d: rows floats.  */
void orc_quantize_rows_f32(const float *x, int64_t ld, int64_t rows, int64_t cols,
                           uint8_t *codes, uint8_t *scales, float *d);
void orc_quantize_rows_bf16(const uint16_t *x, int64_t ld, int64_t rows, int64_t cols,
                            uint8_t *codes, uint8_t *scales, float *d);

/* GEMM operand value b = (+-E2M1) * E4M3 (exact; the row scale d is NOT applied) */
void orc_operand_values(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                        int64_t cols, float *b);
/* full dequantization value = b * d[row] (one binary32 rounding) */
void orc_dequantize(const uint8_t *codes, const uint8_t *scales, const float *d,
                    int64_t rows, int64_t cols, float *out);

/* ---- fused RMSNorm -> quantize ([blog] Method, bullets 2 and 4; [abstract]) ----
 * y = bf16(x * rstd * gamma), yq = Q(y), rstd = 1/sqrt(mean(x^2) + eps). */
void orc_rmsnorm_quant(const uint16_t *x, int64_t ld, const uint16_t *gamma, float eps,
                       int64_t rows, int64_t cols, uint16_t *y, uint8_t *codes,
                       uint8_t *scales, float *d, float *rstd);
/* exact sum of squares of one BF16 row, correctly rounded to binary64 */
double orc_sumsq_bf16(const uint16_t *x, int64_t n);

/* ---- fused SiLU*mul -> quantize ([blog] Method, bullet 2; [abstract]) ---- */
float orc_sigmoid_mul_g(uint16_t g_bits);   /* correctly rounded binary32 of g/(1+exp(-g)) */
int   orc_sigmoid_check_table(void);        /* 0 if every finite BF16 input was decided safely */
void  orc_silu_mul_quant(const uint16_t *g, const uint16_t *u, int64_t ld, int64_t rows,
                         int64_t cols, uint16_t *h,
                         uint8_t *hc, uint8_t *hs, float *hd,
                         uint8_t *gc, uint8_t *gs, float *gd,   /* may be NULL */
                         uint8_t *uc, uint8_t *us, float *ud);  /* may be NULL */

/* ---- cached forward / backward weight layouts ([blog] Method, bullet 4) ----
 * W: N x K BF16 or NULL; if NULL, (fc, fs, fd) is taken as the given forward
 * layout.  Outputs: forward layout (N rows of K) and backward layout (K rows of N). */
void orc_build_weight_layouts(const uint16_t *W, int64_t N, int64_t K,
                              uint8_t *fc, uint8_t *fs, float *fd,
                              uint8_t *bc, uint8_t *bs, float *bd, int use_given_fwd);

/* ---- NVFP4 GEMM with BF16 LoRA term ([blog] Method, bullets 1 and final note;
 * [peft] LoRA: h = W0 x + B A x) ----
 * Generic "TN" form used for both passes:
 *   out[m,n] = bf16( fl32(fl32(acc*da[m])*db[n]) + fl32(s*L[m,n]) (+ C[m,n]) )
 *   acc = sequential FP32 sum over k of a[m,k]*b[n,k] (operand values, exact products)
 *   L[m,n] = sequential FP32 sum over j of T[m,j]*Q[n,j],
 *   T[m,j] = bf16(sequential FP32 sum over k2 of Xl[m,k2]*P[j,k2])
 * Only rows listed in row_idx (n_rows of them) are computed; out is n_rows x N.
 * Forward:  a = Xq, b = W_fwd, Xl = X [M,K], P = A [r,K], Q = B [N,r].
 * dgrad:    a = dYq, b = W_bwd, Xl = dY [M,N], P = B^T, Q = A^T (handled below). */
void orc_gemm_fwd(const uint8_t *xc, const uint8_t *xs, const float *xd,
                  const uint16_t *X, int64_t M, int64_t K,
                  const uint8_t *wc, const uint8_t *ws, const float *wd, int64_t N,
                  const uint16_t *A, const uint16_t *B, int32_t r, float s,
                  const uint16_t *C, const int64_t *row_idx, int64_t n_rows, uint16_t *Y);
void orc_gemm_dgrad(const uint8_t *gc, const uint8_t *gs, const float *gd,
                    const uint16_t *dY, int64_t M, int64_t N,
                    const uint8_t *wc, const uint8_t *ws, const float *wd, int64_t K,
                    const uint16_t *A, const uint16_t *B, int32_t r, float s,
                    const uint16_t *C, const int64_t *row_idx, int64_t n_rows, uint16_t *dX);

/* ---- nonlinear backward from the NVFP4 stash ([blog] Method, bullet 2;
 * [abstract]: quantized RMSNorm outputs reused, gate/up saved in NVFP4) ---- */
float orc_dsilu(uint16_t g_bits);           /* correctly rounded binary32 of d/dg (g sigma(g)) */
int   orc_dsilu_check_table(void);          /* 0 if every finite BF16 input was decided safely */
/* g' = bf16(deq(gq)), u' = bf16(deq(uq)); du = bf16(dh sigma32(g')),
 * dg = bf16((dh u') dsilu32(g')); dgq = Q(dg), duq = Q(du) (outputs may be NULL) */
void  orc_silu_mul_bwd_quant(const uint16_t *dh, int64_t ld, int64_t rows, int64_t cols,
                             const uint8_t *gc, const uint8_t *gs, const float *gd,
                             const uint8_t *uc, const uint8_t *us, const float *ud,
                             uint16_t *dg, uint16_t *du,
                             uint8_t *dgc, uint8_t *dgs, float *dgd,
                             uint8_t *duc, uint8_t *dus, float *dud);
/* exact dot product of a BF16 and a binary32 vector, rounded once to binary64 */
double orc_dot_bf16_f32(const uint16_t *a, const float *b, int64_t n);
/* dx = bf16(((dy gamma) - x^ c) rstd (+ C)), x^ = deq(yq)/gamma, c = fl32(S/H),
 * S = exact sum of dy deq(yq); dxq = Q(dx) (dx, dxq, C may be NULL) */
void  orc_rmsnorm_bwd(const uint16_t *dy, int64_t ld, const uint8_t *yc, const uint8_t *ys,
                      const float *yd, const uint16_t *gamma, const float *rstd,
                      const uint16_t *C, int64_t ldc, int64_t rows, int64_t cols, uint16_t *dx,
                      uint8_t *dxc, uint8_t *dxs, float *dxd);

/* ---- LoRA weight gradients on the NVFP4 stash ([blog] Method, bullet 2 and
 * final note; [peft] LoRA) ----
 * X^ = bf16(deq(Xq)) [M,K]; T^ = s bf16(X^ A^T), T' = s bf16(dY B) [M,r];
 * dB = dY^T T^ [N,r], dA = T'^T X^ [r,K], summed in binary64. */
void orc_lora_grads(const uint8_t *xc, const uint8_t *xs, const float *xd, int64_t M, int64_t K,
                    const uint16_t *dY, int64_t ld_dy, int64_t N, const uint16_t *A, const uint16_t *B,
                    int32_t r, float s, double *dA, double *dB);

/* ---- NVFP4-adapted GPTQ ([blog] Method, bullet 3; [abs]) ----
 * The column sweep of GPTQ over W [N][K] (binary64, destroyed: on return it
 * holds the quantized values) with the upper Cholesky factor U [K][K] of the
 * inverse Hessian, lazy batches of bs columns, and the NVFP4 block rule with
 * the given row scales d [N]: codes [N][K/2], scale bytes [N][K/16]. */
void orc_gptq_sweep(const double *U, double *W, const float *d, int64_t N, int64_t K, int32_t bs,
                    uint8_t *codes, uint8_t *scales);

int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
