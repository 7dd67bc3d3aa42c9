/*
 * oracle_sdm.h -- plain, slow CPU reference of the SDM hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The product path
 * (libsdm.so and its Python binding) never calls it, and the two share no
 * code, headers, helpers or tables.
 *
 * Sources (page titles; sections as printed on the pages):
 *   [SDM]   "Sparse Delta Memory：中文精读笔记" (close-reading notes on
 *           arXiv 2607.07386v1): §2.2 notation, §2.3 product-key addressing,
 *           §2.4 Eq. (3)-(5) write / read, §2.5 Fig. 2 shared-residual form
 *           and the worked counter-example, §2.1 Eq. (2) gated delta rule.
 *   [FwPKM] "Fast-weight Product Key Memory：中文精读笔记", §2.2
 *           (per-half top-k, k^2 candidates, softmax over the selection;
 *           the inverse-distance subkey score), §2.3 (the sigmoid gate).
 *
 * Conventions: all arrays are host memory, row-major and contiguous, fp32 for
 * every floating-point tensor (bf16 inputs are widened exactly by the
 * caller). Accumulations run in double; every stored value is rounded once to
 * fp32. Functions return 0 on success and a negative code on invalid
 * arguments (nothing is written then).
 *
 * Every function has pins in tests/test_oracle_*pins.py; none is unpinned.
 */
#ifndef ORACLE_SDM_H
#define ORACLE_SDM_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_EQ4 0   /* per-slot residual, Eq. (4) as printed   */
#define ORACLE_FIG2 1  /* shared residual read off Fig. 2         */

/* A1: half-scores. q [B,H,T,2,dh], subkeys [H,2,n,dh] -> out [B,H,T,2,n].
 * out[..,j,a] = fp32( sum_c q[..,j,c] * K[h,j,a,c] ), summed in double in c order. */
int oracle_half_scores(const float* q, const float* subkeys, int64_t B, int64_t H,
                       int64_t T, int64_t n, int64_t dh, float* out, int nthreads);

/* A1, inverse-distance variant ([FwPKM] §2.2, FwPKM's default scoring):
 * out[..,j,a] = fp32( -log(1e-3 + sum_c (q[..,j,c] - K[h,j,a,c])^2) ), the
 * squared distance summed in double in c order. Same shapes as above. */
int oracle_half_scores_idw(const float* q, const float* subkeys, int64_t B, int64_t H,
                           int64_t T, int64_t n, int64_t dh, float* out, int nthreads);

/* A2-A4 from given half-scores half [B,H,T,2,n], for k selected slots.
 * idx/wt/score [B,H,T,k]: slots ordered by (score desc, slot asc), softmax
 * weights, fp32 slot scores. score_next [B,H,T] (may be NULL): the (k+1)-th
 * slot score found by the same procedure with k+1, or -INFINITY when k == n*n. */
int oracle_select(const float* half, int64_t B, int64_t H, int64_t T, int64_t n,
                  int64_t k, int32_t* idx, float* wt, float* score, float* score_next,
                  int nthreads);

/* A5-A6: the sparse gated delta scan over tokens 0..T-1, in place on M.
 * idx_w/wt_w [B,H,T,W], idx_r/wt_r [B,H,T,R], alpha/beta [B,H,T], v [B,H,T,dv],
 * M [B,H,N,dv] (in: state before token 0, out: after token T-1), y [B,H,T,dv].
 * form: ORACLE_EQ4 or ORACLE_FIG2. Returns -3 on an out-of-range index and
 * -4 on a repeated write index within one token (checked before any write). */
int oracle_scan(const int32_t* idx_w, const float* wt_w, int64_t W,
                const int32_t* idx_r, const float* wt_r, int64_t R,
                const float* alpha, const float* beta, const float* v,
                float* M, float* y, int64_t B, int64_t H, int64_t T, int64_t N,
                int64_t dv, int form, int nthreads);

/* A5-A6 with the table stored in bfloat16 (a storage variant: the pages'
 * per-layer state size implies 2-byte elements, [SDM] §4.5 Table 3 with the
 * element count of §2.8). Same recurrence, in double, as oracle_scan; every
 * stored table element is rounded once to the nearest bfloat16 (ties to even)
 * instead of to fp32; reads widen the stored bits exactly. Mb [B,H,N,dv]
 * holds the bfloat16 bits (in/out); y [B,H,T,dv] is fp32. Same return codes. */
int oracle_scan_bf16(const int32_t* idx_w, const float* wt_w, int64_t W,
                     const int32_t* idx_r, const float* wt_r, int64_t R,
                     const float* alpha, const float* beta, const float* v,
                     uint16_t* Mb, float* y, int64_t B, int64_t H, int64_t T, int64_t N,
                     int64_t dv, int form, int nthreads);

/* Backward of A5-A6 by reverse-mode differentiation of the whole scan, the
 * tokens walked in reverse with each written row restored from its pre-image
 * ([SDM] §2.9 Appendix A, backward memory). Same index/weight/gate/v inputs as
 * oracle_scan; M_in [B,H,N,dv] is the state before token 0 (not modified);
 * dy [B,H,T,dv] the gradient of y; dM_out [B,H,N,dv] that of the final state
 * (NULL: zero). Outputs: dv_ [B,H,T,dv], dalpha/dbeta [B,H,T], dwt_w [B,H,T,W],
 * dwt_r [B,H,T,R], dM_in [B,H,N,dv] (the gradient of the state before token 0).
 * Derivatives are those of the exact recurrence at the fp32 values the forward
 * stores; the adjoint table and every sum are kept in double. */
int oracle_scan_backward(const int32_t* idx_w, const float* wt_w, int64_t W,
                         const int32_t* idx_r, const float* wt_r, int64_t R,
                         const float* alpha, const float* beta, const float* v,
                         const float* M_in, const float* dy, const float* dM_out,
                         float* dv_, float* dalpha, float* dbeta, float* dwt_w, float* dwt_r,
                         float* dM_in, int64_t B, int64_t H, int64_t T, int64_t N, int64_t dv,
                         int form, int nthreads);

/* Gates of the scan from the layer input ([SDM] §2.4, the definitions under
 * Eq. (3)-(4)): per token and head, with sums in double,
 *   alpha[b,h,t] = fp32( exp(-A[h] * softplus(sum_i W_a[h,i] x[b,t,i] + b_dt[h])) )
 *   beta[b,h,t]  = fp32( sigmoid(sum_i W_b[h,i] x[b,t,i]) )
 * x [B,T,d], W_a and W_b [H,d], b_dt and A [H]; alpha, beta [B,H,T]. */
int oracle_gates(const float* x, const float* W_a, const float* W_b, const float* b_dt,
                 const float* A, int64_t B, int64_t T, int64_t d, int64_t H,
                 float* alpha, float* beta, int nthreads);

/* The per-head output after the read ([SDM] §2.4: RMS-Norm, then an
 * elementwise output gate; the gate's activation is read as the sigmoid of
 * [FwPKM] §2.3): o = fp32( y / sqrt(mean_i y_i^2 + eps) * gamma[h] * sigmoid(g) )
 * per row, in double. y, g, o [B,H,T,dv]; gamma [H,dv]. */
int oracle_output_gate(const float* y, const float* gamma, const float* g, double eps,
                       int64_t B, int64_t H, int64_t T, int64_t dv, float* o, int nthreads);

int oracle_version(void);

#ifdef __cplusplus
}
#endif
#endif
