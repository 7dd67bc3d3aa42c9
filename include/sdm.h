/*
 * sdm.h -- C ABI of the Sparse Delta Memory (SDM) hot path on MI355X (gfx950).
 *
 * The operations follow "Sparse Delta Memory：中文精读笔记" (close-reading notes
 * on arXiv 2607.07386v1), cited below as [SDM], and the product-key
 * addressing of "Fast-weight Product Key Memory：中文精读笔记" §2.2, cited as
 * [FwPKM].
 *
 * Common conventions
 *   - Every tensor pointer is a DEVICE pointer owned by the caller. Tensors are
 *     row-major and contiguous; shapes are given in the comments. Sizes are
 *     int64_t. The library never frees or retains caller memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *     compute calls are asynchronous and ordered on that stream; results are
 *     visible after the caller synchronises it.
 *   - Every call validates its arguments on the host before any launch. On
 *     failure it returns a non-zero sdm_status, writes nothing and launches
 *     nothing; sdm_last_error() then describes the failure (thread-local).
 *     A failed launch returns SDM_ERR_HIP. Faults inside a kernel surface at
 *     the caller's next synchronisation. No C++ exception crosses the ABI.
 *   - Pointers to device tensors must be 16-byte aligned (SDM_ERR_ALIGN).
 *   - Empty work (B, H or T equal to 0) is valid, launches nothing and accepts
 *     NULL tensor pointers (empty tensors need not have storage).
 */
#ifndef SDM_H
#define SDM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDM_ABI_VERSION 7

typedef enum sdm_status {
    SDM_OK = 0,
    SDM_ERR_NULL = 1,         /* a required pointer is NULL                      */
    SDM_ERR_SHAPE = 2,        /* a size is negative or sizes are inconsistent    */
    SDM_ERR_DTYPE = 3,        /* unknown dtype or delta form                     */
    SDM_ERR_ALIGN = 4,        /* a device pointer is not 16-byte aligned         */
    SDM_ERR_UNSUPPORTED = 5,  /* valid but outside the sizes the kernels cover   */
    SDM_ERR_HIP = 6,          /* a HIP launch failed                             */
    SDM_ERR_WORKSPACE = 7     /* workspace missing or too small                  */
} sdm_status;

typedef enum sdm_dtype { SDM_F32 = 0, SDM_BF16 = 1 } sdm_dtype;

/* The two write rules the notes keep side by side ([SDM] §2.4-§2.5):
 *   SDM_DELTA_EQ4:  M[i] <- a M[i] + b w_i (v - a M[i])         (Eq. (4), per slot)
 *   SDM_DELTA_FIG2: vhat = sum_j w_j a M[j];  M[i] <- a M[i] + b w_i (v - vhat)
 *                   (shared residual read off Fig. 2; equals the gated delta
 *                   rule Eq. (2) when every slot is selected).            */
typedef enum sdm_delta_form { SDM_DELTA_EQ4 = 0, SDM_DELTA_FIG2 = 1 } sdm_delta_form;

/* SDM_ABI_VERSION of the loaded library. */
int sdm_abi_version(void);

/* Static text for a status code. */
const char* sdm_status_string(int status);

/* Detail of the last failing call on the calling thread ("" if none). */
const char* sdm_last_error(void);

/*
 * sdm_address -- product-key addressing of both branches ([SDM] §2.3, §2.2
 * notation; [FwPKM] §2.2).
 *
 * For each (b, h, t) and each branch (write with k = W, read with k = R):
 *   half-scores  s_j[a] = <q[.., j, :], subkeys[h, j, a, :]>, j in {0, 1}, a < n_sub
 *                (MFMA contraction, fp32 accumulation);
 *   per half     keep the k_h = min(k, n_sub) best, ordered (score desc, index asc);
 *   combine      slot (a, b) -> row a*n_sub + b with score fp32(s_0[a] + s_1[b]);
 *                the k best candidate slots, ordered (score desc, slot asc);
 *   weights      softmax over the k selected slot scores.
 *
 *   q_w, q_r             [B, H, T, 2, dh]   q_dtype (half 0 then half 1)
 *   subkeys_w, subkeys_r [H, 2, n_sub, dh]  k_dtype == q_dtype (may alias)
 *   idx_w, wt_w          [B, H, T, W]       int32 slots, fp32 weights (out)
 *   idx_r, wt_r          [B, H, T, R]       (out)
 *   score_w, score_r     [B, H, T, W|R]     optional (NULL): fp32 slot scores
 *
 * Supported: q_dtype in {SDM_F32, SDM_BF16}; n_sub a multiple of 16 up to 512;
 * dh a multiple of 8 (fp32) or 32 (bf16) up to 256; 1 <= W, R <= min(64, n_sub^2);
 * B * T < 2^32 tokens per call.
 */
int sdm_address(const void* q_w, const void* q_r, int q_dtype,
                const void* subkeys_w, const void* subkeys_r, int k_dtype,
                int64_t B, int64_t H, int64_t T, int64_t n_sub, int64_t dh,
                int64_t W, int64_t R,
                int32_t* idx_w, float* wt_w, int32_t* idx_r, float* wt_r,
                float* score_w, float* score_r, void* stream);

/*
 * sdm_debug_half_scores -- test hook: only the half-score contraction of
 * sdm_address (same kernel code), for one branch.
 *   q [B, H, T, 2, dh], subkeys [H, 2, n_sub, dh], half [B, H, T, 2, n_sub] fp32 (out).
 * Same support as sdm_address.
 */
int sdm_debug_half_scores(const void* q, int q_dtype, const void* subkeys, int k_dtype,
                          int64_t B, int64_t H, int64_t T, int64_t n_sub, int64_t dh,
                          float* half, void* stream);

/*
 * sdm_address_idw -- sdm_address with FwPKM's inverse-distance subkey score
 * ([FwPKM] §2.2, FwPKM's default scoring) in place of the dot product:
 *   half-scores  s_j[a] = -log(1e-3 + ||q[.., j, :] - subkeys[h, j, a, :]||^2)
 * (computed as ||q||^2 + ||K_a||^2 - 2 <q, K_a>, the inner product on MFMA with
 * fp32 accumulation). Per-half top-k, the outer sum, the selection and the
 * softmax are those of sdm_address, so the weights of the selected slots are
 * the normalised products 1 / ((1e-3 + d_0)(1e-3 + d_1)) of the two halves'
 * squared distances. Arguments, layouts, errors and support as sdm_address.
 */
int sdm_address_idw(const void* q_w, const void* q_r, int q_dtype,
                    const void* subkeys_w, const void* subkeys_r, int k_dtype,
                    int64_t B, int64_t H, int64_t T, int64_t n_sub, int64_t dh,
                    int64_t W, int64_t R,
                    int32_t* idx_w, float* wt_w, int32_t* idx_r, float* wt_r,
                    float* score_w, float* score_r, void* stream);

/*
 * sdm_debug_half_scores_idw -- test hook: the inverse-distance half-scores of
 * sdm_address_idw alone (same kernel code), for one branch. Arguments as
 * sdm_debug_half_scores.
 */
int sdm_debug_half_scores_idw(const void* q, int q_dtype, const void* subkeys, int k_dtype,
                              int64_t B, int64_t H, int64_t T, int64_t n_sub, int64_t dh,
                              float* half, void* stream);

/*
 * sdm_state_init -- per-sequence initial table from the (learned) initial
 * state M0 ([SDM] §2.6): M[b] = M0 for every b.
 *   M0 [H, N, dv] fp32, M [B, H, N, dv] (out) in m_dtype: SDM_F32 (a copy) or
 *   SDM_BF16 (each element rounded to nearest-even bfloat16). dv must be a
 *   multiple of 4.
 */
int sdm_state_init(const float* M0, void* M, int m_dtype, int64_t B, int64_t H, int64_t N,
                   int64_t dv, void* stream);

/*
 * sdm_scan_workspace_bytes -- device workspace sdm_scan_forward needs for these
 * sizes (0 when there is no work, -1 when the sizes are invalid).
 */
int64_t sdm_scan_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t W, int64_t R,
                                 int64_t dv);

/*
 * sdm_scan_forward -- the sparse gated delta recurrence with its sparse read,
 * sequential in t for each (b, h) ([SDM] §2.4 Eq. (3)-(5), §2.5 Fig. 2):
 *   for t = 0 .. T-1:
 *     for i in idx_w[b,h,t,:]:  Mt = alpha[b,h,t] * M[b,h,i,:]              (Eq. 3)
 *                               M[b,h,i,:] = Mt + beta * wt_w_i * (v - P_i)
 *                               P_i = Mt (EQ4)  or  sum_j wt_w_j * alpha * M[b,h,j,:] (FIG2)
 *     y[b,h,t,:] = sum_i wt_r_i * M[b,h,idx_r_i,:]   (after this token's writes, Eq. 5)
 *   Rows that no token selects for writing are never touched (bit-identical).
 *
 *   idx_w, wt_w  [B, H, T, W]   int32 / fp32     idx_r, wt_r [B, H, T, R]
 *   alpha, beta  [B, H, T]      fp32 gates
 *   v            [B, H, T, dv]  v_dtype (SDM_F32 or SDM_BF16)
 *   M            [B, H, N, dv]  m_dtype, in: state before token 0, out: after token T-1
 *   y            [B, H, T, dv]  fp32 (out)
 *   m_dtype      SDM_F32, or SDM_BF16: the table is stored in bfloat16 (the
 *                2-byte state elements the notes' per-layer state size implies,
 *                [SDM] §4.5 Table 3 with §2.8's element count); each update is
 *                computed in fp32 from the widened row and stored rounded to
 *                nearest even, halving the bytes of every row access
 *   workspace    device buffer of >= sdm_scan_workspace_bytes(B,H,T,W,R,dv) bytes,
 *                16-byte aligned; its contents on entry do not matter.
 *
 * The state is in/out, so a sequence split over several calls gives the same
 * result as one call. Preconditions: indices in [0, N) and the W write indices
 * of one token distinct (sdm_address guarantees both). Entries that break the
 * first are skipped (memory-safe, result unspecified); the second gives an
 * unspecified result. Weights are used as given.
 * Supported: 1 <= W, R <= 256, N <= 2^18, dv a multiple of 4 (of 8 for a bf16
 * table), N * dv * 4 < 2^31.
 */
int sdm_scan_forward(const int32_t* idx_w, const float* wt_w, int64_t W,
                     const int32_t* idx_r, const float* wt_r, int64_t R,
                     const float* alpha, const float* beta,
                     const void* v, int v_dtype,
                     void* M, int m_dtype, float* y,
                     int64_t B, int64_t H, int64_t T, int64_t N, int64_t dv,
                     int form, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * sdm_scan_gated_workspace_bytes -- device workspace sdm_scan_forward_gated
 * needs: sdm_scan_workspace_bytes rounded up to 256, plus B*H*T*dv*4 bytes for
 * y in the calls that keep it themselves (0 when there is no work, -1 when the
 * sizes are invalid).
 */
int64_t sdm_scan_gated_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t W, int64_t R,
                                       int64_t dv);

/*
 * sdm_scan_forward_gated -- sdm_scan_forward followed by the head's output step
 * of the SDM layer ([SDM] §2.4: the read, then RMS-Norm and the output gate;
 * the same step as sdm_output_gate):
 *   o[b,h,t,i] = y[b,h,t,i] / sqrt(mean_j y[b,h,t,j]^2 + eps) * gamma[h,i] * sigmoid(g[b,h,t,i])
 * Arguments as sdm_scan_forward and sdm_output_gate, except:
 *   y          [B, H, T, dv] fp32 (out), or NULL: then y is not returned
 *   gamma      [H, dv] fp32; g [B, H, T, dv] g_dtype (SDM_F32 or SDM_BF16);
 *   eps >= 0;  o [B, H, T, dv] fp32 (out), not aliasing y
 *   workspace  >= sdm_scan_gated_workspace_bytes(B,H,T,W,R,dv) bytes, 16-byte aligned
 * The table M and y are bit-identical to sdm_scan_forward's, and o to
 * sdm_output_gate applied to that y. Where the scan splits the table rows into
 * partitions whose partial sums of y a last pass adds (long calls: the usual
 * case), that pass also normalises and gates each row while it holds it in
 * registers (d_v <= 1024), so y is stored only if requested and never read
 * back; otherwise y is stored (to `y`, or the workspace) and the output step
 * runs after the scan. Same support as sdm_scan_forward, and B*H*T < 2^32.
 */
int sdm_scan_forward_gated(const int32_t* idx_w, const float* wt_w, int64_t W,
                           const int32_t* idx_r, const float* wt_r, int64_t R,
                           const float* alpha, const float* beta,
                           const void* v, int v_dtype,
                           void* M, int m_dtype, float* y,
                           const float* gamma, const void* g, int g_dtype, float eps, float* o,
                           int64_t B, int64_t H, int64_t T, int64_t N, int64_t dv,
                           int form, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * sdm_scan_forward_noalloc -- sdm_scan_forward without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). Arguments, layouts,
 * results and support as sdm_scan_forward (the table and y are bit-identical
 * to it), except:
 *   - the scan's scratch (plan records, partial sums, counters) is one array of
 *     64 MiB per GPU inside the library, held from the first call on that GPU
 *     until the process ends; the call allocates and frees nothing;
 *   - calls of more tokens than that scratch holds at once are run as several
 *     launch chunks in order (the same result: the state carries over exactly);
 *     a call whose streams need more than 64 MiB for even one token per launch
 *     (B*H in the thousands) returns SDM_ERR_UNSUPPORTED;
 *   - every call on a GPU uses that GPU's one array, so calls that overlap in
 *     time on one GPU (on different streams or from different threads) race and
 *     give unspecified results; calls on one stream are ordered and safe;
 *   - `stream` selects the GPU (its device), else the current device.
 */
int sdm_scan_forward_noalloc(const int32_t* idx_w, const float* wt_w, int64_t W,
                             const int32_t* idx_r, const float* wt_r, int64_t R,
                             const float* alpha, const float* beta,
                             const void* v, int v_dtype,
                             void* M, int m_dtype, float* y,
                             int64_t B, int64_t H, int64_t T, int64_t N, int64_t dv,
                             int form, void* stream);

/*
 * Training: the forward with pre-images, then the backward that undoes it.
 * ([SDM] §2.9 Appendix A, backward memory: the forward writes the table in
 * place; the backward walks the tokens in reverse and restores each written
 * row from its stored pre-image, so the memory is O(N*dv + T*W*dv) instead of
 * one table per step.)
 */

/*
 * sdm_scan_snapshot_bytes -- bytes of the pre-image buffer for these sizes:
 * B*H*T*W*dv*4 (-1 when the sizes are invalid).
 */
int64_t sdm_scan_snapshot_bytes(int64_t B, int64_t H, int64_t T, int64_t W, int64_t dv);

/*
 * sdm_scan_forward_save -- sdm_scan_forward on an fp32 table (same arguments
 * but m_dtype; M bit-identical to it, y equal up to the order in which the read
 * rows are added) that also
 * stores, for every write, the row as it was before this token's decay:
 *   snap [B, H, T, W, dv] fp32 (out): snap[b,h,t,p,:] = M_{t-1}[b,h,idx_w[b,h,t,p],:]
 * The workspace is the one sdm_scan_workspace_bytes gives. Same support as
 * sdm_scan_forward.
 */
int sdm_scan_forward_save(const int32_t* idx_w, const float* wt_w, int64_t W,
                          const int32_t* idx_r, const float* wt_r, int64_t R,
                          const float* alpha, const float* beta,
                          const void* v, int v_dtype,
                          float* M, float* y, float* snap,
                          int64_t B, int64_t H, int64_t T, int64_t N, int64_t dv,
                          int form, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * sdm_scan_backward_workspace_bytes -- device workspace sdm_scan_backward needs
 * (per-slab partial sums of the weight and gate gradients, and the planner's
 * W + 2R source words per token and stream that let the reverse walk load a
 * token's rows several tokens early); 0 when there is no work, -1 when the
 * sizes are invalid.
 */
int64_t sdm_scan_backward_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t W, int64_t R,
                                          int64_t dv);

/*
 * sdm_scan_backward -- reverse-mode derivatives of one sdm_scan_forward_save
 * call, tokens T-1 .. 0, with the forward's writes undone in place.
 *   idx_w, wt_w, idx_r, wt_r, alpha, beta, v, form: as given to the forward call
 *   snap  [B, H, T, W, dv] fp32: the forward call's pre-images
 *   dy    [B, H, T, dv] fp32: dL/dy
 *   M     [B, H, N, dv] fp32, in: the state after the forward call;
 *         out: the state before it (bit-identical to what the forward got)
 *   dM    [B, H, N, dv] fp32, in: dL/dM after the call (zeros if the final state
 *         does not enter the loss); out: dL/dM before the call
 *   dv_out [B, H, T, dv], dalpha, dbeta [B, H, T], dwt_w [B, H, T, W],
 *   dwt_r [B, H, T, R]: fp32 gradients (out)
 *   workspace: >= sdm_scan_backward_workspace_bytes(B,H,T,W,R,dv) bytes, 16-byte aligned
 * A sequence split into forward calls is differentiated call by call, last
 * call first, passing M and dM along. Preconditions: those of the forward, and
 * also the R read indices of one token distinct (sdm_address guarantees it).
 * Supported: as sdm_scan_forward; W, R <= 256 with ceil(W/G) + ceil(R/G) <= 16
 * wavefronts for some slab width (G = 64 / (S / 4) rows per wavefront, S in
 * {4, 8, 16, 32} dividing dv).
 */
int sdm_scan_backward(const int32_t* idx_w, const float* wt_w, int64_t W,
                      const int32_t* idx_r, const float* wt_r, int64_t R,
                      const float* alpha, const float* beta,
                      const void* v, int v_dtype, const float* snap, const float* dy,
                      float* M, float* dM,
                      float* dv_out, float* dalpha, float* dbeta, float* dwt_w, float* dwt_r,
                      int64_t B, int64_t H, int64_t T, int64_t N, int64_t dv,
                      int form, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * sdm_state_init_backward -- adjoint of sdm_state_init: the gradient of the
 * shared initial state, dM0[h] = sum over b of dM[b, h] (added in b order).
 *   dM [B, H, N, dv] fp32, dM0 [H, N, dv] fp32 (out). dv a multiple of 4.
 */
int sdm_state_init_backward(const float* dM, float* dM0, int64_t B, int64_t H, int64_t N,
                            int64_t dv, void* stream);

/*
 * The steps either side of the scan ([SDM] §2.4).
 *
 * sdm_gates -- the scan's per-head scalar gates from the layer input:
 *   alpha[b,h,t] = exp(-A[h] * softplus(<W_a[h,:], x[b,t,:]> + b_dt[h]))
 *   beta[b,h,t]  = sigmoid(<W_b[h,:], x[b,t,:]>)
 * The projections of all heads are one MFMA contraction over d with fp32
 * accumulation (bf16 or fp32 operands); softplus, exp and sigmoid in fp32.
 *   x [B, T, d] x_dtype; W_a, W_b [H, d] w_dtype == x_dtype; b_dt, A [H] fp32;
 *   alpha, beta [B, H, T] fp32 (out): the layout sdm_scan_forward reads.
 * Supported: d a multiple of 32 (bf16) or 8 (fp32) up to 2^20, H <= 4096,
 * B * T < 2^32 tokens per call.
 */
int sdm_gates(const void* x, int x_dtype, const void* W_a, const void* W_b, int w_dtype,
              const float* b_dt, const float* A, int64_t B, int64_t T, int64_t d, int64_t H,
              float* alpha, float* beta, void* stream);

/*
 * sdm_output_gate -- each head's output after the read: RMS-Norm of the row
 * y[b,h,t,:], then the elementwise output gate; the gate's activation is taken
 * to be the sigmoid ([FwPKM] §2.3's output gate; the SDM notes name the gate
 * without its activation):
 *   o[b,h,t,i] = y[b,h,t,i] / sqrt(mean_j y[b,h,t,j]^2 + eps) * gamma[h,i] * sigmoid(g[b,h,t,i])
 *   y, o [B, H, T, dv] fp32; g [B, H, T, dv] g_dtype (gate pre-activation);
 *   gamma [H, dv] fp32; eps >= 0. o may not alias y. dv a multiple of 4;
 *   B * H * T < 2^32 rows per call.
 * The head-mixing projection W_o that follows is a plain dense layer and is
 * not part of this library.
 */
int sdm_output_gate(const float* y, const float* gamma, const void* g, int g_dtype, float eps,
                    int64_t B, int64_t H, int64_t T, int64_t dv, float* o, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SDM_H */
