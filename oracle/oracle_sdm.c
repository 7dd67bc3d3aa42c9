/*
 * oracle_sdm.c -- plain, slow CPU reference of the SDM hot path.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle_sdm.h). Written from the pages:
 *   [SDM]   "Sparse Delta Memory：中文精读笔记"
 *   [FwPKM] "Fast-weight Product Key Memory：中文精读笔记"
 *
 * Readings where the pages leave a step open (each is pinned by a test):
 *   - slot (a, b) of the outer sum is row a*n + b, a from half 0;
 *   - when k > n each half keeps all n sub-scores (k_h = min(k, n));
 *   - ties are broken by the lower index: per half by sub-index, in the final
 *     selection by slot index;
 *   - half-scores are rounded to fp32 and a slot score is one fp32 add;
 *   - the weights are a plain softmax over the selected fp32 slot scores;
 *   - within one token all write rows are updated first, then the read sees
 *     the updated table (read-after-write).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared -pthread
 * (no fast-math, no FMA contraction: every double operation is rounded as
 * written).
 */
#include "oracle_sdm.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

int oracle_version(void) { return 3; }

/* ------------------------------------------------------------------ */
/* a tiny "run f(i) for i in [0, count) on nthreads threads" helper.   */
/* Work items are independent, so results never depend on nthreads.   */
/* ------------------------------------------------------------------ */
typedef void (*item_fn)(void* ctx, int64_t item);
typedef struct {
    item_fn fn;
    void* ctx;
    int64_t count;
    int tid, nthreads;
} par_arg;

static void* par_body(void* p) {
    par_arg* a = (par_arg*)p;
    for (int64_t i = a->tid; i < a->count; i += a->nthreads) a->fn(a->ctx, i);
    return NULL;
}

static void parallel_for(item_fn fn, void* ctx, int64_t count, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads == 1 || count <= 1) {
        for (int64_t i = 0; i < count; ++i) fn(ctx, i);
        return;
    }
    pthread_t th[256];
    par_arg args[256];
    for (int t = 0; t < nthreads; ++t) {
        args[t].fn = fn; args[t].ctx = ctx; args[t].count = count;
        args[t].tid = t; args[t].nthreads = nthreads;
        pthread_create(&th[t], NULL, par_body, &args[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------ */
/* A1 -- half-scores [SDM §2.3; FwPKM §2.2]: each half-query is scored  */
/* against the n subkeys of its half by a dot product.                 */
/* ------------------------------------------------------------------ */
typedef struct {
    const float *q, *K;
    int64_t H, T, n, dh;
    float* out;
} hs_ctx;

static void hs_item(void* p, int64_t bht) {
    hs_ctx* c = (hs_ctx*)p;
    int64_t h = (bht / c->T) % c->H;
    for (int j = 0; j < 2; ++j) {
        const float* qj = c->q + (bht * 2 + j) * c->dh;
        for (int64_t a = 0; a < c->n; ++a) {
            const float* ka = c->K + ((h * 2 + j) * c->n + a) * c->dh;
            double acc = 0.0;
            for (int64_t i = 0; i < c->dh; ++i) acc += (double)qj[i] * (double)ka[i];
            c->out[(bht * 2 + j) * c->n + a] = (float)acc;
        }
    }
}

int oracle_half_scores(const float* q, const float* subkeys, int64_t B, int64_t H,
                       int64_t T, int64_t n, int64_t dh, float* out, int nthreads) {
    if (!q || !subkeys || !out) return -1;
    if (B < 0 || H < 0 || T < 0 || n < 1 || dh < 1) return -2;
    hs_ctx c = {q, subkeys, H, T, n, dh, out};
    parallel_for(hs_item, &c, B * H * T, nthreads);
    return 0;
}

/* ------------------------------------------------------------------ */
/* A1, inverse-distance variant [FwPKM §2.2]: the default FwPKM score of */
/* a subkey is s = -log(1e-3 + ||q - K_a||^2), so a near subkey scores   */
/* high; the selection that follows is the same outer sum and top-k.    */
/* The squared distance is summed in double over the componentwise      */
/* differences (no expansion into norms and a dot product).             */
/* ------------------------------------------------------------------ */
#define ORACLE_IDW_EPS 1e-3   /* the constant FwPKM §2.2 adds to the squared distance */

static void hs_idw_item(void* p, int64_t bht) {
    hs_ctx* c = (hs_ctx*)p;
    int64_t h = (bht / c->T) % c->H;
    for (int j = 0; j < 2; ++j) {
        const float* qj = c->q + (bht * 2 + j) * c->dh;
        for (int64_t a = 0; a < c->n; ++a) {
            const float* ka = c->K + ((h * 2 + j) * c->n + a) * c->dh;
            double d2 = 0.0;
            for (int64_t i = 0; i < c->dh; ++i) {
                double d = (double)qj[i] - (double)ka[i];
                d2 += d * d;
            }
            c->out[(bht * 2 + j) * c->n + a] = (float)(-log(ORACLE_IDW_EPS + d2));
        }
    }
}

int oracle_half_scores_idw(const float* q, const float* subkeys, int64_t B, int64_t H,
                           int64_t T, int64_t n, int64_t dh, float* out, int nthreads) {
    if (!q || !subkeys || !out) return -1;
    if (B < 0 || H < 0 || T < 0 || n < 1 || dh < 1) return -2;
    hs_ctx c = {q, subkeys, H, T, n, dh, out};
    parallel_for(hs_idw_item, &c, B * H * T, nthreads);
    return 0;
}

/* ------------------------------------------------------------------ */
/* A2-A4 -- product-key selection [SDM §2.3; FwPKM §2.2].              */
/* ------------------------------------------------------------------ */
typedef struct {
    float s;
    int64_t id;
} scored;

/* order: higher score first; equal scores -> lower index first */
static int by_score_then_index(const void* x, const void* y) {
    const scored* a = (const scored*)x;
    const scored* b = (const scored*)y;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->id > b->id) - (a->id < b->id);
}

/* Top-k slots of one token-branch by product keys. h0, h1: the n half-scores
 * of half 0 and half 1. Writes kk slots (kk <= n*n) with their fp32 scores,
 * ordered by (score desc, slot asc). */
static void pkm_topk(const float* h0, const float* h1, int64_t n, int64_t kk,
                     int64_t* slot_out, float* score_out) {
    int64_t kh = kk < n ? kk : n;             /* per-half keep count */
    scored* best0 = (scored*)malloc((size_t)n * sizeof(scored));
    scored* best1 = (scored*)malloc((size_t)n * sizeof(scored));
    scored* cand = (scored*)malloc((size_t)(kh * kh) * sizeof(scored));
    /* A2: per-half top-kh, each half ordered by (score desc, sub-index asc) */
    for (int64_t a = 0; a < n; ++a) { best0[a].s = h0[a]; best0[a].id = a; }
    for (int64_t b = 0; b < n; ++b) { best1[b].s = h1[b]; best1[b].id = b; }
    qsort(best0, (size_t)n, sizeof(scored), by_score_then_index);
    qsort(best1, (size_t)n, sizeof(scored), by_score_then_index);
    /* A3: all kh*kh outer sums; slot score = one fp32 add; slot = a*n + b */
    int64_t m = 0;
    for (int64_t i = 0; i < kh; ++i)
        for (int64_t j = 0; j < kh; ++j) {
            float s = best0[i].s + best1[j].s;
            cand[m].s = s;
            cand[m].id = best0[i].id * n + best1[j].id;
            ++m;
        }
    qsort(cand, (size_t)m, sizeof(scored), by_score_then_index);
    for (int64_t i = 0; i < kk; ++i) { slot_out[i] = cand[i].id; score_out[i] = cand[i].s; }
    free(cand); free(best1); free(best0);
}

typedef struct {
    const float* half;
    int64_t n, k;
    int32_t* idx;
    float *wt, *score, *score_next;
} sel_ctx;

static void sel_item(void* p, int64_t bht) {
    sel_ctx* c = (sel_ctx*)p;
    int64_t n = c->n, k = c->k, N = n * n;
    const float* h0 = c->half + bht * 2 * n;
    const float* h1 = h0 + n;
    int64_t kn = k < N ? k + 1 : k;
    int64_t* slots = (int64_t*)malloc((size_t)kn * sizeof(int64_t));
    float* sc = (float*)malloc((size_t)kn * sizeof(float));

    pkm_topk(h0, h1, n, k, slots, sc);
    /* A4: softmax over the k selected fp32 scores, max-subtracted, in double */
    double mx = (double)sc[0], sum = 0.0;
    double* e = (double*)malloc((size_t)k * sizeof(double));
    for (int64_t i = 0; i < k; ++i) { e[i] = exp((double)sc[i] - mx); sum += e[i]; }
    for (int64_t i = 0; i < k; ++i) {
        c->idx[bht * k + i] = (int32_t)slots[i];
        c->wt[bht * k + i] = (float)(e[i] / sum);
        if (c->score) c->score[bht * k + i] = sc[i];
    }
    if (c->score_next) {
        if (k < N) {
            /* the (k+1)-th slot score may lie outside the k x k grid: rerun with k+1 */
            pkm_topk(h0, h1, n, k + 1, slots, sc);
            c->score_next[bht] = sc[k];
        } else {
            c->score_next[bht] = -INFINITY;
        }
    }
    free(e); free(sc); free(slots);
}

int oracle_select(const float* half, int64_t B, int64_t H, int64_t T, int64_t n,
                  int64_t k, int32_t* idx, float* wt, float* score, float* score_next,
                  int nthreads) {
    if (!half || !idx || !wt) return -1;
    if (B < 0 || H < 0 || T < 0 || n < 1 || k < 1 || k > n * n) return -2;
    sel_ctx c = {half, n, k, idx, wt, score, score_next};
    parallel_for(sel_item, &c, B * H * T, nthreads);
    return 0;
}

/* ------------------------------------------------------------------ */
/* A5-A6 -- sparse gated delta write, then sparse read                 */
/* [SDM §2.4 Eq. (3)-(5); §2.5 Fig. 2 form].                           */
/* ------------------------------------------------------------------ */
typedef struct {
    const int32_t* idx_w; const float* wt_w; int64_t W;
    const int32_t* idx_r; const float* wt_r; int64_t R;
    const float *alpha, *beta, *v;
    float *M, *y;
    int64_t T, N, dv;
    int form;
    uint16_t* Mb;        /* non-NULL: the table is stored in bfloat16 instead of M */
} scan_ctx;

/* Round x to the nearest bfloat16 (8 significant bits, the fp32 exponent
 * range), ties to even; returns its 16 bits. x = m 2^e with 0.5 <= |m| < 1
 * lies where bfloat16 values are 2^(e-8) apart (below the normal range the
 * spacing stays 2^-133). Used only for the bf16-table variant of the scan. */
static uint16_t bf16_round(double x) {
    int e;
    if (x == 0.0) return signbit(x) ? 0x8000u : 0u;
    frexp(x, &e);
    if (e < -125) e = -125;
    double q = ldexp(1.0, e - 8);
    float f = (float)(nearbyint(x / q) * q);   /* exact: at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static double bf16_value(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* element (row, col) of stream s's table, and its update (one rounding to
   the storage type: fp32, or bfloat16 for the bf16-table variant) */
static double tab_get(const scan_ctx* c, int64_t s, int64_t row, int64_t col) {
    int64_t o = (s * c->N + row) * c->dv + col;
    return c->Mb ? bf16_value(c->Mb[o]) : (double)c->M[o];
}
static void tab_put(scan_ctx* c, int64_t s, int64_t row, int64_t col, double x) {
    int64_t o = (s * c->N + row) * c->dv + col;
    if (c->Mb) c->Mb[o] = bf16_round(x);
    else c->M[o] = (float)x;
}

static void scan_item(void* p, int64_t s) {      /* s = b*H + h: one sequence-head */
    scan_ctx* c = (scan_ctx*)p;
    int64_t W = c->W, R = c->R, dv = c->dv;
    double* vhat = (double*)malloc((size_t)dv * sizeof(double));
    for (int64_t t = 0; t < c->T; ++t) {
        int64_t st = s * c->T + t;
        const int32_t* iw = c->idx_w + st * W;
        const float* ww = c->wt_w + st * W;
        const int32_t* ir = c->idx_r + st * R;
        const float* wr = c->wt_r + st * R;
        const float* vt = c->v + st * dv;
        double a = (double)c->alpha[st], b = (double)c->beta[st];

        if (c->form == ORACLE_FIG2) {
            /* shared prediction from the decayed pre-token rows:
               vhat = sum_j k^(j) * alpha * M[j] */
            for (int64_t col = 0; col < dv; ++col) vhat[col] = 0.0;
            for (int64_t j = 0; j < W; ++j)
                for (int64_t col = 0; col < dv; ++col)
                    vhat[col] += (double)ww[j] * (a * tab_get(c, s, iw[j], col));
        }
        /* Eq. (3): decay the selected rows; Eq. (4) or Fig. 2: delta-correct them.
           Unselected rows are not touched at all. */
        for (int64_t j = 0; j < W; ++j) {
            double kw = (double)ww[j];
            for (int64_t col = 0; col < dv; ++col) {
                double mt = a * tab_get(c, s, iw[j], col);
                double pred = (c->form == ORACLE_FIG2) ? vhat[col] : mt;
                tab_put(c, s, iw[j], col, mt + b * kw * ((double)vt[col] - pred));
            }
        }
        /* Eq. (5): weighted read of the R selected rows of the updated table */
        float* yt = c->y + st * dv;
        for (int64_t col = 0; col < dv; ++col) {
            double acc = 0.0;
            for (int64_t j = 0; j < R; ++j)
                acc += (double)wr[j] * tab_get(c, s, ir[j], col);
            yt[col] = (float)acc;
        }
    }
    free(vhat);
}

/* preconditions of the scan: indices in range, write indices of one token
   distinct. 0, or -3 (out of range) / -4 (repeated write index). */
static int check_indices(const int32_t* idx_w, int64_t W, const int32_t* idx_r, int64_t R,
                         int64_t ntok, int64_t N) {
    unsigned char* seen = (unsigned char*)calloc((size_t)N, 1);
    for (int64_t st = 0; st < ntok; ++st) {
        for (int64_t j = 0; j < R; ++j)
            if (idx_r[st * R + j] < 0 || idx_r[st * R + j] >= N) { free(seen); return -3; }
        for (int64_t j = 0; j < W; ++j) {
            int32_t i = idx_w[st * W + j];
            if (i < 0 || i >= N) { free(seen); return -3; }
            if (seen[i]) { free(seen); return -4; }
            seen[i] = 1;
        }
        for (int64_t j = 0; j < W; ++j) seen[idx_w[st * W + j]] = 0;
    }
    free(seen);
    return 0;
}

int oracle_scan(const int32_t* idx_w, const float* wt_w, int64_t W,
                const int32_t* idx_r, const float* wt_r, int64_t R,
                const float* alpha, const float* beta, const float* v,
                float* M, float* y, int64_t B, int64_t H, int64_t T, int64_t N,
                int64_t dv, int form, int nthreads) {
    if (!idx_w || !wt_w || !idx_r || !wt_r || !alpha || !beta || !v || !M || !y) return -1;
    if (B < 0 || H < 0 || T < 0 || N < 1 || dv < 1 || W < 1 || R < 1 || W > N || R > N) return -2;
    if (form != ORACLE_EQ4 && form != ORACLE_FIG2) return -2;
    int rc = check_indices(idx_w, W, idx_r, R, B * H * T, N);
    if (rc) return rc;
    scan_ctx c = {idx_w, wt_w, W, idx_r, wt_r, R, alpha, beta, v, M, y, T, N, dv, form, NULL};
    parallel_for(scan_item, &c, B * H, nthreads);
    return 0;
}

int oracle_scan_bf16(const int32_t* idx_w, const float* wt_w, int64_t W,
                     const int32_t* idx_r, const float* wt_r, int64_t R,
                     const float* alpha, const float* beta, const float* v,
                     uint16_t* Mb, float* y, int64_t B, int64_t H, int64_t T, int64_t N,
                     int64_t dv, int form, int nthreads) {
    if (!idx_w || !wt_w || !idx_r || !wt_r || !alpha || !beta || !v || !Mb || !y) return -1;
    if (B < 0 || H < 0 || T < 0 || N < 1 || dv < 1 || W < 1 || R < 1 || W > N || R > N) return -2;
    if (form != ORACLE_EQ4 && form != ORACLE_FIG2) return -2;
    int rc = check_indices(idx_w, W, idx_r, R, B * H * T, N);
    if (rc) return rc;
    scan_ctx c = {idx_w, wt_w, W, idx_r, wt_r, R, alpha, beta, v, NULL, y, T, N, dv, form, Mb};
    parallel_for(scan_item, &c, B * H, nthreads);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Backward of A5-A6: reverse-mode derivatives of the scan              */
/* [SDM §2.4 Eq. (3)-(5), §2.5 Fig. 2 form; §2.9 Appendix A: the        */
/*  forward writes in place and the backward walks the tokens in        */
/*  reverse, restoring each written row from its pre-image].            */
/*                                                                      */
/* Per token the forward computes, for write rows i_p with pre-images   */
/* m_p = M_{t-1}[i_p] and read rows j_q:                                */
/*   EQ4:  M_t[i_p] = a m_p + b w_p (v - a m_p)                         */
/*   FIG2: M_t[i_p] = a m_p + b w_p (v - a s),  s = sum_p w_p m_p       */
/*   y_t = sum_q r_q M_t[j_q]                                           */
/* With G = dL/dM_t (the adjoint table), token t in reverse order:      */
/*   reads:  dr_q = <dy_t, M_t[j_q]>;  G[j_q] += r_q dy_t                */
/*   writes, with g_p = G[i_p] (after the reads), u = v - a m_p (EQ4)   */
/*   or u = v - a s (FIG2), gh = sum_p w_p g_p:                          */
/*   EQ4:  dv += b w_p g_p;  da += (1 - b w_p) <g_p, m_p>;              */
/*         db += w_p <g_p, u>;  dw_p = b <g_p, u>;                       */
/*         G[i_p] = a (1 - b w_p) g_p                                    */
/*   FIG2: dv = b gh;  da = sum_p <g_p, m_p> - b <gh, s>;  db = <gh, u>; */
/*         dw_p = b <g_p, u> - a b <gh, m_p>;  G[i_p] = a g_p - a b w_p gh */
/*   and M[i_p] = m_p (the undo). After token 0, G = dL/dM_0.            */
/* Here the pre-images are recorded by running the forward first (same  */
/* arithmetic as oracle_scan); G and every sum are kept in double and    */
/* the outputs rounded once to fp32.                                     */
/* ------------------------------------------------------------------ */
typedef struct {
    const int32_t* idx_w; const float* wt_w; int64_t W;
    const int32_t* idx_r; const float* wt_r; int64_t R;
    const float *alpha, *beta, *v, *M_in, *dy, *dM_out;
    float *dv_, *dalpha, *dbeta, *dwt_w, *dwt_r, *dM_in;
    int64_t T, N, dv;
    int form;
} bwd_ctx;

static void bwd_item(void* p, int64_t s) {      /* s = b*H + h: one sequence-head */
    bwd_ctx* c = (bwd_ctx*)p;
    const int64_t W = c->W, R = c->R, dv = c->dv, T = c->T, N = c->N;
    float* Ms = (float*)malloc((size_t)(N * dv) * sizeof(float));
    float* pre = (float*)malloc((size_t)(T * W * dv + 1) * sizeof(float));
    float* yscr = (float*)malloc((size_t)(T * dv + 1) * sizeof(float));
    double* G = (double*)malloc((size_t)(N * dv) * sizeof(double));
    double* g = (double*)malloc((size_t)(W * dv) * sizeof(double));
    double* gh = (double*)malloc((size_t)dv * sizeof(double));
    double* sm = (double*)malloc((size_t)dv * sizeof(double));
    memcpy(Ms, c->M_in + s * N * dv, (size_t)(N * dv) * sizeof(float));

    /* forward pass, recording the pre-image of every written row */
    for (int64_t t = 0; t < T; ++t) {
        const int32_t* iw = c->idx_w + (s * T + t) * W;
        for (int64_t p = 0; p < W; ++p)
            memcpy(pre + (t * W + p) * dv, Ms + (int64_t)iw[p] * dv, (size_t)dv * sizeof(float));
        scan_ctx f = {c->idx_w + (s * T + t) * W, c->wt_w + (s * T + t) * W, W,
                      c->idx_r + (s * T + t) * R, c->wt_r + (s * T + t) * R, R,
                      c->alpha + s * T + t, c->beta + s * T + t, c->v + (s * T + t) * dv,
                      Ms, yscr + t * dv, 1, N, dv, c->form};
        scan_item(&f, 0);
    }

    for (int64_t k = 0; k < N * dv; ++k) G[k] = c->dM_out ? (double)c->dM_out[s * N * dv + k] : 0.0;
    for (int64_t t = T - 1; t >= 0; --t) {
        const int64_t st = s * T + t;
        const int32_t* iw = c->idx_w + st * W;
        const float* ww = c->wt_w + st * W;
        const int32_t* ir = c->idx_r + st * R;
        const float* wr = c->wt_r + st * R;
        const float* vt = c->v + st * dv;
        const float* dyt = c->dy + st * dv;
        const double a = (double)c->alpha[st], b = (double)c->beta[st];

        /* Eq. (5) read of M_t: weight gradients, then the read's adjoint */
        for (int64_t q = 0; q < R; ++q) {
            const float* row = Ms + (int64_t)ir[q] * dv;
            double acc = 0.0;
            for (int64_t col = 0; col < dv; ++col) acc += (double)dyt[col] * (double)row[col];
            c->dwt_r[st * R + q] = (float)acc;
        }
        for (int64_t q = 0; q < R; ++q) {
            double* Gr = G + (int64_t)ir[q] * dv;
            for (int64_t col = 0; col < dv; ++col) Gr[col] += (double)wr[q] * (double)dyt[col];
        }

        /* the write's adjoint, from the pre-images m_p */
        for (int64_t p = 0; p < W; ++p)
            memcpy(g + p * dv, G + (int64_t)iw[p] * dv, (size_t)dv * sizeof(double));
        double da = 0.0, db = 0.0;
        if (c->form == ORACLE_FIG2) {
            for (int64_t col = 0; col < dv; ++col) { gh[col] = 0.0; sm[col] = 0.0; }
            for (int64_t p = 0; p < W; ++p) {
                const float* m = pre + (t * W + p) * dv;
                for (int64_t col = 0; col < dv; ++col) {
                    gh[col] += (double)ww[p] * g[p * dv + col];
                    sm[col] += (double)ww[p] * (double)m[col];
                }
            }
            double ghs = 0.0;
            for (int64_t col = 0; col < dv; ++col) {
                const double u = (double)vt[col] - a * sm[col];
                c->dv_[st * dv + col] = (float)(b * gh[col]);
                db += gh[col] * u;
                ghs += gh[col] * sm[col];
            }
            da = -b * ghs;
            for (int64_t p = 0; p < W; ++p) {
                const float* m = pre + (t * W + p) * dv;
                double gm = 0.0, gu = 0.0, hm = 0.0;
                for (int64_t col = 0; col < dv; ++col) {
                    const double u = (double)vt[col] - a * sm[col];
                    gm += g[p * dv + col] * (double)m[col];
                    gu += g[p * dv + col] * u;
                    hm += gh[col] * (double)m[col];
                }
                da += gm;
                c->dwt_w[st * W + p] = (float)(b * gu - a * b * hm);
                double* Gw = G + (int64_t)iw[p] * dv;
                for (int64_t col = 0; col < dv; ++col)
                    Gw[col] = a * g[p * dv + col] - a * b * (double)ww[p] * gh[col];
            }
        } else {
            for (int64_t col = 0; col < dv; ++col) gh[col] = 0.0;   /* dv accumulator */
            for (int64_t p = 0; p < W; ++p) {
                const float* m = pre + (t * W + p) * dv;
                const double kw = (double)ww[p];
                double gm = 0.0, gu = 0.0;
                for (int64_t col = 0; col < dv; ++col) {
                    const double gc = g[p * dv + col];
                    gm += gc * (double)m[col];
                    gu += gc * ((double)vt[col] - a * (double)m[col]);
                    gh[col] += b * kw * gc;
                }
                da += (1.0 - b * kw) * gm;
                db += kw * gu;
                c->dwt_w[st * W + p] = (float)(b * gu);
                double* Gw = G + (int64_t)iw[p] * dv;
                for (int64_t col = 0; col < dv; ++col) Gw[col] = a * (1.0 - b * kw) * g[p * dv + col];
            }
            for (int64_t col = 0; col < dv; ++col) c->dv_[st * dv + col] = (float)gh[col];
        }
        c->dalpha[st] = (float)da;
        c->dbeta[st] = (float)db;
        /* the undo: rows of token t back to their pre-images (M_{t-1}) */
        for (int64_t p = 0; p < W; ++p)
            memcpy(Ms + (int64_t)iw[p] * dv, pre + (t * W + p) * dv, (size_t)dv * sizeof(float));
    }
    for (int64_t k = 0; k < N * dv; ++k) c->dM_in[s * N * dv + k] = (float)G[k];
    free(Ms); free(pre); free(yscr); free(G); free(g); free(gh); free(sm);
}

int oracle_scan_backward(const int32_t* idx_w, const float* wt_w, int64_t W,
                         const int32_t* idx_r, const float* wt_r, int64_t R,
                         const float* alpha, const float* beta, const float* v,
                         const float* M_in, const float* dy, const float* dM_out,
                         float* dv_, float* dalpha, float* dbeta, float* dwt_w, float* dwt_r,
                         float* dM_in, int64_t B, int64_t H, int64_t T, int64_t N, int64_t dv,
                         int form, int nthreads) {
    if (!idx_w || !wt_w || !idx_r || !wt_r || !alpha || !beta || !v || !M_in || !dy ||
        !dv_ || !dalpha || !dbeta || !dwt_w || !dwt_r || !dM_in) return -1;
    if (B < 0 || H < 0 || T < 0 || N < 1 || dv < 1 || W < 1 || R < 1 || W > N || R > N) return -2;
    if (form != ORACLE_EQ4 && form != ORACLE_FIG2) return -2;
    int rc = check_indices(idx_w, W, idx_r, R, B * H * T, N);
    if (rc) return rc;
    bwd_ctx c = {idx_w, wt_w, W, idx_r, wt_r, R, alpha, beta, v, M_in, dy, dM_out,
                 dv_, dalpha, dbeta, dwt_w, dwt_r, dM_in, T, N, dv, form};
    parallel_for(bwd_item, &c, B * H, nthreads);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Glue either side of the scan [SDM §2.4]: the per-head scalar gates   */
/*   alpha_t = exp(-A softplus(W_a x_t + b_dt)),  beta_t = sigma(W_b x_t) */
/* and, after the read, the per-head RMS-Norm with an elementwise       */
/* output gate (reading: o = y / sqrt(mean(y^2) + eps) * gamma *         */
/* sigmoid(g), the gate's activation being the sigmoid FwPKM §2.3 uses). */
/* ------------------------------------------------------------------ */
typedef struct {
    const float *x, *Wa, *Wb, *bdt, *A;
    int64_t T, d, H;
    float *alpha, *beta;
} gates_ctx;

static double softplus(double z) {    /* log(1 + e^z), without overflow for large z */
    return z > 0.0 ? z + log1p(exp(-z)) : log1p(exp(z));
}

static void gates_item(void* p, int64_t bt) {   /* bt = b*T + t: one token, all heads */
    gates_ctx* c = (gates_ctx*)p;
    int64_t b = bt / c->T, t = bt % c->T;
    const float* xt = c->x + bt * c->d;
    for (int64_t h = 0; h < c->H; ++h) {
        double za = 0.0, zb = 0.0;
        for (int64_t i = 0; i < c->d; ++i) {
            za += (double)c->Wa[h * c->d + i] * (double)xt[i];
            zb += (double)c->Wb[h * c->d + i] * (double)xt[i];
        }
        za += (double)c->bdt[h];
        int64_t o = (b * c->H + h) * c->T + t;    /* [B, H, T] */
        c->alpha[o] = (float)exp(-(double)c->A[h] * softplus(za));
        c->beta[o] = (float)(1.0 / (1.0 + exp(-zb)));
    }
}

int oracle_gates(const float* x, const float* W_a, const float* W_b, const float* b_dt,
                 const float* A, int64_t B, int64_t T, int64_t d, int64_t H,
                 float* alpha, float* beta, int nthreads) {
    if (!x || !W_a || !W_b || !b_dt || !A || !alpha || !beta) return -1;
    if (B < 0 || T < 0 || d < 1 || H < 1) return -2;
    gates_ctx c = {x, W_a, W_b, b_dt, A, T, d, H, alpha, beta};
    parallel_for(gates_item, &c, B * T, nthreads);
    return 0;
}

typedef struct {
    const float *y, *gamma, *g;
    double eps;
    int64_t H, T, dv;
    float* o;
} outg_ctx;

static void outg_item(void* p, int64_t bht) {   /* one (b, h, t) row of d_v values */
    outg_ctx* c = (outg_ctx*)p;
    int64_t h = (bht / c->T) % c->H;
    const float* yr = c->y + bht * c->dv;
    const float* gr = c->g + bht * c->dv;
    double ss = 0.0;
    for (int64_t i = 0; i < c->dv; ++i) ss += (double)yr[i] * (double)yr[i];
    double r = 1.0 / sqrt(ss / (double)c->dv + c->eps);
    for (int64_t i = 0; i < c->dv; ++i) {
        double gate = 1.0 / (1.0 + exp(-(double)gr[i]));
        c->o[bht * c->dv + i] = (float)((double)yr[i] * r * (double)c->gamma[h * c->dv + i] * gate);
    }
}

int oracle_output_gate(const float* y, const float* gamma, const float* g, double eps,
                       int64_t B, int64_t H, int64_t T, int64_t dv, float* o, int nthreads) {
    if (!y || !gamma || !g || !o) return -1;
    if (B < 0 || H < 1 || T < 0 || dv < 1 || !(eps >= 0.0)) return -2;
    outg_ctx c = {y, gamma, g, eps, H, T, dv, o};
    parallel_for(outg_item, &c, B * H * T, nthreads);
    return 0;
}
