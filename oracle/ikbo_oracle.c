/*
 * ikbo_oracle.c -- fp64 CPU oracle of the IKBO hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use this code. It shares nothing with the GPU library: no headers, helpers, tables or
 * kernels. It is deliberately plain and slow: every request-side tensor is copied out once per
 * candidate (the materialised request-to-candidate broadcast that the GPU path avoids), and
 * every product is a plain loop in double precision.
 *
 * Sources (the ROCS paper, arXiv 2607.27744, as read through the paper-archivist reading notes):
 *  - GLM invariant and two-group form: Sec. 3.1.1, Eq. 1-3 (mask M_ij = 1{j <= i}).
 *  - Grouped affine layer: Sec. 3.1.2, Eq. 4; the two-group block matrix with the
 *    request<-candidate block fixed to zero: Eq. 6.
 *  - Pointwise ops per group (the activation): Sec. 3.1.3, Eq. 8.
 *  - Composition of GLM layers (the MLP): Sec. 3.1.5, Eq. 11; queries from an MLP: Eq. 12.
 *  - Candidate-side cross attention over the shared request sequence: Sec. 3.2, Eq. 13 (A^C);
 *    K/V kept at the request batch and selected through the index map m: Sec. 4.1 and 4.3.1.
 *
 * Conventions (the pages give none; these are the readings used throughout):
 *  - Q and O are [C, Lq, H, d]; K and V are [R, L, H, d] (uniform length) or [sum L_r, H, d]
 *    with prefix offsets kv_cu [R+1] (variable length); weights are [N_out, K_in] (y = W x).
 *  - The request of candidate c is the r with off[r] <= c < off[r+1] when the offsets are given
 *    (they are the contiguous grouping of Sec. 4.2.1), else m[c]. When both are given they must
 *    agree; a candidate whose m[c] names another request is counted as a violation and still
 *    takes its request from the offsets. A candidate with no request in [0, R) gives an
 *    all-zero output row and is counted as a violation.
 *  - Softmax is over all L_r keys of the candidate's request; no masking.
 *  - GELU is the exact erf form x * Phi(x), using libm erf.
 * Parity status of each function is stated in its comment; pins live in the tests.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_F64 = 2 };
enum { OR_ACT_NONE = 0, OR_ACT_GELU = 1 };
enum { OR_OK = 0, OR_BAD_ARG = -1, OR_NO_MEMORY = -3 };

/* Widen one stored element to double (bf16 is the top half of an IEEE fp32). */
static double in_at(const void *p, int dtype, int64_t i) {
    if (dtype == OR_F64) return ((const double *)p)[i];
    if (dtype == OR_F32) return (double)((const float *)p)[i];
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* GELU, exact form: x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)). */
double oracle_gelu(double x) { return 0.5 * x * (1.0 + erf(x / sqrt(2.0))); }

static double act_apply(int act, double x) { return act == OR_ACT_GELU ? oracle_gelu(x) : x; }

/* Request of candidate c from the map m and/or the per-request offsets. The offsets, when given,
 * decide (the candidates of a request are stored contiguously, Sec. 4.2.1); m, when also given,
 * must agree with them, and *disagree (may be NULL) is set to 1 when it does not.
 * Returns the request index, or -1 when the candidate has no valid request. */
int64_t oracle_request_of(const int32_t *m, const int32_t *off, int64_t R, int64_t c, int *disagree) {
    int64_t from_m = -1, from_off = -1;
    if (m) {
        from_m = m[c];
        if (from_m < 0 || from_m >= R) from_m = -1;
    }
    if (off) {
        for (int64_t r = 0; r < R; ++r)
            if (off[r] <= c && c < off[r + 1]) { from_off = r; break; }
    }
    if (disagree) *disagree = m && off && from_m != from_off;
    return off ? from_off : from_m;
}

/* ------------------------------------------------------------------------------------------ */
/* Thread pool helper: run fn(ctx, i) for i in [0, n) over nthreads threads, contiguous chunks. */

typedef void (*item_fn)(void *ctx, int64_t i, void *scratch);

typedef struct {
    item_fn fn;
    void *ctx;
    int64_t lo, hi;
    size_t scratch_bytes;
    int failed;
} span_t;

static void *run_span(void *arg) {
    span_t *s = (span_t *)arg;
    void *scratch = s->scratch_bytes ? malloc(s->scratch_bytes) : 0;
    if (s->scratch_bytes && !scratch) { s->failed = 1; return 0; }
    for (int64_t i = s->lo; i < s->hi; ++i) s->fn(s->ctx, i, scratch);
    free(scratch);
    return 0;
}

static int parallel_for(int64_t n, int nthreads, size_t scratch_bytes, item_fn fn, void *ctx) {
    if (n <= 0) return OR_OK;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > n) nthreads = (int)n;
    pthread_t th[256];
    int created[256];
    span_t sp[256];
    int64_t chunk = (n + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        sp[t].fn = fn;
        sp[t].ctx = ctx;
        sp[t].scratch_bytes = scratch_bytes;
        sp[t].failed = 0;
        sp[t].lo = t * chunk < n ? t * chunk : n;
        sp[t].hi = (t + 1) * chunk < n ? (t + 1) * chunk : n;
        created[t] = 0;
        if (sp[t].lo >= sp[t].hi) continue;
        if (nthreads > 1 && pthread_create(&th[t], 0, run_span, &sp[t]) == 0) created[t] = 1;
        else run_span(&sp[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (created[t]) pthread_join(th[t], 0);
    for (int t = 0; t < nthreads; ++t)
        if (sp[t].failed) return OR_NO_MEMORY;
    return OR_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* IKBO-DCA: candidate cross attention A^C = Attn(Q^C, K_{m(c)}, V_{m(c)}), Eq. 13 with the
 * request-batched K/V selected by m (Sec. 4.3.1). Parity: pinned in the tests (single key,
 * Q = 0 mean, key-shift and value-affine invariances, per-request library attention). */

typedef struct {
    const void *q, *k, *v;
    int dtype, qdtype;
    int64_t C, R;
    int Lq, H, d, L;
    const int32_t *kv_cu, *m, *off;
    double scale;
    const int64_t *cands;
    double *out;
    int64_t *viol;      /* per-item violation flag */
} dca_ctx;

static void dca_item(void *vctx, int64_t i, void *scratch) {
    dca_ctx *x = (dca_ctx *)vctx;
    int64_t c = x->cands ? x->cands[i] : i;
    const int H = x->H, d = x->d, Lq = x->Lq;
    double *o = x->out + i * (int64_t)Lq * H * d;
    memset(o, 0, sizeof(double) * (size_t)Lq * H * d);
    x->viol[i] = 0;
    if (c < 0 || c >= x->C) { x->viol[i] = 1; return; }
    int disagree = 0;
    int64_t r = oracle_request_of(x->m, x->off, x->R, c, &disagree);
    if (r < 0 || disagree) x->viol[i] = 1;
    if (r < 0) return;
    int64_t base = x->kv_cu ? x->kv_cu[r] : r * (int64_t)x->L;
    int64_t Lr = x->kv_cu ? (int64_t)x->kv_cu[r + 1] - x->kv_cu[r] : x->L;
    if (Lr <= 0) return;

    /* The explicit broadcast: this candidate's own copy of its request's K and V. */
    double *Kc = (double *)scratch;
    double *Vc = Kc + (size_t)x->L * H * d;
    double *s = Vc + (size_t)x->L * H * d;
    for (int64_t j = 0; j < Lr; ++j)
        for (int h = 0; h < H; ++h)
            for (int e = 0; e < d; ++e) {
                int64_t src = ((base + j) * H + h) * (int64_t)d + e;
                Kc[(j * H + h) * d + e] = in_at(x->k, x->dtype, src);
                Vc[(j * H + h) * d + e] = in_at(x->v, x->dtype, src);
            }

    for (int t = 0; t < Lq; ++t)
        for (int h = 0; h < H; ++h) {
            int64_t qrow = ((c * Lq + t) * (int64_t)H + h) * d;
            /* scores s_j = scale * <q, k_j> */
            for (int64_t j = 0; j < Lr; ++j) {
                double acc = 0.0;
                for (int e = 0; e < d; ++e) acc += in_at(x->q, x->qdtype, qrow + e) * Kc[(j * H + h) * d + e];
                s[j] = x->scale * acc;
            }
            /* softmax over the keys, two passes: max, then exp and sum */
            double mu = s[0];
            for (int64_t j = 1; j < Lr; ++j) mu = s[j] > mu ? s[j] : mu;
            double l = 0.0;
            for (int64_t j = 0; j < Lr; ++j) { s[j] = exp(s[j] - mu); l += s[j]; }
            /* o = sum_j p_j v_j / l */
            double *orow = o + ((int64_t)t * H + h) * d;
            for (int e = 0; e < d; ++e) {
                double acc = 0.0;
                for (int64_t j = 0; j < Lr; ++j) acc += s[j] * Vc[(j * H + h) * d + e];
                orow[e] = acc / l;
            }
        }
}

/* out: [n, Lq, H, d] fp64 for the candidates cands[0..n) (or all C when cands is NULL).
 * kv_cu: [R+1] prefix offsets of variable K/V lengths, or NULL for uniform length L.
 * L: the uniform length, or the largest L_r when kv_cu is given (sizes the expansion buffer).
 * dtype: storage of k and v; qdtype: storage of q (fp64 lets a chained oracle stay in fp64).
 * Returns OR_OK, or a negative code; *violations counts candidates with no valid request or with a
 * map entry that disagrees with the offsets. */
int oracle_dca(const void *q, int64_t C, int Lq, const void *k, const void *v, int64_t R,
               const int32_t *kv_cu, int L, const int32_t *m, const int32_t *off, int H, int d,
               double scale, int dtype, int qdtype, const int64_t *cands, int64_t n, double *out,
               int64_t *violations, int nthreads) {
    if (!q || !k || !v || !out || (!m && !off) || C < 0 || R < 0 || Lq <= 0 || H <= 0 || d <= 0 || L < 0)
        return OR_BAD_ARG;
    if (dtype != OR_F32 && dtype != OR_BF16 && dtype != OR_F64) return OR_BAD_ARG;
    if (qdtype != OR_F32 && qdtype != OR_BF16 && qdtype != OR_F64) return OR_BAD_ARG;
    if (!cands) n = C;
    if (kv_cu)
        for (int64_t r = 0; r < R; ++r)
            if (kv_cu[r + 1] - kv_cu[r] > L) return OR_BAD_ARG;
    dca_ctx x = {q, k, v, dtype, qdtype, C, R, Lq, H, d, L, kv_cu, m, off, scale, cands, out, 0};
    x.viol = (int64_t *)calloc((size_t)(n > 0 ? n : 1), sizeof(int64_t));
    if (!x.viol) return OR_NO_MEMORY;
    size_t scratch = sizeof(double) * ((size_t)2 * (L > 0 ? L : 1) * H * d + (L > 0 ? L : 1));
    int rc = parallel_for(n, nthreads, scratch, dca_item, &x);
    int64_t nv = 0;
    for (int64_t i = 0; i < n; ++i) nv += x.viol[i];
    if (violations) *violations = nv;
    free(x.viol);
    return rc;
}

/* ------------------------------------------------------------------------------------------ */
/* GLM layers. One layer maps u = [u^R; u^C] (K_r + K_c) to phi(W~ u + [b_r; b_c]) (N_r + N_c),
 * with W~ = [[W_RR, 0], [W_CR, W_CC]] built as a full dense matrix whose upper-right block is
 * an explicit zero (Eq. 4 with the mask of Eq. 3, written as Eq. 6). */

typedef struct {
    const void *w_rr, *w_cr, *w_cc;   /* [N_r,K_r], [N_c,K_r], [N_c,K_c] in the run dtype */
    const float *b_r, *b_c;           /* [N_r], [N_c] fp32, or NULL for zero */
    int32_t k_req, k_cand, n_req, n_cand, act;
} oracle_layer;

typedef struct {
    int rows, cols;     /* (N_r + N_c) x (K_r + K_c) */
    double *w;          /* dense masked weight, row-major */
    double *b;          /* [rows] */
    int act;
    int n_req;
} dense_layer;

static int build_dense(const oracle_layer *ly, int dtype, dense_layer *D) {
    int Kr = ly->k_req, Kc = ly->k_cand, Nr = ly->n_req, Nc = ly->n_cand;
    D->rows = Nr + Nc;
    D->cols = Kr + Kc;
    D->act = ly->act;
    D->n_req = Nr;
    D->w = (double *)calloc((size_t)D->rows * D->cols + 1, sizeof(double));
    D->b = (double *)calloc((size_t)D->rows + 1, sizeof(double));
    if (!D->w || !D->b) { free(D->w); free(D->b); return OR_NO_MEMORY; }
    for (int i = 0; i < D->rows; ++i)
        for (int j = 0; j < D->cols; ++j) {
            int out_req = i < Nr, in_req = j < Kr;
            double mask = (in_req || !out_req) ? 1.0 : 0.0;   /* M_ij = 1{input group <= output group} */
            double w = 0.0;
            if (out_req && in_req) w = in_at(ly->w_rr, dtype, (int64_t)i * Kr + j);
            else if (!out_req && in_req) w = in_at(ly->w_cr, dtype, (int64_t)(i - Nr) * Kr + j);
            else if (!out_req && !in_req) w = in_at(ly->w_cc, dtype, (int64_t)(i - Nr) * Kc + (j - Kr));
            D->w[(size_t)i * D->cols + j] = mask * w;
        }
    for (int i = 0; i < Nr; ++i) D->b[i] = ly->b_r ? (double)ly->b_r[i] : 0.0;
    for (int i = 0; i < Nc; ++i) D->b[Nr + i] = ly->b_c ? (double)ly->b_c[i] : 0.0;
    return OR_OK;
}

/* y = phi(W~ u + b), the full dense product including the zero block. */
static void dense_apply(const dense_layer *D, const double *u, double *y) {
    for (int i = 0; i < D->rows; ++i) {
        const double *wr = D->w + (size_t)i * D->cols;
        double acc = 0.0;
        for (int j = 0; j < D->cols; ++j) acc += wr[j] * u[j];
        y[i] = act_apply(D->act, acc + D->b[i]);
    }
}

typedef struct {
    const void *x_r, *x_c;
    int dtype;
    int64_t R, C;
    const int32_t *m, *off;
    int nlayers;
    const dense_layer *L;
    int k_req0, k_cand0, width_max;
    const int64_t *cands;
    double *y_c, *y_r_c;       /* [n, N_c last], [n, N_r last] (optional) */
    int64_t *viol;
} glm_ctx;

static void glm_item(void *vctx, int64_t i, void *scratch) {
    glm_ctx *x = (glm_ctx *)vctx;
    int64_t c = x->cands ? x->cands[i] : i;
    const dense_layer *last = &x->L[x->nlayers - 1];
    int nr_last = last->n_req, nc_last = last->rows - last->n_req;
    double *yc = x->y_c + i * (int64_t)nc_last;
    double *yrc = x->y_r_c ? x->y_r_c + i * (int64_t)nr_last : 0;
    memset(yc, 0, sizeof(double) * (size_t)nc_last);
    if (yrc) memset(yrc, 0, sizeof(double) * (size_t)nr_last);
    x->viol[i] = 0;
    if (c < 0 || c >= x->C) { x->viol[i] = 1; return; }
    int disagree = 0;
    int64_t r = oracle_request_of(x->m, x->off, x->R, c, &disagree);
    if (r < 0 || disagree) x->viol[i] = 1;
    if (r < 0) return;
    double *u = (double *)scratch, *y = u + x->width_max;
    /* The explicit broadcast: u_c = [x_r[m(c)]; x_c[c]]. */
    for (int j = 0; j < x->k_req0; ++j) u[j] = in_at(x->x_r, x->dtype, r * x->k_req0 + j);
    for (int j = 0; j < x->k_cand0; ++j) u[x->k_req0 + j] = in_at(x->x_c, x->dtype, c * x->k_cand0 + j);
    for (int l = 0; l < x->nlayers; ++l) {
        dense_apply(&x->L[l], u, y);
        double *t = u; u = y; y = t;
    }
    for (int j = 0; j < nc_last; ++j) yc[j] = u[nr_last + j];
    if (yrc)
        for (int j = 0; j < nr_last; ++j) yrc[j] = u[j];
}

/* The request-batched request path alone: y_r = phi(W_RR x_r + b_r) layer by layer. */
static void glm_request_rows(const void *x_r, int dtype, int64_t R, int nlayers, const oracle_layer *layers,
                             const dense_layer *D, double *y_r, double *u, double *y) {
    for (int64_t r = 0; r < R; ++r) {
        int w = layers[0].k_req;
        for (int j = 0; j < w; ++j) u[j] = in_at(x_r, dtype, r * w + j);
        for (int l = 0; l < nlayers; ++l) {
            int Nr = layers[l].n_req, Kr = layers[l].k_req;
            for (int i = 0; i < Nr; ++i) {
                const double *wr = D[l].w + (size_t)i * D[l].cols;   /* first K_r columns = W_RR */
                double acc = 0.0;
                for (int j = 0; j < Kr; ++j) acc += wr[j] * u[j];
                y[i] = act_apply(layers[l].act, acc + D[l].b[i]);
            }
            double *t = u; u = y; y = t;
        }
        int nr = layers[nlayers - 1].n_req;
        for (int j = 0; j < nr; ++j) y_r[r * nr + j] = u[j];
    }
}

/* GLM stack (one layer = IKBO-LCB's linear form; two layers = the query MLP of Eq. 12).
 * y_c: [n, N_c(last)] for candidates cands[0..n) (all C if NULL).
 * y_r_c: optional [n, N_r(last)], the request-group output seen from each candidate's
 *        expanded input (must not depend on the candidate, Eq. 11).
 * y_r: optional [R, N_r(last)], the request path evaluated once per request.
 * Layer l+1 must take k_req = layer l's n_req and k_cand = layer l's n_cand. */
int oracle_glm(const void *x_r, int64_t R, const void *x_c, int64_t C, const int32_t *m, const int32_t *off,
               int nlayers, const oracle_layer *layers, int dtype, const int64_t *cands, int64_t n,
               double *y_c, double *y_r_c, double *y_r, int64_t *violations, int nthreads) {
    if (nlayers <= 0 || !layers || !y_c || !x_r || !x_c || (!m && !off) || R < 0 || C < 0) return OR_BAD_ARG;
    if (dtype != OR_F32 && dtype != OR_BF16) return OR_BAD_ARG;
    int width_max = 1;
    for (int l = 0; l < nlayers; ++l) {
        const oracle_layer *ly = &layers[l];
        if (ly->k_req < 0 || ly->k_cand < 0 || ly->n_req < 0 || ly->n_cand < 0) return OR_BAD_ARG;
        if (l > 0 && (ly->k_req != layers[l - 1].n_req || ly->k_cand != layers[l - 1].n_cand)) return OR_BAD_ARG;
        int a = ly->k_req + ly->k_cand, b = ly->n_req + ly->n_cand;
        width_max = a > width_max ? a : width_max;
        width_max = b > width_max ? b : width_max;
    }
    dense_layer *D = (dense_layer *)calloc((size_t)nlayers, sizeof(dense_layer));
    if (!D) return OR_NO_MEMORY;
    int rc = OR_OK;
    for (int l = 0; l < nlayers && rc == OR_OK; ++l) rc = build_dense(&layers[l], dtype, &D[l]);
    if (!cands) n = C;
    glm_ctx x = {x_r, x_c, dtype, R, C, m, off, nlayers, D, layers[0].k_req, layers[0].k_cand, width_max,
                 cands, y_c, y_r_c, 0};
    x.viol = (int64_t *)calloc((size_t)(n > 0 ? n : 1), sizeof(int64_t));
    if (!x.viol) rc = OR_NO_MEMORY;
    if (rc == OR_OK) rc = parallel_for(n, nthreads, sizeof(double) * 2 * (size_t)width_max, glm_item, &x);
    if (rc == OR_OK && y_r) {
        double *buf = (double *)malloc(sizeof(double) * 2 * (size_t)width_max);
        if (!buf) rc = OR_NO_MEMORY;
        else glm_request_rows(x_r, dtype, R, nlayers, layers, D, y_r, buf, buf + width_max);
        free(buf);
    }
    int64_t nv = 0;
    if (x.viol)
        for (int64_t i = 0; i < n; ++i) nv += x.viol[i];
    if (violations) *violations = nv;
    for (int l = 0; l < nlayers; ++l) { free(D[l].w); free(D[l].b); }
    free(D);
    free(x.viol);
    return rc;
}

/* Index checks, one count per fault: with offsets, off[0] != 0 and off[R] != C count once each
 * and every decreasing step off[r + 1] < off[r] once; with a map, every candidate whose m is
 * outside [0, R), and with sorted_flag every candidate whose m is below its predecessor's; with
 * both, every candidate with a valid m that does not lie in [off[m], off[m + 1]). */
int64_t oracle_index_violations(const int32_t *m, const int32_t *off, int64_t C, int64_t R, int sorted_flag) {
    int64_t bad = 0;
    if (off) {
        if (off[0] != 0) ++bad;
        if (off[R] != C) ++bad;
        for (int64_t r = 0; r < R; ++r)
            if (off[r + 1] < off[r]) ++bad;
    }
    if (m) {
        for (int64_t c = 0; c < C; ++c) {
            if (m[c] < 0 || m[c] >= R) { ++bad; continue; }
            if (sorted_flag && c > 0 && m[c] < m[c - 1]) ++bad;
            if (off && !(off[m[c]] <= c && c < off[m[c] + 1])) ++bad;
        }
    }
    return bad;
}
