/*
 * ikbo.h -- C ABI of the IKBO hot path for MI355X (gfx950).
 *
 * In-Kernel Broadcast Optimization, from ROCS (Request-Oriented Compute Sharing,
 * arXiv 2607.27744): request-side tensors stay at their natural batch size B_r = num_req,
 * candidate-side tensors at B_c = num_cand, and an index map m in {0..B_r-1}^{B_c} ties each
 * candidate to its request (Sec. 4, opening paragraph; Sec. 4.1). The request-to-candidate
 * broadcast is resolved inside the consuming kernels and is never materialised in memory.
 *
 * Conventions shared by every entry point
 *  - Pointers to tensors are DEVICE pointers unless a comment says "host". Tensors are dense,
 *    row-major and contiguous; base pointers must be 16-byte aligned (IKBO_MISALIGNED).
 *  - Ownership: the caller owns every buffer. The library allocates no device memory and keeps
 *    no pointer after a call returns. Scratch memory comes from the caller's `workspace`, whose
 *    size the matching *_workspace_size() call returns.
 *  - Asynchrony: work is enqueued on `hip_stream` (a hipStream_t; NULL = the default stream).
 *    IKBO_OK means the work was enqueued, not that it finished.
 *  - Errors: a status code is returned, never an exception. The last failure's text is kept per
 *    host thread (ikbo_last_error_message). Argument checks run before any GPU work, so a call
 *    that returns an error other than IKBO_HIP_ERROR has enqueued nothing.
 *  - Index arrays: cand_to_req (the map m of Sec. 4.1, int32 [num_cand]) and/or
 *    req_cand_offsets (int32 [num_req + 1], candidates of request r are rows off[r]..off[r+1]-1).
 *    At least one is required. The pages store the candidates of one request contiguously
 *    (Sec. 4.2.1); a map that is not grouped is accepted too (grouped on the device by a stable
 *    sort: a request's candidates keep their index order). When both are given they must agree,
 *    and in every entry point the offsets then decide each candidate's request: cand_to_req is
 *    not read. Index CONTENTS (range, order, agreement) are a precondition that ikbo_check_index
 *    verifies; kernels stay memory-safe whatever the contents: a candidate with no request in
 *    range (or outside every offset range) gets an all-zero output row.
 *  - Dtypes: inputs IKBO_F32 or IKBO_BF16; outputs IKBO_F32 or IKBO_BF16; accumulation is
 *    always fp32. A bf16-output call returns the round-to-nearest-even bf16 of what the same
 *    call with an fp32 output returns.
 *  - Results are deterministic run to run (no floating-point atomics).
 */
#ifndef IKBO_H
#define IKBO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IKBO_VERSION 100

/* Status codes */
#define IKBO_OK 0
#define IKBO_INVALID_ARGUMENT 1     /* null pointer, negative size, no index array, bad flag */
#define IKBO_UNSUPPORTED 2          /* dtype combination or head_dim not built */
#define IKBO_MISALIGNED 3           /* base pointer or row width breaks 16-byte alignment */
#define IKBO_WORKSPACE_TOO_SMALL 4  /* workspace_bytes below the *_workspace_size() value */
#define IKBO_HIP_ERROR 5            /* a HIP call or kernel launch failed */

/* Dtype codes */
#define IKBO_F32 0
#define IKBO_BF16 1

/* Activations (applied per group, a pointwise GLM op: Sec. 3.1.3, Eq. 8) */
#define IKBO_ACT_NONE 0
#define IKBO_ACT_GELU 1             /* exact form x * Phi(x) = x/2 (1 + erf(x / sqrt 2)) */

/* Group-local normalisations (Sec. 3.1.3, Eq. 7), of each embedding row over its d values */
#define IKBO_NORM_NONE 0
#define IKBO_NORM_LAYER 1           /* (y - mean) / sqrt(var + eps), biased variance; then * gamma + beta */
#define IKBO_NORM_RMS 2             /* y / sqrt(mean(y^2) + eps); then * gamma + beta */

/* index_flags bits */
#define IKBO_INDEX_SORTED 1u        /* cand_to_req is non-decreasing (candidates grouped) */

int ikbo_version(void);
const char *ikbo_status_string(int status);
const char *ikbo_last_error_message(void);

/* ------------------------------------------------------------------------------------------
 * IKBO-DCA: candidate-side cross attention of Deep Cross Attention (Sec. 3.2, Eq. 13, the
 * A^C term), executed as in Sec. 4.3.1: the kernel takes K and V at the request batch size,
 * resolves each candidate's request, and every candidate of a request reads the same physical
 * K/V rows.
 *
 *   out[c, t, h, :] = sum_j softmax_j(scale * <q[c,t,h,:], k[r,j,h,:]>) * v[r, j, h, :],
 *   with r the request of candidate c and j over the L_r keys of request r.
 *
 * q     [num_cand, q_len, num_heads, head_dim]   (in_dtype)
 * k, v  uniform: [num_req, kv_len, num_heads, head_dim]; variable length (kv_cu_seqlens set):
 *       [kv_cu_seqlens[num_req], num_heads, head_dim], request r owning rows
 *       kv_cu_seqlens[r] .. kv_cu_seqlens[r+1]-1                       (in_dtype)
 * kv_cu_seqlens  device int32 [num_req + 1] or NULL (uniform length kv_len)
 * kv_len         uniform K/V length, or with kv_cu_seqlens an upper bound on L_r (0 = unknown)
 * cand_to_req, req_cand_offsets, index_flags   see the conventions above (the offsets, when
 *       given, define the grouping).
 * num_heads      H >= 1 (queries and keys share the head count)
 * head_dim       bf16: 64 or 128; fp32: a multiple of 4 in [4, 128]
 *       bf16 also needs each request's K (and V) rows to span fewer than 2^31 bytes,
 *       L_r * num_heads * head_dim * 2 < 2^31: a larger kv_len is rejected (IKBO_UNSUPPORTED);
 *       with kv_cu_seqlens and kv_len = 0 a longer request yields NaN output rows.
 * softmax_scale  <= 0 selects 1/sqrt(head_dim)
 * out   [num_cand, q_len, num_heads, head_dim] (out_dtype). Rows of a request with L_r = 0 and
 *       rows of candidates with no valid request are written as zeros.
 * workspace      device scratch of at least ikbo_dca_workspace_size(num_cand, num_req) bytes
 *       (may be NULL when that size is 0).
 * Errors: IKBO_INVALID_ARGUMENT, IKBO_UNSUPPORTED, IKBO_MISALIGNED, IKBO_WORKSPACE_TOO_SMALL,
 *         IKBO_HIP_ERROR.
 * ---------------------------------------------------------------------------------------- */
size_t ikbo_dca_workspace_size(int64_t num_cand, int64_t num_req);

int ikbo_dca_forward(const void *q, int64_t num_cand, int32_t q_len,
                     const void *k, const void *v, int64_t num_req,
                     const int32_t *kv_cu_seqlens, int32_t kv_len,
                     const int32_t *cand_to_req, const int32_t *req_cand_offsets, uint32_t index_flags,
                     int32_t num_heads, int32_t head_dim, float softmax_scale,
                     int32_t in_dtype, int32_t out_dtype, void *out,
                     void *workspace, size_t workspace_bytes, void *hip_stream);

/* ------------------------------------------------------------------------------------------
 * IKBO-DCA without allocation, for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, results and errors are those of ikbo_dca_forward (same kernels, same bits); the
 * scratch that call takes from `workspace` comes instead from a fixed array of
 * IKBO_DCA_NOALLOC_SCRATCH_BYTES bytes that the library keeps on every GPU it runs on, from the
 * first call on that GPU until the process ends. The first call on a device looks the array up
 * (hipGetSymbolAddress, on the current device); no call allocates. Uses the current device's
 * array: hip_stream must belong to the current device.
 * Limit: ikbo_dca_workspace_size(num_cand, num_req) must not exceed the array (about 1.5 million
 *        candidates); larger calls return IKBO_WORKSPACE_TOO_SMALL and enqueue nothing.
 * Calls that overlap on one GPU (on different streams, or from different host threads without
 * stream ordering) share that array and race; calls ordered on one stream do not. Every call sets
 * up the parts of the array it reads (counters are cleared by kernels), so no state carries over
 * from a previous call.
 * ---------------------------------------------------------------------------------------- */
#define IKBO_DCA_NOALLOC_SCRATCH_BYTES (32u << 20)

int ikbo_dca_forward_noalloc(const void *q, int64_t num_cand, int32_t q_len,
                             const void *k, const void *v, int64_t num_req,
                             const int32_t *kv_cu_seqlens, int32_t kv_len,
                             const int32_t *cand_to_req, const int32_t *req_cand_offsets, uint32_t index_flags,
                             int32_t num_heads, int32_t head_dim, float softmax_scale,
                             int32_t in_dtype, int32_t out_dtype, void *out, void *hip_stream);

/* ------------------------------------------------------------------------------------------
 * IKBO-LCB: the GLM-masked two-group linear layer (Sec. 3.1.2, Eq. 4 with the mask of Eq. 3,
 * block form Eq. 6), run as the decomposition of Sec. 4.1, Eq. 14:
 *   [y_r ; Z] = [W_RR ; W_CR] x_r          once per request (request batch),
 *   y_c[c]   = act(W_CC x_c[c] + Z[m(c)] + b_c)   with the Z gather-added in the GEMM epilogue
 *                                                  (Sec. 4.2.1),
 *   y_r[r]   = act(W_RR x_r[r] + b_r).
 * The request<-candidate block W_RC of Eq. 6 is zero by construction and is not an argument.
 *
 * x_req  [num_req, k_req], x_cand [num_cand, k_cand]               (in_dtype)
 * w_rr   [n_req_out, k_req], w_cr [n_cand_out, k_req], w_cc [n_cand_out, k_cand]  (in_dtype)
 * b_r    [n_req_out] fp32 or NULL;  b_c [n_cand_out] fp32 or NULL
 * activation  IKBO_ACT_NONE or IKBO_ACT_GELU, applied to both groups
 * y_req  [num_req, n_req_out] (out_dtype) or NULL to skip the request-group output
 * y_cand [num_cand, n_cand_out] (out_dtype)
 * k_req, k_cand, n_req_out, n_cand_out: >= 0, any value. The alignment rule of Sec. 4.2.4 is
 *       applied inside the call: a bf16 K width that is not a multiple of 8 (16-byte rows) is
 *       zero-padded to the next multiple of 8 in workspace copies of the activations and of the
 *       weights that multiply them (the padded columns add nothing to any sum); fp32 widths need
 *       no padding. Base pointers must still be 16-byte aligned.
 * workspace >= ikbo_lcb_workspace_size(num_cand, num_req, k_req, k_cand, n_req_out, n_cand_out,
 *       in_dtype) bytes; it holds the candidate->request map built from the offsets, Z in fp32,
 *       the request GEMM's split-K partial sums and, for misaligned bf16 K widths, the padded copies.
 * Environment: IKBO_LCB_FUSED=1 runs a bf16 layer as one persistent launch in which request and
 *       candidate tiles share the schedule (Sec. 4.2.3: request items claimed ascending, candidate
 *       tiles descending; each candidate epilogue waits on the ready flags of the request tiles
 *       holding its Z columns). Same results bit for bit; two launches are the default, being
 *       faster on MI355X. Each wait is bounded (0.5 s); a wait that runs out writes the tile as NaN.
 *       IKBO_LCB_FUSED_WAIT_NS sets that bound in nanoseconds; a negative value also keeps the
 *       request tiles from setting their flags (a host-forced test of the bounded waits).
 * ---------------------------------------------------------------------------------------- */
size_t ikbo_lcb_workspace_size(int64_t num_cand, int64_t num_req, int32_t k_req, int32_t k_cand,
                               int32_t n_req_out, int32_t n_cand_out, int32_t in_dtype);

int ikbo_lcb_forward(const void *x_req, int64_t num_req, int32_t k_req,
                     const void *x_cand, int64_t num_cand, int32_t k_cand,
                     const int32_t *cand_to_req, const int32_t *req_cand_offsets, uint32_t index_flags,
                     const void *w_rr, const void *w_cr, const void *w_cc,
                     const float *b_r, const float *b_c,
                     int32_t n_req_out, int32_t n_cand_out, int32_t activation,
                     int32_t in_dtype, int32_t out_dtype, void *y_req, void *y_cand,
                     void *workspace, size_t workspace_bytes, void *hip_stream);

/* ------------------------------------------------------------------------------------------
 * GLM-MLP: a stack of GLM linear layers (each an IKBO-LCB), closed under composition
 * (Sec. 3.1.5, Eq. 11), as used to form DCA queries (Sec. 3.2, Eq. 12). Layer l+1 takes
 * layer l's outputs: k_req(l+1) = n_req_out(l), k_cand(l+1) = n_cand_out(l). Hidden
 * activations live in the workspace, in bf16 for bf16 inputs and fp32 for fp32 inputs; the
 * last layer writes y_req / y_cand in out_dtype. Widths may take any value (each layer applies
 * the zero padding rule of ikbo_lcb_forward to its own inputs).
 * `layers` is a HOST array of num_layers descriptors whose pointer members are device
 * pointers.
 * ---------------------------------------------------------------------------------------- */
typedef struct ikbo_glm_layer {
    const void *w_rr;       /* [n_req_out, k_req] */
    const void *w_cr;       /* [n_cand_out, k_req] */
    const void *w_cc;       /* [n_cand_out, k_cand] */
    const float *b_r;       /* [n_req_out] or NULL */
    const float *b_c;       /* [n_cand_out] or NULL */
    int32_t k_req, k_cand, n_req_out, n_cand_out;
    int32_t activation;
} ikbo_glm_layer;

size_t ikbo_glm_mlp_workspace_size(int64_t num_cand, int64_t num_req, int32_t num_layers,
                                   const ikbo_glm_layer *layers, int32_t in_dtype);

int ikbo_glm_mlp_forward(const void *x_req, int64_t num_req, const void *x_cand, int64_t num_cand,
                         const int32_t *cand_to_req, const int32_t *req_cand_offsets, uint32_t index_flags,
                         int32_t num_layers, const ikbo_glm_layer *layers,
                         int32_t in_dtype, int32_t out_dtype, void *y_req, void *y_cand,
                         void *workspace, size_t workspace_bytes, void *hip_stream);

/* ------------------------------------------------------------------------------------------
 * K/V projection at the request batch size. Sec. 4.1 (the DCA decomposition after Eq. 14): a
 * linear K/V projection commutes with the request-to-candidate broadcast, (S_m) W = (S W)_m, so
 * K and V are projected once per request and the candidates of a request share the result.
 *   k_out[i, :] = W_K s[i, :],   v_out[i, :] = W_V s[i, :]   for every sequence row i.
 * s      [rows, d_in]: the request-side sequence rows of all requests stacked ([R * L, d_in] for
 *        a uniform length L, [sum L_r, d_in] for variable lengths)                 (in_dtype)
 * w_k, w_v  [d_out, d_in] (in_dtype): the pages' S W with W of shape [d_in, d_out], stored
 *        transposed like the LCB weights (row n holds the weights of output n).
 * k_out, v_out  [rows, d_out] (out_dtype). With d_out = num_heads * head_dim they are the
 *        [rows, num_heads, head_dim] K / V that ikbo_dca_forward and ikbo_request_attention read.
 * rows, d_in, d_out >= 0; d_in a multiple of 8 (bf16) / 4 (fp32), else IKBO_MISALIGNED.
 * No workspace. Errors: IKBO_INVALID_ARGUMENT, IKBO_UNSUPPORTED, IKBO_MISALIGNED, IKBO_HIP_ERROR.
 * ---------------------------------------------------------------------------------------- */
int ikbo_kv_project(const void *s, int64_t rows, int32_t d_in, const void *w_k, const void *w_v,
                    int32_t d_out, int32_t in_dtype, int32_t out_dtype, void *k_out, void *v_out,
                    void *hip_stream);

/* ------------------------------------------------------------------------------------------
 * Request-side attention A^R of Deep Cross Attention (Sec. 3.2, Eq. 13, the request term): the
 * queries of request r attend the K/V of request r, at the request batch size (no broadcast):
 *   out[r, t, h, :] = sum_j softmax_j(scale * <q_req[r,t,h,:], k[r,j,h,:]>) * v[r, j, h, :].
 * This is ikbo_dca_forward with one candidate per request (the identity map); with few query
 * rows per request that call runs one-wave, 32-row work tiles.
 * q_req  [num_req, q_len, num_heads, head_dim] (in_dtype)
 * k, v, kv_cu_seqlens, kv_len, num_heads, head_dim, softmax_scale, in_dtype, out_dtype: as for
 *        ikbo_dca_forward (the same head_dim and 2^31-byte limits).
 * out    [num_req, q_len, num_heads, head_dim] (out_dtype); a request with L_r = 0 gets zeros.
 * workspace >= ikbo_request_attention_workspace_size(num_req) bytes.
 * Errors: as ikbo_dca_forward.
 * ---------------------------------------------------------------------------------------- */
size_t ikbo_request_attention_workspace_size(int64_t num_req);

int ikbo_request_attention(const void *q_req, int64_t num_req, int32_t q_len, const void *k, const void *v,
                           const int32_t *kv_cu_seqlens, int32_t kv_len, int32_t num_heads, int32_t head_dim,
                           float softmax_scale, int32_t in_dtype, int32_t out_dtype, void *out,
                           void *workspace, size_t workspace_bytes, void *hip_stream);

/* ------------------------------------------------------------------------------------------
 * GLM factorization machine, two groups (Sec. 3.1.4, Eq. 9 with the block mask, two-group form
 * Eq. 10): pairwise inner products of feature embeddings, masked so the request group sees only
 * request features:
 *   y_req[r]  = X^R_r (X^R_r)^T                                    [n_req_feat, n_req_feat]
 *   y_cand[c] = [ X^C_c (X^R_{m(c)})^T ,  X^C_c (X^C_c)^T ]        [n_cand_feat, n_req_feat + n_cand_feat]
 * The request embeddings are read through the candidate->request index inside the kernel
 * (never expanded to the candidate batch).
 * x_req  [num_req, n_req_feat, dim], x_cand [num_cand, n_cand_feat, dim]      (in_dtype)
 * y_req  [num_req, n_req_feat, n_req_feat] (out_dtype) or NULL to skip the request group
 * y_cand [num_cand, n_cand_feat, n_req_feat + n_cand_feat]                   (out_dtype)
 * cand_to_req, req_cand_offsets, index_flags: see the conventions above (offsets, when given,
 *        define each candidate's request); a candidate without a valid request gets zeros.
 * n_req_feat, n_cand_feat: multiples of 4 (else IKBO_UNSUPPORTED); dim >= 1. bf16 with dim in
 *        {32, 64, 128} and both feature counts <= 64 runs on MFMA; other shapes run a plain
 *        fp32-arithmetic kernel.
 * No workspace. Errors: IKBO_INVALID_ARGUMENT, IKBO_UNSUPPORTED, IKBO_MISALIGNED, IKBO_HIP_ERROR.
 * ---------------------------------------------------------------------------------------- */
int ikbo_fm_forward(const void *x_req, int64_t num_req, int32_t n_req_feat,
                    const void *x_cand, int64_t num_cand, int32_t n_cand_feat, int32_t dim,
                    const int32_t *cand_to_req, const int32_t *req_cand_offsets, uint32_t index_flags,
                    int32_t in_dtype, int32_t out_dtype, void *y_req, void *y_cand, void *hip_stream);

/* ------------------------------------------------------------------------------------------
 * One DCA interaction layer (Sec. 3.2: the query generator of Eq. 12, the two attention halves
 * of Eq. 13, and the concatenation of each attention output with its group's GLM
 * representation that feeds the next layer; stacking layers is "Benefiting from Depth"):
 *   [Q^R | Q^C] = GLM-MLP(x_req, x_cand)               (the glm_layers, as ikbo_glm_mlp_forward)
 *   K^C, V^C = S W_K^C, S W_V^C;  K^R, V^R = S W_K^R, S W_V^R   (once per request, as ikbo_kv_project)
 *   A^C = IKBO-DCA(Q^C, K^C, V^C) (as ikbo_dca_forward);  A^R = Attn(Q^R, K^R, V^R) (as
 *         ikbo_request_attention)
 *   y_req = [Q^R | A^R]  [num_req, 2 W],   y_cand = [Q^C | A^C]  [num_cand, 2 W],   W = q_len *
 *         num_heads * head_dim (each row: the W query values viewed [q_len, num_heads, head_dim],
 *         then the W attention outputs in the same layout).
 * The halves are written in place (strided), so the next layer reads y_req / y_cand as its
 * x_req / x_cand with k_req = k_cand = 2 W. S is this layer's request sequence representation
 * (the shared encoder that produces it is request-only and not part of this call).
 * x_req, x_cand, cand_to_req, req_cand_offsets, index_flags, glm_layers: as ikbo_glm_mlp_forward;
 *        the last glm layer must output W columns per group.
 * seq    [seq_rows, seq_dim] (dtype): R * kv_len rows for a uniform length, sum L_r rows with
 *        kv_cu_seqlens (seq_rows must then equal kv_cu_seqlens[num_req]).
 * w_k_cand, w_v_cand, w_k_req, w_v_req  [num_heads * head_dim, seq_dim] (dtype).
 * q_len, num_heads, head_dim, softmax_scale: as ikbo_dca_forward.
 * dtype  IKBO_BF16 or IKBO_F32 for inputs, weights, intermediates and outputs (fp32 accumulation).
 * workspace >= ikbo_dca_layer_workspace_size(...) bytes (the MLP's, two K/V buffers reused by both
 *        halves, and the attention's).
 * Errors: those of the calls above, plus IKBO_INVALID_ARGUMENT for a query generator whose output
 *         width is not W or a seq_rows that does not match.
 * ---------------------------------------------------------------------------------------- */
size_t ikbo_dca_layer_workspace_size(int64_t num_cand, int64_t num_req, int32_t num_glm_layers,
                                     const ikbo_glm_layer *glm_layers, int64_t seq_rows, int32_t num_heads,
                                     int32_t head_dim, int32_t dtype);

int ikbo_dca_layer_forward(const void *x_req, int64_t num_req, const void *x_cand, int64_t num_cand,
                           const int32_t *cand_to_req, const int32_t *req_cand_offsets, uint32_t index_flags,
                           int32_t num_glm_layers, const ikbo_glm_layer *glm_layers,
                           const void *seq, int64_t seq_rows, int32_t seq_dim,
                           const int32_t *kv_cu_seqlens, int32_t kv_len,
                           const void *w_k_cand, const void *w_v_cand, const void *w_k_req, const void *w_v_req,
                           int32_t q_len, int32_t num_heads, int32_t head_dim, float softmax_scale,
                           int32_t dtype, void *y_req, void *y_cand, void *workspace,
                           size_t workspace_bytes, void *hip_stream);

/* ------------------------------------------------------------------------------------------
 * LCB in its embedding-matrix (row-axis) form, two groups (Sec. 3.1.2, Eq. 5 and the block
 * form Eq. 6), each group's output then normalised on its own (Sec. 3.1.3, Eq. 7):
 *   y_req[r]  = Norm_R( W_RR X^R_r )                                   [n_req_out, dim]
 *   y_cand[c] = Norm_C( W_CR X^R_{m(c)} + W_CC X^C_c )                 [n_cand_out, dim]
 * The request-derived term W_CR X^R_r is computed once per request into the workspace (fp32) and
 * added in the candidate kernel through the candidate->request index (never expanded to the
 * candidate batch). Norm acts on each output row (one embedding) over its dim values.
 * x_req  [num_req, n_req_in, dim], x_cand [num_cand, n_cand_in, dim]           (in_dtype)
 * w_rr   [n_req_out, n_req_in], w_cr [n_cand_out, n_req_in], w_cc [n_cand_out, n_cand_in] (in_dtype)
 * norm   IKBO_NORM_NONE | IKBO_NORM_LAYER | IKBO_NORM_RMS; eps >= 0 (added to the variance or the
 *        mean square; 0 gives inf/NaN on a constant or zero row, as the formula does).
 * gamma_req, beta_req, gamma_cand, beta_cand: fp32 [dim] or NULL (gamma 1, beta 0); used only
 *        when norm is not IKBO_NORM_NONE.
 * y_req  [num_req, n_req_out, dim] (out_dtype) or NULL to skip the request group
 * y_cand [num_cand, n_cand_out, dim] (out_dtype); a candidate without a valid request gets zeros.
 * cand_to_req, req_cand_offsets, index_flags: see the conventions above.
 * n_req_in, n_cand_in >= 1; 1 <= dim <= 256. bf16 with dim in {32, 64, 128} and n_cand_in,
 *        n_cand_out <= 64 runs the candidates on MFMA; other shapes run plain fp32-arithmetic
 *        kernels. The request group always runs the plain kernel (num_req rows only).
 * workspace >= ikbo_lcb_emb_workspace_size(num_req, n_cand_out, dim) bytes when the candidate
 *        group is computed (num_cand > 0 and n_cand_out > 0), else unused.
 * Errors: IKBO_INVALID_ARGUMENT, IKBO_UNSUPPORTED, IKBO_MISALIGNED, IKBO_WORKSPACE_TOO_SMALL,
 *         IKBO_HIP_ERROR.
 * ---------------------------------------------------------------------------------------- */
size_t ikbo_lcb_emb_workspace_size(int64_t num_req, int32_t n_cand_out, int32_t dim);

int ikbo_lcb_emb_forward(const void *x_req, int64_t num_req, int32_t n_req_in,
                         const void *x_cand, int64_t num_cand, int32_t n_cand_in, int32_t dim,
                         const void *w_rr, int32_t n_req_out, const void *w_cr, const void *w_cc,
                         int32_t n_cand_out, const int32_t *cand_to_req, const int32_t *req_cand_offsets,
                         uint32_t index_flags, int32_t norm, const float *gamma_req, const float *beta_req,
                         const float *gamma_cand, const float *beta_cand, float eps, int32_t in_dtype,
                         int32_t out_dtype, void *y_req, void *y_cand, void *workspace,
                         size_t workspace_bytes, void *hip_stream);

/* ------------------------------------------------------------------------------------------
 * Index check (the map m of Sec. 4.1, the contiguous grouping of Sec. 4.2.1): counts, on the
 * device, one violation per fault:
 *   (a) each candidate whose cand_to_req is outside [0, num_req);
 *   (b) with IKBO_INDEX_SORTED, each candidate whose map value is below the previous candidate's;
 *   (c) when both arrays are given, each candidate with a valid map value that does not lie in
 *       [off[m(c)], off[m(c)+1]) (the two forms disagree);
 *   (d) with offsets, off[0] != 0 and off[num_req] != num_cand (one each) and every decreasing
 *       step off[r+1] < off[r].
 * Either index array may be NULL (not both when num_cand > 0). d_violations: device uint64 [1],
 * 8-byte aligned, overwritten with the count (0 = valid) in stream order; the caller reads it
 * after the stream synchronises. Errors: IKBO_INVALID_ARGUMENT, IKBO_MISALIGNED, IKBO_HIP_ERROR.
 * ---------------------------------------------------------------------------------------- */
int ikbo_check_index(const int32_t *cand_to_req, const int32_t *req_cand_offsets,
                     int64_t num_cand, int64_t num_req, uint32_t index_flags,
                     uint64_t *d_violations, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* IKBO_H */
