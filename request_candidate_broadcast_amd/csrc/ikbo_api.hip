// The C ABI of libikbo (declared in include/ikbo.h): argument checks, workspace carving and
// kernel launches on the caller's stream. No device memory is allocated here.
#include "ikbo.h"
#include "ikbo_launch.h"

#include <stdlib.h>

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <mutex>
#include <string>

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return IKBO_OK;
}

int hip_fail(hipError_t e, const char *where) {
    return fail(IKBO_HIP_ERROR, "%s: %s", where, hipGetErrorString(e));
}

#define IKBO_HIP(call)                                   \
    do {                                                 \
        hipError_t e_ = (call);                          \
        if (e_ != hipSuccess) return hip_fail(e_, #call); \
    } while (0)

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool dtype_ok(int32_t d) { return d == IKBO_F32 || d == IKBO_BF16; }

size_t esize(int32_t d) { return d == IKBO_F32 ? 4 : 2; }

// Sequential carve-out of a caller workspace.
struct Carver {
    char *base;
    size_t used = 0;
    explicit Carver(void *b) : base((char *)b) {}
    void *take(size_t bytes) {
        void *p = base ? base + used : nullptr;
        used += align256(bytes);
        return p;
    }
};

// ---- DCA ----------------------------------------------------------------------------------------
// counts [R+1], off [R+1], tiles [R+1], perm [C], then the stable grouping's scratch (used only
// when the map is given without offsets)
size_t dca_ws(int64_t C, int64_t R, Carver *c, int32_t **counts, int32_t **off, int32_t **tiles, int32_t **perm,
              int32_t **sort_scratch = nullptr) {
    Carver local(nullptr);
    Carver &cv = c ? *c : local;
    int32_t *a = (int32_t *)cv.take(sizeof(int32_t) * (size_t)(R + 1));
    int32_t *b = (int32_t *)cv.take(sizeof(int32_t) * (size_t)(R + 1));
    int32_t *t = (int32_t *)cv.take(sizeof(int32_t) * (size_t)(R + 1));
    int32_t *p = (int32_t *)cv.take(sizeof(int32_t) * (size_t)(C > 0 ? C : 1));
    int32_t *g = (int32_t *)cv.take(sizeof(int32_t) * (size_t)ikbo::stable_group_scratch_ints(C > 0 ? C : 1));
    if (counts) *counts = a;
    if (off) *off = b;
    if (tiles) *tiles = t;
    if (perm) *perm = p;
    if (sort_scratch) *sort_scratch = g;
    return cv.used;
}

// ---- LCB ----------------------------------------------------------------------------------------
int32_t lcb_splits(int64_t R, int32_t n_total, int32_t k_req, int32_t in_dtype) {
    return ikbo::request_gemm_splits(R, n_total, k_req, in_dtype == IKBO_F32);
}

// an environment switch that is on when set to a value starting with '1'
bool getenv_flag(const char *name) {
    const char *v = getenv(name);
    return v && v[0] == '1';
}

// Alignment rule (Sec. 4.2.4): a bf16 K width that is not a multiple of 8 elements (16-byte rows)
// is zero-padded to the next multiple of 8, in copies of the activations and of the weights that
// multiply them, so the GEMMs run on whole 16-byte rows; the padded columns multiply zeros and
// change no sum. Bytes of each padded copy one LCB layer needs (0 when its width is aligned).
int64_t round_up8(int64_t k) { return (k + 7) / 8 * 8; }

struct PadSizes {
    size_t xr = 0, wrr = 0, wcr = 0, xc = 0, wcc = 0;
    void take_max(const PadSizes &o) {
        xr = xr > o.xr ? xr : o.xr;
        wrr = wrr > o.wrr ? wrr : o.wrr;
        wcr = wcr > o.wcr ? wcr : o.wcr;
        xc = xc > o.xc ? xc : o.xc;
        wcc = wcc > o.wcc ? wcc : o.wcc;
    }
};

PadSizes lcb_pad_sizes(int64_t C, int64_t R, int32_t k_req, int32_t k_cand, int32_t n_req, int32_t n_cand,
                       int32_t in_dtype) {
    PadSizes p;
    if (in_dtype != IKBO_BF16) return p;      // the fp32 kernel reads elements one by one
    if (k_req % 8) {
        const size_t kp = (size_t)round_up8(k_req) * 2;
        p.xr = kp * (size_t)R;
        p.wrr = kp * (size_t)n_req;
        p.wcr = kp * (size_t)n_cand;
    }
    if (k_cand % 8) {
        const size_t kp = (size_t)round_up8(k_cand) * 2;
        p.xc = kp * (size_t)C;
        p.wcc = kp * (size_t)n_cand;
    }
    return p;
}

struct LcbWs {
    int32_t *map = nullptr;
    float *z = nullptr;
    float *partial = nullptr;
    size_t partial_cap = 0;   // floats
    int32_t *sync = nullptr;  // state of the persistent LCB launch
    int64_t sync_cap = 0;     // int32 words
    // zero-padded copies for misaligned K widths (see lcb_pad_sizes), each at least its size
    void *pad_xr = nullptr, *pad_wrr = nullptr, *pad_wcr = nullptr, *pad_xc = nullptr, *pad_wcc = nullptr;
};

void carve_pads(Carver &cv, const PadSizes &p, LcbWs *w) {
    void *a = cv.take(p.xr), *b = cv.take(p.wrr), *c = cv.take(p.wcr), *d = cv.take(p.xc), *e = cv.take(p.wcc);
    if (w) {
        w->pad_xr = a;
        w->pad_wrr = b;
        w->pad_wcr = c;
        w->pad_xc = d;
        w->pad_wcc = e;
    }
}

size_t lcb_ws(int64_t C, int64_t R, int32_t k_req, int32_t k_cand, int32_t n_req, int32_t n_cand, int32_t in_dtype,
              Carver *c, LcbWs *w) {
    Carver local(nullptr);
    Carver &cv = c ? *c : local;
    const int32_t n_total = n_req + n_cand;
    const int32_t s = lcb_splits(R, n_total, k_req, in_dtype);
    int32_t *map = (int32_t *)cv.take(sizeof(int32_t) * (size_t)(C > 0 ? C : 1));
    float *z = (float *)cv.take(sizeof(float) * (size_t)(R > 0 ? R : 1) * (size_t)(n_cand > 0 ? n_cand : 1));
    float *part = (float *)cv.take(sizeof(float) * (size_t)s * (size_t)(R > 0 ? R : 1) * (size_t)(n_total > 0 ? n_total : 1));
    const int64_t nsync = ikbo::lcb_fused_sync_ints(R > 0 ? R : 1, n_total > 0 ? n_total : 1);
    int32_t *sync = (int32_t *)cv.take(sizeof(int32_t) * (size_t)nsync);
    carve_pads(cv, lcb_pad_sizes(C, R, k_req, k_cand, n_req, n_cand, in_dtype), w);
    if (w) {
        w->map = map;
        w->z = z;
        w->partial = part;
        w->partial_cap = (size_t)s * (size_t)(R > 0 ? R : 1) * (size_t)(n_total > 0 ? n_total : 1);
        w->sync = sync;
        w->sync_cap = nsync;
    }
    return cv.used;
}

// One GLM layer (request GEMM + candidate GEMM with the fused gather epilogue).
int run_lcb(const void *x_req, int64_t R, int32_t k_req, const void *x_cand, int64_t C, int32_t k_cand,
            const int32_t *map, const void *w_rr, const void *w_cr, const void *w_cc, const float *b_r,
            const float *b_c, int32_t n_req, int32_t n_cand, int32_t act, int32_t in_dtype, int32_t out_dtype,
            void *y_req, void *y_cand, int64_t ldo_r, int64_t ldo_c, const LcbWs &ws, hipStream_t s) {
    const int in_f32 = in_dtype == IKBO_F32;
    const bool want_req = y_req != nullptr && n_req > 0;
    // alignment rule: bf16 K widths off a multiple of 8 run on zero-padded copies
    if (!in_f32 && k_req % 8) {
        const int32_t kp = (int32_t)round_up8(k_req);
        if (R > 0) {
            IKBO_HIP(ikbo::launch_pad_rows_bf16(x_req, R, k_req, ws.pad_xr, kp, s));
            x_req = ws.pad_xr;
        }
        if (want_req) {
            IKBO_HIP(ikbo::launch_pad_rows_bf16(w_rr, n_req, k_req, ws.pad_wrr, kp, s));
            w_rr = ws.pad_wrr;
        }
        if (n_cand > 0) {
            IKBO_HIP(ikbo::launch_pad_rows_bf16(w_cr, n_cand, k_req, ws.pad_wcr, kp, s));
            w_cr = ws.pad_wcr;
        }
        k_req = kp;
    }
    if (!in_f32 && k_cand % 8 && n_cand > 0) {
        const int32_t kp = (int32_t)round_up8(k_cand);
        if (C > 0) {
            IKBO_HIP(ikbo::launch_pad_rows_bf16(x_cand, C, k_cand, ws.pad_xc, kp, s));
            x_cand = ws.pad_xc;
        }
        IKBO_HIP(ikbo::launch_pad_rows_bf16(w_cc, n_cand, k_cand, ws.pad_wcc, kp, s));
        w_cc = ws.pad_wcc;
        k_cand = kp;
    }
    // bf16 with both GEMMs on direct copies, IKBO_LCB_FUSED=1: one persistent launch that
    // co-schedules the request tiles and the candidate tiles (Sec. 4.2.3). Its results equal the
    // two launches below bit for bit; on this part the two launches are faster (the split-K
    // request GEMM already fills the GPU for its few microseconds, and the persistent loop adds a
    // claim and a flag check per tile), so they are the default.
    if (R > 0 && C > 0 && n_cand > 0 && !in_f32 && ldo_r == n_req && ldo_c == n_cand && getenv_flag("IKBO_LCB_FUSED")) {
        ikbo::LcbFusedArgs f = {};
        ikbo::GemmArgs &g = f.req;
        g.x = x_req;
        g.M = R;
        g.K = k_req;
        g.ldx = k_req;
        g.w0 = want_req ? w_rr : w_cr;
        g.w1 = w_cr;
        g.n0 = want_req ? n_req : n_cand;
        g.N = (want_req ? n_req : 0) + n_cand;
        g.in_f32 = 0;
        g.partial = ws.partial;
        g.splits = lcb_splits(R, g.N, k_req, in_dtype);
        while (g.splits > 1 && (size_t)g.splits * (size_t)R * (size_t)g.N > ws.partial_cap) --g.splits;
        ikbo::GemmArgs &h = f.cand;
        h.x = x_cand;
        h.M = C;
        h.K = k_cand;
        h.ldx = k_cand;
        h.w0 = w_cc;
        h.w1 = w_cc;
        h.n0 = n_cand;
        h.N = n_cand;
        h.in_f32 = 0;
        h.bias = b_c;
        h.z = ws.z;
        h.ldz = n_cand;
        h.map = map;
        h.R = R;
        h.out = y_cand;
        h.ldo = n_cand;
        h.out_f32 = out_dtype == IKBO_F32;
        h.act = act;
        f.n_split = want_req ? n_req : 0;
        f.bias0 = b_r;
        f.act = act;
        f.out0 = y_req;
        f.out0_f32 = out_dtype == IKBO_F32;
        f.sync = ws.sync;
        f.wait_ticks = ikbo::wall_clock_ticks(0.5);   // a safety bound, never reached when the request tiles run
        f.publish = 1;
        // IKBO_LCB_FUSED_WAIT_NS: the bound in nanoseconds instead; a negative value also keeps the
        // request tiles from setting their ready flags, so every candidate wait gives up after
        // |value| ns (a host-forced test of the timeout path: the launch still ends, with NaN tiles)
        if (const char *w = getenv("IKBO_LCB_FUSED_WAIT_NS")) {
            const long long ns = atoll(w);
            f.wait_ticks = ikbo::wall_clock_ticks((double)(ns < 0 ? -ns : ns) * 1e-9);
            f.publish = ns >= 0;
        }
        if ((size_t)R * (size_t)g.N <= ws.partial_cap && ws.sync_cap >= ikbo::lcb_fused_sync_ints(R, g.N) &&
            ikbo::lcb_fused_supported(g, h)) {
            IKBO_HIP(ikbo::launch_lcb_fused(f, s));
            return IKBO_OK;
        }
    }
    // request-batched GEMM: [Y_r | Z] = x_r [W_RR ; W_CR]^T (Sec. 4.1), split-K + fixed-order reduce
    if (R > 0 && (want_req || n_cand > 0)) {
        ikbo::GemmArgs g = {};
        g.x = x_req;
        g.M = R;
        g.K = k_req;
        g.ldx = k_req;
        g.w0 = want_req ? w_rr : w_cr;
        g.w1 = w_cr;
        g.n0 = want_req ? n_req : n_cand;
        g.N = (want_req ? n_req : 0) + n_cand;
        g.in_f32 = in_f32;
        g.partial = ws.partial;
        g.splits = lcb_splits(R, g.N, k_req, in_dtype);
        while (g.splits > 1 && (size_t)g.splits * (size_t)R * (size_t)g.N > ws.partial_cap) --g.splits;
        if ((size_t)R * (size_t)g.N > ws.partial_cap)
            return fail(IKBO_WORKSPACE_TOO_SMALL, "internal: request GEMM partials exceed the workspace sizing");
        IKBO_HIP(ikbo::launch_gemm(g, s));
        IKBO_HIP(ikbo::launch_splitk_reduce(ws.partial, g.splits, R, g.N, want_req ? n_req : 0, b_r, act, y_req,
                                            out_dtype == IKBO_F32, ldo_r, ws.z, s));
    }
    // candidate GEMM with the broadcast-add fused in the epilogue (Sec. 4.2.1, Eq. 14)
    if (C > 0 && n_cand > 0) {
        ikbo::GemmArgs g = {};
        g.x = x_cand;
        g.M = C;
        g.K = k_cand;
        g.ldx = k_cand;
        g.w0 = w_cc;
        g.w1 = w_cc;
        g.n0 = n_cand;
        g.N = n_cand;
        g.in_f32 = in_f32;
        g.bias = b_c;
        g.z = ws.z;
        g.ldz = n_cand;
        g.map = map;
        g.R = R;
        g.out = y_cand;
        g.ldo = ldo_c;
        g.out_f32 = out_dtype == IKBO_F32;
        g.act = act;
        g.partial = nullptr;
        g.splits = 1;
        IKBO_HIP(ikbo::launch_gemm(g, s));
    }
    return IKBO_OK;
}

int check_index_args(const int32_t *m, const int32_t *off, uint32_t flags, int64_t C) {
    if (!m && !off && C > 0) return fail(IKBO_INVALID_ARGUMENT, "need cand_to_req or req_cand_offsets (both are NULL)");
    if (flags & ~IKBO_INDEX_SORTED) return fail(IKBO_INVALID_ARGUMENT, "unknown index_flags bits 0x%x", flags);
    if ((m && !aligned16(m)) || (off && !aligned16(off)))
        return fail(IKBO_MISALIGNED, "index arrays must be 16-byte aligned");
    return IKBO_OK;
}

int check_layer_dims(int32_t k_req, int32_t k_cand, int32_t n_req, int32_t n_cand, int32_t act, int32_t in_dtype) {
    if (k_req < 0 || k_cand < 0 || n_req < 0 || n_cand < 0)
        return fail(IKBO_INVALID_ARGUMENT, "negative layer width (k_req %d k_cand %d n_req %d n_cand %d)", k_req, k_cand,
                    n_req, n_cand);
    if (act != IKBO_ACT_NONE && act != IKBO_ACT_GELU) return fail(IKBO_INVALID_ARGUMENT, "unknown activation %d", act);
    (void)in_dtype;     // any K width: bf16 widths off a multiple of 8 are zero-padded in the workspace
    return IKBO_OK;
}

}  // namespace

extern "C" {

int ikbo_version(void) { return IKBO_VERSION; }

const char *ikbo_status_string(int status) {
    switch (status) {
    case IKBO_OK: return "IKBO_OK";
    case IKBO_INVALID_ARGUMENT: return "IKBO_INVALID_ARGUMENT";
    case IKBO_UNSUPPORTED: return "IKBO_UNSUPPORTED";
    case IKBO_MISALIGNED: return "IKBO_MISALIGNED";
    case IKBO_WORKSPACE_TOO_SMALL: return "IKBO_WORKSPACE_TOO_SMALL";
    case IKBO_HIP_ERROR: return "IKBO_HIP_ERROR";
    default: return "IKBO_UNKNOWN_STATUS";
    }
}

const char *ikbo_last_error_message(void) { return g_last_error.c_str(); }

size_t ikbo_dca_workspace_size(int64_t num_cand, int64_t num_req) {
    if (num_cand < 0 || num_req < 0) return 0;
    return dca_ws(num_cand, num_req, nullptr, nullptr, nullptr, nullptr, nullptr);
}

// Argument checks of ikbo_dca_forward (nothing enqueued)
static int dca_validate(const void *q, int64_t C, int32_t q_len, const void *k, const void *v, int64_t R,
                        const int32_t *kv_cu_seqlens, int32_t kv_len, const int32_t *cand_to_req,
                        const int32_t *req_cand_offsets, uint32_t index_flags, int32_t num_heads, int32_t head_dim,
                        int32_t in_dtype, int32_t out_dtype, const void *out, const void *workspace,
                        size_t workspace_bytes) {
    if (C < 0 || R < 0 || q_len <= 0 || num_heads <= 0 || head_dim <= 0 || kv_len < 0)
        return fail(IKBO_INVALID_ARGUMENT, "bad sizes (num_cand %lld num_req %lld q_len %d heads %d head_dim %d kv_len %d)",
                    (long long)C, (long long)R, q_len, num_heads, head_dim, kv_len);
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return fail(IKBO_UNSUPPORTED, "dtype in %d out %d", in_dtype, out_dtype);
    if (in_dtype == IKBO_BF16 && head_dim != 64 && head_dim != 128)
        return fail(IKBO_UNSUPPORTED, "bf16 DCA is built for head_dim 64 and 128, got %d", head_dim);
    if (in_dtype == IKBO_BF16 && (int64_t)kv_len * num_heads * head_dim * 2 >= (1LL << 31))
        return fail(IKBO_UNSUPPORTED, "bf16 DCA needs L_r * num_heads * head_dim * 2 < 2^31 bytes (kv_len %d)", kv_len);
    if (in_dtype == IKBO_F32 && (head_dim % 4 || head_dim > 128))
        return fail(IKBO_UNSUPPORTED, "fp32 DCA needs head_dim a multiple of 4 up to 128, got %d", head_dim);
    int rc = check_index_args(cand_to_req, req_cand_offsets, index_flags, C);
    if (rc) return rc;
    if (C > 0 && (!q || !out)) return fail(IKBO_INVALID_ARGUMENT, "q and out must be non-NULL when num_cand > 0");
    if (R > 0 && (!k || !v)) return fail(IKBO_INVALID_ARGUMENT, "k and v must be non-NULL when num_req > 0");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(kv_cu_seqlens) ||
        !aligned16(workspace))
        return fail(IKBO_MISALIGNED, "tensor base pointers must be 16-byte aligned");
    if (C * (int64_t)q_len > 0x7fffffffLL || C > 0x7fffffffLL || R > 0x7ffffffeLL)
        return fail(IKBO_UNSUPPORTED, "num_cand * q_len must fit in int32");
    const size_t need = ikbo_dca_workspace_size(C, R);
    if (workspace_bytes < need || (!workspace && need > 0))
        return fail(IKBO_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes, need);
    return IKBO_OK;
}

// The DCA launches of ikbo_dca_forward, arguments already validated
// q_cs / o_cs: elements from one candidate's query (output) rows to the next's; 0 means packed
// (q_len * num_heads * head_dim).
static int dca_run(const void *q, int64_t C, int32_t q_len, const void *k, const void *v, int64_t R,
                   const int32_t *kv_cu_seqlens, int32_t kv_len, const int32_t *cand_to_req,
                   const int32_t *req_cand_offsets, int32_t num_heads, int32_t head_dim, float softmax_scale,
                   int32_t in_dtype, int32_t out_dtype, void *out, void *workspace, hipStream_t s, int64_t q_cs = 0,
                   int64_t o_cs = 0) {
    if (C == 0) return ok();
    const int in_f32 = in_dtype == IKBO_F32;
    const int64_t row_elems = (int64_t)q_len * num_heads * head_dim;
    if (q_cs == 0) q_cs = row_elems;
    if (o_cs == 0) o_cs = row_elems;
    // the bf16 kernel reads and writes rows in 16-byte pieces
    if (!in_f32 && (q_cs % 8 != 0 || o_cs % 8 != 0))
        return fail(IKBO_MISALIGNED, "candidate row strides must be multiples of 8 elements");
    const int ob = (int)esize(out_dtype);
    // work tile by the average stacked query rows per request: at most 32 one wave, at most 1024
    // four waves (128 rows), else eight (256 rows); a request's last tile is partly empty, and
    // smaller tiles waste fewer rows where requests are short
    const int64_t rows_all = C * (int64_t)q_len;
    const int mode = in_f32 ? 0 : rows_all <= 32 * R ? 1 : rows_all <= 1024 * R ? 2 : 0;

    Carver cv(workspace);
    int32_t *counts, *off, *tiles, *perm, *sort_scratch;
    dca_ws(C, R, &cv, &counts, &off, &tiles, &perm, &sort_scratch);
    const int32_t bm = ikbo::dca_block_m(head_dim, in_f32, mode);
    const int32_t *perm_used = nullptr;
    if (req_cand_offsets) {
        // the offsets define the grouping (cand_to_req, if also given, is not read)
        IKBO_HIP(ikbo::launch_scan_tiles(nullptr, req_cand_offsets, R, C, q_len, num_heads, bm, off, nullptr, tiles, s));
        IKBO_HIP(ikbo::launch_zero_uncovered(req_cand_offsets, R, C, out, row_elems, o_cs, ob, s));
    } else {
        // group an arbitrary map: counts -> offsets and tiles, then a stable sort of the candidates
        // by request (each request's candidates keep their index order); rows without a valid
        // request are zeroed
        IKBO_HIP(ikbo::launch_fill_i32(counts, R + 1, 0, s));
        IKBO_HIP(ikbo::launch_histogram(cand_to_req, C, R, counts, s));
        IKBO_HIP(ikbo::launch_scan_tiles(counts, nullptr, R, C, q_len, num_heads, bm, off, nullptr, tiles, s));
        IKBO_HIP(ikbo::launch_stable_group(cand_to_req, C, R, perm, sort_scratch, s));
        IKBO_HIP(ikbo::launch_zero_invalid_rows(cand_to_req, C, R, out, row_elems, o_cs, ob, s));
        perm_used = perm;
    }
    if (R == 0) return ok();
    ikbo::DcaArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.C = C;
    a.R = R;
    a.Lq = q_len;
    a.H = num_heads;
    a.D = head_dim;
    a.L = kv_cu_seqlens ? 0 : kv_len;
    a.kv_cu = kv_cu_seqlens;
    a.off = off;
    a.perm = perm_used;
    a.tile_start = tiles;
    a.grid_tiles = (int64_t)num_heads * ((C * q_len) / bm + R + 1);
    a.scale = softmax_scale > 0.0f ? softmax_scale : (float)(1.0 / sqrt((double)head_dim));
    a.in_f32 = in_f32;
    a.out_f32 = out_dtype == IKBO_F32;
    a.mode = mode;
    a.q_cs = q_cs;
    a.o_cs = o_cs;
    IKBO_HIP(ikbo::launch_dca(a, s));
    return ok();
}

int ikbo_dca_forward(const void *q, int64_t num_cand, int32_t q_len, const void *k, const void *v, int64_t num_req,
                     const int32_t *kv_cu_seqlens, int32_t kv_len, const int32_t *cand_to_req,
                     const int32_t *req_cand_offsets, uint32_t index_flags, int32_t num_heads, int32_t head_dim,
                     float softmax_scale, int32_t in_dtype, int32_t out_dtype, void *out, void *workspace,
                     size_t workspace_bytes, void *hip_stream) {
    const int rc = dca_validate(q, num_cand, q_len, k, v, num_req, kv_cu_seqlens, kv_len, cand_to_req, req_cand_offsets,
                                index_flags, num_heads, head_dim, in_dtype, out_dtype, out, workspace, workspace_bytes);
    if (rc) return rc;
    return dca_run(q, num_cand, q_len, k, v, num_req, kv_cu_seqlens, kv_len, cand_to_req, req_cand_offsets, num_heads,
                   head_dim, softmax_scale, in_dtype, out_dtype, out, workspace, (hipStream_t)hip_stream);
}

// ---- IKBO-DCA without allocation ------------------------------------------------------------------
// Scratch for callers that cannot allocate: one fixed array on every GPU the library runs on, held
// until the process ends. In host code `scratch` is a host-side stand-in for the symbol, not a
// device address: its device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[IKBO_DCA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices];     // device address of `scratch` on each device, once looked up

// The device address of the current device's scratch array (looked up on its first use).
int current_device_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(IKBO_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(IKBO_HIP_ERROR, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return IKBO_OK;
}
}  // namespace

int ikbo_dca_forward_noalloc(const void *q, int64_t num_cand, int32_t q_len, const void *k, const void *v,
                             int64_t num_req, const int32_t *kv_cu_seqlens, int32_t kv_len, const int32_t *cand_to_req,
                             const int32_t *req_cand_offsets, uint32_t index_flags, int32_t num_heads,
                             int32_t head_dim, float softmax_scale, int32_t in_dtype, int32_t out_dtype, void *out,
                             void *hip_stream) {
    if (num_cand < 0 || num_req < 0)
        return fail(IKBO_INVALID_ARGUMENT, "bad sizes (num_cand %lld num_req %lld)", (long long)num_cand,
                    (long long)num_req);
    const size_t need = ikbo_dca_workspace_size(num_cand, num_req);
    if (need > (size_t)IKBO_DCA_NOALLOC_SCRATCH_BYTES)
        return fail(IKBO_WORKSPACE_TOO_SMALL, "num_cand %lld / num_req %lld need %zu bytes of scratch, above the fixed "
                    "%zu-byte array of ikbo_dca_forward_noalloc (use ikbo_dca_forward with a workspace)",
                    (long long)num_cand, (long long)num_req, need, (size_t)IKBO_DCA_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    int rc = current_device_scratch(&ws);
    if (rc) return rc;
    rc = dca_validate(q, num_cand, q_len, k, v, num_req, kv_cu_seqlens, kv_len, cand_to_req, req_cand_offsets,
                      index_flags, num_heads, head_dim, in_dtype, out_dtype, out, ws, IKBO_DCA_NOALLOC_SCRATCH_BYTES);
    if (rc) return rc;
    return dca_run(q, num_cand, q_len, k, v, num_req, kv_cu_seqlens, kv_len, cand_to_req, req_cand_offsets, num_heads,
                   head_dim, softmax_scale, in_dtype, out_dtype, out, ws, (hipStream_t)hip_stream);
}

// ---- request-side attention ---------------------------------------------------------------------
size_t ikbo_request_attention_workspace_size(int64_t num_req) {
    if (num_req < 0) return 0;
    return align256(sizeof(int32_t) * (size_t)(num_req + 1)) + ikbo_dca_workspace_size(num_req, num_req);
}

// q_cs / o_cs: elements between consecutive requests' query (output) rows; 0 means packed.
// Argument checks of the request-side attention (nothing enqueued)
static int request_attention_check(const void *q_req, int64_t num_req, int32_t q_len, const void *k, const void *v,
                                   const int32_t *kv_cu_seqlens, int32_t kv_len, int32_t num_heads, int32_t head_dim,
                                   int32_t in_dtype, int32_t out_dtype, const void *out, void *workspace,
                                   size_t workspace_bytes) {
    const int64_t R = num_req;
    if (R < 0) return fail(IKBO_INVALID_ARGUMENT, "negative num_req");
    const size_t need = ikbo_request_attention_workspace_size(R);
    if (workspace_bytes < need || !workspace)
        return fail(IKBO_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes, need);
    if (!aligned16(workspace)) return fail(IKBO_MISALIGNED, "tensor base pointers must be 16-byte aligned");
    Carver cv(workspace);
    int32_t *ident = (int32_t *)cv.take(sizeof(int32_t) * (size_t)(R + 1));
    return dca_validate(q_req, R, q_len, k, v, R, kv_cu_seqlens, kv_len, nullptr, ident, IKBO_INDEX_SORTED, num_heads,
                        head_dim, in_dtype, out_dtype, out, (char *)workspace + cv.used, workspace_bytes - cv.used);
}

static int request_attention_impl(const void *q_req, int64_t num_req, int32_t q_len, const void *k, const void *v,
                                  const int32_t *kv_cu_seqlens, int32_t kv_len, int32_t num_heads, int32_t head_dim,
                                  float softmax_scale, int32_t in_dtype, int32_t out_dtype, void *out, void *workspace,
                                  size_t workspace_bytes, void *hip_stream, int64_t q_cs, int64_t o_cs) {
    const int64_t R = num_req;
    const int rc = request_attention_check(q_req, R, q_len, k, v, kv_cu_seqlens, kv_len, num_heads, head_dim, in_dtype,
                                           out_dtype, out, workspace, workspace_bytes);
    if (rc) return rc;
    if (R == 0) return ok();
    // the identity map as offsets (request r is candidate r), then the DCA over it
    Carver cv(workspace);
    int32_t *ident = (int32_t *)cv.take(sizeof(int32_t) * (size_t)(R + 1));
    void *rest = (char *)workspace + cv.used;
    hipStream_t s = (hipStream_t)hip_stream;
    IKBO_HIP(ikbo::launch_iota_i32(ident, R + 1, s));
    return dca_run(q_req, R, q_len, k, v, R, kv_cu_seqlens, kv_len, nullptr, ident, num_heads, head_dim, softmax_scale,
                   in_dtype, out_dtype, out, rest, s, q_cs, o_cs);
}

int ikbo_request_attention(const void *q_req, int64_t num_req, int32_t q_len, const void *k, const void *v,
                           const int32_t *kv_cu_seqlens, int32_t kv_len, int32_t num_heads, int32_t head_dim,
                           float softmax_scale, int32_t in_dtype, int32_t out_dtype, void *out, void *workspace,
                           size_t workspace_bytes, void *hip_stream) {
    return request_attention_impl(q_req, num_req, q_len, k, v, kv_cu_seqlens, kv_len, num_heads, head_dim,
                                  softmax_scale, in_dtype, out_dtype, out, workspace, workspace_bytes, hip_stream, 0, 0);
}

// ---- GLM factorization machine -------------------------------------------------------------------
int ikbo_fm_forward(const void *x_req, int64_t num_req, int32_t n_req_feat, const void *x_cand, int64_t num_cand,
                    int32_t n_cand_feat, int32_t dim, const int32_t *cand_to_req, const int32_t *req_cand_offsets,
                    uint32_t index_flags, int32_t in_dtype, int32_t out_dtype, void *y_req, void *y_cand,
                    void *hip_stream) {
    const int64_t R = num_req, C = num_cand;
    if (R < 0 || C < 0 || n_req_feat < 0 || n_cand_feat < 0 || dim <= 0)
        return fail(IKBO_INVALID_ARGUMENT, "bad sizes (num_req %lld num_cand %lld n_req_feat %d n_cand_feat %d dim %d)",
                    (long long)R, (long long)C, n_req_feat, n_cand_feat, dim);
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return fail(IKBO_UNSUPPORTED, "dtype in %d out %d", in_dtype, out_dtype);
    if (n_req_feat % 4 || n_cand_feat % 4)
        return fail(IKBO_UNSUPPORTED, "feature counts must be multiples of 4 (got %d, %d)", n_req_feat, n_cand_feat);
    int rc = check_index_args(cand_to_req, req_cand_offsets, index_flags, C);
    if (rc) return rc;
    const bool want_req = y_req != nullptr && R > 0 && n_req_feat > 0;
    if (C > 0 && (n_cand_feat > 0) && (!x_cand || !y_cand))
        return fail(IKBO_INVALID_ARGUMENT, "x_cand and y_cand must be non-NULL when num_cand > 0");
    if ((want_req || (C > 0 && n_req_feat > 0)) && R > 0 && !x_req)
        return fail(IKBO_INVALID_ARGUMENT, "x_req is NULL");
    const void *ptrs[] = {x_req, x_cand, y_req, y_cand};
    for (const void *p : ptrs)
        if (!aligned16(p)) return fail(IKBO_MISALIGNED, "tensor base pointers must be 16-byte aligned");
    if (C * (int64_t)n_cand_feat * (n_req_feat + n_cand_feat) > (1LL << 62))
        return fail(IKBO_UNSUPPORTED, "output too large");
    if ((C == 0 || n_cand_feat == 0) && !want_req) return ok();
    ikbo::FmArgs a = {};
    a.x_r = x_req;
    a.x_c = x_cand;
    a.y_r = want_req ? y_req : nullptr;
    a.y_c = y_cand;
    a.R = R;
    a.C = n_cand_feat > 0 ? C : 0;
    a.n_r = n_req_feat;
    a.n_c = n_cand_feat;
    a.d = dim;
    a.map = cand_to_req;
    a.off = req_cand_offsets;
    a.in_f32 = in_dtype == IKBO_F32;
    a.out_f32 = out_dtype == IKBO_F32;
    IKBO_HIP(ikbo::launch_fm(a, (hipStream_t)hip_stream));
    return ok();
}

// ---- LCB, embedding-matrix form, with the group-local norm ----------------------------------------
size_t ikbo_lcb_emb_workspace_size(int64_t num_req, int32_t n_cand_out, int32_t dim) {
    if (num_req < 0 || n_cand_out < 0 || dim < 0) return 0;
    return align256(sizeof(float) * (size_t)num_req * (size_t)n_cand_out * (size_t)dim);
}

int ikbo_lcb_emb_forward(const void *x_req, int64_t num_req, int32_t n_req_in, const void *x_cand, int64_t num_cand,
                         int32_t n_cand_in, int32_t dim, const void *w_rr, int32_t n_req_out, const void *w_cr,
                         const void *w_cc, int32_t n_cand_out, const int32_t *cand_to_req,
                         const int32_t *req_cand_offsets, uint32_t index_flags, int32_t norm, const float *gamma_req,
                         const float *beta_req, const float *gamma_cand, const float *beta_cand, float eps,
                         int32_t in_dtype, int32_t out_dtype, void *y_req, void *y_cand, void *workspace,
                         size_t workspace_bytes, void *hip_stream) {
    const int64_t R = num_req, C = num_cand;
    if (R < 0 || C < 0 || n_req_in < 1 || n_cand_in < 1 || n_req_out < 0 || n_cand_out < 0 || dim < 1)
        return fail(IKBO_INVALID_ARGUMENT,
                    "bad sizes (num_req %lld num_cand %lld n_req_in %d n_cand_in %d n_req_out %d n_cand_out %d dim %d)",
                    (long long)R, (long long)C, n_req_in, n_cand_in, n_req_out, n_cand_out, dim);
    if (dim > ikbo::kLcbeMaxDim) return fail(IKBO_UNSUPPORTED, "dim %d above %d", dim, ikbo::kLcbeMaxDim);
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return fail(IKBO_UNSUPPORTED, "dtype in %d out %d", in_dtype, out_dtype);
    if (norm != IKBO_NORM_NONE && norm != IKBO_NORM_LAYER && norm != IKBO_NORM_RMS)
        return fail(IKBO_INVALID_ARGUMENT, "unknown norm %d", norm);
    if (!(eps >= 0.0f) || eps > 3.0e38f) return fail(IKBO_INVALID_ARGUMENT, "eps must be finite and >= 0");
    int rc = check_index_args(cand_to_req, req_cand_offsets, index_flags, C);
    if (rc) return rc;
    const bool want_req = y_req != nullptr && R > 0 && n_req_out > 0;
    const bool want_cand = C > 0 && n_cand_out > 0;
    if (want_cand && (!x_cand || !y_cand || !w_cc || (R > 0 && (!w_cr || !x_req))))
        return fail(IKBO_INVALID_ARGUMENT, "x_cand, y_cand, w_cc, w_cr and x_req must be non-NULL for the candidate group");
    if (want_req && (!x_req || !w_rr)) return fail(IKBO_INVALID_ARGUMENT, "x_req and w_rr must be non-NULL");
    const void *ptrs[] = {x_req, x_cand, w_rr, w_cr, w_cc, gamma_req, beta_req, gamma_cand, beta_cand, y_req, y_cand, workspace};
    for (const void *p : ptrs)
        if (!aligned16(p)) return fail(IKBO_MISALIGNED, "tensor base pointers must be 16-byte aligned");
    const size_t need = want_cand ? ikbo_lcb_emb_workspace_size(R, n_cand_out, dim) : 0;
    if (need && (workspace_bytes < need || !workspace))
        return fail(IKBO_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes, need);
    if (!want_req && !want_cand) return ok();
    ikbo::LcbeArgs a = {};
    a.x_r = x_req;
    a.x_c = x_cand;
    a.w_rr = w_rr;
    a.w_cr = w_cr;
    a.w_cc = w_cc;
    a.g_r = gamma_req;
    a.b_r = beta_req;
    a.g_c = gamma_cand;
    a.b_c = beta_cand;
    a.z = want_cand && R > 0 ? (float *)workspace : nullptr;
    a.y_r = want_req ? y_req : nullptr;
    a.y_c = want_cand ? y_cand : nullptr;
    a.R = R;
    a.C = want_cand ? C : 0;
    a.n_r = n_req_in;
    a.n_c = n_cand_in;
    a.k_r = n_req_out;
    a.k_c = n_cand_out;
    a.d = dim;
    a.map = cand_to_req;
    a.off = req_cand_offsets;
    a.in_f32 = in_dtype == IKBO_F32;
    a.out_f32 = out_dtype == IKBO_F32;
    a.norm = norm;
    a.eps = eps;
    IKBO_HIP(ikbo::launch_lcbe(a, (hipStream_t)hip_stream));
    return ok();
}

// ---- K/V projection -----------------------------------------------------------------------------
// Argument checks of the K/V projection (nothing enqueued)
static int kv_project_check(const void *s_rows, int64_t rows, int32_t d_in, const void *w_k, const void *w_v,
                            int32_t d_out, int32_t in_dtype, int32_t out_dtype, const void *k_out, const void *v_out) {
    if (rows < 0 || d_in < 0 || d_out < 0)
        return fail(IKBO_INVALID_ARGUMENT, "bad sizes (rows %lld d_in %d d_out %d)", (long long)rows, d_in, d_out);
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return fail(IKBO_UNSUPPORTED, "dtype in %d out %d", in_dtype, out_dtype);
    if (rows == 0 || d_out == 0) return IKBO_OK;
    if (!s_rows || !w_k || !w_v || !k_out || !v_out) return fail(IKBO_INVALID_ARGUMENT, "a tensor pointer is NULL");
    const void *ptrs[] = {s_rows, w_k, w_v, k_out, v_out};
    for (const void *p : ptrs)
        if (!aligned16(p)) return fail(IKBO_MISALIGNED, "tensor base pointers must be 16-byte aligned");
    if (d_in % (in_dtype == IKBO_F32 ? 4 : 8)) return fail(IKBO_MISALIGNED, "d_in must keep 16-byte rows (got %d)", d_in);
    return IKBO_OK;
}

int ikbo_kv_project(const void *s_rows, int64_t rows, int32_t d_in, const void *w_k, const void *w_v, int32_t d_out,
                    int32_t in_dtype, int32_t out_dtype, void *k_out, void *v_out, void *hip_stream) {
    const int rc = kv_project_check(s_rows, rows, d_in, w_k, w_v, d_out, in_dtype, out_dtype, k_out, v_out);
    if (rc) return rc;
    if (rows == 0 || d_out == 0) return ok();
    const int in_f32 = in_dtype == IKBO_F32;
    hipStream_t s = (hipStream_t)hip_stream;
    // one GEMM per projection: out = s W^T, no bias, no activation, no gather
    for (int which = 0; which < 2; ++which) {
        ikbo::GemmArgs g = {};
        g.x = s_rows;
        g.M = rows;
        g.K = d_in;
        g.ldx = d_in;
        g.w0 = which ? w_v : w_k;
        g.w1 = g.w0;
        g.n0 = d_out;
        g.N = d_out;
        g.in_f32 = in_f32;
        g.out = which ? v_out : k_out;
        g.ldo = d_out;
        g.out_f32 = out_dtype == IKBO_F32;
        IKBO_HIP(ikbo::launch_gemm(g, s));
    }
    return ok();
}

size_t ikbo_lcb_workspace_size(int64_t num_cand, int64_t num_req, int32_t k_req, int32_t k_cand, int32_t n_req_out,
                               int32_t n_cand_out, int32_t in_dtype) {
    if (num_cand < 0 || num_req < 0 || k_req < 0 || k_cand < 0 || n_req_out < 0 || n_cand_out < 0 || !dtype_ok(in_dtype))
        return 0;
    return lcb_ws(num_cand, num_req, k_req, k_cand, n_req_out, n_cand_out, in_dtype, nullptr, nullptr);
}

int ikbo_lcb_forward(const void *x_req, int64_t num_req, int32_t k_req, const void *x_cand, int64_t num_cand,
                     int32_t k_cand, const int32_t *cand_to_req, const int32_t *req_cand_offsets, uint32_t index_flags,
                     const void *w_rr, const void *w_cr, const void *w_cc, const float *b_r, const float *b_c,
                     int32_t n_req_out, int32_t n_cand_out, int32_t activation, int32_t in_dtype, int32_t out_dtype,
                     void *y_req, void *y_cand, void *workspace, size_t workspace_bytes, void *hip_stream) {
    const int64_t C = num_cand, R = num_req;
    if (C < 0 || R < 0) return fail(IKBO_INVALID_ARGUMENT, "negative num_cand / num_req");
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return fail(IKBO_UNSUPPORTED, "dtype in %d out %d", in_dtype, out_dtype);
    int rc = check_layer_dims(k_req, k_cand, n_req_out, n_cand_out, activation, in_dtype);
    if (rc) return rc;
    rc = check_index_args(cand_to_req, req_cand_offsets, index_flags, C);
    if (rc) return rc;
    if (R > 0 && k_req > 0 && !x_req) return fail(IKBO_INVALID_ARGUMENT, "x_req is NULL");
    if (C > 0 && k_cand > 0 && !x_cand) return fail(IKBO_INVALID_ARGUMENT, "x_cand is NULL");
    if (C > 0 && n_cand_out > 0 && !y_cand) return fail(IKBO_INVALID_ARGUMENT, "y_cand is NULL");
    if (n_cand_out > 0 && ((k_req > 0 && !w_cr) || (k_cand > 0 && !w_cc)))
        return fail(IKBO_INVALID_ARGUMENT, "w_cr / w_cc is NULL");
    if (y_req && n_req_out > 0 && k_req > 0 && !w_rr) return fail(IKBO_INVALID_ARGUMENT, "w_rr is NULL");
    const void *ptrs[] = {x_req, x_cand, w_rr, w_cr, w_cc, b_r, b_c, y_req, y_cand, workspace};
    for (const void *p : ptrs)
        if (!aligned16(p)) return fail(IKBO_MISALIGNED, "tensor base pointers must be 16-byte aligned");
    const size_t need = ikbo_lcb_workspace_size(C, R, k_req, k_cand, n_req_out, n_cand_out, in_dtype);
    if (workspace_bytes < need || !workspace) return fail(IKBO_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes, need);
    hipStream_t s = (hipStream_t)hip_stream;
    Carver cv(workspace);
    LcbWs ws;
    lcb_ws(C, R, k_req, k_cand, n_req_out, n_cand_out, in_dtype, &cv, &ws);
    // the offsets, when given, define each candidate's request (as in every entry point)
    const int32_t *map = cand_to_req;
    if (req_cand_offsets) {
        IKBO_HIP(ikbo::launch_offsets_to_map(req_cand_offsets, R, C, ws.map, s));
        map = ws.map;
    }
    rc = run_lcb(x_req, R, k_req, x_cand, C, k_cand, map, w_rr, w_cr, w_cc, b_r, b_c, n_req_out, n_cand_out, activation,
                 in_dtype, out_dtype, y_req, y_cand, n_req_out, n_cand_out, ws, s);
    return rc ? rc : ok();
}

static PadSizes glm_pad_sizes(int64_t C, int64_t R, int32_t num_layers, const ikbo_glm_layer *layers, int32_t in_dtype) {
    PadSizes p;
    for (int l = 0; l < num_layers; ++l)
        p.take_max(lcb_pad_sizes(C, R, layers[l].k_req, layers[l].k_cand, layers[l].n_req_out, layers[l].n_cand_out,
                                 in_dtype));
    return p;
}

size_t ikbo_glm_mlp_workspace_size(int64_t num_cand, int64_t num_req, int32_t num_layers, const ikbo_glm_layer *layers,
                                   int32_t in_dtype) {
    if (num_cand < 0 || num_req < 0 || num_layers <= 0 || !layers || !dtype_ok(in_dtype)) return 0;
    int32_t max_kr = 0, max_nr = 0, max_nc = 0, max_ntot = 0;
    for (int l = 0; l < num_layers; ++l) {
        const ikbo_glm_layer &ly = layers[l];
        if (ly.k_req > max_kr) max_kr = ly.k_req;
        if (ly.n_req_out > max_nr) max_nr = ly.n_req_out;
        if (ly.n_cand_out > max_nc) max_nc = ly.n_cand_out;
        if (ly.n_req_out + ly.n_cand_out > max_ntot) max_ntot = ly.n_req_out + ly.n_cand_out;
    }
    Carver cv(nullptr);
    // map, Z and partials sized for the widest layer (split counts checked per layer at run time)
    int32_t smax = 1;
    for (int l = 0; l < num_layers; ++l) {
        int32_t sl = lcb_splits(num_req, layers[l].n_req_out + layers[l].n_cand_out, layers[l].k_req, in_dtype);
        if (sl > smax) smax = sl;
    }
    cv.take(sizeof(int32_t) * (size_t)(num_cand > 0 ? num_cand : 1));
    cv.take(sizeof(float) * (size_t)(num_req > 0 ? num_req : 1) * (size_t)(max_nc > 0 ? max_nc : 1));
    cv.take(sizeof(float) * (size_t)smax * (size_t)(num_req > 0 ? num_req : 1) * (size_t)(max_ntot > 0 ? max_ntot : 1));
    cv.take(sizeof(int32_t) * (size_t)ikbo::lcb_fused_sync_ints(num_req > 0 ? num_req : 1, max_ntot > 0 ? max_ntot : 1));
    carve_pads(cv, glm_pad_sizes(num_cand, num_req, num_layers, layers, in_dtype), nullptr);
    if (num_layers > 1) {
        const size_t e = esize(in_dtype);
        for (int b = 0; b < 2; ++b) {
            cv.take(e * (size_t)(num_req > 0 ? num_req : 1) * (size_t)(max_nr > 0 ? max_nr : 1));
            cv.take(e * (size_t)(num_cand > 0 ? num_cand : 1) * (size_t)(max_nc > 0 ? max_nc : 1));
        }
    }
    return cv.used;
}

// Argument checks of the GLM-MLP (nothing enqueued)
static int glm_mlp_check(const void *x_req, int64_t num_req, const void *x_cand, int64_t num_cand,
                         const int32_t *cand_to_req, const int32_t *req_cand_offsets, uint32_t index_flags,
                         int32_t num_layers, const ikbo_glm_layer *layers, int32_t in_dtype, int32_t out_dtype,
                         const void *y_req, const void *y_cand, const void *workspace, size_t workspace_bytes) {
    const int64_t C = num_cand, R = num_req;
    if (C < 0 || R < 0) return fail(IKBO_INVALID_ARGUMENT, "negative num_cand / num_req");
    if (num_layers <= 0 || !layers) return fail(IKBO_INVALID_ARGUMENT, "need num_layers >= 1 and a host layer array");
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return fail(IKBO_UNSUPPORTED, "dtype in %d out %d", in_dtype, out_dtype);
    int rc = check_index_args(cand_to_req, req_cand_offsets, index_flags, C);
    if (rc) return rc;
    for (int l = 0; l < num_layers; ++l) {
        const ikbo_glm_layer &ly = layers[l];
        rc = check_layer_dims(ly.k_req, ly.k_cand, ly.n_req_out, ly.n_cand_out, ly.activation, in_dtype);
        if (rc) return fail(rc, "layer %d: %s", l, g_last_error.c_str());
        if (l > 0 && (ly.k_req != layers[l - 1].n_req_out || ly.k_cand != layers[l - 1].n_cand_out))
            return fail(IKBO_INVALID_ARGUMENT, "layer %d input widths (%d, %d) do not match layer %d outputs (%d, %d)", l,
                        ly.k_req, ly.k_cand, l - 1, layers[l - 1].n_req_out, layers[l - 1].n_cand_out);
        const void *ptrs[] = {ly.w_rr, ly.w_cr, ly.w_cc, ly.b_r, ly.b_c};
        for (const void *p : ptrs)
            if (!aligned16(p)) return fail(IKBO_MISALIGNED, "layer %d: weight pointers must be 16-byte aligned", l);
        if ((ly.n_cand_out > 0 && ((ly.k_req > 0 && !ly.w_cr) || (ly.k_cand > 0 && !ly.w_cc))) ||
            (ly.n_req_out > 0 && ly.k_req > 0 && !ly.w_rr))
            return fail(IKBO_INVALID_ARGUMENT, "layer %d: NULL weight", l);
    }
    const ikbo_glm_layer &last = layers[num_layers - 1];
    if (C > 0 && last.n_cand_out > 0 && !y_cand) return fail(IKBO_INVALID_ARGUMENT, "y_cand is NULL");
    if ((R > 0 && layers[0].k_req > 0 && !x_req) || (C > 0 && layers[0].k_cand > 0 && !x_cand))
        return fail(IKBO_INVALID_ARGUMENT, "x_req / x_cand is NULL");
    const void *ptrs[] = {x_req, x_cand, y_req, y_cand, workspace};
    for (const void *p : ptrs)
        if (!aligned16(p)) return fail(IKBO_MISALIGNED, "tensor base pointers must be 16-byte aligned");
    const size_t need = ikbo_glm_mlp_workspace_size(C, R, num_layers, layers, in_dtype);
    if (workspace_bytes < need || !workspace)
        return fail(IKBO_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes, need);
    return IKBO_OK;
}

// The GLM-MLP with the last layer's outputs written with row strides ldo_r / ldo_c (0: packed).
static int glm_mlp_impl(const void *x_req, int64_t num_req, const void *x_cand, int64_t num_cand,
                        const int32_t *cand_to_req, const int32_t *req_cand_offsets, uint32_t index_flags,
                        int32_t num_layers, const ikbo_glm_layer *layers, int32_t in_dtype, int32_t out_dtype,
                        void *y_req, void *y_cand, int64_t ldo_r, int64_t ldo_c, void *workspace,
                        size_t workspace_bytes, void *hip_stream) {
    const int64_t C = num_cand, R = num_req;
    int rc = glm_mlp_check(x_req, R, x_cand, C, cand_to_req, req_cand_offsets, index_flags, num_layers, layers,
                           in_dtype, out_dtype, y_req, y_cand, workspace, workspace_bytes);
    if (rc) return rc;
    hipStream_t s = (hipStream_t)hip_stream;
    int32_t max_nr = 0, max_nc = 0, max_ntot = 0, smax = 1;
    for (int l = 0; l < num_layers; ++l) {
        if (layers[l].n_req_out > max_nr) max_nr = layers[l].n_req_out;
        if (layers[l].n_cand_out > max_nc) max_nc = layers[l].n_cand_out;
        if (layers[l].n_req_out + layers[l].n_cand_out > max_ntot) max_ntot = layers[l].n_req_out + layers[l].n_cand_out;
        int32_t sl = lcb_splits(R, layers[l].n_req_out + layers[l].n_cand_out, layers[l].k_req, in_dtype);
        if (sl > smax) smax = sl;
    }
    Carver cv(workspace);
    LcbWs ws;
    ws.map = (int32_t *)cv.take(sizeof(int32_t) * (size_t)(C > 0 ? C : 1));
    ws.z = (float *)cv.take(sizeof(float) * (size_t)(R > 0 ? R : 1) * (size_t)(max_nc > 0 ? max_nc : 1));
    ws.partial_cap = (size_t)smax * (size_t)(R > 0 ? R : 1) * (size_t)(max_ntot > 0 ? max_ntot : 1);
    ws.partial = (float *)cv.take(sizeof(float) * ws.partial_cap);
    ws.sync_cap = ikbo::lcb_fused_sync_ints(R > 0 ? R : 1, max_ntot > 0 ? max_ntot : 1);
    ws.sync = (int32_t *)cv.take(sizeof(int32_t) * (size_t)ws.sync_cap);
    carve_pads(cv, glm_pad_sizes(C, R, num_layers, layers, in_dtype), &ws);
    void *hr[2] = {nullptr, nullptr}, *hc[2] = {nullptr, nullptr};
    const size_t e = esize(in_dtype);
    if (num_layers > 1)
        for (int b = 0; b < 2; ++b) {
            hr[b] = cv.take(e * (size_t)(R > 0 ? R : 1) * (size_t)(max_nr > 0 ? max_nr : 1));
            hc[b] = cv.take(e * (size_t)(C > 0 ? C : 1) * (size_t)(max_nc > 0 ? max_nc : 1));
        }
    // the offsets, when given, define each candidate's request (as in every entry point)
    const int32_t *map = cand_to_req;
    if (req_cand_offsets) {
        IKBO_HIP(ikbo::launch_offsets_to_map(req_cand_offsets, R, C, ws.map, s));
        map = ws.map;
    }
    const void *xr = x_req, *xc = x_cand;
    for (int l = 0; l < num_layers; ++l) {
        const ikbo_glm_layer &ly = layers[l];
        const bool is_last = l + 1 == num_layers;
        void *yr = is_last ? y_req : hr[l & 1];
        void *yc = is_last ? y_cand : hc[l & 1];
        const int64_t lr = is_last && ldo_r ? ldo_r : ly.n_req_out, lc = is_last && ldo_c ? ldo_c : ly.n_cand_out;
        rc = run_lcb(xr, R, ly.k_req, xc, C, ly.k_cand, map, ly.w_rr, ly.w_cr, ly.w_cc, ly.b_r, ly.b_c, ly.n_req_out,
                     ly.n_cand_out, ly.activation, in_dtype, is_last ? out_dtype : in_dtype, yr, yc, lr, lc, ws, s);
        if (rc) return rc;
        xr = yr;
        xc = yc;
    }
    return ok();
}

int ikbo_glm_mlp_forward(const void *x_req, int64_t num_req, const void *x_cand, int64_t num_cand,
                         const int32_t *cand_to_req, const int32_t *req_cand_offsets, uint32_t index_flags,
                         int32_t num_layers, const ikbo_glm_layer *layers, int32_t in_dtype, int32_t out_dtype,
                         void *y_req, void *y_cand, void *workspace, size_t workspace_bytes, void *hip_stream) {
    return glm_mlp_impl(x_req, num_req, x_cand, num_cand, cand_to_req, req_cand_offsets, index_flags, num_layers, layers,
                        in_dtype, out_dtype, y_req, y_cand, 0, 0, workspace, workspace_bytes, hip_stream);
}

// ---- one DCA interaction layer ------------------------------------------------------------------
size_t ikbo_dca_layer_workspace_size(int64_t num_cand, int64_t num_req, int32_t num_glm_layers,
                                     const ikbo_glm_layer *glm_layers, int64_t seq_rows, int32_t num_heads,
                                     int32_t head_dim, int32_t dtype) {
    if (num_cand < 0 || num_req < 0 || seq_rows < 0 || num_heads <= 0 || head_dim <= 0 || !dtype_ok(dtype)) return 0;
    const size_t g = ikbo_glm_mlp_workspace_size(num_cand, num_req, num_glm_layers, glm_layers, dtype);
    if (g == 0) return 0;
    const size_t kv = align256(esize(dtype) * (size_t)(seq_rows > 0 ? seq_rows : 1) * (size_t)num_heads * (size_t)head_dim);
    const size_t da = ikbo_dca_workspace_size(num_cand, num_req), ra = ikbo_request_attention_workspace_size(num_req);
    return align256(g) + 2 * kv + align256(da > ra ? da : ra);
}

int ikbo_dca_layer_forward(const void *x_req, int64_t num_req, const void *x_cand, int64_t num_cand,
                           const int32_t *cand_to_req, const int32_t *req_cand_offsets, uint32_t index_flags,
                           int32_t num_glm_layers, const ikbo_glm_layer *glm_layers, const void *seq, int64_t seq_rows,
                           int32_t seq_dim, const int32_t *kv_cu_seqlens, int32_t kv_len, const void *w_k_cand,
                           const void *w_v_cand, const void *w_k_req, const void *w_v_req, int32_t q_len,
                           int32_t num_heads, int32_t head_dim, float softmax_scale, int32_t dtype, void *y_req,
                           void *y_cand, void *workspace, size_t workspace_bytes, void *hip_stream) {
    const int64_t C = num_cand, R = num_req;
    if (C < 0 || R < 0 || seq_rows < 0 || seq_dim <= 0 || q_len <= 0 || num_heads <= 0 || head_dim <= 0)
        return fail(IKBO_INVALID_ARGUMENT, "bad sizes (num_cand %lld num_req %lld seq_rows %lld seq_dim %d q_len %d heads %d "
                    "head_dim %d)", (long long)C, (long long)R, (long long)seq_rows, seq_dim, q_len, num_heads, head_dim);
    if (!dtype_ok(dtype)) return fail(IKBO_UNSUPPORTED, "dtype %d", dtype);
    if (num_glm_layers <= 0 || !glm_layers) return fail(IKBO_INVALID_ARGUMENT, "need num_glm_layers >= 1 and a host layer array");
    const int64_t W = (int64_t)q_len * num_heads * head_dim;
    const ikbo_glm_layer &last = glm_layers[num_glm_layers - 1];
    if (last.n_req_out != W || last.n_cand_out != W)
        return fail(IKBO_INVALID_ARGUMENT, "the query generator's last layer must output q_len * num_heads * head_dim = %lld "
                    "columns per group (got %d, %d)", (long long)W, last.n_req_out, last.n_cand_out);
    if (!kv_cu_seqlens && seq_rows != R * (int64_t)kv_len)
        return fail(IKBO_INVALID_ARGUMENT, "seq_rows %lld must be num_req * kv_len = %lld", (long long)seq_rows,
                    (long long)(R * (int64_t)kv_len));
    if (R > 0 && (!y_req || !seq || !w_k_cand || !w_v_cand || !w_k_req || !w_v_req))
        return fail(IKBO_INVALID_ARGUMENT, "y_req, seq and the four K/V weights must be non-NULL when num_req > 0");
    if (C > 0 && !y_cand) return fail(IKBO_INVALID_ARGUMENT, "y_cand is NULL");
    const size_t need = ikbo_dca_layer_workspace_size(C, R, num_glm_layers, glm_layers, seq_rows, num_heads, head_dim, dtype);
    if (!workspace || workspace_bytes < need)
        return fail(IKBO_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes, need);
    if (!aligned16(workspace) || !aligned16(y_req) || !aligned16(y_cand))
        return fail(IKBO_MISALIGNED, "tensor base pointers must be 16-byte aligned");
    if ((W * (int64_t)esize(dtype)) % 16)
        return fail(IKBO_MISALIGNED, "q_len * num_heads * head_dim must keep 16-byte halves of the output rows");
    const size_t e = esize(dtype);
    Carver cv(workspace);
    const size_t g_bytes = ikbo_glm_mlp_workspace_size(C, R, num_glm_layers, glm_layers, dtype);
    void *ws_glm = cv.take(g_bytes);
    const size_t kv_bytes = e * (size_t)(seq_rows > 0 ? seq_rows : 1) * (size_t)num_heads * (size_t)head_dim;
    void *kbuf = cv.take(kv_bytes), *vbuf = cv.take(kv_bytes);
    void *ws_att = (char *)workspace + cv.used;
    const size_t att_bytes = workspace_bytes - cv.used;
    const int64_t ld = 2 * W;                                  // rows of [Q | A]
    char *a_req = (char *)y_req + W * e, *a_cand = (char *)y_cand + W * e;
    // every stage's arguments are checked before the first launch, so an error other than
    // IKBO_HIP_ERROR leaves the outputs untouched
    int rc = glm_mlp_check(x_req, R, x_cand, C, cand_to_req, req_cand_offsets, index_flags, num_glm_layers, glm_layers,
                           dtype, dtype, y_req, y_cand, ws_glm, g_bytes);
    if (rc) return rc;
    if (R > 0) {
        const int32_t hd = num_heads * head_dim;
        rc = kv_project_check(seq, seq_rows, seq_dim, w_k_cand, w_v_cand, hd, dtype, dtype, kbuf, vbuf);
        if (!rc) rc = kv_project_check(seq, seq_rows, seq_dim, w_k_req, w_v_req, hd, dtype, dtype, kbuf, vbuf);
        if (!rc && C > 0)
            rc = dca_validate(y_cand, C, q_len, kbuf, vbuf, R, kv_cu_seqlens, kv_len, cand_to_req, req_cand_offsets,
                              index_flags, num_heads, head_dim, dtype, dtype, a_cand, ws_att, att_bytes);
        if (!rc)
            rc = request_attention_check(y_req, R, q_len, kbuf, vbuf, kv_cu_seqlens, kv_len, num_heads, head_dim, dtype,
                                         dtype, a_req, ws_att, att_bytes);
        if (rc) return rc;
    }
    // Eq. 12: the query generator (LCB_i and MLP_i), its outputs in the left halves
    rc = glm_mlp_impl(x_req, R, x_cand, C, cand_to_req, req_cand_offsets, index_flags, num_glm_layers, glm_layers,
                      dtype, dtype, y_req, y_cand, ld, ld, ws_glm, g_bytes, hip_stream);
    if (rc) return rc;
    if (R == 0) {
        // no request: every candidate's attention half is zero (no valid request)
        if (C > 0) IKBO_HIP(ikbo::launch_zero_uncovered(req_cand_offsets, 0, C, a_cand, W, ld, (int)e, (hipStream_t)hip_stream));
        return ok();
    }
    // Eq. 13, candidate half: K^C, V^C of S once per request, then IKBO-DCA into the right halves
    rc = ikbo_kv_project(seq, seq_rows, seq_dim, w_k_cand, w_v_cand, num_heads * head_dim, dtype, dtype, kbuf, vbuf,
                         hip_stream);
    if (rc) return rc;
    if (C > 0) {
        rc = dca_run(y_cand, C, q_len, kbuf, vbuf, R, kv_cu_seqlens, kv_len, cand_to_req, req_cand_offsets, num_heads,
                     head_dim, softmax_scale, dtype, dtype, a_cand, ws_att, (hipStream_t)hip_stream, ld, ld);
        if (rc) return rc;
    }
    // Eq. 13, request half: K^R, V^R (the same buffers, stream-ordered after the DCA), then A^R
    rc = ikbo_kv_project(seq, seq_rows, seq_dim, w_k_req, w_v_req, num_heads * head_dim, dtype, dtype, kbuf, vbuf,
                         hip_stream);
    if (rc) return rc;
    return request_attention_impl(y_req, R, q_len, kbuf, vbuf, kv_cu_seqlens, kv_len, num_heads, head_dim,
                                  softmax_scale, dtype, dtype, a_req, ws_att, att_bytes, hip_stream, ld, ld);
}

int ikbo_check_index(const int32_t *cand_to_req, const int32_t *req_cand_offsets, int64_t num_cand, int64_t num_req,
                     uint32_t index_flags, uint64_t *d_violations, void *hip_stream) {
    if (num_cand < 0 || num_req < 0) return fail(IKBO_INVALID_ARGUMENT, "negative sizes");
    if (!d_violations) return fail(IKBO_INVALID_ARGUMENT, "d_violations is NULL");
    int rc = check_index_args(cand_to_req, req_cand_offsets, index_flags, 1);
    if (rc) return rc;
    if (((uintptr_t)d_violations & 7u) != 0) return fail(IKBO_MISALIGNED, "d_violations must be 8-byte aligned");
    IKBO_HIP(ikbo::launch_check_index(cand_to_req, req_cand_offsets, num_cand, num_req, index_flags, d_violations,
                                      (hipStream_t)hip_stream));
    return ok();
}

}  // extern "C"
