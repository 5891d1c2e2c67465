// Host-side launch entry points of the IKBO kernels (internal to libikbo; not the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ikbo {

// ---- index prologue (ikbo_index.hip) ----------------------------------------------------------
// Fill n int32 with a value (a kernel, not hipMemsetAsync, so it is safe under graph capture).
hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t value, hipStream_t s);
// p[i] = i for i < n
hipError_t launch_iota_i32(int32_t *p, int64_t n, hipStream_t s);
// counts[r] += 1 for every candidate with 0 <= m[c] < R.
hipError_t launch_histogram(const int32_t *m, int64_t C, int64_t R, int32_t *counts, hipStream_t s);
// From counts (counts != null) or from offsets: writes off_out[0..R] (exclusive scan of counts, or a
// sanitised copy of the offsets), cursor[0..R) = off_out[r] (may be null), and
// tile_start[0..R] = prefix of H * ceil(rows_r / block_m) with rows_r = candidates_r * q_len.
hipError_t launch_scan_tiles(const int32_t *counts, const int32_t *off_in, int64_t R, int64_t C, int32_t q_len,
                             int32_t heads, int32_t block_m, int32_t *off_out, int32_t *cursor,
                             int32_t *tile_start, hipStream_t s);
// Stable grouping of an arbitrary map: perm lists the candidates with a valid request sorted by
// request, each request's candidates in increasing index order, then those without one. scratch
// holds stable_group_scratch_ints(C) int32.
int64_t stable_group_scratch_ints(int64_t C);
hipError_t launch_stable_group(const int32_t *m, int64_t C, int64_t R, int32_t *perm, int32_t *scratch, hipStream_t s);
// Rows of `out` of candidates whose m is outside [0, R) are zeroed (row_elems elements of out_bytes
// each, rows row_stride elements apart).
hipError_t launch_zero_invalid_rows(const int32_t *m, int64_t C, int64_t R, void *out, int64_t row_elems,
                                    int64_t row_stride, int out_bytes, hipStream_t s);
// m_out[c] = r with off[r] <= c < off[r+1] (binary search over a sanitised view), -1 when none.
hipError_t launch_offsets_to_map(const int32_t *off, int64_t R, int64_t C, int32_t *m_out, hipStream_t s);
// Zero rows of `out` for candidates outside [clamp(off[0]), clamp(off[R])) (row_elems elements,
// rows row_stride elements apart).
hipError_t launch_zero_uncovered(const int32_t *off, int64_t R, int64_t C, void *out, int64_t row_elems,
                                 int64_t row_stride, int out_bytes, hipStream_t s);
hipError_t launch_check_index(const int32_t *m, const int32_t *off, int64_t C, int64_t R, uint32_t flags,
                              uint64_t *d_count, hipStream_t s);

// ---- IKBO-DCA (ikbo_dca.hip) -----------------------------------------------------------------
struct DcaArgs {
    const void *q, *k, *v;
    void *out;
    int64_t C, R;
    int32_t Lq, H, D, L;
    const int32_t *kv_cu;       // [R+1] or null (uniform L)
    const int32_t *off;         // [R+1] grouping (sanitised)
    const int32_t *perm;        // [C] or null (identity)
    const int32_t *tile_start;  // [R+1], tile_start[R] = number of tiles
    int64_t grid_tiles;         // upper bound on tile_start[R], sizes the grid
    float scale;
    int32_t in_f32, out_f32;
    int32_t mode;               // bf16 work tile: 0 eight waves (256 rows), 1 one wave (32), 2 four waves (128)
    int64_t q_cs, o_cs;         // elements from one candidate's q (out) rows to the next's (>= Lq H D)
};
// Rows of stacked candidate queries covered by one DCA work tile, per path.
int32_t dca_block_m(int32_t D, int in_f32, int mode);
hipError_t launch_dca(const DcaArgs &a, hipStream_t s);

// ---- GEMMs for IKBO-LCB (ikbo_gemm.hip) ------------------------------------------------------
struct GemmArgs {
    const void *x;              // activations [M, K], row stride ldx elements
    int64_t M;
    int32_t K;
    int64_t ldx;
    const void *w0, *w1;        // weight rows n < n0 from w0 (row n), else from w1 (row n - n0); K contiguous
    int32_t n0, N;
    int32_t in_f32;
    // direct epilogue: out[m, n] = act(acc + bias[n] + (z ? z[map[m], n] : 0)); rows whose map is
    // outside [0, R) are written as zeros when z is set
    const float *bias;
    const float *z;
    int64_t ldz;
    const int32_t *map;
    int64_t R;
    void *out;
    int64_t ldo;
    int32_t out_f32, act;
    // split-K: when partial != null the kernel writes fp32 partial sums [split][M][N] instead
    float *partial;
    int32_t splits;
};
hipError_t launch_gemm(const GemmArgs &a, hipStream_t s);
// Sum the split-K partials in a fixed order, then columns n < n_split go to out0 = act(sum + bias0)
// ([M, n_split] with row stride ld0, out dtype) and columns n >= n_split go to out1 = sum (fp32,
// [M, N - n_split]).
hipError_t launch_splitk_reduce(const float *partial, int32_t splits, int64_t M, int32_t N, int32_t n_split,
                                const float *bias0, int32_t act, void *out0, int32_t out0_f32, int64_t ld0,
                                float *out1, hipStream_t s);
// Zero-padded copy of bf16 rows: dst [rows, kp] (kp a multiple of 8, 16-byte aligned) holds src
// [rows, k] (any k <= kp) in its first k columns and zeros after them.
hipError_t launch_pad_rows_bf16(const void *src, int64_t rows, int32_t k, void *dst, int32_t kp, hipStream_t s);
// Split count the request GEMM uses for an M x N x K problem.
int32_t request_gemm_splits(int64_t M, int32_t N, int32_t K, int in_f32);

// One persistent launch for an LCB layer (bf16): the request GEMM's split-K tiles are taken first
// from a device-wide counter; the last split of a request tile to finish sums the partials in
// split order and applies the request-group epilogue (out0 = act(sum + bias0) for columns below
// n_split, Z = sum above), then releases that tile's ready flag. Candidate tiles are taken next
// from one counter per XCD; each runs its main loop, then acquires the ready flags of the request
// tiles holding its Z columns before the fused epilogue. Results equal launch_gemm +
// launch_splitk_reduce + launch_gemm bit for bit.
struct LcbFusedArgs {
    GemmArgs req;           // request GEMM: partial = [splits][R][N] fp32, splits >= 1
    GemmArgs cand;          // candidate GEMM: z = the request GEMM's Z output
    int32_t n_split;        // request columns below n_split are Y_r, the rest Z
    const float *bias0;
    int32_t act;
    void *out0;             // Y_r [R, n_split] or null when n_split == 0
    int32_t out0_f32;
    int32_t *sync;          // lcb_fused_sync_ints(...) int32, zeroed by launch_lcb_fused
    int64_t wait_ticks;     // bound on each flag wait, in ticks of the device's constant wall clock;
                            // a wait that runs out sets sync[9] and poisons the tile's output with NaN
    int32_t publish;        // 1: request tiles set their ready flags; 0 (a test of the bounded
                            // waits, set from the host): they never do, so every wait gives up
};
// ticks of the device's constant wall clock (wall_clock64) in the given number of seconds
int64_t wall_clock_ticks(double seconds);
// int32 words of synchronisation state for a request GEMM of M rows and N columns
int64_t lcb_fused_sync_ints(int64_t M, int32_t N);
// whether launch_lcb_fused supports these two GEMMs (bf16 with direct copies)
bool lcb_fused_supported(const GemmArgs &req, const GemmArgs &cand);
hipError_t launch_lcb_fused(const LcbFusedArgs &f, hipStream_t s);

// ---- GLM factorization machine (ikbo_fm.hip) -----------------------------------------------------
struct FmArgs {
    const void *x_r, *x_c;      // [R, n_r, d], [C, n_c, d]
    void *y_r, *y_c;            // [R, n_r, n_r] or null, [C, n_c, n_r + n_c]
    int64_t R, C;
    int32_t n_r, n_c, d;
    const int32_t *map, *off;   // candidate -> request; offsets [R + 1] take precedence when set
    int32_t in_f32, out_f32;
    int64_t chunk;              // items per wave (set by launch_fm)
};
// whether launch_fm takes the MFMA path (bf16, d in {32, 64, 128}, n_r and n_c <= 64)
bool fm_mfma_supported(const FmArgs &a);
hipError_t launch_fm(const FmArgs &a, hipStream_t s);

// ---- LCB, embedding-matrix form, with the group-local norm (ikbo_lcbe.hip) -----------------------
struct LcbeArgs {
    const void *x_r, *x_c;              // [R, n_r, d], [C, n_c, d]
    const void *w_rr, *w_cr, *w_cc;     // [k_r, n_r], [k_c, n_r], [k_c, n_c]
    const float *g_r, *b_r, *g_c, *b_c; // [d] each, or null (gamma 1, beta 0)
    float *z;                           // [R, k_c, d] fp32: W_CR X^R once per request
    void *y_r, *y_c;                    // [R, k_r, d] or null, [C, k_c, d]
    int64_t R, C;
    int32_t n_r, n_c, k_r, k_c, d;
    const int32_t *map, *off;           // candidate -> request; offsets [R + 1] take precedence when set
    int32_t in_f32, out_f32, norm;      // norm: 0 none, 1 LayerNorm, 2 RMSNorm (per embedding row)
    float eps;
    int64_t chunk;                      // candidates per wave (set by launch_lcbe)
};
constexpr int kLcbeMaxDim = 256;
// whether launch_lcbe takes the MFMA path for the candidates (bf16, d in {32, 64, 128},
// n_c and k_c <= 64)
bool lcbe_mfma_supported(const LcbeArgs &a);
hipError_t launch_lcbe(const LcbeArgs &a, hipStream_t s);

}  // namespace ikbo
