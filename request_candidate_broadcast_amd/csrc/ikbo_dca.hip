// IKBO-DCA kernels: candidate-side cross attention (ROCS Sec. 3.2, Eq. 13, the A^C term) that
// reads K and V at the request batch size and resolves each candidate's request in the kernel
// (Sec. 4.3.1). All candidates of a request read the same physical K/V rows.
//
// Work decomposition (MI355X design, not the pages' Hopper one):
//  - The query rows of request r are the rows of its candidates, each with Lq tokens, stacked in
//    candidate order: row i of request r is token i % Lq of candidate off[r] + i / Lq (through
//    perm when the map was not grouped). Stacking candidates fills the MFMA tiles even when one
//    candidate has few query tokens (the pages make the same point for short candidate queries,
//    Sec. 4.3.2).
//  - A work tile is (request r, head h, block of BLOCK_M stacked rows). Tiles are numbered
//    request-major, then head, then row block, so the tiles that stream the same (r, h) K/V
//    are consecutive; each XCD takes one contiguous range of tile numbers (xcd_tile), so those
//    tiles run together on one XCD and share its L2 (the MI355X form of the grid reorder of
//    Sec. 4.3.1).
//  - bf16 path: 8 waves x 32 query rows. The K/V tile of BLOCK_N keys is staged once in LDS
//    (double-buffered) and read by all 8 waves. Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16 so each lane owns one query column: the softmax max is a per-lane
//    reduction plus one exchange between the two 32-lane halves, and the per-lane partial sums are
//    combined once at the end. The accumulator of S^T is reused in registers as the B operand of
//    O^T += V^T P^T; V^T comes from LDS through ds_read_b64_tr_b16, which transposes 16-bit data
//    across each 16-lane group.
//  - Online softmax in the exp2 domain with the softmax scale folded into one FMA, and lazy
//    rescaling: a query's reference max is only raised when the tile max exceeds it by more than
//    kTau (log2 units), so most tiles skip the O rescale; the final O / l is exact in real
//    arithmetic for any reference value. The decision is per query, so a row's result does not
//    depend on which other rows share its tile.
#include "ikbo_device.h"
#include "ikbo_launch.h"

#include <math.h>

#include <type_traits>

namespace ikbo {

namespace {


__device__ __forceinline__ int64_t clamp64(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Locate a tile: largest r with tile_start[r] <= t (tile_start[0] = 0, non-decreasing).
__device__ __forceinline__ int64_t find_request(const int32_t *tile_start, int64_t R, int64_t t) {
    int64_t lo = 0, hi = R;
    while (hi - lo > 1) {
        int64_t mid = (lo + hi) >> 1;
        if (tile_start[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

// LDS swizzles (16-byte chunk index XOR a function of the key row) so that the MFMA operand
// reads of K (ds_read_b128, 32 consecutive keys at one chunk) and the transposed reads of V
// (ds_read_b64_tr_b16, 4 consecutive keys x 2 chunks per 16 lanes) hit distinct banks.
template <int D>
__device__ __forceinline__ int swz_k(int key) { return D == 128 ? (key & 15) : ((key >> 1) & 7); }
__device__ __forceinline__ int swz_v(int key) { return (key & 3) << 1; }

struct TileInfo {
    int64_t r, h, qb, rows, cand0, kv_row0, Lr;
};

__device__ __forceinline__ bool decode_tile(const DcaArgs &a, int block_m, TileInfo &ti) {
    const int64_t total = a.tile_start[a.R];
    const int64_t t = xcd_tile(blockIdx.x, total);
    if (t < 0) return false;
    const int64_t r = find_request(a.tile_start, a.R, t);
    const int64_t c0 = clamp64(a.off[r], 0, a.C);
    const int64_t c1 = clamp64(a.off[r + 1], c0, a.C);
    const int64_t rows = (c1 - c0) * a.Lq;
    const int64_t nqb = (rows + block_m - 1) / block_m;
    if (nqb == 0) return false;
    const int64_t local = t - a.tile_start[r];
    ti.r = r;
    ti.h = local / nqb;
    ti.qb = local % nqb;
    if (ti.h >= a.H) return false;
    ti.rows = rows;
    ti.cand0 = c0;
    if (a.kv_cu) {
        ti.kv_row0 = a.kv_cu[r];
        ti.Lr = (int64_t)a.kv_cu[r + 1] - a.kv_cu[r];
    } else {
        ti.kv_row0 = r * (int64_t)a.L;
        ti.Lr = a.L;
    }
    if (ti.Lr < 0) ti.Lr = 0;
    return true;
}

// Candidate index and token of stacked row `srow` of a tile.
__device__ __forceinline__ void row_source(const DcaArgs &a, const TileInfo &ti, int64_t srow, int64_t &cand, int &tok) {
    int64_t cl = srow / a.Lq;
    tok = (int)(srow - cl * a.Lq);
    cand = ti.cand0 + cl;
    if (a.perm) cand = a.perm[cand];
}

// ----------------------------------------------------------------------------------------------
// bf16 inputs, D in {64, 128}, MFMA path.
//
// Template parameters: NW waves per workgroup, NG groups of 32 query columns per wave, NKB
// 32-key blocks per K/V tile, NBUF LDS stages, LATE = copy the next tiles in after this tile's
// V fragments are read (else at the top of the tile). With NG = 2 the work of one tile is
// ordered so the softmax VALU work of one group overlaps the MFMA work of the other
// (scheduling fences keep the phases apart):
//   A: S0 = K Q0^T                     (MFMA)
//   B: S1 = K Q1^T        | softmax(S0) (MFMA | VALU)
//   C: O0 += V^T P0^T     | softmax(S1)
//   D: O1 += V^T P1^T
// K fragments are read from LDS once per tile and used by every group, likewise the V^T
// fragments. K/V tiles are copied global -> LDS directly (no register staging); one barrier per
// tile.

// Cross-half combine: v_permlane32_swap exchanges the two 32-lane halves, so the max (or sum) of
// both results is the value over lanes l and l ^ 32.
__device__ __forceinline__ float half_swap_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Masks keys at or past L_r in the last tile: s[kb][j] holds key kb*32 + 8*(j/4) + 4*half + j%4.
template <int NKB>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[NKB], int rem, int half) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (kb * 32 + 8 * (j >> 2) + 4 * half + (j & 3) >= rem) s[kb][j] = -INFINITY;
}

// Max over the lane's scores of one tile, then over the two 32-lane halves (one query column).
template <int NKB>
__device__ __forceinline__ float tile_max(const f32x16 (&s)[NKB]) {
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int j = (kb == 0 ? 2 : 0); j < 16; ++j) mx = fmaxf(mx, s[kb][j]);
    return half_swap_max(mx);
}

// p = 2^(s * scale * log2(e) - m_ref) against a fixed per-query reference; accumulates the row
// sum and packs the bf16 B operands of the PV MFMAs.
template <int NKB>
__device__ __forceinline__ void exp_tile(f32x16 (&s)[NKB], bf16x8 (&pb)[NKB][2], float &l, float cl2, float mneg) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][j], cl2, mneg));
            s[kb][j] = p;
            l += p;
        }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[kb][u][e] = (__bf16)s[kb][8 * u + e];
}

template <int D, int NW, int NG, int NKB, int NBUF, bool LATE>
__global__ __launch_bounds__(NW * 64) void dca_bf16_kernel(DcaArgs a) {
    constexpr int BN = NKB * 32;                       // keys per tile
    constexpr int BM = NW * NG * 32;                   // stacked query rows per workgroup
    constexpr int CPR = D / 8;                         // 16-byte chunks per key row
    constexpr int kTileChunks = BN * CPR;              // chunks per K (or V) tile
    constexpr int kThreads = NW * 64;
    constexpr int kLoadPasses = kTileChunks / kThreads;
    static_assert(kTileChunks % kThreads == 0, "tile load must split evenly");
    constexpr int kCopiesPerTile = 2 * kLoadPasses;    // global -> LDS instructions per tile (K and V)
    static_assert(NBUF == 2 || (NBUF == 3 && LATE), "three stages are filled late");
    constexpr int KS = D / 16;                         // k16 steps over the head dim
    constexpr int DB = D / 32;                         // 32-row blocks of O^T

    __shared__ uint4 smem[NBUF][2][kTileChunks];       // [stage][K=0 / V=1][chunk]

    TileInfo ti;
    if (!decode_tile(a, BM, ti)) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, half = lane >> 5;
    const int64_t HD = (int64_t)a.H * D;

    // ---- the lane's query rows (one column of S^T per group) ----
    bool rvalid[NG];
    int64_t cand[NG];
    int tok[NG];
    bf16x8 qf[NG][KS];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int64_t srow = ti.qb * BM + wave * (NG * 32) + g * 32 + l32;
        rvalid[g] = srow < ti.rows;
        cand[g] = 0;
        tok[g] = 0;
        if (rvalid[g]) row_source(a, ti, srow, cand[g], tok[g]);
        const uint16_t *qp = (const uint16_t *)a.q + ((cand[g] * a.Lq + tok[g]) * HD + ti.h * D) + half * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 u = rvalid[g] ? *(const uint4 *)(qp + ks * 16) : make_uint4(0, 0, 0, 0);
            qf[g][ks] = __builtin_bit_cast(bf16x8, u);
        }
    }

    // ---- K/V tile copies: global -> LDS direct ----
    // Each wave instruction fills 64 consecutive 16-byte LDS slots; the lane that fills slot
    // (key, c') reads chunk c' ^ swizzle(key) of that key row, which realises the swizzled layout.
    // Rows past L_r are read from row L_r - 1 instead: their scores are masked to -inf, so they
    // get weight exactly 0 and their finite values do not matter.
    const uint16_t *kbase = (const uint16_t *)a.k + ti.kv_row0 * HD + ti.h * D;
    const uint16_t *vbase = (const uint16_t *)a.v + ti.kv_row0 * HD + ti.h * D;
    const int Lr = (int)ti.Lr;
    auto dma = [&](int n0, int st) {
#pragma unroll
        for (int p = 0; p < kLoadPasses; ++p) {
            const int slot0 = p * kThreads + wave * 64;
            const int slot = slot0 + lane, key = slot / CPR, chp = slot % CPR;
            const int row = min(n0 + key, Lr - 1);
            const int64_t roff = (int64_t)row * HD;
            copy16_to_lds(kbase + roff + (chp ^ swz_k<D>(key)) * 8, &smem[st][0][slot0]);
            copy16_to_lds(vbase + roff + (chp ^ swz_v(key)) * 8, &smem[st][1][slot0]);
        }
    };

    const float cl2 = a.scale * 1.4426950408889634f;

    // lane constants of the transposed V read
    const int g16 = lane >> 4, s16 = lane & 15;
    const int tr_dsub = (g16 & 1) * 16 + 4 * (s16 & 3);
    const int tr_key = 4 * (g16 >> 1) + (s16 >> 2);

    // K fragments of one tile (A operands of S^T = K Q^T)
    auto k_frags = [&](int st, bf16x8 (&kf)[KS][NKB]) {
        const uint4 *ks_lds = smem[st][0];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int key = kb * 32 + l32, ch = ks * 2 + half;
                kf[ks][kb] = __builtin_bit_cast(bf16x8, ks_lds[key * CPR + (ch ^ swz_k<D>(key))]);
            }
    };
    auto s_tile = [&](const bf16x8 (&kf)[KS][NKB], const bf16x8 (&q)[KS], f32x16 (&s)[NKB]) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) s[kb][j] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s[kb] = mfma_32x32x16_bf16(kf[ks][kb], q[ks], s[kb]);
    };
    // V^T fragments of one tile (A operands of O^T += V^T P^T) through the transposing LDS read
    auto v_frags = [&](int st, bf16x8 (&vf)[DB][NKB][2]) {
        const char *vs_lds = (const char *)smem[st][1];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int dcol = db * 32 + tr_dsub;
            const int chunk = dcol >> 3, sub = (dcol & 7) * 2;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int key0 = kb * 32 + 16 * u + tr_key;
                    const int key1 = key0 + 8;
                    i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(vs_lds + (key0 * CPR + (chunk ^ swz_v(key0))) * 16 + sub));
                    i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(vs_lds + (key1 * CPR + (chunk ^ swz_v(key1))) * 16 + sub));
                    typedef short i16x8 __attribute__((ext_vector_type(8)));
                    vf[db][kb][u] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
                }
        }
    };
    auto pv_tile = [&](const bf16x8 (&vf)[DB][NKB][2], const bf16x8 (&pb)[NKB][2], f32x16 (&o)[DB]) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int u = 0; u < 2; ++u) o[db] = mfma_32x32x16_bf16(vf[db][kb][u], pb[kb][u], o[db]);
    };

    const int ntiles = (Lr + BN - 1) / BN;
    const bool ragged = (Lr % BN) != 0;

    // ---- one pass over the keys ----
    // Softmax weights are taken against a fixed per-query reference m_ref (no running rescale of
    // O): O' = sum_j 2^(s_j c - m_ref) v_j and l' = sum_j 2^(s_j c - m_ref) give O = O' / l' exactly
    // in real arithmetic for any m_ref. With INIT the reference is the max of the first tile;
    // later tiles may exceed it, and a query whose sums overflow is redone with its true max.
    // With MAXONLY the pass only computes scores and leaves each query's exact max in m_ref.
    f32x16 o[NG][DB];
    float l[NG], mref[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        l[g] = 0.0f;
        mref[g] = 0.0f;
    }
    auto pass = [&](auto init, auto maxonly) {
        constexpr bool INIT = decltype(init)::value;
        constexpr bool MAXONLY = decltype(maxonly)::value;
        float mx[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            l[g] = 0.0f;
            mx[g] = -INFINITY;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) o[g][db][j] = 0.0f;
        }
        // prologue: the first tile (and with three stages the second) in flight, the first landed
        if (ntiles > 0) dma(0, 0);
        if (NBUF == 3 && ntiles > 1) {
            dma(BN, 1);
            wait_vmcnt<kCopiesPerTile>();
        } else {
            wait_all();
        }
        __syncthreads();
        auto tile = [&](int it, auto first, auto masked) {
            constexpr bool FIRST = decltype(first)::value;
            constexpr bool MASK = decltype(masked)::value;
            const int st = it % NBUF;
            const int n0 = it * BN;
            const int ahead = it + NBUF - 1;               // the tile copied in during this one
            const bool copy = ahead < ntiles;
            if (!LATE && copy) dma(ahead * BN, ahead % NBUF);
            f32x16 s[NG][NKB];
            bf16x8 p[NG][NKB][2];
            bf16x8 kf[KS][NKB];
            bf16x8 vf[DB][NKB][2];
            k_frags(st, kf);
            auto softmax = [&](int g) {
                if (MASK) mask_tile<NKB>(s[g], Lr - n0, half);
                if (MAXONLY) {
                    mx[g] = fmaxf(mx[g], tile_max<NKB>(s[g]));
                } else {
                    if (INIT && FIRST) mref[g] = tile_max<NKB>(s[g]) * cl2;
                    exp_tile<NKB>(s[g], p[g], l[g], cl2, -mref[g]);
                }
            };
            s_tile(kf, qf[0], s[0]);                                         // A
            sched_fence();
            if (NG == 2) {
                s_tile(kf, qf[NG - 1], s[NG - 1]);                           // B
                softmax(0);
                sched_fence();
            } else {
                softmax(0);
            }
            if (!MAXONLY) v_frags(st, vf);
            if (LATE && copy) dma(ahead * BN, ahead % NBUF);
            if (!MAXONLY) {
                pv_tile(vf, p[0], o[0]);                                     // C
                if (NG == 2) {
                    softmax(NG - 1);
                    sched_fence();
                    pv_tile(vf, p[NG - 1], o[NG - 1]);                       // D
                }
            } else if (NG == 2) {
                softmax(NG - 1);
            }
            // the next tile must have landed; with three stages the one after may stay in flight
            if (NBUF == 3 && it + 2 < ntiles) wait_vmcnt<kCopiesPerTile>();
            else wait_vmcnt<0>();
            __syncthreads();
        };
        const std::true_type T;
        const std::false_type F;
        if (ntiles == 1) {
            if (ragged) tile(0, T, T); else tile(0, T, F);
        } else if (ntiles > 1) {
            tile(0, T, F);
            for (int it = 1; it + 1 < ntiles; ++it) tile(it, F, F);
            if (ragged) tile(ntiles - 1, F, T); else tile(ntiles - 1, F, F);
        }
        if (MAXONLY) {
#pragma unroll
            for (int g = 0; g < NG; ++g) mref[g] = mx[g] * cl2;
        }
    };

    pass(std::true_type(), std::false_type());

    // ---- overflow check: redo the tile for the queries whose sums left the fp32 range ----
    bool bad[NG];
    bool any_bad = false;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        bool b = !(half_swap_sum(l[g]) < INFINITY);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) b |= !(fabsf(o[g][db][j]) < INFINITY);
        // a query column lives in lanes l and l ^ 32: both halves must take the same decision
        bad[g] = half_swap_max(b ? 1.0f : 0.0f) > 0.0f && rvalid[g];
        any_bad |= bad[g];
    }
    if (__syncthreads_or(any_bad)) {
        float keep[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) keep[g] = mref[g];
        pass(std::false_type(), std::true_type());               // exact max per query
#pragma unroll
        for (int g = 0; g < NG; ++g) mref[g] = bad[g] ? mref[g] : keep[g];
        pass(std::false_type(), std::false_type());              // redo; unchanged queries repeat bit for bit
    }

    // ---- epilogue: O = O^T / l, store rows ----
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const float l_tot = half_swap_sum(l[g]);
        if (!rvalid[g]) continue;
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        const int64_t obase = (cand[g] * a.Lq + tok[g]) * HD + ti.h * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d = db * 32 + 8 * jj + 4 * half;
                const float v0 = o[g][db][4 * jj + 0] * inv, v1 = o[g][db][4 * jj + 1] * inv;
                const float v2 = o[g][db][4 * jj + 2] * inv, v3 = o[g][db][4 * jj + 3] * inv;
                if (a.out_f32) {
                    *(float4 *)((float *)a.out + obase + d) = make_float4(v0, v1, v2, v3);
                } else {
                    *(uint2 *)((uint16_t *)a.out + obase + d) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
                }
            }
    }
}

// The configuration the library launches, per head dim.
template <int D>
struct DcaBf16Config {
    static constexpr int NW = 4, NG = 2, NKB = 2, NBUF = 3;
    static constexpr bool LATE = true;
    static constexpr int BM = NW * NG * 32;
};

// ----------------------------------------------------------------------------------------------
// fp32 inputs, any D that is a multiple of 4 up to 128. 16 query rows per workgroup, 16 lanes
// per row; each lane owns the head dims e = sub, sub + 16, ... Exact online softmax with expf.
constexpr int kF32Rows = 16;
constexpr int kF32Keys = 32;

__global__ __launch_bounds__(256) void dca_f32_kernel(DcaArgs a) {
    __shared__ float ks[kF32Keys][128];
    __shared__ float vs[kF32Keys][128];
    TileInfo ti;
    if (!decode_tile(a, kF32Rows, ti)) return;
    const int D = a.D;
    const int tid = threadIdx.x, qi = tid >> 4, sub = tid & 15;
    const int64_t HD = (int64_t)a.H * D;
    const int64_t srow = ti.qb * kF32Rows + qi;
    const bool rvalid = srow < ti.rows;
    int64_t cand = 0;
    int tok = 0;
    if (rvalid) row_source(a, ti, srow, cand, tok);
    const float *qp = (const float *)a.q + (cand * a.Lq + tok) * HD + ti.h * D;
    float qv[8], ov[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int e = sub + 16 * k;
        qv[k] = (rvalid && e < D) ? qp[e] : 0.0f;
        ov[k] = 0.0f;
    }
    const float *kb = (const float *)a.k + ti.kv_row0 * HD + ti.h * D;
    const float *vb = (const float *)a.v + ti.kv_row0 * HD + ti.h * D;
    float m_run = -INFINITY, l_run = 0.0f;
    for (int64_t n0 = 0; n0 < ti.Lr; n0 += kF32Keys) {
        __syncthreads();
        for (int i = tid; i < kF32Keys * D; i += 256) {
            const int key = i / D, e = i % D;
            const bool ok = n0 + key < ti.Lr;
            ks[key][e] = ok ? kb[(n0 + key) * HD + e] : 0.0f;
            vs[key][e] = ok ? vb[(n0 + key) * HD + e] : 0.0f;
        }
        __syncthreads();
        float sc[kF32Keys];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < kF32Keys; ++j) {
            float part = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int e = sub + 16 * k;
                if (e < D) part = __builtin_fmaf(qv[k], ks[j][e], part);
            }
            part += __shfl_xor(part, 8, 16);
            part += __shfl_xor(part, 4, 16);
            part += __shfl_xor(part, 2, 16);
            part += __shfl_xor(part, 1, 16);
            sc[j] = (n0 + j < ti.Lr) ? part * a.scale : -INFINITY;
            mx = fmaxf(mx, sc[j]);
        }
        const float m_new = fmaxf(m_run, mx);
        const float alpha = expf(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int k = 0; k < 8; ++k) ov[k] *= alpha;
#pragma unroll
        for (int j = 0; j < kF32Keys; ++j) {
            const float p = expf(sc[j] - m_new);
            l_run += p;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int e = sub + 16 * k;
                if (e < D) ov[k] = __builtin_fmaf(p, vs[j][e], ov[k]);
            }
        }
    }
    if (!rvalid) return;
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    const int64_t obase = (cand * a.Lq + tok) * HD + ti.h * D;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int e = sub + 16 * k;
        if (e < D) {
            const float val = ov[k] * inv;
            if (a.out_f32) ((float *)a.out)[obase + e] = val;
            else ((uint16_t *)a.out)[obase + e] = f32_to_bf16(val);
        }
    }
}

}  // namespace

int32_t dca_block_m(int32_t D, int in_f32) {
    if (in_f32) return kF32Rows;
    return D == 128 ? DcaBf16Config<128>::BM : DcaBf16Config<64>::BM;
}

hipError_t launch_dca(const DcaArgs &a, hipStream_t s) {
    if (a.grid_tiles <= 0) return hipSuccess;
    const int64_t grid = ((a.grid_tiles + kNumXcd - 1) / kNumXcd) * kNumXcd;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (a.in_f32) {
        hipLaunchKernelGGL(dca_f32_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
    } else if (a.D == 128) {
        using C = DcaBf16Config<128>;
        hipLaunchKernelGGL((dca_bf16_kernel<128, C::NW, C::NG, C::NKB, C::NBUF, C::LATE>), dim3((unsigned)grid),
                           dim3(C::NW * 64), 0, s, a);
    } else if (a.D == 64) {
        using C = DcaBf16Config<64>;
        hipLaunchKernelGGL((dca_bf16_kernel<64, C::NW, C::NG, C::NKB, C::NBUF, C::LATE>), dim3((unsigned)grid),
                           dim3(C::NW * 64), 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ikbo
