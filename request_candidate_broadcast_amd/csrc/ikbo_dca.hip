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
//    and read by all 8 waves. Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16 so each lane owns one query column: the softmax max is a per-lane
//    reduction plus one exchange between the two 32-lane halves, and the per-lane partial sums are
//    combined once at the end. The bf16 weights P^T are the B operand of O^T += V^T P^T; V^T comes
//    from LDS through ds_read_b64_tr_b16, which transposes 16-bit data across each 16-lane group.
//  - Softmax in the exp2 domain with the softmax scale folded into one FMA, against a fixed
//    per-query reference (the max of the first tile), so O is never rescaled; O / l is exact in
//    real arithmetic for any reference. The scores stay fp32 products of the bf16 inputs: folding
//    the scale into bf16 Q fragments instead would save the FMA but round every score by up to
//    2^-9 of its size, which large keys turn into errors past the accuracy bar. A query whose sums
//    leave the fp32 range is redone with its exact max (a rare second and third pass over its
//    keys); the decision is per query, so a row's result does not depend on which other rows
//    share its tile.
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
// Template parameters: NW waves per workgroup, each owning 32 query rows (one column of S^T per
// lane); NKB 32-key blocks per K/V tile; KPD / VPD how many k16 steps of K fragments / 32-dim
// blocks of V^T fragments are read ahead of the MFMAs that use them. Two LDS stages. Eight
// waves put two on every SIMD, so the softmax VALU work of one overlaps the MFMAs of the other in
// hardware; streaming the fragments from LDS step by step (instead of holding a whole tile) keeps
// a wave within the 256 registers that two waves per SIMD leave it. One barrier per tile.
//
// LDS layout: K rows are padded to D*2 + 16 bytes, so 16 consecutive keys read at one 16-byte
// column fall in 16 distinct bank groups without a swizzle, and every K operand read is one
// per-lane base plus a compile-time offset. V rows are padded to D*2 + 64 bytes, so the transposed
// reads (4 keys x 64 bytes per 32 lanes) hit distinct banks, again base plus constant. Tiles are
// copied with buffer loads straight into LDS: each wave instruction fills 64 consecutive 16-byte
// slots, so a lane's source is the (key, column) of its slot. Pad slots, and keys at or past L_r
// (the buffer range covers the request's rows only), read as zeros without touching memory.
// Each stage is its own LDS variable and stage indices are compile-time constants (the tile loop
// is unrolled by the stage count), so reads of one stage are not held back by copies into another.

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

// Masks the keys at or past `rem` of one 32-key block: s[j] holds key 8*(j/4) + 4*half + j%4.
__device__ __forceinline__ void mask_block(f32x16 &s, int rem, int half) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
        if (8 * (j >> 2) + 4 * half + (j & 3) >= rem) s[j] = -INFINITY;
}

// Max over the lane's scores of one 32-key block, then over the two 32-lane halves (one query).
__device__ __forceinline__ float block_max(const f32x16 &s) {
    float mx = fmaxf(s[0], s[1]);
#pragma unroll
    for (int j = 2; j < 16; ++j) mx = fmaxf(mx, s[j]);
    return half_swap_max(mx);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// p = 2^(s * scale * log2(e) - m_ref) for one 32-key block against a fixed per-query reference;
// packs the bf16 B operands of the PV MFMAs and adds the packed (rounded) weights to the row sum,
// so the sum normalises exactly the weights the PV MFMAs use.
__device__ __forceinline__ void exp_block(f32x16 &s, bf16x8 (&pb)[2], float &l, float cl2, float mneg) {
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], cl2, mneg));
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            // a pair at a time: one v_cvt_pk_bf16_f32 per two weights
            const bf16x2 pr = cvt_bf16x2(s[8 * u + e], s[8 * u + e + 1]);
            pb[u][e] = pr[0];
            pb[u][e + 1] = pr[1];
            l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
        }
    }
}

// Occupancy: at least two waves per SIMD for the multi-wave tiles; the four-wave d = 64 tile (the
// ragged, short-request workloads, with little MFMA work per key tile) is held to 168 registers so
// that three workgroups share a CU, which measured faster than two.
template <int D, int NW>
constexpr int dca_min_waves() { return NW == 4 && D == 64 ? 3 : NW >= 4 ? 2 : 1; }

template <int D, int NW, int NKB, int KPD, int VPD>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(dca_min_waves<D, NW>(), 8))) void dca_bf16_kernel(DcaArgs a) {
    constexpr int BN = NKB * 32;                       // keys per tile
    constexpr int BM = NW * 32;                        // stacked query rows per workgroup
    constexpr int CPR = D / 8;                         // 16-byte chunks per key row
    constexpr int KSR = CPR + 1, VSR = CPR + 4;        // 16-byte slots per padded K / V row
    constexpr int VROW = VSR * 16;                     // bytes per padded V row
    // wave instructions per K / V tile (64 slots each); wave w issues instructions w, w + NW, ...
    constexpr int kInstrK = (BN * KSR + 63) / 64, kInstrV = (BN * VSR + 63) / 64;
    constexpr int kPassK = (kInstrK + NW - 1) / NW, kPassV = (kInstrV + NW - 1) / NW;
    constexpr int kCopiesPerTile = kPassK + kPassV;     // at most, per wave
    constexpr int NBUF = 2;     // LDS stages: the copies of the next tile are waited for at each barrier
    constexpr int KS = D / 16, DB = D / 32;
    constexpr uint32_t kOutOfRange = 0x80000000u;

    __shared__ uint4 k_s0[kInstrK * 64], k_s1[kInstrK * 64];
    __shared__ uint4 v_s0[kInstrV * 64], v_s1[kInstrV * 64];
    auto k_lds = [&](auto S) __attribute__((always_inline)) -> uint4 * {
        if constexpr (decltype(S)::value == 0) return k_s0;
        else return k_s1;
    };
    auto v_lds = [&](auto S) __attribute__((always_inline)) -> uint4 * {
        if constexpr (decltype(S)::value == 0) return v_s0;
        else return v_s1;
    };

    TileInfo ti;
    if (!decode_tile(a, BM, ti)) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, half = lane >> 5;
    const int64_t HD = (int64_t)a.H * D;

    const float cl2 = a.scale * 1.4426950408889634f;

    // ---- the lane's query row (one column of S^T) ----
    const int64_t srow = ti.qb * BM + wave * 32 + l32;
    const bool rvalid = srow < ti.rows;
    // four-wave tiles (short requests): a wave none of whose 32 rows is in the request (the
    // request's last, partly filled work tile) skips the score, softmax and PV work of the main
    // pass and only copies and meets the barriers (the eight-wave tile gains nothing from it)
    const bool active = NW != 4 || __builtin_amdgcn_readfirstlane((int)(ti.qb * BM + wave * 32 < ti.rows)) != 0;
    int64_t cand = 0;
    int tok = 0;
    if (rvalid) row_source(a, ti, srow, cand, tok);
    bf16x8 qf[KS];
    {
        const uint16_t *qp = (const uint16_t *)a.q + (cand * a.q_cs + tok * HD + ti.h * D) + half * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 u = rvalid ? *(const uint4 *)(qp + ks * 16) : make_uint4(0, 0, 0, 0);
            qf[ks] = __builtin_bit_cast(bf16x8, u);
        }
    }

    // ---- K/V tile copies: buffer -> LDS ----
    const uint16_t *kbase = uniform_ptr((const uint16_t *)a.k + ti.kv_row0 * HD + ti.h * D);
    const uint16_t *vbase = uniform_ptr((const uint16_t *)a.v + ti.kv_row0 * HD + ti.h * D);
    const int Lr = __builtin_amdgcn_readfirstlane((int)ti.Lr);
    uint32_t koff[kPassK], voff[kPassV];
#pragma unroll
    for (int p = 0; p < kPassK; ++p) {
        const int slot = (p * NW + wave) * 64 + lane, key = slot / KSR, c = slot % KSR;
        koff[p] = key < BN && c < CPR ? (uint32_t)(key * HD + c * 8) * 2 : kOutOfRange;
    }
#pragma unroll
    for (int p = 0; p < kPassV; ++p) {
        const int slot = (p * NW + wave) * 64 + lane, key = slot / VSR, c = slot % VSR;
        voff[p] = key < BN && c < CPR ? (uint32_t)(key * HD + c * 8) * 2 : kOutOfRange;
    }
    // Buffer resources over the request's K / V rows (keys at or past L_r read as zeros); the
    // tile's first row goes into the lane offsets. The host keeps L_r * H * D * 2 below 2^31.
    const uint32_t req_bytes = (uint32_t)((int64_t)Lr * HD * 2);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase, req_bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase, req_bytes);
    // copy number c (K passes, then V passes) of the tile of keys n0 .. n0 + BN - 1 into stage S
    auto copy = [&](int c, int n0, auto S) __attribute__((always_inline)) {
        const uint32_t toff = (uint32_t)min((int64_t)n0 * HD * 2, (int64_t)0x7fff0000);
        if (c < kPassK) {
            if (c * NW + wave < kInstrK) buffer_copy16_to_lds(kr, koff[c] + toff, k_lds(S) + (c * NW + wave) * 64);
        } else {
            const int p = c - kPassK;
            if (p * NW + wave < kInstrV) buffer_copy16_to_lds(vr, voff[p] + toff, v_lds(S) + (p * NW + wave) * 64);
        }
    };
    auto dma = [&](int n0, auto S) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < kCopiesPerTile; ++c) copy(c, n0, S);
    };

    const int g16 = lane >> 4, s16 = lane & 15;
    const int tr_dsub = (g16 & 1) * 16 + 4 * (s16 & 3);
    const int tr_key = 4 * (g16 >> 1) + (s16 >> 2);
    const int k_lane = l32 * KSR + half;
    const int v_lane = tr_key * VROW + tr_dsub * 2;

    // a request whose K/V block does not fit the 31-bit buffer range gets NaN rows (the host
    // rejects such calls when it knows a bound on L_r)
    const bool fits = (int64_t)Lr * HD * 2 < (1LL << 31);
    const int ntiles = fits ? (Lr + BN - 1) / BN : 0;
    const bool ragged = (Lr % BN) != 0;

    f32x16 o[DB];
    float l = 0.0f, mref = 0.0f, mx = -INFINITY;
    auto clear = [&]() __attribute__((always_inline)) {
        l = 0.0f;
        mx = -INFINITY;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) o[db][j] = 0.0f;
    };
    clear();

    bf16x8 pb[NKB][2];      // bf16 weights of the last scored tile (B operands of the PV MFMAs)
    const f32x16 zero16 = {};

    // The score / softmax / PV parts below act on the 32-key blocks kb in [KB0, KB1) of a tile.
    f32x16 sc[NKB];         // scores of the last tile whose MFMAs ran
    // S^T = K Q^T for the tile in stage S into sc, K fragments streamed per k16 step;
    // hook(ks) runs before the MFMAs of k16 step ks (the copies of the next tile are spread there)
    auto scores = [&](auto S, auto KB0, auto KB1, auto hook) __attribute__((always_inline)) {
        constexpr int B0 = KB0, B1 = KB1, NB = B1 - B0;
        const uint4 *kp = k_lds(S) + k_lane;
        bf16x8 kf[KPD + 1][NB];      // KPD steps of reads in flight ahead of the MFMAs
        static_for<KPD>([&](auto ks) {
#pragma unroll
            for (int b = 0; b < NB; ++b) kf[ks][b] = __builtin_bit_cast(bf16x8, kp[(B0 + b) * 32 * KSR + ks * 2]);
        });
        static_for<KS>([&](auto ks) {
            constexpr int cur = ks % (KPD + 1);
            hook(ks);
            if constexpr (ks + KPD < KS) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    kf[(ks + KPD) % (KPD + 1)][b] = __builtin_bit_cast(bf16x8, kp[(B0 + b) * 32 * KSR + (ks + KPD) * 2]);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b)
                sc[B0 + b] = mfma_32x32x16_bf16(kf[cur][b], qf[ks], ks == 0 ? zero16 : sc[B0 + b]);
            sched_fence();     // keeps the reads KPD steps ahead, not hoisted further (registers)
        });
    };
    // Softmax weights of tile `it` from sc into pb (MAXONLY: the per-query max only). MASK: the
    // ragged last tile. INIT: the main pass's first tile, which sets m_ref (a whole tile's blocks
    // must be present).
    auto softmax = [&](int it, auto KB0, auto KB1, auto mask, auto init, auto maxonly) __attribute__((always_inline)) {
        constexpr int B0 = KB0, B1 = KB1;
        constexpr bool MASK = decltype(mask)::value;
        constexpr bool INIT = decltype(init)::value;
        constexpr bool MAXONLY = decltype(maxonly)::value;
        static_assert(!INIT || (B0 == 0 && B1 == NKB), "the reference is the max of a whole tile");
#pragma unroll
        for (int kb = B0; kb < B1; ++kb)
            if (MASK) mask_block(sc[kb], Lr - it * BN - kb * 32, half);
        if constexpr (MAXONLY) {
#pragma unroll
            for (int kb = B0; kb < B1; ++kb) mx = fmaxf(mx, block_max(sc[kb]));
        } else {
            if constexpr (INIT) {
                float m0 = block_max(sc[0]);
#pragma unroll
                for (int kb = 1; kb < NKB; ++kb) m0 = fmaxf(m0, block_max(sc[kb]));
                mref = m0 * cl2;
            }
#pragma unroll
            for (int kb = B0; kb < B1; ++kb) exp_block(sc[kb], pb[kb], l, cl2, -mref);
        }
    };
    auto no_hook = [](auto) {};
    // O^T += V^T P^T for the tile in stage S with the weights in pb, V^T streamed per 32 dims
    auto pv = [&](auto S, auto KB0, auto KB1, auto hook) __attribute__((always_inline)) {
        constexpr int B0 = KB0, B1 = KB1, NB = B1 - B0;
        const char *vp = (const char *)v_lds(S) + v_lane;
        bf16x8 vf[VPD + 1][NB][2];
        auto vload = [&](int db, int set) __attribute__((always_inline)) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int o0 = ((B0 + b) * 32 + 16 * u) * VROW + db * 64;
                    i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vp + o0));
                    i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vp + o0 + 8 * VROW));
                    vf[set][b][u] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
                }
        };
        static_for<VPD>([&](auto db) { vload(db, db); });
        static_for<DB>([&](auto db) {
            constexpr int cur = db % (VPD + 1);
            hook(db);
            if constexpr (db + VPD < DB) vload(db + VPD, (db + VPD) % (VPD + 1));
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int u = 0; u < 2; ++u) o[db] = mfma_32x32x16_bf16(vf[cur][b][u], pb[B0 + b][u], o[db]);
            sched_fence();
        });
    };
    const IC<0> K0;
    const IC<NKB> KN;
    const std::true_type T;
    const std::false_type F;
    // One whole tile, nothing else in flight (the overflow redo)
    auto tile = [&](int it, auto S, auto mask, auto maxonly) __attribute__((always_inline)) {
        scores(S, K0, KN, no_hook);
        softmax(it, K0, KN, mask, F, maxonly);
        if constexpr (!decltype(maxonly)::value) pv(S, K0, KN, no_hook);
        wait_vmcnt<0>();
        barrier_lds();
    };
    auto redo_tile = [&](int it, auto maxonly) __attribute__((always_inline)) {
        if (ragged && it == ntiles - 1) tile(it, IC<0>{}, T, maxonly);
        else tile(it, IC<0>{}, F, maxonly);
    };

    // ---- main pass ----
    // The copies of tile it + 1 go out one per k16 step of tile it's scores, so the eight waves
    // do not queue all their copies at once right after the barrier; the copy unit is fed while
    // the MFMAs run (kCPS copies per step: one with eight waves, more when fewer waves share a
    // tile's copies). Each barrier waits for the whole next tile.
    constexpr int kCPS = (kCopiesPerTile + KS - 1) / KS;
    auto step = [&](int it, auto S, auto mask, auto init) __attribute__((always_inline)) {
        auto copies_s = [&](auto ks) __attribute__((always_inline)) {
            static_for<kCPS>([&](auto u) __attribute__((always_inline)) {
                constexpr int c = decltype(ks)::value * kCPS + decltype(u)::value;
                if constexpr (c < kCopiesPerTile) copy(c, (it + 1) * BN, IC<(S + 1) % NBUF>{});
            });
        };
        if (active) {
            scores(S, K0, KN, copies_s);
            softmax(it, K0, KN, mask, init, F);
            pv(S, K0, KN, no_hook);
        } else {
            // no row of this wave is in the request: only its share of the next tile's copies
            static_for<KS>(copies_s);
        }
        wait_vmcnt<0>();     // tile it + 1 landed
        barrier_lds();
    };
    if (ntiles > 0) {
        dma(0, IC<0>{});
        wait_vmcnt<0>();
        barrier_lds();
        // the first tile (it sets m_ref) is peeled off, so the loop's softmax has no branch on it
        if (ragged && ntiles == 1) step(0, IC<0>{}, T, T);
        else step(0, IC<0>{}, F, T);
        const int nfull = ragged ? ntiles - 1 : ntiles;
        for (int it0 = 1; it0 < nfull; it0 += NBUF)
            static_for<NBUF>([&](auto J) {
                if (it0 + J < nfull) step(it0 + J, IC<(1 + J) % NBUF>{}, F, F);
            });
        if (ragged && ntiles > 1) {
            const int st = (ntiles - 1) % NBUF;
            static_for<NBUF>([&](auto S) {
                if (st == S) step(ntiles - 1, S, T, F);
            });
        }
    }

    // ---- overflow check and redo, one tile copied at a time ----
    bool b = !(half_swap_sum(l) < INFINITY);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) b |= !(fabsf(o[db][j]) < INFINITY);
    const bool bad = half_swap_max(b ? 1.0f : 0.0f) > 0.0f && rvalid;
    if (__syncthreads_or(bad)) {
        const float keep = mref;
        clear();
        for (int it = 0; it < ntiles; ++it) {
            dma(it * BN, IC<0>{});
            wait_vmcnt<0>();
            barrier_lds();
            redo_tile(it, T);
        }
        mref = bad ? mx * cl2 : keep;
        clear();
        for (int it = 0; it < ntiles; ++it) {
            dma(it * BN, IC<0>{});
            wait_vmcnt<0>();
            barrier_lds();
            redo_tile(it, F);
        }
    }

    // ---- epilogue: O = O^T / l ----
    const float l_tot = half_swap_sum(l);
    const float inv = !fits ? __builtin_nanf("") : l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int64_t obase = cand * a.o_cs + tok * HD + ti.h * D;
    if (a.out_f32) {
        if (!rvalid) return;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d = db * 32 + 8 * jj + 4 * half;
                *(float4 *)((float *)a.out + obase + d) = make_float4(o[db][4 * jj] * inv, o[db][4 * jj + 1] * inv,
                                                                      o[db][4 * jj + 2] * inv, o[db][4 * jj + 3] * inv);
            }
        return;
    }
    // bf16: a lane holds 4-dim pieces of its row, so direct stores would put 8 bytes into each of
    // 32 rows. The wave's 32 rows (2D bytes each) go through its own area of the K/V stages, idle
    // since the last barrier, and leave as whole rows, CPR lanes per row, with the non-temporal
    // hint (whole lines). The 16-byte chunks are XOR-swizzled, and rows 16-31 hold the two 8-byte
    // halves of each chunk swapped, so that no two rows of a 32-lane write, and no two chunks of a
    // whole-row read, fall on the same banks.
    // Rows start on 16 bytes: the host checks the base and a candidate stride of 8k elements.
    constexpr int RPI = 64 / CPR;                       // rows per store instruction
    static_assert(NW <= 8 && 64 * CPR <= kInstrK * 64 && 64 * CPR <= kInstrV * 64, "O staging: two waves per stage buffer");
    const int sbuf = wave >> 1;
    uint4 *const stg = (sbuf == 0 ? k_s0 : sbuf == 1 ? k_s1 : sbuf == 2 ? v_s0 : v_s1) + (wave & 1) * 32 * CPR;
    auto swz = [](int r) __attribute__((always_inline)) { return CPR >= 16 ? (r & 15) : ((r >> 1) & 7); };
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float v0 = o[db][4 * jj + 0] * inv, v1 = o[db][4 * jj + 1] * inv;
            const float v2 = o[db][4 * jj + 2] * inv, v3 = o[db][4 * jj + 3] * inv;
            *(uint2 *)((char *)(stg + l32 * CPR + ((db * 4 + jj) ^ swz(l32))) + 8 * (half ^ (l32 >> 4))) =
                make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
        }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");     // the wave's LDS writes first
    __builtin_amdgcn_wave_barrier();
    const int64_t omark = rvalid ? obase : -1;               // row r's lanes are r and r + 32
    const int fr = lane / CPR, fc = lane % CPR;
#pragma unroll
    for (int k = 0; k < 32 / RPI; ++k) {
        const int r = fr + k * RPI;
        const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)omark, r);
        const int32_t hi = __shfl((int)(omark >> 32), r);
        const int64_t ob = (int64_t)(((uint64_t)(uint32_t)hi << 32) | lo);
        uint4 val = stg[r * CPR + (fc ^ swz(r))];
        if ((r >> 4) & 1) val = make_uint4(val.z, val.w, val.x, val.y);
        if (ob >= 0) store_nt16((uint16_t *)a.out + ob + fc * 8, val);
    }
}

// The configurations the library launches, per head dim: 8 waves x 32 query rows, 64-key tiles,
// K and V^T fragments read one step ahead of their MFMAs (mode 0); for requests with a few hundred
// stacked query rows, 4 waves of 32 rows, two or three workgroups per CU (mode 2: a request's last
// work tile is on average half as empty); and for requests with very few rows (the request-side
// attention has q_len rows per request), one wave of 32 rows (mode 1). Each row's arithmetic is
// the same in all three, so are the results.
template <int D, int MODE = 0>
struct DcaBf16Config {
    static constexpr int NW = MODE == 1 ? 1 : MODE == 2 ? 4 : 8, NKB = 2, KPD = 1, VPD = 1;
    static constexpr int BM = NW * 32;
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
    const float *qp = (const float *)a.q + cand * a.q_cs + tok * HD + ti.h * D;
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
    const int64_t obase = cand * a.o_cs + tok * HD + ti.h * D;
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

int32_t dca_block_m(int32_t D, int in_f32, int mode) {
    if (in_f32) return kF32Rows;
    if (mode == 1) return D == 128 ? DcaBf16Config<128, 1>::BM : DcaBf16Config<64, 1>::BM;
    if (mode == 2) return D == 128 ? DcaBf16Config<128, 2>::BM : DcaBf16Config<64, 2>::BM;
    return D == 128 ? DcaBf16Config<128>::BM : DcaBf16Config<64>::BM;
}

hipError_t launch_dca(const DcaArgs &a, hipStream_t s) {
    if (a.grid_tiles <= 0) return hipSuccess;
    const int64_t grid = ((a.grid_tiles + kNumXcd - 1) / kNumXcd) * kNumXcd;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (a.in_f32) {
        hipLaunchKernelGGL(dca_f32_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
    } else if (a.D == 128 || a.D == 64) {
#define IKBO_DCA_LAUNCH(DD, SM)                                                                                         \
    do {                                                                                                               \
        using C = DcaBf16Config<DD, SM>;                                                                               \
        hipLaunchKernelGGL((dca_bf16_kernel<DD, C::NW, C::NKB, C::KPD, C::VPD>), dim3((unsigned)grid),                     \
                           dim3(C::NW * 64), 0, s, a);                                                                 \
    } while (0)
        if (a.D == 128) {
            if (a.mode == 1) IKBO_DCA_LAUNCH(128, 1);
            else if (a.mode == 2) IKBO_DCA_LAUNCH(128, 2);
            else IKBO_DCA_LAUNCH(128, 0);
        } else {
            if (a.mode == 1) IKBO_DCA_LAUNCH(64, 1);
            else if (a.mode == 2) IKBO_DCA_LAUNCH(64, 2);
            else IKBO_DCA_LAUNCH(64, 0);
        }
#undef IKBO_DCA_LAUNCH
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ikbo
