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

namespace ikbo {

namespace {

constexpr int kBlockN = 64;        // keys per LDS tile
constexpr int kWavesBf16 = 8;      // waves per workgroup (2 per SIMD)
constexpr int kBlockMBf16 = kWavesBf16 * 32;
constexpr float kTau = 8.0f;       // lazy-rescale threshold, log2 units (p <= 2^8)

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
template <int D>
__global__ __launch_bounds__(kWavesBf16 * 64) void dca_bf16_kernel(DcaArgs a) {
    constexpr int CPR = D / 8;                         // 16-byte chunks per key row
    constexpr int kTileChunks = kBlockN * CPR;         // chunks per K (or V) tile
    constexpr int kThreads = kWavesBf16 * 64;
    constexpr int kLoadPasses = kTileChunks / kThreads;
    static_assert(kTileChunks % kThreads == 0, "tile load must split evenly");
    constexpr int KS = D / 16;                         // k16 steps over the head dim
    constexpr int DB = D / 32;                         // 32-row blocks of O^T

    __shared__ uint4 smem[2][2][kTileChunks];          // [stage][K=0 / V=1][chunk]

    TileInfo ti;
    if (!decode_tile(a, kBlockMBf16, ti)) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, half = lane >> 5;
    const int64_t HD = (int64_t)a.H * D;

    // ---- this lane's query row (column of S^T) ----
    const int64_t srow = ti.qb * kBlockMBf16 + wave * 32 + l32;
    const bool rvalid = srow < ti.rows;
    int64_t cand = 0;
    int tok = 0;
    if (rvalid) row_source(a, ti, srow, cand, tok);
    bf16x8 qf[KS];
    {
        const uint16_t *qp = (const uint16_t *)a.q + ((cand * a.Lq + tok) * HD + ti.h * D) + half * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 u = rvalid ? *(const uint4 *)(qp + ks * 16) : make_uint4(0, 0, 0, 0);
            qf[ks] = __builtin_bit_cast(bf16x8, u);
        }
    }

    // ---- K/V tile loader ----
    const uint16_t *kbase = (const uint16_t *)a.k + ti.kv_row0 * HD + ti.h * D;
    const uint16_t *vbase = (const uint16_t *)a.v + ti.kv_row0 * HD + ti.h * D;
    const int64_t Lr = ti.Lr;
    uint4 pk[kLoadPasses], pv[kLoadPasses];
    auto gload = [&](int64_t n0) {
#pragma unroll
        for (int p = 0; p < kLoadPasses; ++p) {
            const int qd = tid + p * kThreads, key = qd / CPR, ch = qd % CPR;
            if (n0 + key < Lr) {
                const int64_t off = (n0 + key) * HD + ch * 8;
                pk[p] = *(const uint4 *)(kbase + off);
                pv[p] = *(const uint4 *)(vbase + off);
            } else {
                pk[p] = make_uint4(0, 0, 0, 0);
                pv[p] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto lstore = [&](int st) {
#pragma unroll
        for (int p = 0; p < kLoadPasses; ++p) {
            const int qd = tid + p * kThreads, key = qd / CPR, ch = qd % CPR;
            smem[st][0][key * CPR + (ch ^ swz_k<D>(key))] = pk[p];
            smem[st][1][key * CPR + (ch ^ swz_v(key))] = pv[p];
        }
    };

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;
    const float cl2 = a.scale * 1.4426950408889634f;

    const int64_t ntiles = (Lr + kBlockN - 1) / kBlockN;
    if (ntiles > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();

    // lane constants of the transposed V read
    const int g16 = lane >> 4, s16 = lane & 15;
    const int tr_dsub = (g16 & 1) * 16 + 4 * (s16 & 3);   // + db * 32
    const int tr_key = 4 * (g16 >> 1) + (s16 >> 2);        // + kb * 32 + 16 u + 8 t

    for (int64_t it = 0; it < ntiles; ++it) {
        const int st = (int)(it & 1);
        const int64_t n0 = it * kBlockN;
        if (it + 1 < ntiles) gload(n0 + kBlockN);

        // ---- S^T = K Q^T for 64 keys (two 32-key blocks) ----
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) s[kb][j] = 0.0f;
        const uint4 *ks_lds = smem[st][0];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int key = kb * 32 + l32, ch = ks * 2 + half;
                bf16x8 af = __builtin_bit_cast(bf16x8, ks_lds[key * CPR + (ch ^ swz_k<D>(key))]);
                s[kb] = mfma_32x32x16_bf16(af, qf[ks], s[kb]);
            }
        }

        // ---- online softmax (exp2 domain, lazy rescale) ----
        if (n0 + kBlockN > Lr) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int64_t key = n0 + kb * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
                    if (key >= Lr) s[kb][j] = -INFINITY;
                }
        }
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kb][j]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = mx * cl2;
        const bool need = m_new > m_run + kTau;
        if (__any(need)) {
            const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            if (need) m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
        }
        bf16x8 pb[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][j], cl2, -m_run));
                s[kb][j] = p;
                l_run += p;
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) pb[kb][u][e] = (__bf16)s[kb][8 * u + e];
        }

        // ---- O^T += V^T P^T ----
        const char *vs_lds = (const char *)smem[st][1];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int dcol = db * 32 + tr_dsub;
            const int chunk = dcol >> 3, sub = (dcol & 7) * 2;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int key0 = kb * 32 + 16 * u + tr_key;
                    const int key1 = key0 + 8;
                    i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(vs_lds + (key0 * CPR + (chunk ^ swz_v(key0))) * 16 + sub));
                    i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(vs_lds + (key1 * CPR + (chunk ^ swz_v(key1))) * 16 + sub));
                    typedef short i16x8 __attribute__((ext_vector_type(8)));
                    i16x8 av = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
                    o[db] = mfma_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb[kb][u], o[db]);
                }
        }

        if (it + 1 < ntiles) lstore(st ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O^T / l, store rows ----
    if (!rvalid) return;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int64_t obase = (cand * a.Lq + tok) * HD + ti.h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int d = db * 32 + 8 * jj + 4 * half;
            const float v0 = o[db][4 * jj + 0] * inv, v1 = o[db][4 * jj + 1] * inv;
            const float v2 = o[db][4 * jj + 2] * inv, v3 = o[db][4 * jj + 3] * inv;
            if (a.out_f32) {
                *(float4 *)((float *)a.out + obase + d) = make_float4(v0, v1, v2, v3);
            } else {
                *(uint2 *)((uint16_t *)a.out + obase + d) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
            }
        }
}

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
    (void)D;
    return in_f32 ? kF32Rows : kBlockMBf16;
}

hipError_t launch_dca(const DcaArgs &a, hipStream_t s) {
    if (a.grid_tiles <= 0) return hipSuccess;
    const int64_t grid = ((a.grid_tiles + kNumXcd - 1) / kNumXcd) * kNumXcd;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (a.in_f32) {
        hipLaunchKernelGGL(dca_f32_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
    } else if (a.D == 128) {
        hipLaunchKernelGGL(dca_bf16_kernel<128>, dim3((unsigned)grid), dim3(kWavesBf16 * 64), 0, s, a);
    } else if (a.D == 64) {
        hipLaunchKernelGGL(dca_bf16_kernel<64>, dim3((unsigned)grid), dim3(kWavesBf16 * 64), 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ikbo
