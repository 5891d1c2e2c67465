// GEMM kernels of IKBO-LCB (ROCS Sec. 4.1 Eq. 14 and Sec. 4.2).
//
// Both operands are K-contiguous ("NT"): activations X [M, K] and weights W [N, K], computing
// C[m, n] = sum_k X[m, k] W[n, k]. The bf16 kernel computes C^T = W X^T with
// v_mfma_f32_32x32x16_bf16 (A operand = W rows, B operand = X rows), so each lane of the fp32
// accumulator owns one activation row and groups of 4 consecutive output columns. That makes the
// fused epilogue of Sec. 4.2.1 cheap: one request-index lookup m[row] per lane and row, then
// 16-byte reads of the request-derived term Z[m[row], n..n+3], added in registers before the
// activation and the single store. The candidate GEMM result is never written to memory on its own.
//
// Tile 256 x 256 x 64, 8 waves (2 along N x 4 along M, each 128 x 64), two LDS stages filled by
// direct buffer -> LDS copies of the next k tile while the current one is multiplied. Tiles are numbered with the N tile fastest and each
// XCD takes a contiguous range, so the N tiles that share one block of activation rows run
// together on one XCD and read those rows through its L2.
//
// The request GEMM ([Y_r | Z] = x_r [W_RR; W_CR]^T, a small M = num_req) runs split-K into fp32
// partial sums, reduced in a fixed order by a second kernel that also applies the request-group
// epilogue; results are deterministic.
#include <type_traits>

#include "ikbo_device.h"
#include "ikbo_launch.h"

namespace ikbo {

namespace {

// bf16 configuration: 4 x 2 waves, each 64 activation rows x 128 output columns, 64-deep k tiles
// in two LDS stages
constexpr int kWGM = 4, kWGN = 2, kTM = 64, kTN = 128;
constexpr int BM = kWGM * kTM, BN = kWGN * kTN, BK = 64;
constexpr int kGemmGroupM = 8;     // row blocks per tile group of the one-tile-per-workgroup GEMM
constexpr int kGemmThreads = kWGM * kWGN * 64;

__device__ __forceinline__ float apply_act(int act, float x) { return act == 1 ? gelu_exact(x) : x; }

// A float read past the XCD's L2 (agent-coherent), for data other XCDs wrote during this launch.
__device__ __forceinline__ float load_coherent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Epilogue for 4 consecutive columns col..col+3 of one row. ZCOH: Z was written during this launch
// by other workgroups (it is read only after the flags of the request tiles holding its columns are
// set). When every 128-byte line of Z holds columns of one 256-column request tile only (row
// stride a multiple of 32 floats, Z 128-byte aligned), no line can reach this XCD's caches before
// its final values (caches start the launch invalidated) and plain loads read them. Otherwise a
// line can also hold columns of a tile not yet final when it is first read, and Z is read with
// agent-coherent loads, past the L2.
template <bool ZCOH = false>
__device__ __forceinline__ void epilogue4(const GemmArgs &a, int64_t row, int64_t zrow, bool row_ok, int64_t col,
                                          float v0, float v1, float v2, float v3) {
    const bool zcoh = ZCOH && ((a.ldz & 31) != 0 || ((uintptr_t)a.z & 127) != 0);
    float v[4] = {v0, v1, v2, v3};
    const bool full = col + 3 < a.N;
    if (!row_ok) {
        v[0] = v[1] = v[2] = v[3] = 0.0f;
    } else {
        if (a.bias) {
            if (full) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] += a.bias[col + e];
            } else {
                for (int e = 0; e < 4; ++e)
                    if (col + e < a.N) v[e] += a.bias[col + e];
            }
        }
        if (a.z) {
            const float *zp = a.z + zrow * a.ldz + col;
            if (full && (a.ldz & 3) == 0) {
                if (zcoh) {
                    const uint64_t *zq = (const uint64_t *)zp;
                    const uint64_t lo = __hip_atomic_load(zq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    const uint64_t hi = __hip_atomic_load(zq + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    v[0] += __uint_as_float((uint32_t)lo); v[1] += __uint_as_float((uint32_t)(lo >> 32));
                    v[2] += __uint_as_float((uint32_t)hi); v[3] += __uint_as_float((uint32_t)(hi >> 32));
                } else {
                    const float4 zz = *(const float4 *)zp;
                    v[0] += zz.x; v[1] += zz.y; v[2] += zz.z; v[3] += zz.w;
                }
            } else {
                for (int e = 0; e < 4; ++e)
                    if (col + e < a.N) v[e] += zcoh ? load_coherent(zp + e) : zp[e];
            }
        }
        if (a.act) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = apply_act(a.act, v[e]);
        }
    }
    if (a.out_f32) {
        float *op = (float *)a.out + row * a.ldo + col;
        if (full && (a.ldo & 3) == 0) {
            *(float4 *)op = make_float4(v[0], v[1], v[2], v[3]);
        } else {
            for (int e = 0; e < 4; ++e)
                if (col + e < a.N) op[e] = v[e];
        }
    } else {
        uint16_t *op = (uint16_t *)a.out + row * a.ldo + col;
        if (full && (a.ldo & 3) == 0) {
            *(uint2 *)op = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
            for (int e = 0; e < 4; ++e)
                if (col + e < a.N) op[e] = f32_to_bf16(v[e]);
        }
    }
}

// Resolve a row's request for the gather: returns false when the row's request is out of range.
__device__ __forceinline__ bool row_request(const GemmArgs &a, int64_t row, int64_t &zrow) {
    zrow = 0;
    if (!a.z) return true;
    const int32_t r = a.map[row];
    zrow = r;
    return r >= 0 && r < a.R;
}

// ----------------------------------------------------------------------------------------------
// ----------------------------------------------------------------------------------------------
// bf16 GEMM, templated on the wave grid (WGM along M x WGN along N), the per-wave tile (TM
// activation rows x TN output columns, in 32x32x16 MFMA blocks), the k-tile depth TBK and the
// number of LDS stages NBUF.
//
// DMA: tiles go global -> LDS directly with buffer loads (each wave instruction fills 64
// consecutive 16-byte slots; the lane filling slot (row, c') reads chunk c' ^ swizzle(row)). This
// needs K to be a multiple of TBK and a tile that does not straddle the w0 / w1 boundary; rows past
// M or N fall outside the tile's buffer range and read as zeros. Otherwise the next tile is staged
// through registers (any K that is a multiple of 8). With NBUF stages tile it + NBUF - 1 is copied
// during tile it into the stage that tile it - 1 used, and only tile it + 1 is waited for.
//
// Each stage is its own LDS variable and the stage index is a compile-time constant everywhere
// (the k loop is unrolled by NBUF): reads of one stage then carry an alias scope distinct from the
// copies in flight into another, so the compiler does not hold them back until those land.
// Fragments for k step ks + 1 are read into a second register set before the MFMAs of step ks.
// LDS chunk swizzle for rows of CPR 16-byte chunks: 16 consecutive rows read at one logical chunk
// land in 16 distinct 16-byte bank groups.
template <int CPR>
__device__ __forceinline__ int swzc(int row) { return CPR == 8 ? ((row >> 1) & 7) : ((row >> 2) & 3); }

// Tile geometry of a bf16 GEMM configuration.
template <int WGM, int WGN, int TM, int TN, int TBK>
struct GemmShape {
    static constexpr int T = WGM * WGN * 64;
    static constexpr int TBM = WGM * TM, TBN = WGN * TN;
    static constexpr int CPR = TBK / 8;                       // 16-byte chunks per tile row
    static constexpr int XCH = TBM * CPR, WCH = TBN * CPR;    // chunks per X / W tile
};

constexpr uint32_t kOutOfRange = 0x80000000u;      // past every tile's buffer range (< 2^31 bytes)

// Direct-copy state of one output tile: buffer resources over its activation and weight rows (rows
// past M / N read as zeros), this lane's byte offset in each (pass p adds p * T / CPR rows), and
// its k tiles (nk from kbeg, visited from krot on, wrapping).
struct DmaTile {
    __amdgpu_buffer_rsrc_t xr, wr;
    uint32_t xvoff, wvoff;
    int nk, krot, kbeg;
};

// k tiles of split sp, and the first one visited. The N tiles that share a block of activation rows
// run side by side on one XCD; starting each one k tile further along (nt mod 4) staggers them, so
// one of them misses L2 on a given activation tile and the others find it there, instead of all of
// them waiting on the same miss.
template <int TBK>
__device__ __forceinline__ void k_range(const GemmArgs &a, int nt, int sp, int32_t k_per_split, int &kbeg, int &kend,
                                        int &nk, int &krot) {
    kbeg = sp * k_per_split;
    kend = min(a.K, kbeg + k_per_split);
    nk = kend > kbeg ? (kend - kbeg + TBK - 1) / TBK : 0;
    krot = nk > 0 ? (nt & 3) % nk : 0;
}

template <class G, int TBK>
__device__ __forceinline__ DmaTile dma_tile(const GemmArgs &a, int mt, int nt, int sp, int32_t k_per_split, int wave,
                                            int lane) {
    constexpr int TBM = G::TBM, TBN = G::TBN, CPR = G::CPR;
    DmaTile t;
    int kend;
    k_range<TBK>(a, nt, sp, k_per_split, t.kbeg, kend, t.nk, t.krot);
    const int64_t m0 = (int64_t)mt * TBM;
    const int n0 = nt * TBN;
    const int row = (wave * 64 + lane) / CPR;
    const int ch = (lane % CPR) ^ swzc<CPR>(row);
    const int64_t mrows = min((int64_t)TBM, a.M - m0);
    t.xr = make_rsrc((const uint16_t *)a.x + m0 * a.ldx, (uint32_t)(mrows * a.ldx * 2));
    t.xvoff = (uint32_t)(row * a.ldx + ch * 8) * 2;
    const bool second = n0 >= a.n0;     // a tile never straddles the w0 / w1 boundary here
    const int nend = second ? a.N : min(a.N, a.n0);
    const uint16_t *wbase = second ? (const uint16_t *)a.w1 + (int64_t)(n0 - a.n0) * a.K
                                   : (const uint16_t *)a.w0 + (int64_t)n0 * a.K;
    t.wr = make_rsrc(wbase, (uint32_t)(min(TBN, nend - n0) * a.K * 2));
    t.wvoff = (uint32_t)(row * a.K + ch * 8) * 2;
    return t;
}

// Copies step kt of a tile into one LDS stage (xs / ws); steps at or past nk read out of range.
template <class G, int TBK>
__device__ __forceinline__ void dma_fetch(const GemmArgs &a, const DmaTile &t, int kt, uint4 *xs, uint4 *ws, int wave) {
    constexpr int T = G::T, CPR = G::CPR, XP = G::XCH / T, WP = G::WCH / T;
    int ktr = kt + t.krot;
    if (ktr >= t.nk) ktr -= t.nk;
    const int k0 = t.kbeg + ktr * TBK;
    const bool in = kt < t.nk;
#pragma unroll
    for (int p = 0; p < XP; ++p)
        buffer_copy16_to_lds(t.xr, in ? t.xvoff + (uint32_t)(p * (T / CPR) * a.ldx + k0) * 2 : kOutOfRange,
                             xs + p * T + wave * 64);
#pragma unroll
    for (int p = 0; p < WP; ++p)
        buffer_copy16_to_lds(t.wr, in ? t.wvoff + (uint32_t)(p * (T / CPR) * a.K + k0) * 2 : kOutOfRange,
                             ws + p * T + wave * 64);
}

struct NoHook {
    __device__ void operator()() const {}
};

// The mark of an output tile whose result is not available: NaN in columns col..col+3 below N.
__device__ __forceinline__ void store_nan4(const GemmArgs &a, int64_t row, int64_t col) {
    for (int e = 0; e < 4; ++e)
        if (col + e < a.N) {
            if (a.out_f32) ((float *)a.out)[row * a.ldo + col + e] = __builtin_nanf("");
            else ((uint16_t *)a.out)[row * a.ldo + col + e] = 0x7fc0;
        }
}

// One output tile (mt, nt) over the k range of split sp. sx[s] / sw[s] are the LDS stages of the
// activation / weight tiles (the caller's __shared__ arrays, one per stage). pre_epilogue() runs
// between the main loop and the epilogue (every thread); when it returns a bool, false (the same
// in every thread) makes the epilogue store the NaN mark in every output element of the tile
// instead of its result, reading neither bias nor Z. mid_epilogue() runs once inside the epilogue,
// after the loads of its first column group are issued (LDS is free by then: a copy issued there
// does not delay those loads, which it would when issued before them). prefetched: the caller has
// already copied step 0 into stage 0 with dma_fetch (direct copies, two stages).
template <int WGM, int WGN, int TM, int TN, int TBK, int NBUF, bool DMA, bool PARTIAL, bool ZCOH, bool STG,
          typename Pre, typename Mid = NoHook>
__device__ __forceinline__ void gemm_tile(const GemmArgs &a, int mt, int nt, int sp, int32_t k_per_split,
                                          uint4 *const *sx, uint4 *const *sw, Pre pre_epilogue,
                                          bool prefetched = false, Mid mid_epilogue = Mid()) {
    using G = GemmShape<WGM, WGN, TM, TN, TBK>;
    constexpr int T = G::T, TBM = G::TBM, TBN = G::TBN, CPR = G::CPR, XCH = G::XCH, WCH = G::WCH;
    constexpr int XP = XCH / T, WP = WCH / T;          // load passes
    static_assert(XCH % T == 0 && WCH % T == 0, "tile load must split evenly");
    constexpr int MB = TM / 32, NB = TN / 32;
    constexpr int kCopies = XP + WP;
    static_assert(NBUF == 2 || DMA, "more than two stages need the direct copies");
    static_assert(NBUF <= 4 && (NBUF - 2) * kCopies < 64, "vmcnt range");
    static_assert(!DMA || (T / CPR) % 16 == 0, "direct copies: the chunk swizzle must repeat every pass");
    auto xs = [&](auto S) -> uint4 * { return sx[decltype(S)::value]; };
    auto ws = [&](auto S) -> uint4 * { return sw[decltype(S)::value]; };

    const int64_t m0 = (int64_t)mt * TBM;
    const int n0 = nt * TBN;
    int kbeg, kend, nk, krot;
    k_range<TBK>(a, nt, sp, k_per_split, kbeg, kend, nk, krot);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);     // uniform: LDS copy bases in SGPRs
    const int l32 = lane & 31, half = lane >> 5;
    const int wn = wave / WGM, wm = wave % WGM;

    // Register-staged path: source row pointers of this thread's copies (rows past M / N repeat the
    // last valid row; their results are never stored).
    constexpr int NP = DMA ? 1 : (XP > WP ? XP : WP);
    const uint16_t *xsrc[NP];
    const uint16_t *wsrc[NP];
    int xslot[NP], wslot[NP];
    // Direct path: the tile's buffer resources and lane offsets.
    DmaTile dt;
    if constexpr (DMA) {
        dt = dma_tile<G, TBK>(a, mt, nt, sp, k_per_split, wave, lane);
    } else {
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            const int slot = tid + p * T;
            const int row = slot / CPR, chp = slot % CPR;
            int64_t gm = m0 + row;
            if (gm >= a.M) gm = a.M - 1;
            xsrc[p] = (const uint16_t *)a.x + gm * a.ldx + chp * 8;
            xslot[p] = row * CPR + (chp ^ swzc<CPR>(row));
        }
#pragma unroll
        for (int p = 0; p < WP; ++p) {
            const int slot = tid + p * T;
            const int row = slot / CPR, chp = slot % CPR;
            int gn = n0 + row;
            if (gn >= a.N) gn = a.N - 1;
            const uint16_t *wp = gn < a.n0 ? (const uint16_t *)a.w0 + (int64_t)gn * a.K
                                           : (const uint16_t *)a.w1 + (int64_t)(gn - a.n0) * a.K;
            wsrc[p] = wp + chp * 8;
            wslot[p] = row * CPR + (chp ^ swzc<CPR>(row));
        }
    }
    uint4 px[NP], pw[NP];
    auto fetch = [&](int kt, auto st) {
        if constexpr (DMA) {
            dma_fetch<G, TBK>(a, dt, kt, xs(st), ws(st), wave);
        } else {
            int ktr = kt + krot;     // rotated k order, see k_range
            if (ktr >= nk) ktr -= nk;
            const int k0 = kbeg + ktr * TBK;
#pragma unroll
            for (int p = 0; p < XP; ++p) {
                const int ch = (tid + p * T) % CPR;
                px[p] = (k0 + ch * 8 < kend) ? *(const uint4 *)(xsrc[p] + k0) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int p = 0; p < WP; ++p) {
                const int ch = (tid + p * T) % CPR;
                pw[p] = (k0 + ch * 8 < kend) ? *(const uint4 *)(wsrc[p] + k0) : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto commit = [&](auto st) {   // register-staged path: write the fetched tile to LDS
        if constexpr (!DMA) {
#pragma unroll
            for (int p = 0; p < XP; ++p) xs(st)[xslot[p]] = px[p];
#pragma unroll
            for (int p = 0; p < WP; ++p) ws(st)[wslot[p]] = pw[p];
        }
    };
    f32x16 acc[NB][MB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // fragments of one 16-deep k step: NB from the weight tile (A operand), MB from the activation
    // tile (B operand); two register sets so step ks + 1 is read while step ks multiplies
    constexpr int KS = TBK / 16;
    bf16x8 af[2][NB], bfr[2][MB];
    auto load_frags = [&](auto st, int ks, auto set) {
        const int ch = ks * 2 + half;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int row = wn * TN + i * 32 + l32;
            af[set][i] = __builtin_bit_cast(bf16x8, ws(st)[row * CPR + (ch ^ swzc<CPR>(row))]);
        }
#pragma unroll
        for (int j = 0; j < MB; ++j) {
            const int row = wm * TM + j * 32 + l32;
            bfr[set][j] = __builtin_bit_cast(bf16x8, xs(st)[row * CPR + (ch ^ swzc<CPR>(row))]);
        }
    };
    auto compute = [&](auto st) {
        load_frags(st, 0, IC<0>{});
        static_for<KS>([&](auto ks) {
            constexpr int cur = ks & 1;
            // the next step's reads go out before this step's MFMAs, into the other register set
            if constexpr (ks + 1 < KS) load_frags(st, ks + 1, IC<cur ^ 1>{});
            sched_fence();
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int j = 0; j < MB; ++j) acc[i][j] = mfma_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j]);
        });
    };

    if constexpr (DMA) {
        // Every step copies one tile. Tiles at or past nk are read out of range (zeros, no memory
        // access), so the loop has no data-dependent branch and a fixed number of copies in flight;
        // it runs to a multiple of NBUF steps, the extra ones multiplying zeros.
        if (!prefetched) static_for<NBUF - 1>([&](auto S) { fetch(S, S); });
        else static_for<NBUF - 2>([&](auto S) { fetch(S + 1, IC<S + 1>{}); });
        wait_vmcnt<(NBUF - 2) * kCopies>();                   // tile 0 landed
        barrier_lds();
        for (int base = 0; base < nk; base += NBUF) {
            static_for<NBUF>([&](auto S) {
                // the stage of tile base + S + NBUF - 1 held the tile consumed before the last barrier
                fetch(base + S + NBUF - 1, IC<(S + NBUF - 1) % NBUF>{});
                compute(S);
                wait_vmcnt<(NBUF - 2) * kCopies>();           // tile base + S + 1 landed
                barrier_lds();
            });
        }
        wait_vmcnt<0>();     // no copy may still be writing LDS when the workgroup ends
    } else {
        if (nk > 0) {
            fetch(0, IC<0>{});
            commit(IC<0>{});
        }
        barrier_lds();
        for (int base = 0; base < nk; base += 2) {
            static_for<2>([&](auto S) {
                const int it = base + S;
                if (it < nk) {
                    if (it + 1 < nk) fetch(it + 1, IC<1 - S>{});
                    compute(S);
                    if (it + 1 < nk) commit(IC<1 - S>{});
                    barrier_lds();
                }
            });
        }
    }

    bool mark = false;
    if constexpr (std::is_same_v<decltype(pre_epilogue()), bool>) mark = !pre_epilogue();
    else pre_epilogue();

    // ---- epilogue ----
    // Fast form, uniform per tile: every column of the tile inside N and 16-byte output / Z rows.
    // For each 32-column group i the bias and Z values of the lane's MB rows are loaded together
    // before any of the group's results is stored, so a tile waits on NB load round trips instead
    // of one per 4 columns (the stores may alias the loads, which keeps the compiler from moving
    // loads past them). The branches on bias / Z / coherent reads are taken once per tile.
    const int cw = n0 + wn * TN;     // first output column of this wave
    const bool fast = n0 + TBN <= a.N &&
                      (PARTIAL ? (a.N & 3) == 0 : ((a.ldo & 3) == 0 && (!a.z || (a.ldz & 3) == 0)));
    if (fast) {
        int64_t rowj[MB];
        bool rin[MB];
#pragma unroll
        for (int j = 0; j < MB; ++j) {
            rowj[j] = m0 + wm * TM + j * 32 + l32;
            rin[j] = rowj[j] < a.M;
        }
        if constexpr (PARTIAL) {
            mid_epilogue();
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                if (!rin[j]) continue;
                float *pp = a.partial + ((int64_t)sp * a.M + rowj[j]) * a.N + cw + 4 * half;
#pragma unroll
                for (int i = 0; i < NB; ++i)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        *(float4 *)(pp + i * 32 + 8 * jj) = make_float4(acc[i][j][4 * jj], acc[i][j][4 * jj + 1],
                                                                        acc[i][j][4 * jj + 2], acc[i][j][4 * jj + 3]);
            }
        } else {
            // each row's request (rows whose request is out of range are written as zeros)
            int64_t zoff[MB];
            bool rok[MB];
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                bool ok = rin[j];
                int64_t zr = 0;
                if (a.z) {
                    const int32_t r = rin[j] ? a.map[rowj[j]] : 0;
                    ok = rin[j] && r >= 0 && r < a.R;
                    zr = ok ? r : 0;
                }
                zoff[j] = zr * a.ldz;
                rok[j] = ok;
            }
            const bool zcoh = ZCOH && a.z && ((a.ldz & 31) != 0 || ((uintptr_t)a.z & 127) != 0);
            bool any_bad = false;
#pragma unroll
            for (int j = 0; j < MB; ++j) any_bad |= !rok[j];
            const bool all_ok = __builtin_amdgcn_ballot_w64(any_bad) == 0;     // no row of the wave zeroed
            // row bases: every access below is the base plus a compile-time offset
            const float *zb[MB];
            char *ob[MB];
            const int osz = a.out_f32 ? 4 : 2;
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                zb[j] = a.z ? a.z + zoff[j] + cw + 4 * half : nullptr;
                ob[j] = (char *)a.out + (rowj[j] * a.ldo + cw + 4 * half) * osz;
            }
            const float *bb = a.bias ? a.bias + cw + 4 * half : nullptr;
            // Staged stores. A lane holds 4-column pieces of one row, so a direct store puts 8 or 16
            // bytes into each of 32 rows. Instead the wave's results for 128 output bytes of each of
            // its rows (two 32-column groups in bf16, one in fp32) go to a per-wave area of LDS stage
            // 1, which is free once the main loop has ended (with two stages its last copy lands in
            // stage 0, and a persistent caller prefetches only into stage 0), and leave as whole
            // 128-byte row pieces, 8 rows per store (non-temporal: the output is streamed). 16-byte
            // chunks are XOR-swizzled by (row >> 1) & 7, and in bf16 rows 16-31 of a 32-row block
            // hold the two 8-byte halves of each chunk swapped, so no two rows of a 32-lane write,
            // and no two chunks of a whole-row read, fall on the same banks.
            constexpr int NW2 = WGM * WGN / 2;
            static_assert(NBUF == 2 && WGM * WGN % 2 == 0 && NW2 * TM * 8 <= XCH && NW2 * TM * 8 <= WCH,
                          "output staging: each wave's TM x 128-byte area must fit in LDS stage 1");
            char *const stg = (char *)(wave < NW2 ? sx[1] + wave * TM * 8 : sw[1] + (wave - NW2) * TM * 8);
            // addresses: a wave-uniform base (SGPRs) plus one 32-bit lane offset
            const int srow = lane >> 3, sch = lane & 7;
            const int64_t wrow0 = m0 + wm * TM;
            const int64_t obase_el = wrow0 * a.ldo + cw;
            char *const obase = (char *)a.out +
                                (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(obase_el >> 32)) << 32) |
                                          (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)obase_el)) * osz;
            const uint32_t loff = (uint32_t)(srow * a.ldo * osz) + sch * 16;
            const int64_t ostep = 8 * a.ldo * osz;
            const int rows_here = (int)min((int64_t)TM, a.M - wrow0) - srow;     // this lane's rows: srow + 8k
            auto flush = [&](int col_bytes, bool swapped) __attribute__((always_inline)) {
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");     // the wave's LDS writes first
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int k = 0; k < TM / 8; ++k) {
                    const int row = srow + 8 * k;
                    uint4 val = *(const uint4 *)(stg + row * 128 + (sch ^ ((row >> 1) & 7)) * 16);
                    if (swapped && ((row >> 4) & 1)) val = make_uint4(val.z, val.w, val.x, val.y);
                    if (8 * k < rows_here) store_nt16(obase + k * ostep + col_bytes + loff, val);
                }
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");     // reads before the next writes
                __builtin_amdgcn_wave_barrier();
            };
            auto body = [&](auto HB, auto HZ, auto HC) __attribute__((always_inline)) {
                static_for<NB>([&](auto I) __attribute__((always_inline)) {
                    constexpr int i = decltype(I)::value;
                    float4 bv[4], zv[MB][4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int c = i * 32 + 8 * jj;
                        if constexpr (decltype(HB)::value) bv[jj] = *(const float4 *)(bb + c);
                        else bv[jj] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
                        for (int j = 0; j < MB; ++j) {
                            if constexpr (!decltype(HZ)::value) {
                                zv[j][jj] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                            } else if constexpr (decltype(HC)::value) {
                                const uint64_t *zq = (const uint64_t *)(zb[j] + c);
                                const uint64_t lo = __hip_atomic_load(zq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                                const uint64_t hi = __hip_atomic_load(zq + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                                zv[j][jj] = make_float4(__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                                                        __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32)));
                            } else {
                                zv[j][jj] = *(const float4 *)(zb[j] + c);
                            }
                        }
                    }
                    if constexpr (i == 0) mid_epilogue();
                    // pre-activation values of the group, then the activation (one branch per group)
                    float v[MB][16];
#pragma unroll
                    for (int j = 0; j < MB; ++j)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            v[j][4 * jj + 0] = acc[i][j][4 * jj + 0] + bv[jj].x + zv[j][jj].x;
                            v[j][4 * jj + 1] = acc[i][j][4 * jj + 1] + bv[jj].y + zv[j][jj].y;
                            v[j][4 * jj + 2] = acc[i][j][4 * jj + 2] + bv[jj].z + zv[j][jj].z;
                            v[j][4 * jj + 3] = acc[i][j][4 * jj + 3] + bv[jj].w + zv[j][jj].w;
                        }
                    if (a.act == 1) {
#pragma unroll
                        for (int j = 0; j < MB; ++j)
#pragma unroll
                            for (int e = 0; e < 16; ++e) v[j][e] = gelu_exact(v[j][e]);
                    }
                    if (!all_ok) {
#pragma unroll
                        for (int j = 0; j < MB; ++j)
#pragma unroll
                            for (int e = 0; e < 16; ++e) v[j][e] = rok[j] ? v[j][e] : 0.0f;
                    }
                    if (mark) {
#pragma unroll
                        for (int j = 0; j < MB; ++j)
#pragma unroll
                            for (int e = 0; e < 16; ++e) v[j][e] = __builtin_nanf("");
                    }
                    if constexpr (STG) {
                        const int sw7 = (l32 >> 1) & 7, hs = half ^ ((l32 >> 4) & 1);
                        if (a.out_f32) {
#pragma unroll
                            for (int j = 0; j < MB; ++j)
#pragma unroll
                                for (int jj = 0; jj < 4; ++jj)
                                    *(float4 *)(stg + (j * 32 + l32) * 128 + ((2 * jj + half) ^ sw7) * 16) =
                                        make_float4(v[j][4 * jj], v[j][4 * jj + 1], v[j][4 * jj + 2], v[j][4 * jj + 3]);
                            flush(i * 128, false);
                        } else {
#pragma unroll
                            for (int j = 0; j < MB; ++j)
#pragma unroll
                                for (int jj = 0; jj < 4; ++jj)
                                    *(uint2 *)(stg + (j * 32 + l32) * 128 + (((i & 1) * 4 + jj) ^ sw7) * 16 + 8 * hs) =
                                        make_uint2(pack_bf16x2(v[j][4 * jj], v[j][4 * jj + 1]),
                                                   pack_bf16x2(v[j][4 * jj + 2], v[j][4 * jj + 3]));
                            if constexpr ((i & 1) == 1 || i == NB - 1) flush((i >> 1) * 128, true);
                        }
                    } else if (a.out_f32) {
#pragma unroll
                        for (int j = 0; j < MB; ++j)
                            if (rin[j])
#pragma unroll
                                for (int jj = 0; jj < 4; ++jj)
                                    *(float4 *)(ob[j] + (i * 32 + 8 * jj) * 4) =
                                        make_float4(v[j][4 * jj], v[j][4 * jj + 1], v[j][4 * jj + 2], v[j][4 * jj + 3]);
                    } else {
#pragma unroll
                        for (int j = 0; j < MB; ++j)
                            if (rin[j])
#pragma unroll
                                for (int jj = 0; jj < 4; ++jj)
                                    *(uint2 *)(ob[j] + (i * 32 + 8 * jj) * 2) =
                                        make_uint2(pack_bf16x2(v[j][4 * jj], v[j][4 * jj + 1]),
                                                   pack_bf16x2(v[j][4 * jj + 2], v[j][4 * jj + 3]));
                    }
                });
            };
            const std::true_type T;
            const std::false_type F;
            if (mark) {
                body(F, F, F);
            } else if (a.bias) {
                if (!a.z) body(T, F, F);
                else if (zcoh) body(T, T, T);
                else body(T, T, F);
            } else {
                if (!a.z) body(F, F, F);
                else if (zcoh) body(F, T, T);
                else body(F, T, F);
            }
        }
        return;
    }
    mid_epilogue();
#pragma unroll
    for (int j = 0; j < MB; ++j) {
        const int64_t row = m0 + wm * TM + j * 32 + l32;
        if (row >= a.M) continue;
        if (PARTIAL) {
            float *pp = a.partial + ((int64_t)sp * a.M + row) * a.N;
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int64_t col = n0 + wn * TN + i * 32 + 8 * jj + 4 * half;
                    for (int e = 0; e < 4; ++e)
                        if (col + e < a.N) pp[col + e] = acc[i][j][4 * jj + e];
                }
        } else if (mark) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) store_nan4(a, row, n0 + wn * TN + i * 32 + 8 * jj + 4 * half);
        } else {
            int64_t zrow;
            const bool ok = row_request(a, row, zrow);
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int64_t col = n0 + wn * TN + i * 32 + 8 * jj + 4 * half;
                    if (col < a.N)
                        epilogue4<ZCOH>(a, row, zrow, ok, col, acc[i][j][4 * jj], acc[i][j][4 * jj + 1], acc[i][j][4 * jj + 2],
                                  acc[i][j][4 * jj + 3]);
                }
        }
    }
}

// One LDS variable per stage: the compiler gives each its own alias scope, so reading one stage
// does not wait for copies still in flight into another.
#define IKBO_GEMM_LDS(G, NBUF)                                                                                         \
    __shared__ uint4 sx0[G::XCH], sx1[G::XCH], sx2[NBUF > 2 ? G::XCH : 1], sx3[NBUF > 3 ? G::XCH : 1];              \
    __shared__ uint4 sw0[G::WCH], sw1[G::WCH], sw2[NBUF > 2 ? G::WCH : 1], sw3[NBUF > 3 ? G::WCH : 1];              \
    uint4 *const sx[4] = {sx0, sx1, sx2, sx3};                                                                      \
    uint4 *const sw[4] = {sw0, sw1, sw2, sw3}

template <int WGM, int WGN, int TM, int TN, int TBK, int NBUF, bool DMA, bool PARTIAL, bool STG>
__global__ __launch_bounds__(WGM *WGN * 64) void gemm_bf16_t(GemmArgs a, int32_t tiles_m, int32_t tiles_n,
                                                            int32_t k_per_split) {
    using G = GemmShape<WGM, WGN, TM, TN, TBK>;
    IKBO_GEMM_LDS(G, NBUF);
    const int64_t total = (int64_t)tiles_m * tiles_n * a.splits;
    int64_t t = xcd_tile(blockIdx.x, total);
    if (t < 0) return;
    int nt, mt, sp;
    if constexpr (!PARTIAL) {
        // groups of kGemmGroupM row blocks: within a group the column tile changes slowest, so
        // consecutive tiles share one weight tile and the column tiles of a row block (which
        // share its activation tile) are kGemmGroupM tiles apart, still running together on
        // the XCD
        const int64_t gsz = (int64_t)kGemmGroupM * tiles_n, g = t / gsz, r = t % gsz;
        const int64_t rows = min((int64_t)kGemmGroupM, (int64_t)tiles_m - g * kGemmGroupM);
        nt = (int)(r / rows);
        mt = (int)(g * kGemmGroupM + r % rows);
        sp = 0;
    } else {
        nt = (int)(t % tiles_n);
        t /= tiles_n;
        mt = (int)(t % tiles_m);
        sp = (int)(t / tiles_m);
    }
    gemm_tile<WGM, WGN, TM, TN, TBK, NBUF, DMA, PARTIAL, false, STG>(a, mt, nt, sp, k_per_split, sx, sw, [] {});
}

// ----------------------------------------------------------------------------------------------
// fp32 inputs: a plain LDS-tiled FMA GEMM (64 x 64 tile, 16-deep k steps, 4 x 4 per thread), same
// epilogue and split-K contract as the bf16 kernel.
constexpr int FBM = 64, FBN = 64, FBK = 16;

template <bool PARTIAL>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a, int32_t tiles_m, int32_t tiles_n, int32_t k_per_split) {
    __shared__ float xs[FBK][FBM + 4];
    __shared__ float ws[FBK][FBN + 4];
    const int64_t total = (int64_t)tiles_m * tiles_n * a.splits;
    int64_t t = xcd_tile(blockIdx.x, total);
    if (t < 0) return;
    const int nt = (int)(t % tiles_n);
    t /= tiles_n;
    const int mt = (int)(t % tiles_m);
    const int sp = (int)(t / tiles_m);
    const int64_t m0 = (int64_t)mt * FBM;
    const int n0 = nt * FBN;
    const int kbeg = sp * k_per_split;
    const int kend = min(a.K, kbeg + k_per_split);
    const int tid = threadIdx.x, tm = tid >> 4, tn = tid & 15;
    float acc[4][4] = {};
    for (int k0 = kbeg; k0 < kend; k0 += FBK) {
        for (int i = tid; i < FBM * FBK; i += 256) {
            const int r = i / FBK, kk = i % FBK;
            const int64_t gm = m0 + r;
            const int gk = k0 + kk;
            xs[kk][r] = (gm < a.M && gk < kend) ? ((const float *)a.x)[gm * a.ldx + gk] : 0.0f;
            const int gn = n0 + r;
            float wv = 0.0f;
            if (gn < a.N && gk < kend)
                wv = gn < a.n0 ? ((const float *)a.w0)[(int64_t)gn * a.K + gk] : ((const float *)a.w1)[(int64_t)(gn - a.n0) * a.K + gk];
            ws[kk][r] = wv;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < FBK; ++kk) {
            float xv[4], wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) { xv[i] = xs[kk][tm * 4 + i]; wv[i] = ws[kk][tn * 4 + i]; }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(xv[i], wv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + tm * 4 + i;
        if (row >= a.M) continue;
        const int64_t col = n0 + tn * 4;
        if (col >= a.N) continue;
        if (PARTIAL) {
            float *pp = a.partial + ((int64_t)sp * a.M + row) * a.N;
            for (int j = 0; j < 4; ++j)
                if (col + j < a.N) pp[col + j] = acc[i][j];
        } else {
            int64_t zrow;
            const bool ok = row_request(a, row, zrow);
            epilogue4(a, row, zrow, ok, col, acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        }
    }
}

// One element of the split-K reduction: partials summed in split order, then the request-group
// epilogue (columns below n_split) or the raw sum into Z. COH: the partials were written during
// this launch by other workgroups and are read with agent-coherent loads.
template <bool COH = false>
__device__ __forceinline__ void reduce_elem(const float *partial, int32_t splits, int64_t M, int32_t N, int32_t n_split,
                                            const float *bias0, int32_t act, void *out0, int32_t out0_f32, int64_t ld0,
                                            float *out1, int64_t row, int32_t col) {
    const int64_t total = M * N, i = row * N + col;
    float s = 0.0f;
    for (int sp = 0; sp < splits; ++sp) s += COH ? load_coherent(partial + (int64_t)sp * total + i) : partial[(int64_t)sp * total + i];
    if (col < n_split) {
        float v = s + (bias0 ? bias0[col] : 0.0f);
        v = apply_act(act, v);
        if (out0_f32) ((float *)out0)[row * ld0 + col] = v;
        else ((uint16_t *)out0)[row * ld0 + col] = f32_to_bf16(v);
    } else {
        out1[row * (N - n_split) + (col - n_split)] = s;
    }
}

// Four consecutive columns col .. col + 3 of the split-K reduction (N and n_split multiples of 4,
// splits <= kMaxSplits): the partials of every split are loaded before the first add (a load per
// split beyond `splits` rereads the last one and is not added), then summed in split order, which
// gives the same bits as reduce_elem.
constexpr int kMaxSplits = 16;
template <bool COH = false>
__device__ __forceinline__ void reduce_quad(const float *partial, int32_t splits, int64_t M, int32_t N, int32_t n_split,
                                            const float *bias0, int32_t act, void *out0, int32_t out0_f32, int64_t ld0,
                                            float *out1, int64_t row, int32_t col) {
    const int64_t total = M * N, i = row * N + col;
    float4 p[kMaxSplits];
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp) {
        const float *q = partial + (int64_t)min(sp, splits - 1) * total + i;
        if constexpr (COH) {
            const uint64_t lo = __hip_atomic_load((const uint64_t *)q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint64_t hi = __hip_atomic_load((const uint64_t *)q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            p[sp] = make_float4(__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                                __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32)));
        } else {
            p[sp] = *(const float4 *)q;
        }
    }
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp)
        if (sp < splits) {
            v[0] += p[sp].x; v[1] += p[sp].y; v[2] += p[sp].z; v[3] += p[sp].w;
        }
    if (col < n_split) {
        if (bias0) {
            const float4 b = *(const float4 *)(bias0 + col);
            v[0] += b.x; v[1] += b.y; v[2] += b.z; v[3] += b.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = apply_act(act, v[e]);
        if (out0_f32) *(float4 *)((float *)out0 + row * ld0 + col) = make_float4(v[0], v[1], v[2], v[3]);
        else *(uint2 *)((uint16_t *)out0 + row * ld0 + col) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    } else {
        *(float4 *)(out1 + row * (N - n_split) + (col - n_split)) = make_float4(v[0], v[1], v[2], v[3]);
    }
}

__device__ __forceinline__ bool reduce_quads_ok(int32_t splits, int32_t N, int32_t n_split) {
    return splits >= 1 && splits <= kMaxSplits && (N & 3) == 0 && (n_split & 3) == 0;
}

__global__ void splitk_reduce_kernel(const float *partial, int32_t splits, int64_t M, int32_t N, int32_t n_split,
                                     const float *bias0, int32_t act, void *out0, int32_t out0_f32, int64_t ld0,
                                     float *out1) {
    const int64_t total = M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if (reduce_quads_ok(splits, N, n_split)) {
        for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < total / 4; q += stride) {
            const int64_t row = 4 * q / N;
            reduce_quad(partial, splits, M, N, n_split, bias0, act, out0, out0_f32, ld0, out1, row, (int32_t)(4 * q - row * N));
        }
        return;
    }
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t row = i / N;
        reduce_elem(partial, splits, M, N, n_split, bias0, act, out0, out0_f32, ld0, out1, row, (int32_t)(i - row * N));
    }
}

// Zero-padded copy of bf16 rows (the alignment rule of Sec. 4.2.4): dst[r, j] = src[r, j] for j < k
// and 0 for k <= j < kp, with src rows k elements long and dst rows kp (a multiple of 8). One
// thread per 16-byte chunk of a destination row; the source rows are not 16-byte aligned, so their
// elements are read one by one.
__global__ void pad_rows_bf16_kernel(const uint16_t *src, int64_t rows, int32_t k, uint16_t *dst, int32_t kp) {
    const int64_t chunks = kp / 8, total = rows * chunks;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / chunks;
        const int32_t j0 = (int32_t)(i - r * chunks) * 8;
        const uint16_t *sp = src + r * k;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = j0 + 2 * e < k ? sp[j0 + 2 * e] : 0u;
            const uint32_t hi = j0 + 2 * e + 1 < k ? sp[j0 + 2 * e + 1] : 0u;
            w[e] = lo | (hi << 16);
        }
        *(uint4 *)(dst + r * kp + j0) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// ----------------------------------------------------------------------------------------------
// Persistent LCB layer (request/candidate co-scheduling, ROCS Sec. 4.2.3). sync layout (int32):
// [0] request item counter, [1 .. 8] candidate tile counter of each XCD, [9] wait ran out,
// [16 .. 16 + Q) arrivals per request tile, [16 + Q .. 16 + 2Q) ready flags (Q request tiles).
constexpr int kSyncHead = 16;

// A flag is read with a compare-exchange that never matches (flags hold 0 or 1): an atomic, so it
// sees the device-wide value as the claim and arrival counters do. It is relaxed: the data a flag
// guards is read with agent-coherent loads after the flag is seen, so no acquire fence (on this
// part an L2 invalidate) is needed. A flag is set by a release fence (the writer's data reaches
// memory) and an atomic exchange.
__device__ __forceinline__ int32_t flag_poll(int32_t *p) {
    int32_t v = 2;
    __hip_atomic_compare_exchange_strong(p, &v, 2, __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return v;
}
__device__ __forceinline__ void flag_release(int32_t *p, int32_t v) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Values every lane of a wave holds alike, moved to scalar registers so that the branches and loop
// exits they decide are uniform. The control flow of the persistent loop below must be uniform:
// with a loop exit that the compiler takes as divergent (a value read from LDS into a vector
// register), it may run the loop for the other lanes while the one lane that claims items and
// sets flags waits outside it, and the workgroup never ends.
// lane 0 of the calling wave applies op, every lane gets its result (call with all lanes active)
template <typename Op>
__device__ __forceinline__ int32_t lane0(int lane, Op op) {
    int32_t v = 0;
    if (lane == 0) v = op();
    return __builtin_amdgcn_readfirstlane(v);
}

template <bool DMA_R, bool DMA_C, bool STG>
__global__ __launch_bounds__(kGemmThreads) void lcb_fused_kernel(LcbFusedArgs f) {
    using G = GemmShape<kWGM, kWGN, kTM, kTN, BK>;
    IKBO_GEMM_LDS(G, 2);
    __shared__ int64_t s_item;
    __shared__ int32_t s_flag;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int xcd = blockIdx.x % kNumXcd;
    const GemmArgs &rq = f.req, &cd = f.cand;
    const int32_t rtm = (int32_t)((rq.M + BM - 1) / BM), rtn = (rq.N + BN - 1) / BN;
    const int32_t splits = rq.splits;
    const int64_t req_tiles = (int64_t)rtm * rtn, req_items = req_tiles * splits;
    const int32_t rkps = (int32_t)((((int64_t)rq.K + splits - 1) / splits + BK - 1) / BK * BK);
    const int32_t ctn = (cd.N + BN - 1) / BN;
    const int64_t cand_tiles = ((cd.M + BM - 1) / BM) * ctn;
    const int64_t per_xcd = (cand_tiles + kNumXcd - 1) / kNumXcd;
    const int64_t c_beg = xcd * per_xcd, c_end = min(cand_tiles, c_beg + per_xcd);
    int32_t *arrive = f.sync + kSyncHead, *ready = f.sync + kSyncHead + req_tiles;
    using CG = GemmShape<kWGM, kWGN, kTM, kTN, BK>;

    // wave 0 claims the next item (request items first, then this XCD's candidate tiles) and
    // hands it to the workgroup through LDS. Bidirectional order (Sec. 4.2.3): request items go
    // out ascending from one device-wide counter, candidate tiles descending from the end of each
    // XCD's range (with claims the balance comes from the claims themselves; the order is the
    // pages').
    auto claim = [&]() -> int64_t {
        if (wave == 0) {
            int64_t it = -1;
            const int32_t r = lane0(lane, [&] { return atomicAdd(&f.sync[0], 1); });
            if (r < req_items) {
                it = r;
            } else {
                const int64_t c = c_end - 1 - lane0(lane, [&] { return atomicAdd(&f.sync[1 + xcd], 1); });
                if (c >= c_beg) it = req_items + c;
            }
            if (lane == 0) s_item = it;
        }
        __syncthreads();
        const int64_t it = uniform64(s_item);
        __syncthreads();
        return it;
    };
    // request tiles wave 0 has seen ready (the first 64), so later tiles do not poll them again
    uint64_t known = 0;
    int64_t item = claim();
    bool prefetched = false;
    for (;;) {
        if (item < 0) break;
        if (item < req_items) {
            // request tile, one k split; splits of a tile are consecutive items
            const int64_t tile = item / splits;
            const int sp = (int)(item % splits);
            const int mt = (int)(tile / rtn), nt = (int)(tile % rtn);
            gemm_tile<kWGM, kWGN, kTM, kTN, BK, 2, DMA_R, true, false, false>(rq, mt, nt, sp, rkps, sx, sw, [] {});
            // every wave's partial stores have reached the L2; one release (an L2 write-back) by
            // wave 0 then puts them in memory before the arrival is counted
            wait_vmcnt<0>();
            __syncthreads();
            if (wave == 0) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                const int32_t a = lane0(lane, [&] { return atomicAdd(&arrive[tile], 1); });
                if (lane == 0) s_flag = a == splits - 1;
            }
            __syncthreads();
            if (__builtin_amdgcn_readfirstlane(s_flag)) {
                // the last split of the tile: every other split's partials reached memory before its
                // arrival was counted; they are read with coherent loads
                const int64_t m0 = (int64_t)mt * BM;
                const int n0 = nt * BN;
                float *z = const_cast<float *>(cd.z);
                if (reduce_quads_ok(splits, rq.N, f.n_split)) {
                    for (int i = tid; i < BM * BN / 4; i += kGemmThreads) {
                        const int64_t row = m0 + i / (BN / 4);
                        const int col = n0 + 4 * (i % (BN / 4));
                        if (row < rq.M && col < rq.N)
                            reduce_quad<true>(rq.partial, splits, rq.M, rq.N, f.n_split, f.bias0, f.act, f.out0,
                                              f.out0_f32, f.n_split, z, row, col);
                    }
                } else {
                    for (int i = tid; i < BM * BN; i += kGemmThreads) {
                        const int64_t row = m0 + i / BN;
                        const int col = n0 + i % BN;
                        if (row < rq.M && col < rq.N)
                            reduce_elem<true>(rq.partial, splits, rq.M, rq.N, f.n_split, f.bias0, f.act, f.out0,
                                              f.out0_f32, f.n_split, z, row, col);
                    }
                }
                wait_vmcnt<0>();                   // Z and Y_r have reached the L2 ...
                __syncthreads();
                if (wave == 0 && lane == 0 && f.publish) flag_release(&ready[tile], 1);   // ... memory, then the flag
            }
            item = claim();
            prefetched = false;
        } else {
            const int64_t c = item - req_items;
            const int mt = (int)(c / ctn), nt = (int)(c % ctn);
            int64_t next = -1;
            // After the main loop: wave 0 waits for the request tiles holding Z columns
            // nt * BN .. nt * BN + BN - 1 (all request row blocks; bounded in time, and once any wait
            // has run out, sync[9], every wait stops) and claims this XCD's next candidate tile,
            // whose first k step then goes into LDS stage 0 (free once the main loop has ended)
            // while this tile's epilogue runs (issued in the epilogue, after its first loads).
            auto pre = [&] {
                if (wave == 0) {
                    const int tn0 = (f.n_split + nt * BN) / BN;
                    const int tn1 = min(rtn - 1, (f.n_split + min(cd.N, nt * BN + BN) - 1) / BN);
                    const int64_t deadline = (int64_t)wall_clock64() + f.wait_ticks;
                    bool ok = true;
                    for (int tm = 0; tm < rtm && ok; ++tm)
                        for (int tn = tn0; tn <= tn1 && ok; ++tn) {
                            const int64_t ti = (int64_t)tm * rtn + tn;
                            if (ti < 64 && ((known >> ti) & 1)) continue;
                            if (lane0(lane, [&] { return flag_poll(&f.sync[9]); }) != 0) ok = false;
                            while (ok && lane0(lane, [&] { return flag_poll(&ready[ti]); }) == 0) {
                                if ((int64_t)wall_clock64() > deadline ||
                                    lane0(lane, [&] { return flag_poll(&f.sync[9]); }) != 0) {
                                    ok = false;
                                    lane0(lane, [&] {
                                        return __hip_atomic_exchange(&f.sync[9], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                                    });
                                } else {
                                    __builtin_amdgcn_s_sleep(4);
                                }
                            }
                            if (ok && ti < 64) known |= 1ull << ti;
                        }
                    const int64_t c2 = c_end - 1 - lane0(lane, [&] { return atomicAdd(&f.sync[1 + xcd], 1); });
                    if (lane == 0) {
                        s_flag = ok;
                        s_item = c2 >= c_beg ? req_items + c2 : -1;
                    }
                }
                __syncthreads();
                next = uniform64(s_item);
                return __builtin_amdgcn_readfirstlane(s_flag) != 0;
            };
            auto mid = [&] {
                if constexpr (DMA_C) {
                    if (next >= 0) {
                        const int64_t c2 = next - req_items;
                        const DmaTile t = dma_tile<CG, BK>(cd, (int)(c2 / ctn), (int)(c2 % ctn), 0, cd.K, wave, lane);
                        dma_fetch<CG, BK>(cd, t, 0, sx[0], sw[0], wave);
                    }
                }
            };
            // the epilogue reads Z with plain loads when its lines hold one request tile each, else
            // with coherent loads; no acquire fence, which would invalidate the XCD's L2 (and the
            // weight and activation tiles the other workgroups there hold) per tile
            // when a wait ran out, pre returns false and the epilogue marks the whole tile NaN without
            // reading Z: a line of Z read before its tile is final could otherwise stay in this XCD's
            // L2 and reach a later tile's plain loads
            gemm_tile<kWGM, kWGN, kTM, kTN, BK, 2, DMA_C, false, true, STG>(cd, mt, nt, 0, cd.K, sx, sw, pre, prefetched, mid);
            item = next;
            prefetched = DMA_C && next >= 0;
        }
    }
    wait_vmcnt<0>();     // no copy may still be writing LDS when the workgroup ends
}

}  // namespace

int32_t request_gemm_splits(int64_t M, int32_t N, int32_t K, int in_f32) {
    const int64_t bm = in_f32 ? FBM : BM, bn = in_f32 ? FBN : BN, bk = in_f32 ? FBK : BK;
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    if (tiles <= 0 || K <= 0) return 1;
    int64_t s = (256 + tiles - 1) / tiles;        // aim for about one workgroup per CU
    const int64_t ksteps = (K + bk - 1) / bk;
    if (s > ksteps / 2) s = ksteps / 2;           // keep at least two k steps per split
    if (s > 16) s = 16;
    if (s < 1) s = 1;
    return (int32_t)s;
}

// the direct-copy conditions of launch_gemm for one bf16 GEMM with k split kps
static bool gemm_dma_ok(const GemmArgs &a, int32_t kps) {
    return a.K % BK == 0 && kps % BK == 0 && a.ldx % 8 == 0 && ((uintptr_t)a.x & 15) == 0 &&
           ((uintptr_t)a.w0 & 15) == 0 && ((uintptr_t)a.w1 & 15) == 0 && (a.n0 >= a.N || a.n0 % BN == 0) &&
           (int64_t)BM * a.ldx * 2 < (1LL << 31) && (int64_t)BN * a.K * 2 < (1LL << 31);
}

// the staged epilogue stores 16-byte pieces of output rows: 16-byte aligned output and rows
static bool out_staging_ok(const GemmArgs &a) {
    return ((uintptr_t)a.out & 15) == 0 && (a.out_f32 || (a.ldo & 7) == 0);
}

static int32_t k_per_split(const GemmArgs &a) {
    const int splits = a.partial ? (a.splits > 0 ? a.splits : 1) : 1;
    int32_t kps = (int32_t)((((int64_t)a.K + splits - 1) / splits + BK - 1) / BK * BK);
    return kps <= 0 ? BK : kps;
}

hipError_t launch_gemm(const GemmArgs &a, hipStream_t s) {
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    const int splits = a.partial ? (a.splits > 0 ? a.splits : 1) : 1;
    GemmArgs b = a;
    b.splits = splits;
    const int bm = a.in_f32 ? FBM : BM, bn = a.in_f32 ? FBN : BN, bk = a.in_f32 ? FBK : BK;
    const int64_t tm = (a.M + bm - 1) / bm, tn = (a.N + bn - 1) / bn;
    int32_t kps = (int32_t)((((int64_t)a.K + splits - 1) / splits + bk - 1) / bk * bk);
    if (kps <= 0) kps = bk;
    const int64_t total = tm * tn * splits;
    const int64_t grid = ((total + kNumXcd - 1) / kNumXcd) * kNumXcd;
    if (grid > 0x7fffffffLL || tm > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (a.in_f32) {
        if (a.partial) hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, b, (int32_t)tm, (int32_t)tn, kps);
        else hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, b, (int32_t)tm, (int32_t)tn, kps);
    } else {
        // direct copies: k tiles whole, 16-byte aligned rows, buffer ranges within 32 bits, and no
        // tile across the w0 / w1 boundary
        const bool dma = gemm_dma_ok(a, kps);
#define IKBO_GEMM(D, P, S)                                                                                           \
    hipLaunchKernelGGL((gemm_bf16_t<kWGM, kWGN, kTM, kTN, BK, 2, D, P, S>), dim3((unsigned)grid), dim3(kGemmThreads),   \
                       0, s, b, (int32_t)tm, (int32_t)tn, kps)
        const bool stg = out_staging_ok(a);
        if (dma) {
            if (a.partial) IKBO_GEMM(true, true, false);
            else if (stg) IKBO_GEMM(true, false, true);
            else IKBO_GEMM(true, false, false);
        } else {
            if (a.partial) IKBO_GEMM(false, true, false);
            else if (stg) IKBO_GEMM(false, false, true);
            else IKBO_GEMM(false, false, false);
        }
#undef IKBO_GEMM
    }
    return hipGetLastError();
}

int64_t wall_clock_ticks(double seconds) {
    static int khz = 0;
    if (khz <= 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
            khz <= 0)
            khz = 100000;     // 100 MHz
    }
    return (int64_t)(seconds * 1e3 * khz);
}

int64_t lcb_fused_sync_ints(int64_t M, int32_t N) {
    return kSyncHead + 2 * ((M + BM - 1) / BM) * (int64_t)((N + BN - 1) / BN);
}

bool lcb_fused_supported(const GemmArgs &req, const GemmArgs &cand) {
    return !req.in_f32 && !cand.in_f32 && req.partial && req.splits >= 1 && req.M > 0 && cand.M > 0 &&
           req.N > 0 && cand.N > 0 && gemm_dma_ok(req, k_per_split(req)) && gemm_dma_ok(cand, cand.K);
}

hipError_t launch_lcb_fused(const LcbFusedArgs &f, hipStream_t s) {
    if (!lcb_fused_supported(f.req, f.cand)) return hipErrorInvalidValue;
    const int64_t nsync = lcb_fused_sync_ints(f.req.M, f.req.N);
    hipError_t e = launch_fill_i32(f.sync, nsync, 0, s);
    if (e != hipSuccess) return e;
    static int cus = 0;
    if (cus <= 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
    }
    // one workgroup per CU (the LDS stages take 128 KiB), a multiple of the XCD count
    const int64_t items = (int64_t)((f.req.M + BM - 1) / BM) * ((f.req.N + BN - 1) / BN) * f.req.splits +
                          ((f.cand.M + BM - 1) / BM) * ((f.cand.N + BN - 1) / BN);
    int64_t grid = min((int64_t)cus, items);
    grid = ((grid + kNumXcd - 1) / kNumXcd) * kNumXcd;
    if (out_staging_ok(f.cand)) hipLaunchKernelGGL((lcb_fused_kernel<true, true, true>), dim3((unsigned)grid), dim3(kGemmThreads), 0, s, f);
    else hipLaunchKernelGGL((lcb_fused_kernel<true, true, false>), dim3((unsigned)grid), dim3(kGemmThreads), 0, s, f);
    return hipGetLastError();
}

hipError_t launch_pad_rows_bf16(const void *src, int64_t rows, int32_t k, void *dst, int32_t kp, hipStream_t s) {
    const int64_t total = rows * (int64_t)(kp / 8);
    if (total <= 0) return hipSuccess;
    int64_t g = (total + 255) / 256;
    if (g > 65536) g = 65536;
    hipLaunchKernelGGL(pad_rows_bf16_kernel, dim3((unsigned)g), dim3(256), 0, s, (const uint16_t *)src, rows, k,
                       (uint16_t *)dst, kp);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float *partial, int32_t splits, int64_t M, int32_t N, int32_t n_split,
                                const float *bias0, int32_t act, void *out0, int32_t out0_f32, int64_t ld0,
                                float *out1, hipStream_t s) {
    const int64_t total = M * N;
    if (total <= 0) return hipSuccess;
    int64_t g = (total + 255) / 256;
    if (g > 65536) g = 65536;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)g), dim3(256), 0, s, partial, splits, M, N, n_split, bias0,
                       act, out0, out0_f32, ld0, out1);
    return hipGetLastError();
}

}  // namespace ikbo
