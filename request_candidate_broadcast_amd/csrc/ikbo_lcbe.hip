// ROCSified LCB in its embedding-matrix (row-axis) form, two groups (ROCS Sec. 3.1.2, Eq. 5-6),
// followed by the group-local normalisation of Sec. 3.1.3, Eq. 7:
//   Y^R_r = Norm_R( W_RR X^R_r )                                     [k_r, d]
//   Y^C_c = Norm_C( W_CR X^R_{m(c)} + W_CC X^C_c )                   [k_c, d]
// The request-derived term Z_r = W_CR X^R_r (the contribution the pages single out after Eq. 6)
// is computed once per request, at the request batch size, into an fp32 workspace, and added to
// each candidate's product in the candidate kernel's epilogue through m: the broadcast is
// resolved in the kernel, never materialised. Norm is per embedding row over d (LayerNorm with
// the biased variance, or RMSNorm), then * gamma + beta of the row's group.
//
// Candidate kernel (bf16, d in {32, 64, 128}, n_c and k_c <= 64): one wave per candidate, each
// wave taking a contiguous run of candidates so a request's Z rows are loaded once per run. The
// contraction runs over the embedding rows of X^C (its slow axis), so X^C_c goes to a per-wave
// LDS tile and comes back transposed (ds_read_b64_tr_b16, 16-bit data transposed across each
// 16-lane group) as the A operand of v_mfma_f32_32x32x16_bf16; W_CC is the B operand, held in
// registers for the whole launch. Products are computed transposed (D^T = X^T W^T) so each lane
// owns one output row o: the row statistics of the norm are a per-lane sum plus one exchange
// between the two 32-lane halves. Results go through an LDS stage and leave as whole rows,
// consecutive lanes on consecutive 16-byte chunks. The next candidate's X^C is loaded into
// registers while the current one is computed. HBM-bound: 2 n_c d bytes in and k_c d outputs
// per candidate for 2 k_c n_c d FLOP.
//
// Request kernel and the generic candidate kernel (fp32 inputs, other shapes): one wave per
// output row, lanes over d, products summed in index order in fp32.
#include "ikbo_device.h"
#include "ikbo_launch.h"

#include <math.h>

namespace ikbo {
namespace {

constexpr int kLeWaves = 4;            // waves per workgroup (every kernel here)

// One input element; the dtype is a template parameter so no load sits behind a branch.
template <bool F32>
__device__ __forceinline__ float le_in(const void *p, int64_t i) {
    if constexpr (F32) return ((const float *)p)[i];
    else return __uint_as_float((uint32_t)((const uint16_t *)p)[i] << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s);
    return v;
}

// Sum over lanes l and l ^ 32 (v_permlane32_swap hands each half the other's value).
__device__ __forceinline__ float halves_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Keeps the compiler from moving LDS accesses of this wave across the point: the tile and the
// stage are written and read by different lanes of the same wave.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Eq. 7 on one output row held by a whole wave: lane l holds columns l + 64 t (t < T), valid
// below d. Leaves v normalised, times gamma plus beta.
template <int T>
__device__ __forceinline__ void norm_row(float (&v)[T], int d, int lane, int norm, float eps, const float *g,
                                         const float *b) {
    if (norm == 0) return;
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < T; ++t)
        if (lane + 64 * t < d) s += norm == 1 ? v[t] : v[t] * v[t];
    s = wave_sum(s);
    float shift = 0.0f, rstd;
    if (norm == 1) {
        shift = s / (float)d;
        float q = 0.0f;
#pragma unroll
        for (int t = 0; t < T; ++t)
            if (lane + 64 * t < d) q += (v[t] - shift) * (v[t] - shift);
        rstd = 1.0f / sqrtf(wave_sum(q) / (float)d + eps);
    } else {
        rstd = 1.0f / sqrtf(s / (float)d + eps);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int j = lane + 64 * t;
        if (j < d) v[t] = (v[t] - shift) * rstd * (g ? g[j] : 1.0f) + (b ? b[j] : 0.0f);
    }
}

__device__ __forceinline__ void store_out(void *y, int out_f32, int64_t i, float v) {
    if (out_f32) ((float *)y)[i] = v;
    else ((uint16_t *)y)[i] = f32_to_bf16(v);
}

// Request side: per request r, rows [0, kr) are Y^R (= W_RR X^R_r, normalised) and rows
// [kr, kr + kc) are Z_r = W_CR X^R_r (fp32, no norm); kr = 0 without y_r, kc = 0 without z.
template <bool F32>
__global__ __launch_bounds__(kLeWaves * 64) void lcbe_request_kernel(LcbeArgs a) {
    constexpr int T = kLcbeMaxDim / 64;
    const int lane = threadIdx.x & 63;
    const int kr = a.y_r ? a.k_r : 0, kc = a.z ? a.k_c : 0, per = kr + kc;
    const int64_t rows = a.R * per;
    for (int64_t w = (int64_t)blockIdx.x * kLeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); w < rows;
         w += (int64_t)gridDim.x * kLeWaves) {
        const int64_t r = w / per;
        const int o = (int)(w - r * per);
        const bool is_y = o < kr;
        const void *wsrc = is_y ? a.w_rr : a.w_cr;
        const int orow = is_y ? o : o - kr;
        float v[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int j = lane + 64 * t;
            float s = 0.0f;
            // unrolled so the loads of eight k are in flight together (the sum stays in k order)
            if (j < a.d)
#pragma unroll 8
                for (int k = 0; k < a.n_r; ++k)
                    s = __builtin_fmaf(le_in<F32>(wsrc, (int64_t)orow * a.n_r + k),
                                       le_in<F32>(a.x_r, (r * a.n_r + k) * a.d + j), s);
            v[t] = s;
        }
        if (!is_y) {
#pragma unroll
            for (int t = 0; t < T; ++t)
                if (lane + 64 * t < a.d) a.z[(r * a.k_c + orow) * a.d + lane + 64 * t] = v[t];
            continue;
        }
        norm_row<T>(v, a.d, lane, a.norm, a.eps, a.g_r, a.b_r);
#pragma unroll
        for (int t = 0; t < T; ++t)
            if (lane + 64 * t < a.d) store_out(a.y_r, a.out_f32, (r * a.k_r + o) * a.d + lane + 64 * t, v[t]);
    }
}

// Candidates, any shape and dtype: one wave per output row (c, o).
template <bool F32>
__global__ __launch_bounds__(kLeWaves * 64) void lcbe_cand_generic_kernel(LcbeArgs a) {
    constexpr int T = kLcbeMaxDim / 64;
    const int lane = threadIdx.x & 63;
    const int64_t rows = a.C * a.k_c;
    for (int64_t w = (int64_t)blockIdx.x * kLeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); w < rows;
         w += (int64_t)gridDim.x * kLeWaves) {
        const int64_t c = w / a.k_c;
        const int o = (int)(w - c * a.k_c);
        int64_t cursor = -1;
        const int64_t r = uniform64(cand_request(a.off, a.map, a.R, c, cursor));
        float v[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int j = lane + 64 * t;
            float s = 0.0f;
            if (j < a.d && r >= 0) {
#pragma unroll 8
                for (int k = 0; k < a.n_c; ++k)
                    s = __builtin_fmaf(le_in<F32>(a.w_cc, (int64_t)o * a.n_c + k),
                                       le_in<F32>(a.x_c, (c * a.n_c + k) * a.d + j), s);
                s += a.z[(r * a.k_c + o) * a.d + j];
            }
            v[t] = s;
        }
        if (r >= 0) norm_row<T>(v, a.d, lane, a.norm, a.eps, a.g_c, a.b_c);
#pragma unroll
        for (int t = 0; t < T; ++t)
            if (lane + 64 * t < a.d) store_out(a.y_c, a.out_f32, w * a.d + lane + 64 * t, v[t]);
    }
}

// JB = d / 32 column blocks, KST = 16-row k steps over the padded n_c, OB = 32-row output blocks
// (k_c <= 32 OB), WPE = waves per SIMD the register budget is sized for.
template <int JB, int KST, int OB, int WPE>
__global__ __launch_bounds__(kLeWaves * 64) __attribute__((amdgpu_waves_per_eu(WPE, 8))) void lcbe_cand_kernel(LcbeArgs a) {
    constexpr int D = 32 * JB;
    constexpr int NP = 16 * KST;                          // input rows in the tile (zero past n_c)
    constexpr int XROW = 2 * D + (D == 32 ? 0 : 64);      // bytes per tile row: rows 4 apart hit other banks
    constexpr int SW = D + 4;                             // stage row stride (floats)
    constexpr int XBYTES = NP * XROW, SBYTES = 32 * SW * 4;
    constexpr int REGION = XBYTES > SBYTES ? XBYTES : SBYTES;
    constexpr int CPR = D / 8;                            // 16-byte chunks per input row
    constexpr int NLD = NP * CPR / 64;                    // chunks per lane per tile
    constexpr int C8 = D / 8;                             // 8-column chunks per output row
    constexpr int RPI = 64 / C8;                          // output rows per flush step
    constexpr bool PREFETCH = NLD <= 4;                   // next tile in registers during this one
    constexpr bool ZCACHE = OB * JB <= 2;                 // a request's Z rows in registers per run
    static_assert(NP * CPR % 64 == 0, "tile chunks must fill whole waves");
    // The tile and the stage share one region: a candidate's tile is read into registers before
    // its stage is written, and the next tile is written after the stage has been flushed.
    __shared__ __attribute__((aligned(16))) char region_all[kLeWaves][REGION];
    __shared__ float2 stat_all[kLeWaves][32];             // per output row: mean, 1 / std
    __shared__ float gb[2][D];                            // gamma, beta of the candidate group

    const int lane = threadIdx.x & 63, l32 = lane & 31, half = lane >> 5;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int i = threadIdx.x; i < 2 * D; i += kLeWaves * 64) {
        const float *src = i < D ? a.g_c : a.b_c;
        gb[i / D][i % D] = src ? src[i % D] : (i < D ? 1.0f : 0.0f);
    }
    __syncthreads();

    char *reg = region_all[wid];
    float *st = (float *)reg;
    float2 *stat = stat_all[wid];
    const int64_t wave = (int64_t)blockIdx.x * kLeWaves + wid;
    const int64_t c0 = wave * a.chunk, c1 = min(a.C, c0 + a.chunk);
    if (c0 >= c1) return;

    // W_CC as B operand fragments: lane (o = l32, half) of k step s holds W_CC[o, k] for the eight
    // k the transposed tile read gives the A operand: 16 s + 4 half + {0..3}, 16 s + 8 + 4 half + {0..3}
    const uint16_t *wcc = (const uint16_t *)a.w_cc;
    bf16x8 wf[OB][KST];
#pragma unroll
    for (int ob = 0; ob < OB; ++ob)
#pragma unroll
        for (int s = 0; s < KST; ++s) {
            const int o = 32 * ob + l32;
            uint32_t p[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                uint32_t two = 0;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int e = 2 * t + u;
                    const int k = 16 * s + (e < 4 ? 4 * half + e : 8 + 4 * half + (e - 4));
                    const uint32_t bits = (o < a.k_c && k < a.n_c) ? wcc[o * a.n_c + k] : 0u;
                    two |= bits << (16 * u);
                }
                p[t] = two;
            }
            wf[ob][s] = __builtin_bit_cast(bf16x8, make_uint4(p[0], p[1], p[2], p[3]));
        }

    // transposed-read address of this lane within a 16-row, 32-column block of the tile
    const int g16 = lane >> 4, s16 = lane & 15;
    const int tr_off = (4 * (g16 >> 1) + (s16 >> 2)) * XROW + ((g16 & 1) * 16 + 4 * (s16 & 3)) * 2;

    const uint16_t *xc = (const uint16_t *)a.x_c;
    const int valid = a.n_c * CPR;                        // chunks of the tile that hold data
    uint4 pf[NLD];
    auto fetch = [&](int64_t c) __attribute__((always_inline)) {
        const uint4 *src = (const uint4 *)(xc + c * a.n_c * D);
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int q = lane + 64 * i;
            pf[i] = q < valid ? src[q] : make_uint4(0, 0, 0, 0);
        }
    };
    auto put = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int q = lane + 64 * i;
            *(uint4 *)(reg + (q / CPR) * XROW + (q % CPR) * 16) = pf[i];
        }
    };
    // Z rows of request r for output block ob, column block jb, in the accumulator layout
    auto zload = [&](int64_t r, int ob, int jb, float4 (&z)[4]) __attribute__((always_inline)) {
        const int o = 32 * ob + l32;
        const float *zr = a.z + (r * a.k_c + o) * D + 32 * jb + 4 * half;
#pragma unroll
        for (int g = 0; g < 4; ++g) z[g] = o < a.k_c ? *(const float4 *)(zr + 8 * g) : make_float4(0.f, 0.f, 0.f, 0.f);
    };

    float4 zf[ZCACHE ? OB : 1][ZCACHE ? JB : 1][4];
    int64_t have_r = -1, cursor = -1;
    const int q8 = lane % C8, r8 = lane / C8;
    if (PREFETCH) fetch(c0);
    for (int64_t c = c0; c < c1; ++c) {
        const int64_t r = uniform64(cand_request(a.off, a.map, a.R, c, cursor));
        if (!PREFETCH) fetch(c);
        wave_lds_fence();
        put();
        wave_lds_fence();
        if (PREFETCH && c + 1 < c1) fetch(c + 1);
        const int64_t ybase = c * a.k_c * D;
        if (r < 0) {
            for (int i = lane; i < a.k_c * D / 4; i += 64) {
                if (a.out_f32) *(float4 *)((float *)a.y_c + ybase + 4 * i) = make_float4(0.f, 0.f, 0.f, 0.f);
                else *(uint2 *)((uint16_t *)a.y_c + ybase + 4 * i) = make_uint2(0, 0);
            }
            continue;
        }
        if (ZCACHE && r != have_r) {
#pragma unroll
            for (int ob = 0; ob < OB; ++ob)
#pragma unroll
                for (int jb = 0; jb < JB; ++jb) zload(r, ob, jb, zf[ZCACHE ? ob : 0][ZCACHE ? jb : 0]);
            have_r = r;
        }
        // every fragment of the tile before the stage (same memory) is written
        bf16x8 xf[JB][KST];
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
#pragma unroll
            for (int s = 0; s < KST; ++s) {
                const char *p = reg + 16 * s * XROW + 64 * jb + tr_off;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 8 * XROW));
                xf[jb][s] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        wave_lds_fence();
#pragma unroll
        for (int ob = 0; ob < OB; ++ob) {
            if (32 * ob >= a.k_c) break;
            // Row statistics of output row 32 ob + l32 over this lane's columns, merged block by
            // block (Chan et al.'s pairwise update of count, mean and sum of squared deviations;
            // RMSNorm keeps the plain sum of squares in m2).
            float mean = 0.0f, m2 = 0.0f;
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                // lane (o = l32, half): acc[4 g + t] is column 32 jb + 8 g + 4 half + t of row 32 ob + o
                f32x16 acc;
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
                for (int s = 0; s < KST; ++s) acc = mfma_32x32x16_bf16(xf[jb][s], wf[ob][s], acc);
                float4 zb[4];
                if (ZCACHE) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) zb[g] = zf[ZCACHE ? ob : 0][ZCACHE ? jb : 0][g];
                } else {
                    zload(r, ob, jb, zb);
                }
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    acc[4 * g] += zb[g].x;
                    acc[4 * g + 1] += zb[g].y;
                    acc[4 * g + 2] += zb[g].z;
                    acc[4 * g + 3] += zb[g].w;
                }
                if (a.norm == 1) {
                    float sb = 0.0f;
#pragma unroll
                    for (int e = 0; e < 16; ++e) sb += acc[e];
                    const float mb = sb * (1.0f / 16);
                    float qb = 0.0f;
#pragma unroll
                    for (int e = 0; e < 16; ++e) qb += (acc[e] - mb) * (acc[e] - mb);
                    const float na = 16.0f * jb, nn = na + 16.0f, delta = mb - mean;
                    mean += delta * (16.0f / nn);
                    m2 += qb + delta * delta * (na * 16.0f / nn);
                } else if (a.norm == 2) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) m2 += acc[e] * acc[e];
                }
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *(float4 *)(st + l32 * SW + 32 * jb + 8 * g + 4 * half) =
                        make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
            }
            if (a.norm) {
                // the two halves hold D / 2 columns each of the same row
                float rstd;
                if (a.norm == 1) {
                    const float tot = halves_sum(mean);
                    const float delta = tot - 2.0f * mean;          // other half's mean minus this one's
                    const float m2t = halves_sum(m2) + delta * delta * (0.25f * D);
                    mean = 0.5f * tot;
                    rstd = 1.0f / sqrtf(m2t * (1.0f / D) + a.eps);
                } else {
                    rstd = 1.0f / sqrtf(halves_sum(m2) * (1.0f / D) + a.eps);
                    mean = 0.0f;
                }
                if (half == 0) stat[l32] = make_float2(mean, rstd);
            }
            wave_lds_fence();
            // whole rows out: lane takes columns 8 q8 .. 8 q8 + 7 of rows r8, r8 + RPI, ...
            const int nrows = min(32, a.k_c - 32 * ob);
            // gamma and beta of the lane's columns, read here rather than held across the loop:
            // the offset is an opaque zero, so the compiler cannot hoist these reads out of it
            int zero;
            asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
            float gg[8], bb[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                gg[t] = a.norm ? gb[0][8 * q8 + t + zero] : 1.0f;
                bb[t] = a.norm ? gb[1][8 * q8 + t + zero] : 0.0f;
            }
#pragma unroll
            for (int it = 0; it < 32 / RPI; ++it) {
                const int row = it * RPI + r8;
                if (row >= nrows) continue;
                const float4 u = *(const float4 *)(st + row * SW + 8 * q8);
                const float4 v = *(const float4 *)(st + row * SW + 8 * q8 + 4);
                float o8[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
                if (a.norm) {
                    const float2 ms = stat[row];
#pragma unroll
                    for (int t = 0; t < 8; ++t) o8[t] = __builtin_fmaf((o8[t] - ms.x) * ms.y, gg[t], bb[t]);
                }
                const int64_t yo = ybase + (int64_t)(32 * ob + row) * D + 8 * q8;
                if (a.out_f32) {
                    float4 *yp = (float4 *)((float *)a.y_c + yo);
                    yp[0] = make_float4(o8[0], o8[1], o8[2], o8[3]);
                    yp[1] = make_float4(o8[4], o8[5], o8[6], o8[7]);
                } else {
                    store_nt16((uint16_t *)a.y_c + yo,
                               make_uint4(pack_bf16x2(o8[0], o8[1]), pack_bf16x2(o8[2], o8[3]), pack_bf16x2(o8[4], o8[5]),
                                          pack_bf16x2(o8[6], o8[7])));
                }
            }
            wave_lds_fence();
        }
    }
}

}  // namespace

bool lcbe_mfma_supported(const LcbeArgs &a) {
    return !a.in_f32 && (a.d == 32 || a.d == 64 || a.d == 128) && a.n_c >= 1 && a.n_c <= 64 && a.k_c >= 1 &&
           a.k_c <= 64;
}

hipError_t launch_lcbe(const LcbeArgs &a0, hipStream_t s) {
    LcbeArgs a = a0;
    const int64_t per = (a.y_r ? a.k_r : 0) + (a.z ? a.k_c : 0);
    const int64_t rrows = a.R * per;
    if (rrows > 0) {
        int64_t grid = (rrows + kLeWaves - 1) / kLeWaves;
        if (grid > 65536) grid = 65536;
        if (a.in_f32) hipLaunchKernelGGL(lcbe_request_kernel<true>, dim3((unsigned)grid), dim3(kLeWaves * 64), 0, s, a);
        else hipLaunchKernelGGL(lcbe_request_kernel<false>, dim3((unsigned)grid), dim3(kLeWaves * 64), 0, s, a);
    }
    if (a.C > 0 && a.k_c > 0) {
        if (lcbe_mfma_supported(a)) {
            // contiguous runs per wave: enough waves to fill 256 CUs x 32 waves, runs of >= 8
            int64_t waves = (a.C + 7) / 8;
            if (waves > 256 * 32) waves = 256 * 32;
            a.chunk = (a.C + waves - 1) / waves;
            waves = (a.C + a.chunk - 1) / a.chunk;
            const int64_t grid = (waves + kLeWaves - 1) / kLeWaves;
            if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
            const int kst = a.n_c <= 32 ? 2 : 4, ob = a.k_c <= 32 ? 1 : 2;
#define IKBO_LE(JB, KST, OB, WPE) \
    hipLaunchKernelGGL((lcbe_cand_kernel<JB, KST, OB, WPE>), dim3((unsigned)grid), dim3(kLeWaves * 64), 0, s, a)
#define IKBO_LE_D(JB, W1, W2, W3, W4)              \
    do {                                            \
        if (kst == 2 && ob == 1) IKBO_LE(JB, 2, 1, W1); \
        else if (kst == 2) IKBO_LE(JB, 2, 2, W2);   \
        else if (ob == 1) IKBO_LE(JB, 4, 1, W3);    \
        else IKBO_LE(JB, 4, 2, W4);                 \
    } while (0)
            if (a.d == 32) IKBO_LE_D(1, 4, 2, 3, 2);
            else if (a.d == 64) IKBO_LE_D(2, 3, 3, 2, 2);
            else IKBO_LE_D(4, 2, 2, 1, 1);
#undef IKBO_LE_D
#undef IKBO_LE
        } else {
            int64_t grid = (a.C * a.k_c + kLeWaves - 1) / kLeWaves;
            if (grid > 65536) grid = 65536;
            if (a.in_f32)
                hipLaunchKernelGGL(lcbe_cand_generic_kernel<true>, dim3((unsigned)grid), dim3(kLeWaves * 64), 0, s, a);
            else
                hipLaunchKernelGGL(lcbe_cand_generic_kernel<false>, dim3((unsigned)grid), dim3(kLeWaves * 64), 0, s, a);
        }
    }
    return hipGetLastError();
}

}  // namespace ikbo
