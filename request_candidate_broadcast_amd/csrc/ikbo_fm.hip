// GLM factorization machine with the request-candidate broadcast resolved in the kernel (ROCS
// Sec. 3.1.4, Eq. 9-10, two groups):
//   y_c[c] = [ X^C_c (X^R_{m(c)})^T ,  X^C_c (X^C_c)^T ]   [n_c, n_r + n_c]
//   y_r[r] =   X^R_r (X^R_r)^T                              [n_r, n_r]
// The request embeddings stay at the request batch size and are read through m.
//
// bf16 path (d in {32, 64, 128}, n_r and n_c up to 64): one wave per item (candidate or request),
// each wave taking a contiguous run of items, so with grouped candidates a request's fragments are
// loaded once per run. Products on v_mfma_f32_32x32x16_bf16, 32 embedding rows per block, computed
// transposed (D^T = B A^T) so each lane owns one output row and four consecutive columns per store.
// A lane (l32, half) reads one contiguous half-row of its embedding row (d bytes) and splits it into
// d/16 chunks of 8, chunk e feeding k step e: the same permutation of the contraction index on both
// operands, so the products summed are the definition's. The candidate's own fragments are both
// operands of the X^C (X^C)^T block. The workload is HBM-bound (d/2 FLOP per byte at bf16 in, bf16
// out), so the design is about streaming: small register footprint, many waves per CU. Results go
// through a per-wave LDS stage: the 32 x W row block of an output is written there from the
// accumulators, then stored as whole rows, consecutive lanes on consecutive 16-byte chunks, so the
// L2 receives full-line writes (stored straight from the accumulator layout, each instruction
// would write 16 bytes into each of 32 rows: four times the write requests).
#include "ikbo_device.h"
#include "ikbo_launch.h"

namespace ikbo {
namespace {

constexpr int kFmWaves = 4;            // waves per workgroup
constexpr int kFmRowsMax = 64;         // n_r, n_c <= 64 (two 32-row blocks) on the MFMA path

// Rows [0, nrows) of a [nrows, 16 * KS] bf16 matrix as MFMA fragments (rows >= nrows read as zero).
template <int KS>
__device__ __forceinline__ void fm_rows(const uint16_t *x, int nrows, int l32, int half, bf16x8 (&f)[KS]) {
    constexpr int D = 16 * KS;
    if (l32 < nrows) {
        const uint4 *p = (const uint4 *)(x + (int64_t)l32 * D + half * (D / 2));
#pragma unroll
        for (int e = 0; e < KS; ++e) f[e] = __builtin_bit_cast(bf16x8, p[e]);
    } else {
#pragma unroll
        for (int e = 0; e < KS; ++e) f[e] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    }
}

// One 32 x 32 accumulator block into the wave's LDS stage (fp32, row stride SW floats): lane
// (l32, half) holds row l32, columns col0 + 8 jj + 4 half + {0..3}; columns past ncols (a multiple
// of 4) are skipped.
__device__ __forceinline__ void fm_stage(float *st, int SW, int l32, int half, int col0, int ncols, const f32x16 &acc) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int col = 8 * jj + 4 * half;
        if (col < ncols)
            *(float4 *)(st + l32 * SW + col0 + col) = make_float4(acc[4 * jj], acc[4 * jj + 1], acc[4 * jj + 2], acc[4 * jj + 3]);
    }
}

// Rows [0, nrows) (at most 32) of the stage, W columns each (a multiple of 4), to the output at
// element offset base with row stride W: consecutive lanes take consecutive chunks (16 bytes, or 8
// for bf16 rows whose length is not a multiple of 8, which keeps every store naturally aligned).
// The stage is written by other lanes of the same wave: wavefront-scope fences on both sides keep
// the compiler from moving these reads above those writes or the next block's writes above them.
__device__ __forceinline__ void fm_flush(const float *st, int SW, void *y, int out_f32, int64_t base, int W, int nrows,
                                         int lane) {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (out_f32) {
        const int cpr = W / 4;
        for (int i = lane; i < nrows * cpr; i += 64) {
            const int row = i / cpr, q = i - row * cpr;
            store_nt16((float *)y + base + (int64_t)row * W + 4 * q, *(const uint4 *)(st + row * SW + 4 * q));
        }
    } else if (W % 8 == 0) {
        const int cpr = W / 8;
        for (int i = lane; i < nrows * cpr; i += 64) {
            const int row = i / cpr, q = i - row * cpr;
            const float4 u = *(const float4 *)(st + row * SW + 8 * q);
            const float4 v = *(const float4 *)(st + row * SW + 8 * q + 4);
            store_nt16((uint16_t *)y + base + (int64_t)row * W + 8 * q,
                       make_uint4(pack_bf16x2(u.x, u.y), pack_bf16x2(u.z, u.w), pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)));
        }
    } else {
        const int cpr = W / 4;
        for (int i = lane; i < nrows * cpr; i += 64) {
            const int row = i / cpr, q = i - row * cpr;
            const float4 u = *(const float4 *)(st + row * SW + 4 * q);
            *(uint2 *)((uint16_t *)y + base + (int64_t)row * W + 4 * q) =
                make_uint2(pack_bf16x2(u.x, u.y), pack_bf16x2(u.z, u.w));
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ void fm_zero(void *y, int out_f32, int64_t base, int64_t n, int lane) {
    for (int64_t i = 4 * lane; i < n; i += 256) {
        if (out_f32) *(float4 *)((float *)y + base + i) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        else *(uint2 *)((uint16_t *)y + base + i) = make_uint2(0, 0);
    }
}

__device__ __forceinline__ int64_t fm_request(const FmArgs &a, int64_t c, int64_t &cursor) {
    return cand_request(a.off, a.map, a.R, c, cursor);
}

// KS = d / 16 k steps, NB = 32-row blocks per group (1: n_r, n_c <= 32; 2: <= 64), WPE = waves per
// SIMD the register budget is sized for (fragments of both groups stay in registers).
template <int KS, int NB, int WPE>
__global__ __launch_bounds__(kFmWaves * 64) __attribute__((amdgpu_waves_per_eu(WPE, 8))) void fm_bf16_kernel(FmArgs a) {
    constexpr int D = 16 * KS;
    constexpr int kFmMaxBlocks = NB;
    constexpr int SW = 64 * NB + 4;                        // stage row stride (floats): W <= 64 NB
    __shared__ float stage_all[kFmWaves][32 * SW];
    const int lane = threadIdx.x & 63, l32 = lane & 31, half = lane >> 5;
    const int64_t wave = (int64_t)blockIdx.x * kFmWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t items = a.C + (a.y_r ? a.R : 0);
    const int64_t i0 = wave * a.chunk, i1 = min(items, i0 + a.chunk);
    const int rbr = (a.n_r + 31) / 32, rbc = (a.n_c + 31) / 32;
    const int W = a.n_r + a.n_c;
    const uint16_t *xr = (const uint16_t *)a.x_r, *xc = (const uint16_t *)a.x_c;
    float *st = stage_all[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];
    bf16x8 fr[kFmMaxBlocks][KS], fc[kFmMaxBlocks][KS];
    int64_t have_r = -1, cursor = -1;
    for (int64_t it = i0; it < i1; ++it) {
        if (it < a.C) {
            const int64_t c = it;
            const int64_t r = uniform64(fm_request(a, c, cursor));
            const int64_t base = c * a.n_c * W;
            if (r < 0) {
                fm_zero(a.y_c, a.out_f32, base, (int64_t)a.n_c * W, lane);
                continue;
            }
            if (r != have_r) {
#pragma unroll
                for (int b = 0; b < kFmMaxBlocks; ++b)
                    if (b < rbr) fm_rows<KS>(xr + (r * a.n_r + 32 * b) * D, a.n_r - 32 * b, l32, half, fr[b]);
                have_r = r;
            }
#pragma unroll
            for (int b = 0; b < kFmMaxBlocks; ++b)
                if (b < rbc) fm_rows<KS>(xc + (c * a.n_c + 32 * b) * D, a.n_c - 32 * b, l32, half, fc[b]);
#pragma unroll
            for (int rb = 0; rb < kFmMaxBlocks; ++rb) {
                if (rb >= rbc) continue;
                // request-candidate block(s): columns [0, n_r)
#pragma unroll
                for (int cb = 0; cb < kFmMaxBlocks; ++cb) {
                    if (cb >= rbr) continue;
                    f32x16 acc;
#pragma unroll
                    for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
#pragma unroll
                    for (int e = 0; e < KS; ++e) acc = mfma_32x32x16_bf16(fr[cb][e], fc[rb][e], acc);
                    fm_stage(st, SW, l32, half, 32 * cb, a.n_r - 32 * cb, acc);
                }
                // candidate-candidate block(s): columns [n_r, n_r + n_c)
#pragma unroll
                for (int cb = 0; cb < kFmMaxBlocks; ++cb) {
                    if (cb >= rbc) continue;
                    f32x16 acc;
#pragma unroll
                    for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
#pragma unroll
                    for (int e = 0; e < KS; ++e) acc = mfma_32x32x16_bf16(fc[cb][e], fc[rb][e], acc);
                    fm_stage(st, SW, l32, half, a.n_r + 32 * cb, a.n_c - 32 * cb, acc);
                }
                fm_flush(st, SW, a.y_c, a.out_f32, base + (int64_t)32 * rb * W, W, min(32, a.n_c - 32 * rb), lane);
            }
        } else {
            // request group: y_r[r] = X^R_r (X^R_r)^T
            const int64_t r = it - a.C;
            const int64_t base = r * a.n_r * a.n_r;
#pragma unroll
            for (int b = 0; b < kFmMaxBlocks; ++b)
                if (b < rbr) fm_rows<KS>(xr + (r * a.n_r + 32 * b) * D, a.n_r - 32 * b, l32, half, fr[b]);
            have_r = -1;
#pragma unroll
            for (int rb = 0; rb < kFmMaxBlocks; ++rb) {
                if (rb >= rbr) continue;
#pragma unroll
                for (int cb = 0; cb < kFmMaxBlocks; ++cb) {
                    if (cb >= rbr) continue;
                    f32x16 acc;
#pragma unroll
                    for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
#pragma unroll
                    for (int e = 0; e < KS; ++e) acc = mfma_32x32x16_bf16(fr[cb][e], fr[rb][e], acc);
                    fm_stage(st, SW, l32, half, 32 * cb, a.n_r - 32 * cb, acc);
                }
                fm_flush(st, SW, a.y_r, a.out_f32, base + (int64_t)32 * rb * a.n_r, a.n_r, min(32, a.n_r - 32 * rb), lane);
            }
        }
    }
}

// Any d (fp32 inputs, or bf16 with a width the MFMA path is not built for): one thread per output
// element, fp32 products summed in index order.
__device__ __forceinline__ float fm_in(const void *p, int in_f32, int64_t i) {
    if (in_f32) return ((const float *)p)[i];
    return __uint_as_float((uint32_t)((const uint16_t *)p)[i] << 16);
}

__global__ void fm_generic_kernel(FmArgs a) {
    const int W = a.n_r + a.n_c;
    const int64_t nc_out = a.C * a.n_c * W, nr_out = a.y_r ? a.R * a.n_r * a.n_r : 0;
    for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < nc_out + nr_out;
         g += (int64_t)gridDim.x * blockDim.x) {
        float s = 0.0f;
        void *y;
        int64_t o;
        if (g < nc_out) {
            const int64_t c = g / ((int64_t)a.n_c * W);
            const int64_t rem = g - c * a.n_c * W;
            const int i = (int)(rem / W), n = (int)(rem % W);
            int64_t cur = -1;
            const int64_t r = fm_request(a, c, cur);
            if (r >= 0) {
                const int64_t pa = (c * a.n_c + i) * a.d;
                const int64_t pb = n < a.n_r ? (r * a.n_r + n) * a.d : (c * a.n_c + (n - a.n_r)) * a.d;
                const void *xb = n < a.n_r ? a.x_r : a.x_c;
                for (int k = 0; k < a.d; ++k) s = __builtin_fmaf(fm_in(a.x_c, a.in_f32, pa + k), fm_in(xb, a.in_f32, pb + k), s);
            }
            y = a.y_c;
            o = g;
        } else {
            const int64_t h = g - nc_out;
            const int64_t r = h / ((int64_t)a.n_r * a.n_r);
            const int64_t rem = h - r * a.n_r * a.n_r;
            const int i = (int)(rem / a.n_r), n = (int)(rem % a.n_r);
            const int64_t pa = (r * a.n_r + i) * a.d, pb = (r * a.n_r + n) * a.d;
            for (int k = 0; k < a.d; ++k) s = __builtin_fmaf(fm_in(a.x_r, a.in_f32, pa + k), fm_in(a.x_r, a.in_f32, pb + k), s);
            y = a.y_r;
            o = h;
        }
        if (a.out_f32) ((float *)y)[o] = s;
        else ((uint16_t *)y)[o] = f32_to_bf16(s);
    }
}

}  // namespace

bool fm_mfma_supported(const FmArgs &a) {
    return !a.in_f32 && (a.d == 32 || a.d == 64 || a.d == 128) && a.n_r <= kFmRowsMax && a.n_c <= kFmRowsMax;
}

hipError_t launch_fm(const FmArgs &a0, hipStream_t s) {
    FmArgs a = a0;
    const int64_t items = a.C + (a.y_r ? a.R : 0);
    if (items <= 0) return hipSuccess;
    if (fm_mfma_supported(a)) {
        // contiguous runs of items per wave: enough waves to fill 256 CUs x 32 waves, each run at
        // least 8 items long
        int64_t waves = (items + 7) / 8;
        if (waves > 256 * 32) waves = 256 * 32;
        a.chunk = (items + waves - 1) / waves;
        waves = (items + a.chunk - 1) / a.chunk;
        const int64_t grid = (waves + kFmWaves - 1) / kFmWaves;
        if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        const bool one = a.n_r <= 32 && a.n_c <= 32;
#define IKBO_FM(KS, NB, WPE) hipLaunchKernelGGL((fm_bf16_kernel<KS, NB, WPE>), dim3((unsigned)grid), dim3(kFmWaves * 64), 0, s, a)
        if (a.d == 32) {
            if (one) IKBO_FM(2, 1, 4);
            else IKBO_FM(2, 2, 2);
        } else if (a.d == 64) {
            if (one) IKBO_FM(4, 1, 4);
            else IKBO_FM(4, 2, 2);
        } else {
            if (one) IKBO_FM(8, 1, 2);
            else IKBO_FM(8, 2, 1);
        }
#undef IKBO_FM
    } else {
        const int64_t total = a.C * a.n_c * (a.n_r + a.n_c) + (a.y_r ? a.R * a.n_r * a.n_r : 0);
        int64_t grid = (total + 255) / 256;
        if (grid > 65536) grid = 65536;
        hipLaunchKernelGGL(fm_generic_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace ikbo
