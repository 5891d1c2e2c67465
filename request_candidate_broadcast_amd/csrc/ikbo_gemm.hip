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
// Tile 256 x 256 x 64, 8 waves (2 along N x 4 along M, each 128 x 64), LDS double-buffered with
// register-staged prefetch of the next k-tile. Tiles are numbered with the N tile fastest and each
// XCD takes a contiguous range, so the N tiles that share one block of activation rows run
// together on one XCD and read those rows through its L2.
//
// The request GEMM ([Y_r | Z] = x_r [W_RR; W_CR]^T, a small M = num_req) runs split-K into fp32
// partial sums, reduced in a fixed order by a second kernel that also applies the request-group
// epilogue; results are deterministic.
#include "ikbo_device.h"
#include "ikbo_launch.h"

namespace ikbo {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kGemmWaves = 8;
constexpr int kGemmThreads = kGemmWaves * 64;
constexpr int WM = 64, WN = 128;                 // per-wave tile (M x N)
constexpr int MB = WM / 32, NB = WN / 32;        // 32x32 accumulator blocks per wave
constexpr int kChunksPerRow = BK / 8;            // 16-byte chunks per tile row
constexpr int kTileChunks = BM * kChunksPerRow;  // 2048 per operand tile
constexpr int kLoadPasses = kTileChunks / kGemmThreads;

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ float apply_act(int act, float x) { return act == 1 ? gelu_exact(x) : x; }

// Epilogue for 4 consecutive columns col..col+3 of one row.
__device__ __forceinline__ void epilogue4(const GemmArgs &a, int64_t row, int64_t zrow, bool row_ok, int64_t col,
                                          float v0, float v1, float v2, float v3) {
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
                const float4 zz = *(const float4 *)zp;
                v[0] += zz.x; v[1] += zz.y; v[2] += zz.z; v[3] += zz.w;
            } else {
                for (int e = 0; e < 4; ++e)
                    if (col + e < a.N) v[e] += zp[e];
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
template <bool PARTIAL>
__global__ __launch_bounds__(kGemmThreads) void gemm_bf16_kernel(GemmArgs a, int32_t tiles_m, int32_t tiles_n,
                                                                 int32_t k_per_split) {
    __shared__ uint4 sx[2][kTileChunks];
    __shared__ uint4 sw[2][kTileChunks];

    const int64_t total = (int64_t)tiles_m * tiles_n * a.splits;
    int64_t t = xcd_tile(blockIdx.x, total);
    if (t < 0) return;
    const int nt = (int)(t % tiles_n);
    t /= tiles_n;
    const int mt = (int)(t % tiles_m);
    const int sp = (int)(t / tiles_m);
    const int64_t m0 = (int64_t)mt * BM;
    const int n0 = nt * BN;
    const int kbeg = sp * k_per_split;
    const int kend = min(a.K, kbeg + k_per_split);
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, half = lane >> 5;
    const int wn = wave >> 2, wm = wave & 3;

    // per-thread global source rows for the tile loads
    const uint16_t *xrow[kLoadPasses];
    const uint16_t *wrow[kLoadPasses];
#pragma unroll
    for (int p = 0; p < kLoadPasses; ++p) {
        const int q = tid + p * kGemmThreads, row = q >> 3, ch = q & 7;
        const int64_t gm = m0 + row;
        xrow[p] = gm < a.M ? (const uint16_t *)a.x + gm * a.ldx + ch * 8 : nullptr;
        const int gn = n0 + row;
        const uint16_t *wp = nullptr;
        if (gn < a.N) wp = gn < a.n0 ? (const uint16_t *)a.w0 + (int64_t)gn * a.K : (const uint16_t *)a.w1 + (int64_t)(gn - a.n0) * a.K;
        wrow[p] = wp ? wp + ch * 8 : nullptr;
    }
    uint4 px[kLoadPasses], pw[kLoadPasses];
    auto gload = [&](int k0) {
#pragma unroll
        for (int p = 0; p < kLoadPasses; ++p) {
            const int q = tid + p * kGemmThreads, ch = q & 7;
            const bool kin = k0 + ch * 8 < kend;
            px[p] = (xrow[p] && kin) ? *(const uint4 *)(xrow[p] + k0) : make_uint4(0, 0, 0, 0);
            pw[p] = (wrow[p] && kin) ? *(const uint4 *)(wrow[p] + k0) : make_uint4(0, 0, 0, 0);
        }
    };
    auto lstore = [&](int st) {
#pragma unroll
        for (int p = 0; p < kLoadPasses; ++p) {
            const int q = tid + p * kGemmThreads, row = q >> 3, ch = q & 7;
            sx[st][row * 8 + (ch ^ swz(row))] = px[p];
            sw[st][row * 8 + (ch ^ swz(row))] = pw[p];
        }
    };

    f32x16 acc[NB][MB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (nk > 0) {
        gload(kbeg);
        lstore(0);
    }
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
        const int st = it & 1;
        if (it + 1 < nk) gload(kbeg + (it + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int ch = ks * 2 + half;
            bf16x8 af[NB], bfr[MB];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int row = wn * WN + i * 32 + l32;
                af[i] = __builtin_bit_cast(bf16x8, sw[st][row * 8 + (ch ^ swz(row))]);
            }
#pragma unroll
            for (int j = 0; j < MB; ++j) {
                const int row = wm * WM + j * 32 + l32;
                bfr[j] = __builtin_bit_cast(bf16x8, sx[st][row * 8 + (ch ^ swz(row))]);
            }
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int j = 0; j < MB; ++j) acc[i][j] = mfma_32x32x16_bf16(af[i], bfr[j], acc[i][j]);
        }
        if (it + 1 < nk) lstore(st ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----
#pragma unroll
    for (int j = 0; j < MB; ++j) {
        const int64_t row = m0 + wm * WM + j * 32 + l32;
        if (row >= a.M) continue;
        if (PARTIAL) {
            float *pp = a.partial + ((int64_t)sp * a.M + row) * a.N;
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int64_t col = n0 + wn * WN + i * 32 + 8 * jj + 4 * half;
                    for (int e = 0; e < 4; ++e)
                        if (col + e < a.N) pp[col + e] = acc[i][j][4 * jj + e];
                }
        } else {
            int64_t zrow;
            const bool ok = row_request(a, row, zrow);
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int64_t col = n0 + wn * WN + i * 32 + 8 * jj + 4 * half;
                    if (col < a.N)
                        epilogue4(a, row, zrow, ok, col, acc[i][j][4 * jj], acc[i][j][4 * jj + 1], acc[i][j][4 * jj + 2],
                                  acc[i][j][4 * jj + 3]);
                }
        }
    }
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

__global__ void splitk_reduce_kernel(const float *partial, int32_t splits, int64_t M, int32_t N, int32_t n_split,
                                     const float *bias0, int32_t act, void *out0, int32_t out0_f32, float *out1) {
    const int64_t total = M * N;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / N;
        const int32_t col = (int32_t)(i - row * N);
        float s = 0.0f;
        for (int sp = 0; sp < splits; ++sp) s += partial[(int64_t)sp * total + i];
        if (col < n_split) {
            float v = s + (bias0 ? bias0[col] : 0.0f);
            v = apply_act(act, v);
            if (out0_f32) ((float *)out0)[row * n_split + col] = v;
            else ((uint16_t *)out0)[row * n_split + col] = f32_to_bf16(v);
        } else {
            out1[row * (N - n_split) + (col - n_split)] = s;
        }
    }
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
        if (a.partial) hipLaunchKernelGGL(gemm_bf16_kernel<true>, dim3((unsigned)grid), dim3(kGemmThreads), 0, s, b, (int32_t)tm, (int32_t)tn, kps);
        else hipLaunchKernelGGL(gemm_bf16_kernel<false>, dim3((unsigned)grid), dim3(kGemmThreads), 0, s, b, (int32_t)tm, (int32_t)tn, kps);
    }
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float *partial, int32_t splits, int64_t M, int32_t N, int32_t n_split,
                                const float *bias0, int32_t act, void *out0, int32_t out0_f32, float *out1,
                                hipStream_t s) {
    const int64_t total = M * N;
    if (total <= 0) return hipSuccess;
    int64_t g = (total + 255) / 256;
    if (g > 65536) g = 65536;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)g), dim3(256), 0, s, partial, splits, M, N, n_split, bias0,
                       act, out0, out0_f32, out1);
    return hipGetLastError();
}

}  // namespace ikbo
