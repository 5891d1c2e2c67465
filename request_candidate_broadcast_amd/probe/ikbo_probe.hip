// Ceiling probes for the roofline: the rates a kernel of this part can reach on its own, measured
// beside the published peaks (bf16 dense MFMA, HBM, the transcendental unit the softmax uses, and
// LDS reads).
// Each probe is a bounded loop over registers or a grid-stride pass over a buffer; none depends
// on the method. The caller times the launch (events on the stream) and divides the work below.
#include "ikbo_probe.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Four independent v_mfma_f32_32x32x16_bf16 chains per wave, `iters` rounds: 4 * 32768 FLOP per
// wave per round. Operands come from the lane index so nothing folds; one float per thread is
// stored so nothing is dropped.
__global__ __launch_bounds__(256) void probe_mfma_kernel(float *out, int64_t iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1e-3f * (float)((lane + e) & 7));
        b[e] = (__bf16)(1e-3f * (float)((lane * 3 + e) & 7));
    }
    f32x16 c0, c1, c2, c3;
#pragma unroll
    for (int e = 0; e < 16; ++e) c0[e] = c1[e] = c2[e] = c3[e] = 0.0f;
    for (int64_t i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Eight independent chains y <- 2^(-y) per thread (y stays in [0.5, 1]): 8 v_exp_f32 per thread
// per round, the negation folded into the instruction.
__global__ __launch_bounds__(256) void probe_exp2_kernel(float *out, int64_t iters) {
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = 0.5f + 0.01f * (float)((threadIdx.x + k) & 31);
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = __builtin_amdgcn_exp2f(-y[k]);
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += y[k];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Chunk k (< 4) of lane l of wave w in step j: each wave owns 256 consecutive 16-byte chunks per
// step (4 KiB), each of its 4 loads a contiguous 1 KiB, and the waves of the grid cover 4 * nthr
// consecutive chunks per step.
__device__ __forceinline__ int64_t probe_chunk(int64_t j, int64_t nthr, int64_t t, int k) {
    return j * 4 * nthr + (t >> 6) * 256 + k * 64 + (t & 63);
}

// dst <- src with four 16-byte loads in flight per lane (all issued before the stores); chunks past
// the last whole step are copied one per lane.
__global__ __launch_bounds__(256) void probe_copy_kernel(const uint4 *src, uint4 *dst, int64_t n16) {
    const int64_t nthr = (int64_t)gridDim.x * blockDim.x, t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t steps = n16 / (4 * nthr);
    for (int64_t j = 0; j < steps; ++j) {
        uint4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = src[probe_chunk(j, nthr, t, k)];
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[probe_chunk(j, nthr, t, k)] = v[k];
    }
    for (int64_t i = steps * 4 * nthr + t; i < n16; i += nthr) dst[i] = src[i];
}

// Reads src once, four 16-byte loads in flight per lane, one word per thread written.
__global__ __launch_bounds__(256) void probe_read_kernel(const uint4 *src, int64_t n16, uint32_t *out) {
    const int64_t nthr = (int64_t)gridDim.x * blockDim.x, t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t steps = n16 / (4 * nthr);
    uint32_t x = 0;
    for (int64_t j = 0; j < steps; ++j) {
        uint4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = src[probe_chunk(j, nthr, t, k)];
#pragma unroll
        for (int k = 0; k < 4; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    for (int64_t i = steps * 4 * nthr + t; i < n16; i += nthr) {
        const uint4 v = src[i];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[t] = x;
}

// LDS reads: each block fills 32 KiB of LDS with one runtime value, then every wave issues 16 reads
// per round, `iters` rounds, at addresses that move with the round (so no read leaves the loop).
// TR = false: ds_read_b128, lane l at 16 l of a 1 KiB block (1 KiB per wave instruction).
// TR = true: ds_read_b64_tr_b16 (512 B per wave instruction) over rows of 320 bytes (128 16-bit
// elements plus 32 of padding), each 16-lane group reading 4 rows by 64 bytes, in pairs 8 rows
// apart. Every read returns copies of the fill value, so the xor of each round's reads is 0 and
// every thread writes 0.
typedef short probe_i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) probe_i16x4 probe_lds_i16x4;

template <bool TR>
__global__ __launch_bounds__(256) void probe_lds_kernel(uint32_t *out, int64_t iters) {
    __shared__ uint4 buf[2048];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t h = (uint32_t)(iters * 2654435761LL) & 0xffffu;
    const uint32_t w = h | (h << 16);
    for (int i = tid; i < 2048; i += 256) buf[i] = make_uint4(w, w, w, w);
    __syncthreads();
    const int g16 = lane >> 4, s16 = lane & 15;
    const int tr_base = (4 * (g16 >> 1) + (s16 >> 2)) * 320 + ((g16 & 1) * 16 + 4 * (s16 & 3)) * 2;
    uint32_t acc = 0;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            if constexpr (TR) {
                const int off = (int)((it + k) & 1) * 8192 + tr_base + ((k >> 2) & 1) * 32 * 320 + (k & 3) * 64 +
                                (k >> 3) * 8 * 320;
                const probe_i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (probe_lds_i16x4 *)((__attribute__((address_space(3))) char *)buf + off));
                acc ^= (uint32_t)(uint16_t)r[0] ^ (uint32_t)(uint16_t)r[1] ^ (uint32_t)(uint16_t)r[2] ^
                       (uint32_t)(uint16_t)r[3];
            } else {
                const uint4 v = buf[(int)((it * 16 + k + wave * 5) & 31) * 64 + lane];
                acc ^= v.x ^ v.y ^ v.z ^ v.w;
            }
        }
    }
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

int ikbo_probe_launch(int32_t kind, void *buf, size_t bytes, int64_t iters, int64_t blocks, void *hip_stream) {
    hipStream_t s = (hipStream_t)hip_stream;
    if (!buf || blocks <= 0 || blocks > 0x7fffffffLL || iters < 0) return 1;
    const dim3 grid((unsigned)blocks), block(256);
    const size_t per_thread_out = (size_t)blocks * 256 * 4;
    switch (kind) {
        case IKBO_PROBE_MFMA_BF16:
            if (bytes < per_thread_out) return 1;
            hipLaunchKernelGGL(probe_mfma_kernel, grid, block, 0, s, (float *)buf, iters);
            break;
        case IKBO_PROBE_EXP2:
            if (bytes < per_thread_out) return 1;
            hipLaunchKernelGGL(probe_exp2_kernel, grid, block, 0, s, (float *)buf, iters);
            break;
        case IKBO_PROBE_COPY: {
            // the first half of buf is copied onto the second half
            const int64_t n16 = (int64_t)(bytes / 2 / 16);
            if (n16 <= 0 || ((uintptr_t)buf & 15)) return 1;
            hipLaunchKernelGGL(probe_copy_kernel, grid, block, 0, s, (const uint4 *)buf, (uint4 *)buf + n16, n16);
            break;
        }
        case IKBO_PROBE_READ: {
            // reads all of buf but the last blocks * 256 words, which receive the per-thread results
            if (bytes <= per_thread_out + 16 || ((uintptr_t)buf & 15)) return 1;
            const int64_t n16 = (int64_t)((bytes - per_thread_out) / 16);
            hipLaunchKernelGGL(probe_read_kernel, grid, block, 0, s, (const uint4 *)buf, n16,
                               (uint32_t *)((char *)buf + (size_t)n16 * 16));
            break;
        }
        case IKBO_PROBE_LDS_B128:
            if (bytes < per_thread_out) return 1;
            hipLaunchKernelGGL(probe_lds_kernel<false>, grid, block, 0, s, (uint32_t *)buf, iters);
            break;
        case IKBO_PROBE_LDS_TR16:
            if (bytes < per_thread_out) return 1;
            hipLaunchKernelGGL(probe_lds_kernel<true>, grid, block, 0, s, (uint32_t *)buf, iters);
            break;
        default:
            return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
