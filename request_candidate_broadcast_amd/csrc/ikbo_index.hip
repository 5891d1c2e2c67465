// Index prologue of the IKBO kernels: the candidate -> request map m and the per-request
// candidate offsets (ROCS Sec. 4.1: m in {0..B_r-1}^{B_c}; Sec. 4.2.1: the candidates of a request
// are usually stored contiguously). Converts between the two forms, groups an ungrouped map with
// a counting sort (integer atomics only, so the resulting grouping is exact), builds the DCA
// tile table, and checks index contents.
#include "ikbo_device.h"
#include "ikbo_launch.h"

namespace ikbo {

namespace {

__device__ __forceinline__ int64_t clampi(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }

__global__ void fill_i32_kernel(int32_t *p, int64_t n, int32_t v) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

__global__ void iota_i32_kernel(int32_t *p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = (int32_t)i;
}

__global__ void histogram_kernel(const int32_t *m, int64_t C, int64_t R, int32_t *counts) {
    for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < C; c += (int64_t)gridDim.x * blockDim.x) {
        const int32_t r = m[c];
        if (r >= 0 && r < R) atomicAdd(&counts[r], 1);
    }
}

// One workgroup of 1024 threads scans R entries in chunks, carrying the running totals.
__global__ __launch_bounds__(1024) void scan_tiles_kernel(const int32_t *counts, const int32_t *off_in, int64_t R,
                                                          int64_t C, int32_t q_len, int32_t heads, int32_t block_m,
                                                          int32_t *off_out, int32_t *cursor, int32_t *tile_start) {
    __shared__ int64_t s_cnt[1024];
    __shared__ int64_t s_til[1024];
    __shared__ int64_t carry_c, carry_t;
    const int tid = threadIdx.x;
    if (tid == 0) { carry_c = 0; carry_t = 0; }
    __syncthreads();
    for (int64_t base = 0; base < R; base += 1024) {
        const int64_t r = base + tid;
        int64_t n = 0;
        if (r < R) {
            if (counts) {
                n = counts[r];
            } else {
                const int64_t c0 = clampi(off_in[r], 0, C);
                const int64_t c1 = clampi(off_in[r + 1], c0, C);
                n = c1 - c0;
            }
        }
        const int64_t rows = n * q_len;
        const int64_t tiles = heads * ((rows + block_m - 1) / block_m);
        s_cnt[tid] = n;
        s_til[tid] = tiles;
        __syncthreads();
        // inclusive Hillis-Steele scan
        for (int d = 1; d < 1024; d <<= 1) {
            int64_t a = tid >= d ? s_cnt[tid - d] : 0, b = tid >= d ? s_til[tid - d] : 0;
            __syncthreads();
            s_cnt[tid] += a;
            s_til[tid] += b;
            __syncthreads();
        }
        if (r < R) {
            const int64_t excl_c = carry_c + s_cnt[tid] - n;
            const int64_t excl_t = carry_t + s_til[tid] - tiles;
            if (counts) {
                off_out[r] = (int32_t)excl_c;
            } else {
                off_out[r] = (int32_t)clampi(off_in[r], 0, C);
            }
            if (cursor) cursor[r] = off_out[r];
            tile_start[r] = (int32_t)excl_t;
        }
        __syncthreads();
        if (tid == 1023) {
            carry_c += s_cnt[1023];
            carry_t += s_til[1023];
        }
        __syncthreads();
    }
    if (tid == 0) {
        if (counts) off_out[R] = (int32_t)carry_c;
        else off_out[R] = (int32_t)clampi(off_in[R], 0, C);
        tile_start[R] = (int32_t)carry_t;
    }
}

__global__ void scatter_kernel(const int32_t *m, int64_t C, int64_t R, int32_t *cursor, int32_t *perm, void *out,
                               int64_t row_elems, int64_t row_stride, int out_bytes) {
    for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < C; c += (int64_t)gridDim.x * blockDim.x) {
        const int32_t r = m[c];
        if (r >= 0 && r < R) {
            const int32_t pos = atomicAdd(&cursor[r], 1);
            perm[pos] = (int32_t)c;
        } else if (out) {
            char *row = (char *)out + c * row_stride * out_bytes;
            for (int64_t i = 0; i < row_elems * out_bytes; i += 4) *(uint32_t *)(row + i) = 0u;
        }
    }
}

__global__ void offsets_to_map_kernel(const int32_t *off, int64_t R, int64_t C, int32_t *m_out) {
    for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < C; c += (int64_t)gridDim.x * blockDim.x) {
        // largest r with clamp(off[r]) <= c, on the running-max sanitised offsets
        int64_t lo = 0, hi = R;   // search in [0, R)
        int32_t found = -1;
        if (R > 0 && clampi(off[0], 0, C) <= c) {
            while (hi - lo > 1) {
                const int64_t mid = (lo + hi) >> 1;
                if (clampi(off[mid], 0, C) <= c) lo = mid; else hi = mid;
            }
            if (c < clampi(off[lo + 1], 0, C)) found = (int32_t)lo;
        }
        m_out[c] = found;
    }
}

__global__ void zero_uncovered_kernel(const int32_t *off, int64_t R, int64_t C, void *out, int64_t row_elems,
                                      int64_t row_stride, int out_bytes) {
    const int64_t c0 = R > 0 ? clampi(off[0], 0, C) : C;
    const int64_t c1 = R > 0 ? clampi(off[R], c0, C) : C;
    const int64_t words = row_elems * out_bytes / 4;
    for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < C; c += (int64_t)gridDim.x * blockDim.x) {
        if (c >= c0 && c < c1) continue;
        uint32_t *row = (uint32_t *)((char *)out + c * row_stride * out_bytes);
        for (int64_t i = 0; i < words; ++i) row[i] = 0u;
    }
}

__global__ void check_index_kernel(const int32_t *m, const int32_t *off, int64_t C, int64_t R, uint32_t flags,
                                   unsigned long long *count) {
    unsigned long long bad = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (off) {
        if (g == 0) {
            if (off[0] != 0) ++bad;
            if (off[R] != C) ++bad;
        }
        for (int64_t r = g; r < R; r += stride)
            if (off[r + 1] < off[r]) ++bad;
    }
    if (m) {
        for (int64_t c = g; c < C; c += stride) {
            const int32_t r = m[c];
            if (r < 0 || r >= R) { ++bad; continue; }
            if ((flags & 1u) && c > 0 && r < m[c - 1]) ++bad;
            if (off && !(off[r] <= c && c < off[r + 1])) ++bad;
        }
    }
    if (bad) atomicAdd(count, bad);
}

unsigned grid_for(int64_t n, int threads) {
    int64_t g = (n + threads - 1) / threads;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return (unsigned)g;
}

}  // namespace

hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t value, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, p, n, value);
    return hipGetLastError();
}

hipError_t launch_iota_i32(int32_t *p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(iota_i32_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_histogram(const int32_t *m, int64_t C, int64_t R, int32_t *counts, hipStream_t s) {
    if (C <= 0) return hipSuccess;
    hipLaunchKernelGGL(histogram_kernel, dim3(grid_for(C, 256)), dim3(256), 0, s, m, C, R, counts);
    return hipGetLastError();
}

hipError_t launch_scan_tiles(const int32_t *counts, const int32_t *off_in, int64_t R, int64_t C, int32_t q_len,
                             int32_t heads, int32_t block_m, int32_t *off_out, int32_t *cursor, int32_t *tile_start,
                             hipStream_t s) {
    hipLaunchKernelGGL(scan_tiles_kernel, dim3(1), dim3(1024), 0, s, counts, off_in, R, C, q_len, heads, block_m,
                       off_out, cursor, tile_start);
    return hipGetLastError();
}

hipError_t launch_scatter(const int32_t *m, int64_t C, int64_t R, int32_t *cursor, int32_t *perm, void *out,
                          int64_t row_elems, int64_t row_stride, int out_bytes, hipStream_t s) {
    if (C <= 0) return hipSuccess;
    hipLaunchKernelGGL(scatter_kernel, dim3(grid_for(C, 256)), dim3(256), 0, s, m, C, R, cursor, perm, out,
                       row_elems, row_stride, out_bytes);
    return hipGetLastError();
}

hipError_t launch_offsets_to_map(const int32_t *off, int64_t R, int64_t C, int32_t *m_out, hipStream_t s) {
    if (C <= 0) return hipSuccess;
    hipLaunchKernelGGL(offsets_to_map_kernel, dim3(grid_for(C, 256)), dim3(256), 0, s, off, R, C, m_out);
    return hipGetLastError();
}

hipError_t launch_zero_uncovered(const int32_t *off, int64_t R, int64_t C, void *out, int64_t row_elems,
                                 int64_t row_stride, int out_bytes, hipStream_t s) {
    if (C <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_uncovered_kernel, dim3(grid_for(C, 256)), dim3(256), 0, s,
                       off, R, C, out, row_elems, row_stride, out_bytes);
    return hipGetLastError();
}

hipError_t launch_check_index(const int32_t *m, const int32_t *off, int64_t C, int64_t R, uint32_t flags,
                              uint64_t *d_count, hipStream_t s) {
    hipError_t e = launch_fill_i32((int32_t *)d_count, 2, 0, s);   // a kernel, safe under graph capture
    if (e != hipSuccess) return e;
    const int64_t n = C > R ? C : R;
    hipLaunchKernelGGL(check_index_kernel, dim3(grid_for(n > 0 ? n : 1, 256)), dim3(256), 0, s, m, off, C, R, flags,
                       (unsigned long long *)d_count);
    return hipGetLastError();
}

}  // namespace ikbo
