// Device-side helpers shared by the IKBO kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace ikbo {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWave = 64;
constexpr int kNumXcd = 8;   // MI355X: 8 accelerator dies; workgroups go round-robin over them

// bf16 <-> fp32. The conversion down is round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

// 16-byte store with the non-temporal hint, for streamed outputs written in whole 128-byte lines
// (8 lanes per line): the lines go out without displacing operand tiles that other workgroups
// still read from L2. Stores that cover only part of a line are slower with the hint (the L2 no
// longer merges them), so they keep plain stores.
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt16(void *p, uint4 v) {
    const nt_u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (nt_u32x4 *)p);
}

// Two values at once: one v_cvt_pk_bf16_f32 (the same rounding as f32_to_bf16 on each).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x2_t cvt_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_convertvector(v, bf16x2_t);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, cvt_bf16x2(lo, hi));
}

// GELU, exact form x Phi(x) = x/2 (1 + erf(x / sqrt 2)), with erf from the rational approximation of
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26: for u >= 0,
// erf(u) = 1 - t P(t) exp(-u^2), t = 1 / (1 + p u), P(t) = a1 + a2 t + a3 t^2 + a4 t^3 + a5 t^4, with
// |error| <= 1.5e-7. With u = |x| / sqrt 2 both signs of x give
//   GELU(x) = max(x, 0) - |x| t (P(t) / 2) exp(-x^2 / 2),
// which needs no 1 + erf (that sum loses the small tail for negative x) and no branch: one
// reciprocal, one exp2 and a dozen FMA-class operations, where the library erff spends several
// times that on range reduction and branches (GELU is the larger part of the GEMM epilogues).
// |x| is capped at the largest float in the product so that GELU(+-inf) = +inf / 0; a NaN input
// reaches the result through t. The cap and max(x, 0) are integer min / max on the bit patterns
// (for floats >= 0 the integer order is the float order; a signed max with 0 maps every negative
// float to +0), which needs none of the NaN-quieting the float min / max carry.
__device__ __forceinline__ float gelu_exact(float x) {
    const float ax = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.23164188769779495f, ax, 1.0f));   // p / sqrt 2
    float q = __builtin_fmaf(0.5307027145f, t, -0.7265760135f);                               // a5 / 2, a4 / 2
    q = __builtin_fmaf(q, t, 0.7107068705f);                                                  // a3 / 2
    q = __builtin_fmaf(q, t, -0.142248368f);                                                  // a2 / 2
    q = __builtin_fmaf(q, t, 0.127414796f);                                                   // a1 / 2
    const float axm = __uint_as_float(min(__float_as_uint(ax), 0x7f7fffffu));
    const float h = (axm * t) * q;
    const float e = __builtin_amdgcn_exp2f((x * x) * -0.72134752044448170f);                  // exp(-x^2 / 2)
    const float relu = __int_as_float(max(__float_as_int(x), 0));
    return __builtin_fmaf(-h, e, relu);
}

__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Compile-time loop: f(IC<0>), f(IC<1>), ..., f(IC<N-1>).
template <int I>
using IC = std::integral_constant<int, I>;
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(IC<I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Thin wrappers of target builtins, so generic lambdas inside kernels only call device functions.
// No instruction is moved across a scheduling fence.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// s_waitcnt vmcnt(N) leaving expcnt (7) and lgkmcnt (15) free; vmcnt is split over bits 3:0
// and 15:14
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }
// Workgroup barrier without the memory fences of __syncthreads(). Those fences make the compiler
// wait for every load in flight (vmcnt 0), direct global -> LDS copies included, which defeats
// copies meant to stay in flight across the barrier. Callers wait for the copies they need
// (wait_vmcnt) before calling this; it waits for the wave's own LDS accesses (lgkmcnt 0), and the
// asm memory clobber keeps the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("s_barrier" ::: "memory");
}
// Direct global -> LDS copy of 16 bytes per lane: the wave's 64 lanes fill 64 consecutive 16-byte
// LDS slots starting at lds_wave_base (taken from the first lane), lane i slot i.
__device__ __forceinline__ void copy16_to_lds(const void *src, void *lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds_wave_base, 16, 0, 0);
}

// A 64-bit value every lane holds alike, in scalar registers (branches on it are uniform)
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Request of candidate c for kernels that walk candidates in increasing order: from the offsets
// [R + 1] when given (one binary search when cursor < 0, then a linear advance from the previous
// candidate's request), else from the map; -1 when the candidate has no valid request.
__device__ __forceinline__ int64_t cand_request(const int32_t *off, const int32_t *map, int64_t R, int64_t c,
                                                int64_t &cursor) {
    if (off) {
        if (cursor < 0) {
            int64_t lo = 0, hi = R;          // last r with off[r] <= c
            while (hi - lo > 1) {
                const int64_t mid = (lo + hi) / 2;
                if (off[mid] <= c) lo = mid;
                else hi = mid;
            }
            cursor = lo;
        }
        while (cursor < R && off[cursor + 1] <= c) ++cursor;
        if (cursor >= R || off[cursor] > c) return -1;
        return cursor;
    }
    const int32_t r = map[c];
    return (r >= 0 && r < R) ? r : -1;
}

// A pointer that is the same in every lane, moved to scalar registers.
template <typename T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
    const uint64_t u = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (T *)(((uint64_t)hi << 32) | lo);
}

// Raw buffer resource over [base, base + bytes): loads at offsets past the end return zero. The
// last word is the gfx9-family default (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
// Buffer -> LDS copy of 16 bytes per lane from byte offset voff (out-of-range lanes write zeros);
// LDS slots as in copy16_to_lds.
__device__ __forceinline__ void buffer_copy16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, void *lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_wave_base, 16, voff, 0, 0, 0);
}

// Map a hardware workgroup id to a logical tile so that each XCD works through one contiguous
// range of logical tiles (consecutive tiles share request K/V or GEMM operands, and share an L2
// only when they run on the same XCD). Returns -1 for ids past the end.
__device__ __forceinline__ int64_t xcd_tile(int64_t bid, int64_t num_tiles) {
    const int64_t per_xcd = (num_tiles + kNumXcd - 1) / kNumXcd;
    const int64_t xcd = bid % kNumXcd, slot = bid / kNumXcd;
    if (slot >= per_xcd) return -1;
    const int64_t t = xcd * per_xcd + slot;
    return t < num_tiles ? t : -1;
}

}  // namespace ikbo
