// Device-side helpers shared by the IKBO kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// GELU, exact form x * Phi(x) = x/2 (1 + erf(x / sqrt 2)).
__device__ __forceinline__ float gelu_exact(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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
