// gla_common.hpp -- element types, conversions and MFMA wrappers for gfx950.
//
// Device code here targets CDNA4 (gfx950) only: 64-lane wavefronts and the
// v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x4_f32 matrix instructions.
//
// MFMA 16x16 lane layout used throughout (wave of 64 lanes, n = lane % 16,
// g = lane / 16):
//   accumulator  D[4g + r][n]  in register r (r = 0..3)
//   A operand    A[n][k] for the lane's k-set,  B operand  B[k][n] for the same
//                k-set.  Only the pairing of A's and B's k-sets matters, so any
//                k permutation used identically on both sides is valid.
//   bf16 16x16x32: 8 k values per lane; fp32 16x16x4: 1 k value per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return static_cast<bf16>(x); }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename E> __device__ __forceinline__ E from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return to_bf16(x); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// sigmoid on the hardware exp2 and reciprocal (about 1 ulp each)
__device__ __forceinline__ float fast_sigmoid(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

// A wave-uniform fp32 value moved to a scalar register (bit pattern preserved;
// the readfirstlane builtin itself operates on 32-bit integers).
__device__ __forceinline__ float uniform_f32(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// lambda^n for integer n >= 0 with lambda^0 = 1 (also for lambda = 0): binary
// powering in double (at most ~17 squarings for the sizes used here, relative
// error ~1e-15), rounded once to fp32.  No ratio of powers is ever formed and
// no transcendental function is evaluated.
__device__ __forceinline__ float pow_int(float lam, int n) {
    double result = 1.0, base = static_cast<double>(lam);
    for (unsigned e = static_cast<unsigned>(n); e != 0u; e >>= 1) {
        if (e & 1u) result *= base;
        base *= base;
    }
    return static_cast<float>(result);
}

}  // namespace gla
