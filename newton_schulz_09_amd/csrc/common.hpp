// Shared device/host definitions for the Muon HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

typedef uint16_t bf16_t;  // bfloat16 bit pattern as stored in HBM and LDS

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxGroup = 128;      // matrices per pass (kernel-argument pointer tables)
constexpr int kMaxNormBlocks = 256; // partial sums per matrix in the norm reduction
constexpr int kThreads = 256;       // threads per workgroup for every kernel

// Host pointer tables passed by value as kernel arguments.
struct ConstPtrTable {
    const float* p[kMaxGroup];
};
struct PtrTable {
    float* p[kMaxGroup];
};

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// float32 -> bfloat16, round to nearest, ties to even: gfx950's
// v_cvt_pk_bf16_f32 (NaN comes out quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Two float32 -> two bfloat16 (same rounding) packed as lo | hi << 16, one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// float64 -> bfloat16 with a single rounding (nearest, ties to even) for the
// normal bf16 range: round the float64 significand at bf16's 8-bit width in
// the integer domain, then the result converts to float32 exactly.  Values
// below the smallest normal bf16 (2^-126) go through float32 first.
__device__ __forceinline__ bf16_t f64_to_bf16(double d) {
    double ad = fabs(d);
    if (!(ad >= 0x1p-126) || ad > 0x1.fep127) {  // tiny, zero, huge, inf or NaN
        return f32_to_bf16(static_cast<float>(d));
    }
    uint64_t u = static_cast<uint64_t>(__double_as_longlong(d));
    const uint64_t lsb = (u >> 45) & 1ull;  // 52 - 7 fraction bits dropped
    u += 0x00000fffffffffffull + lsb;
    u &= ~0x00001fffffffffffull;
    float f = static_cast<float>(__longlong_as_double(static_cast<long long>(u)));
    return static_cast<bf16_t>(__float_as_uint(f) >> 16);
}

// The float32 quotient q (within ~2 ulps of the exact one) cannot be rounded
// to bf16 directly: it lies within 8 ulps of a bf16 rounding midpoint, or is
// not a normal float32 (zero excepted).
__device__ __forceinline__ bool cast_needs_f64(float q) {
    const uint32_t bits = __float_as_uint(q);
    const uint32_t mag = bits & 0x7fffffffu;
    const bool near_mid = ((bits & 0xffffu) - 0x7ff8u) <= 16u;
    return near_mid || (mag != 0u && mag < 0x01000000u) || mag >= 0x7f800000u;
}

}  // namespace muon
