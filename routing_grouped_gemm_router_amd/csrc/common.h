// common.h -- internal helpers shared by the libmoe HIP sources (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

#define MOE_DEV __device__ __forceinline__

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

namespace moe {

constexpr int kWave = 64;

// bfloat16 <-> fp32 on raw 16-bit patterns.
MOE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
MOE_DEV uint16_t f32_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;   // nearest, ties to even
    const uint32_t q = (u >> 16) | 0x40u;                          // NaN stays a quiet NaN
    return (uint16_t)(((u & 0x7fffffffu) > 0x7f800000u) ? q : r);  // a select, no branch
}

MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

MOE_DEV float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
MOE_DEV float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T>
MOE_DEV T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

inline moe_status launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

// Number of compute units of the current device (cached per device).
int num_cus();

}  // namespace moe
