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

// fp32 -> bf16, round to nearest even (IEEE conversion; CDNA4 does it in one
// instruction, v_cvt_pk_bf16_f32, two values at a time); NaN stays a NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
MOE_DEV uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

MOE_DEV float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
MOE_DEV float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T>
MOE_DEV T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// lane moves inside a quad of lanes (DPP, no LDS)
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7 - i within each 8 lanes
constexpr int kDppRowShl4 = 0x104;    // lane i <- lane i + 4 within each 16 lanes (others keep 0)
constexpr int kDppRowShl8 = 0x108;    // lane i <- lane i + 8 within each 16 lanes (others keep 0)
constexpr int kDppRowRor4 = 0x124;    // each 16 lanes rotated by 4 (row_ror:4)
constexpr int kDppRowRor8 = 0x128;    // each 16 lanes rotated by 8 (row_ror:8)
template <int CTRL>
MOE_DEV int dpp_move(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
MOE_DEV float dpp_move(float v) {
    return __int_as_float(dpp_move<CTRL>(__float_as_int(v)));
}

// max of v over lanes i and i ^ 16 (within each 32 lanes) and over lanes i
// and i ^ 32: v_permlane16_swap / v_permlane32_swap exchange the odd 16-lane
// (32-lane) rows of one operand with the even rows of the other, so with v as
// both operands the two results hold v and its partner lane's v (VALU, no LDS)
MOE_DEV float max_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
MOE_DEV float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

inline moe_status launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

// Number of compute units of the current device.
int num_cus();

// Bytes of the device array moe_route_noalloc uses instead of a workspace.
constexpr size_t kRouteNoAllocScratchBytes = MOE_ROUTE_NOALLOC_SCRATCH_BYTES;

}  // namespace moe
