// mx_encode.h -- the OCP MXFP8 encoding steps shared by the quantisers
// (mxfp8.hip) and the grouped GEMM's quantising SwiGLU epilogue (gemm.hip):
// the E8M0 scale byte of a 32-element block and the E4M3 bytes of its
// elements. The format, the rounding and the NaN rules are described at the
// top of mxfp8.hip.
#pragma once

#include "common.h"

namespace moe {

MOE_DEV uint32_t mx_scale_byte(float amax) {
    const int ef = (int)((__float_as_uint(amax) >> 23) & 0xff);
    return (uint32_t)max(ef - 8, 0);
}

// four elements, scaled by 2^(127 - sb), to four E4M3 bytes (first element
// lowest). With no NaN in the wave (the rule): each value is clamped to
// +-448 * 2^(sb - 127) by one v_med3_f32 and the pair converted by
// v_cvt_scalef32_pk_fp8_f32, which takes the E8M0 byte as the exponent field
// of its scale operand and divides by it (checked on the GPU on every bf16
// pattern and every scale byte 0..254: the same bytes as the form below).
// med3 maps a NaN to a finite value, so a wave that holds one takes the
// select form, which scales with ldexp, saturates and patches NaN signs.
//
// The form for four values none of which is a NaN (a condition on the lane's
// own values).
MOE_DEV uint32_t e4m3x4_finite(float a, float b, float c, float d, uint32_t sb) {
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    const float x[4] = {a, b, c, d};
    const float scale = __uint_as_float(sb << 23);
    const float bound = sb + 8 < 255 ? __uint_as_float(((sb + 8) << 23) | 0x600000u)
                                     : __builtin_inff();   // 448 * 2^(sb - 127)
    float cl[4];
#pragma unroll
    for (int i = 0; i < 4; i++) cl[i] = __builtin_amdgcn_fmed3f(x[i], -bound, bound);
    const s16x2 z = {0, 0};
    const s16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, cl[0], cl[1], scale, false);
    const s16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, cl[2], cl[3], scale, true);
    return (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
}

// The form for any values, NaN included.
MOE_DEV uint32_t e4m3x4_select(float a, float b, float c, float d, uint32_t sb) {
    const float x[4] = {a, b, c, d};
    const int sh = 127 - (int)sb;
    float cl[4];
    uint32_t pnan = 0;                                  // positive NaNs: 0xff -> 0x7f
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float v = ldexpf(x[i], sh);
        cl[i] = fabsf(v) > 448.0f ? copysignf(448.0f, v) : v;
        pnan |= ((int32_t)__float_as_uint(v) > 0x7f800000) ? 0x80u << (8 * i) : 0u;
    }
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl[0], cl[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(cl[2], cl[3], w, true);
    return (uint32_t)w ^ pnan;
}

MOE_DEV bool any_nan4(float a, float b, float c, float d) {
    return __builtin_isnan(a) || __builtin_isnan(b) || __builtin_isnan(c) || __builtin_isnan(d);
}

// The wave takes the first form unless one of its lanes holds a NaN.
MOE_DEV uint32_t e4m3x4(float a, float b, float c, float d, uint32_t sb) {
    return __ballot(any_nan4(a, b, c, d)) == 0 ? e4m3x4_finite(a, b, c, d, sb)
                                               : e4m3x4_select(a, b, c, d, sb);
}

}  // namespace moe
