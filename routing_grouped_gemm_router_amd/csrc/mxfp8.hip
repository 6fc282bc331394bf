// mxfp8.hip -- OCP MXFP8 quantisation on the GPU.
//
// MXFP8 cuts GEMM time, saved activations and the dispatch payload while an
// fp32 master copy of the weights is kept (kongchang.com, "caveats behind the
// numbers"); the format is the OCP one with one shared scale per 32 elements
// (same section). Per OCP Microscaling v1.0: E8M0 shared exponent
// floor(log2 amax) - 8 (8 = E4M3's largest exponent), clamped to
// [-127, 127]; elements x * 2^-shared rounded to nearest even E4M3 (bias 7,
// no infinities) and saturated to +-448.
//
// Both the scale and the element encodings are done with integer operations
// on the fp32 bit pattern:
//   scale byte = max(biased fp32 exponent of amax - 8, 0)   (zero and fp32
//                subnormal amax give byte 0, i.e. 2^-127)
//   element    = fp32 mantissa rounded from 23 to 3 bits (ties to even) and
//                exponent rebased from bias 127 to 7 in the normal range;
//                rint(|v| * 2^9) in the subnormal range (|v| < 2^-6).
// The kernels are HBM-bound: one read of the input, one write of the bytes.
#include "common.h"

namespace moe {

MOE_DEV uint32_t mx_scale_byte(float amax) {
    const int ef = (int)((__float_as_uint(amax) >> 23) & 0xff);
    return (uint32_t)max(ef - 8, 0);
}

// v already multiplied by 2^-shared
MOE_DEV uint32_t e4m3_rne_sat(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7fu;          // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;         // >= 448 (and inf): saturate
    if (a >= 0x3c800000u) {                            // >= 2^-6: normal E4M3
        uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);  // round 20 bits off, ties to even
        r >>= 20;                                      // [fp32 exponent | 3-bit mantissa]
        return sign | (r - (120u << 3));               // rebias 127 -> 7
    }
    const float m = rintf(__uint_as_float(a) * 512.0f);   // subnormal: m * 2^-9, m in 0..8
    return sign | (uint32_t)m;
}

template <bool BF16>
MOE_DEV float load_elem(const void *p, int64_t i) {
    if constexpr (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
    else return reinterpret_cast<const float *>(p)[i];
}

// axis 1: 4 threads per 32-element block, 8 consecutive elements each.
template <bool BF16>
__global__ __launch_bounds__(256) void mx_quant_rows(const void *__restrict__ in, int64_t n_blocks,
                                                     int64_t cols,
                                                     const int32_t *__restrict__ row_map,
                                                     uint8_t *__restrict__ q,
                                                     uint8_t *__restrict__ scale) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = gid >> 2;
    const bool ok = blk < n_blocks;
    // input chunk of 8 elements: same position, or the mapped row
    int64_t src = gid;
    if (row_map && ok) {
        const int64_t r = gid * 8 / cols, c8 = gid - r * (cols / 8);
        src = (int64_t)row_map[r] * (cols / 8) + c8;
    }
    float f[8];
    if (ok) {
        if constexpr (BF16) {
            const uint4 v = reinterpret_cast<const uint4 *>(in)[src];
            f[0] = lo_bf16(v.x); f[1] = hi_bf16(v.x); f[2] = lo_bf16(v.y); f[3] = hi_bf16(v.y);
            f[4] = lo_bf16(v.z); f[5] = hi_bf16(v.z); f[6] = lo_bf16(v.w); f[7] = hi_bf16(v.w);
        } else {
            const float4 a = reinterpret_cast<const float4 *>(in)[src * 2];
            const float4 b = reinterpret_cast<const float4 *>(in)[src * 2 + 1];
            f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
            f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++) f[i] = 0.f;
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(f[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const uint32_t sb = mx_scale_byte(amax);
    if (!ok) return;
    const int sh = 127 - (int)sb;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        lo |= e4m3_rne_sat(ldexpf(f[i], sh)) << (8 * i);
        hi |= e4m3_rne_sat(ldexpf(f[i + 4], sh)) << (8 * i);
    }
    reinterpret_cast<uint2 *>(q)[gid] = make_uint2(lo, hi);
    if ((threadIdx.x & 3) == 0) scale[blk] = (uint8_t)sb;
}

// axis 0, grouped and transposed: one workgroup per 32-row block (global
// block index over all groups), one thread per column.
template <bool BF16>
__global__ __launch_bounds__(256) void mx_quant_cols(const void *__restrict__ in, int64_t rows,
                                                     int64_t cols,
                                                     const int32_t *__restrict__ group_offsets,
                                                     int n_groups,
                                                     const int32_t *__restrict__ row_map,
                                                     uint8_t *__restrict__ q,
                                                     uint8_t *__restrict__ scale) {
    __shared__ int32_t s_bb[1025];   // block base of each group
    __shared__ int32_t s_go[1025];
    const int tid = threadIdx.x;
    for (int g = tid; g <= n_groups; g += 256)
        s_go[g] = group_offsets ? group_offsets[g] : (g == 0 ? 0 : (int32_t)rows);
    __syncthreads();
    if (tid == 0) {
        int32_t acc = 0;
        for (int g = 0; g < n_groups; g++) {
            s_bb[g] = acc;
            acc += 4 * ((s_go[g + 1] - s_go[g] + 127) / 128);   // groups padded to 128 rows
        }
        s_bb[n_groups] = acc;
    }
    __syncthreads();
    const int B = blockIdx.x;
    if (B >= s_bb[n_groups]) return;
    int lo = 0, hi = n_groups - 1;     // group: largest g with s_bb[g] <= B and a block
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (s_bb[mid] <= B) lo = mid; else hi = mid - 1;
    }
    // skip empty groups that share the same base
    while (lo + 1 < n_groups && s_bb[lo + 1] <= B) lo++;
    const int g = lo;
    const int64_t len = s_go[g + 1] - s_go[g];
    const int nb = s_bb[g + 1] - s_bb[g];
    const int b = B - s_bb[g];
    const int64_t r0 = s_go[g] + (int64_t)b * 32;
    const int n = (int)max<int64_t>(0, min<int64_t>(32, len - (int64_t)b * 32));
    uint8_t *qg = q + (int64_t)s_bb[g] * 32 * cols;
    uint8_t *sg = scale + (int64_t)s_bb[g] * cols;
    for (int64_t c = tid; c < cols; c += 256) {
        float f[32];
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 32; i++) {
            const int64_t rr = row_map ? (int64_t)(i < n ? row_map[r0 + i] : 0) : r0 + i;
            f[i] = i < n ? load_elem<BF16>(in, rr * cols + c) : 0.f;
            amax = fmaxf(amax, fabsf(f[i]));
        }
        const uint32_t sb = mx_scale_byte(amax);
        const int sh = 127 - (int)sb;
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            w[i] = 0;
#pragma unroll
            for (int j = 0; j < 4; j++)
                w[i] |= (4 * i + j < n ? e4m3_rne_sat(ldexpf(f[4 * i + j], sh)) : 0u) << (8 * j);
        }
        uint4 *dst = reinterpret_cast<uint4 *>(qg + c * (int64_t)nb * 32 + (int64_t)b * 32);
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
        sg[c * nb + b] = (uint8_t)sb;
    }
}

moe_status mxfp8_quantize_launch(const void *in, moe_dtype in_dt, int64_t rows, int64_t cols,
                                 int axis, const int32_t *group_offsets, int n_groups,
                                 const int32_t *row_map, uint8_t *q, uint8_t *scale,
                                 hipStream_t s) {
    const bool bf = in_dt == MOE_BF16;
    if (axis == 1) {
        const int64_t n_blocks = rows * cols / 32;
        const unsigned grid = (unsigned)((n_blocks * 4 + 255) / 256);
        if (bf) mx_quant_rows<true><<<grid, 256, 0, s>>>(in, n_blocks, cols, row_map, q, scale);
        else mx_quant_rows<false><<<grid, 256, 0, s>>>(in, n_blocks, cols, row_map, q, scale);
    } else {
        // upper bound of the padded block count: sum_g 4*ceil(len_g/128)
        const unsigned grid = (unsigned)(rows / 32 + 4 * (int64_t)n_groups + 4);
        if (bf) mx_quant_cols<true><<<grid, 256, 0, s>>>(in, rows, cols, group_offsets, n_groups, row_map, q, scale);
        else mx_quant_cols<false><<<grid, 256, 0, s>>>(in, rows, cols, group_offsets, n_groups, row_map, q, scale);
    }
    return launch_status();
}

// size in bytes of the column-block layout's element array (scale array =
// this / 32) for `rows` rows in n_groups groups: (rows/32 + 4*n_groups + 4) blocks
size_t mxfp8_col_blocks(int64_t rows, int n_groups) {
    return (size_t)(rows / 32 + 4 * (int64_t)n_groups + 4);
}

}  // namespace moe
