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
// The scale is taken from the fp32 bit pattern:
//   scale byte = max(biased fp32 exponent of amax - 8, 0)   (zero and fp32
//                subnormal amax give byte 0, i.e. 2^-127)
// The elements x * 2^-shared are encoded by the CDNA4 conversion instructions
// (OCP E4M3, round to nearest even) on inputs clamped to +-448 (after the
// scaling), which is the saturation. Waves without a NaN clamp with
// v_med3_f32 and convert with v_cvt_scalef32_pk_fp8_f32, which applies the
// shared exponent itself; a wave with a NaN scales with ldexp and converts
// with v_cvt_pk_fp8_f32, whose only departure from the format is a NaN,
// written as 0xff whatever the sign, so a positive NaN is patched to 0x7f.
// Checked on the GPU: the ldexp form against an integer encoding of the
// format (mantissa rounded from 23 to 3 bits ties to even, exponent rebased
// from 127 to 7; rint(|v| * 2^9) below 2^-6) on all 2^32 fp32 patterns,
// identical except NaN's sign, which the patch restores; the scaled form
// against the ldexp form on all 2^32 non-NaN fp32 patterns for scale bytes
// 0, 1, 64, 119, 120, 127, 134, 200, 246, 254 and on every bf16 pattern for
// every scale byte 0..254, identical.
// Each kernel reads its input once and writes each output once; the encoding
// arithmetic is about half of the time of the both-layouts kernels, memory
// traffic the rest.
#include "common.h"
#include "mx_encode.h"

namespace moe {

template <bool BF16>
MOE_DEV float load_elem(const void *p, int64_t i) {
    if constexpr (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
    else return reinterpret_cast<const float *>(p)[i];
}

// axis 1: 2 threads per 32-element block, 16 consecutive elements each
// (32 B of bf16 in, one 16-B store out).
template <bool BF16>
__global__ __launch_bounds__(256) void mx_quant_rows(const void *__restrict__ in, int64_t n_blocks,
                                                     int64_t cols,
                                                     const int32_t *__restrict__ row_map,
                                                     uint8_t *__restrict__ q,
                                                     uint8_t *__restrict__ scale) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 16-element chunk
    const int64_t blk = gid >> 1;
    const bool ok = blk < n_blocks;
    int64_t src = gid * 16;                                          // element offset of the chunk
    if (row_map && ok) {
        const int64_t r = src / cols;
        src = (int64_t)row_map[r] * cols + (src - r * cols);
    }
    float f[16];
    if (ok) {
        if constexpr (BF16) {
            const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(in) + src);
            const uint4 v0 = p[0], v1 = p[1];
            const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int i = 0; i < 8; i++) { f[2 * i] = lo_bf16(w[i]); f[2 * i + 1] = hi_bf16(w[i]); }
        } else {
            const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(in) + src);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float4 a = p[i];
                f[4 * i] = a.x; f[4 * i + 1] = a.y; f[4 * i + 2] = a.z; f[4 * i + 3] = a.w;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; i++) f[i] = 0.f;
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i++) amax = fmaxf(amax, fabsf(f[i]));
    amax = fmaxf(amax, dpp_move<kDppXor1>(amax));
    const uint32_t sb = mx_scale_byte(amax);
    if (!ok) return;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++) w[i] = e4m3x4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3], sb);
    reinterpret_cast<uint4 *>(q)[gid] = make_uint4(w[0], w[1], w[2], w[3]);
    if ((threadIdx.x & 1) == 0) scale[blk] = (uint8_t)sb;
}

// Inclusive prefix sum over a 256-thread workgroup (s_w: 4 ints of LDS).
MOE_DEV int block_incl_scan(int v, int *s_w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    if (lane == 63) s_w[wave] = v;
    __syncthreads();
    for (int w = 0; w < wave; w++) v += s_w[w];
    return v;
}

// Unit geometry of the grouped column-block layout. A group's output is a
// sequence of 128-row units (4 blocks of 32 rows); units are numbered over all
// groups. Every workgroup first builds s_ub (first unit of each group, by a
// parallel prefix sum of ceil(len/128)) and s_go (the offsets).
struct ColUnits {
    int32_t ub[1025];
    int32_t go[1025];
    int w[4];
};

MOE_DEV int col_units_init(ColUnits &cu, const int32_t *group_offsets, int ng, int64_t rows) {
    const int tid = threadIdx.x;
    int u[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int g = 4 * tid + i;
        u[i] = 0;
        if (g < ng) {
            const int32_t a = group_offsets ? group_offsets[g] : 0;
            const int32_t b = group_offsets ? group_offsets[g + 1] : (int32_t)rows;
            cu.go[g] = a;
            if (g == ng - 1) cu.go[ng] = b;
            u[i] = (b - a + 127) / 128;
        }
        sum += u[i];
    }
    int ex = block_incl_scan(sum, cu.w) - sum;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int g = 4 * tid + i;
        if (g < ng) cu.ub[g] = ex;
        ex += u[i];
        if (g == ng - 1) cu.ub[ng] = ex;
    }
    __syncthreads();
    return cu.ub[ng];
}

struct UnitGeom {
    int64_t r0, nb, bb;   // first input row, blocks of the group, first block of the group
    int j, n;             // unit within the group, valid rows (1..128)
};

MOE_DEV UnitGeom unit_geom(const ColUnits &cu, int ng, int unit) {
    int lo = 0, hi = ng - 1;              // largest g with ub[g] <= unit (it has units)
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu.ub[mid] <= unit) lo = mid; else hi = mid - 1;
    }
    UnitGeom u;
    u.j = unit - cu.ub[lo];
    u.nb = 4 * (int64_t)(cu.ub[lo + 1] - cu.ub[lo]);
    u.bb = 4 * (int64_t)cu.ub[lo];
    u.r0 = (int64_t)cu.go[lo] + 128 * (int64_t)u.j;
    u.n = (int)min<int64_t>(128, (int64_t)cu.go[lo + 1] - u.r0);
    return u;
}

// Encode 32 values (one column block) to 32 E4M3 bytes at dst (16-B aligned)
// and return the scale byte.
MOE_DEV uint32_t encode_block32(const float *f, uint8_t *dst) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(f[i]));
    const uint32_t sb = mx_scale_byte(amax);
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; i++) w[i] = e4m3x4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3], sb);
    uint4 *d = reinterpret_cast<uint4 *>(dst);
    d[0] = make_uint4(w[0], w[1], w[2], w[3]);
    d[1] = make_uint4(w[4], w[5], w[6], w[7]);
    return sb;
}

// axis 0, fp32 input (weights; once per weight update). Persistent over
// units like the bf16 kernel below: a workgroup owns 64 columns and walks
// units blockIdx.y, blockIdx.y + gridDim.y, ...; the next unit's 32 KiB tile
// is loaded into registers while the current one is encoded. The 128 x 64
// tile is read with 16-B row loads, transposed through LDS, and each thread
// encodes one 32-row block of one column; 4 neighbouring threads write the
// column's 128 contiguous bytes.
// BOTH: the loaded rows are also quantised along the columns into the
// row-major axis-1 layout (q1, s1): a 32-column block is 8 neighbouring
// lanes of one row, so the fp32 masters are read once for both orientations.
template <bool BOTH>
__global__ __launch_bounds__(256) void mx_quant_cols_f32(const float *__restrict__ in, int64_t rows,
                                                         int64_t cols,
                                                         const int32_t *__restrict__ group_offsets,
                                                         int n_groups,
                                                         const int32_t *__restrict__ row_map,
                                                         uint8_t *__restrict__ q,
                                                         uint8_t *__restrict__ scale,
                                                         uint8_t *__restrict__ q1,
                                                         uint8_t *__restrict__ s1) {
    constexpr int TP = 129;               // LDS pitch (floats) of one column: conflict-free writes
    __shared__ float s_t[64 * TP];
    __shared__ ColUnits cu;
    const int tid = threadIdx.x;
    const int ng = group_offsets ? n_groups : 1;
    const int n_units = col_units_init(cu, group_offsets, ng, rows);
    const int64_t c0 = (int64_t)blockIdx.x * 64;
    const int ch = tid & 15, rr = tid >> 4;   // 4 columns per load, 16 loads per row
    const bool cok = c0 + 4 * ch < cols;

    float4 v[8];                          // rows rr + 16 p
    auto load = [&](const UnitGeom &u) {
#pragma unroll
        for (int p = 0; p < 8; p++) {
            const int r = rr + 16 * p;
            v[p] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < u.n && cok) {
                const int64_t src = row_map ? (int64_t)row_map[u.r0 + r] : u.r0 + r;
                v[p] = *reinterpret_cast<const float4 *>(in + src * cols + c0 + 4 * ch);
            }
        }
    };
    int unit = blockIdx.y;
    if (unit >= n_units) return;          // uniform over the workgroup
    UnitGeom u = unit_geom(cu, ng, unit);
    load(u);
    while (true) {
#pragma unroll
        for (int p = 0; p < 8; p++) {
            const int r = rr + 16 * p;
            s_t[(4 * ch) * TP + r] = v[p].x;
            s_t[(4 * ch + 1) * TP + r] = v[p].y;
            s_t[(4 * ch + 2) * TP + r] = v[p].z;
            s_t[(4 * ch + 3) * TP + r] = v[p].w;
            if constexpr (BOTH) {
                // from 0, so that NaN elements never enter the block maximum
                float am = fmaxf(fmaxf(fmaxf(0.f, fabsf(v[p].x)), fabsf(v[p].y)),
                                 fmaxf(fabsf(v[p].z), fabsf(v[p].w)));
                // max over the 8 lanes of the block (lane moves, no LDS)
                am = fmaxf(am, dpp_move<kDppXor1>(am));
                am = fmaxf(am, dpp_move<kDppXor2>(am));
                am = fmaxf(am, dpp_move<kDppHalfMirror>(am));
                if (r < u.n && cok) {
                    const uint32_t sb = mx_scale_byte(am);
                    const uint32_t w = e4m3x4(v[p].x, v[p].y, v[p].z, v[p].w, sb);
                    *reinterpret_cast<uint32_t *>(q1 + (u.r0 + r) * cols + c0 + 4 * ch) = w;
                    if ((ch & 7) == 0) s1[(u.r0 + r) * (cols / 32) + (c0 + 4 * ch) / 32] = (uint8_t)sb;
                }
            }
        }
        __syncthreads();
        const UnitGeom cur = u;
        const int next = unit + gridDim.y;
        if (next < n_units) {             // prefetch the next tile while this one is encoded
            u = unit_geom(cu, ng, next);
            load(u);
        }
        const int cc = tid >> 2, b = tid & 3;
        const int64_t c = c0 + cc;
        if (c < cols) {
            float f[32];
#pragma unroll
            for (int i = 0; i < 32; i++) f[i] = s_t[cc * TP + 32 * b + i];
            const uint32_t sb = encode_block32(f, q + cur.bb * 32 * cols + c * cur.nb * 32 + 128 * (int64_t)cur.j + 32 * b);
            scale[cur.bb * cols + c * cur.nb + 4 * cur.j + b] = (uint8_t)sb;
        }
        if (next >= n_units) break;
        unit = next;
        __syncthreads();                  // s_t is rewritten by the next unit
    }
}

// axis 0, bf16 input (activations and gradients, every step). Persistent over
// units: a workgroup owns 128 columns and walks units blockIdx.y,
// blockIdx.y + gridDim.y, ...; the next unit's 32 KiB tile is loaded into
// registers while the current one is encoded. Sixteen lanes read a row's 256
// bytes: thread (ch = tid % 16, q = tid / 16) loads 8 columns of rows
// 2q + {0, 1} + 32k. LDS holds the tile transposed as packed row pairs (dword
// = rows 2i, 2i+1 of one column, pitch 65 dwords); the column-block reads
// are conflict-free. Column tiles vary fastest over the grid, so
// neighbouring workgroups stream the same input rows.
// BOTH: the tile is also quantised along its rows into the row-major axis-1
// layout (q1, s1), row index = position in the grouped order, which saves a
// second read of tensors needed in both orientations. Each lane pair writes
// 16 bytes, so a row's 128 bytes go out as one full line, and its four scale
// bytes as one word.
// row_scale (with row_map): the rows quantised are round_bf16(row_scale[r] *
// in[row_map[r]]), formed as they are loaded: the MXFP8 backward's dy rows
// (each routed row's gate times its token's dOut row, rounded to bf16 as the
// combine backward would store them) without a stored copy.
template <bool BOTH>
__global__ __launch_bounds__(256) void mx_quant_cols_bf16(const uint16_t *__restrict__ in,
                                                          int64_t rows, int64_t cols,
                                                          const int32_t *__restrict__ group_offsets,
                                                          int n_groups,
                                                          const int32_t *__restrict__ row_map,
                                                          const float *__restrict__ row_scale,
                                                          uint8_t *__restrict__ q,
                                                          uint8_t *__restrict__ scale,
                                                          uint8_t *__restrict__ q1,
                                                          uint8_t *__restrict__ s1) {
    constexpr int TP = 65;
    __shared__ uint32_t s_t[128 * TP];
    __shared__ ColUnits cu;
    const int tid = threadIdx.x, lane = tid & 63;
    const int ng = group_offsets ? n_groups : 1;
    const int n_units = col_units_init(cu, group_offsets, ng, rows);
    const int64_t c0 = (int64_t)blockIdx.x * 128;
    const int ch = tid & 15, qr = tid >> 4;
    // cols % 32 == 0: the four 8-column chunks of a 32-column block are all
    // in range or all out
    const bool cok = c0 + 8 * ch < cols;
    // a row's four scale bytes as one word: whole tile, word-aligned rows
    const bool full_row = c0 + 128 <= cols && cols % 128 == 0 && ((uintptr_t)s1 & 3) == 0;

    uint4 v[8];                           // v[p]: row 2qr + (p & 1) + 32 (p >> 1)
    // row_map: this thread's source rows (and row_scale: their scales) of the
    // next unit to load, read one unit ahead so that the tile loads do not
    // wait on the index loads
    int32_t ri[8];
    float rs[8], rs_v[8];                 // scales of the next unit; of the loaded one
    auto rows_of = [&](const UnitGeom &u) {
#pragma unroll
        for (int p = 0; p < 8; p++) {
            const int r = 2 * qr + (p & 1) + 32 * (p >> 1);
            const bool ok = r < u.n && cok;
            ri[p] = ok ? row_map[u.r0 + r] : 0;
            if (row_scale) rs[p] = ok ? row_scale[u.r0 + r] : 0.f;
        }
    };
    auto load = [&](const UnitGeom &u) {
#pragma unroll
        for (int p = 0; p < 8; p++) {
            const int r = 2 * qr + (p & 1) + 32 * (p >> 1);
            v[p] = make_uint4(0, 0, 0, 0);
            if (r < u.n && cok) {
                const int64_t src = row_map ? (int64_t)ri[p] : u.r0 + r;
                v[p] = *reinterpret_cast<const uint4 *>(in + src * cols + c0 + 8 * ch);
            }
            if (row_scale) rs_v[p] = rs[p];
        }
    };
    int unit = blockIdx.y;
    if (unit >= n_units) return;          // uniform over the workgroup
    UnitGeom u = unit_geom(cu, ng, unit);
    if (row_map) rows_of(u);
    load(u);
    if (row_map && unit + (int)gridDim.y < n_units) rows_of(unit_geom(cu, ng, unit + gridDim.y));
    while (true) {
        if (row_scale) {                  // the scaled rows, rounded to bf16
#pragma unroll
            for (int p = 0; p < 8; p++) {
                uint32_t w[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
#pragma unroll
                for (int e = 0; e < 4; e++) w[e] = pack_bf16x2(rs_v[p] * lo_bf16(w[e]), rs_v[p] * hi_bf16(w[e]));
                v[p] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
        // registers -> LDS (packed row pairs)
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint4 a = v[2 * k], b = v[2 * k + 1];     // rows r, r+1
            const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
            const int pr = qr + 16 * k;                      // row pair index
#pragma unroll
            for (int e = 0; e < 4; e++) {
                s_t[(8 * ch + 2 * e) * TP + pr] = (wa[e] & 0xffffu) | (wb[e] << 16);
                s_t[(8 * ch + 2 * e + 1) * TP + pr] = (wa[e] >> 16) | (wb[e] & 0xffff0000u);
            }
        }
        if constexpr (BOTH) {             // 32-column block = 4 neighbouring lanes of one row
#pragma unroll
            for (int p = 0; p < 8; p++) {
                const int r = 2 * qr + (p & 1) + 32 * (p >> 1);
                const uint32_t w[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
                float f[8];
#pragma unroll
                for (int e = 0; e < 4; e++) { f[2 * e] = lo_bf16(w[e]); f[2 * e + 1] = hi_bf16(w[e]); }
                float am = 0.f;
#pragma unroll
                for (int e = 0; e < 8; e++) am = fmaxf(am, fabsf(f[e]));
                // max over the block's 4 lanes (lane moves, no LDS)
                am = fmaxf(am, dpp_move<kDppXor1>(am));
                am = fmaxf(am, dpp_move<kDppXor2>(am));
                const uint32_t sb = mx_scale_byte(am);
                const uint32_t lo4 = e4m3x4(f[0], f[1], f[2], f[3], sb);
                const uint32_t hi4 = e4m3x4(f[4], f[5], f[6], f[7], sb);
                // the odd lane's 8 bytes go out with the even lane's store
                const uint32_t plo = (uint32_t)dpp_move<kDppXor1>((int)lo4);
                const uint32_t phi = (uint32_t)dpp_move<kDppXor1>((int)hi4);
                // the row's four scale bytes (lanes rl, rl + 4, rl + 8, rl + 12)
                // as one word in lane rl
                const uint32_t s2 = sb | ((uint32_t)dpp_move<kDppRowShl4>((int)sb) << 8);
                const uint32_t s4 = s2 | ((uint32_t)dpp_move<kDppRowShl8>((int)s2) << 16);
                if (r < u.n && cok) {
                    uint8_t *qrow = q1 + (u.r0 + r) * cols + c0;
                    if ((ch & 1) == 0)
                        *reinterpret_cast<uint4 *>(qrow + 8 * ch) = make_uint4(lo4, hi4, plo, phi);
                    uint8_t *srow = s1 + (u.r0 + r) * (cols / 32) + c0 / 32;
                    if (full_row) {
                        if (ch == 0) *reinterpret_cast<uint32_t *>(srow) = s4;
                    } else if ((ch & 3) == 0) {
                        srow[ch / 4] = (uint8_t)sb;
                    }
                }
            }
        }
        __syncthreads();
        const UnitGeom cur = u;
        const int next = unit + gridDim.y;
        if (next < n_units) {             // prefetch the next tile while this one is encoded
            u = unit_geom(cu, ng, next);
            load(u);
            if (row_map && next + (int)gridDim.y < n_units) rows_of(unit_geom(cu, ng, next + gridDim.y));
        }
#pragma unroll
        for (int pass = 0; pass < 2; pass++) {
            const int cc = (tid >> 2) + 64 * pass, b = tid & 3;
            const int64_t c = c0 + cc;
            if (c < cols) {
                float f[32];
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const uint32_t w = s_t[cc * TP + 16 * b + i];
                    f[2 * i] = lo_bf16(w);
                    f[2 * i + 1] = hi_bf16(w);
                }
                const uint32_t sb = encode_block32(f, q + cur.bb * 32 * cols + c * cur.nb * 32 + 128 * (int64_t)cur.j + 32 * b);
                scale[cur.bb * cols + c * cur.nb + 4 * cur.j + b] = (uint8_t)sb;
            }
        }
        if (next >= n_units) break;
        unit = next;
        __syncthreads();                  // s_t is rewritten by the next unit
    }
}

#ifndef MOE_COLS_PER_CU
#define MOE_COLS_PER_CU 3
#endif
constexpr int kColsPerCU = MOE_COLS_PER_CU;   // the bf16 tile's 41 KiB of LDS: three workgroups per CU
constexpr int kColsPerCUF32 = 4;          // the fp32 tile's 33 KiB of LDS: four workgroups per CU

// column tiles along x; units (upper bound sum_g ceil(len_g/128) <= rows/128 + groups) along
// y, `per_cu` workgroups per CU in all when the kernel walks several units
static dim3 cols_grid(int64_t rows, int64_t cols, int ng, int per_cu, int tile_cols) {
    const int64_t xt = (cols + tile_cols - 1) / tile_cols;
    int64_t y = rows / 128 + ng + 1;
    if (per_cu > 0) {
        const int64_t want = ((int64_t)num_cus() * per_cu + xt - 1) / xt;
        if (want < y) y = want;
    }
    if (y > 65535) y = 65535;
    return dim3((unsigned)xt, (unsigned)(y < 1 ? 1 : y));
}

moe_status mxfp8_quantize_launch(const void *in, moe_dtype in_dt, int64_t rows, int64_t cols,
                                 int axis, const int32_t *group_offsets, int n_groups,
                                 const int32_t *row_map, uint8_t *q, uint8_t *scale,
                                 hipStream_t s) {
    const bool bf = in_dt == MOE_BF16;
    if (axis == 1) {
        const int64_t n_blocks = rows * cols / 32;
        const unsigned grid = (unsigned)((n_blocks * 2 + 255) / 256);
        if (bf) mx_quant_rows<true><<<grid, 256, 0, s>>>(in, n_blocks, cols, row_map, q, scale);
        else mx_quant_rows<false><<<grid, 256, 0, s>>>(in, n_blocks, cols, row_map, q, scale);
    } else {
        const int ng = group_offsets ? n_groups : 1;
        if (bf)
            mx_quant_cols_bf16<false><<<cols_grid(rows, cols, ng, kColsPerCU, 128), 256, 0, s>>>(
                (const uint16_t *)in, rows, cols, group_offsets, n_groups, row_map, nullptr, q,
                scale, nullptr, nullptr);
        else
            mx_quant_cols_f32<false><<<cols_grid(rows, cols, ng, kColsPerCUF32, 64), 256, 0, s>>>(
                (const float *)in, rows, cols, group_offsets, n_groups, row_map, q, scale, nullptr,
                nullptr);
    }
    return launch_status();
}

// bf16 or fp32 [rows, cols] in grouped row order -> both the row-major
// axis-1 layout (q1, s1) and the grouped column-block layout (q0, s0), from
// one read.
moe_status mxfp8_quantize_both_launch(const void *in, moe_dtype in_dt, int64_t rows, int64_t cols,
                                      const int32_t *group_offsets, int n_groups, uint8_t *q1,
                                      uint8_t *s1, uint8_t *q0, uint8_t *s0, hipStream_t s,
                                      const int32_t *row_map, const float *row_scale) {
    const int ng = group_offsets ? n_groups : 1;
    if ((row_map || row_scale) && in_dt != MOE_BF16) return MOE_ERR_DTYPE;
    if (row_scale && !row_map) return MOE_ERR_NULL;
    if (in_dt == MOE_BF16)
        mx_quant_cols_bf16<true><<<cols_grid(rows, cols, ng, kColsPerCU, 128), 256, 0, s>>>(
            (const uint16_t *)in, rows, cols, group_offsets, n_groups, row_map, row_scale, q0, s0,
            q1, s1);
    else
        mx_quant_cols_f32<true><<<cols_grid(rows, cols, ng, kColsPerCUF32, 64), 256, 0, s>>>(
            (const float *)in, rows, cols, group_offsets, n_groups, nullptr, q0, s0, q1, s1);
    return launch_status();
}

// size in bytes of the column-block layout's element array (scale array =
// this / 32) for `rows` rows in n_groups groups: (rows/32 + 4*n_groups + 4) blocks
size_t mxfp8_col_blocks(int64_t rows, int n_groups) {
    return (size_t)(rows / 32 + 4 * (int64_t)n_groups + 4);
}

}  // namespace moe
