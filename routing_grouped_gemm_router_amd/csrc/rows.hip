// rows.hip -- HBM-bound row movers: dispatch, combine and their backwards.
//
// Row-wise dispatch writes each selected token row straight into the expert
// input buffers, which removes a separate reordering pass (bytechap.com, "How
// it works"; kongchang.com, "capacity tax"). Here it is a scatter in token
// order: each token row is read from HBM once and stored to its k rows, so the
// traffic is the algorithmic minimum (T*d read, T*k*d written). Rows are whole
// contiguous runs of d elements, so every wave issues full 16-byte-per-lane
// (1 KiB per instruction) loads and stores; staging them through LDS would
// only add a round trip.
//
// One wave per token row in every kernel; four tokens per 256-thread block.
#include "common.h"

namespace moe {

constexpr int kRowWaves = 4;
constexpr int kUnroll = 4;   // combine kernels: 16-byte column chunks per lane in flight together

// Non-temporal 16-byte loads of rows read exactly once (the combine kernels'
// gathered rows, the combine backward's dOut): measured in the layer step at
// T=16384, d=2048, k=4 bf16, combine 64 -> 58 us and the unpermute backward
// 72 -> 67 us. Stores stay ordinary: the next kernel reads x_perm and dy_perm
// while they are still in the last-level cache (non-temporal stores made the
// dispatch 53 -> 65 us and the GEMMs reading its output ~4 % slower).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
MOE_DEV uint4 ld16_nt(const uint4 *p) {
    const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(w.x, w.y, w.z, w.w);
}

// ---------------------------------------------------------------------------
// dispatch: x_perm[token_pos[t, j]] = x[t]

template <int KMAX>
__global__ __launch_bounds__(256) void permute_rows16(const uint4 *__restrict__ x, int64_t T,
                                                      int n16, int k,
                                                      const int32_t *__restrict__ token_pos,
                                                      uint4 *__restrict__ x_perm) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6);
    if (t >= T) return;
    int32_t pos[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; j++) pos[j] = j < k ? token_pos[t * k + j] : -1;
    const uint4 *src = x + t * n16;
    int c = lane;
    // four 16-byte loads in flight per lane, then k stores of each
    for (; c + 3 * 64 < n16; c += 4 * 64) {
        uint4 v0 = src[c], v1 = src[c + 64], v2 = src[c + 128], v3 = src[c + 192];
#pragma unroll
        for (int j = 0; j < KMAX; j++) {
            if (pos[j] < 0) continue;
            uint4 *dst = x_perm + (int64_t)pos[j] * n16;
            dst[c] = v0; dst[c + 64] = v1; dst[c + 128] = v2; dst[c + 192] = v3;
        }
    }
    for (; c < n16; c += 64) {
        uint4 v = src[c];
#pragma unroll
        for (int j = 0; j < KMAX; j++)
            if (pos[j] >= 0) x_perm[(int64_t)pos[j] * n16 + c] = v;
    }
}

// byte-granular variant for short rows (MXFP8 scale rows of d/32 bytes)
__global__ __launch_bounds__(256) void permute_rows_bytes(const uint8_t *__restrict__ x, int64_t T,
                                                          int nbytes, int k,
                                                          const int32_t *__restrict__ token_pos,
                                                          uint8_t *__restrict__ x_perm) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6);
    if (t >= T) return;
    for (int j = 0; j < k; j++) {
        int32_t p = token_pos[t * k + j];
        if (p < 0) continue;
        for (int c = lane; c < nbytes; c += 64) x_perm[(int64_t)p * nbytes + c] = x[t * nbytes + c];
    }
}

// ---------------------------------------------------------------------------
// combine: out[t] = sum_j g[t,j] * y[token_pos[t,j]]   (fp32 sum, ascending j)
// unpermute backward is the same with unit gates: dX[t] = sum_j dx_perm[...]

template <bool BF16>
MOE_DEV void load_f32(const uint4 &v, float *f) {
    if constexpr (BF16) {
        f[0] = lo_bf16(v.x); f[1] = hi_bf16(v.x); f[2] = lo_bf16(v.y); f[3] = hi_bf16(v.y);
        f[4] = lo_bf16(v.z); f[5] = hi_bf16(v.z); f[6] = lo_bf16(v.w); f[7] = hi_bf16(v.w);
    } else {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
}

template <bool BF16>
MOE_DEV uint4 store_f32(const float *f) {
    uint4 v;
    if constexpr (BF16) {
        v.x = pack_bf16x2(f[0], f[1]); v.y = pack_bf16x2(f[2], f[3]);
        v.z = pack_bf16x2(f[4], f[5]); v.w = pack_bf16x2(f[6], f[7]);
    } else {
        v.x = __float_as_uint(f[0]); v.y = __float_as_uint(f[1]);
        v.z = __float_as_uint(f[2]); v.w = __float_as_uint(f[3]);
    }
    return v;
}

template <bool BF16, bool UNIT, int KMAX>
__global__ __launch_bounds__(256) void combine_rows(const uint4 *__restrict__ y,
                                                    const float *__restrict__ gate,
                                                    const int32_t *__restrict__ token_pos,
                                                    int64_t T, int n16, int k,
                                                    uint4 *__restrict__ out) {
    constexpr int EPV = BF16 ? 8 : 4;   // elements per 16-byte vector
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6);
    if (t >= T) return;
    int32_t pos[KMAX];
    float g[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; j++) {
        pos[j] = j < k ? token_pos[t * k + j] : -1;
        g[j] = (j < k && !UNIT) ? gate[t * k + j] : 1.f;
    }
    // kUnroll column chunks per lane at a time: all their row loads are in
    // flight before the first sum
    for (int c0 = lane; c0 < n16; c0 += 64 * kUnroll) {
        uint4 v[kUnroll][KMAX];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int c = c0 + 64 * u;
#pragma unroll
            for (int j = 0; j < KMAX; j++)
                if (c < n16 && pos[j] >= 0) v[u][j] = ld16_nt(y + (int64_t)pos[j] * n16 + c);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int c = c0 + 64 * u;
            if (c >= n16) break;
            float acc[EPV];
#pragma unroll
            for (int i = 0; i < EPV; i++) acc[i] = 0.f;
#pragma unroll
            for (int j = 0; j < KMAX; j++) {
                if (pos[j] < 0) continue;
                float f[EPV];
                load_f32<BF16>(v[u][j], f);
#pragma unroll
                for (int i = 0; i < EPV; i++) acc[i] = UNIT ? acc[i] + f[i] : fmaf(g[j], f[i], acc[i]);
            }
            out[t * n16 + c] = store_f32<BF16>(acc);
        }
    }
}

// ---------------------------------------------------------------------------
// combine backward with the router backward fused in:
//   dy_perm[p_j] = round(g_j * dOut[t]),  dg_j = <dOut[t], y_perm[p_j]>
//   dlogits[t, e_j] = g_j (dg_j - sum_i g_i dg_i); 0 for unselected experts
// The gates sum to one, so the router term is evaluated as
//   g_j sum_i g_i (dg_j - dg_i),
// which equals it exactly but has no cancellation: with one gate near 1
// (a confident router) the first form subtracts two nearly equal sums and
// loses about log2(1 / (1 - g)) bits in fp32.
// DY = false (the MXFP8 backward, whose quantiser forms dy_perm itself from
// dOut and the gates): no dy rows; row_gate[p_j] = g_j instead.

template <bool BF16, int KMAX, bool DY = true>
__global__ __launch_bounds__(256) void combine_bwd_rows(
    const uint4 *__restrict__ dout, const uint4 *__restrict__ y, const float *__restrict__ gate,
    const int32_t *__restrict__ topk_idx, const int32_t *__restrict__ token_pos, int64_t T,
    int n16, int k, int E, uint4 *__restrict__ dy, float *__restrict__ dlogits,
    float *__restrict__ dgate) {
    constexpr int EPV = BF16 ? 8 : 4;
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6);
    if (t >= T) return;
    int32_t pos[KMAX], ex[KMAX];
    float g[KMAX], dot[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; j++) {
        pos[j] = j < k ? token_pos[t * k + j] : -1;
        ex[j] = j < k ? topk_idx[t * k + j] : -1;
        g[j] = j < k ? gate[t * k + j] : 0.f;
        dot[j] = 0.f;
    }
    for (int c0 = lane; c0 < n16; c0 += 64 * kUnroll) {
        uint4 vo[kUnroll], v[kUnroll][KMAX];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int c = c0 + 64 * u;
            if (c < n16) vo[u] = ld16_nt(dout + t * n16 + c);
#pragma unroll
            for (int j = 0; j < KMAX; j++)
                if (c < n16 && pos[j] >= 0) v[u][j] = ld16_nt(y + (int64_t)pos[j] * n16 + c);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int c = c0 + 64 * u;
            if (c >= n16) break;
            float fo[EPV];
            load_f32<BF16>(vo[u], fo);
#pragma unroll
            for (int j = 0; j < KMAX; j++) {
                if (pos[j] < 0) continue;
                float fy[EPV], fd[EPV];
                load_f32<BF16>(v[u][j], fy);
#pragma unroll
                for (int i = 0; i < EPV; i++) {
                    dot[j] = fmaf(fo[i], fy[i], dot[j]);
                    fd[i] = g[j] * fo[i];
                }
                if constexpr (DY) dy[(int64_t)pos[j] * n16 + c] = store_f32<BF16>(fd);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < KMAX; j++) {
        dot[j] = wave_sum(dot[j]);
        if (pos[j] < 0) dot[j] = 0.f;   // dropped row: its gate had no effect
    }
    float rg[KMAX];                      // router gradient of slot j
#pragma unroll
    for (int j = 0; j < KMAX; j++) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < KMAX; i++) s = fmaf(g[i], dot[j] - dot[i], s);
        rg[j] = g[j] * s;
    }
    for (int e = lane; e < E; e += 64) {
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < KMAX; j++)
            if (ex[j] == e) v = rg[j];
        dlogits[t * E + e] = v;
    }
    if (dgate && lane == 0) {
#pragma unroll
        for (int j = 0; j < KMAX; j++)
            if (j < k) dgate[t * k + j] = dot[j];
    }
    if (!DY && lane == 0) {
        float *row_gate = reinterpret_cast<float *>(dy);
#pragma unroll
        for (int j = 0; j < KMAX; j++)
            if (pos[j] >= 0) row_gate[pos[j]] = g[j];
    }
}

// ---------------------------------------------------------------------------
// launchers

#define MOE_KSWITCH(k, F) \
    ((k) <= 1 ? F(1) : (k) <= 2 ? F(2) : (k) <= 4 ? F(4) : F(8))

moe_status permute_launch(const void *x, const uint8_t *x_scale, moe_dtype dt, int64_t T, int d,
                          int k, const int32_t *token_pos, void *x_perm, uint8_t *x_perm_scale,
                          hipStream_t s) {
    if (T == 0) return MOE_OK;
    const int esize = dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 2 : 1;
    const int n16 = (int)((int64_t)d * esize / 16);
    const unsigned nb = (unsigned)((T + kRowWaves - 1) / kRowWaves);
#define L(K)                                                                                  \
    (permute_rows16<K><<<nb, 256, 0, s>>>(reinterpret_cast<const uint4 *>(x), T, n16, k,     \
                                          token_pos, reinterpret_cast<uint4 *>(x_perm)), 0)
    MOE_KSWITCH(k, L);
#undef L
    if (dt == MOE_MXFP8)
        permute_rows_bytes<<<nb, 256, 0, s>>>(x_scale, T, d / 32, k, token_pos, x_perm_scale);
    return launch_status();
}

moe_status combine_launch(const void *y, moe_dtype dt, const float *gate,
                          const int32_t *token_pos, int64_t T, int d, int k, void *out,
                          bool unit_gate, hipStream_t s) {
    if (T == 0) return MOE_OK;
    const bool bf = dt == MOE_BF16;
    const int n16 = d * (bf ? 2 : 4) / 16;
    const unsigned nb = (unsigned)((T + kRowWaves - 1) / kRowWaves);
    const uint4 *yy = reinterpret_cast<const uint4 *>(y);
    uint4 *oo = reinterpret_cast<uint4 *>(out);
#define L(K)                                                                                      \
    (bf ? (unit_gate ? (combine_rows<true, true, K><<<nb, 256, 0, s>>>(yy, gate, token_pos, T, n16, k, oo), 0) \
                     : (combine_rows<true, false, K><<<nb, 256, 0, s>>>(yy, gate, token_pos, T, n16, k, oo), 0)) \
        : (unit_gate ? (combine_rows<false, true, K><<<nb, 256, 0, s>>>(yy, gate, token_pos, T, n16, k, oo), 0) \
                     : (combine_rows<false, false, K><<<nb, 256, 0, s>>>(yy, gate, token_pos, T, n16, k, oo), 0)))
    MOE_KSWITCH(k, L);
#undef L
    return launch_status();
}

// row_gate_only (bf16): dy receives the gate of each routed row (fp32, T*k
// entries) instead of the dy rows.
moe_status combine_bwd_launch(const void *dout, const void *y, moe_dtype dt, const float *gate,
                              const int32_t *topk_idx, const int32_t *token_pos, int64_t T,
                              int d, int k, int E, void *dy, float *dlogits, float *dgate,
                              hipStream_t s, bool row_gate_only) {
    if (T == 0) return MOE_OK;
    const bool bf = dt == MOE_BF16;
    if (row_gate_only && !bf) return MOE_ERR_DTYPE;
    const int n16 = d * (bf ? 2 : 4) / 16;
    const unsigned nb = (unsigned)((T + kRowWaves - 1) / kRowWaves);
    const uint4 *dd = reinterpret_cast<const uint4 *>(dout);
    const uint4 *yy = reinterpret_cast<const uint4 *>(y);
    uint4 *oo = reinterpret_cast<uint4 *>(dy);
#define L(K)                                                                                        \
    (row_gate_only ? (combine_bwd_rows<true, K, false><<<nb, 256, 0, s>>>(dd, yy, gate, topk_idx,  \
                                                        token_pos, T, n16, k, E, oo, dlogits, dgate), 0) \
    : bf ? (combine_bwd_rows<true, K><<<nb, 256, 0, s>>>(dd, yy, gate, topk_idx, token_pos, T, n16, \
                                                        k, E, oo, dlogits, dgate), 0)               \
        : (combine_bwd_rows<false, K><<<nb, 256, 0, s>>>(dd, yy, gate, topk_idx, token_pos, T,   \
                                                         n16, k, E, oo, dlogits, dgate), 0))
    MOE_KSWITCH(k, L);
#undef L
    return launch_status();
}

}  // namespace moe
