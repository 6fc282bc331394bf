// gemm.hip -- device-scheduled grouped GEMM for the expert FFNs.
//
// The pages' grouped GEMM runs the uneven per-expert shapes produced by
// routing in one kernel and is scheduled on the device, so experts are never
// padded to one capacity and the host never learns the group sizes
// (kongchang.com, "routing is a systems problem"; bytechap.com, "How it
// works": small matmuls merged into larger batches).
//
// Design for gfx950:
//  * persistent grid (a fixed number of workgroups per CU). Each workgroup
//    reads the group offsets from device memory into LDS, scans ceil(c_e/BM)
//    into a tile table, and walks tile ids t = blockIdx.x, += gridDim.x. A
//    tile id maps to (m-tile, n-tile) with the n-tile fastest; with a grid
//    that is a multiple of 8, tile t runs on XCD t % 8, so a given weight
//    panel (expert, n-tile) is always read by the same XCD and reused from
//    that XCD's L2 across the expert's m-tiles.
//  * bf16 MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulators; each wave owns a
//    (BM/WM) x (BN/WN) block of 32x32 MFMA tiles.
//  * both operands are staged into LDS K-contiguous ([rows][64] bf16, 16-byte
//    chunks XOR-swizzled by row) so every MFMA operand fetch is one
//    ds_read_b128. Operands that are K-contiguous in HBM (activations in
//    FWD/DGRAD, weights in FWD) are copied chunk by chunk; operands that are
//    M/N-contiguous (weights in DGRAD, both operands of WGRAD) are loaded as
//    8x8 bf16 blocks with coalesced 16-byte loads and transposed in registers.
//  * double-buffered LDS with a register prefetch of the next K block: one
//    barrier per K step.
//  * epilogues: plain store; SwiGLU forward (the weight panel is laid out so
//    each wave holds the gate and up columns of the same hidden unit in the
//    same registers, so H' = silu(a) * b is formed from the fp32
//    accumulators); SwiGLU backward (reads the stored a, b).
#include <type_traits>

#include "common.h"

namespace moe {

struct GemmArgs {
    const void *A;
    const void *B;
    void *C;
    const void *aux;
    void *aux_out;
    const int32_t *offsets;
    int64_t rows;
    int M, N, K;
    int E;
    int h;          // hidden width (SwiGLU epilogues)
};

// ---------------------------------------------------------------------------
// tile table shared by the kernels

// Loads offsets[0..E] into s_off and builds s_tile[e] = sum_{e'<e} ceil(c_e'/BM).
// Needs blockDim.x >= 256 (E <= 256). Returns the total number of m-tiles.
MOE_DEV int build_tile_table(const int32_t *offsets, int E, int BM, int32_t *s_off,
                             int32_t *s_tile) {
    const int tid = threadIdx.x;
    if (tid <= E) s_off[tid] = offsets[tid];
    __syncthreads();
    int32_t c = tid < E ? (s_off[tid + 1] - s_off[tid] + BM - 1) / BM : 0;
    if (tid < 256) s_tile[tid + 1] = c;
    if (tid == 0) s_tile[0] = 0;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        int32_t v = (tid < 256 && tid >= o) ? s_tile[tid + 1 - o] : 0;
        __syncthreads();
        if (tid < 256) s_tile[tid + 1] += v;
        __syncthreads();
    }
    return s_tile[E];
}

// group of a global m-tile: largest e with s_tile[e] <= mt
MOE_DEV int find_group(const int32_t *s_tile, int E, int mt) {
    int lo = 0, hi = E;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (s_tile[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    return lo;
}

MOE_DEV float silu_f(float a) { return a / (1.f + __expf(-a)); }

// ---------------------------------------------------------------------------
// bf16 MFMA kernel

constexpr int kBK = 64;

MOE_DEV int swz(int row, int kc) { return row * 8 + (kc ^ (row & 7)); }

// K-contiguous operand tile [R rows][64 k] -> registers. row_ptr(r) gives the
// address of the row's element k=0 (or null when the row is out of range).
template <int R, int NT>
struct KcStage {
    static constexpr int CH = R * 8 / NT;
    static_assert(CH >= 1 && R * 8 % NT == 0, "tile/thread mismatch");
    uint4 v[CH];
    template <typename RowFn>
    MOE_DEV void load(RowFn row_ptr, int k0, int K) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < CH; i++) {
            const int id = tid + i * NT, row = id >> 3, kc = id & 7;
            const uint16_t *p = row_ptr(row);
            const int kk = k0 + kc * 8;
            if (p != nullptr && kk < K)
                v[i] = *reinterpret_cast<const uint4 *>(p + kk);
            else
                v[i] = make_uint4(0, 0, 0, 0);
        }
    }
    MOE_DEV void store(uint4 *lds) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < CH; i++) {
            const int id = tid + i * NT, row = id >> 3, kc = id & 7;
            lds[swz(row, kc)] = v[i];
        }
    }
};

// M/N-contiguous operand: global [k][ld] with the tile's R columns contiguous.
// Each working thread loads an 8(k) x 8(col) block and transposes it.
template <int R, int NT>
struct McStage {
    static constexpr int NBLK = R;                       // (64/8) * (R/8)
    static constexpr int PER = (NBLK + NT - 1) / NT;
    uint4 v[PER][8];
    // base: pointer to element (k=0 of the tile, col=0 of the tile);
    // ld: row pitch in elements; kvalid: rows [0, kvalid) are valid;
    // cvalid: columns [0, cvalid) are valid (multiple of 8).
    MOE_DEV void load(const uint16_t *base, int64_t ld, int k0, int kvalid, int cvalid) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int b = tid + i * NT;
            const int mb = b % (R / 8), kb = b / (R / 8);
            const bool okc = (b < NBLK) && (mb * 8 < cvalid);
#pragma unroll
            for (int ii = 0; ii < 8; ii++) {
                const int kr = k0 + kb * 8 + ii;
                if (okc && kr < kvalid)
                    v[i][ii] = *reinterpret_cast<const uint4 *>(base + (int64_t)kr * ld + mb * 8);
                else
                    v[i][ii] = make_uint4(0, 0, 0, 0);
            }
        }
    }
    MOE_DEV void store(uint4 *lds) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int b = tid + i * NT;
            if (b >= NBLK) continue;
            const int mb = b % (R / 8), kb = b / (R / 8);
            const uint32_t *w = reinterpret_cast<const uint32_t *>(v[i]);   // w[ii*4 + c]
#pragma unroll
            for (int c = 0; c < 4; c++) {
                uint4 lo, hi;   // columns 2c and 2c+1, eight k values each
                uint32_t *l = reinterpret_cast<uint32_t *>(&lo);
                uint32_t *hh = reinterpret_cast<uint32_t *>(&hi);
#pragma unroll
                for (int p = 0; p < 4; p++) {
                    const uint32_t a = w[(2 * p) * 4 + c], bq = w[(2 * p + 1) * 4 + c];
                    l[p] = (a & 0xffffu) | (bq << 16);
                    hh[p] = (a >> 16) | (bq & 0xffff0000u);
                }
                const int r0 = mb * 8 + 2 * c;
                lds[swz(r0, kb)] = lo;
                lds[swz(r0 + 1, kb)] = hi;
            }
        }
    }
};

template <int MODE, int EPI, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM *WN * 64) void gg_bf16(GemmArgs g) {
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM >= 1 && TN >= 1, "wave tile");
    static_assert(EPI != MOE_EPI_SWIGLU_FWD || TN % 2 == 0, "SwiGLU pairs gate/up sub-tiles");
    constexpr bool A_KC = MODE != MOE_GG_WGRAD;
    constexpr bool B_KC = MODE == MOE_GG_FWD;

    __shared__ __attribute__((aligned(16))) uint4 lds_a[2][BM * 8];
    __shared__ __attribute__((aligned(16))) uint4 lds_b[2][BN * 8];
    __shared__ int32_t s_off[257];
    __shared__ int32_t s_tile[257];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int E = g.E;

    int n_tiles, total;
    if constexpr (MODE == MOE_GG_WGRAD) {
        if (tid <= E) s_off[tid] = g.offsets[tid];
        __syncthreads();
        n_tiles = (g.N + BN - 1) / BN;
        total = E * ((g.M + BM - 1) / BM) * n_tiles;
    } else {
        const int mt = build_tile_table(g.offsets, E, BM, s_off, s_tile);
        n_tiles = (EPI == MOE_EPI_SWIGLU_FWD) ? (g.h + BN / 2 - 1) / (BN / 2)
                                              : (g.N + BN - 1) / BN;
        total = mt * n_tiles;
    }

    const uint16_t *A = reinterpret_cast<const uint16_t *>(g.A);
    const uint16_t *B = reinterpret_cast<const uint16_t *>(g.B);

    using AStageT = typename std::conditional<A_KC, KcStage<BM, NT>, McStage<BM, NT>>::type;
    using BStageT = typename std::conditional<B_KC, KcStage<BN, NT>, McStage<BN, NT>>::type;

    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        // ---- decode the tile
        int e, row0 = 0, row_end = 0, m0 = 0, n0, nt, klen;
        if constexpr (MODE == MOE_GG_WGRAD) {
            const int mtiles = (g.M + BM - 1) / BM;
            nt = tile % n_tiles;
            const int rest = tile / n_tiles;
            const int mtl = rest % mtiles;
            e = rest / mtiles;
            m0 = mtl * BM;
            row0 = s_off[e];
            klen = s_off[e + 1] - row0;     // reduction over the group's rows
        } else {
            nt = tile % n_tiles;
            const int mt = tile / n_tiles;
            e = find_group(s_tile, E, mt);
            row0 = s_off[e] + (mt - s_tile[e]) * BM;
            row_end = s_off[e + 1];
            klen = g.K;
        }
        n0 = nt * BN;

        // ---- operand row pointers
        auto a_row = [&](int r) -> const uint16_t * {
            const int gr = row0 + r;
            return gr < row_end ? A + (int64_t)gr * g.K : nullptr;
        };
        auto b_row = [&](int n) -> const uint16_t * {
            // FWD: B[e] is [N, K]; SwiGLU lays the panel out per wave as
            // [gate rows | up rows] of the same hidden units
            int wrow;
            if constexpr (EPI == MOE_EPI_SWIGLU_FWD) {
                const int wc = n / WTN, off = n % WTN, half = WTN / 2;
                const int j = nt * (BN / 2) + wc * half + (off % half);
                if (j >= g.h) return nullptr;
                wrow = off < half ? j : g.h + j;
            } else {
                wrow = n0 + n;
                if (wrow >= g.N) return nullptr;
            }
            return B + ((int64_t)e * g.N + wrow) * g.K;
        };

        AStageT sa;
        BStageT sb;
        auto load_stage = [&](int k0) {
            if constexpr (A_KC) sa.load(a_row, k0, klen);
            else sa.load(A + (int64_t)row0 * g.M + m0, g.M, k0, klen, g.M - m0);
            if constexpr (MODE == MOE_GG_FWD) sb.load(b_row, k0, klen);
            else if constexpr (MODE == MOE_GG_DGRAD)
                sb.load(B + (int64_t)e * g.K * g.N + n0, g.N, k0, klen, g.N - n0);
            else sb.load(B + (int64_t)row0 * g.N + n0, g.N, k0, klen, g.N - n0);
        };

        f32x16 acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++)
#pragma unroll
                for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

        const int nk = (klen + kBK - 1) / kBK;
        if (nk > 0) {
            load_stage(0);
            sa.store(lds_a[0]);
            sb.store(lds_b[0]);
            __syncthreads();
        }
        for (int kt = 0; kt < nk; kt++) {
            const int cur = kt & 1;
            if (kt + 1 < nk) load_stage((kt + 1) * kBK);
            const uint4 *la = lds_a[cur];
            const uint4 *lb = lds_b[cur];
#pragma unroll
            for (int kk = 0; kk < kBK / 16; kk++) {
                const int kc = kk * 2 + (lane >> 5);
                bf16x8 fa[TM], fb[TN];
#pragma unroll
                for (int i = 0; i < TM; i++) {
                    const int r = wm * WTM + i * 32 + (lane & 31);
                    uint4 u = la[swz(r, kc)];
                    fa[i] = __builtin_bit_cast(bf16x8, u);
                }
#pragma unroll
                for (int j = 0; j < TN; j++) {
                    const int r = wn * WTN + j * 32 + (lane & 31);
                    uint4 u = lb[swz(r, kc)];
                    fb[j] = __builtin_bit_cast(bf16x8, u);
                }
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int j = 0; j < TN; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
            }
            if (kt + 1 < nk) {
                sa.store(lds_a[cur ^ 1]);
                sb.store(lds_b[cur ^ 1]);
            }
            __syncthreads();
        }

        // ---- epilogue. acc[i][j][v] holds row (v/4)*8 + (lane/32)*4 + v%4 and
        // column lane%32 of the wave's (i, j) 32x32 tile.
        const int col_l = lane & 31;
        if constexpr (MODE == MOE_GG_WGRAD) {
            float *C = reinterpret_cast<float *>(g.C) + (int64_t)e * g.M * g.N;
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++) {
                    const int n = n0 + wn * WTN + j * 32 + col_l;
                    if (n >= g.N) continue;
#pragma unroll
                    for (int v = 0; v < 16; v++) {
                        const int m = m0 + wm * WTM + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
                        if (m < g.M) C[(int64_t)m * g.N + n] = acc[i][j][v];
                    }
                }
        } else if constexpr (EPI == MOE_EPI_SWIGLU_FWD) {
            uint16_t *AB = reinterpret_cast<uint16_t *>(g.C);
            uint16_t *HP = reinterpret_cast<uint16_t *>(g.aux_out);
            const int h = g.h;
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN / 2; j++) {
                    const int jj = nt * (BN / 2) + wn * (WTN / 2) + j * 32 + col_l;
                    if (jj >= h) continue;
#pragma unroll
                    for (int v = 0; v < 16; v++) {
                        const int r = row0 + wm * WTM + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
                        if (r >= row_end) continue;
                        const float a = acc[i][j][v], b = acc[i][j + TN / 2][v];
                        AB[(int64_t)r * 2 * h + jj] = f32_to_bf16(a);
                        AB[(int64_t)r * 2 * h + h + jj] = f32_to_bf16(b);
                        HP[(int64_t)r * h + jj] = f32_to_bf16(silu_f(a) * b);
                    }
                }
        } else if constexpr (EPI == MOE_EPI_SWIGLU_BWD) {
            const uint16_t *AB = reinterpret_cast<const uint16_t *>(g.aux);
            uint16_t *dAB = reinterpret_cast<uint16_t *>(g.C);
            const int h = g.h;
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++) {
                    const int jj = n0 + wn * WTN + j * 32 + col_l;
                    if (jj >= h) continue;
#pragma unroll
                    for (int v = 0; v < 16; v++) {
                        const int r = row0 + wm * WTM + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
                        if (r >= row_end) continue;
                        const float a = bf16_to_f32(AB[(int64_t)r * 2 * h + jj]);
                        const float b = bf16_to_f32(AB[(int64_t)r * 2 * h + h + jj]);
                        const float dh = acc[i][j][v];
                        const float s = 1.f / (1.f + __expf(-a));
                        dAB[(int64_t)r * 2 * h + jj] = f32_to_bf16(dh * b * s * (1.f + a * (1.f - s)));
                        dAB[(int64_t)r * 2 * h + h + jj] = f32_to_bf16(dh * a * s);
                    }
                }
        } else {
            uint16_t *C = reinterpret_cast<uint16_t *>(g.C);
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++) {
                    const int n = n0 + wn * WTN + j * 32 + col_l;
                    if (n >= g.N) continue;
#pragma unroll
                    for (int v = 0; v < 16; v++) {
                        const int r = row0 + wm * WTM + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
                        if (r < row_end) C[(int64_t)r * g.N + n] = f32_to_bf16(acc[i][j][v]);
                    }
                }
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 kernel (correctness dtype): 64x64 tiles, 256 threads, 4x4 outputs per
// thread, fp32 FMA. A thread owns rows 4*ty..4*ty+3 and columns
// {2tx, 2tx+1, 32+2tx, 32+2tx+1}, so in the SwiGLU forward layout (tile
// columns 0..31 = gate, 32..63 = up of the same hidden units) it holds both
// halves of each pair.

template <int MODE, int EPI>
__global__ __launch_bounds__(256) void gg_f32(GemmArgs g) {
    constexpr int BM = 64, BN = 64, BKF = 16;
    __shared__ float As[BKF][BM + 1];
    __shared__ float Bs[BKF][BN + 1];
    __shared__ int32_t s_off[257];
    __shared__ int32_t s_tile[257];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int E = g.E;
    const float *A = reinterpret_cast<const float *>(g.A);
    const float *B = reinterpret_cast<const float *>(g.B);

    int n_tiles, total;
    if constexpr (MODE == MOE_GG_WGRAD) {
        if (tid <= E) s_off[tid] = g.offsets[tid];
        __syncthreads();
        n_tiles = (g.N + BN - 1) / BN;
        total = E * ((g.M + BM - 1) / BM) * n_tiles;
    } else {
        const int mt = build_tile_table(g.offsets, E, BM, s_off, s_tile);
        n_tiles = (EPI == MOE_EPI_SWIGLU_FWD) ? (g.h + 31) / 32 : (g.N + BN - 1) / BN;
        total = mt * n_tiles;
    }
    int cols[4] = {2 * tx, 2 * tx + 1, 32 + 2 * tx, 33 + 2 * tx};

    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        int e, row0, row_end = 0, m0 = 0, nt, klen;
        nt = tile % n_tiles;
        if constexpr (MODE == MOE_GG_WGRAD) {
            const int mtiles = (g.M + BM - 1) / BM;
            const int rest = tile / n_tiles;
            m0 = (rest % mtiles) * BM;
            e = rest / mtiles;
            row0 = s_off[e];
            klen = s_off[e + 1] - row0;
        } else {
            const int mt = tile / n_tiles;
            e = find_group(s_tile, E, mt);
            row0 = s_off[e] + (mt - s_tile[e]) * BM;
            row_end = s_off[e + 1];
            klen = g.K;
        }
        const int n0 = nt * BN;
        // column index (in B's N space) of tile column c; -1 if out of range
        auto bcol = [&](int c) -> int {
            if constexpr (EPI == MOE_EPI_SWIGLU_FWD) {
                const int j = nt * 32 + (c & 31);
                if (j >= g.h) return -1;
                return c < 32 ? j : g.h + j;
            } else {
                const int n = n0 + c;
                return n < g.N ? n : -1;
            }
        };
        float acc[4][4] = {};
        for (int k0 = 0; k0 < klen; k0 += BKF) {
            for (int i = tid; i < BKF * BM; i += 256) {
                const int kk = i % BKF, m = i / BKF;   // A tile element (m, kk)
                const int k = k0 + kk;
                float va = 0.f;
                if constexpr (MODE == MOE_GG_WGRAD) {
                    if (k < klen && m0 + m < g.M) va = A[(int64_t)(row0 + k) * g.M + m0 + m];
                } else {
                    if (k < klen && row0 + m < row_end) va = A[(int64_t)(row0 + m) * g.K + k];
                }
                As[kk][m] = va;
                const int c = m;                         // B tile element (c, kk)
                float vb = 0.f;
                const int bc = bcol(c);
                if (k < klen && bc >= 0) {
                    if constexpr (MODE == MOE_GG_FWD) vb = B[((int64_t)e * g.N + bc) * g.K + k];
                    else if constexpr (MODE == MOE_GG_DGRAD) vb = B[((int64_t)e * g.K + k) * g.N + bc];
                    else vb = B[(int64_t)(row0 + k) * g.N + bc];
                }
                Bs[kk][c] = vb;
            }
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < BKF; kk++) {
                float a[4], b[4];
#pragma unroll
                for (int i = 0; i < 4; i++) a[i] = As[kk][ty * 4 + i];
#pragma unroll
                for (int j = 0; j < 4; j++) b[j] = Bs[kk][cols[j]];
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int j = 0; j < 4; j++) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
            }
            __syncthreads();
        }
        // epilogue
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int ml = ty * 4 + i;
            if constexpr (MODE == MOE_GG_WGRAD) {
                if (m0 + ml >= g.M) continue;
                float *C = reinterpret_cast<float *>(g.C) + ((int64_t)e * g.M + m0 + ml) * g.N;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int bc = bcol(cols[j]);
                    if (bc >= 0) C[bc] = acc[i][j];
                }
            } else {
                const int r = row0 + ml;
                if (r >= row_end) continue;
                if constexpr (EPI == MOE_EPI_SWIGLU_FWD) {
                    float *AB = reinterpret_cast<float *>(g.C) + (int64_t)r * 2 * g.h;
                    float *HP = reinterpret_cast<float *>(g.aux_out) + (int64_t)r * g.h;
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        const int jj = nt * 32 + cols[j];
                        if (jj >= g.h) continue;
                        const float a = acc[i][j], b = acc[i][j + 2];
                        AB[jj] = a;
                        AB[g.h + jj] = b;
                        HP[jj] = silu_f(a) * b;
                    }
                } else if constexpr (EPI == MOE_EPI_SWIGLU_BWD) {
                    const float *ABr = reinterpret_cast<const float *>(g.aux) + (int64_t)r * 2 * g.h;
                    float *dAB = reinterpret_cast<float *>(g.C) + (int64_t)r * 2 * g.h;
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const int jj = bcol(cols[j]);
                        if (jj < 0) continue;
                        const float a = ABr[jj], b = ABr[g.h + jj], dh = acc[i][j];
                        const float s = 1.f / (1.f + expf(-a));
                        dAB[jj] = dh * b * s * (1.f + a * (1.f - s));
                        dAB[g.h + jj] = dh * a * s;
                    }
                } else {
                    float *C = reinterpret_cast<float *>(g.C) + (int64_t)r * g.N;
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const int bc = bcol(cols[j]);
                        if (bc >= 0) C[bc] = acc[i][j];
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// launch

template <int MODE, int EPI>
static void launch_bf16(const GemmArgs &a, hipStream_t s) {
    constexpr int BM = 128, BN = 128, WM = 2, WN = 2;
    const int grid = num_cus() * 2;
    gg_bf16<MODE, EPI, BM, BN, WM, WN><<<grid, WM * WN * 64, 0, s>>>(a);
}

template <int MODE, int EPI>
static void launch_f32(const GemmArgs &a, hipStream_t s) {
    const int grid = num_cus() * 4;
    gg_f32<MODE, EPI><<<grid, 256, 0, s>>>(a);
}

moe_status gemm_launch(const moe_gemm_desc *d, hipStream_t s) {
    GemmArgs a;
    a.A = d->A; a.B = d->B; a.C = d->C; a.aux = d->aux; a.aux_out = d->aux_out;
    a.offsets = d->offsets; a.rows = d->rows; a.M = d->M; a.N = d->N; a.K = d->K;
    a.E = d->n_groups;
    a.h = d->epilogue == MOE_EPI_SWIGLU_FWD ? d->N / 2 : d->N;
    const bool bf = d->dtype == MOE_BF16;
#define GO(MODE, EPI) (bf ? launch_bf16<MODE, EPI>(a, s) : launch_f32<MODE, EPI>(a, s))
    if (d->mode == MOE_GG_FWD) {
        if (d->epilogue == MOE_EPI_SWIGLU_FWD) GO(MOE_GG_FWD, MOE_EPI_SWIGLU_FWD);
        else GO(MOE_GG_FWD, MOE_EPI_NONE);
    } else if (d->mode == MOE_GG_DGRAD) {
        if (d->epilogue == MOE_EPI_SWIGLU_BWD) GO(MOE_GG_DGRAD, MOE_EPI_SWIGLU_BWD);
        else GO(MOE_GG_DGRAD, MOE_EPI_NONE);
    } else {
        GO(MOE_GG_WGRAD, MOE_EPI_NONE);
    }
#undef GO
    return launch_status();
}

}  // namespace moe
