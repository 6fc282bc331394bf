// copy_plan.h -- where the grouped GEMM's global -> LDS copies read from.
//
// The grouped GEMM (gemm.hip) stages its operands with 16-byte copies, one
// per lane and instruction, and the MXFP8 block scales with 4- or 16-byte
// copies. Every source address is an operand base plus offsets computed by
// the functions below, which compile for the host as well as the device:
// the kernels call them to set up their copies, and moe_gemm_copy_walk
// (walk.hip) calls the same functions on the host to walk every copy a
// launch would issue and bound it against the operand's extent.
#pragma once

#include <stdint.h>

#include "moe.h"

#define MOE_HD __host__ __device__ __forceinline__

namespace moe {

// Each pipeline step covers 128 bytes of K per row: 64 bf16 or 128 fp8.
constexpr int kStepBytes = 128;

struct GemmArgs {
    const void *A;
    const void *B;
    void *C;
    const void *aux;
    void *aux_out;
    const int32_t *offsets;
    const uint8_t *a_scale;   // MXFP8 E8M0 scales
    const uint8_t *b_scale;
    int64_t rows;
    int M, N, K;
    int E;
    int h;          // hidden width (SwiGLU epilogues)
    int accumulate; // WGRAD: add to C instead of overwriting it
    // MXFP8 SwiGLU forward with H' stored quantised (aux_out: its E4M3 rows)
    uint8_t *aux_out_scale;
    uint8_t *aux_out_cols;
    uint8_t *aux_out_cols_scale;
};

// K-layout LDS tile: [R rows][128 bytes]. LDS has 64 4-byte banks, i.e. two
// 128-byte rows per bank cycle; XOR-swizzling the 16-byte chunks with
// (row/2) % 8 puts the 16 rows that a ds_read_b128 serves per cycle on 16
// different 16-byte bank groups (measured: 2x the read rate of a row % 8
// swizzle, 7x that of no swizzle).
MOE_HD int kl_swz(int row) { return (row >> 1) & 7; }
MOE_HD int kl_chunk(int row, int kc) { return row * 8 + (kc ^ kl_swz(row)); }

MOE_HD int imin(int a, int b) { return a < b ? a : b; }

// Copy geometry of one operand tile per stage: every instruction writes 64
// lanes x 16 bytes to a contiguous 1 KiB of LDS, so each lane picks the
// global chunk that belongs at its LDS position. NW waves share the copy,
// IPW instructions each.
//
// KL = true : K-layout tile [R rows][128 bytes]; source rows are K-contiguous.
// KL = false: MN-layout tile [64 k][R cols] bf16; the source is [k][ld],
//             columns contiguous.
//
// Rows past the operand's end (KL) and columns past it (MN) are read from
// the last valid row / column instead: they meet only output rows or columns
// that the epilogue does not store. K past the reduction's end is different
// (it would add to valid outputs): a step that reaches past klim takes zeros
// for those chunks.
template <int R, bool KL, int NW>
struct CopyGeom {
    static constexpr int CHUNKS = R * 8;
    static constexpr int IPW = CHUNKS / 64 / NW;
    static constexpr int STEP = KL ? kStepBytes : 64;   // K per step: bytes (KL) or rows (MN)
    static_assert(IPW >= 1 && CHUNKS % (64 * NW) == 0, "tile/wave mismatch");
    static_assert(KL || R >= 128, "MN-layout swizzle needs >= 16 chunks per row");

    // chunk position of lane `lane`'s instruction i: (row, 16-byte column)
    MOE_HD static int pos(int i, int wave, int lane) { return (wave * IPW + i) * 64 + lane; }
    // the chunk's K position: byte offset in the step (KL) or k row (MN)
    MOE_HD static int kpos(int i, int wave, int lane) {
        const int p = pos(i, wave, lane);
        if constexpr (KL) return ((p & 7) ^ kl_swz(p >> 3)) * 16;
        else return p / (R / 8);
    }
    // KL: byte offset of the chunk from the tile origin at step 0, given
    // row_off(r) = byte offset of tile row r's K run (< 2^32)
    template <typename RowFn>
    MOE_HD static uint32_t kl_off(int i, int wave, int lane, RowFn row_off) {
        const int p = pos(i, wave, lane);
        const int row = p >> 3, kc = (p & 7) ^ kl_swz(row);
        return row_off(row) + (uint32_t)(kc * 16);
    }
    // MN: the same for a tile whose element (k = 0, col 0) is the origin, ld =
    // row pitch in bytes, cvalid = valid columns (>= 1)
    MOE_HD static uint32_t mn_off(int i, int wave, int lane, int64_t ld, int cvalid) {
        const int p = pos(i, wave, lane);
        const int k = p / (R / 8), c = (p % (R / 8)) ^ ((k & 3) << 2);
        const int cs = c * 8 < cvalid ? c : (cvalid - 1) >> 3;
        return (uint32_t)(k * ld + cs * 16);
    }
    // bytes the tile origin advances per step
    MOE_HD static int64_t kstride(int64_t ld) { return KL ? (int64_t)kStepBytes : 64 * ld; }
    // whether instruction i of step kt copies real data (else the zero chunk)
    MOE_HD static bool in_k(int i, int wave, int lane, int kt, int klim) {
        const int k0 = kt * STEP;
        return k0 + STEP <= klim || k0 + kpos(i, wave, lane) < klim;
    }
};

// Byte offsets of the stores of the MXFP8 SwiGLU forward that writes H'
// quantised (used by the kernel's epilogue and by the host walk of those
// stores, moe_gemm_hp_store_walk). A consumer wave holds rows r0 .. r0+63 and
// hidden units j0 .. j0+31; lane = 32 half + 4 qd + rq, column c = j0 + lane % 32.
// The group's column-block layout covers blocks [bb, bb + nb) (bb = 4 x the
// group's first 128-row unit, nb = 4 x its units), one nb*32-byte run per
// hidden unit; lr is a row within the group.
struct HpStores {
    // 16 bytes of column c, rows lr + 16 half .. + 15 of a 32-row block
    MOE_HD static int64_t col_q(int64_t bb, int64_t nb, int h, int c, int lr, int half) {
        return bb * 32 * h + (int64_t)c * nb * 32 + lr + half * 16;
    }
    // the scale byte of column c's 32-row block starting at lr
    MOE_HD static int64_t col_s(int64_t bb, int64_t nb, int h, int c, int lr) {
        return bb * h + (int64_t)c * nb + (lr >> 5);
    }
    // 4 bytes of routed row `row`, units j0 + 4 qd .. + 3
    MOE_HD static int64_t row_q(int64_t row, int h, int j0, int qd) {
        return row * h + j0 + 4 * qd;
    }
    // the scale byte of the row's block j0 / 32
    MOE_HD static int64_t row_s(int64_t row, int h, int j0) { return row * (h >> 5) + (j0 >> 5); }
};

// coordinates of one output tile
struct TileC {
    int e;        // group (expert)
    int row0;     // FWD/DGRAD: first routed row of the tile; WGRAD: the group's first row
    int row_end;  // FWD/DGRAD: one past the group's last row
    int m0, n0;   // WGRAD: first output row; first output column (B row / column)
    int nt;       // n-tile index
    int klim;     // K extent: bytes of K per A row (KL A), or rows (bf16 WGRAD)
    int kpad;     // MXFP8 WGRAD: the group's rows rounded up to 128 (bytes per row)
    int sb0;      // MXFP8 WGRAD: the group's first 128-row block in the column layout
};

// Per-tile copy sources of the grouped GEMM: MODE, epilogue, element type,
// tile size and the consumer-wave tile width WTN (the SwiGLU forward lays the
// B panel out per consumer wave). Offsets are in bytes from the operand's
// base pointer.
template <int MODE, int EPI, bool FP8, int BM, int BN, int WTN>
struct TilePlan {
    static constexpr bool A_KL = FP8 || MODE != MOE_GG_WGRAD;
    static constexpr bool B_KL = FP8 || MODE == MOE_GG_FWD;
    static constexpr int ESZ = FP8 ? 1 : 2;
    static constexpr int ASTEP = A_KL ? kStepBytes : 64;   // K per step of A: bytes, or rows

    MOE_HD static int nk_of(int klim) { return (klim + ASTEP - 1) / ASTEP; }
    // B's K extent in its own unit (bf16 DGRAD: A counts bytes, B rows)
    MOE_HD static int b_klim(int klim) { return (A_KL && !B_KL) ? klim / ESZ : klim; }

    // n-tiles across the output
    MOE_HD static int n_tiles(const GemmArgs &g) {
        return (MODE != MOE_GG_WGRAD && EPI == MOE_EPI_SWIGLU_FWD) ? (g.h + BN / 2 - 1) / (BN / 2)
                                                                 : (g.N + BN - 1) / BN;
    }
    // FWD/DGRAD: tile (group e, its m-tile mt_e, n-tile nt); off = offsets[0..E]
    MOE_HD static TileC row_tile(const GemmArgs &g, const int32_t *off, int e, int mt_e, int nt) {
        TileC t;
        t.e = e;
        t.row0 = off[e] + mt_e * BM;
        t.row_end = off[e + 1];
        t.m0 = 0;
        t.nt = nt;
        t.n0 = nt * BN;
        t.klim = g.K * ESZ;
        t.kpad = 0;
        t.sb0 = 0;
        return t;
    }
    // WGRAD: tile (group e, output m-tile mi, n-tile nt); blk[e] = sum over
    // e' < e of ceil(c_e' / 128) (MXFP8 only)
    MOE_HD static TileC wgrad_tile(const int32_t *off, const int32_t *blk, int e, int mi, int nt) {
        TileC t;
        t.e = e;
        t.row0 = off[e];
        t.row_end = 0;
        t.m0 = mi * BM;
        t.nt = nt;
        t.n0 = nt * BN;
        if constexpr (FP8) {
            t.sb0 = blk[e];
            t.kpad = (blk[e + 1] - t.sb0) * 128;
            t.klim = t.kpad;                       // bytes of K per row
        } else {
            t.sb0 = 0;
            t.kpad = 0;
            t.klim = off[e + 1] - t.row0;          // reduction over the group's rows
        }
        return t;
    }

    // B row (of B's N rows) of tile column n, clamped into range. SwiGLU
    // forward: each consumer wave's columns are gate rows, then the up rows
    // of the same hidden units.
    MOE_HD static int b_row_clamped(const GemmArgs &g, const TileC &t, int n) {
        if constexpr (MODE == MOE_GG_FWD && EPI == MOE_EPI_SWIGLU_FWD) {
            const int wc = n / WTN, off = n % WTN, half = WTN / 2;
            const int j = imin(t.nt * (BN / 2) + wc * half + (off % half), g.h - 1);
            return off < half ? j : g.h + j;
        } else {
            return imin(t.n0 + n, g.N - 1);
        }
    }
    // the same without the clamp: -1 for a column past the end
    MOE_HD static int b_row_index(const GemmArgs &g, const TileC &t, int n) {
        if constexpr (MODE == MOE_GG_FWD && EPI == MOE_EPI_SWIGLU_FWD) {
            const int wc = n / WTN, off = n % WTN, half = WTN / 2;
            const int j = t.nt * (BN / 2) + wc * half + (off % half);
            if (j >= g.h) return -1;
            return off < half ? j : g.h + j;
        } else {
            const int r = t.n0 + n;
            return r < g.N ? r : -1;
        }
    }

    // A tile origin, and its row offsets (K layout) or pitch and valid
    // columns (MN layout)
    MOE_HD static int64_t a_origin(const GemmArgs &g, const TileC &t) {
        if constexpr (MODE == MOE_GG_WGRAD) {
            // MXFP8 column-block layout: group e's A is [M][kpad] at byte sb0*128*M
            if constexpr (FP8) return (int64_t)t.sb0 * 128 * g.M + (int64_t)t.m0 * t.kpad;
            else return ((int64_t)t.row0 * g.M + t.m0) * 2;
        } else {
            return (int64_t)t.row0 * g.K * ESZ;
        }
    }
    // K layout: byte offset of tile row r's K run from the origin (rows past
    // the end read the last valid one); offsets stay below 2^32 (the host
    // bounds MXFP8 WGRAD to 2^24 rows)
    MOE_HD static uint32_t a_row_off(const GemmArgs &g, const TileC &t, int r) {
        if constexpr (MODE == MOE_GG_WGRAD) {
            return (uint32_t)imin(r, g.M - 1 - t.m0) * (uint32_t)t.kpad;
        } else {
            const int last = t.row_end - t.row0 - 1;   // a tile has at least one row
            return (uint32_t)imin(r, last) * (uint32_t)(g.K * ESZ);
        }
    }
    MOE_HD static int64_t a_ld(const GemmArgs &g) { return (int64_t)g.M * 2; }
    MOE_HD static int a_cvalid(const GemmArgs &g, const TileC &t) { return g.M - t.m0; }

    MOE_HD static int64_t b_origin(const GemmArgs &g, const TileC &t) {
        if constexpr (MODE == MOE_GG_WGRAD) {
            if constexpr (FP8) return (int64_t)t.sb0 * 128 * g.N + (int64_t)t.n0 * t.kpad;
            else return ((int64_t)t.row0 * g.N + t.n0) * 2;
        } else if constexpr (B_KL) {
            return (int64_t)t.e * g.N * g.K * ESZ;
        } else {
            return ((int64_t)t.e * g.K * g.N + t.n0) * 2;
        }
    }
    MOE_HD static uint32_t b_row_off(const GemmArgs &g, const TileC &t, int n) {
        if constexpr (MODE == MOE_GG_WGRAD) {
            return (uint32_t)imin(n, g.N - 1 - t.n0) * (uint32_t)t.kpad;
        } else {
            return (uint32_t)b_row_clamped(g, t, n) * (uint32_t)(g.K * ESZ);
        }
    }
    MOE_HD static int64_t b_ld(const GemmArgs &g) { return (int64_t)g.N * 2; }
    MOE_HD static int b_cvalid(const GemmArgs &g, const TileC &t) { return g.N - t.n0; }

    // MXFP8: the E8M0 bytes of the stage's scale row sr ([A rows | B rows])
    // for step 0, as (operand 0 = A scales / 1 = B scales, byte offset); -1
    // for a row that has none (those copy zeros). One byte per 32 K elements,
    // so step kt's 4 bytes start at offset + 4 kt.
    MOE_HD static int scale_operand(int sr) { return sr < BM ? 0 : (sr < BM + BN ? 1 : -1); }
    MOE_HD static int64_t scale_off(const GemmArgs &g, const TileC &t, int sr) {
        if constexpr (MODE == MOE_GG_WGRAD) {
            const int nbk = t.kpad / 32;           // scale blocks per row of the group
            if (sr < BM) {
                const int m = t.m0 + sr;
                return m < g.M ? (int64_t)t.sb0 * 4 * g.M + (int64_t)m * nbk : -1;
            }
            if (sr < BM + BN) {
                const int c = t.n0 + sr - BM;
                return c < g.N ? (int64_t)t.sb0 * 4 * g.N + (int64_t)c * nbk : -1;
            }
            return -1;
        } else {
            const int nbk = g.K / 32;
            if (sr < BM) {
                const int gr = t.row0 + sr;
                return gr < t.row_end ? (int64_t)gr * nbk : -1;
            }
            if (sr < BM + BN) {
                const int br = b_row_index(g, t, sr - BM);
                return br >= 0 ? ((int64_t)t.e * g.N + br) * nbk : -1;
            }
            return -1;
        }
    }
    // MXFP8: scales copied 16 bytes per row every 4th step (FWD/DGRAD when
    // every row's scales come in whole 16-byte groups; WGRAD always -- the
    // column-block scale array is sized by mxfp8_col_blocks, whose spare
    // blocks keep a 16-byte read past the end of a column's last, partial
    // group in bounds), else 4 bytes per step
    MOE_HD static bool scale_batched(const GemmArgs &g) {
        return FP8 && (MODE == MOE_GG_WGRAD || (g.K / 32) % 16 == 0);
    }
};

}  // namespace moe
