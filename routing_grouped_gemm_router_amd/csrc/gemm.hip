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
//    into a tile table, and walks an XCD-aware tile list (below): a weight
//    panel (expert, n-tile) is read by one XCD and reused from that XCD's L2
//    across the expert's m-tiles.
//  * bf16 MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulators; each wave owns a
//    (BM/WM) x (BN/WN) block of 32x32 MFMA tiles.
//  * operands reach LDS by direct global -> LDS copies (global_load_lds_dwordx4)
//    through a 3-stage pipeline of 128-byte K steps, one workgroup barrier
//    per step. K-contiguous operands (activations in FWD/DGRAD, weights in
//    FWD, every MXFP8 operand) are staged [rows][128 bytes] with XOR-swizzled
//    16-byte chunks, so an MFMA operand is one ds_read_b128; M/N-contiguous
//    bf16 operands (weights in DGRAD, both operands of WGRAD) are staged as
//    they lie and read with the transposing ds_read_b64_tr_b16.
//  * epilogues: plain store; SwiGLU forward (the weight panel is laid out so
//    each wave holds the gate and up columns of the same hidden unit in the
//    same registers, so H' = silu(a) * b is formed from the fp32
//    accumulators); SwiGLU backward (reads the stored a, b). A wave tile
//    that lies wholly inside the output is stored without per-element
//    checks, from a scalar base and one 32-bit offset per lane.
//  * two kernels share the tiles, schedules, LDS layouts and MFMA order, so
//    they give the same bits: gg_ws (bf16 and MXFP8 FWD, DGRAD, WGRAD) splits
//    the workgroup into consumer waves (fragment reads, MFMAs, epilogue) and
//    producer waves (every global -> LDS copy), so the copies never wait on
//    the epilogue's stores and the producers run ahead across tiles;
//    gg_mfma (the SwiGLU backward, bf16 and MXFP8, whose epilogue stages dH'
//    in the stage buffers; every role with -DMOE_GG_MFMA_ALL=1) has every
//    wave do both.
//  * copy sources come from copy_plan.h, which moe_gemm_copy_walk also runs on
//    the host to bound every copy of a launch.
#include <type_traits>
#include <utility>
#include <vector>

#include "common.h"
#include "copy_plan.h"
#include "mx_encode.h"

namespace moe {

// ---------------------------------------------------------------------------
// tile table shared by the kernels

// Copies offsets[0..E] (E + 1 entries, up to 257) into LDS with a strided
// loop, so the copy is whole for any block size; ends with a barrier.
MOE_DEV void load_offsets(const int32_t *offsets, int E, int32_t *s_off) {
    for (int i = threadIdx.x; i <= E; i += blockDim.x) s_off[i] = offsets[i];
    __syncthreads();
}

// Loads offsets[0..E] into s_off and builds s_tile[e] = sum_{e'<e} ceil(c_e'/BM).
// The scan needs blockDim.x >= 256 (E <= 256). Returns the total number of m-tiles.
MOE_DEV int build_tile_table(const int32_t *offsets, int E, int BM, int32_t *s_off,
                             int32_t *s_tile) {
    const int tid = threadIdx.x;
    load_offsets(offsets, E, s_off);
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

// silu(a) = a * sigmoid(a), the sigmoid by the hardware reciprocal (1 ulp)
// instead of a correctly rounded divide: the SwiGLU epilogues' VALU work is
// exposed between tiles (GEMM2 dgrad + SwiGLU backward 6 % faster; the
// results differ from the divided form in a few bf16 roundings)
MOE_DEV float silu_f(float a) { return a * __builtin_amdgcn_rcpf(1.f + __expf(-a)); }

// ---------------------------------------------------------------------------
// XCD-aware tile schedule
//
// MI355X has 8 XCDs with a private L2 each, and consecutive workgroup ids go
// to consecutive XCDs. The persistent grid (a multiple of 8 workgroups) is
// therefore split per XCD: workgroup b serves XCD x = b % 8 as its (b / 8)-th
// worker. Each expert's m-tiles are cut into chunks of about kChunkM m-tiles
// (below); chunk c belongs to XCD c % 8, and an XCD walks its chunks' tiles in
// order with the m-tile fastest.
// The ~32 CUs of an XCD thus work on all m-tiles of one chunk and a few of its
// weight panels at a time: each weight panel is fetched into that XCD's L2
// once and shared by all of the chunk's m-tiles, and the chunk's activation
// rows are shared by the concurrent panels. (With the n-tile fastest, the
// concurrent tiles would touch every panel of the expert and stream the whole
// weight matrix, larger than the L2, once per pair of m-tiles.)
// WGRAD gives whole experts to XCDs (hot experts are split over all XCDs, see
// build_wgrad_schedule) and orders an expert's output tiles in groups of
// kWgGroupM m-tiles, m-tile fastest within a group, so the concurrent tiles
// form a block that shares both operand panels.
// Correctness does not depend on the XCD mapping: every tile id is owned by
// exactly one workgroup.

constexpr int kMaxChunks = 1920;      // chunk list: kMaxChunks/8 entries per XCD (+1)
constexpr int kXcdChunks = kMaxChunks / 8;
#ifndef MOE_CHUNK_M
#define MOE_CHUNK_M 8
#endif
// m-tiles per chunk: an expert of fewer than twice this many stays on one XCD.
// Measured (bf16 GEMM1, GEMM2, GEMM1 dgrad): E = 8 with 32 m-tiles per expert
// 20 % faster with chunks of 8 than of 16; Zipf routing 7-8 % faster; E = 128
// (4-9 m-tiles per expert: one chunk either way) unchanged; chunks of 4 lose
// 10 % at E = 128 bf16 and MXFP8, where they split experts.
constexpr int kChunkM = MOE_CHUNK_M;
#ifndef MOE_WG_GROUP_M
#define MOE_WG_GROUP_M 8
#endif
constexpr int kWgGroupM = MOE_WG_GROUP_M;   // WGRAD: m-tiles per tile group

struct RowSchedule {
    int n_tiles;      // n-tiles per m-tile
    int chm;          // m-tiles per chunk
    int total;        // tiles owned by this workgroup's XCD
};

// s_tile: exclusive prefix of m-tiles per group (from build_tile_table).
// Builds s_chunk (chunk prefix per group, E+1) and s_xpre (tile prefix over
// this XCD's chunks, up to kMaxChunks/8 + 1 entries). blockDim.x >= 256.
// A group of mt_e m-tiles is cut into max(1, round(mt_e / chm)) chunks of
// equal size up to one m-tile (the first mt_e % n chunks one larger): no
// chunk is a sliver that would cost its XCD a whole weight-matrix read for
// little work, and the chunks dealt to the XCDs are alike, so the XCDs'
// totals are too.
MOE_DEV int chunk_count(int mt_e, int chm) { return mt_e > 0 ? max(1, (mt_e + chm / 2) / chm) : 0; }
// m-tiles of chunk ci of a group of mt_e m-tiles, and its first m-tile
MOE_DEV int chunk_mtiles(int mt_e, int chm, int ci) {
    const int n = chunk_count(mt_e, chm);
    return mt_e / n + (ci < mt_e % n ? 1 : 0);
}
MOE_DEV int chunk_first(int mt_e, int chm, int ci) {
    const int n = chunk_count(mt_e, chm);
    return ci * (mt_e / n) + min(ci, mt_e % n);
}

MOE_DEV RowSchedule build_row_schedule(const int32_t *s_tile, int E, int n_tiles, int xcd,
                                       int32_t *s_chunk, int32_t *s_xpre) {
    const int tid = threadIdx.x;
    const int mt_total = s_tile[E];
    // chunk size: at least kChunkM m-tiles, more when needed to stay within kMaxChunks
    const int chm = max(kChunkM, (mt_total + (kMaxChunks - 256) - 1) / (kMaxChunks - 256));
    int32_t nc = 0;
    if (tid < E) nc = chunk_count(s_tile[tid + 1] - s_tile[tid], chm);
    if (tid < 256) s_chunk[tid + 1] = nc;
    if (tid == 0) s_chunk[0] = 0;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        int32_t v = (tid < 256 && tid >= o) ? s_chunk[tid + 1 - o] : 0;
        __syncthreads();
        if (tid < 256) s_chunk[tid + 1] += v;
        __syncthreads();
    }
    const int C = s_chunk[E];
    const int cx = C > xcd ? (C - xcd + 7) / 8 : 0;     // chunks of this XCD (<= 256)
    int32_t t = 0;
    if (tid < cx) {
        const int c = xcd + 8 * tid;
        const int e = find_group(s_chunk, E, c);
        const int ci = c - s_chunk[e];
        const int mt_e = s_tile[e + 1] - s_tile[e];
        t = chunk_mtiles(mt_e, chm, ci) * n_tiles;
    }
    // (C <= kMaxChunks by the choice of chm, so cx <= kXcdChunks)
    if (tid < kXcdChunks) s_xpre[tid + 1] = t;
    if (tid == 0) s_xpre[0] = 0;
    __syncthreads();
    for (int o = 1; o < kXcdChunks; o <<= 1) {
        int32_t v = (tid < kXcdChunks && tid >= o) ? s_xpre[tid + 1 - o] : 0;
        __syncthreads();
        if (tid < kXcdChunks) s_xpre[tid + 1] += v;
        __syncthreads();
    }
    RowSchedule r;
    r.n_tiles = n_tiles;
    r.chm = chm;
    r.total = s_xpre[cx];
    (void)cx;
    return r;
}

// position p of this XCD's list -> (group e, m-tile index within e, n-tile)
MOE_DEV void decode_row_tile(const RowSchedule &rs, const int32_t *s_tile, const int32_t *s_chunk,
                             const int32_t *s_xpre, int E, int xcd, int p, int &e, int &mt_e,
                             int &nt) {
    int lo = 0, hi = kXcdChunks;          // largest lc with s_xpre[lc] <= p
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (s_xpre[mid] <= p) lo = mid; else hi = mid - 1;
    }
    // entries past this XCD's chunk count repeat the total, which is > p
    const int c = xcd + 8 * lo;
    const int o = p - s_xpre[lo];
    e = find_group(s_chunk, E, c);
    // m-tile fastest within the chunk: the XCD's concurrent tiles cover all
    // of the chunk's m-tiles and a few weight panels, so each weight panel
    // is fetched into the XCD's L2 once and shared by the chunk's m-tiles
    const int ci = c - s_chunk[e];
    const int cm = chunk_mtiles(s_tile[e + 1] - s_tile[e], rs.chm, ci);
    mt_e = chunk_first(s_tile[e + 1] - s_tile[e], rs.chm, ci) + o % cm;
    nt = o / cm;
}

// WGRAD schedule. Every expert has the same number of output tiles (per_e);
// its cost grows with its row count. An expert with more than twice the mean
// rows is split into 8 equal tile chunks, chunk x on XCD x, at the head of
// every XCD's list (the longest work starts first); the other experts stay
// whole and are dealt round-robin over the XCDs in index order, so their
// operands are read by a single XCD. Without the split, one very hot expert
// (skewed routing) would keep a single XCD busy long after the others.
// s_scan: 257 ints of scratch; s_list: split experts at [0, 128), this XCD's
// whole experts at [128, 160). (At most E/2 experts can exceed twice the mean.)
struct WgSchedule {
    int n_split, n_light, cs, total;
};

MOE_DEV WgSchedule build_wgrad_schedule(const int32_t *s_off, int E, int per_e, int xcd,
                                        int32_t *s_scan, int32_t *s_list) {
    const int tid = threadIdx.x;
    const int R = s_off[E];
    const int thresh = 2 * ((R + E - 1) / E);
    const bool can_split = per_e % 8 == 0;
    int fl = 0;
    if (tid < E && can_split) fl = (s_off[tid + 1] - s_off[tid] > thresh) ? 1 : 0;
    if (tid < 256) s_scan[tid + 1] = fl;
    if (tid == 0) s_scan[0] = 0;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        int32_t v = (tid < 256 && tid >= o) ? s_scan[tid + 1 - o] : 0;
        __syncthreads();
        if (tid < 256) s_scan[tid + 1] += v;
        __syncthreads();
    }
    const int n_split = s_scan[E];
    if (tid < E) {
        const int before = s_scan[tid];
        if (fl) {
            s_list[before] = tid;
        } else {
            const int lr = tid - before;         // rank among the whole experts
            if ((lr & 7) == xcd) s_list[128 + (lr >> 3)] = tid;
        }
    }
    __syncthreads();
    WgSchedule w;
    w.n_split = n_split;
    const int n_whole = E - n_split;
    w.n_light = n_whole > xcd ? (n_whole - xcd + 7) / 8 : 0;
    w.cs = per_e / 8;
    w.total = n_split * w.cs + w.n_light * per_e;
    return w;
}

// A worker's next position in its XCD's WGRAD list. Without split experts:
// a fixed stride (the tiles cost about the same, and workers in step share
// the operand panels of neighbouring tiles). With them the list starts with
// the long split tiles, and a fixed stride would give the workers that take
// those also their full share of the rest: the rounds of `workers` positions
// are then walked forward and backward in turn (under Zipf routing, whose
// hottest expert has 23 % of the rows, the weight gradients ran 10 % faster;
// with no expert split the snake cost 4 % and is not used).
MOE_DEV int wgrad_next(const WgSchedule &ws, int pos, int worker, int workers) {
    if (ws.n_split == 0) return pos + workers;
    const int r = pos / workers + 1;
    return r * workers + ((r & 1) ? workers - 1 - worker : worker);
}

// position p of this XCD's WGRAD list -> (group e, output m-tile mi, n-tile nt).
// An expert's tiles come in groups of kWgGroupM m-tiles, m-tile fastest within
// a group: the XCD's concurrent tiles form a block of m-tiles x n-tiles, so
// both operand panels are shared from L2 by several tiles.
MOE_DEV void decode_wgrad_tile(const WgSchedule &ws, const int32_t *s_list, int xcd, int p,
                               int mtiles, int n_tiles, int &e, int &mi, int &nt) {
    const int per_e = mtiles * n_tiles;
    int tt;
    if (p < ws.n_split * ws.cs) {          // this XCD's chunk of a split expert
        e = s_list[p / ws.cs];
        tt = xcd * ws.cs + p % ws.cs;
    } else {                               // a whole expert of this XCD
        const int p2 = p - ws.n_split * ws.cs;
        e = s_list[128 + p2 / per_e];
        tt = p2 % per_e;
    }
    const int grp = tt / (kWgGroupM * n_tiles), first_m = grp * kWgGroupM;
    const int gm = min(mtiles - first_m, kWgGroupM);
    const int tg = tt - grp * kWgGroupM * n_tiles;
    mi = first_m + tg % gm;
    nt = tg / gm;
}

// ---------------------------------------------------------------------------
// MFMA kernel: bf16 (v_mfma_f32_32x32x16_bf16) and MXFP8
// (v_mfma_scale_f32_32x32x64_f8f6f4 with E8M0 block scales)


typedef short v4i16 __attribute__((ext_vector_type(4)));
#define MOE_LDS __attribute__((address_space(3)))

// Source of the LDS copies of chunks past the K extent (and of the MXFP8
// scale words of rows that have none): zero-initialised device memory.
__device__ uint4 g_zero_chunk[64] = {};

// (K-layout LDS tiles: kl_chunk in copy_plan.h)

// MN-layout LDS tile (bf16 only): [64 k][R] bf16, i.e. the global tile copied
// as is. Chunk c of row k sits at c ^ ((k & 3) << 2): the four k rows that one
// transpose read touches fall in four different 64-byte bank windows.
template <int R>
MOE_DEV int mn_chunk(int k, int c) { return k * (R / 8) + (c ^ ((k & 3) << 2)); }

// Stores of the fp32 weight gradients and of dAB. With MOE_NT_STORE they are
// non-temporal: the outputs stream out without displacing the operand panels
// that other tiles of the XCD are still reading from L2 (measured: the MXFP8
// GEMM1 weight gradient at E=128, d=4096 runs 7% faster).
#ifndef MOE_NT_STORE
#define MOE_NT_STORE 1
#endif
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
MOE_DEV void store_f32(float *p, float v) {
    if constexpr (MOE_NT_STORE) __builtin_nontemporal_store(v, p);
    else *p = v;
}
MOE_DEV void store16(void *p, uint4 v) {
    if constexpr (MOE_NT_STORE) {
        u32x4 w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
    } else {
        *reinterpret_cast<uint4 *>(p) = v;
    }
}

// A condition that holds for the whole wave or for none of its lanes, taken
// from lane 0 so that the branch on it is a scalar one.
MOE_DEV bool wave_full(bool c) { return __builtin_amdgcn_readfirstlane((int)c) != 0; }

// Byte address of element (row, col) of a row-major matrix with ld elements
// per row, for wave-uniform row and col (kept in scalar registers), and the
// byte offset of lane l's first accumulator element from there: row
// (l / 32) * 4, column l % 32 of the MFMA output layout.
template <typename T>
MOE_DEV char *wave_base(T *p, int row, int col, int ld) {
    row = __builtin_amdgcn_readfirstlane(row);
    col = __builtin_amdgcn_readfirstlane(col);
    return reinterpret_cast<char *>(p + ((int64_t)row * ld + col));
}
template <int ES>
MOE_DEV uint32_t lane_off(int lane, int ld) { return (uint32_t)(((lane >> 5) * 4 * ld + (lane & 31)) * ES); }

// Wait until at most N vector-memory instructions of this wave are in flight
// (they complete in issue order).
template <int N>
MOE_DEV void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for the LDS pipeline: this wave's LDS reads have
// completed (lgkmcnt(0)), then s_barrier, then an acquire fence on LDS only so
// later LDS reads stay below the barrier. No global-memory fence: that would
// drain the LDS copies that are still in flight for later stages.
MOE_DEV void lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Copy 16 (dma16) or 4 (dma4) bytes per lane from global memory straight into
// LDS: lane l's bytes land at lds_wave_base + size * l (lds_wave_base is
// wave-uniform, passed in M0). Issued through inline asm so that the only
// waits on these copies are the explicit ones of the pipeline below
// (wait_vmem + lds_sync); the instructions have no result registers, and the
// "memory" clobber keeps LDS reads from moving across them.
MOE_DEV void dma16(const void *src, const void *lds_wave_base) {
    // wave-uniform by construction; readfirstlane keeps it in an SGPR for M0
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const MOE_LDS void *)lds_wave_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(m0v)
                 : "memory", "m0");
}
MOE_DEV void dma4(const void *src, const void *lds_wave_base) {
    // wave-uniform by construction; readfirstlane keeps it in an SGPR for M0
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const MOE_LDS void *)lds_wave_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(src), "s"(m0v)
                 : "memory", "m0");
}

// The same copy with the address split into a wave-uniform base in SGPRs
// and a 32-bit per-lane offset: advancing a whole tile by one K step is then
// a scalar add, with no per-lane address arithmetic.
MOE_DEV void dma16s(uint32_t voff, const char *sbase, const void *lds_wave_base) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const MOE_LDS void *)lds_wave_base);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(m0v)
                 : "memory", "m0");
}

// a pointer that is equal in every lane, moved into scalar registers (the
// builtin returns a signed int: each half is widened from uint32_t, or a low
// word with bit 31 set would be sign-extended over the high word)
MOE_DEV const char *uniform_ptr(const char *p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const char *>((uintptr_t)((hi << 32) | lo));
}

// One operand tile per stage, copied HBM -> LDS by global_load_lds_dwordx4
// with the geometry of CopyGeom (copy_plan.h): the tile origin in SGPRs,
// advanced by one scalar add per K step, plus a fixed 32-bit offset per lane
// and instruction.
template <int R, bool KL, int NW>
struct DmaTile : CopyGeom<R, KL, NW> {
    using G = CopyGeom<R, KL, NW>;
    static constexpr int IPW = G::IPW;
    static constexpr int STEP = G::STEP;
    const char *base;          // tile origin at step 0 (wave-uniform)
    int64_t kstride;           // bytes to advance per step
    uint32_t voff[IPW];        // per lane and instruction: byte offset of its chunk

    // KL: row_off(r) -> byte offset from b of tile row r's K run (< 2^32)
    template <typename RowFn>
    MOE_DEV void setup_kl(const char *b, RowFn row_off, int wave, int lane) {
        base = uniform_ptr(b);
#pragma unroll
        for (int i = 0; i < IPW; i++) voff[i] = G::kl_off(i, wave, lane, row_off);
        kstride = G::kstride(0);
    }
    // MN: b = element (k = 0, col 0) of the tile, ld = row pitch in bytes,
    // cvalid = valid columns (>= 1)
    MOE_DEV void setup_mn(const char *b, int64_t ld, int cvalid, int wave, int lane) {
        base = uniform_ptr(b);
#pragma unroll
        for (int i = 0; i < IPW; i++) voff[i] = G::mn_off(i, wave, lane, ld, cvalid);
        kstride = G::kstride(ld);
    }
    // enqueue the copy of step kt; klim = K bytes (KL) or K rows (MN)
    MOE_DEV void issue(uint4 *lds, int kt, int klim, int wave) const {
        const int k0 = kt * STEP;
        const char *b = base + (int64_t)kt * kstride;
        if (k0 + STEP <= klim) {
#pragma unroll
            for (int i = 0; i < IPW; i++) dma16s(voff[i], b, lds + (wave * IPW + i) * 64);
        } else {
            const int lane = threadIdx.x & 63;
#pragma unroll
            for (int i = 0; i < IPW; i++) {
                const bool ok = G::in_k(i, wave, lane, kt, klim);
                const void *s = ok ? (const void *)(b + voff[i]) : (const void *)&g_zero_chunk[lane];
                dma16(s, lds + (wave * IPW + i) * 64);
            }
        }
    }
    // bf16 MFMA operand for rows/cols r0..r0+31, k slice kk (16 wide):
    // lanes 0-31 get k 16*kk..+7, lanes 32-63 k 16*kk+8..+15
    MOE_DEV static bf16x8 frag(const uint4 *lds, int r0, int kk, int lane) {
        if constexpr (KL) {
            return __builtin_bit_cast(bf16x8, lds[kl_chunk(r0 + (lane & 31), kk * 2 + (lane >> 5))]);
        } else {
            // ds_read_b64_tr_b16: within a 16-lane group, lane i receives element
            // (i % 4) of the 8-byte segments read by lanes 4j + i/4, j = 0..3. Lane
            // s reads columns m0 + 4*(s%4)..+3 of row k0 + s/4, so lane i ends up
            // with column m0 + i at rows k0..k0+3.
            const int grp = lane >> 4, s = lane & 15;
            const int m = r0 + (grp & 1) * 16 + 4 * (s & 3);
            const int k = kk * 16 + (grp >> 1) * 8 + (s >> 2);
            const char *base = reinterpret_cast<const char *>(lds);
            const int o0 = mn_chunk<R>(k, m >> 3) * 16 + (m & 7) * 2;
            const int o1 = mn_chunk<R>(k + 4, m >> 3) * 16 + (m & 7) * 2;
            v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS v4i16 *)(base + o0));
            v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS v4i16 *)(base + o1));
            typedef short v8i16 __attribute__((ext_vector_type(8)));
            v8i16 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
            return __builtin_bit_cast(bf16x8, r);
        }
    }
    // fp8 MFMA operand (32x32x64) for rows r0..r0+31, K slice s (64 wide) of the
    // step: lane l holds K 16*(l/32)..+15 of the slice in dwords 0-3 and
    // 32+16*(l/32)..+15 in dwords 4-7 (layout measured on the GPU)
    MOE_DEV static i32x8 frag8(const uint4 *lds, int r0, int s, int lane) {
        static_assert(KL, "fp8 operands are K-contiguous");
        const int row = r0 + (lane & 31), half = lane >> 5;
        const uint4 c0 = lds[kl_chunk(row, s * 4 + half)];
        const uint4 c1 = lds[kl_chunk(row, s * 4 + 2 + half)];
        i32x8 r = {(int)c0.x, (int)c0.y, (int)c0.z, (int)c0.w,
                   (int)c1.x, (int)c1.y, (int)c1.z, (int)c1.w};
        return r;
    }
};

// STAGES LDS buffers; the copy of step kt+STAGES-1 is enqueued while step kt
// is multiplied, so STAGES-1 copies are in flight behind the MFMAs.
// FP8: operands are MXFP8 (E4M3 bytes, K-contiguous in every mode) and each
// stage also holds the E8M0 scale words (4 blocks = one 128-byte step) of its
// A rows and B rows, copied with one 4-byte LDS-DMA per wave.
// ACC (WGRAD only): C += the product instead of C = (a separate
// instantiation, so the overwriting kernel carries none of its code)
template <int MODE, int EPI, bool FP8, int BM, int BN, int WM, int WN, int STAGES, int WPE,
          bool ACC = false>
__global__ __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void gg_mfma(GemmArgs g) {
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM >= 1 && TN >= 1, "wave tile");
    static_assert(STAGES >= 2 && STAGES <= 3, "pipeline depth");
    static_assert(EPI != MOE_EPI_SWIGLU_FWD || TN % 2 == 0, "SwiGLU pairs gate/up sub-tiles");
    // FP8: the stage's BM + BN scale words are copied SPW per lane
    constexpr int SPW = FP8 ? (BM + BN + NW * 64 - 1) / (NW * 64) : 0;
    constexpr bool A_KL = FP8 || MODE != MOE_GG_WGRAD;
    constexpr bool B_KL = FP8 || MODE == MOE_GG_FWD;
    using AT = DmaTile<BM, A_KL, NW>;
    using BT = DmaTile<BN, B_KL, NW>;
    constexpr int IPS_MAIN = AT::IPW + BT::IPW;   // operand copy instructions / wave / stage
    constexpr int IPS = IPS_MAIN + SPW;           // with one scale word per step

    // LDS pool: STAGES x (A tile | B tile | scale words) during the K loop;
    // reused after it to stage the output tile for coalesced stores (the
    // copies into LDS are issued through inline asm, so the compiler tracks no
    // LDS writes of its own here and a single array serves every stage)
    // FP8 scale words, after the stages: either per step (SPW 4-byte copies
    // per lane into a per-stage area) or, when every row's scales come in
    // whole 16-byte groups (K % 512 == 0), 16 bytes per row covering 4 steps,
    // copied every 4th step into one slot of a 2-slot ring. A 4-byte copy
    // touches 64 cache lines for 256 bytes, so the ring cuts the L1 work of
    // the scales 4x.
    constexpr int SCALE_U4 = SPW * NW * 64 * 4 / 16;              // per-stage area
    constexpr int SROWS = FP8 ? ((BM + BN + 63) / 64) * 64 : 0;   // ring rows per slot
    constexpr int SREG_U4 = FP8 ? (2 * SROWS > STAGES * SCALE_U4 ? 2 * SROWS : STAGES * SCALE_U4) : 0;
    constexpr int STAGE_U4 = (BM + BN) * 8;
    constexpr bool F32_STAGE = MODE == MOE_GG_WGRAD || EPI == MOE_EPI_SWIGLU_BWD;
    constexpr int PF = BN * 4 + 32;      // fp32 staging pitch (bytes)
    constexpr int PB = BN * 2 + 16;      // bf16 staging pitch (bytes)
    constexpr int PH = BN + 16;          // H' staging pitch (bytes)
    // the output tile is staged in passes of EP_ROWS rows, as many rows per
    // pass as fit in the LDS budget of the pool
    constexpr int EP_ROW_BYTES = F32_STAGE ? PF : (EPI == MOE_EPI_SWIGLU_FWD ? PB + PH : PB);
    constexpr int POOL_BUDGET = 152 * 1024;
    constexpr int EP_ROWS = BM * EP_ROW_BYTES <= POOL_BUDGET       ? BM
                          : (BM / 2) * EP_ROW_BYTES <= POOL_BUDGET ? BM / 2
                                                                   : BM / 4;
    constexpr int EP_PASSES = BM / EP_ROWS;
    static_assert(EP_ROWS % 32 == 0 && EP_ROWS * EP_ROW_BYTES <= POOL_BUDGET, "epilogue staging");
    constexpr int EPI_BYTES = EP_ROWS * EP_ROW_BYTES;
    constexpr int POOL_U4 = STAGES * STAGE_U4 + SREG_U4 > (EPI_BYTES + 15) / 16
                                ? STAGES * STAGE_U4 + SREG_U4
                                : (EPI_BYTES + 15) / 16;
    __shared__ __attribute__((aligned(1024))) uint4 lds_pool[POOL_U4];
    __shared__ int32_t s_off[257];
    __shared__ int32_t s_tile[257];
    __shared__ int32_t s_chunk[257];
    __shared__ int32_t s_xpre[kXcdChunks + 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int E = g.E;

    const int xcd = blockIdx.x & 7, worker = blockIdx.x >> 3, workers = gridDim.x >> 3;
    int n_tiles, total;
    RowSchedule rs;
    WgSchedule ws;
    if constexpr (MODE == MOE_GG_WGRAD) {
        // experts to XCDs by build_wgrad_schedule (hot experts split over all
        // XCDs, the others whole). FP8: s_tile[e] = sum_{e'<e} ceil(c_e'/128), the 128-row step base of
        // each expert in the column-block MXFP8 layout.
        if constexpr (FP8) build_tile_table(g.offsets, E, 128, s_off, s_tile);
        else load_offsets(g.offsets, E, s_off);
        n_tiles = (g.N + BN - 1) / BN;
        const int per_e = ((g.M + BM - 1) / BM) * n_tiles;
        ws = build_wgrad_schedule(s_off, E, per_e, xcd, s_chunk, s_xpre);
        total = ws.total;
    } else {
        build_tile_table(g.offsets, E, BM, s_off, s_tile);
        n_tiles = (EPI == MOE_EPI_SWIGLU_FWD) ? (g.h + BN / 2 - 1) / (BN / 2)
                                              : (g.N + BN - 1) / BN;
        rs = build_row_schedule(s_tile, E, n_tiles, xcd, s_chunk, s_xpre);
        total = rs.total;
    }

    const char *A = reinterpret_cast<const char *>(g.A);
    const char *B = reinterpret_cast<const char *>(g.B);
    const uint8_t *AS = g.a_scale;
    const uint8_t *BS = g.b_scale;

    using P = TilePlan<MODE, EPI, FP8, BM, BN, WTN>;
    // FP8: scales batched 16 bytes per row every 4th step, or 4 bytes per step
    const bool sbatch = P::scale_batched(g);
    (void)sbatch;

    auto decode = [&](int pos) {
        if constexpr (MODE == MOE_GG_WGRAD) {
            int e, mi, nt;
            decode_wgrad_tile(ws, s_xpre, xcd, pos, (g.M + BM - 1) / BM, n_tiles, e, mi, nt);
            // FP8: s_tile holds each group's first 128-row block of the column layout
            return P::wgrad_tile(s_off, s_tile, e, mi, nt);
        } else {
            int e, mt_e, nt;
            decode_row_tile(rs, s_tile, s_chunk, s_xpre, E, xcd, pos, e, mt_e, nt);
            return P::row_tile(g, s_off, e, mt_e, nt);
        }
    };

    // per-lane copy sources of a tile (operand chunks and FP8 scale words)
    AT ta;
    BT tb;
    const char *ssrc[SPW > 0 ? SPW : 1];
    auto setup = [&](const TileC &t) {
        if constexpr (A_KL) {
            ta.setup_kl(A + P::a_origin(g, t), [&](int r) { return P::a_row_off(g, t, r); }, wave, lane);
        } else {
            ta.setup_mn(A + P::a_origin(g, t), P::a_ld(g), P::a_cvalid(g, t), wave, lane);
        }
        if constexpr (B_KL) {
            tb.setup_kl(B + P::b_origin(g, t), [&](int n) { return P::b_row_off(g, t, n); }, wave, lane);
        } else {
            tb.setup_mn(B + P::b_origin(g, t), P::b_ld(g), P::b_cvalid(g, t), wave, lane);
        }
        // FP8: sources of this lane's scale words (rows sr of the stage's
        // [A rows | B rows | unused] scale array) for step 0
        if constexpr (FP8) {
#pragma unroll
            for (int q = 0; q < SPW; q++) {
                const int sr = (q * NW + wave) * 64 + lane;
                const int64_t o = P::scale_off(g, t, sr);
                ssrc[q] = o < 0 ? nullptr : (const char *)(P::scale_operand(sr) == 0 ? AS : BS) + o;
            }
        }
    };

    auto stage = [&](auto I) {
        constexpr int i = decltype(I)::value;
        return lds_pool + i * STAGE_U4;
    };
    // enqueue the copies of K step kt of the tile set up last (klim: its K extent)
    auto issue = [&](auto I, int kt, int klim) {
        constexpr int si = decltype(I)::value;
        uint4 *st = stage(I);
        if constexpr (FP8) {
            // batched scales first: a later wait for this stage's operands then
            // also covers them (copies complete in issue order)
            if (sbatch && (kt & 3) == 0) {
                uint4 *ring = lds_pool + STAGES * STAGE_U4 + ((kt >> 2) & 1) * SROWS;
#pragma unroll
                for (int q = 0; q < SPW; q++) {
                    if ((q * NW + wave) * 64 >= BM + BN) continue;   // wave-uniform
                    const void *s = ssrc[q] ? (const void *)(ssrc[q] + (kt >> 2) * 16)
                                            : (const void *)&g_zero_chunk[threadIdx.x & 63];
                    dma16(s, ring + (q * NW + wave) * 64);
                }
            }
        }
        ta.issue(st, kt, klim, wave);
        // bf16 DGRAD: klim is A's K extent in bytes; B (MN layout) counts K rows
        tb.issue(st + BM * 8, kt, P::b_klim(klim), wave);
        if constexpr (FP8) {
            if (!sbatch) {
                uint4 *sarea = lds_pool + STAGES * STAGE_U4 + si * SCALE_U4;
#pragma unroll
                for (int q = 0; q < SPW; q++) {
                    const void *s = ssrc[q] ? (const void *)(ssrc[q] + kt * 4)
                                            : (const void *)&g_zero_chunk[threadIdx.x & 63];
                    dma4(s, sarea + (q * NW + wave) * 16);
                }
            }
        }
    };
    auto nk_of = [](int klim) { return P::nk_of(klim); };
    // start the pipeline of a tile: its first STAGES-1 steps
    auto prologue = [&](const TileC &t) {
        const int n = nk_of(t.klim);
        if (0 < n) issue(std::integral_constant<int, 0>(), 0, t.klim);
        if constexpr (STAGES > 2)
            if (1 < n) issue(std::integral_constant<int, 1>(), 1, t.klim);
    };

    // The epilogue writes the outputs straight from the accumulators (except
    // the SwiGLU backward, which reads a, b with 16-byte row loads and goes
    // through LDS). It needs no LDS, so the next tile's first steps are
    // enqueued before it: their load latency overlaps the epilogue's stores.
    constexpr bool DIRECT_EPI = EPI != MOE_EPI_SWIGLU_BWD;

    int pos = worker;
    if (pos >= total) return;                     // uniform over the workgroup
    TileC cur = decode(pos);
    setup(cur);
    prologue(cur);
    while (true) {
        f32x16 acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++)
#pragma unroll
                for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;
        const int klim = cur.klim;
        const int nk = nk_of(klim);
        // one K step with stage buffer CUR (compile time)
        auto step = [&](auto CUR, int kt) {
            constexpr int cur = decltype(CUR)::value;
            constexpr int nb = (cur + STAGES - 1) % STAGES;
            // copies of later stages may stay in flight; step kt's must be done
            // (batched scales: per-stage counts vary; IPS_MAIN only over-waits)
            if (kt + STAGES - 2 < nk) {
                if (sbatch) wait_vmem<(STAGES - 2) * IPS_MAIN>();
                else wait_vmem<(STAGES - 2) * IPS>();
            } else {
                wait_vmem<0>();
            }
            lds_sync();
            if (kt + STAGES - 1 < nk) issue(std::integral_constant<int, nb>(), kt + STAGES - 1, klim);
            const uint4 *sa = stage(CUR);
            const uint4 *sb = sa + BM * 8;
            if constexpr (FP8) {
                uint32_t swa[TM], swb[TN];
                if (sbatch) {
                    const uint32_t *rw = reinterpret_cast<const uint32_t *>(
                        lds_pool + STAGES * STAGE_U4 + ((kt >> 2) & 1) * SROWS);
                    const int w = kt & 3;
#pragma unroll
                    for (int i = 0; i < TM; i++) swa[i] = rw[(wm * WTM + i * 32 + (lane & 31)) * 4 + w];
#pragma unroll
                    for (int j = 0; j < TN; j++) swb[j] = rw[(BM + wn * WTN + j * 32 + (lane & 31)) * 4 + w];
                } else {
                    const uint32_t *sw = reinterpret_cast<const uint32_t *>(
                        lds_pool + STAGES * STAGE_U4 + cur * SCALE_U4);
#pragma unroll
                    for (int i = 0; i < TM; i++) swa[i] = sw[wm * WTM + i * 32 + (lane & 31)];
#pragma unroll
                    for (int j = 0; j < TN; j++) swb[j] = sw[BM + wn * WTN + j * 32 + (lane & 31)];
                }
                // operand fragments double-buffered in registers: the LDS reads
                // of K slice sl+1 are issued before the MFMAs of slice sl
                i32x8 fa[2][TM], fb[2][TN];
#pragma unroll
                for (int i = 0; i < TM; i++) fa[0][i] = AT::frag8(sa, wm * WTM + i * 32, 0, lane);
#pragma unroll
                for (int j = 0; j < TN; j++) fb[0][j] = BT::frag8(sb, wn * WTN + j * 32, 0, lane);
#pragma unroll
                for (int sl = 0; sl < 2; sl++) {
                    if (MODE != MOE_GG_WGRAD && sl == 0) {
                        // row GEMMs: the reads of slice 1 go one between each
                        // two MFMAs of slice 0, as in the bf16 path
                        const int sh = 8 * (lane >> 5);
#pragma unroll
                        for (int t = 0; t < TM * TN; t++) {
                            if (t < TM) fa[1][t] = AT::frag8(sa, wm * WTM + t * 32, 1, lane);
                            else if (t < TM + TN) fb[1][t - TM] = BT::frag8(sb, wn * WTN + (t - TM) * 32, 1, lane);
                            __builtin_amdgcn_sched_barrier(0);
                            const int i = t / TN, j = t % TN;
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                fa[0][i], fb[0][j], acc[i][j], 0, 0, 0,
                                (int)((swa[i] >> sh) & 0xff), 0, (int)((swb[j] >> sh) & 0xff));
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        continue;
                    }
                    if (sl + 1 < 2) {
#pragma unroll
                        for (int i = 0; i < TM; i++) fa[1][i] = AT::frag8(sa, wm * WTM + i * 32, 1, lane);
#pragma unroll
                        for (int j = 0; j < TN; j++) fb[1][j] = BT::frag8(sb, wn * WTN + j * 32, 1, lane);
                    }
                    __builtin_amdgcn_sched_barrier(0);   // keep the prefetch above the MFMAs
                    // lane l supplies the scale of (row l%32, block 2*sl + l/32)
                    const int sh = 8 * (2 * sl + (lane >> 5));
#pragma unroll
                    for (int i = 0; i < TM; i++)
#pragma unroll
                        for (int j = 0; j < TN; j++)
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                fa[sl][i], fb[sl][j], acc[i][j], 0, 0, 0,
                                (int)((swa[i] >> sh) & 0xff), 0, (int)((swb[j] >> sh) & 0xff));
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                // operand fragments double-buffered in registers: the LDS reads
                // of K slice kk+1 are issued while the MFMAs of slice kk run
                bf16x8 fa[2][TM], fb[2][TN];
#pragma unroll
                for (int i = 0; i < TM; i++) fa[0][i] = AT::frag(sa, wm * WTM + i * 32, 0, lane);
#pragma unroll
                for (int j = 0; j < TN; j++) fb[0][j] = BT::frag(sb, wn * WTN + j * 32, 0, lane);
#pragma unroll
                for (int kk = 0; kk < 4; kk++) {
                    const int cb = kk & 1, nb2 = cb ^ 1;
                    if constexpr (MODE != MOE_GG_WGRAD) {
                        // one fragment read between consecutive MFMAs: the LDS
                        // requests of the CU arrive spread over the slice
                        // (measured 2-4% faster on the row GEMMs; the weight
                        // gradients run 2-6% slower this way)
                        static_assert(TM + TN <= TM * TN, "one read per MFMA slot");
#pragma unroll
                        for (int t = 0; t < TM * TN; t++) {
                            if (kk + 1 < 4) {
                                if (t < TM) fa[nb2][t] = AT::frag(sa, wm * WTM + t * 32, kk + 1, lane);
                                else if (t < TM + TN)
                                    fb[nb2][t - TM] = BT::frag(sb, wn * WTN + (t - TM) * 32, kk + 1, lane);
                            }
                            __builtin_amdgcn_sched_barrier(0);
                            acc[t / TN][t % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                fa[cb][t / TN], fb[cb][t % TN], acc[t / TN][t % TN], 0, 0, 0);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    } else {
                        if (kk + 1 < 4) {
#pragma unroll
                            for (int i = 0; i < TM; i++) fa[nb2][i] = AT::frag(sa, wm * WTM + i * 32, kk + 1, lane);
#pragma unroll
                            for (int j = 0; j < TN; j++) fb[nb2][j] = BT::frag(sb, wn * WTN + j * 32, kk + 1, lane);
                        }
                        __builtin_amdgcn_sched_barrier(0);   // keep the prefetch above the MFMAs
#pragma unroll
                        for (int i = 0; i < TM; i++)
#pragma unroll
                            for (int j = 0; j < TN; j++)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cb][i], fb[cb][j], acc[i][j], 0, 0, 0);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        };
        for (int kt = 0; kt < nk; kt += STAGES) {
            step(std::integral_constant<int, 0>(), kt);
            if (kt + 1 < nk) step(std::integral_constant<int, 1>(), kt + 1);
            if constexpr (STAGES > 2)
                if (kt + 2 < nk) step(std::integral_constant<int, 2>(), kt + 2);
        }

        int npos = pos + workers;
        if constexpr (MODE == MOE_GG_WGRAD) npos = wgrad_next(ws, pos, worker, workers);
        const bool has_next = npos < total;
        TileC nxt = cur;
        if constexpr (DIRECT_EPI) {
            // An accumulating weight gradient reads C in its epilogue; those
            // reads go out before the next tile's copies, which they would
            // otherwise wait behind (vector-memory loads return in issue order).
            constexpr bool epi_first = MODE == MOE_GG_WGRAD && ACC;
            if (!epi_first && has_next) {
                nxt = decode(npos);
                setup(nxt);
                lds_sync();                       // every wave is done with this tile's stages
                prologue(nxt);
            }
            // acc[i][j][v] holds row (v/4)*8 + (lane/32)*4 + v%4 and column
            // lane%32 of the wave's (i, j) 32x32 tile
            const int col_l = lane & 31;
            if constexpr (MODE == MOE_GG_WGRAD) {
                float *C = reinterpret_cast<float *>(g.C) + (int64_t)cur.e * g.M * g.N;
                auto row_of = [&](int i, int v) {
                    return cur.m0 + wm * WTM + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
                };
                if constexpr (epi_first) {
                    // C += the tile, one fp32 add per element. Every old value
                    // of the wave's tile is loaded before the first store: with
                    // loads and stores both in flight the compiler would wait
                    // for all memory operations before each use of a loaded
                    // value
                    float old[TM][TN][16];
#pragma unroll
                    for (int i = 0; i < TM; i++)
#pragma unroll
                        for (int j = 0; j < TN; j++) {
                            const int n = cur.n0 + wn * WTN + j * 32 + col_l;
#pragma unroll
                            for (int v = 0; v < 16; v++) {
                                const int m = row_of(i, v);
                                old[i][j][v] = (m < g.M && n < g.N) ? C[(int64_t)m * g.N + n] : 0.f;
                            }
                        }
                    // one wait for all of them, on the path every lane takes
                    // (the stores below sit in masked branches)
                    wait_vmem<0>();
#pragma unroll
                    for (int i = 0; i < TM; i++)
#pragma unroll
                        for (int j = 0; j < TN; j++) {
                            const int n = cur.n0 + wn * WTN + j * 32 + col_l;
#pragma unroll
                            for (int v = 0; v < 16; v++) {
                                const int m = row_of(i, v);
                                if (m < g.M && n < g.N) store_f32(C + (int64_t)m * g.N + n, old[i][j][v] + acc[i][j][v]);
                            }
                        }
                } else {
#pragma unroll
                    for (int i = 0; i < TM; i++)
#pragma unroll
                        for (int j = 0; j < TN; j++) {
                            const int n = cur.n0 + wn * WTN + j * 32 + col_l;
#pragma unroll
                            for (int v = 0; v < 16; v++) {
                                const int m = row_of(i, v);
                                if (m < g.M && n < g.N) store_f32(C + (int64_t)m * g.N + n, acc[i][j][v]);
                            }
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
                        const int jj = cur.nt * (BN / 2) + wn * (WTN / 2) + j * 32 + col_l;
#pragma unroll
                        for (int v = 0; v < 16; v++) {
                            const int grow = cur.row0 + wm * WTM + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
                            if (grow < cur.row_end && jj < h) {
                                const float a = acc[i][j][v], b = acc[i][j + TN / 2][v];
                                uint16_t *abr = AB + (int64_t)grow * 2 * h;
                                abr[jj] = f32_to_bf16(a);
                                abr[h + jj] = f32_to_bf16(b);
                                HP[(int64_t)grow * h + jj] = f32_to_bf16(silu_f(a) * b);
                            }
                        }
                    }
            } else {
                uint16_t *C = reinterpret_cast<uint16_t *>(g.C);
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int j = 0; j < TN; j++) {
                        const int n = cur.n0 + wn * WTN + j * 32 + col_l;
#pragma unroll
                        for (int v = 0; v < 16; v++) {
                            const int grow = cur.row0 + wm * WTM + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
                            if (grow < cur.row_end && n < g.N)
                                C[(int64_t)grow * g.N + n] = f32_to_bf16(acc[i][j][v]);
                        }
                    }
            }
            if (epi_first && has_next) {
                nxt = decode(npos);
                setup(nxt);
                lds_sync();
                prologue(nxt);
            }
        } else {
            // ---- epilogue. acc[i][j][v] holds row (v/4)*8 + (lane/32)*4 + v%4 and
            // column lane%32 of the wave's (i, j) 32x32 tile. Each pass writes the
            // 32-row sub-tiles that fall in rows [pr0, pr0 + EP_ROWS) of the tile
            // to LDS, then copies those rows out with 16-byte accesses.
            char *stg = reinterpret_cast<char *>(lds_pool);
            const int col_l = lane & 31;
            constexpr int NT = NW * 64;
    #pragma unroll
            for (int pass = 0; pass < EP_PASSES; pass++) {
                const int pr0 = pass * EP_ROWS;
                lds_sync();                               // stage buffers / previous pass no longer read
    #pragma unroll
                for (int i = 0; i < TM; i++) {
                    const int rb = wm * WTM + i * 32;     // wave-uniform
                    if (rb < pr0 || rb >= pr0 + EP_ROWS) continue;
    #pragma unroll
                    for (int j = 0; j < (EPI == MOE_EPI_SWIGLU_FWD ? TN / 2 : TN); j++)
    #pragma unroll
                        for (int v = 0; v < 16; v++) {
                            const int r = rb - pr0 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
                            if constexpr (F32_STAGE) {
                                const int c = wn * WTN + j * 32 + col_l;
                                *reinterpret_cast<float *>(stg + r * PF + c * 4) = acc[i][j][v];
                            } else if constexpr (EPI == MOE_EPI_SWIGLU_FWD) {
                                const int jt = wn * (WTN / 2) + j * 32 + col_l;
                                const float a = acc[i][j][v], b = acc[i][j + TN / 2][v];
                                uint16_t *abr = reinterpret_cast<uint16_t *>(stg + r * PB);
                                abr[jt] = f32_to_bf16(a);
                                abr[BN / 2 + jt] = f32_to_bf16(b);
                                reinterpret_cast<uint16_t *>(stg + EP_ROWS * PB + r * PH)[jt] =
                                    f32_to_bf16(silu_f(a) * b);
                            } else {
                                const int c = wn * WTN + j * 32 + col_l;
                                reinterpret_cast<uint16_t *>(stg + r * PB)[c] = f32_to_bf16(acc[i][j][v]);
                            }
                        }
                }
                lds_sync();
                if constexpr (MODE == MOE_GG_WGRAD) {
                    float *C = reinterpret_cast<float *>(g.C) + (int64_t)cur.e * g.M * g.N;
                    constexpr int CPR = BN / 4;
                    for (int it = tid; it < EP_ROWS * CPR; it += NT) {
                        const int r = it / CPR, c = it % CPR;
                        const int m = cur.m0 + pr0 + r, n = cur.n0 + c * 4;
                        if (m < g.M && n < g.N)
                            store16(C + (int64_t)m * g.N + n,
                                    *reinterpret_cast<const uint4 *>(stg + r * PF + c * 16));
                    }
                } else if constexpr (EPI == MOE_EPI_SWIGLU_BWD) {
                    const uint16_t *AB = reinterpret_cast<const uint16_t *>(g.aux);
                    uint16_t *dAB = reinterpret_cast<uint16_t *>(g.C);
                    const int h = g.h;
                    // each thread's (row, 8-column) chunks of the pass, GRP at a
                    // time: their a and b loads are issued together and waited
                    // for once, on the path every lane takes (with loads and
                    // stores both in flight the compiler would otherwise wait
                    // for everything before each chunk)
                    constexpr int CPR = BN / 8;
                    constexpr int ITERS = (EP_ROWS * CPR + NT - 1) / NT;
                    constexpr int GRP = ITERS < 2 ? ITERS : 2;
                    for (int q0 = 0; q0 < ITERS; q0 += GRP) {
                        uint4 la[GRP], lb[GRP];
#pragma unroll
                        for (int u = 0; u < GRP; u++) {
                            const int it = tid + (q0 + u) * NT;
                            const int r = it / CPR, c = it % CPR;
                            const int grow = cur.row0 + pr0 + r, jj = cur.n0 + c * 8;
                            if (q0 + u < ITERS && it < EP_ROWS * CPR && grow < cur.row_end && jj < h) {
                                const uint16_t *abr = AB + (int64_t)grow * 2 * h;
                                la[u] = *reinterpret_cast<const uint4 *>(abr + jj);
                                lb[u] = *reinterpret_cast<const uint4 *>(abr + h + jj);
                            }
                        }
                        wait_vmem<0>();
#pragma unroll
                        for (int u = 0; u < GRP; u++) {
                            const int it = tid + (q0 + u) * NT;
                            const int r = it / CPR, c = it % CPR;
                            const int grow = cur.row0 + pr0 + r, jj = cur.n0 + c * 8;
                            if (q0 + u >= ITERS || it >= EP_ROWS * CPR || grow >= cur.row_end || jj >= h) continue;
                            const uint4 ua = la[u], ub = lb[u];
                            const float4 d0 = *reinterpret_cast<const float4 *>(stg + r * PF + c * 32);
                            const float4 d1 = *reinterpret_cast<const float4 *>(stg + r * PF + c * 32 + 16);
                            const float dh[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
                            const uint32_t wa[4] = {ua.x, ua.y, ua.z, ua.w}, wb[4] = {ub.x, ub.y, ub.z, ub.w};
                            uint32_t oa[4], ob[4];
#pragma unroll
                            for (int w = 0; w < 4; w++) {
                                float da2[2], db2[2];
#pragma unroll
                                for (int hh = 0; hh < 2; hh++) {
                                    const float a = hh ? hi_bf16(wa[w]) : lo_bf16(wa[w]);
                                    const float b = hh ? hi_bf16(wb[w]) : lo_bf16(wb[w]);
                                    const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-a));
                                    const float d = dh[2 * w + hh];
                                    da2[hh] = d * b * sg * (1.f + a * (1.f - sg));
                                    db2[hh] = d * a * sg;
                                }
                                oa[w] = pack_bf16x2(da2[0], da2[1]);
                                ob[w] = pack_bf16x2(db2[0], db2[1]);
                            }
                            uint16_t *dr = dAB + (int64_t)grow * 2 * h;
                            store16(dr + jj, make_uint4(oa[0], oa[1], oa[2], oa[3]));
                            store16(dr + h + jj, make_uint4(ob[0], ob[1], ob[2], ob[3]));
                        }
                    }
                } else if constexpr (EPI == MOE_EPI_SWIGLU_FWD) {
                    uint16_t *AB = reinterpret_cast<uint16_t *>(g.C);
                    uint16_t *HP = reinterpret_cast<uint16_t *>(g.aux_out);
                    const int h = g.h, j0 = cur.nt * (BN / 2);
                    constexpr int CPR = BN / 8;           // gate half then up half
                    for (int it = tid; it < EP_ROWS * CPR; it += NT) {
                        const int r = it / CPR, c = it % CPR;
                        const int grow = cur.row0 + pr0 + r;
                        const int half = c >= CPR / 2, jj = j0 + (c - half * (CPR / 2)) * 8;
                        if (grow >= cur.row_end || jj >= h) continue;
                        store16(AB + (int64_t)grow * 2 * h + half * h + jj,
                                *reinterpret_cast<const uint4 *>(stg + r * PB + c * 16));
                    }
                    constexpr int CPH = BN / 16;
                    for (int it = tid; it < EP_ROWS * CPH; it += NT) {
                        const int r = it / CPH, c = it % CPH;
                        const int grow = cur.row0 + pr0 + r, jj = j0 + c * 8;
                        if (grow >= cur.row_end || jj >= h) continue;
                        store16(HP + (int64_t)grow * h + jj,
                                *reinterpret_cast<const uint4 *>(stg + EP_ROWS * PB + r * PH + c * 16));
                    }
                } else {
                    uint16_t *C = reinterpret_cast<uint16_t *>(g.C);
                    constexpr int CPR = BN / 8;
                    for (int it = tid; it < EP_ROWS * CPR; it += NT) {
                        const int r = it / CPR, c = it % CPR;
                        const int grow = cur.row0 + pr0 + r, n = cur.n0 + c * 8;
                        if (grow < cur.row_end && n < g.N)
                            store16(C + (int64_t)grow * g.N + n,
                                    *reinterpret_cast<const uint4 *>(stg + r * PB + c * 16));
                    }
                }
            }
            if (has_next) {
                nxt = decode(npos);
                setup(nxt);
                lds_sync();                       // the staging buffer is no longer read
                prologue(nxt);
            }
        }
        if (!has_next) break;
        cur = nxt;
        pos = npos;
    }
}

// ---------------------------------------------------------------------------
// Grouped GEMM with split roles (bf16 and MXFP8; FWD, DGRAD, WGRAD). The
// workgroup's waves 0..NC-1 are consumers: LDS fragment reads, MFMAs and the
// tile's epilogue. Waves NC..NC+NP-1 are producers: they issue every
// global -> LDS copy and wait only on those. A wave's vector-memory counter
// covers its loads and stores together, so with one role per wave the
// consumers never wait on the copies and a tile's stores drain while the next
// tile is multiplied; the producers run up to STAGES-1 steps ahead, across
// tile boundaries.
// One workgroup barrier per K step, numbered over the workgroup's tiles:
// before barrier G the producers have landed step G and the consumers have
// finished reading step G-1, whose buffer the producers refill after it.
// MXFP8 block scales: either 4 bytes per row and step into the step's stage,
// or (when batched) 16 bytes per row covering 4 steps of a tile into one slot
// of a 2-slot ring. A batch is started only once the consumers are done with
// the batch that last held its slot: when the batch before it has a single
// step (a tile of K % 512 in (0, 128]), the producers wait one more barrier.
// Tiles, schedules, LDS layouts and the order of every MFMA over K are those
// of gg_mfma, so both kernels give the same bits.

template <int MODE, int EPI, bool FP8, int BM, int BN, int WM, int WN, int NP, int STAGES,
          bool ACC = false>
__global__ __launch_bounds__((WM * WN + NP) * 64) __attribute__((amdgpu_waves_per_eu(3, 3)))
void gg_ws(GemmArgs g) {
    constexpr int NC = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM >= 1 && TN >= 1, "wave tile");
    static_assert(EPI != MOE_EPI_SWIGLU_FWD || TN % 2 == 0, "SwiGLU pairs gate/up sub-tiles");
    static_assert(EPI != MOE_EPI_SWIGLU_BWD, "the SwiGLU backward runs on gg_mfma");
    static_assert(STAGES == 3, "the producers' wait assumes one step in flight behind the next");
    constexpr bool A_KL = FP8 || MODE != MOE_GG_WGRAD;
    constexpr bool B_KL = FP8 || MODE == MOE_GG_FWD;
    using AT = DmaTile<BM, A_KL, NP>;
    using BT = DmaTile<BN, B_KL, NP>;
    constexpr int IPP = AT::IPW + BT::IPW;          // operand copies per producer wave per step
    constexpr int STAGE_U4 = (BM + BN) * 8;
    // MXFP8 scales: SPW rows per producer lane; per-step areas (one per
    // stage) or the batched 2-slot ring, in the same region
    constexpr int SPW = FP8 ? (BM + BN + NP * 64 - 1) / (NP * 64) : 0;
    constexpr int SCALE_U4 = SPW * NP * 64 * 4 / 16;
    constexpr int SROWS = FP8 ? ((BM + BN + 63) / 64) * 64 : 0;
    constexpr int SREG_U4 = FP8 ? (2 * SROWS > STAGES * SCALE_U4 ? 2 * SROWS : STAGES * SCALE_U4) : 0;
    __shared__ __attribute__((aligned(1024))) uint4 lds_pool[STAGES * STAGE_U4 + SREG_U4];
    __shared__ int32_t s_off[257];
    __shared__ int32_t s_tile[257];
    __shared__ int32_t s_chunk[257];
    __shared__ int32_t s_xpre[kXcdChunks + 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = wave >= NC;
    const int E = g.E;
    const int xcd = blockIdx.x & 7, worker = blockIdx.x >> 3, workers = gridDim.x >> 3;
    int n_tiles, total;
    RowSchedule rs;
    WgSchedule ws;
    if constexpr (MODE == MOE_GG_WGRAD) {
        // MXFP8: s_tile[e] = the group's first 128-row block of the column layout
        if constexpr (FP8) build_tile_table(g.offsets, E, 128, s_off, s_tile);
        else load_offsets(g.offsets, E, s_off);
        n_tiles = (g.N + BN - 1) / BN;
        ws = build_wgrad_schedule(s_off, E, ((g.M + BM - 1) / BM) * n_tiles, xcd, s_chunk, s_xpre);
        total = ws.total;
    } else {
        build_tile_table(g.offsets, E, BM, s_off, s_tile);
        n_tiles = (EPI == MOE_EPI_SWIGLU_FWD) ? (g.h + BN / 2 - 1) / (BN / 2) : (g.N + BN - 1) / BN;
        rs = build_row_schedule(s_tile, E, n_tiles, xcd, s_chunk, s_xpre);
        total = rs.total;
    }
    const char *A = reinterpret_cast<const char *>(g.A);
    const char *B = reinterpret_cast<const char *>(g.B);

    using P = TilePlan<MODE, EPI, FP8, BM, BN, WTN>;
    const bool sbatch = P::scale_batched(g);
    (void)sbatch;
    auto decode = [&](int pos) {
        if constexpr (MODE == MOE_GG_WGRAD) {
            int e, mi, nt;
            decode_wgrad_tile(ws, s_xpre, xcd, pos, (g.M + BM - 1) / BM, n_tiles, e, mi, nt);
            return P::wgrad_tile(s_off, FP8 ? s_tile : nullptr, e, mi, nt);
        } else {
            int e, mt_e, nt;
            decode_row_tile(rs, s_tile, s_chunk, s_xpre, E, xcd, pos, e, mt_e, nt);
            return P::row_tile(g, s_off, e, mt_e, nt);
        }
    };
    auto nk_of = [](int klim) { return P::nk_of(klim); };
    auto stage = [&](int s) { return lds_pool + s * STAGE_U4; };
    // a worker's next tile position (WGRAD: the walk of WgSchedule)
    auto next_pos = [&](int pos) {
        if constexpr (MODE == MOE_GG_WGRAD) return wgrad_next(ws, pos, worker, workers);
        else return pos + workers;
    };

    if (producer) {
        const int pw = wave - NC;
        AT ta;
        BT tb;
        const char *ssrc[SPW > 0 ? SPW : 1];
        auto setup = [&](const TileC &t) {
            if constexpr (A_KL) {
                ta.setup_kl(A + P::a_origin(g, t), [&](int r) { return P::a_row_off(g, t, r); }, pw, lane);
            } else {
                ta.setup_mn(A + P::a_origin(g, t), P::a_ld(g), P::a_cvalid(g, t), pw, lane);
            }
            if constexpr (B_KL) {
                tb.setup_kl(B + P::b_origin(g, t), [&](int n) { return P::b_row_off(g, t, n); }, pw, lane);
            } else {
                tb.setup_mn(B + P::b_origin(g, t), P::b_ld(g), P::b_cvalid(g, t), pw, lane);
            }
            if constexpr (FP8) {
#pragma unroll
                for (int q = 0; q < SPW; q++) {
                    const int sr = (q * NP + pw) * 64 + lane;
                    const int64_t o = P::scale_off(g, t, sr);
                    ssrc[q] = o < 0 ? nullptr : (const char *)(P::scale_operand(sr) == 0 ? g.a_scale : g.b_scale) + o;
                }
            }
        };
        // issue cursor over the workgroup's tiles that have steps
        int ip = worker, ikt = 0, iklim = 0;
        auto seek = [&]() {
            while (ip < total) {
                const TileC t = decode(ip);
                if (nk_of(t.klim) > 0) {
                    iklim = t.klim;
                    setup(t);
                    break;
                }
                ip = next_pos(ip);
            }
            ikt = 0;
        };
        // batched scales: batches started, and the last step of the latest
        // batch of each ring slot's parity
        int nbatch = 0, bend[2] = {-1, -1};
        // enqueue the next step (global index x) into stage x % STAGES
        auto issue_next = [&](int x) {
            uint4 *st = stage(x % STAGES);
            if constexpr (FP8) {
                // scales first: a wait for this step's operand copies then
                // also covers them (copies complete in issue order)
                if (sbatch) {
                    if ((ikt & 3) == 0) {
                        if (nbatch > 0) bend[(nbatch - 1) & 1] = x - 1;
                        uint4 *ring = lds_pool + STAGES * STAGE_U4 + (nbatch & 1) * SROWS;
#pragma unroll
                        for (int q = 0; q < SPW; q++) {
                            if ((q * NP + pw) * 64 >= BM + BN) continue;   // wave-uniform
                            const void *src = ssrc[q] ? (const void *)(ssrc[q] + (ikt >> 2) * 16)
                                                      : (const void *)&g_zero_chunk[lane];
                            dma16(src, ring + (q * NP + pw) * 64);
                        }
                        nbatch++;
                    }
                } else {
                    uint4 *sarea = lds_pool + STAGES * STAGE_U4 + (x % STAGES) * SCALE_U4;
#pragma unroll
                    for (int q = 0; q < SPW; q++) {
                        const void *src = ssrc[q] ? (const void *)(ssrc[q] + ikt * 4)
                                                  : (const void *)&g_zero_chunk[lane];
                        dma4(src, sarea + (q * NP + pw) * 16);
                    }
                }
            }
            ta.issue(st, ikt, iklim, pw);
            // bf16 DGRAD: iklim is A's K extent in bytes; B (MN layout) counts K rows
            tb.issue(st + BM * 8, ikt, P::b_klim(iklim), pw);
            if (++ikt == nk_of(iklim)) {
                ip = next_pos(ip);
                seek();
            }
        };
        // issue every step the consumers' progress allows: done = steps they
        // have finished reading; a step's stage is free once the step
        // STAGES before it is done, a batch's ring slot once the batch two
        // before it is
        int issued = 0;
        auto pump = [&](int done, int limit) {
            while (ip < total && issued <= limit) {
                if (FP8 && sbatch && (ikt & 3) == 0 && bend[nbatch & 1] >= done) break;
                issue_next(issued);
                issued++;
            }
        };
        seek();
        pump(0, STAGES - 2);
        for (int G = 0; G < issued; G++) {
            // step G must have landed; at most one step after it is in flight
            // (each step's last IPP copies are its operands, issued last)
            if (issued - 1 - G >= STAGES - 2) wait_vmem<(STAGES - 2) * IPP>();
            else wait_vmem<0>();
            lds_sync();                  // barrier G
            pump(G, G + STAGES - 1);
        }
        return;
    }

    // consumers
    const int wm = wave / WN, wn = wave % WN;
    f32x16 acc[TM][TN];
    auto zero = [&]() {
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++)
#pragma unroll
                for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;
    };
    // acc[i][j][v] holds row (v/4)*8 + (lane/32)*4 + v%4 and column lane%32
    // of the wave's (i, j) 32x32 block
    const int col_l = lane & 31;
    auto row_in = [&](int i, int v) { return wm * WTM + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3); };
    // MXFP8 SwiGLU forward with H' stored quantised: A||B in bf16 as in the
    // plain epilogue; H' rounded to bf16 as that epilogue would store it, then
    // encoded in both MXFP8 layouts (the bytes the both-layout quantiser
    // writes for those values). A wave holds 64 rows x 32 hidden units: one
    // 32-element block of each row (h and the wave's first unit are
    // multiples of 32) and, per 32-row half i, one 32-row block of each
    // unit's column (the tile's rows start a 128-row unit of the group).
    auto swiglu_fwd_mx = [&](const TileC &t, int r0, int j0) {
      if constexpr (FP8 && EPI == MOE_EPI_SWIGLU_FWD) {
        static_assert(TN == 2 && TM == 2, "one hidden-unit block and two 32-row blocks per wave");
        const int h = g.h;
        if (j0 >= h) return;                        // wave-uniform: no unit in range
        uint16_t *AB = reinterpret_cast<uint16_t *>(g.C);
        uint8_t *q1 = reinterpret_cast<uint8_t *>(g.aux_out);
        const int e = t.e;
        // the group's blocks [bb, bb + nb) of the column-block layout
        const int64_t bb = 4 * (int64_t)s_tile[e], nb = 4 * (int64_t)(s_tile[e + 1] - s_tile[e]);
        const int c = j0 + col_l;
        const int half = lane >> 5, qd = (lane & 31) >> 2, rq = lane & 3;
        const int lrow0 = r0 - s_off[e];            // within the group; a multiple of 64
        const bool rows_full = wave_full(r0 + WTM <= t.row_end);
        char *abw = wave_base(AB, r0, j0, 2 * h);
        const uint32_t lab = lane_off<2>(lane, 2 * h);
        // A||B stores and H' as the plain epilogue rounds it; rows past the
        // group's end are the column layout's zero padding
        float hq[TM][16];
        bool nan = false;
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int ro = i * 32 + (v >> 2) * 8 + half * 4 + (v & 3);
                const bool ok = rows_full || r0 + ro < t.row_end;
                const float a = acc[i][0][v], b = acc[i][1][v];
                if (ok) {
                    char *abr = abw + (int64_t)(i * 32 + (v >> 2) * 8 + (v & 3)) * 2 * h * 2;
                    *reinterpret_cast<uint16_t *>(abr + lab) = f32_to_bf16(a);
                    *reinterpret_cast<uint16_t *>(abr + (int64_t)h * 2 + lab) = f32_to_bf16(b);
                }
                hq[i][v] = ok ? bf16_to_f32(f32_to_bf16(silu_f(a) * b)) : 0.f;
                nan |= __builtin_isnan(hq[i][v]);
            }
        // one encoder form for the whole tile (the same bytes either way)
        const bool finite = __ballot(nan) == 0;
        auto enc = [&](float x0, float x1, float x2, float x3, uint32_t sb) {
            return finite ? e4m3x4_finite(x0, x1, x2, x3, sb) : e4m3x4_select(x0, x1, x2, x3, sb);
        };
        // column layout: the lane's unit, rows i*32 .. i*32+31 of the wave
        // (16 in the lane, 16 in lane ^ 32: rows gq*8 + half*4 + 0..3). Two
        // 32-lane swaps hand the lower half of the block's rows to half 0 and
        // the upper half to half 1, so each lane stores 16 contiguous bytes.
#pragma unroll
        for (int i = 0; i < TM; i++) {
            float am = 0.f;
#pragma unroll
            for (int v = 0; v < 16; v++) am = fmaxf(am, fabsf(hq[i][v]));
            const uint32_t sbc = mx_scale_byte(max_xor32(am));
            uint32_t w[4];
#pragma unroll
            for (int gq = 0; gq < 4; gq++)
                w[gq] = enc(hq[i][4 * gq], hq[i][4 * gq + 1], hq[i][4 * gq + 2], hq[i][4 * gq + 3], sbc);
            // half 0 sends rows 16..19, 24..27 and receives 4..7, 12..15; half 1
            // the other way round
            uint32_t got[2];
#pragma unroll
            for (int m = 0; m < 2; m++) {
                const uint32_t send = half ? w[m] : w[m + 2];
                const auto r = __builtin_amdgcn_permlane32_swap(send, send, false, false);
                got[m] = half ? r[0] : r[1];
            }
            const uint4 out = half ? make_uint4(got[0], w[2], got[1], w[3])
                                   : make_uint4(w[0], got[0], w[1], got[1]);
            const int lr = lrow0 + i * 32;
            *reinterpret_cast<uint4 *>(g.aux_out_cols + HpStores::col_q(bb, nb, h, c, lr, half)) = out;
            if (half == 0) g.aux_out_cols_scale[HpStores::col_s(bb, nb, h, c, lr)] = (uint8_t)sbc;
        }
        // row layout: a 4 x 4 transpose inside each quad of lanes gives lane
        // 4 qd + rq the units 4 qd .. 4 qd + 3 of row i*32 + gq*8 + half*4 + rq;
        // that row's block is the lanes qd = 0..7 with the same rq
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int gq = 0; gq < 4; gq++) {
                float x[4] = {hq[i][4 * gq], hq[i][4 * gq + 1], hq[i][4 * gq + 2], hq[i][4 * gq + 3]};
                float p[4];
#pragma unroll
                for (int k = 0; k < 4; k++) p[k] = dpp_move<kDppXor2>(x[k ^ 2]);
#pragma unroll
                for (int k = 0; k < 4; k++)
                    if (((k >> 1) & 1) != ((rq >> 1) & 1)) x[k] = p[k];
#pragma unroll
                for (int k = 0; k < 4; k++) p[k] = dpp_move<kDppXor1>(x[k ^ 1]);
#pragma unroll
                for (int k = 0; k < 4; k++)
                    if ((k & 1) != (rq & 1)) x[k] = p[k];
                float amr = fmaxf(fmaxf(fmaxf(0.f, fabsf(x[0])), fabsf(x[1])),
                                  fmaxf(fabsf(x[2]), fabsf(x[3])));
                amr = fmaxf(amr, dpp_move<kDppRowRor4>(amr));
                amr = fmaxf(amr, dpp_move<kDppRowRor8>(amr));
                const uint32_t sbr = mx_scale_byte(max_xor16(amr));
                const uint32_t w = enc(x[0], x[1], x[2], x[3], sbr);
                const int ro = i * 32 + gq * 8 + half * 4 + rq;
                if (rows_full || r0 + ro < t.row_end) {
                    *reinterpret_cast<uint32_t *>(q1 + HpStores::row_q(r0 + ro, h, j0, qd)) = w;
                    if (qd == 0) g.aux_out_scale[HpStores::row_s(r0 + ro, h, j0)] = (uint8_t)sbr;
                }
            }
      }
    };
    auto epilogue = [&](const TileC &t) {
        if constexpr (MODE == MOE_GG_WGRAD) {
            float *C = reinterpret_cast<float *>(g.C) + (int64_t)t.e * g.M * g.N;
            // the wave's 64x64 part lies inside C: stores without per-element
            // checks, from one per-lane base (row (lane/32)*4, column lane%32)
            const bool full = wave_full(t.m0 + wm * WTM + WTM <= g.M && t.n0 + wn * WTN + WTN <= g.N);
            const char *Cw = wave_base(C, t.m0 + wm * WTM, t.n0 + wn * WTN, g.N);
            const uint32_t lo = lane_off<4>(lane, g.N);
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++) {
                    const int n = t.n0 + wn * WTN + j * 32 + col_l;
                    if constexpr (ACC) {
                        // C += the block, one fp32 add per element; its old
                        // values are all loaded before the first store
                        float old[16];
#pragma unroll
                        for (int v = 0; v < 16; v++) {
                            const int m = t.m0 + row_in(i, v);
                            old[v] = (m < g.M && n < g.N) ? C[(int64_t)m * g.N + n] : 0.f;
                        }
                        wait_vmem<0>();
#pragma unroll
                        for (int v = 0; v < 16; v++) {
                            const int m = t.m0 + row_in(i, v);
                            if (m < g.M && n < g.N) store_f32(C + (int64_t)m * g.N + n, old[v] + acc[i][j][v]);
                        }
                    } else if (full) {
#pragma unroll
                        for (int v = 0; v < 16; v++)
                            store_f32(reinterpret_cast<float *>(
                                          (char *)Cw + ((int64_t)(i * 32 + (v >> 2) * 8 + (v & 3)) * g.N + j * 32) * 4 + lo),
                                      acc[i][j][v]);
                    } else {
#pragma unroll
                        for (int v = 0; v < 16; v++) {
                            const int m = t.m0 + row_in(i, v);
                            if (m < g.M && n < g.N) store_f32(C + (int64_t)m * g.N + n, acc[i][j][v]);
                        }
                    }
                }
        } else if constexpr (EPI == MOE_EPI_SWIGLU_FWD) {
            uint16_t *AB = reinterpret_cast<uint16_t *>(g.C);
            uint16_t *HP = reinterpret_cast<uint16_t *>(g.aux_out);
            const int h = g.h;
            const int r0 = t.row0 + wm * WTM, j0 = t.nt * (BN / 2) + wn * (WTN / 2);
            if constexpr (FP8) {
                if (g.aux_out_scale != nullptr) {       // uniform: a kernel argument
                    swiglu_fwd_mx(t, r0, j0);
                    return;
                }
            }
            if (wave_full(r0 + WTM <= t.row_end && j0 + WTN / 2 <= h)) {
                // the wave's rows and hidden units are all in range
                char *abw = wave_base(AB, r0, j0, 2 * h);
                char *hpw = wave_base(HP, r0, j0, h);
                const uint32_t lab = lane_off<2>(lane, 2 * h), lhp = lane_off<2>(lane, h);
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int j = 0; j < TN / 2; j++)
#pragma unroll
                        for (int v = 0; v < 16; v++) {
                            const int64_t ro = i * 32 + (v >> 2) * 8 + (v & 3);
                            const float a = acc[i][j][v], b = acc[i][j + TN / 2][v];
                            char *abr = abw + (ro * 2 * h + j * 32) * 2;
                            *reinterpret_cast<uint16_t *>(abr + lab) = f32_to_bf16(a);
                            *reinterpret_cast<uint16_t *>(abr + (int64_t)h * 2 + lab) = f32_to_bf16(b);
                            *reinterpret_cast<uint16_t *>(hpw + (ro * h + j * 32) * 2 + lhp) =
                                f32_to_bf16(silu_f(a) * b);
                        }
                return;
            }
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN / 2; j++) {
                    const int jj = j0 + j * 32 + col_l;
#pragma unroll
                    for (int v = 0; v < 16; v++) {
                        const int grow = t.row0 + row_in(i, v);
                        if (grow < t.row_end && jj < h) {
                            const float a = acc[i][j][v], b = acc[i][j + TN / 2][v];
                            uint16_t *abr = AB + (int64_t)grow * 2 * h;
                            abr[jj] = f32_to_bf16(a);
                            abr[h + jj] = f32_to_bf16(b);
                            HP[(int64_t)grow * h + jj] = f32_to_bf16(silu_f(a) * b);
                        }
                    }
                }
        } else {
            uint16_t *C = reinterpret_cast<uint16_t *>(g.C);
            const int r0 = t.row0 + wm * WTM, n0 = t.n0 + wn * WTN;
            if (wave_full(r0 + WTM <= t.row_end && n0 + WTN <= g.N)) {
                char *cw = wave_base(C, r0, n0, g.N);
                const uint32_t lo = lane_off<2>(lane, g.N);
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int j = 0; j < TN; j++)
#pragma unroll
                        for (int v = 0; v < 16; v++)
                            *reinterpret_cast<uint16_t *>(
                                cw + ((int64_t)(i * 32 + (v >> 2) * 8 + (v & 3)) * g.N + j * 32) * 2 + lo) =
                                f32_to_bf16(acc[i][j][v]);
                return;
            }
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++) {
                    const int n = n0 + j * 32 + col_l;
#pragma unroll
                    for (int v = 0; v < 16; v++) {
                        const int grow = t.row0 + row_in(i, v);
                        if (grow < t.row_end && n < g.N) C[(int64_t)grow * g.N + n] = f32_to_bf16(acc[i][j][v]);
                    }
                }
        }
    };
    // one K step from buffer st: fragments double-buffered in registers
    auto step = [&](int st) {
        const uint4 *sa = stage(st);
        const uint4 *sb = sa + BM * 8;
        bf16x8 fa[2][TM], fb[2][TN];
#pragma unroll
        for (int i = 0; i < TM; i++) fa[0][i] = AT::frag(sa, wm * WTM + i * 32, 0, lane);
#pragma unroll
        for (int j = 0; j < TN; j++) fb[0][j] = BT::frag(sb, wn * WTN + j * 32, 0, lane);
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
            const int cb = kk & 1, nb2 = cb ^ 1;
            if constexpr (MODE != MOE_GG_WGRAD) {
                // row GEMMs: one fragment read of the next slice between two MFMAs
#pragma unroll
                for (int t = 0; t < TM * TN; t++) {
                    if (kk + 1 < 4) {
                        if (t < TM) fa[nb2][t] = AT::frag(sa, wm * WTM + t * 32, kk + 1, lane);
                        else if (t < TM + TN)
                            fb[nb2][t - TM] = BT::frag(sb, wn * WTN + (t - TM) * 32, kk + 1, lane);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    acc[t / TN][t % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        fa[cb][t / TN], fb[cb][t % TN], acc[t / TN][t % TN], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                if (kk + 1 < 4) {
#pragma unroll
                    for (int i = 0; i < TM; i++) fa[nb2][i] = AT::frag(sa, wm * WTM + i * 32, kk + 1, lane);
#pragma unroll
                    for (int j = 0; j < TN; j++) fb[nb2][j] = BT::frag(sb, wn * WTN + j * 32, kk + 1, lane);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int j = 0; j < TN; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cb][i], fb[cb][j], acc[i][j], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // one MXFP8 K step (128 bytes: two 64-wide slices) from buffer st; the
    // scale words from the ring slot of its batch (word kt % 4) or from the
    // step's own area
    auto step8 = [&](int st, int kt, int slot) {
      if constexpr (FP8) {
        const uint4 *sa = stage(st);
        const uint4 *sb = sa + BM * 8;
        uint32_t swa[TM], swb[TN];
        if (sbatch) {
            const uint32_t *rw =
                reinterpret_cast<const uint32_t *>(lds_pool + STAGES * STAGE_U4 + slot * SROWS);
            const int w = kt & 3;
#pragma unroll
            for (int i = 0; i < TM; i++) swa[i] = rw[(wm * WTM + i * 32 + (lane & 31)) * 4 + w];
#pragma unroll
            for (int j = 0; j < TN; j++) swb[j] = rw[(BM + wn * WTN + j * 32 + (lane & 31)) * 4 + w];
        } else {
            const uint32_t *sw =
                reinterpret_cast<const uint32_t *>(lds_pool + STAGES * STAGE_U4 + st * SCALE_U4);
#pragma unroll
            for (int i = 0; i < TM; i++) swa[i] = sw[wm * WTM + i * 32 + (lane & 31)];
#pragma unroll
            for (int j = 0; j < TN; j++) swb[j] = sw[BM + wn * WTN + j * 32 + (lane & 31)];
        }
        i32x8 fa[2][TM], fb[2][TN];
#pragma unroll
        for (int i = 0; i < TM; i++) fa[0][i] = AT::frag8(sa, wm * WTM + i * 32, 0, lane);
#pragma unroll
        for (int j = 0; j < TN; j++) fb[0][j] = BT::frag8(sb, wn * WTN + j * 32, 0, lane);
#pragma unroll
        for (int sl = 0; sl < 2; sl++) {
            // lane l supplies the scale of (row l % 32, block 2 sl + l / 32)
            const int sh = 8 * (2 * sl + (lane >> 5));
            if (MODE != MOE_GG_WGRAD && sl == 0) {
                // row GEMMs: the reads of slice 1 go one between each two MFMAs
#pragma unroll
                for (int t = 0; t < TM * TN; t++) {
                    if (t < TM) fa[1][t] = AT::frag8(sa, wm * WTM + t * 32, 1, lane);
                    else if (t < TM + TN) fb[1][t - TM] = BT::frag8(sb, wn * WTN + (t - TM) * 32, 1, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    const int i = t / TN, j = t % TN;
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fa[0][i], fb[0][j], acc[i][j], 0, 0, 0, (int)((swa[i] >> sh) & 0xff), 0,
                        (int)((swb[j] >> sh) & 0xff));
                    __builtin_amdgcn_sched_barrier(0);
                }
                continue;
            }
            if (sl == 0) {
#pragma unroll
                for (int i = 0; i < TM; i++) fa[1][i] = AT::frag8(sa, wm * WTM + i * 32, 1, lane);
#pragma unroll
                for (int j = 0; j < TN; j++) fb[1][j] = BT::frag8(sb, wn * WTN + j * 32, 1, lane);
            }
            __builtin_amdgcn_sched_barrier(0);   // keep the prefetch above the MFMAs
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fa[sl][i], fb[sl][j], acc[i][j], 0, 0, 0, (int)((swa[i] >> sh) & 0xff), 0,
                        (int)((swb[j] >> sh) & 0xff));
            __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    int G = 0, nbatch = 0;
    for (int pos = worker; pos < total; pos = next_pos(pos)) {
        const TileC t = decode(pos);
        const int nk = nk_of(t.klim);
        if (ACC && nk == 0) continue;              // accumulating: an empty group leaves C as it is
        zero();
        for (int kt = 0; kt < nk; kt++, G++) {
            lds_sync();                             // barrier G: step G is in buffer G % STAGES
            if constexpr (FP8) {
                if (sbatch && (kt & 3) == 0) nbatch++;
                step8(G % STAGES, kt, (nbatch - 1) & 1);
            } else {
                step(G % STAGES);
            }
        }
        epilogue(t);                                // its stores drain while the next tile runs
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
        load_offsets(g.offsets, E, s_off);
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
                    if (bc >= 0) C[bc] = g.accumulate ? C[bc] + acc[i][j] : acc[i][j];
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

// Tile configuration of gg_mfma (the SwiGLU backward): rows x columns of the
// output tile, the wave grid, LDS stages and workgroups per CU of the
// persistent grid.
#ifndef MOE_ROW_BM
#define MOE_ROW_BM 128      // FWD / DGRAD: routed rows per tile
#endif
#ifndef MOE_ROW_BN
#define MOE_ROW_BN 256
#endif
#ifndef MOE_ROW_STAGES
#define MOE_ROW_STAGES 3
#endif
#ifndef MOE_ROW_OCC
#define MOE_ROW_OCC 1
#endif
#ifndef MOE_ROW_WPE
#define MOE_ROW_WPE 2
#endif

#ifndef MOE_ROW_WM
#define MOE_ROW_WM 2
#endif
#ifndef MOE_ROW_WN
#define MOE_ROW_WN 4
#endif

// gg_ws, bf16 and MXFP8: 8 consumer waves (2 x 4, 64 x 64 each) and 4
// producer waves on the same 128 x 256 tiles and 3 stages as gg_mfma
constexpr int kWsBM = 128, kWsBN = 256, kWsWM = 2, kWsWN = 4, kWsNP = 4, kWsStages = 3;

template <int MODE, int EPI, bool FP8>
static void launch_ws(const GemmArgs &a, hipStream_t s) {
    const int grid = (num_cus() + 7) / 8 * 8;
    constexpr int threads = (kWsWM * kWsWN + kWsNP) * 64;
    if constexpr (MODE == MOE_GG_WGRAD) {
        if (a.accumulate) {
            gg_ws<MODE, EPI, FP8, kWsBM, kWsBN, kWsWM, kWsWN, kWsNP, kWsStages, true>
                <<<grid, threads, 0, s>>>(a);
            return;
        }
    }
    gg_ws<MODE, EPI, FP8, kWsBM, kWsBN, kWsWM, kWsWN, kWsNP, kWsStages><<<grid, threads, 0, s>>>(a);
}

// A build with -DMOE_GG_MFMA_ALL=1 runs every role on gg_mfma (every wave
// copies and multiplies), the kernel gg_ws was split from: the same tiles,
// schedules and MFMA order, so the same bits, for comparing the two.
#ifndef MOE_GG_MFMA_ALL
#define MOE_GG_MFMA_ALL 0
#endif

template <int MODE, int EPI, bool FP8>
static void launch_mfma(const GemmArgs &a, hipStream_t s) {
    // every role on the split-role kernel except the SwiGLU backward, whose
    // epilogue stages dH' through the LDS stage buffers and reads a, b as
    // 16-byte rows (measured 2 % faster than a register-direct form)
    if constexpr (EPI != MOE_EPI_SWIGLU_BWD && !MOE_GG_MFMA_ALL) {
        launch_ws<MODE, EPI, FP8>(a, s);
    } else {
        const int grid = (num_cus() * MOE_ROW_OCC + 7) / 8 * 8;
        gg_mfma<MODE, EPI, FP8, MOE_ROW_BM, MOE_ROW_BN, MOE_ROW_WM, MOE_ROW_WN, MOE_ROW_STAGES,
                MOE_ROW_WPE><<<grid, MOE_ROW_WM * MOE_ROW_WN * 64, 0, s>>>(a);
    }
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
    a.a_scale = d->a_scale; a.b_scale = d->b_scale;
    a.E = d->n_groups;
    a.h = d->epilogue == MOE_EPI_SWIGLU_FWD ? d->N / 2 : d->N;
    a.accumulate = d->accumulate;
    a.aux_out_scale = d->aux_out_scale;
    a.aux_out_cols = d->aux_out_cols;
    a.aux_out_cols_scale = d->aux_out_cols_scale;
    // the comparison build's gg_mfma has no quantising SwiGLU epilogue
    if (MOE_GG_MFMA_ALL && d->aux_out_scale) return MOE_ERR_DTYPE;
#define GO(MODE, EPI)                                                          \
    (d->dtype == MOE_BF16    ? launch_mfma<MODE, EPI, false>(a, s)             \
     : d->dtype == MOE_MXFP8 ? launch_mfma<MODE, EPI, true>(a, s)              \
                             : launch_f32<MODE, EPI>(a, s))
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

// ---------------------------------------------------------------------------
// host walk of the copies (moe_gemm_copy_walk)

namespace {

struct Walker {
    moe_copy_walk *w;
    void read(int op, int64_t off, int64_t bytes) {
        w->copies++;
        if (off < w->lowest[op]) w->lowest[op] = off;
        if (off + bytes > w->end[op]) w->end[op] = off + bytes;
        if (w->first_bad < 0 && (off < 0 || off + bytes > w->extent[op])) {
            w->first_bad = op;
            w->bad_offset = off;
            w->bad_bytes = bytes;
        }
    }
    void zero(int64_t n) {
        w->copies += n;
        w->zero_copies += n;
    }
};

// One operand of one tile: every wave, lane and instruction of the copy
// over nk steps. A source is affine in the step with a non-negative stride,
// so its lowest and highest addresses are at the first and at the last
// step that copies real data; the steps in between are counted.
template <typename Geom, typename OffFn>
void walk_operand(Walker &wk, int op, int nwaves, int64_t origin, int64_t kstride, int nk,
                  int klim, OffFn voff_of) {
    for (int wave = 0; wave < nwaves; wave++)
        for (int lane = 0; lane < 64; lane++)
            for (int i = 0; i < Geom::IPW; i++) {
                const int64_t base = origin + voff_of(i, wave, lane);
                int last = -1, n_in = 0;
                for (int kt = nk - 1; kt >= 0 && kt >= nk - 2; kt--)
                    if (Geom::in_k(i, wave, lane, kt, klim)) { last = kt; break; }
                // only the last step can be partial: steps before it copy real data
                if (last >= 0) n_in = last + 1;
                if (n_in > 0) {
                    wk.read(op, base, 16);
                    if (last > 0) wk.read(op, base + (int64_t)last * kstride, 16);
                    wk.w->copies += n_in - (last > 0 ? 2 : 1);
                }
                wk.zero(nk - n_in);
            }
}

template <int MODE, int EPI, bool FP8, int BM, int BN, int WM, int WN, int NCOPY>
void walk_kernel(const GemmArgs &g, const int32_t *off, moe_copy_walk *w) {
    using P = TilePlan<MODE, EPI, FP8, BM, BN, BN / WN>;
    using AG = CopyGeom<BM, P::A_KL, NCOPY>;
    using BG = CopyGeom<BN, P::B_KL, NCOPY>;
    // MXFP8: SPW scale rows per lane of the NCOPY copying waves
    constexpr int SPW = FP8 ? (BM + BN + NCOPY * 64 - 1) / (NCOPY * 64) : 0;
    Walker wk{w};
    const int E = g.E;
    const int n_tiles = P::n_tiles(g);
    const bool sbatch = P::scale_batched(g);
    std::vector<int32_t> blk(E + 1, 0);
    for (int e = 0; e < E; e++) blk[e + 1] = blk[e] + (off[e + 1] - off[e] + 127) / 128;
    auto walk_tile = [&](const TileC &t) {
        const int nk = P::nk_of(t.klim);
        if (nk == 0) return;
        if constexpr (P::A_KL) {
            walk_operand<AG>(wk, 0, NCOPY, P::a_origin(g, t), AG::kstride(0), nk, t.klim,
                             [&](int i, int wave, int lane) {
                                 return (int64_t)AG::kl_off(i, wave, lane, [&](int r) { return P::a_row_off(g, t, r); });
                             });
        } else {
            walk_operand<AG>(wk, 0, NCOPY, P::a_origin(g, t), AG::kstride(P::a_ld(g)), nk, t.klim,
                             [&](int i, int wave, int lane) {
                                 return (int64_t)AG::mn_off(i, wave, lane, P::a_ld(g), P::a_cvalid(g, t));
                             });
        }
        const int bk = P::b_klim(t.klim);
        if constexpr (P::B_KL) {
            walk_operand<BG>(wk, 1, NCOPY, P::b_origin(g, t), BG::kstride(0), nk, bk,
                             [&](int i, int wave, int lane) {
                                 return (int64_t)BG::kl_off(i, wave, lane, [&](int n) { return P::b_row_off(g, t, n); });
                             });
        } else {
            walk_operand<BG>(wk, 1, NCOPY, P::b_origin(g, t), BG::kstride(P::b_ld(g)), nk, bk,
                             [&](int i, int wave, int lane) {
                                 return (int64_t)BG::mn_off(i, wave, lane, P::b_ld(g), P::b_cvalid(g, t));
                             });
        }
        if constexpr (FP8) {
            for (int q = 0; q < SPW; q++)
                for (int wave = 0; wave < NCOPY; wave++) {
                    if (sbatch && (q * NCOPY + wave) * 64 >= BM + BN) continue;
                    for (int lane = 0; lane < 64; lane++) {
                        const int sr = (q * NCOPY + wave) * 64 + lane;
                        const int64_t o = P::scale_off(g, t, sr);
                        const int op = 2 + (P::scale_operand(sr) == 1 ? 1 : 0);
                        const int n = sbatch ? (nk + 3) / 4 : nk;   // batched: steps 0, 4, 8, ...
                        if (o < 0) { wk.zero(n); continue; }
                        const int64_t step = sbatch ? 16 : 4;
                        wk.read(op, o, step);
                        if (n > 1) wk.read(op, o + (int64_t)(n - 1) * step, step);
                        w->copies += n - (n > 1 ? 2 : 1);
                    }
                }
        }
    };
    if constexpr (MODE == MOE_GG_WGRAD) {
        const int mtiles = (g.M + BM - 1) / BM;
        for (int e = 0; e < E; e++)
            for (int mi = 0; mi < mtiles; mi++)
                for (int nt = 0; nt < n_tiles; nt++) walk_tile(P::wgrad_tile(off, blk.data(), e, mi, nt));
    } else {
        for (int e = 0; e < E; e++) {
            const int mt = (off[e + 1] - off[e] + BM - 1) / BM;
            for (int m = 0; m < mt; m++)
                for (int nt = 0; nt < n_tiles; nt++) walk_tile(P::row_tile(g, off, e, m, nt));
        }
    }
}

template <int MODE, int EPI>
void walk_mode(const GemmArgs &a, const int32_t *off, bool fp8, moe_copy_walk *w) {
    // the SwiGLU backward runs on gg_mfma (every wave copies), the rest on
    // the split-role kernel (its producer waves copy)
    if constexpr (EPI == MOE_EPI_SWIGLU_BWD) {
        if (fp8)
            walk_kernel<MODE, EPI, true, MOE_ROW_BM, MOE_ROW_BN, MOE_ROW_WM, MOE_ROW_WN,
                        MOE_ROW_WM * MOE_ROW_WN>(a, off, w);
        else
            walk_kernel<MODE, EPI, false, MOE_ROW_BM, MOE_ROW_BN, MOE_ROW_WM, MOE_ROW_WN,
                        MOE_ROW_WM * MOE_ROW_WN>(a, off, w);
    } else {
        if (fp8) walk_kernel<MODE, EPI, true, kWsBM, kWsBN, kWsWM, kWsWN, kWsNP>(a, off, w);
        else walk_kernel<MODE, EPI, false, kWsBM, kWsBN, kWsWM, kWsWN, kWsNP>(a, off, w);
    }
}

}  // namespace

// the launch configuration of gemm_launch, walked on the host
// Every store of the MXFP8 SwiGLU forward's quantised H' (the four outputs
// as operands 0..3 of the walk), over the tiles gg_ws computes: group e's
// 128-row units times the n-tiles of BN / 2 hidden units, each consumer
// wave and lane, with the offsets the epilogue uses (HpStores).
moe_status gemm_hp_store_walk(const moe_gemm_desc *d, const int32_t *off, moe_copy_walk *w) {
    constexpr int BM = kWsBM, BN = kWsBN, WM = kWsWM, WN = kWsWN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    static_assert(WTM == 64 && WTN == 64, "the epilogue's wave tile");
    const int h = d->N / 2, E = d->n_groups;
    w->copies = w->zero_copies = 0;
    for (int i = 0; i < 4; i++) {
        w->lowest[i] = INT64_MAX;
        w->end[i] = 0;
    }
    w->first_bad = -1;
    w->bad_offset = w->bad_bytes = 0;
    Walker wk{w};
    const int n_tiles = (h + BN / 2 - 1) / (BN / 2);
    int64_t ub = 0;                                   // 128-row units before group e
    for (int e = 0; e < E; e++) {
        const int rows_e = off[e + 1] - off[e];
        const int units = (rows_e + BM - 1) / BM;
        const int64_t bb = 4 * ub, nb = 4 * (int64_t)units;
        for (int mt = 0; mt < units; mt++)
            for (int nt = 0; nt < n_tiles; nt++)
                for (int wm = 0; wm < WM; wm++)
                    for (int wn = 0; wn < WN; wn++) {
                        const int j0 = nt * (BN / 2) + wn * (WTN / 2);
                        if (j0 >= h) continue;
                        const int r0 = off[e] + mt * BM + wm * WTM;
                        const int lrow0 = r0 - off[e];
                        for (int lane = 0; lane < 64; lane++) {
                            const int half = lane >> 5, qd = (lane & 31) >> 2, rq = lane & 3;
                            const int c = j0 + (lane & 31);
                            for (int i = 0; i < 2; i++) {
                                const int lr = lrow0 + i * 32;
                                wk.read(2, HpStores::col_q(bb, nb, h, c, lr, half), 16);
                                if (half == 0) wk.read(3, HpStores::col_s(bb, nb, h, c, lr), 1);
                                for (int gq = 0; gq < 4; gq++) {
                                    const int64_t row = r0 + i * 32 + gq * 8 + half * 4 + rq;
                                    if (row >= off[e + 1]) continue;
                                    wk.read(0, HpStores::row_q(row, h, j0, qd), 4);
                                    if (qd == 0) wk.read(1, HpStores::row_s(row, h, j0), 1);
                                }
                            }
                        }
                    }
        ub += units;
    }
    return MOE_OK;
}

moe_status gemm_copy_walk(const moe_gemm_desc *d, const int32_t *off, moe_copy_walk *w) {
    GemmArgs a{};
    a.rows = d->rows; a.M = d->M; a.N = d->N; a.K = d->K;
    a.E = d->n_groups;
    a.h = d->epilogue == MOE_EPI_SWIGLU_FWD ? d->N / 2 : d->N;
    w->copies = w->zero_copies = 0;
    for (int i = 0; i < 4; i++) {
        w->lowest[i] = INT64_MAX;
        w->end[i] = 0;
    }
    w->first_bad = -1;
    w->bad_offset = w->bad_bytes = 0;
    const bool fp8 = d->dtype == MOE_MXFP8;
    if (d->mode == MOE_GG_FWD) {
        if (d->epilogue == MOE_EPI_SWIGLU_FWD) walk_mode<MOE_GG_FWD, MOE_EPI_SWIGLU_FWD>(a, off, fp8, w);
        else walk_mode<MOE_GG_FWD, MOE_EPI_NONE>(a, off, fp8, w);
    } else if (d->mode == MOE_GG_DGRAD) {
        if (d->epilogue == MOE_EPI_SWIGLU_BWD) walk_mode<MOE_GG_DGRAD, MOE_EPI_SWIGLU_BWD>(a, off, fp8, w);
        else walk_mode<MOE_GG_DGRAD, MOE_EPI_NONE>(a, off, fp8, w);
    } else {
        walk_mode<MOE_GG_WGRAD, MOE_EPI_NONE>(a, off, fp8, w);
    }
    return MOE_OK;
}

}  // namespace moe
