// route.hip -- GPU-resident top-k routing and its metadata.
//
// The routing decisions and the metadata derived from them (all-to-all split
// sizes, per-expert group sizes) are computed and kept on the GPU, so the host
// only enqueues work (Ai2 Olmo-core 3, kongchang.com, "routing is a systems
// problem"; bytechap.com, "How it works").
//
// Three kernels, no host round trip and no order-dependent atomics:
//  1. route_select: one workgroup per 64-token chunk, G = 8 lanes per token.
//     Each lane reads every G-th 16-byte piece of its token's logits (all
//     loads in flight at once) and keeps their top k (descending fp32 logit,
//     equal logits -> lower index): each piece is sorted by a four-input
//     sorting network and bitonic-merged into the lane's list, and the G
//     lists of a token are bitonic-merged across lanes with DPP moves. Lane j
//     of the token owns selection j; the gates are the softmax over the k
//     selected logits. Each wave ranks its (token, slot) pairs inside the
//     chunk (rank = number of lanes below with the same expert, found with
//     one ballot per bit of the expert index); the waves' counts are
//     combined in LDS. Per-chunk expert counts go to the workspace.
//  2. route_scan: one workgroup per expert scans its counts over chunks
//     (exclusive), giving each chunk its base inside the expert's group, and
//     the expert's total.
//  3. route_place: scans the E totals (in LDS) into offsets / tile offsets
//     and writes token_pos = offsets[e] + chunk base + rank and the inverse
//     maps sorted_token / sorted_slot.
#include <mutex>

#include "common.h"

namespace moe {

constexpr int kChunk = 64;      // tokens per chunk
constexpr int kMaxE = 256;

// A candidate is (logit v, expert i); i < 0 marks an empty slot.
// (v, i) ranks above (bv, bi): it is not empty and (bv, bi) is, or its logit
// is larger, or the logits are equal (IEEE comparison, so -0 and +0 are
// equal) and its index is lower. Bitwise, not short-circuit, so that it
// compiles to selects.
MOE_DEV bool route_better(float v, int i, float bv, int bi) {
    return (i >= 0) & ((bi < 0) | (v > bv) | ((v == bv) & (i < bi)));
}

// compare-exchange: afterwards (v[a], i[a]) ranks at or above (v[b], i[b])
template <int N>
MOE_DEV void route_cx(float (&v)[N], int (&i)[N], int a, int b) {
    const bool sw = route_better(v[b], i[b], v[a], i[a]);
    const float va = v[a], vb = v[b];
    const int ia = i[a], ib = i[b];
    v[a] = sw ? vb : va; i[a] = sw ? ib : ia;
    v[b] = sw ? va : vb; i[b] = sw ? ia : ib;
}

// (bv, bi) <- the best KP of the sorted lists (bv, bi) and (ov, oi), sorted.
// Pairing slot j of one list with slot KP-1-j of the other and keeping the
// better of each pair leaves exactly the best KP, as a bitonic sequence,
// which log2(KP) rounds of compare-exchanges sort (Batcher's bitonic merge).
template <int KP>
MOE_DEV void route_merge(float (&bv)[KP], int (&bi)[KP], const float (&ov)[KP], const int (&oi)[KP]) {
#pragma unroll
    for (int j = 0; j < KP; j++) {
        const bool t = route_better(ov[KP - 1 - j], oi[KP - 1 - j], bv[j], bi[j]);
        bv[j] = t ? ov[KP - 1 - j] : bv[j];
        bi[j] = t ? oi[KP - 1 - j] : bi[j];
    }
#pragma unroll
    for (int st = KP / 2; st > 0; st >>= 1)
#pragma unroll
        for (int j = 0; j < KP; j++)
            if ((j & st) == 0) route_cx<KP>(bv, bi, j, j + st);
}

// merge four candidates (experts e0 .. e0+3) into the sorted list
template <int KP>
MOE_DEV void route_take4(float (&bv)[KP], int (&bi)[KP], float4 x, int e0) {
    float v[4] = {x.x, x.y, x.z, x.w};
    int i[4] = {e0, e0 + 1, e0 + 2, e0 + 3};
    // sorting network on four (Knuth's five comparators)
    route_cx<4>(v, i, 0, 1); route_cx<4>(v, i, 2, 3);
    route_cx<4>(v, i, 0, 2); route_cx<4>(v, i, 1, 3);
    route_cx<4>(v, i, 1, 2);
    float ov[KP];
    int oi[KP];
#pragma unroll
    for (int j = 0; j < KP; j++) {
        ov[j] = j < 4 ? v[j < 4 ? j : 0] : -INFINITY;
        oi[j] = j < 4 ? i[j < 4 ? j : 0] : -1;
    }
    route_merge<KP>(bv, bi, ov, oi);
}

// merge one candidate into the sorted list
template <int KP>
MOE_DEV void route_take1(float (&bv)[KP], int (&bi)[KP], float x, int e) {
    float ov[KP];
    int oi[KP];
#pragma unroll
    for (int j = 0; j < KP; j++) { ov[j] = j ? -INFINITY : x; oi[j] = j ? -1 : e; }
    route_merge<KP>(bv, bi, ov, oi);
}

// lane moves inside a row of lanes (DPP, no LDS): xor 1 and xor 2 within
// quads, then the half-row mirror. Applied in this order, each pairs every
// lane with one holding the other half of the lists merged so far, so after
// the three rounds all 8 lanes of an aligned group hold the merge of all 8.

template <int KP, int CTRL>
MOE_DEV void route_merge_lanes(float (&bv)[KP], int (&bi)[KP]) {
    float ov[KP];
    int oi[KP];
#pragma unroll
    for (int j = 0; j < KP; j++) {
        ov[j] = __int_as_float(dpp_move<CTRL>(__float_as_int(bv[j])));
        oi[j] = dpp_move<CTRL>(bi[j]);
    }
    route_merge<KP>(bv, bi, ov, oi);
}

template <int K>
__global__ __launch_bounds__(kChunk * 8) void route_select(const float *__restrict__ logits, int64_t T,
                                                          int E, int k, int32_t *__restrict__ topk_idx,
                                                          float *__restrict__ topk_gate,
                                                          int32_t *__restrict__ rank_out,
                                                          int32_t *__restrict__ chunk_counts) {
    constexpr int G = 8;                                // lanes per token
    constexpr int KP = K <= 1 ? 1 : K <= 2 ? 2 : K <= 4 ? 4 : 8;   // list length (power of two)
    constexpr int NT = kChunk * G, NWAVE = NT / 64;
    constexpr int NV = kMaxE / 4 / G;                  // 16-byte pieces of a token row per lane (E = 256)
    __shared__ int32_t cnt[NWAVE][kMaxE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t chunk = blockIdx.x;
    const int64_t t0 = chunk * kChunk;
    const int ntok = (int)min<int64_t>(kChunk, T - t0);

    for (int i = tid; i < NWAVE * kMaxE; i += NT) (&cnt[0][0])[i] = 0;

    // lane `part` of token `tok` holds the logits of experts 4(part + G c) ..
    // + 3, c = 0, 1, ...: the token's G lanes read its row in 16-byte pieces,
    // every load in flight before the first comparison
    const int tok = tid / G, part = tid % G;
    const bool active = tok < ntok;
    float bv[KP];
    int bi[KP];
#pragma unroll
    for (int j = 0; j < KP; j++) { bv[j] = -INFINITY; bi[j] = -1; }
    if (active) {
        const float *row = logits + (t0 + tok) * E;
        if ((E & 3) == 0) {
            float4 v[NV];
#pragma unroll
            for (int c = 0; c < NV; c++) {
                const int e0 = 4 * (part + G * c);
                if (e0 < E) v[c] = *reinterpret_cast<const float4 *>(row + e0);
            }
#pragma unroll
            for (int c = 0; c < NV; c++) {
                const int e0 = 4 * (part + G * c);
                if (e0 < E) route_take4<KP>(bv, bi, v[c], e0);
            }
        } else {
            for (int e = part; e < E; e += G) route_take1<KP>(bv, bi, row[e], e);
        }
    }
    // merge the G = 8 lists of the token (an aligned group of 8 lanes)
    route_merge_lanes<KP, kDppXor1>(bv, bi);
    route_merge_lanes<KP, kDppXor2>(bv, bi);
    route_merge_lanes<KP, kDppHalfMirror>(bv, bi);

    // this lane's selection: slot `part` of its token; gates = softmax over
    // the k selected logits
    const bool owns = active && part < K;
    int my_e = -1;
    float my_g = 0.f;
    {
        const float m = bv[0];
        float z = 0.f, mine = 0.f;
#pragma unroll
        for (int j = 0; j < K; j++) {
            const float ex = expf(bv[j] - m);
            z += ex;
            if (j == part) { mine = ex; my_e = bi[j]; }
        }
        my_g = mine / z;
    }
    if (owns) {
        const int64_t t = t0 + tok;
        topk_idx[t * k + part] = my_e;
        topk_gate[t * k + part] = my_g;
    }
    __syncthreads();                                   // counts zeroed

    // rank inside the wave: lanes below with the same expert (the lanes of
    // one token hold distinct experts, so they are exactly earlier tokens).
    // The lanes with the same expert are found bit by bit of the expert
    // index: one ballot per bit.
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const uint64_t own_m = __ballot(owns);
    uint64_t same = own_m;
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    for (int b = 0; b < nbits; b++) {
        const bool bit = (my_e >> b) & 1;
        const uint64_t mb = __ballot(owns && bit);
        same &= bit ? mb : (own_m & ~mb);
    }
    int rank = __popcll(same & below);
    if (owns && rank == 0) cnt[wave][my_e] = __popcll(same);   // one writer per expert
    __syncthreads();
    if (owns) {
#pragma unroll
        for (int w = 0; w < NWAVE; w++)
            if (w < wave) rank += cnt[w][my_e];
        rank_out[(t0 + tok) * k + part] = rank;
    }
    for (int e = tid; e < E; e += NT) {
        int32_t c = 0;
#pragma unroll
        for (int w = 0; w < NWAVE; w++) c += cnt[w][e];
        chunk_counts[chunk * E + e] = c;
    }
}

// One workgroup per expert: exclusive scan of its per-chunk counts (in place)
// and the expert's total.
__global__ __launch_bounds__(256) void route_scan(int32_t *__restrict__ chunk_counts,
                                                  int64_t nchunks, int E,
                                                  int32_t *__restrict__ counts) {
    __shared__ int32_t part[256];
    const int e = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t per = (nchunks + 255) / 256;
    const int64_t c0 = min<int64_t>(nchunks, tid * per), c1 = min<int64_t>(nchunks, c0 + per);
    int32_t s = 0;
    for (int64_t c = c0; c < c1; c++) s += chunk_counts[c * E + e];
    part[tid] = s;
    __syncthreads();
    // Hillis-Steele inclusive scan over 256 partial sums
    for (int o = 1; o < 256; o <<= 1) {
        int32_t v = tid >= o ? part[tid - o] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int32_t run = part[tid] - s;   // exclusive
    for (int64_t c = c0; c < c1; c++) {
        int32_t v = chunk_counts[c * E + e];
        chunk_counts[c * E + e] = run;
        run += v;
    }
    if (tid == 255) counts[e] = part[255];
}

// offsets / tile offsets (every block recomputes them in LDS; block 0 stores
// them) and the final positions.
__global__ __launch_bounds__(256) void route_place(
    const int32_t *__restrict__ counts, const int32_t *__restrict__ chunk_base, int64_t T, int E,
    int k, int tile_m, const int32_t *__restrict__ topk_idx, int32_t *__restrict__ token_pos,
    int32_t *__restrict__ sorted_token, int32_t *__restrict__ sorted_slot,
    int32_t *__restrict__ offsets, int32_t *__restrict__ tile_offsets) {
    __shared__ int32_t off[kMaxE + 1];
    __shared__ int32_t toff[kMaxE + 1];
    const int tid = threadIdx.x;
    int32_t c = tid < E ? counts[tid] : 0;
    int32_t tc = (c + tile_m - 1) / tile_m;
    off[tid + 1] = c;
    toff[tid + 1] = tc;
    if (tid == 0) { off[0] = 0; toff[0] = 0; }
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        int32_t v = tid >= o ? off[tid + 1 - o] : 0;
        int32_t w = tid >= o ? toff[tid + 1 - o] : 0;
        __syncthreads();
        off[tid + 1] += v;
        toff[tid + 1] += w;
        __syncthreads();
    }
    if (blockIdx.x == 0) {
        for (int e = tid; e <= E; e += 256) {
            offsets[e] = off[e];
            tile_offsets[e] = toff[e];
        }
    }
    const int64_t t = (int64_t)blockIdx.x * 256 + tid;
    if (t >= T) return;
    const int64_t chunk = t / kChunk;
    const int64_t R = T * k;
    for (int j = 0; j < k; j++) {
        const int e = topk_idx[t * k + j];
        if ((unsigned)e >= (unsigned)E) continue;      // never for route_select's output
        const int32_t p = off[e] + chunk_base[chunk * E + e] + token_pos[t * k + j];
        token_pos[t * k + j] = p;
        if ((uint64_t)p >= (uint64_t)R) continue;
        sorted_token[p] = (int32_t)t;
        sorted_slot[p] = j;
    }
}

moe_status route_launch(const float *logits, int64_t T, int E, int k, int tile_m,
                        int32_t *topk_idx, float *topk_gate, int32_t *counts, int32_t *offsets,
                        int32_t *token_pos, int32_t *sorted_token, int32_t *sorted_slot,
                        int32_t *tile_offsets, void *ws, hipStream_t s) {
    const int64_t nchunks = (T + kChunk - 1) / kChunk;
    int32_t *chunk_counts = reinterpret_cast<int32_t *>(ws);
    if (nchunks > 0) {
        dim3 g((unsigned)nchunks);
        switch (k) {
#define MOE_RS(K) \
    case K: route_select<K><<<g, kChunk * 8, 0, s>>>(logits, T, E, k, topk_idx, topk_gate, token_pos, chunk_counts); break;
            MOE_RS(1) MOE_RS(2) MOE_RS(3) MOE_RS(4) MOE_RS(5) MOE_RS(6) MOE_RS(7) MOE_RS(8)
#undef MOE_RS
            default: return MOE_ERR_SHAPE;
        }
    }
    route_scan<<<E, 256, 0, s>>>(chunk_counts, nchunks, E, counts);
    const int64_t nb = T > 0 ? (T + 255) / 256 : 1;
    route_place<<<(unsigned)nb, 256, 0, s>>>(counts, chunk_counts, T, E, k, tile_m, topk_idx,
                                             token_pos, sorted_token, sorted_slot, offsets,
                                             tile_offsets);
    return launch_status();
}


// ---------------------------------------------------------------------------
// moe_route without a caller workspace: the per-chunk expert counts go to
// this file-scope array, one copy per GPU, held until the process ends. In
// host code `g_route_scratch` is only a stand-in for the symbol, not a device
// address: the address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that address reaches a kernel.
static __device__ __align__(256) uint8_t g_route_scratch[kRouteNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::once_flag g_scratch_once[kMaxDevices];
static void *g_scratch_ptr[kMaxDevices];

static void *route_scratch(int dev) {
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_ptr[dev] =
            hipGetSymbolAddress(&p, HIP_SYMBOL(g_route_scratch)) == hipSuccess ? p : nullptr;
    });
    return g_scratch_ptr[dev];
}

moe_status route_noalloc_launch(const float *logits, int64_t T, int E, int k, int tile_m,
                                int32_t *topk_idx, float *topk_gate, int32_t *counts,
                                int32_t *offsets, int32_t *token_pos, int32_t *sorted_token,
                                int32_t *sorted_slot, int32_t *tile_offsets, hipStream_t s) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_LAUNCH;
    void *ws = route_scratch(dev);
    if (!ws) return MOE_ERR_LAUNCH;
    // every chunk count the kernels read is written first by route_select in
    // the same call, so nothing left by an earlier call needs clearing
    return route_launch(logits, T, E, k, tile_m, topk_idx, topk_gate, counts, offsets, token_pos,
                        sorted_token, sorted_slot, tile_offsets, ws, s);
}

}  // namespace moe
