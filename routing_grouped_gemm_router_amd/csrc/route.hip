// route.hip -- GPU-resident top-k routing and its metadata.
//
// The routing decisions and the metadata derived from them (all-to-all split
// sizes, per-expert group sizes) are computed and kept on the GPU, so the host
// only enqueues work (Ai2 Olmo-core 3, kongchang.com, "routing is a systems
// problem"; bytechap.com, "How it works").
//
// Three kernels, no host round trip and no order-dependent atomics:
//  1. route_select: one wave per 64-token chunk. The chunk's [64, E] logits
//     are read with coalesced 16-byte loads into LDS; each lane then selects
//     its token's top k (descending fp32 logit, equal logits -> lower index),
//     computes the gates (softmax over the k selected logits), and the wave
//     ranks every (token, expert) pair inside the chunk with one ballot per
//     expert: rank = popcount(ballot & lanes-below). Per-chunk expert counts
//     go to the workspace.
//  2. route_scan: one workgroup per expert scans its counts over chunks
//     (exclusive), giving each chunk its base inside the expert's group, and
//     the expert's total.
//  3. route_place: scans the E totals (in LDS) into offsets / tile offsets
//     and writes token_pos = offsets[e] + chunk base + rank and the inverse
//     maps sorted_token / sorted_slot.
#include "common.h"

namespace moe {

constexpr int kChunk = 64;      // tokens per chunk = one wave
constexpr int kMaxE = 256;

template <int KMAX>
__global__ __launch_bounds__(64) void route_select(const float *__restrict__ logits, int64_t T,
                                                   int E, int k, int32_t *__restrict__ topk_idx,
                                                   float *__restrict__ topk_gate,
                                                   int32_t *__restrict__ rank_out,
                                                   int32_t *__restrict__ chunk_counts) {
    __shared__ float tile[kChunk * (kMaxE + 1)];
    __shared__ int32_t cnt[kMaxE];
    const int lane = threadIdx.x;
    const int64_t chunk = blockIdx.x;
    const int64_t t0 = chunk * kChunk;
    const int ntok = (int)min<int64_t>(kChunk, T - t0);
    const int stride = E + 1;

    // coalesced load of the contiguous [ntok, E] block of logits
    const float *src = logits + t0 * E;
    const int total = ntok * E;
    if ((E & 3) == 0) {
        const float4 *src4 = reinterpret_cast<const float4 *>(src);
        for (int i = lane; i < total / 4; i += kChunk) {
            float4 v = src4[i];
            int e0 = (i * 4) % E, r = (i * 4) / E;
            float *dst = tile + r * stride + e0;
            dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
        }
    } else {
        for (int i = lane; i < total; i += kChunk) tile[(i / E) * stride + (i % E)] = src[i];
    }
    __syncthreads();

    // per-lane top-k by insertion (kept sorted: value descending, index ascending)
    float bv[KMAX];
    int bi[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; j++) { bv[j] = -INFINITY; bi[j] = -1; }
    const bool active = lane < ntok;
    if (active) {
        const float *row = tile + lane * stride;
        for (int e = 0; e < E; e++) {
            float cv = row[e];
            int ci = e;
            bool shifting = false;
#pragma unroll
            for (int j = 0; j < KMAX; j++) {
                if (j < k) {
                    // a later (higher) index only overtakes a strictly smaller value;
                    // once inserted, the rest of the list shifts down by one
                    bool take = shifting || bi[j] < 0 || cv > bv[j];
                    if (take) {
                        float tv = bv[j]; int ti = bi[j];
                        bv[j] = cv; bi[j] = ci;
                        cv = tv; ci = ti;
                        shifting = true;
                    }
                }
            }
        }
        // gates: softmax over the selected logits
        float m = bv[0], z = 0.f;
        float ex[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; j++) {
            ex[j] = (j < k) ? expf(bv[j] - m) : 0.f;
            z += ex[j];
        }
        const int64_t t = t0 + lane;
#pragma unroll
        for (int j = 0; j < KMAX; j++) {
            if (j < k) {
                topk_idx[t * k + j] = bi[j];
                topk_gate[t * k + j] = ex[j] / z;
            }
        }
    }

    // rank of each (token, expert) inside the chunk: one ballot per expert
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int rank[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; j++) rank[j] = 0;
    for (int e = 0; e < E; e++) {
        bool sel = false;
#pragma unroll
        for (int j = 0; j < KMAX; j++) sel |= (j < k) && active && (bi[j] == e);
        uint64_t m = __ballot(sel);
        int r = __popcll(m & below);
#pragma unroll
        for (int j = 0; j < KMAX; j++)
            if (j < k && bi[j] == e) rank[j] = r;
        if (lane == 0) cnt[e] = __popcll(m);
    }
    if (active) {
        const int64_t t = t0 + lane;
#pragma unroll
        for (int j = 0; j < KMAX; j++)
            if (j < k) rank_out[t * k + j] = rank[j];
    }
    __syncthreads();
    for (int e = lane; e < E; e += kChunk) chunk_counts[chunk * E + e] = cnt[e];
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
    for (int j = 0; j < k; j++) {
        int e = topk_idx[t * k + j];
        int32_t p = off[e] + chunk_base[chunk * E + e] + token_pos[t * k + j];
        token_pos[t * k + j] = p;
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
        dim3 g((unsigned)nchunks), b(kChunk);
        if (k <= 1)
            route_select<1><<<g, b, 0, s>>>(logits, T, E, k, topk_idx, topk_gate, token_pos, chunk_counts);
        else if (k <= 2)
            route_select<2><<<g, b, 0, s>>>(logits, T, E, k, topk_idx, topk_gate, token_pos, chunk_counts);
        else if (k <= 4)
            route_select<4><<<g, b, 0, s>>>(logits, T, E, k, topk_idx, topk_gate, token_pos, chunk_counts);
        else
            route_select<8><<<g, b, 0, s>>>(logits, T, E, k, topk_idx, topk_gate, token_pos, chunk_counts);
    }
    route_scan<<<E, 256, 0, s>>>(chunk_counts, nchunks, E, counts);
    const int64_t nb = T > 0 ? (T + 255) / 256 : 1;
    route_place<<<(unsigned)nb, 256, 0, s>>>(counts, chunk_counts, T, E, k, tile_m, topk_idx,
                                             token_pos, sorted_token, sorted_slot, offsets,
                                             tile_offsets);
    return launch_status();
}

}  // namespace moe
