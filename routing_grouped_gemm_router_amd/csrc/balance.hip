// balance.hip -- load-balance statistics and the auxiliary balancing loss.
//
// The report reads the load-balancing loss as part of the routing interface
// and names a failure mode, "token gerrymandering": the loss improves while
// the imbalance between experts gets worse (Ai2 Olmo-core 3, kongchang.com,
// "routing is a systems problem"; bytechap.com, "Key details" and "What you
// can do": watch for it in the routing metrics). The pages give no formula;
// the loss here is the published Switch Transformer balancing loss (Fedus,
// Zoph and Shazeer, 2021) with top-k routing:
//   f_e = c_e / (T k)                  fraction of routed rows sent to expert e
//   P_e = (1/T) sum_t softmax(l_t)_e   mean router probability of expert e
//   L   = alpha * E * sum_e f_e P_e
// L depends on the logits only through P (the counts are a step function of
// them), so dL/dl_{t,e} = (alpha E / T) p_{t,e} (f_e - sum_j p_{t,j} f_j).
// Next to L the statistics report the hard load, so that the two can be
// watched side by side: the balance term L optimises (E sum f P, 1 when
// uniform) against E sum f^2 and the max / min load over the mean, from the
// device counts.
//
// Three kernels, deterministic (fixed-order sums, no atomics):
//  1. lb_partial: one workgroup per 64-token chunk; each wave takes every
//     4th token (all its rows loaded first), computes the softmax (wave max,
//     wave sum), adds p to the wave's running sums and, if asked, adds the
//     loss gradient to dlogits. The four waves' sums are added in wave order
//     into the chunk's row of the workspace.
//  2. lb_reduce: one workgroup per expert sums its column of chunk rows
//     (fp64, fixed tree order) into P_e.
//  3. lb_stats: one workgroup reduces the statistics in fp64 in a fixed
//     tree order.
#include "common.h"

namespace moe {

constexpr int kLbChunk = 64;     // tokens per workgroup
constexpr int kLbMaxE = 256;

MOE_DEV float wave_max_f(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// every lane gets lane 0's value (the butterfly sums of different lanes
// associate differently)
MOE_DEV float wave_uniform(float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); }

template <int EPL>   // experts per lane: ceil(E / 64)
__global__ __launch_bounds__(256) void lb_partial(const float *__restrict__ logits,
                                                  const int32_t *__restrict__ counts, int64_t T, int E,
                                                  int k, float coef, float *__restrict__ partial,
                                                  float *__restrict__ dlogits) {
    __shared__ float f_s[kLbMaxE];
    __shared__ float acc_s[4][kLbMaxE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t chunk = blockIdx.x;
    const int64_t t0 = chunk * kLbChunk, t1 = min<int64_t>(T, t0 + kLbChunk);
    const float rows = (float)((double)T * k);
    for (int e = tid; e < E; e += 256) f_s[e] = (float)counts[e] / rows;
    __syncthreads();

    float f[EPL], pacc[EPL];
#pragma unroll
    for (int j = 0; j < EPL; j++) {
        const int e = lane + 64 * j;
        f[j] = e < E ? f_s[e] : 0.f;
        pacc[j] = 0.f;
    }
    // the wave's tokens t0 + wave + 4i, i < kLbChunk / 4: all rows loaded
    // before the first softmax
    constexpr int NTW = kLbChunk / 4;
    float l[NTW][EPL];
    // with a gradient, the current dlogits rows too: loaded with the logits,
    // before the first store (a load used while stores are in flight would
    // wait for all of them)
    float dl[NTW][EPL];
#pragma unroll
    for (int i = 0; i < NTW; i++) {
        const int64_t t = t0 + wave + 4 * i;
#pragma unroll
        for (int j = 0; j < EPL; j++) {
            const int e = lane + 64 * j;
            l[i][j] = (t < t1 && e < E) ? logits[t * E + e] : -INFINITY;
            dl[i][j] = (dlogits && t < t1 && e < E) ? dlogits[t * E + e] : 0.f;
        }
    }
#pragma unroll
    for (int i = 0; i < NTW; i++) {
        const int64_t t = t0 + wave + 4 * i;
        if (t >= t1) break;                               // wave-uniform
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < EPL; j++) m = fmaxf(m, l[i][j]);
        m = wave_uniform(wave_max_f(m));
        float ex[EPL], z = 0.f;
#pragma unroll
        for (int j = 0; j < EPL; j++) {
            ex[j] = (lane + 64 * j < E) ? expf(l[i][j] - m) : 0.f;
            z += ex[j];
        }
        z = wave_uniform(wave_sum(z));
        float p[EPL], sf = 0.f;
#pragma unroll
        for (int j = 0; j < EPL; j++) {
            p[j] = ex[j] / z;
            pacc[j] += p[j];
            sf += p[j] * f[j];
        }
        if (dlogits) {
            sf = wave_uniform(wave_sum(sf));
            float *drow = dlogits + t * E;
#pragma unroll
            for (int j = 0; j < EPL; j++) {
                const int e = lane + 64 * j;
                if (e < E) drow[e] = dl[i][j] + coef * p[j] * (f[j] - sf);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < EPL; j++) {
        const int e = lane + 64 * j;
        if (e < E) acc_s[wave][e] = pacc[j];
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256)
        partial[chunk * E + e] = ((acc_s[0][e] + acc_s[1][e]) + acc_s[2][e]) + acc_s[3][e];
}

// fixed-order tree sum over the 256 threads of the block (fp64)
MOE_DEV double block_sum_d(double v, double *red) {
    const int tid = threadIdx.x;
    red[tid] = v;
    __syncthreads();
#pragma unroll
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) red[tid] += red[tid + o];
        __syncthreads();
    }
    const double r = red[0];
    __syncthreads();
    return r;
}

// one block per expert: P_e = (1/T) sum over chunks of the partial sums,
// each thread summing every 256th chunk, then a fixed-order tree
__global__ __launch_bounds__(256) void lb_reduce(const float *__restrict__ partial, int64_t nchunks,
                                                 int E, int64_t T, double *__restrict__ P) {
    __shared__ double red[256];
    const int e = blockIdx.x, tid = threadIdx.x;
    double s = 0.0;
    for (int64_t ch = tid; ch < nchunks; ch += 256) s += (double)partial[ch * E + e];
    s = block_sum_d(s, red);
    if (tid == 0) P[e] = s / (double)T;
}

__global__ __launch_bounds__(256) void lb_stats(const double *__restrict__ Pv,
                                                const int32_t *__restrict__ counts, int64_t T, int E,
                                                int k, float alpha, float *__restrict__ stats) {
    __shared__ double red[256];
    __shared__ int32_t cmax_s[256], cmin_s[256];
    const int tid = threadIdx.x;
    const bool in = tid < E;
    const double rows = (double)T * k;
    const double P = in ? Pv[tid] : 0.0;
    const int32_t c = in ? counts[tid] : 0;
    const double f = (double)c / rows;
    const double mean = rows / E;
    const double fp = block_sum_d(in ? f * P : 0.0, red);
    const double ff = block_sum_d(in ? f * f : 0.0, red);
    const double pp = block_sum_d(in ? P * P : 0.0, red);
    const double var = block_sum_d(in ? ((double)c - mean) * ((double)c - mean) : 0.0, red) / E;
    const double empty = block_sum_d(in && c == 0 ? 1.0 : 0.0, red);
    cmax_s[tid] = in ? c : INT32_MIN;
    cmin_s[tid] = in ? c : INT32_MAX;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) {
            cmax_s[tid] = max(cmax_s[tid], cmax_s[tid + o]);
            cmin_s[tid] = min(cmin_s[tid], cmin_s[tid + o]);
        }
        __syncthreads();
    }
    if (tid == 0) {
        stats[0] = (float)(alpha * E * fp);
        stats[1] = (float)(E * fp);
        stats[2] = (float)(E * ff);
        stats[3] = (float)(E * pp);
        stats[4] = (float)(cmax_s[0] / mean);
        stats[5] = (float)(cmin_s[0] / mean);
        stats[6] = (float)(sqrt(var) / mean);
        stats[7] = (float)empty;
    }
}

__global__ void lb_zero_stats(float *stats) {
    if (threadIdx.x < MOE_LB_NSTATS) stats[threadIdx.x] = 0.f;
}

// workspace: the chunk partial sums (fp32 [nchunks][E]), then P (fp64 [E])
static size_t lb_partial_bytes(int64_t nchunks, int E) {
    return ((size_t)nchunks * E * sizeof(float) + 255) & ~(size_t)255;
}

moe_status load_balance_launch(const float *logits, const int32_t *counts, int64_t T, int E, int k,
                               float alpha, float *stats, float *dlogits, void *ws, hipStream_t s) {
    if (T == 0) {
        lb_zero_stats<<<1, 64, 0, s>>>(stats);
        return launch_status();
    }
    const int64_t nchunks = (T + kLbChunk - 1) / kLbChunk;
    float *partial = reinterpret_cast<float *>(ws);
    const float coef = (float)((double)alpha * E / (double)T);
    const dim3 g((unsigned)nchunks);
    switch ((E + 63) / 64) {
        case 1: lb_partial<1><<<g, 256, 0, s>>>(logits, counts, T, E, k, coef, partial, dlogits); break;
        case 2: lb_partial<2><<<g, 256, 0, s>>>(logits, counts, T, E, k, coef, partial, dlogits); break;
        case 3: lb_partial<3><<<g, 256, 0, s>>>(logits, counts, T, E, k, coef, partial, dlogits); break;
        default: lb_partial<4><<<g, 256, 0, s>>>(logits, counts, T, E, k, coef, partial, dlogits); break;
    }
    double *P = reinterpret_cast<double *>(reinterpret_cast<char *>(ws) + lb_partial_bytes(nchunks, E));
    lb_reduce<<<E, 256, 0, s>>>(partial, nchunks, E, T, P);
    lb_stats<<<1, 256, 0, s>>>(P, counts, T, E, k, alpha, stats);
    return launch_status();
}

size_t load_balance_ws_bytes(int64_t T, int E) {
    return lb_partial_bytes((T + kLbChunk - 1) / kLbChunk, E) + (size_t)E * sizeof(double);
}

}  // namespace moe
