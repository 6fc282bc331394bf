// pad.hip -- the padded-capacity alternative, kept for comparison.
//
// The report measures the device-scheduled grouped GEMM against padding every
// expert's batch to one uniform capacity (Ai2 Olmo-core 3, kongchang.com,
// "routing is a systems problem"); padding costs compute and memory for the
// empty rows (same page, on grouped GEMM). This file supplies the two pieces
// that turn the dropless metadata into that layout, so the same row kernels
// and the same grouped GEMM run on it and only the padding differs:
//   * expert e owns rows [e*C, (e+1)*C); of its routed rows (ascending token
//     order) the first C keep their rank, the rest are dropped (position -1:
//     no dispatch, no combine contribution, gates not renormalised);
//   * rows of an expert beyond its kept count are zero, so they add nothing
//     to the weight gradients.
#include "common.h"

namespace moe {

// token_pos_pad[t, j] = e*C + rank if rank < C else -1, with
// rank = token_pos[t, j] - offsets[e], e = topk_idx[t, j]; offsets_pad[e] = e*C.
__global__ __launch_bounds__(256) void capacity_pad_kernel(const int32_t *__restrict__ topk_idx,
                                                           const int32_t *__restrict__ token_pos,
                                                           const int32_t *__restrict__ offsets,
                                                           int64_t n, int E, int C,
                                                           int32_t *__restrict__ token_pos_pad,
                                                           int32_t *__restrict__ offsets_pad) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i <= E && offsets_pad) offsets_pad[i] = (int32_t)(i * C);
    if (i >= n) return;
    const int e = topk_idx[i];
    const int32_t rank = token_pos[i] - offsets[e];
    token_pos_pad[i] = rank < C ? e * C + rank : -1;
}

// Zero rows [e*C + min(c_e, C), (e+1)*C) of every expert e (c_e from the
// dropless offsets); one grid row of blocks per expert, 16 bytes per thread.
__global__ __launch_bounds__(256) void capacity_zero_kernel(uint4 *__restrict__ buf,
                                                            const int32_t *__restrict__ offsets,
                                                            int C, int64_t row16) {
    const int e = blockIdx.y;
    const int32_t c = offsets[e + 1] - offsets[e];
    const int64_t r0 = (int64_t)e * C + (c < C ? c : C);
    const int64_t n = ((int64_t)(e + 1) * C - r0) * row16;   // 16-byte units to clear
    uint4 *p = buf + r0 * row16;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = make_uint4(0, 0, 0, 0);
}

moe_status capacity_pad_launch(const int32_t *topk_idx, const int32_t *token_pos,
                               const int32_t *offsets, int64_t T, int E, int k, int C,
                               int32_t *token_pos_pad, int32_t *offsets_pad, hipStream_t s) {
    const int64_t n = T * k;
    const int64_t work = n > E + 1 ? n : E + 1;
    capacity_pad_kernel<<<(unsigned)((work + 255) / 256), 256, 0, s>>>(
        topk_idx, token_pos, offsets, n, E, C, token_pos_pad, offsets_pad);
    return launch_status();
}

moe_status capacity_zero_launch(void *buf, moe_dtype dt, const int32_t *offsets, int E, int C,
                                int cols, hipStream_t s) {
    const int64_t row16 = (int64_t)cols * (dt == MOE_F32 ? 4 : 2) / 16;
    // enough blocks per expert to cover a full capacity's rows in a few passes
    const int64_t per_e = ((int64_t)C * row16 + 1023) / 1024;
    const dim3 grid((unsigned)(per_e < 1 ? 1 : (per_e > 1024 ? 1024 : per_e)), (unsigned)E);
    capacity_zero_kernel<<<grid, 256, 0, s>>>(reinterpret_cast<uint4 *>(buf), offsets, C, row16);
    return launch_status();
}

}  // namespace moe
