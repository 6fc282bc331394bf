// api.hip -- the C ABI of libmoe: argument checks, then kernel launches.
//
// Every entry point validates host-visible scalars and pointers first and
// returns before enqueueing anything on a validation error; it never reads
// device memory, allocates, copies device->host or synchronises.
#include <string.h>

#include "common.h"

namespace moe {

moe_status route_launch(const float *logits, int64_t T, int E, int k, int tile_m,
                        int32_t *topk_idx, float *topk_gate, int32_t *counts, int32_t *offsets,
                        int32_t *token_pos, int32_t *sorted_token, int32_t *sorted_slot,
                        int32_t *tile_offsets, void *ws, hipStream_t s);
moe_status route_noalloc_launch(const float *logits, int64_t T, int E, int k, int tile_m,
                                int32_t *topk_idx, float *topk_gate, int32_t *counts,
                                int32_t *offsets, int32_t *token_pos, int32_t *sorted_token,
                                int32_t *sorted_slot, int32_t *tile_offsets, hipStream_t s);
moe_status permute_launch(const void *x, const uint8_t *x_scale, moe_dtype dt, int64_t T, int d,
                          int k, const int32_t *token_pos, void *x_perm, uint8_t *x_perm_scale,
                          hipStream_t s);
moe_status combine_launch(const void *y, moe_dtype dt, const float *gate,
                          const int32_t *token_pos, int64_t T, int d, int k, void *out,
                          bool unit_gate, hipStream_t s);
moe_status combine_bwd_launch(const void *dout, const void *y, moe_dtype dt, const float *gate,
                              const int32_t *topk_idx, const int32_t *token_pos, int64_t T,
                              int d, int k, int E, void *dy, float *dlogits, float *dgate,
                              hipStream_t s, bool row_gate_only = false);
moe_status gemm_launch(const moe_gemm_desc *d, hipStream_t s);
moe_status gemm_copy_walk(const moe_gemm_desc *d, const int32_t *host_offsets, moe_copy_walk *w);
moe_status gemm_hp_store_walk(const moe_gemm_desc *d, const int32_t *host_offsets, moe_copy_walk *w);
moe_status mxfp8_quantize_launch(const void *in, moe_dtype in_dt, int64_t rows, int64_t cols,
                                 int axis, const int32_t *group_offsets, int n_groups,
                                 const int32_t *row_map, uint8_t *q, uint8_t *scale,
                                 hipStream_t s);
moe_status mxfp8_quantize_both_launch(const void *in, moe_dtype in_dt, int64_t rows, int64_t cols,
                                      const int32_t *group_offsets, int n_groups, uint8_t *q1,
                                      uint8_t *s1, uint8_t *q0, uint8_t *s0, hipStream_t s,
                                      const int32_t *row_map = nullptr,
                                      const float *row_scale = nullptr);
size_t mxfp8_col_blocks(int64_t rows, int n_groups);
moe_status capacity_pad_launch(const int32_t *topk_idx, const int32_t *token_pos,
                               const int32_t *offsets, int64_t T, int E, int k, int C,
                               int32_t *token_pos_pad, int32_t *offsets_pad, hipStream_t s);
moe_status capacity_zero_launch(void *buf, moe_dtype dt, const int32_t *offsets, int E, int C,
                                int cols, hipStream_t s);
moe_status load_balance_launch(const float *logits, const int32_t *counts, int64_t T, int E, int k,
                               float alpha, float *stats, float *dlogits, void *ws, hipStream_t s);
size_t load_balance_ws_bytes(int64_t T, int E);

// Queried at every launch (a host-side lookup in the runtime, no device
// work), so the library holds no mutable state for it.
int num_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        n = 256;
    return n;
}

static bool routing_shape_ok(int64_t T, int32_t E, int32_t k) {
    return T >= 0 && E >= 1 && E <= 256 && k >= 1 && k <= 8 && k <= E &&
           T * (int64_t)k < ((int64_t)1 << 31);
}

static bool width_ok(int32_t w) { return w >= 32 && w <= 16384 && w % 32 == 0; }
// the expert hidden width h: GEMM1 is 2h wide, so 2h is held to the GEMM limit
static bool hidden_ok(int32_t h) { return width_ok(h) && 2 * h <= 16384; }

static size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

static bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

// sub-buffers of the MXFP8 backward workspace (byte offsets, 256-aligned):
// region A holds one row-quantised operand at a time, region B two
// column-block operands at a time (the call reuses them in sequence)
struct MxBwdLayout {
    size_t a_q, a_s, b0_q, b0_s, b1_q, b1_s, total;
};
static MxBwdLayout mx_bwd_layout(int64_t R, int d, int h, int E) {
    MxBwdLayout L;
    const size_t wmax = (size_t)(2 * h > d ? 2 * h : d);
    const size_t nbc = mxfp8_col_blocks(R, E);
    L.a_q = 0;
    L.a_s = round256((size_t)R * wmax);
    const size_t regA = L.a_s + round256((size_t)R * wmax / 32);
    // B: (dy rows along d, H' rows along h) then (dAB rows along 2h, x rows along d);
    // slot 0 holds d or 2h columns, slot 1 h or d
    const size_t w1 = (size_t)(h > d ? h : d);
    const size_t c0 = nbc * 32 * wmax, c1 = nbc * 32 * w1;
    L.b0_q = regA;
    L.b0_s = L.b0_q + round256(c0);
    L.b1_q = L.b0_s + round256(c0 / 32);
    L.b1_s = L.b1_q + round256(c1);
    L.total = L.b1_s + round256(c1 / 32);
    return L;
}

// records the caller's stage event i (if any) on s
static moe_status stage_mark(const moe_bwd_desc *b, int i, hipStream_t s) {
    if (!b->stage_events || !b->stage_events[i]) return MOE_OK;
    return hipEventRecord((hipEvent_t)b->stage_events[i], s) == hipSuccess ? MOE_OK
                                                                             : MOE_ERR_LAUNCH;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char *moe_status_str(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is null";
        case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: a size is out of range or inconsistent";
        case MOE_ERR_DTYPE: return "MOE_ERR_DTYPE: unsupported dtype/mode/epilogue";
        case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
        case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH: the HIP runtime reported a launch error";
        default: return "unknown moe_status";
    }
}

int32_t moe_version(void) { return 102; }

size_t moe_route_workspace_size(int64_t T, int32_t E, int32_t k) {
    (void)k;
    if (T < 0 || E < 1) return 0;
    return round256(sizeof(int32_t) * (size_t)E * (size_t)((T + 63) / 64));
}

moe_status moe_route(const float *logits, int64_t T, int32_t E, int32_t k, int32_t tile_m,
                     int32_t *topk_idx, float *topk_gate, int32_t *counts, int32_t *offsets,
                     int32_t *token_pos, int32_t *sorted_token, int32_t *sorted_slot,
                     int32_t *tile_offsets, void *ws, size_t ws_bytes, void *stream) {
    if (!routing_shape_ok(T, E, k) || tile_m < 1) return MOE_ERR_SHAPE;
    if (!counts || !offsets || !tile_offsets) return MOE_ERR_NULL;
    if (T > 0 && (!logits || !topk_idx || !topk_gate || !token_pos || !sorted_token ||
                  !sorted_slot || !ws))
        return MOE_ERR_NULL;
    if (T > 0 && !aligned16(logits)) return MOE_ERR_ALIGN;
    if (ws_bytes < moe_route_workspace_size(T, E, k)) return MOE_ERR_WORKSPACE;
    return route_launch(logits, T, E, k, tile_m, topk_idx, topk_gate, counts, offsets, token_pos,
                        sorted_token, sorted_slot, tile_offsets, ws, (hipStream_t)stream);
}

moe_status moe_route_noalloc(const float *logits, int64_t T, int32_t E, int32_t k, int32_t tile_m,
                             int32_t *topk_idx, float *topk_gate, int32_t *counts,
                             int32_t *offsets, int32_t *token_pos, int32_t *sorted_token,
                             int32_t *sorted_slot, int32_t *tile_offsets, void *stream) {
    if (!routing_shape_ok(T, E, k) || tile_m < 1) return MOE_ERR_SHAPE;
    if (!counts || !offsets || !tile_offsets) return MOE_ERR_NULL;
    if (T > 0 && (!logits || !topk_idx || !topk_gate || !token_pos || !sorted_token ||
                  !sorted_slot))
        return MOE_ERR_NULL;
    if (T > 0 && !aligned16(logits)) return MOE_ERR_ALIGN;
    if (moe_route_workspace_size(T, E, k) > MOE_ROUTE_NOALLOC_SCRATCH_BYTES)
        return MOE_ERR_WORKSPACE;
    return route_noalloc_launch(logits, T, E, k, tile_m, topk_idx, topk_gate, counts, offsets,
                                token_pos, sorted_token, sorted_slot, tile_offsets,
                                (hipStream_t)stream);
}

moe_status moe_permute(const void *x, const uint8_t *x_scale, moe_dtype dt, int64_t T, int32_t d,
                       int32_t k, const int32_t *token_pos, void *x_perm, uint8_t *x_perm_scale,
                       void *stream) {
    if (dt != MOE_F32 && dt != MOE_BF16 && dt != MOE_MXFP8) return MOE_ERR_DTYPE;
    if (T < 0 || k < 1 || k > 8 || T * (int64_t)k >= ((int64_t)1 << 31) || !width_ok(d))
        return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!x || !token_pos || !x_perm) return MOE_ERR_NULL;
    if (dt == MOE_MXFP8 && (!x_scale || !x_perm_scale)) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_ALIGN;
    return permute_launch(x, x_scale, dt, T, d, k, token_pos, x_perm, x_perm_scale,
                          (hipStream_t)stream);
}

moe_status moe_combine(const void *y_perm, moe_dtype dt, const float *topk_gate,
                       const int32_t *token_pos, int64_t T, int32_t d, int32_t k, void *out,
                       void *stream) {
    if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_DTYPE;
    if (T < 0 || k < 1 || k > 8 || T * (int64_t)k >= ((int64_t)1 << 31) || !width_ok(d))
        return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!y_perm || !topk_gate || !token_pos || !out) return MOE_ERR_NULL;
    if (!aligned16(y_perm) || !aligned16(out)) return MOE_ERR_ALIGN;
    return combine_launch(y_perm, dt, topk_gate, token_pos, T, d, k, out, false,
                          (hipStream_t)stream);
}

// the descriptor's mode, dtype, epilogue and shapes (no pointers)
static moe_status check_gemm_shape(const moe_gemm_desc *g) {
    if (!g) return MOE_ERR_NULL;
    if (g->mode < MOE_GG_FWD || g->mode > MOE_GG_WGRAD) return MOE_ERR_DTYPE;
    if (g->dtype != MOE_F32 && g->dtype != MOE_BF16 && g->dtype != MOE_MXFP8) return MOE_ERR_DTYPE;
    // H' stored quantised: the MXFP8 SwiGLU forward only
    if (g->aux_out_scale && (g->dtype != MOE_MXFP8 || g->epilogue != MOE_EPI_SWIGLU_FWD))
        return MOE_ERR_DTYPE;
    if (g->dtype == MOE_MXFP8) {
        if (g->mode != MOE_GG_WGRAD && g->K % 128) return MOE_ERR_SHAPE;
        // WGRAD: the 256 rows of a B tile in a group's column block (pitch:
        // the group's rows rounded up to 128 bytes) are addressed with 32-bit
        // offsets from one base
        if (g->mode == MOE_GG_WGRAD && g->rows > ((int64_t)1 << 24)) return MOE_ERR_SHAPE;
    }
    if (g->epilogue == MOE_EPI_SWIGLU_FWD && g->mode != MOE_GG_FWD) return MOE_ERR_DTYPE;
    if (g->epilogue == MOE_EPI_SWIGLU_BWD && g->mode != MOE_GG_DGRAD) return MOE_ERR_DTYPE;
    if (g->epilogue < MOE_EPI_NONE || g->epilogue > MOE_EPI_SWIGLU_BWD) return MOE_ERR_DTYPE;
    if (g->accumulate != 0 && (g->accumulate != 1 || g->mode != MOE_GG_WGRAD)) return MOE_ERR_DTYPE;
    if (g->n_groups < 1 || g->n_groups > 256) return MOE_ERR_SHAPE;
    if (g->rows < 0 || g->rows >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
    if (g->mode == MOE_GG_WGRAD) {
        if (!width_ok(g->M) || !width_ok(g->N)) return MOE_ERR_SHAPE;
    } else {
        if (!width_ok(g->N) || !width_ok(g->K)) return MOE_ERR_SHAPE;
        if (g->epilogue == MOE_EPI_SWIGLU_FWD && (g->N / 2) % 32) return MOE_ERR_SHAPE;
    }
    return MOE_OK;
}

static moe_status check_gemm(const moe_gemm_desc *g) {
    moe_status st = check_gemm_shape(g);
    if (st != MOE_OK) return st;
    if (g->dtype == MOE_MXFP8) {
        if (!g->a_scale || !g->b_scale) return MOE_ERR_NULL;
        if (!aligned4(g->a_scale) || !aligned4(g->b_scale)) return MOE_ERR_ALIGN;
    }
    // with no rows, the row-indexed operands may be empty (null) buffers; WGRAD
    // still writes its (zero) weight gradients
    const bool rows_needed = g->rows > 0;
    if (!g->offsets) return MOE_ERR_NULL;
    if (!g->B && (rows_needed || g->mode != MOE_GG_WGRAD)) return MOE_ERR_NULL;
    if (rows_needed && !g->A) return MOE_ERR_NULL;
    if ((rows_needed || g->mode == MOE_GG_WGRAD) && !g->C) return MOE_ERR_NULL;
    if (rows_needed && g->epilogue == MOE_EPI_SWIGLU_FWD && !g->aux_out) return MOE_ERR_NULL;
    if (rows_needed && g->aux_out_scale && (!g->aux_out_cols || !g->aux_out_cols_scale))
        return MOE_ERR_NULL;
    if (g->aux_out_scale && (!aligned4(g->aux_out_scale) ||
                             (g->aux_out_cols && !aligned16(g->aux_out_cols)) ||
                             (g->aux_out_cols_scale && !aligned4(g->aux_out_cols_scale))))
        return MOE_ERR_ALIGN;
    if (rows_needed && g->epilogue == MOE_EPI_SWIGLU_BWD && !g->aux) return MOE_ERR_NULL;
    if ((g->A && !aligned16(g->A)) || !aligned16(g->B) || (g->C && !aligned16(g->C)))
        return MOE_ERR_ALIGN;
    if (g->aux && !aligned16(g->aux)) return MOE_ERR_ALIGN;
    if (g->aux_out && !aligned16(g->aux_out)) return MOE_ERR_ALIGN;
    if (g->ws_bytes < moe_grouped_gemm_workspace_size(g)) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

size_t moe_grouped_gemm_workspace_size(const moe_gemm_desc *g) {
    (void)g;
    return 0;
}

moe_status moe_grouped_gemm(const moe_gemm_desc *g, void *stream) {
    moe_status st = check_gemm(g);
    if (st != MOE_OK) return st;
    if (g->rows == 0 && g->mode != MOE_GG_WGRAD) return MOE_OK;   // every group is empty
    return gemm_launch(g, (hipStream_t)stream);
}

moe_status moe_gemm_copy_walk(const moe_gemm_desc *g, const int32_t *host_offsets,
                              moe_copy_walk *w) {
    moe_status st = check_gemm_shape(g);
    if (st != MOE_OK) return st;
    if (!host_offsets || !w) return MOE_ERR_NULL;
    if (g->dtype == MOE_F32) return MOE_ERR_DTYPE;
    if (host_offsets[0] != 0 || host_offsets[g->n_groups] != g->rows) return MOE_ERR_SHAPE;
    for (int e = 0; e < g->n_groups; e++)
        if (host_offsets[e + 1] < host_offsets[e]) return MOE_ERR_SHAPE;
    return gemm_copy_walk(g, host_offsets, w);
}

moe_status moe_gemm_hp_store_walk(const moe_gemm_desc *g, const int32_t *host_offsets,
                                  moe_copy_walk *w) {
    moe_status st = check_gemm_shape(g);
    if (st != MOE_OK) return st;
    if (!host_offsets || !w) return MOE_ERR_NULL;
    if (g->dtype != MOE_MXFP8 || g->mode != MOE_GG_FWD || g->epilogue != MOE_EPI_SWIGLU_FWD)
        return MOE_ERR_DTYPE;
    if (host_offsets[0] != 0 || host_offsets[g->n_groups] != g->rows) return MOE_ERR_SHAPE;
    for (int e = 0; e < g->n_groups; e++)
        if (host_offsets[e + 1] < host_offsets[e]) return MOE_ERR_SHAPE;
    return gemm_hp_store_walk(g, host_offsets, w);
}

size_t moe_backward_workspace_size(const moe_bwd_desc *b) {
    if (!b || b->dtype != MOE_MXFP8) return 0;
    return mx_bwd_layout(b->T * b->k, b->d, b->h, b->E).total;
}

moe_status moe_backward_workspace_layout(const moe_bwd_desc *b, moe_bwd_ws_layout *out) {
    if (!b || !out) return MOE_ERR_NULL;
    if (b->dtype != MOE_MXFP8) return MOE_ERR_DTYPE;
    if (!routing_shape_ok(b->T, b->E, b->k) || !width_ok(b->d) || !hidden_ok(b->h) ||
        b->d % 128 || b->h % 128 || b->T * b->k > ((int64_t)1 << 24))
        return MOE_ERR_SHAPE;
    const MxBwdLayout L = mx_bwd_layout(b->T * b->k, b->d, b->h, b->E);
    out->row_q = L.a_q; out->row_s = L.a_s;
    out->col0_q = L.b0_q; out->col0_s = L.b0_s;
    out->col1_q = L.b1_q; out->col1_s = L.b1_s;
    out->total = L.total;
    return MOE_OK;
}

static moe_status backward_mxfp8(const moe_bwd_desc *b, hipStream_t s);

moe_status moe_backward(const moe_bwd_desc *b, void *stream) {
    if (!b) return MOE_ERR_NULL;
    if (b->dtype == MOE_MXFP8) return backward_mxfp8(b, (hipStream_t)stream);
    if (b->dtype != MOE_F32 && b->dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (b->accumulate_dw != 0 && b->accumulate_dw != 1) return MOE_ERR_DTYPE;
    if (!routing_shape_ok(b->T, b->E, b->k) || !width_ok(b->d) || !hidden_ok(b->h))
        return MOE_ERR_SHAPE;
    if (!b->dw1 || !b->dw2 || !b->offsets || !b->w1 || !b->w2) return MOE_ERR_NULL;
    const bool any = b->T > 0;
    if (any && (!b->x_perm || !b->ab || !b->hp || !b->y_perm || !b->topk_gate || !b->topk_idx ||
                !b->token_pos || !b->dout || !b->dx || !b->dlogits || !b->dy_perm || !b->dab ||
                !b->dx_perm))
        return MOE_ERR_NULL;
    const void *al[] = {b->x_perm, b->ab, b->hp, b->y_perm, b->w1, b->w2, b->dout, b->dx,
                        b->dw1, b->dw2, b->dy_perm, b->dab, b->dx_perm};
    for (const void *p : al)
        if (p && !aligned16(p)) return MOE_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    const int64_t R = b->T * b->k;
    moe_status st = combine_bwd_launch(b->dout, b->y_perm, b->dtype, b->topk_gate, b->topk_idx,
                                       b->token_pos, b->T, b->d, b->k, b->E, b->dy_perm,
                                       b->dlogits, b->dgate, s);
    if (st != MOE_OK || (st = stage_mark(b, 0, s)) != MOE_OK) return st;
    moe_gemm_desc g;
    memset(&g, 0, sizeof(g));
    g.dtype = b->dtype;
    g.n_groups = b->E;
    g.rows = R;
    g.offsets = b->offsets;
    // GEMM2 dgrad with the SwiGLU backward: dAB from dy_perm . W2[e]
    g.mode = MOE_GG_DGRAD; g.epilogue = MOE_EPI_SWIGLU_BWD;
    g.N = b->h; g.K = b->d;
    g.A = b->dy_perm; g.B = b->w2; g.C = b->dab; g.aux = b->ab;
    if (R > 0 && (st = gemm_launch(&g, s)) != MOE_OK) return st;
    if ((st = stage_mark(b, 1, s)) != MOE_OK) return st;
    // GEMM2 wgrad: dW2[e] = dy^T H'
    g.mode = MOE_GG_WGRAD; g.epilogue = MOE_EPI_NONE; g.aux = nullptr;
    g.accumulate = b->accumulate_dw;
    g.M = b->d; g.N = b->h; g.K = 0;
    g.A = b->dy_perm; g.B = b->hp; g.C = b->dw2;
    if ((st = gemm_launch(&g, s)) != MOE_OK || (st = stage_mark(b, 2, s)) != MOE_OK) return st;
    // GEMM1 dgrad: dx_perm = dAB . W1[e]
    g.mode = MOE_GG_DGRAD; g.accumulate = 0; g.M = 0; g.N = b->d; g.K = 2 * b->h;
    g.A = b->dab; g.B = b->w1; g.C = b->dx_perm;
    if (R > 0 && (st = gemm_launch(&g, s)) != MOE_OK) return st;
    if ((st = stage_mark(b, 3, s)) != MOE_OK) return st;
    // unpermute backward: dX[t] = sum_j dx_perm[token_pos[t, j]], straight
    // after dx_perm is written (read back while it is still cached, and ahead
    // of the weight gradient's 2 GiB of fp32 stores)
    if ((st = combine_launch(b->dx_perm, b->dtype, nullptr, b->token_pos, b->T, b->d, b->k, b->dx,
                             true, s)) != MOE_OK ||
        (st = stage_mark(b, 4, s)) != MOE_OK)
        return st;
    // GEMM1 wgrad: dW1[e] = dAB^T x
    g.mode = MOE_GG_WGRAD; g.accumulate = b->accumulate_dw; g.M = 2 * b->h; g.N = b->d; g.K = 0;
    g.A = b->dab; g.B = b->x_perm; g.C = b->dw1;
    if ((st = gemm_launch(&g, s)) != MOE_OK) return st;
    return stage_mark(b, 5, s);
}

static moe_status backward_mxfp8(const moe_bwd_desc *b, hipStream_t s) {
    if (b->accumulate_dw != 0 && b->accumulate_dw != 1) return MOE_ERR_DTYPE;
    if (!routing_shape_ok(b->T, b->E, b->k) || !width_ok(b->d) || !hidden_ok(b->h) ||
        b->d % 128 || b->h % 128)
        return MOE_ERR_SHAPE;
    // the weight gradients address 256 rows of a group's column block with
    // 32-bit offsets (as moe_grouped_gemm's MXFP8 WGRAD)
    if (b->T * b->k > ((int64_t)1 << 24)) return MOE_ERR_SHAPE;
    if (!b->dw1 || !b->dw2 || !b->offsets || !b->w1t || !b->w1t_scale || !b->w2t ||
        !b->w2t_scale)
        return MOE_ERR_NULL;
    const bool any = b->T > 0;
    if (!b->hp_cols != !b->hp_cols_scale) return MOE_ERR_NULL;
    if (any && (!b->x || !b->sorted_token || !b->ab || (!b->hp && !b->hp_cols) || !b->y_perm || !b->topk_gate ||
                !b->topk_idx || !b->token_pos || !b->dout || !b->dx || !b->dlogits ||
                !b->dy_perm || !b->dab || !b->dx_perm || !b->ws))
        return MOE_ERR_NULL;
    const void *al[] = {b->x, b->ab, b->hp, b->y_perm, b->dout, b->dx, b->dw1, b->dw2,
                        b->dy_perm, b->dab, b->dx_perm, b->w1t, b->w2t, b->ws, b->hp_cols};
    for (const void *p : al)
        if (p && !aligned16(p)) return MOE_ERR_ALIGN;
    if (!aligned4(b->w1t_scale) || !aligned4(b->w2t_scale)) return MOE_ERR_ALIGN;
    if (b->hp_cols_scale && !aligned4(b->hp_cols_scale)) return MOE_ERR_ALIGN;
    const int64_t R = b->T * b->k;
    const int d = b->d, h = b->h, E = b->E;
    const MxBwdLayout L = mx_bwd_layout(R, d, h, E);
    if (b->ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    char *ws = reinterpret_cast<char *>(b->ws);
    uint8_t *aq = (uint8_t *)(ws + L.a_q), *as = (uint8_t *)(ws + L.a_s);
    uint8_t *b0q = (uint8_t *)(ws + L.b0_q), *b0s = (uint8_t *)(ws + L.b0_s);
    uint8_t *b1q = (uint8_t *)(ws + L.b1_q), *b1s = (uint8_t *)(ws + L.b1_s);
    moe_status st;
    // combine backward + router backward (bf16). dy_perm is not stored: the
    // combine backward leaves each routed row's gate in its first 4*T*k bytes
    // and the quantiser below forms dy = round_bf16(gate * dOut[token]) as it
    // reads the dOut rows
    float *row_gate = reinterpret_cast<float *>(b->dy_perm);
    if ((st = combine_bwd_launch(b->dout, b->y_perm, MOE_BF16, b->topk_gate, b->topk_idx,
                                 b->token_pos, b->T, d, b->k, E, row_gate, b->dlogits,
                                 b->dgate, s, true)) != MOE_OK ||
        (st = stage_mark(b, 0, s)) != MOE_OK)
        return st;
    moe_gemm_desc g;
    memset(&g, 0, sizeof(g));
    g.dtype = MOE_MXFP8;
    g.n_groups = E;
    g.rows = R;
    g.offsets = b->offsets;
    // dy along d (GEMM2 dgrad) and along rows per expert (GEMM2 wgrad), from
    // one read of the dOut rows
    if ((st = R > 0 ? mxfp8_quantize_both_launch(b->dout, MOE_BF16, R, d, b->offsets, E, aq, as, b0q,
                                                  b0s, s, b->sorted_token, row_gate)
                    : MOE_OK) != MOE_OK ||
        (st = stage_mark(b, 1, s)) != MOE_OK)
        return st;
    if (R > 0) {
        // GEMM2 dgrad + SwiGLU backward: dy . W2t
        g.mode = MOE_GG_DGRAD; g.epilogue = MOE_EPI_SWIGLU_BWD; g.N = h; g.K = d;
        g.A = aq; g.a_scale = as; g.B = b->w2t; g.b_scale = b->w2t_scale;
        g.C = b->dab; g.aux = b->ab;
        if ((st = gemm_launch(&g, s)) != MOE_OK) return st;
    }
    if ((st = stage_mark(b, 2, s)) != MOE_OK) return st;
    // GEMM2 wgrad: dy and H' along rows, per expert (H' quantised here unless
    // the caller brings it in that layout)
    if (!b->hp_cols &&
        (st = mxfp8_quantize_launch(b->hp, MOE_BF16, R, h, 0, b->offsets, E, nullptr, b1q, b1s,
                                    s)) != MOE_OK)
        return st;
    if ((st = stage_mark(b, 3, s)) != MOE_OK) return st;
    g.mode = MOE_GG_WGRAD; g.epilogue = MOE_EPI_NONE; g.aux = nullptr; g.M = d; g.N = h; g.K = 0;
    g.accumulate = b->accumulate_dw;
    g.A = b0q; g.a_scale = b0s; g.C = b->dw2;
    g.B = b->hp_cols ? b->hp_cols : b1q;
    g.b_scale = b->hp_cols ? b->hp_cols_scale : b1s;
    if ((st = gemm_launch(&g, s)) != MOE_OK || (st = stage_mark(b, 4, s)) != MOE_OK) return st;
    // dAB along 2h (GEMM1 dgrad) and along rows per expert (GEMM1 wgrad), one read
    if ((st = R > 0 ? mxfp8_quantize_both_launch(b->dab, MOE_BF16, R, 2 * h, b->offsets, E, aq, as, b0q,
                                                  b0s, s)
                    : mxfp8_quantize_launch(b->dab, MOE_BF16, R, 2 * h, 0, b->offsets, E,
                                            nullptr, b0q, b0s, s)) != MOE_OK ||
        (st = stage_mark(b, 5, s)) != MOE_OK)
        return st;
    if (R > 0) {
        // GEMM1 dgrad: dAB . W1t
        g.mode = MOE_GG_DGRAD; g.accumulate = 0; g.M = 0; g.N = d; g.K = 2 * h;
        g.A = aq; g.a_scale = as; g.B = b->w1t; g.b_scale = b->w1t_scale; g.C = b->dx_perm;
        if ((st = gemm_launch(&g, s)) != MOE_OK) return st;
    }
    if ((st = stage_mark(b, 6, s)) != MOE_OK) return st;
    // unpermute backward, straight after dx_perm is written
    if ((st = combine_launch(b->dx_perm, MOE_BF16, nullptr, b->token_pos, b->T, d, b->k, b->dx,
                             true, s)) != MOE_OK ||
        (st = stage_mark(b, 7, s)) != MOE_OK)
        return st;
    // GEMM1 wgrad: dAB and x[sorted_token] along rows, per expert
    if ((st = mxfp8_quantize_launch(b->x, MOE_BF16, R, d, 0, b->offsets, E, b->sorted_token, b1q,
                                    b1s, s)) != MOE_OK ||
        (st = stage_mark(b, 8, s)) != MOE_OK)
        return st;
    g.mode = MOE_GG_WGRAD; g.accumulate = b->accumulate_dw; g.M = 2 * h; g.N = d; g.K = 0;
    g.A = b0q; g.a_scale = b0s; g.B = b1q; g.b_scale = b1s; g.C = b->dw1;
    if ((st = gemm_launch(&g, s)) != MOE_OK) return st;
    return stage_mark(b, 9, s);
}

size_t mxfp8_col_blocks(int64_t rows, int32_t n_groups) { return moe::mxfp8_col_blocks(rows, n_groups); }

moe_status mxfp8_quantize_both(const void *in, moe_dtype in_dt, int64_t rows, int64_t cols,
                               const int32_t *group_offsets, int32_t n_groups, uint8_t *q_rows,
                               uint8_t *s_rows, uint8_t *q_cols, uint8_t *s_cols, void *stream) {
    if (in_dt != MOE_F32 && in_dt != MOE_BF16) return MOE_ERR_DTYPE;
    if (rows < 0 || cols < 32 || cols % 32 || rows >= ((int64_t)1 << 31) ||
        cols >= ((int64_t)1 << 20))
        return MOE_ERR_SHAPE;
    if (group_offsets && (n_groups < 1 || n_groups > 1024)) return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    if (!in || !q_rows || !s_rows || !q_cols || !s_cols) return MOE_ERR_NULL;
    if (!aligned16(in) || !aligned16(q_rows) || !aligned16(q_cols)) return MOE_ERR_ALIGN;
    return mxfp8_quantize_both_launch(in, in_dt, rows, cols, group_offsets,
                                      group_offsets ? n_groups : 1, q_rows, s_rows, q_cols, s_cols,
                                      (hipStream_t)stream);
}

moe_status moe_capacity_pad(const int32_t *topk_idx, const int32_t *token_pos,
                            const int32_t *offsets, int64_t T, int32_t E, int32_t k,
                            int32_t capacity, int32_t *token_pos_pad, int32_t *offsets_pad,
                            void *stream) {
    if (!routing_shape_ok(T, E, k) || capacity < 0 ||
        (int64_t)E * capacity >= ((int64_t)1 << 31))
        return MOE_ERR_SHAPE;
    if (!offsets_pad) return MOE_ERR_NULL;
    if (T > 0 && (!topk_idx || !token_pos || !offsets || !token_pos_pad)) return MOE_ERR_NULL;
    return capacity_pad_launch(topk_idx, token_pos, offsets, T, E, k, capacity, token_pos_pad,
                               offsets_pad, (hipStream_t)stream);
}

moe_status moe_capacity_zero_rows(void *buf, moe_dtype dt, const int32_t *offsets, int32_t E,
                                  int32_t capacity, int32_t cols, void *stream) {
    if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_DTYPE;
    if (E < 1 || E > 256 || capacity < 0 || !width_ok(cols) ||
        (int64_t)E * capacity >= ((int64_t)1 << 31))
        return MOE_ERR_SHAPE;
    if (capacity == 0) return MOE_OK;
    if (!buf || !offsets) return MOE_ERR_NULL;
    if (!aligned16(buf)) return MOE_ERR_ALIGN;
    return capacity_zero_launch(buf, dt, offsets, E, capacity, cols, (hipStream_t)stream);
}

size_t moe_load_balance_workspace_size(int64_t T, int32_t E) {
    if (T < 0 || E < 1 || E > 256) return 0;
    return load_balance_ws_bytes(T, E);
}

moe_status moe_load_balance(const float *logits, const int32_t *counts, int64_t T, int32_t E,
                            int32_t k, float alpha, float *stats, float *dlogits, void *ws,
                            size_t ws_bytes, void *stream) {
    if (!routing_shape_ok(T, E, k)) return MOE_ERR_SHAPE;
    if (!stats) return MOE_ERR_NULL;
    if (T > 0 && (!logits || !counts || !ws)) return MOE_ERR_NULL;
    if (!aligned4(logits) || !aligned4(stats) || !aligned4(dlogits) || !aligned16(ws))
        return MOE_ERR_ALIGN;
    if (ws_bytes < load_balance_ws_bytes(T, E)) return MOE_ERR_WORKSPACE;
    return load_balance_launch(logits, counts, T, E, k, alpha, stats, dlogits, ws,
                               (hipStream_t)stream);
}

moe_status mxfp8_quantize(const void *in, moe_dtype in_dt, int64_t rows, int64_t cols,
                          int32_t axis, const int32_t *group_offsets, int32_t n_groups,
                          const int32_t *row_map, uint8_t *q, uint8_t *scale, void *stream) {
    if (in_dt != MOE_F32 && in_dt != MOE_BF16) return MOE_ERR_DTYPE;
    if (rows < 0 || cols < 32 || cols % 32 || rows >= ((int64_t)1 << 31) ||
        cols >= ((int64_t)1 << 20))
        return MOE_ERR_SHAPE;
    if (axis != 0 && axis != 1) return MOE_ERR_SHAPE;
    if (axis == 0 && group_offsets && (n_groups < 1 || n_groups > 1024)) return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    if (!in || !q || !scale) return MOE_ERR_NULL;
    if (!aligned16(in) || !aligned16(q)) return MOE_ERR_ALIGN;
    return mxfp8_quantize_launch(in, in_dt, rows, cols, axis, group_offsets,
                                 group_offsets ? n_groups : 1, row_map, q, scale,
                                 (hipStream_t)stream);
}

}  // extern "C"
