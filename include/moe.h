/*
 * moe.h -- C ABI of libmoe: the MoE expert layer on one MI355X (gfx950).
 *
 * The layer (as the pages describe it in prose):
 *   - each token activates a few of E experts (e.g. 4 of 128)
 *     [Ai2 Olmo-core 3, kongchang.com, section "capacity tax"];
 *   - routing is computed on the GPU and its metadata (the split sizes and the
 *     per-expert group sizes) stays there, so the host enqueues work without
 *     waiting for a device-to-host copy [kongchang.com, "routing is a systems
 *     problem"; aizyradar.cn, "What changed"; bytechap.com, "How it works"];
 *   - only the selected token rows are written straight into the experts'
 *     input buffers [kongchang.com, "capacity tax"; bytechap.com, "How it
 *     works"];
 *   - a device-scheduled grouped GEMM runs the uneven per-expert shapes
 *     without padding every expert to one capacity [kongchang.com, "routing is
 *     a systems problem"];
 *   - MXFP8 (OCP, one shared scale per 32 elements) is used for the GEMMs and
 *     the dispatch payload [kongchang.com, "caveats behind the numbers";
 *     aikraft.ru, "Technical optimisations"].
 * The pages give no router function, FFN shape or API; this header fixes them
 * (softmax top-k router, SwiGLU experts, the calls below).
 *
 * Conventions for every call
 *   - Tensor arguments are DEVICE pointers to dense row-major buffers that the
 *     caller allocates and owns. The library never allocates, frees, copies
 *     device->host or synchronises; it only enqueues kernels on `stream`
 *     (a hipStream_t; NULL = the default stream). Every call can therefore be
 *     captured in a HIP graph.
 *   - Scratch memory, where a call needs it, comes in through (ws, ws_bytes);
 *     the matching *_workspace_size() gives the minimum.
 *   - Validation looks only at host-visible scalars and pointers (null,
 *     16-byte alignment, shape limits); device data is never inspected. On a
 *     validation error nothing is enqueued. After enqueueing, a launch error
 *     is reported as MOE_ERR_LAUNCH.
 *   - Limits: 1 <= E <= 256; 1 <= k <= min(E, 8); 0 <= T; T*k < 2^31;
 *     d and h multiples of 32; d <= 16384, h <= 8192 (GEMM1 is 2h wide;
 *     every GEMM width N, K, M <= 16384).
 *   - Non-finite logits are outside the contract: outputs are then
 *     unspecified, but no kernel indexes out of bounds.
 *   - Stateless and re-entrant: concurrent calls on different streams are
 *     safe given distinct output and workspace buffers (moe_route_noalloc,
 *     which keeps its scratch in the library, is the one exception).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,       /* a required pointer is null */
    MOE_ERR_SHAPE = 2,      /* a size is out of range or inconsistent */
    MOE_ERR_DTYPE = 3,      /* unsupported dtype / mode / epilogue combination */
    MOE_ERR_ALIGN = 4,      /* a tensor pointer is not 16-byte aligned */
    MOE_ERR_WORKSPACE = 5,  /* workspace smaller than *_workspace_size() */
    MOE_ERR_LAUNCH = 6      /* the HIP runtime reported an error at launch */
};

typedef int32_t moe_dtype;
enum {
    MOE_F32 = 0,    /* fp32 storage */
    MOE_BF16 = 1,   /* bfloat16 storage, fp32 accumulation */
    MOE_MXFP8 = 2   /* OCP MXFP8: E4M3 bytes + one E8M0 byte per 32 elements */
};

/* Human-readable name of a status code (static string). */
const char *moe_status_str(moe_status s);

/* ABI version of this header (major * 100 + minor). 101: moe_bwd_desc ends
 * with hp_cols, hp_cols_scale (zero them when unused), and the MXFP8
 * backward uses dy_perm as scratch. 102: moe_gemm_desc ends with
 * aux_out_cols, aux_out_cols_scale, and aux_out_scale selects the MXFP8
 * SwiGLU forward that stores H' quantised (zero all three when unused). */
int32_t moe_version(void);

/* ------------------------------------------------------------------ */
/* Routing                                                              */

/* Bytes of scratch moe_route needs: 4 * E * ceil(T / 64), rounded up to 256. */
size_t moe_route_workspace_size(int64_t T, int32_t E, int32_t k);

/* Top-k softmax routing and the layer's routing metadata, all on device.
 *   logits       [T, E] fp32 (router scores; an input: the router's linear
 *                layer is outside this call)
 *   topk_idx     [T, k] int32 out: the k experts of each token, best first;
 *                experts are compared by fp32 logit, equal logits (IEEE, so
 *                -0 == +0) go to the lower expert index
 *   topk_gate    [T, k] fp32 out: softmax over the k selected logits (the full
 *                softmax renormalised over the top k); sums to 1 per token
 *   counts       [E] int32 out: rows routed to each expert (the group sizes)
 *   offsets      [E+1] int32 out: exclusive prefix sum of counts; expert e owns
 *                rows [offsets[e], offsets[e+1]) of every permuted buffer
 *   token_pos    [T, k] int32 out: row of (token t, slot j) in the permuted
 *                buffers = offsets[e] + #{t' < t that selected e}; rows inside
 *                a group are therefore in ascending token order
 *   sorted_token [T*k] int32 out: token of each permuted row (inverse map)
 *   sorted_slot  [T*k] int32 out: slot j of each permuted row
 *   tile_offsets [E+1] int32 out: exclusive prefix sum of ceil(counts/tile_m),
 *                for callers running their own tiled GEMM (moe_grouped_gemm
 *                derives its own schedule from offsets); tile_m >= 1
 * Indices, counts, offsets and positions are bit-exact and deterministic
 * (no order-dependent atomics). T = 0 writes zero counts and offsets. */
moe_status moe_route(const float *logits, int64_t T, int32_t E, int32_t k, int32_t tile_m,
                     int32_t *topk_idx, float *topk_gate, int32_t *counts, int32_t *offsets,
                     int32_t *token_pos, int32_t *sorted_token, int32_t *sorted_slot,
                     int32_t *tile_offsets, void *ws, size_t ws_bytes, void *stream);

/* moe_route for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, outputs and errors as moe_route without (ws, ws_bytes).
 * Its scratch is a MOE_ROUTE_NOALLOC_SCRATCH_BYTES (4 MiB) array that the
 * library holds on each GPU it runs on until the process ends; the call
 * allocates nothing. Sizes whose moe_route_workspace_size(T, E, k) exceeds
 * it (T > 524288 at E = 128, T > 262144 at E = 256) return
 * MOE_ERR_WORKSPACE with nothing enqueued. All calls on one GPU share its
 * array: calls that overlap in time on one GPU (different streams, or
 * threads) race and must be serialised by the caller. What an earlier call
 * left in the array is never read. The first call on a device looks up the
 * array's address (with that device current); a failed lookup returns
 * MOE_ERR_LAUNCH. */
#define MOE_ROUTE_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
moe_status moe_route_noalloc(const float *logits, int64_t T, int32_t E, int32_t k, int32_t tile_m,
                             int32_t *topk_idx, float *topk_gate, int32_t *counts,
                             int32_t *offsets, int32_t *token_pos, int32_t *sorted_token,
                             int32_t *sorted_slot, int32_t *tile_offsets, void *stream);

/* ------------------------------------------------------------------ */
/* Dispatch and combine                                                 */

/* Row-wise dispatch: every token row is read once and written to its k rows
 * of the per-expert buffer: x_perm[token_pos[t, j]] = x[t], bit for bit.
 *   x        [T, d] in dtype dt (MXFP8: E4M3 bytes)
 *   x_scale  [T, d/32] E8M0 bytes (MXFP8 only, else ignored)
 *   token_pos[T, k] int32; entries < 0 are dropped rows (padded baseline)
 *   x_perm   [T*k, d] out (rows of dropped entries are not written)
 *   x_perm_scale [T*k, d/32] out (MXFP8 only) */
moe_status moe_permute(const void *x, const uint8_t *x_scale, moe_dtype dt, int64_t T, int32_t d,
                       int32_t k, const int32_t *token_pos, void *x_perm, uint8_t *x_perm_scale,
                       void *stream);

/* Gate-weighted combine back to token order:
 *   out[t] = sum_{j<k} topk_gate[t, j] * y_perm[token_pos[t, j]]
 * summed in fp32 in ascending j, then rounded (to nearest even) to dt.
 * Entries with token_pos < 0 contribute nothing. dt is MOE_F32 or MOE_BF16
 * (y_perm and out share it). */
moe_status moe_combine(const void *y_perm, moe_dtype dt, const float *topk_gate,
                       const int32_t *token_pos, int64_t T, int32_t d, int32_t k, void *out,
                       void *stream);

/* ------------------------------------------------------------------ */
/* Device-scheduled grouped GEMM                                         */

enum { MOE_GG_FWD = 0, MOE_GG_DGRAD = 1, MOE_GG_WGRAD = 2 };
enum { MOE_EPI_NONE = 0, MOE_EPI_SWIGLU_FWD = 1, MOE_EPI_SWIGLU_BWD = 2 };

/* One grouped GEMM over E groups of rows. Group g owns rows
 * [offsets[g], offsets[g+1]) of the row-indexed operands; offsets is read on
 * the device, so the host never learns the group sizes. A persistent grid
 * walks every tile of every group; groups of 0 rows cost nothing in FWD and
 * DGRAD and produce zeros in WGRAD.
 *
 * mode MOE_GG_FWD:   C[r, n]    = sum_k A[r, k] * B[g][n, k]
 *                    A [rows, K], B [E, N, K], C [rows, N]
 * mode MOE_GG_DGRAD: C[r, n]    = sum_k A[r, k] * B[g][k, n]
 *                    A [rows, K], B [E, K, N], C [rows, N]
 * mode MOE_GG_WGRAD: C[g][m, n] = sum_{r in g} A[r, m] * B[r, n]
 *                    A [rows, M], B [rows, N], C [E, M, N] fp32, overwritten,
 *                    or with accumulate = 1: C[g][m, n] += that sum (one
 *                    fp32 add per element; a group of 0 rows leaves C[g]
 *                    unchanged). For gradient accumulation over
 *                    micro-batches between optimizer steps, the window the
 *                    report's data-parallel setup keeps the weights for
 *                    (kongchang.com, "capacity tax").
 *
 * epilogue MOE_EPI_SWIGLU_FWD (mode FWD, N = 2h, B = W1 [E, 2h, d]):
 *   C = AB [rows, 2h] (gate pre-activation a in columns 0..h-1, up b in
 *   h..2h-1) and aux_out = H' [rows, h] = silu(a) * b computed from the fp32
 *   accumulators.
 * epilogue MOE_EPI_SWIGLU_BWD (mode DGRAD, N = h, A = dy [rows, d],
 *   B = W2 [E, d, h]): the product dH' [rows, h] is not stored; with
 *   aux = AB [rows, 2h] and s = sigmoid(a): C = dAB [rows, 2h] with
 *   dA = dH' * b * s * (1 + a (1 - s)) in columns 0..h-1 and
 *   dB = dH' * silu(a) in h..2h-1.
 *
 * dtype MOE_F32 or MOE_BF16: A, B and C (except WGRAD's fp32 C) have that
 * dtype; accumulation is fp32; stores round to nearest even.
 * dtype MOE_MXFP8: operands are E4M3 bytes with E8M0 scales (a_scale,
 * b_scale; 4-byte aligned), one per 32 elements along the reduction, and
 * both operands are given K-contiguous in every mode:
 *   FWD / DGRAD: A [rows, K] with scales [rows, K/32]; B [E, N, K] with
 *     scales [E, N, K/32] (for DGRAD that is the weight in its second
 *     orientation, e.g. mxfp8_quantize axis 0 of W[e] per expert); K % 128 == 0;
 *     C (and AB / H' / dAB of the epilogues) is bf16;
 *   WGRAD: A and B in the column-block layout of mxfp8_quantize (axis 0,
 *     groups = offsets): A holds the [rows, M] operand, B the [rows, N]
 *     operand; C [E, M, N] fp32. Their scale arrays must be sized by
 *     mxfp8_col_blocks (the kernel may read up to 12 bytes past the last
 *     used scale byte, into the spare blocks). rows <= 2^24 (MOE_ERR_SHAPE
 *     otherwise): the kernel addresses the 256 rows of a B tile in one
 *     group's column block with 32-bit offsets from one base.
 * epilogue MOE_EPI_SWIGLU_FWD with dtype MOE_MXFP8 and aux_out_scale set: H'
 *   is not stored in bf16 but handed to GEMM2 and to GEMM2's weight
 *   gradient already quantised, in the two layouts mxfp8_quantize_both
 *   writes for it (groups = offsets), from the bf16-rounded values the plain
 *   epilogue would store (the same bytes, padding rows of the column layout
 *   written as zeros):
 *     aux_out            E4M3 [rows, h], blocks of 32 along h (axis 1),
 *     aux_out_scale      E8M0 [rows, h/32],
 *     aux_out_cols       E4M3 column-block layout along the rows of each
 *                        group (axis 0), sized by mxfp8_col_blocks(rows, E),
 *     aux_out_cols_scale its E8M0 scales.
 *   All four must be set (aux_out and aux_out_cols 16-byte aligned, the
 *   scales 4-byte aligned) or aux_out_scale null. MXFP8 quantisation of a GEMM input along its own
 *   reduction axis is the pages' recipe (aikraft.ru, technical
 *   optimisations: MXFP8 with 32-element scales); doing it in the producing
 *   GEMM saves the bf16 H' round trip through HBM.
 * aux_out_cols and aux_out_cols_scale are ignored unless aux_out_scale is
 * set; aux_out_scale must be null for every other epilogue and dtype.
 */
typedef struct moe_gemm_desc {
    int32_t mode;          /* MOE_GG_* */
    int32_t dtype;         /* MOE_F32 | MOE_BF16 | MOE_MXFP8 */
    int32_t epilogue;      /* MOE_EPI_* */
    int32_t n_groups;      /* E */
    int64_t rows;          /* total rows of the row-indexed operands (T*k) */
    int32_t M, N, K;       /* FWD/DGRAD: N, K used (M is per group); WGRAD: M, N */
    const int32_t *offsets;  /* device [n_groups + 1] */
    const void *A;
    const void *B;
    void *C;
    const uint8_t *a_scale;  /* MXFP8 */
    const uint8_t *b_scale;  /* MXFP8 */
    const void *aux;         /* SWIGLU_BWD: AB [rows, 2h] */
    void *aux_out;           /* SWIGLU_FWD: H' [rows, h] */
    uint8_t *aux_out_scale;  /* SWIGLU_FWD with MXFP8: H' quantised along h, scales */
    void *ws;                /* scratch (split-K partials); may be null if ws_bytes = 0 */
    size_t ws_bytes;
    int32_t accumulate;      /* WGRAD only: 1 = C[g] += the product (fp32 add), 0 = overwrite */
    uint8_t *aux_out_cols;        /* SWIGLU_FWD with MXFP8 and aux_out_scale: H' along rows */
    uint8_t *aux_out_cols_scale;  /* ... and its scales */
} moe_gemm_desc;

/* Scratch bytes moe_grouped_gemm needs for this descriptor (0 when none). */
size_t moe_grouped_gemm_workspace_size(const moe_gemm_desc *g);

moe_status moe_grouped_gemm(const moe_gemm_desc *g, void *stream);

/* Host-side bound of the grouped GEMM's reads: no device work, no GPU
 * needed. Walks, on the host, every global -> LDS copy that
 * moe_grouped_gemm would issue for descriptor g, in the kernel
 * configuration the library launches for g's dtype and mode, with the group
 * offsets host_offsets[0 .. n_groups] (host memory, non-decreasing, from 0
 * to g->rows). Only g's mode, dtype, epilogue, n_groups, rows, M, N and K
 * are used; its pointers are neither read nor dereferenced. The walk
 * computes each copy's source with the same code the kernels run
 * (copy_plan.h), so it checks the copies against the operand extents the
 * caller states: w->extent[i] bytes readable from A, B, a_scale, b_scale
 * (i = 0..3; the scale extents matter for MXFP8 only). On return w holds
 * the number of copies (16-byte operand chunks and MXFP8 scale reads) and
 * of those that take zeros instead of memory (K past a group's end), the
 * lowest and one-past-highest byte read from each operand, and the first
 * read outside [0, extent) if any (first_bad = operand index, else -1).
 * MOE_ERR_DTYPE for MOE_F32 (its kernel stages through registers, not
 * through these copies) and for invalid modes; MOE_ERR_SHAPE for shapes
 * moe_grouped_gemm rejects or offsets that do not match rows. */
typedef struct moe_copy_walk {
    int64_t extent[4];      /* in: readable bytes of A, B, a_scale, b_scale */
    int64_t copies;         /* out */
    int64_t zero_copies;
    int64_t lowest[4];      /* INT64_MAX for an operand nothing was read from */
    int64_t end[4];         /* 0 for an operand nothing was read from */
    int32_t first_bad;      /* -1: every read in bounds */
    int64_t bad_offset;     /* first out-of-bounds read: its byte offset */
    int64_t bad_bytes;      /* and its size */
} moe_copy_walk;

moe_status moe_gemm_copy_walk(const moe_gemm_desc *g, const int32_t *host_offsets,
                              moe_copy_walk *w);

/* Host-side bound of the stores of the MXFP8 SwiGLU forward that writes H'
 * quantised (moe_grouped_gemm with aux_out_scale set): no device work, no
 * GPU needed. Walks every store its epilogue would issue for descriptor g
 * (mode FWD, epilogue SWIGLU_FWD, dtype MXFP8; only n_groups, rows and N = 2h
 * are used) with the group offsets host_offsets[0 .. n_groups], computing
 * each store's byte offset with the code the kernel runs. The four outputs
 * are the walk's operands: w->extent[0..3] = writable bytes of aux_out,
 * aux_out_scale, aux_out_cols, aux_out_cols_scale. On return w->copies is the
 * number of stores, lowest / end the lowest and one-past-highest byte
 * written in each output, first_bad the first output written outside
 * [0, extent) (-1 if none). MOE_ERR_DTYPE for any other mode, epilogue or
 * dtype; MOE_ERR_SHAPE as for moe_gemm_copy_walk. */
moe_status moe_gemm_hp_store_walk(const moe_gemm_desc *g, const int32_t *host_offsets,
                                  moe_copy_walk *w);

/* ------------------------------------------------------------------ */
/* Backward of the whole layer                                          */

/* Backward of route -> permute -> GEMM1 + SwiGLU -> GEMM2 -> combine.
 * Enqueues, in order: combine-bwd with the router backward fused in
 * (dy_perm, dgate, dlogits), GEMM2-dgrad with the SwiGLU backward (dAB),
 * GEMM2-wgrad (dW2), GEMM1-dgrad (dx_perm), unpermute-bwd (dX),
 * GEMM1-wgrad (dW1). Saved forward tensors and the three intermediates are
 * caller-owned buffers.
 *   dlogits[t, e] = g_i (dg_i - sum_j g_j dg_j) for e = topk_idx[t, i]
 *   (evaluated as g_i sum_j g_j (dg_i - dg_j), equal since the gates sum to
 *   one, so a confident router's small gradients lose no precision), and
 *   exactly 0 for unselected experts, with dg_j = <dOut[t], y_perm[row]>.
 * dtype MOE_F32 or MOE_BF16: activations, weights, dOut, dX and the
 * intermediates in that dtype. dW1, dW2, dlogits and dgate are fp32.
 * dtype MOE_MXFP8: activations, dOut, dX and the intermediates are bf16
 * (x_perm is not needed; x and sorted_token are); the four backward GEMMs
 * run in MXFP8 on operands the call quantises itself into ws: dy_perm along
 * d and along rows, H' along rows, dAB along 2h and along rows, and the rows
 * x[sorted_token] along rows. dy_perm is quantised as it is formed from the
 * dOut rows and the gates, and never stored: the dy_perm buffer serves as
 * scratch (its first 4*T*k bytes receive each routed row's gate, fp32) and
 * does not hold dy_perm on return. The weights come pre-quantised in their second
 * orientation (w1t/w1t_scale = W1[e] along 2h as [E, d, 2h];
 * w2t/w2t_scale = W2[e] along d as [E, h, d]; see mxfp8_quantize axis 0),
 * i.e. once per weight update. Needs d % 128 == 0, h % 128 == 0 and
 * T*k <= 2^24 (the bound of MXFP8 WGRAD in moe_grouped_gemm). */
typedef struct moe_bwd_desc {
    int32_t dtype;
    int32_t d, h, E, k;
    int64_t T;
    /* saved from the forward */
    const void *x_perm;        /* [T*k, d] */
    const void *ab;            /* [T*k, 2h] */
    const void *hp;            /* [T*k, h] */
    const void *y_perm;        /* [T*k, d] */
    const float *topk_gate;    /* [T, k] */
    const int32_t *topk_idx;   /* [T, k] */
    const int32_t *token_pos;  /* [T, k] */
    const int32_t *offsets;    /* [E+1] */
    const void *w1;            /* [E, 2h, d] */
    const void *w2;            /* [E, d, h] */
    const void *dout;          /* [T, d] */
    /* outputs */
    void *dx;                  /* [T, d] */
    float *dlogits;            /* [T, E] */
    float *dw1;                /* [E, 2h, d] */
    float *dw2;                /* [E, d, h] */
    float *dgate;              /* [T, k], may be null */
    /* caller-owned intermediates */
    void *dy_perm;             /* [T*k, d] */
    void *dab;                 /* [T*k, 2h] */
    void *dx_perm;             /* [T*k, d] */
    /* MXFP8 only */
    const void *x;                 /* [T, d] bf16 layer input */
    const int32_t *sorted_token;   /* [T*k] from moe_route */
    const uint8_t *w1t;            /* [E, d, 2h] E4M3 */
    const uint8_t *w1t_scale;      /* [E, d, 2h/32] */
    const uint8_t *w2t;            /* [E, h, d] E4M3 */
    const uint8_t *w2t_scale;      /* [E, h, d/32] */
    void *ws;                      /* scratch, moe_backward_workspace_size bytes */
    size_t ws_bytes;
    int32_t accumulate_dw;         /* 1: dW1, dW2 += this micro-batch's gradients; 0: overwrite */
    /* Optional (null = none): MOE_BWD_MAX_STAGES hipEvent_t handles (null
     * entries skipped), created by the caller. Event i is recorded on the
     * stream right after the call's i-th kernel is enqueued, so a caller can
     * time each stage on the stream it runs on. Stages, bf16 / f32:
     *   0 combine-bwd + router-bwd, 1 GEMM2 dgrad + SwiGLU-bwd, 2 GEMM2 wgrad,
     *   3 GEMM1 dgrad, 4 unpermute-bwd, 5 GEMM1 wgrad;
     * MXFP8:
     *   0 combine-bwd + router-bwd, 1 quantise dy (both layouts),
     *   2 GEMM2 dgrad + SwiGLU-bwd, 3 quantise H' (columns), 4 GEMM2 wgrad,
     *   5 quantise dAB (both layouts), 6 GEMM1 dgrad, 7 unpermute-bwd,
     *   8 quantise x[sorted_token] (columns), 9 GEMM1 wgrad.
     * A stage with no work (T = 0, or stage 3 with hp_cols given) still
     * records its event. A failed record returns MOE_ERR_LAUNCH. */
    void *const *stage_events;
    /* MXFP8 only, optional (null = none): H' already quantised along rows per
     * expert (the column-block layout of mxfp8_quantize axis 0 with `offsets`,
     * mxfp8_col_blocks(T*k, E) blocks; e.g. from the forward's
     * mxfp8_quantize_both of H', which also gives GEMM2's operand). When
     * given, GEMM2-wgrad uses it and `hp` is not read (it may be null). */
    const uint8_t *hp_cols;        /* mxfp8_col_blocks(T*k, E) * 32 * h bytes */
    const uint8_t *hp_cols_scale;  /* mxfp8_col_blocks(T*k, E) * h bytes */
} moe_bwd_desc;

#define MOE_BWD_MAX_STAGES 10

size_t moe_backward_workspace_size(const moe_bwd_desc *b);

/* Where the MXFP8 backward keeps its quantised operands inside ws (byte
 * offsets, 256-aligned, in this order, each region up to the next offset):
 *   row_q, row_s   dy along d, then dAB along 2h (row blocks) and scales;
 *   col0_q, col0_s dy, then dAB, in the column-block layout per expert;
 *   col1_q, col1_s H', then the gathered x rows, column-block layout;
 *   total          = moe_backward_workspace_size(b).
 * MOE_ERR_DTYPE unless b->dtype is MOE_MXFP8; MOE_ERR_SHAPE as
 * moe_backward. Lets a caller (and the tests) check the regions against the
 * operand sizes of mxfp8_quantize and the reads of moe_gemm_copy_walk. */
typedef struct moe_bwd_ws_layout {
    size_t row_q, row_s, col0_q, col0_s, col1_q, col1_s, total;
} moe_bwd_ws_layout;

moe_status moe_backward_workspace_layout(const moe_bwd_desc *b, moe_bwd_ws_layout *out);

moe_status moe_backward(const moe_bwd_desc *b, void *stream);

/* ------------------------------------------------------------------ */
/* MXFP8 quantisation (OCP Microscaling v1.0)                            */

/* Quantise a [rows, cols] fp32 or bf16 matrix to MXFP8: per block of 32
 * elements, the E8M0 shared exponent is floor(log2(amax)) - 8 (8 = the E4M3
 * maximum exponent), clamped to [-127, 127], -127 for an all-zero block; the
 * elements are x * 2^-shared rounded to nearest even E4M3 and saturated to
 * +-448 (OCP E4M3: bias 7, no infinities, NaN = S.1111.111).
 *   axis = 1: blocks along each row (cols % 32 == 0). q [rows, cols] E4M3,
 *             scale [rows, cols/32].
 *   axis = 0: blocks along each column, for a GEMM that reduces over rows.
 *             Rows are split into n_groups groups by group_offsets (device,
 *             n_groups+1 entries; null = one group of all rows, n_groups
 *             ignored); blocks restart at each group and a group's last block
 *             may be short. Output is transposed per group and each group is
 *             padded to a multiple of 4 blocks (128 rows): with
 *             nb_g = 4*ceil(len_g/128) and bb_g = sum_{g'<g} nb_g',
 *               q[bb_g*32*cols + c*nb_g*32 + i] = element (o_g + i, c) for
 *               i < len_g, and 0 for len_g <= i < nb_g*32;
 *               scale[bb_g*cols + c*nb_g + b] = block b of column c
 *               (blocks wholly past len_g: scale byte 0).
 *             Size q for mxfp8_col_blocks(rows, n_groups) * 32 * cols bytes
 *             and scale for mxfp8_col_blocks(rows, n_groups) * cols bytes.
 *             n_groups <= 1024.
 * row_map (device, nullable): input row r is in[row_map[r]] (a fused
 * gather, e.g. x[sorted_token] for the permuted rows).
 * in_dt: MOE_F32 or MOE_BF16. */
moe_status mxfp8_quantize(const void *in, moe_dtype in_dt, int64_t rows, int64_t cols,
                          int32_t axis, const int32_t *group_offsets, int32_t n_groups,
                          const int32_t *row_map, uint8_t *q, uint8_t *scale, void *stream);

/* Worst-case block count of the column-block layout: rows/32 + 4*n_groups + 4. */
size_t mxfp8_col_blocks(int64_t rows, int32_t n_groups);

/* Both orientations from one read of the input: q_rows / s_rows exactly as
 * mxfp8_quantize with axis = 1, and q_cols / s_cols exactly as axis = 0 with
 * these groups. Its use here is the once-per-optimizer-step re-quantisation
 * of the fp32 master weights (the report keeps FP32 masters and quantises to
 * MXFP8 for the GEMMs, kongchang.com "caveats behind the numbers"): W [E*R, C] along C
 * for the forward GEMMs and, per expert (group_offsets = e*R), along R for
 * the backward ones, reading the 4-byte masters once instead of twice. Same
 * limits, layouts and alignment as mxfp8_quantize (no row_map). */
moe_status mxfp8_quantize_both(const void *in, moe_dtype in_dt, int64_t rows, int64_t cols,
                               const int32_t *group_offsets, int32_t n_groups, uint8_t *q_rows,
                               uint8_t *s_rows, uint8_t *q_cols, uint8_t *s_cols, void *stream);

/* ------------------------------------------------------------------ */
/* Padded-capacity alternative (for comparison)                         */

/* The report measures the device-scheduled grouped GEMM against padding every
 * expert's batch to one uniform capacity (Ai2 Olmo-core 3, kongchang.com,
 * "routing is a systems problem"). These two calls turn the dropless routing
 * metadata of moe_route into that layout, so that moe_permute, the grouped
 * GEMM, moe_combine and moe_backward run on it unchanged:
 *   expert e owns rows [e*C, (e+1)*C) of [E*C, .] buffers; its routed rows
 *   keep their rank in ascending token order, the ones of rank >= C are
 *   dropped (position -1: not dispatched, no contribution to the output, no
 *   gradient, gates not renormalised).
 *
 * moe_capacity_pad: token_pos_pad[t, j] = e*C + r if r < C, else -1, where
 * e = topk_idx[t, j] and r = token_pos[t, j] - offsets[e]; offsets_pad[e] =
 * e*C for e = 0..E (device, E+1 entries). Inputs are moe_route's outputs.
 * Needs E*C < 2^31.
 *
 * moe_capacity_zero_rows: zeroes the unused capacity rows of a [E*C, cols]
 * buffer (dt = MOE_F32 or MOE_BF16, 16-byte aligned), i.e. rows
 * [e*C + min(c_e, C), (e+1)*C) of every expert, with c_e from the dropless
 * offsets. Call it on the dispatch buffer after moe_permute and on dy_perm
 * before moe_backward, so empty rows contribute nothing to dW. */
moe_status moe_capacity_pad(const int32_t *topk_idx, const int32_t *token_pos,
                            const int32_t *offsets, int64_t T, int32_t E, int32_t k,
                            int32_t capacity, int32_t *token_pos_pad, int32_t *offsets_pad,
                            void *stream);
moe_status moe_capacity_zero_rows(void *buf, moe_dtype dt, const int32_t *offsets, int32_t E,
                                  int32_t capacity, int32_t cols, void *stream);

/* ------------------------------------------------------------------ */
/* Load-balance statistics and the auxiliary balancing loss             */

/* The report reads the load-balancing loss as part of the routing interface
 * and names "token gerrymandering": the loss improves while the imbalance
 * between experts grows (Ai2 Olmo-core 3, kongchang.com, "routing is a
 * systems problem"; bytechap.com, "What you can do": monitor it in the
 * routing metrics). The pages print no formula. This call computes the
 * published Switch Transformer balancing loss (Fedus, Zoph and Shazeer 2021)
 * for top-k routing, next to the hard-load statistics it can drift from:
 *   f_e = counts[e] / (T k),  P_e = (1/T) sum_t softmax(logits[t, :])_e,
 *   L = alpha * E * sum_e f_e P_e.
 * stats (device, MOE_LB_NSTATS fp32, written):
 *   [0] L                 [1] E sum f P (what L/alpha measures; 1 if uniform)
 *   [2] E sum f^2 (hard balance of the counts; 1 if perfectly even)
 *   [3] E sum P^2 (balance of the router probabilities)
 *   [4] max_e c_e / mean   [5] min_e c_e / mean   (mean = T k / E)
 *   [6] coefficient of variation of the counts    [7] experts with no row
 * All zero for T = 0.
 * dlogits (device [T, E] fp32, nullable): if given, dL/dlogits is ADDED to it
 *   (call after moe_backward, which overwrites dlogits with the layer's
 *   gradient); the counts are treated as constants, so
 *   dL/dlogits[t, e] = (alpha E / T) p[t, e] (f_e - sum_j p[t, j] f_j).
 * counts: moe_route's counts (device [E] int32). logits: the routing input
 * (device [T, E] fp32). Limits as moe_route. Deterministic: fixed-order
 * sums, no atomics. Workspace: moe_load_balance_workspace_size(T, E) bytes,
 * 16-byte aligned, caller-owned. */
#define MOE_LB_NSTATS 8
size_t moe_load_balance_workspace_size(int64_t T, int32_t E);
moe_status moe_load_balance(const float *logits, const int32_t *counts, int64_t T, int32_t E,
                            int32_t k, float alpha, float *stats, float *dlogits, void *ws,
                            size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
