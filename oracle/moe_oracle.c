/*
 * moe_oracle.c -- plain, slow CPU oracle for the MoE expert layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may load, call or link
 * this file: only the test suite, the smoke check and the bench's CPU-baseline
 * leg do. It shares no code, header or table with the HIP library.
 *
 * What it computes (the pages describe the layer only in prose):
 *   - every token activates a few of E experts, e.g. 4 of 128, so the active
 *     work per token is fixed while the pool grows
 *     [Ai2 Olmo-core 3, kongchang.com, section "capacity tax"];
 *   - routing metadata (split sizes, per-expert group sizes) is computed on
 *     the GPU [same page, "routing is a systems problem"; aizyradar.cn,
 *     "What changed"];
 *   - the selected token rows are written into the experts' input buffers
 *     [bytechap.com, "How it works"], the expert FFNs run on the uneven
 *     groups [kongchang.com, "routing is a systems problem"], and the results
 *     are weighted and returned to token order.
 * Where the pages are silent this file takes the plainest reading:
 *   - router: softmax over the k selected logits (equal to the full softmax
 *     renormalised over the top k), so each token's gates sum to one;
 *   - selection on fp32 logits, descending, equal logits -> lower expert index
 *     (IEEE equality, so -0 == +0);
 *   - rows inside an expert's group in ascending token order;
 *   - expert FFN = SwiGLU (Shazeer, "GLU Variants Improve Transformer", 2020):
 *     W1[e] is [2h, d] with gate rows 0..h-1 and up rows h..2h-1, W2[e] is
 *     [d, h]; H' = silu(a) * b;
 *   - MXFP8 = the OCP Microscaling v1.0 MXFP8 format the pages name
 *     [kongchang.com, "caveats behind the numbers": one shared scale per 32
 *     elements]: E8M0 shared exponent floor(log2 amax) - 8, E4M3 elements
 *     rounded to nearest even and saturated to +-448.
 *
 * Arithmetic: every dot product is a sequential fp64 sum in ascending index
 * order; values are rounded to the storage dtype only where the layer stores
 * a tensor. Threads split work by output row; each output element is written
 * by exactly one thread, so results do not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_F64 2 /* no storage rounding: used to check gradients by finite differences */

/* ------------------------------------------------------------------ */
/* parallel for (static partition, one output row per index)           */

typedef void (*or_body)(int64_t i, void *ctx);
static int g_threads = 1;

void oracle_set_threads(int n) { g_threads = n < 1 ? 1 : (n > 256 ? 256 : n); }
int oracle_get_threads(void) { return g_threads; }

struct pf_arg { int64_t lo, hi; or_body f; void *ctx; };

static void *pf_run(void *p) {
    struct pf_arg *a = (struct pf_arg *)p;
    for (int64_t i = a->lo; i < a->hi; i++) a->f(i, a->ctx);
    return NULL;
}

static void parallel_for(int64_t n, or_body f, void *ctx) {
    int nt = g_threads;
    if (n <= 0) return;
    if (nt > n) nt = (int)n;
    if (nt <= 1) {
        for (int64_t i = 0; i < n; i++) f(i, ctx);
        return;
    }
    pthread_t th[256];
    struct pf_arg a[256];
    for (int t = 0; t < nt; t++) {
        a[t].lo = n * t / nt;
        a[t].hi = n * (t + 1) / nt;
        a[t].f = f;
        a[t].ctx = ctx;
        pthread_create(&th[t], NULL, pf_run, &a[t]);
    }
    for (int t = 0; t < nt; t++) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------ */
/* rounding to storage dtypes                                           */

/* Nearest bfloat16 value of x (ties to even), returned as a double.
 * bfloat16 keeps 8 significant bits and fp32's exponent range; below 2^-126
 * its step is fixed at 2^-133. */
double oracle_round_bf16(double x) {
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    int e;
    frexp(x, &e);                       /* |x| = m 2^e, m in [0.5, 1) */
    if (e < -125) e = -125;             /* subnormal range: fixed quantum */
    double q = nearbyint(ldexp(x, 8 - e));  /* default mode: ties to even */
    double r = ldexp(q, e - 8);
    const double bf16_max = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    if (fabs(r) > bf16_max) r = copysign(INFINITY, x);
    return r;
}

double oracle_round_f32(double x) { return (double)(float)x; }

static double round_to(int dt, double x) {
    if (dt == OR_F64) return x;
    return dt == OR_BF16 ? oracle_round_bf16(x) : oracle_round_f32(x);
}

static double silu(double a) { return a / (1.0 + exp(-a)); }
static double sigmoid(double a) { return 1.0 / (1.0 + exp(-a)); }

/* ------------------------------------------------------------------ */
/* routing                                                              */

/* Top-k selection, gates, per-expert counts, offsets, row positions.
 *   topk_idx[t,j]  : the j-th best expert of token t (logit descending,
 *                    equal logits -> lower index)
 *   topk_gate[t,j] : exp(l_j - m) / sum_{i<k} exp(l_i - m) in fp64, m = the
 *                    token's top logit, rounded to fp32
 *   counts[e]      : rows routed to e;  offsets[e] = sum_{e'<e} counts[e']
 *   token_pos[t,j] : offsets[e] + #{t' < t : t' selected e}, e = topk_idx[t,j]
 *   sorted_token / sorted_slot : inverse of token_pos
 *   tile_offsets[e]: sum_{e'<e} ceil(counts[e'] / tile_m)
 * Returns 0, or -1 on bad arguments. */
int oracle_route(const float *logits, int64_t T, int32_t E, int32_t k, int32_t tile_m,
                 int32_t *topk_idx, float *topk_gate, int32_t *counts, int32_t *offsets,
                 int32_t *token_pos, int32_t *sorted_token, int32_t *sorted_slot,
                 int32_t *tile_offsets) {
    if (E < 1 || k < 1 || k > E || T < 0 || tile_m < 1) return -1;
    char *taken = (char *)malloc((size_t)E);
    for (int64_t t = 0; t < T; t++) {
        const float *l = logits + t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++) {
                if (taken[e]) continue;
                /* strict '>' while scanning upward keeps the lower index on ties */
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            topk_idx[t * k + j] = best;
        }
        double m = (double)l[topk_idx[t * k]];
        double z = 0.0;
        for (int j = 0; j < k; j++) z += exp((double)l[topk_idx[t * k + j]] - m);
        for (int j = 0; j < k; j++)
            topk_gate[t * k + j] = (float)(exp((double)l[topk_idx[t * k + j]] - m) / z);
    }
    free(taken);

    for (int e = 0; e < E; e++) counts[e] = 0;
    for (int64_t i = 0; i < T * k; i++) counts[topk_idx[i]]++;
    offsets[0] = 0;
    tile_offsets[0] = 0;
    for (int e = 0; e < E; e++) {
        offsets[e + 1] = offsets[e] + counts[e];
        tile_offsets[e + 1] = tile_offsets[e] + (counts[e] + tile_m - 1) / tile_m;
    }
    int32_t *next = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    for (int e = 0; e < E; e++) next[e] = offsets[e];
    for (int64_t t = 0; t < T; t++)
        for (int j = 0; j < k; j++) {
            int e = topk_idx[t * k + j];
            int32_t p = next[e]++;
            token_pos[t * k + j] = p;
            sorted_token[p] = (int32_t)t;
            sorted_slot[p] = j;
        }
    free(next);
    return 0;
}

/* ------------------------------------------------------------------ */
/* expert FFN, one routed row at a time                                 */

struct rows_ctx {
    int64_t n; int32_t d, h, dt;
    const double *x;                /* [n, d] rows fed to the experts */
    const int32_t *expert;          /* [n] */
    const double *const *W1;        /* per expert [2h, d] */
    const double *const *W2;        /* per expert [d, h]  */
    double *ab, *hp, *y;            /* [n,2h], [n,h], [n,d] */
    const double *hp_in;            /* optional: H' fed to GEMM2 instead of hp */
};

static void rows_fwd_body(int64_t r, void *vc) {
    struct rows_ctx *c = (struct rows_ctx *)vc;
    const int d = c->d, h = c->h;
    const double *x = c->x + r * d;
    const double *w1 = c->W1[c->expert[r]];
    const double *w2 = c->W2[c->expert[r]];
    double *ab = c->ab + r * 2 * h, *hp = c->hp + r * h, *y = c->y + r * d;
    /* GEMM1: a_j = sum_c x_c W1[j,c], b_j = sum_c x_c W1[h+j,c]; store AB rounded */
    for (int j = 0; j < h; j++) {
        double a = 0.0, b = 0.0;
        for (int q = 0; q < d; q++) {
            a += x[q] * w1[(int64_t)j * d + q];
            b += x[q] * w1[(int64_t)(h + j) * d + q];
        }
        ab[j] = round_to(c->dt, a);
        ab[h + j] = round_to(c->dt, b);
        /* SwiGLU from the unrounded pre-activations */
        hp[j] = round_to(c->dt, silu(a) * b);
    }
    /* GEMM2 consumes the stored (rounded) H' -- or a caller-given one */
    const double *g2 = c->hp_in ? c->hp_in + r * h : hp;
    for (int q = 0; q < d; q++) {
        double s = 0.0;
        for (int j = 0; j < h; j++) s += g2[j] * w2[(int64_t)q * h + j];
        y[q] = round_to(c->dt, s);
    }
}

/* Forward of the expert FFN for n rows: AB (rounded), H' (rounded), y (rounded).
 * Row r uses expert expert[r] and input row x[r]. If hp_in is non-null, GEMM2
 * reads it instead of the freshly computed H' (lets a caller feed a quantised
 * H'). All outputs are doubles holding values of the storage dtype. */
void oracle_rows_fwd(int64_t n, int32_t d, int32_t h, int32_t dt, const double *x,
                     const int32_t *expert, const double *const *W1, const double *const *W2,
                     const double *hp_in, double *ab, double *hp, double *y) {
    struct rows_ctx c = {n, d, h, dt, x, expert, W1, W2, ab, hp, y, hp_in};
    parallel_for(n, rows_fwd_body, &c);
}

struct bwd_ctx {
    int64_t n; int32_t d, h, dt;
    const int32_t *expert;
    const double *const *W1, *const *W2;
    const double *dy;     /* [n,d]  stored dy_perm rows (already rounded) */
    const double *ab;     /* [n,2h] stored AB rows */
    double *dab;          /* [n,2h] */
    double *dx;           /* [n,d]  */
    const double *dab_in; /* optional: dAB fed to the dgrad instead of dab */
};

static void rows_bwd_body(int64_t r, void *vc) {
    struct bwd_ctx *c = (struct bwd_ctx *)vc;
    const int d = c->d, h = c->h;
    const double *w1 = c->W1[c->expert[r]];
    const double *w2 = c->W2[c->expert[r]];
    const double *dy = c->dy + r * d, *ab = c->ab + r * 2 * h;
    double *dab = c->dab + r * 2 * h, *dx = c->dx + r * d;
    /* dH'_j = sum_q dy_q W2[q, j]  (not stored);  SwiGLU backward from the
       stored a, b:  s = sigmoid(a), dA = dH' b s (1 + a (1 - s)), dB = dH' silu(a) */
    /* loops run q (resp. j) outermost so the weights are read row by row;
       every output element still sums its terms in ascending order */
    double *g = (double *)calloc((size_t)(h > d ? h : d), sizeof(double));
    for (int q = 0; q < d; q++)
        for (int j = 0; j < h; j++) g[j] += dy[q] * w2[(int64_t)q * h + j];
    for (int j = 0; j < h; j++) {
        double a = ab[j], b = ab[h + j], s = sigmoid(a);
        dab[j] = round_to(c->dt, g[j] * b * s * (1.0 + a * (1.0 - s)));
        dab[h + j] = round_to(c->dt, g[j] * a * s);
    }
    const double *g1 = c->dab_in ? c->dab_in + r * 2 * h : dab;
    /* dx_q = sum_j dAB_j W1[j, q] */
    for (int q = 0; q < d; q++) g[q] = 0.0;
    for (int j = 0; j < 2 * h; j++)
        for (int q = 0; q < d; q++) g[q] += g1[j] * w1[(int64_t)j * d + q];
    for (int q = 0; q < d; q++) dx[q] = round_to(c->dt, g[q]);
    free(g);
}

/* Backward of the expert FFN for n rows, given the stored dy_perm rows and
 * stored AB rows: dAB (rounded) and dx_perm (rounded). */
void oracle_rows_bwd(int64_t n, int32_t d, int32_t h, int32_t dt, const int32_t *expert,
                     const double *const *W1, const double *const *W2, const double *dy,
                     const double *ab, const double *dab_in, double *dab, double *dx) {
    struct bwd_ctx c = {n, d, h, dt, expert, W1, W2, dy, ab, dab, dx, dab_in};
    parallel_for(n, rows_bwd_body, &c);
}

/* ------------------------------------------------------------------ */
/* weight gradients of one expert (K-grouped: a sum over its rows)      */

struct wg_ctx {
    int64_t n; int32_t m, nn;
    const double *a;   /* [n, m] */
    const double *b;   /* [n, nn] */
    double *c;         /* [m, nn] */
};

static void wgrad_body(int64_t i, void *vc) {
    struct wg_ctx *c = (struct wg_ctx *)vc;
    double *out = c->c + i * c->nn;
    for (int j = 0; j < c->nn; j++) out[j] = 0.0;
    for (int64_t r = 0; r < c->n; r++) {
        double av = c->a[r * c->m + i];
        const double *brow = c->b + r * c->nn;
        for (int j = 0; j < c->nn; j++) out[j] += av * brow[j];
    }
    for (int j = 0; j < c->nn; j++) out[j] = (double)(float)out[j];
}

/* C[i, j] = round_f32( sum_{r=0}^{n-1} A[r, i] * B[r, j] ), r ascending.
 * With n = 0 the result is all zeros. Used for dW2[e] = dy^T H' and
 * dW1[e] = dAB^T x over the rows of expert e. */
void oracle_wgrad(int64_t n, int32_t m, int32_t nn, const double *a, const double *b, double *c) {
    struct wg_ctx ctx = {n, m, nn, a, b, c};
    parallel_for(m, wgrad_body, &ctx);
}

/* ------------------------------------------------------------------ */
/* combine, its backward, unpermute backward, router backward            */

/* out[t] = round( sum_{j<k} g[t,j] * y_perm[token_pos[t,j]] ), j ascending. */
void oracle_combine(int64_t T, int32_t d, int32_t k, int32_t dt, const float *gate,
                    const int32_t *token_pos, const double *y_perm, double *out) {
    for (int64_t t = 0; t < T; t++)
        for (int q = 0; q < d; q++) {
            double s = 0.0;
            for (int j = 0; j < k; j++)
                s += (double)gate[t * k + j] * y_perm[(int64_t)token_pos[t * k + j] * d + q];
            out[t * d + q] = round_to(dt, s);
        }
}

/* Combine backward for the rows of token t:
 *   dy_perm[token_pos[t,j]] = round(g[t,j] * dOut[t])
 *   dgate[t,j]              = sum_q dOut[t,q] * y_perm[token_pos[t,j], q]   */
void oracle_combine_bwd(int64_t T, int32_t d, int32_t k, int32_t dt, const float *gate,
                        const int32_t *token_pos, const double *dout, const double *y_perm,
                        double *dy_perm, double *dgate) {
    for (int64_t t = 0; t < T; t++)
        for (int j = 0; j < k; j++) {
            int64_t p = token_pos[t * k + j];
            double g = (double)gate[t * k + j], s = 0.0;
            for (int q = 0; q < d; q++) {
                dy_perm[p * d + q] = round_to(dt, g * dout[t * d + q]);
                s += dout[t * d + q] * y_perm[p * d + q];
            }
            dgate[t * k + j] = s;
        }
}

/* dlogits[t, e] = g_i (dg_i - sum_j g_j dg_j) where e = topk_idx[t,i]; every
 * unselected expert gets exactly 0 (the derivative of a softmax over the
 * selected logits). Rounded to fp32. */
void oracle_router_bwd(int64_t T, int32_t E, int32_t k, const int32_t *topk_idx,
                       const float *gate, const double *dgate, double *dlogits) {
    for (int64_t t = 0; t < T; t++) {
        double dot = 0.0;
        for (int j = 0; j < k; j++) dot += (double)gate[t * k + j] * dgate[t * k + j];
        for (int e = 0; e < E; e++) dlogits[t * E + e] = 0.0;
        for (int j = 0; j < k; j++) {
            double g = (double)gate[t * k + j];
            dlogits[t * E + topk_idx[t * k + j]] = (double)(float)(g * (dgate[t * k + j] - dot));
        }
    }
}

/* dX[t] = round( sum_{j<k} dx_perm[token_pos[t,j]] ), j ascending. */
void oracle_unpermute_bwd(int64_t T, int32_t d, int32_t k, int32_t dt,
                          const int32_t *token_pos, const double *dx_perm, double *dx) {
    for (int64_t t = 0; t < T; t++)
        for (int q = 0; q < d; q++) {
            double s = 0.0;
            for (int j = 0; j < k; j++) s += dx_perm[(int64_t)token_pos[t * k + j] * d + q];
            dx[t * d + q] = round_to(dt, s);
        }
}

/* ------------------------------------------------------------------ */
/* MXFP8 (OCP Microscaling v1.0, MXFP8 = E4M3 elements + E8M0 scale)     */

/* E4M3 (bias 7, no infinities, NaN = S.1111.111, max normal 448): encode v
 * with round-to-nearest-even and saturation to +-448. */
uint8_t oracle_e4m3_encode(double v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return sign | 0x7F;
    double a = fabs(v);
    if (a >= 448.0) return sign | 0x7E;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    int E = e - 1;                    /* a = 1.f * 2^E */
    if (E < -6) E = -6;               /* subnormals: step 2^-9 */
    double r = ldexp(nearbyint(ldexp(a, 3 - E)), E - 3);
    if (r == 0.0) return sign;
    if (r > 448.0) r = 448.0;
    frexp(r, &e);
    E = e - 1;
    if (E < -6) return sign | (uint8_t)ldexp(r, 9);           /* 0.mmm * 2^-6 */
    return sign | (uint8_t)((E + 7) << 3) | (uint8_t)(ldexp(r, 3 - E) - 8.0);
}

double oracle_e4m3_decode(uint8_t q) {
    double s = (q & 0x80) ? -1.0 : 1.0;
    int ef = (q >> 3) & 0xF, m = q & 7;
    if (ef == 0xF && m == 7) return NAN;
    if (ef == 0) return s * ldexp((double)m, -9);
    return s * ldexp(8.0 + m, ef - 7 - 3);
}

/* Shared exponent of a block: floor(log2(amax)) - 8, clamped to [-127, 127];
 * a block of zeros gets -127. Returned as the E8M0 byte (exponent + 127). */
uint8_t oracle_mx_scale(double amax) {
    if (!(amax > 0.0)) return 0;
    int e;
    frexp(amax, &e);                  /* floor(log2 amax) = e - 1 */
    int s = (e - 1) - 8;
    if (s < -127) s = -127;
    if (s > 127) s = 127;
    return (uint8_t)(s + 127);
}

/* Quantise a [rows, cols] fp32 matrix to MXFP8.
 *   axis = 1: blocks of 32 consecutive elements along each row (cols % 32 == 0).
 *             q is [rows, cols]; scale is [rows, cols/32].
 *   axis = 0: blocks of 32 consecutive rows within each column, for a GEMM
 *             whose reduction runs over rows. Rows are split into groups by
 *             group_offsets (n_groups+1 entries; null = one group of all rows);
 *             blocks restart at every group start and a group's last block may
 *             be short. The output is transposed per group and each group is
 *             padded to a multiple of 4 blocks (128 rows): with
 *             nb_g = 4*ceil(len_g/128) and bb_g = sum_{g'<g} nb_g',
 *               q[bb_g*32*cols + c*(nb_g*32) + i] = element (o_g + i, c),
 *                 i < len_g; positions len_g <= i < nb_g*32 hold 0;
 *               scale[bb_g*cols + c*nb_g + b] = block b of column c of group g
 *               (blocks wholly past len_g hold scale byte 0).
 * Returns 0, or -1 on bad arguments. */
/* One 32-element block of row r (axis 1). */
struct mxq_rows_ctx { const float *in; int64_t cols; uint8_t *q, *scale; };
static void mxq_rows_body(int64_t r, void *vc) {
    const struct mxq_rows_ctx *c = (const struct mxq_rows_ctx *)vc;
    const int64_t cols = c->cols;
    for (int64_t b = 0; b < cols / 32; b++) {
        const float *v = c->in + r * cols + b * 32;
        double amax = 0.0;
        for (int i = 0; i < 32; i++) if (fabs((double)v[i]) > amax) amax = fabs((double)v[i]);
        uint8_t sb = oracle_mx_scale(amax);
        c->scale[r * (cols / 32) + b] = sb;
        for (int i = 0; i < 32; i++)
            c->q[r * cols + b * 32 + i] = oracle_e4m3_encode(ldexp((double)v[i], 127 - sb));
    }
}

/* Every block of column col of one group (axis 0). */
struct mxq_cols_ctx { const float *in; int64_t cols, row0, len, nb; uint8_t *qg, *sg; };
static void mxq_cols_body(int64_t col, void *vc) {
    const struct mxq_cols_ctx *c = (const struct mxq_cols_ctx *)vc;
    const int64_t cols = c->cols, len = c->len, nb = c->nb;
    for (int64_t b = 0; b < nb; b++) {
        int64_t i0 = b * 32, i1 = i0 + 32 < len ? i0 + 32 : len;
        double amax = 0.0;
        for (int64_t i = i0; i < i1; i++) {
            double v = fabs((double)c->in[(c->row0 + i) * cols + col]);
            if (v > amax) amax = v;
        }
        uint8_t sb = oracle_mx_scale(amax);
        c->sg[col * nb + b] = sb;
        for (int64_t i = i0; i < i0 + 32; i++)
            c->qg[col * nb * 32 + i] = i < i1
                ? oracle_e4m3_encode(ldexp((double)c->in[(c->row0 + i) * cols + col], 127 - sb))
                : 0;
    }
}

/* Blocks are independent and each is written by one thread (rows for axis 1,
 * columns of a group for axis 0), so the bytes do not depend on the thread
 * count. */
int oracle_mxfp8_quantize(const float *in, int64_t rows, int64_t cols, int32_t axis,
                          const int32_t *group_offsets, int32_t n_groups,
                          uint8_t *q, uint8_t *scale) {
    if (axis == 1) {
        if (cols % 32) return -1;
        struct mxq_rows_ctx c = {in, cols, q, scale};
        parallel_for(rows, mxq_rows_body, &c);
        return 0;
    }
    if (axis != 0) return -1;
    int32_t single[2] = {0, (int32_t)rows};
    const int32_t *go = group_offsets ? group_offsets : single;
    int32_t ng = group_offsets ? n_groups : 1;
    int64_t bb = 0;
    for (int g = 0; g < ng; g++) {
        int64_t len = go[g + 1] - go[g], nb = 4 * ((len + 127) / 128);
        struct mxq_cols_ctx c = {in, cols, go[g], len, nb, q + bb * 32 * cols, scale + bb * cols};
        if (nb) parallel_for(cols, mxq_cols_body, &c);
        bb += nb;
    }
    return 0;
}

/* Exact values of an MXFP8 tensor in [rows, cols] order (the inverse of
 * oracle_mxfp8_quantize's layouts): out[r, c] = E4M3 value * 2^(scale - 127). */
struct mxd_ctx { const uint8_t *q, *scale; int64_t cols, row0, len, nb; double *out; int axis; };
static void mxd_rows_body(int64_t r, void *vc) {
    const struct mxd_ctx *c = (const struct mxd_ctx *)vc;
    for (int64_t j = 0; j < c->cols; j++)
        c->out[r * c->cols + j] = ldexp(oracle_e4m3_decode(c->q[r * c->cols + j]),
                                        (int)c->scale[r * (c->cols / 32) + j / 32] - 127);
}
static void mxd_cols_body(int64_t col, void *vc) {
    const struct mxd_ctx *c = (const struct mxd_ctx *)vc;
    for (int64_t i = 0; i < c->len; i++)
        c->out[(c->row0 + i) * c->cols + col] =
            ldexp(oracle_e4m3_decode(c->q[col * c->nb * 32 + i]),
                  (int)c->scale[col * c->nb + i / 32] - 127);
}
int oracle_mxfp8_dequantize(const uint8_t *q, const uint8_t *scale, int64_t rows, int64_t cols,
                            int32_t axis, const int32_t *group_offsets, int32_t n_groups,
                            double *out) {
    if (axis == 1) {
        if (cols % 32) return -1;
        struct mxd_ctx c = {q, scale, cols, 0, rows, 0, out, 1};
        parallel_for(rows, mxd_rows_body, &c);
        return 0;
    }
    if (axis != 0) return -1;
    int32_t single[2] = {0, (int32_t)rows};
    const int32_t *go = group_offsets ? group_offsets : single;
    int32_t ng = group_offsets ? n_groups : 1;
    int64_t bb = 0;
    for (int g = 0; g < ng; g++) {
        int64_t len = go[g + 1] - go[g], nb = 4 * ((len + 127) / 128);
        struct mxd_ctx c = {q + bb * 32 * cols, scale + bb * cols, cols, go[g], len, nb, out, 0};
        if (nb) parallel_for(cols, mxd_cols_body, &c);
        bb += nb;
    }
    return 0;
}

/* Exact value of an MXFP8 element: E4M3 value times 2^(scale - 127). */
double oracle_mxfp8_value(uint8_t q, uint8_t scale) {
    return ldexp(oracle_e4m3_decode(q), (int)scale - 127);
}
