/*
 * oracle.c -- plain, slow CPU oracle of the padding-free MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no source with the GPU library.
 *
 * What it computes (sources are the three web pages on X-MoE):
 *   - "5.4 MoE模型在分布式训练中的应用", section 训练流程 (MoE-layer forward):
 *     gate scores per token, dispatch to experts, local expert compute,
 *     combine back by token ownership; backward runs along the reverse path.
 *   - X-MoE article (adg.csdn.net), section 2.1.1 "PFT数据结构创新": the
 *     Padding-Free Token buffer holds token_ids (position in the input),
 *     expert_ids (target expert), tokens_per_expert (count per expert),
 *     combine_weights (weights used at combine) and x (the token rows).
 *   - same article, section 2.1.2 "跨平台核函数优化": the gather copies row
 *     token_ids[r] of the input into row r of the buffer; the expert GEMM walks
 *     the experts in ascending id and multiplies each expert's rows, in their
 *     original order and without padding, by that expert's weights.
 * The pages give no router or FFN formula.  Readings (also listed in the design
 * notes): softmax over the E experts of s = z*inv_tau + logit_bias with
 * z = x.Wg; top-k of sel = s + select_bias ordered by (sel desc, expert asc);
 * weights = the unrenormalised probabilities p[t, e]; SwiGLU experts
 * FFN(x) = (silu(x.W1) * (x.W3)).W2 with silu(a) = a / (1 + exp(-a)); the
 * backward is the exact gradient with the selection held fixed.
 *
 * Conventions: inputs are read through a dtype tag (fp32, bf16 bit patterns,
 * or fp64) and widened exactly to double; every sum is accumulated in double;
 * floating outputs are double.  The only fp32 rounding points are the ones
 * that decide an integer: the router scores s and the selection keys sel are
 * rounded to fp32 (modes 0 and 1), because the GPU takes its top-k decision in
 * fp32.  Mode 2 keeps everything in double (finite-difference checks).
 *
 * Rows: the expert, combine and transpose steps work on a generic row list.
 * Row r carries token row_token[r], expert row_expert[r] and weight row_w[r].
 * The end-to-end oracle uses slot order (r = t*k + j) and never builds the
 * PFT; per-step checks use the PFT order.  Either way the arithmetic is the
 * definition, row by row.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };
enum { ORC_OK = 0, ORC_EINVAL = 1, ORC_EROUTE = 2, ORC_ENOMEM = 3 };

/* ------------------------------------------------------------------ inputs */

static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double ld(const void *p, int dt, int64_t i) {
    if (dt == ORC_F32) return (double)((const float *)p)[i];
    if (dt == ORC_BF16) return bf16_to_double(((const uint16_t *)p)[i]);
    return ((const double *)p)[i];
}

/* acc[0..n) += a * w[off .. off+n) */
static void axpy(double *acc, double a, const void *w, int dt, int64_t off, int64_t n) {
    if (dt == ORC_BF16) {
        const uint16_t *p = (const uint16_t *)w + off;
        for (int64_t j = 0; j < n; ++j) acc[j] += a * bf16_to_double(p[j]);
    } else if (dt == ORC_F32) {
        const float *p = (const float *)w + off;
        for (int64_t j = 0; j < n; ++j) acc[j] += a * (double)p[j];
    } else {
        const double *p = (const double *)w + off;
        for (int64_t j = 0; j < n; ++j) acc[j] += a * p[j];
    }
}

/* sum_j v[j] * w[off + j] */
static double dot(const double *v, const void *w, int dt, int64_t off, int64_t n) {
    double s = 0.0;
    if (dt == ORC_BF16) {
        const uint16_t *p = (const uint16_t *)w + off;
        for (int64_t j = 0; j < n; ++j) s += v[j] * bf16_to_double(p[j]);
    } else if (dt == ORC_F32) {
        const float *p = (const float *)w + off;
        for (int64_t j = 0; j < n; ++j) s += v[j] * (double)p[j];
    } else {
        const double *p = (const double *)w + off;
        for (int64_t j = 0; j < n; ++j) s += v[j] * p[j];
    }
    return s;
}

static void load_row(double *dst, const void *src, int dt, int64_t off, int64_t n) {
    for (int64_t j = 0; j < n; ++j) dst[j] = ld(src, dt, off + j);
}

static int g_threads = 0;
void orc_set_threads(int n) { g_threads = n; }
int orc_get_threads(void) {
#ifdef _OPENMP
    return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
    return 1;
#endif
}
#define NT orc_get_threads()

/* ----------------------------------------------------------------- routing */

static double silu(double a) { return a / (1.0 + exp(-a)); }
static double sigm(double a) { return 1.0 / (1.0 + exp(-a)); }

/*
 * Gate: z = X[t].Wg, s = z*inv_tau + logit_bias, p = softmax_E(s),
 * sel = s + select_bias, S_t = the k largest sel under (sel desc, expert asc);
 * slot j holds the j-th of them, topk_w[t,j] = p[t, topk_ids[t,j]].
 *   mode 0: z accumulated in fp32 with one fused multiply-add per term in
 *           ascending feature order, starting from +0; s, sel in fp32.
 *   mode 1: z = exact sum (double) rounded once to fp32; s, sel in fp32.
 *   mode 2: everything in double.
 * Outputs (any may be NULL except topk_ids): topk_w [T,k], scores s [T,E],
 * probs p [T,E], margin [T] = sel_(k) - sel_(k+1) (0 when k == E).
 */
int orc_route(const void *x, int x_dt, const void *wg, int wg_dt, int64_t T, int d, int E, int k,
              int mode, double inv_tau, const float *logit_bias, const float *select_bias,
              int32_t *topk_ids, double *topk_w, double *scores, double *probs, double *margin) {
    if (!x || !wg || !topk_ids || T < 0 || d < 1 || E < 1 || k < 1 || k > E || mode < 0 || mode > 2)
        return ORC_EINVAL;
    /* Wg transposed to [E][d] in double (exact widening), so each dot product
       walks contiguous memory */
    double *wgt = (double *)malloc(sizeof(double) * (size_t)d * E);
    if (!wgt) return ORC_ENOMEM;
    for (int i = 0; i < d; ++i)
        for (int e = 0; e < E; ++e) wgt[(int64_t)e * d + i] = ld(wg, wg_dt, (int64_t)i * E + e);
    int rc = ORC_OK;
#pragma omp parallel num_threads(NT)
    {
        double *xr = (double *)malloc(sizeof(double) * (size_t)d);
        double *s = (double *)malloc(sizeof(double) * (size_t)E);
        double *sel = (double *)malloc(sizeof(double) * (size_t)E);
        double *p = (double *)malloc(sizeof(double) * (size_t)E);
        char *taken = (char *)malloc((size_t)E);
        const int ok = (xr && s && sel && p && taken) ? 1 : 0;
        if (!ok) {
#pragma omp atomic write
            rc = ORC_ENOMEM;
        }
        {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < T; ++t) {
                if (!ok) continue;
                load_row(xr, x, x_dt, t * (int64_t)d, d);
                for (int e = 0; e < E; ++e) {
                    if (mode == 0) {
                        float acc = 0.0f;
                        const double *we = wgt + (int64_t)e * d;
                        for (int i = 0; i < d; ++i) acc = fmaf((float)xr[i], (float)we[i], acc);
                        float a = acc * (float)inv_tau;
                        if (logit_bias) a = a + logit_bias[e];
                        float b = select_bias ? a + select_bias[e] : a;
                        s[e] = a;
                        sel[e] = b;
                    } else {
                        const double *we = wgt + (int64_t)e * d;
                        double z = 0.0;
                        for (int i = 0; i < d; ++i) z += xr[i] * we[i];
                        if (mode == 1) {
                            float a = (float)z * (float)inv_tau;
                            if (logit_bias) a = a + logit_bias[e];
                            float b = select_bias ? a + select_bias[e] : a;
                            s[e] = a;
                            sel[e] = b;
                        } else {
                            double a = z * inv_tau + (logit_bias ? (double)logit_bias[e] : 0.0);
                            s[e] = a;
                            sel[e] = a + (select_bias ? (double)select_bias[e] : 0.0);
                        }
                    }
                }
                /* softmax over all E experts, max-shifted, in double */
                double mx = s[0];
                for (int e = 1; e < E; ++e) if (s[e] > mx) mx = s[e];
                double den = 0.0;
                for (int e = 0; e < E; ++e) { p[e] = exp(s[e] - mx); den += p[e]; }
                for (int e = 0; e < E; ++e) p[e] /= den;
                /* top-k by repeated selection; strict '>' keeps the lower index on ties */
                memset(taken, 0, (size_t)E);
                double last = 0.0;
                for (int j = 0; j < k; ++j) {
                    int best = -1;
                    for (int e = 0; e < E; ++e)
                        if (!taken[e] && (best < 0 || sel[e] > sel[best])) best = e;
                    taken[best] = 1;
                    topk_ids[t * k + j] = best;
                    if (topk_w) topk_w[t * k + j] = p[best];
                    last = sel[best];
                }
                if (margin) {
                    if (k == E) margin[t] = 0.0;
                    else {
                        int nb = -1;
                        for (int e = 0; e < E; ++e)
                            if (!taken[e] && (nb < 0 || sel[e] > sel[nb])) nb = e;
                        margin[t] = last - sel[nb];
                    }
                }
                if (scores) memcpy(scores + t * (int64_t)E, s, sizeof(double) * (size_t)E);
                if (probs) memcpy(probs + t * (int64_t)E, p, sizeof(double) * (size_t)E);
            }
        }
        free(xr); free(s); free(sel); free(p); free(taken);
    }
    free(wgt);
    return rc;
}

/* ------------------------------------------------------------------- PFT */

/*
 * Padding-Free Token buffer from a routing result, by nested loops:
 * for each expert e in ascending order, for each token t in ascending order,
 * for each slot j of t that chose e, append one row.  Row r then holds
 * token_ids[r] = t, expert_ids[r] = e, combine_weights[r] = topk_w[t,j] (a
 * bit-for-bit copy) and slot_to_row[t*k+j] = r.  offsets[e] is the first row
 * of expert e, offsets[E] the row count; tokens_per_expert[e] its row count.
 * Nothing is padded and nothing is dropped: a valid routing yields T*k rows.
 * Returns ORC_EROUTE if an id is out of range or a token repeats an expert.
 */
int orc_build_pft(const int32_t *topk_ids, const float *topk_w, int64_t T, int E, int k,
                  int32_t *token_ids, int32_t *expert_ids, int32_t *tokens_per_expert,
                  int32_t *offsets, float *combine_weights, int32_t *slot_to_row) {
    if (!topk_ids || T < 0 || E < 1 || k < 1 || k > E) return ORC_EINVAL;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int32_t e = topk_ids[t * k + j];
            if (e < 0 || e >= E) return ORC_EROUTE;
            for (int i = 0; i < j; ++i)
                if (topk_ids[t * k + i] == e) return ORC_EROUTE;
        }
    int64_t r = 0;
    for (int e = 0; e < E; ++e) {
        if (offsets) offsets[e] = (int32_t)r;
        int64_t cnt = 0;
        for (int64_t t = 0; t < T; ++t)
            for (int j = 0; j < k; ++j)
                if (topk_ids[t * k + j] == e) {
                    if (token_ids) token_ids[r] = (int32_t)t;
                    if (expert_ids) expert_ids[r] = e;
                    if (combine_weights) combine_weights[r] = topk_w ? topk_w[t * k + j] : 0.0f;
                    if (slot_to_row) slot_to_row[t * k + j] = (int32_t)r;
                    ++r;
                    ++cnt;
                }
        if (tokens_per_expert) tokens_per_expert[e] = (int32_t)cnt;
    }
    if (offsets) offsets[E] = (int32_t)r;
    return r == T * (int64_t)k ? ORC_OK : ORC_EROUTE;
}

/* ---------------------------------------------------------------- gather */

/* xs[r, :] = x[row_token[r], :] -- the dispatch copy, widened to double. */
int orc_gather(const void *x, int x_dt, const int32_t *row_token, int64_t rows, int64_t T, int d,
               double *xs) {
    if (!x || !row_token || !xs || d < 1) return ORC_EINVAL;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t t = row_token[r];
        if (t < 0 || t >= T) return ORC_EINVAL;
        load_row(xs + r * d, x, x_dt, t * (int64_t)d, d);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------ expert FFN */

/*
 * Work list for the expert loops: the rows of each expert in ascending row
 * order, cut into blocks of at most ORC_BLOCK rows so each expert's weight rows
 * are reused across a block while they sit in cache.
 */
#define ORC_BLOCK 32
typedef struct { int e; int64_t n; int64_t *rows; } orc_item;

static int64_t build_items(const int32_t *row_expert, int64_t rows, int E, orc_item **items_out,
                           int64_t **rowbuf_out) {
    int64_t *cnt = (int64_t *)calloc((size_t)E + 1, sizeof(int64_t));
    int64_t *rowbuf = (int64_t *)malloc(sizeof(int64_t) * (size_t)(rows > 0 ? rows : 1));
    if (!cnt || !rowbuf) { free(cnt); free(rowbuf); return -1; }
    for (int64_t r = 0; r < rows; ++r) {
        int e = row_expert[r];
        if (e < 0 || e >= E) { free(cnt); free(rowbuf); return -2; }
        cnt[e + 1]++;
    }
    for (int e = 0; e < E; ++e) cnt[e + 1] += cnt[e];
    int64_t *fill = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
    if (!fill) { free(cnt); free(rowbuf); return -1; }
    for (int e = 0; e < E; ++e) fill[e] = cnt[e];
    for (int64_t r = 0; r < rows; ++r) rowbuf[fill[row_expert[r]]++] = r;
    free(fill);
    int64_t nitems = 0;
    for (int e = 0; e < E; ++e) nitems += (cnt[e + 1] - cnt[e] + ORC_BLOCK - 1) / ORC_BLOCK;
    orc_item *items = (orc_item *)malloc(sizeof(orc_item) * (size_t)(nitems > 0 ? nitems : 1));
    if (!items) { free(cnt); free(rowbuf); return -1; }
    int64_t it = 0;
    for (int e = 0; e < E; ++e)
        for (int64_t b = cnt[e]; b < cnt[e + 1]; b += ORC_BLOCK) {
            items[it].e = e;
            items[it].rows = rowbuf + b;
            items[it].n = (cnt[e + 1] - b) < ORC_BLOCK ? (cnt[e + 1] - b) : ORC_BLOCK;
            ++it;
        }
    free(cnt);
    *items_out = items;
    *rowbuf_out = rowbuf;
    return nitems;
}

/* The input row of row r: xs row r, or x row row_token[r] when row_token is given. */
static int64_t in_row(const int32_t *row_token, int64_t r) { return row_token ? row_token[r] : r; }

/*
 * Forward of the SwiGLU experts, one row at a time:
 *   H1 = x.W1[e], H3 = x.W3[e], A = silu(H1) * H3, Ye = A.W2[e]
 * with W1, W3 [E, d, h] and W2 [E, h, d] row-major.  Optional outputs
 * h1, h3, act [rows, h]; required ye [rows, d].
 */
int orc_ffn(const void *xs, int xs_dt, const int32_t *row_token, const int32_t *row_expert,
            int64_t rows, int d, int h, int E, const void *w1, const void *w3, const void *w2,
            int w_dt, double *h1_out, double *h3_out, double *act_out, double *ye) {
    if (!xs || !row_expert || !w1 || !w3 || !w2 || !ye || d < 1 || h < 1 || E < 1) return ORC_EINVAL;
    orc_item *items = NULL;
    int64_t *rowbuf = NULL;
    int64_t nitems = build_items(row_expert, rows, E, &items, &rowbuf);
    if (nitems < 0) return nitems == -2 ? ORC_EINVAL : ORC_ENOMEM;
    int rc = ORC_OK;
#pragma omp parallel num_threads(NT)
    {
        double *X = (double *)malloc(sizeof(double) * ORC_BLOCK * (size_t)d);
        double *H1 = (double *)malloc(sizeof(double) * ORC_BLOCK * (size_t)h);
        double *H3 = (double *)malloc(sizeof(double) * ORC_BLOCK * (size_t)h);
        double *Y = (double *)malloc(sizeof(double) * ORC_BLOCK * (size_t)d);
        const int ok = (X && H1 && H3 && Y) ? 1 : 0;
        if (!ok) {
#pragma omp atomic write
            rc = ORC_ENOMEM;
        }
        {
#pragma omp for schedule(dynamic, 1)
            for (int64_t it = 0; it < nitems; ++it) {
                if (!ok) continue;
                const orc_item *w = &items[it];
                const int64_t e = w->e, nb = w->n;
                for (int64_t b = 0; b < nb; ++b)
                    load_row(X + b * d, xs, xs_dt, in_row(row_token, w->rows[b]) * d, d);
                memset(H1, 0, sizeof(double) * (size_t)(nb * h));
                memset(H3, 0, sizeof(double) * (size_t)(nb * h));
                memset(Y, 0, sizeof(double) * (size_t)(nb * d));
                for (int i = 0; i < d; ++i) {
                    const int64_t off = (e * d + i) * (int64_t)h;
                    for (int64_t b = 0; b < nb; ++b) {
                        axpy(H1 + b * h, X[b * d + i], w1, w_dt, off, h);
                        axpy(H3 + b * h, X[b * d + i], w3, w_dt, off, h);
                    }
                }
                /* H1 now holds x.W1; overwrite H3 by A = silu(H1) * H3 after saving */
                for (int64_t b = 0; b < nb; ++b) {
                    const int64_t r = w->rows[b];
                    for (int j = 0; j < h; ++j) {
                        const double a1 = H1[b * h + j], a3 = H3[b * h + j];
                        if (h1_out) h1_out[r * h + j] = a1;
                        if (h3_out) h3_out[r * h + j] = a3;
                        H3[b * h + j] = silu(a1) * a3;
                        if (act_out) act_out[r * h + j] = H3[b * h + j];
                    }
                }
                for (int j = 0; j < h; ++j) {
                    const int64_t off = (e * h + j) * (int64_t)d;
                    for (int64_t b = 0; b < nb; ++b) axpy(Y + b * d, H3[b * h + j], w2, w_dt, off, d);
                }
                for (int64_t b = 0; b < nb; ++b)
                    memcpy(ye + w->rows[b] * d, Y + b * d, sizeof(double) * (size_t)d);
            }
        }
        free(X); free(H1); free(H3); free(Y);
    }
    free(items);
    free(rowbuf);
    return rc;
}

/*
 * Backward of the SwiGLU experts given dYe [rows, d] (upstream gradient of Ye):
 *   dA = dYe.W2[e]^T, dH1 = dA * H3 * sig(H1) * (1 + H1 * (1 - sig(H1))),
 *   dH3 = dA * silu(H1), dXs = dH1.W1[e]^T + dH3.W3[e]^T,
 *   dW1[e] = sum_rows x^T dH1, dW3[e] = sum_rows x^T dH3, dW2[e] = sum_rows A^T dYe,
 * with H1, H3, A recomputed in double.  Weight gradients are accumulated over
 * the expert's rows in ascending row order; an expert with no rows gets an
 * explicit zero gradient.  dw1/dw3 [E,d,h], dw2 [E,h,d], dxs [rows,d];
 * dh1/dh3/da [rows,h] optional.  Each expert's rows are handled by one thread, so
 * the weight-gradient sums need no reduction across threads.
 */
int orc_ffn_bwd(const void *xs, int xs_dt, const int32_t *row_token, const int32_t *row_expert,
                int64_t rows, int d, int h, int E, const void *w1, const void *w3, const void *w2,
                int w_dt, const void *dye, int dye_dt, double *dxs, double *dh1_out, double *dh3_out,
                double *da_out, double *dw1, double *dw3, double *dw2) {
    if (!xs || !row_expert || !w1 || !w3 || !w2 || !dye || d < 1 || h < 1 || E < 1) return ORC_EINVAL;
    orc_item *items = NULL;
    int64_t *rowbuf = NULL;
    int64_t nitems = build_items(row_expert, rows, E, &items, &rowbuf);
    if (nitems < 0) return nitems == -2 ? ORC_EINVAL : ORC_ENOMEM;
    if (dw1) memset(dw1, 0, sizeof(double) * (size_t)E * d * h);
    if (dw3) memset(dw3, 0, sizeof(double) * (size_t)E * d * h);
    if (dw2) memset(dw2, 0, sizeof(double) * (size_t)E * d * h);
    int rc = ORC_OK;
#pragma omp parallel num_threads(NT)
    {
        double *X = (double *)malloc(sizeof(double) * (size_t)d);
        double *G = (double *)malloc(sizeof(double) * (size_t)d);
        double *H1 = (double *)malloc(sizeof(double) * (size_t)h);
        double *H3 = (double *)malloc(sizeof(double) * (size_t)h);
        double *DA = (double *)malloc(sizeof(double) * (size_t)h);
        double *D1 = (double *)malloc(sizeof(double) * (size_t)h);
        double *D3 = (double *)malloc(sizeof(double) * (size_t)h);
        double *A = (double *)malloc(sizeof(double) * (size_t)h);
        double *DX = (double *)malloc(sizeof(double) * (size_t)d);
        const int ok = (X && G && H1 && H3 && DA && D1 && D3 && A && DX) ? 1 : 0;
        if (!ok) {
#pragma omp atomic write
            rc = ORC_ENOMEM;
        }
        {
            /* one expert per iteration: its weight-gradient sums stay with one thread */
#pragma omp for schedule(dynamic, 1)
            for (int e = 0; e < E; ++e) {
                if (!ok) continue;
                for (int64_t it = 0; it < nitems; ++it) {
                    if (items[it].e != e) continue;
                    for (int64_t b = 0; b < items[it].n; ++b) {
                        const int64_t r = items[it].rows[b];
                        load_row(X, xs, xs_dt, in_row(row_token, r) * d, d);
                        load_row(G, dye, dye_dt, r * d, d);
                        memset(H1, 0, sizeof(double) * (size_t)h);
                        memset(H3, 0, sizeof(double) * (size_t)h);
                        for (int i = 0; i < d; ++i) {
                            axpy(H1, X[i], w1, w_dt, ((int64_t)e * d + i) * h, h);
                            axpy(H3, X[i], w3, w_dt, ((int64_t)e * d + i) * h, h);
                        }
                        for (int j = 0; j < h; ++j) {
                            DA[j] = dot(G, w2, w_dt, ((int64_t)e * h + j) * d, d);
                            const double sg = sigm(H1[j]);
                            A[j] = H1[j] * sg * H3[j];
                            D1[j] = DA[j] * H3[j] * sg * (1.0 + H1[j] * (1.0 - sg));
                            D3[j] = DA[j] * H1[j] * sg;
                        }
                        for (int i = 0; i < d; ++i) {
                            const int64_t off = ((int64_t)e * d + i) * h;
                            DX[i] = dot(D1, w1, w_dt, off, h) + dot(D3, w3, w_dt, off, h);
                        }
                        if (dxs) memcpy(dxs + r * d, DX, sizeof(double) * (size_t)d);
                        if (dh1_out) memcpy(dh1_out + r * h, D1, sizeof(double) * (size_t)h);
                        if (dh3_out) memcpy(dh3_out + r * h, D3, sizeof(double) * (size_t)h);
                        if (da_out) memcpy(da_out + r * h, DA, sizeof(double) * (size_t)h);
                        if (dw1 || dw3)
                            for (int i = 0; i < d; ++i) {
                                double *p1 = dw1 ? dw1 + ((int64_t)e * d + i) * h : NULL;
                                double *p3 = dw3 ? dw3 + ((int64_t)e * d + i) * h : NULL;
                                for (int j = 0; j < h; ++j) {
                                    if (p1) p1[j] += X[i] * D1[j];
                                    if (p3) p3[j] += X[i] * D3[j];
                                }
                            }
                        if (dw2)
                            for (int j = 0; j < h; ++j) {
                                double *p2 = dw2 + ((int64_t)e * h + j) * d;
                                for (int c = 0; c < d; ++c) p2[c] += A[j] * G[c];
                            }
                    }
                }
            }
        }
        free(X); free(G); free(H1); free(H3); free(DA); free(D1); free(D3); free(A); free(DX);
    }
    free(items);
    free(rowbuf);
    return rc;
}

/*
 * The same weight gradients as orc_ffn_bwd, restricted to one expert e and a
 * list of hidden columns: dw1c/dw3c [d, ncols] hold dW1[e][:, cols] and
 * dW3[e][:, cols]; dw2c [ncols, d] holds dW2[e][cols, :].  Each needed H1, H3,
 * dA entry is recomputed from its definition, so a full-size layer can be
 * checked on a few columns.
 */
int orc_ffn_wgrad_cols(const void *xs, int xs_dt, const int32_t *row_token, const int32_t *row_expert,
                       int64_t rows, int d, int h, int E, const void *w1, const void *w3,
                       const void *w2, int w_dt, const void *dye, int dye_dt, int e,
                       const int32_t *cols, int ncols, double *dw1c, double *dw3c, double *dw2c) {
    if (!xs || !row_expert || !w1 || !w3 || !w2 || !dye || !cols || e < 0 || e >= E || ncols < 1)
        return ORC_EINVAL;
    for (int c = 0; c < ncols; ++c) if (cols[c] < 0 || cols[c] >= h) return ORC_EINVAL;
    memset(dw1c, 0, sizeof(double) * (size_t)d * ncols);
    memset(dw3c, 0, sizeof(double) * (size_t)d * ncols);
    memset(dw2c, 0, sizeof(double) * (size_t)d * ncols);
    /* parallel over columns: each column's sums belong to one thread */
    int rc = ORC_OK;
#pragma omp parallel num_threads(NT)
    {
        double *X = (double *)malloc(sizeof(double) * (size_t)d);
        double *G = (double *)malloc(sizeof(double) * (size_t)d);
        const int ok = (X && G) ? 1 : 0;
        if (!ok) {
#pragma omp atomic write
            rc = ORC_ENOMEM;
        }
        {
#pragma omp for schedule(dynamic, 1)
            for (int c = 0; c < ncols; ++c) {
                if (!ok) continue;
                const int j = cols[c];
                for (int64_t r = 0; r < rows; ++r) {
                    if (row_expert[r] != e) continue;
                    load_row(X, xs, xs_dt, in_row(row_token, r) * d, d);
                    load_row(G, dye, dye_dt, r * d, d);
                    double a1 = 0.0, a3 = 0.0;
                    for (int i = 0; i < d; ++i) {
                        a1 += X[i] * ld(w1, w_dt, ((int64_t)e * d + i) * h + j);
                        a3 += X[i] * ld(w3, w_dt, ((int64_t)e * d + i) * h + j);
                    }
                    const double da = dot(G, w2, w_dt, ((int64_t)e * h + j) * d, d);
                    const double sg = sigm(a1);
                    const double g1 = da * a3 * sg * (1.0 + a1 * (1.0 - sg));
                    const double g3 = da * a1 * sg;
                    const double act = a1 * sg * a3;
                    for (int i = 0; i < d; ++i) {
                        dw1c[(int64_t)i * ncols + c] += X[i] * g1;
                        dw3c[(int64_t)i * ncols + c] += X[i] * g3;
                        dw2c[(int64_t)c * d + i] += act * G[i];
                    }
                }
            }
        }
        free(X); free(G);
    }
    return rc;
}

/* --------------------------------------------------------------- combine */

/*
 * Combine by token ownership: y[t] = sum over rows r with row_token[r] == t of
 * row_w[r] * ye[r]  (+ y_add[t] when given).  y [T, d].
 */
int orc_combine(const double *ye, const int32_t *row_token, const double *row_w, int64_t rows,
                int64_t T, int d, const void *y_add, int add_dt, double *y) {
    if (!ye || !row_token || !row_w || !y || d < 1) return ORC_EINVAL;
    for (int64_t i = 0; i < T * d; ++i) y[i] = 0.0;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t t = row_token[r];
        if (t < 0 || t >= T) return ORC_EINVAL;
        for (int c = 0; c < d; ++c) y[t * d + c] += row_w[r] * ye[r * d + c];
    }
    if (y_add)
        for (int64_t i = 0; i < T * d; ++i) y[i] += ld(y_add, add_dt, i);
    return ORC_OK;
}

/*
 * Backward of the combine for fixed weights:
 *   dye[r] = row_w[r] * dy[row_token[r]]         (gradient of the expert output)
 *   dw[r]  = <dy[row_token[r]], ye[r]>           (gradient of the weight)
 */
int orc_combine_bwd(const void *dy, int dy_dt, const double *ye, const int32_t *row_token,
                    const double *row_w, int64_t rows, int64_t T, int d, double *dye, double *dw) {
    if (!dy || !ye || !row_token || !row_w || d < 1) return ORC_EINVAL;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t t = row_token[r];
        if (t < 0 || t >= T) return ORC_EINVAL;
        double s = 0.0;
        for (int c = 0; c < d; ++c) {
            const double g = ld(dy, dy_dt, t * d + c);
            if (dye) dye[r * d + c] = row_w[r] * g;
            s += g * ye[r * d + c];
        }
        if (dw) dw[r] = s;
    }
    return ORC_OK;
}

/*
 * Transpose of the gather: dx[t] = sum over rows r with row_token[r] == t of
 * dxs[r]  (+ dx_add[t] when given).
 */
int orc_scatter_add(const void *dxs, int dxs_dt, const int32_t *row_token, int64_t rows, int64_t T,
                    int d, const void *dx_add, int add_dt, double *dx) {
    if (!dxs || !row_token || !dx || d < 1) return ORC_EINVAL;
    for (int64_t i = 0; i < T * d; ++i) dx[i] = dx_add ? ld(dx_add, add_dt, i) : 0.0;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t t = row_token[r];
        if (t < 0 || t >= T) return ORC_EINVAL;
        for (int c = 0; c < d; ++c) dx[t * d + c] += ld(dxs, dxs_dt, r * d + c);
    }
    return ORC_OK;
}

/* ---------------------------------------------------------- router backward */

/*
 * Backward of the gate through the probabilities (the selection is piecewise
 * constant, so it carries no gradient; the biases get none either):
 *   p = softmax(s[t]),  g[t,e] = dtopk_w[t,j] where e == topk_ids[t,j], else 0,
 *   c_t = sum_j p[t, topk_ids[t,j]] * dtopk_w[t,j],
 *   dz[t,e] = p[t,e] * (g[t,e] - c_t) * inv_tau,
 *   dx[t,i] = sum_e dz[t,e] * Wg[i,e],   dwg[i,e] = sum_t x[t,i] * dz[t,e].
 * scores s [T,E] are the softmax inputs of the forward.  dz, dx, dwg may be NULL.
 */
int orc_route_bwd(const double *scores, const int32_t *topk_ids, const double *dtopk_w,
                  const void *x, int x_dt, const void *wg, int wg_dt, int64_t T, int d, int E, int k,
                  double inv_tau, double *dz_out, double *dx, double *dwg) {
    if (!scores || !topk_ids || !dtopk_w || !x || !wg || d < 1 || E < 1 || k < 1 || k > E)
        return ORC_EINVAL;
    double *dz = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * E);
    if (!dz) return ORC_ENOMEM;
#pragma omp parallel for num_threads(NT) schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double *s = scores + t * E;
        double *z = dz + t * E;
        double mx = s[0];
        for (int e = 1; e < E; ++e) if (s[e] > mx) mx = s[e];
        double den = 0.0;
        for (int e = 0; e < E; ++e) { z[e] = exp(s[e] - mx); den += z[e]; }
        for (int e = 0; e < E; ++e) z[e] /= den;          /* z holds p for now */
        double c = 0.0;
        for (int j = 0; j < k; ++j) c += z[topk_ids[t * k + j]] * dtopk_w[t * k + j];
        double g[1024];
        double *gp = E <= 1024 ? g : (double *)calloc((size_t)E, sizeof(double));
        if (E <= 1024) memset(g, 0, sizeof(double) * (size_t)E);
        for (int j = 0; j < k; ++j) gp[topk_ids[t * k + j]] = dtopk_w[t * k + j];
        for (int e = 0; e < E; ++e) z[e] = z[e] * (gp[e] - c) * inv_tau;
        if (gp != g) free(gp);
        if (dx)
            for (int i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int e = 0; e < E; ++e) acc += z[e] * ld(wg, wg_dt, (int64_t)i * E + e);
                dx[t * d + i] = acc;
            }
    }
    if (dwg) {
        /* blocks of 16 features per thread; each (i, e) sum runs over t ascending */
        const int nblk = (d + 15) / 16;
#pragma omp parallel for num_threads(NT) schedule(dynamic, 1)
        for (int b = 0; b < nblk; ++b) {
            const int i0 = b * 16, i1 = (i0 + 16 < d) ? i0 + 16 : d;
            double xv[16];
            for (int i = i0; i < i1; ++i)
                for (int e = 0; e < E; ++e) dwg[(int64_t)i * E + e] = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                for (int i = i0; i < i1; ++i) xv[i - i0] = ld(x, x_dt, t * d + i);
                const double *z = dz + t * E;
                for (int i = i0; i < i1; ++i) {
                    double *row = dwg + (int64_t)i * E;
                    for (int e = 0; e < E; ++e) row[e] += xv[i - i0] * z[e];
                }
            }
        }
    }
    if (dz_out) memcpy(dz_out, dz, sizeof(double) * (size_t)T * E);
    free(dz);
    return ORC_OK;
}
