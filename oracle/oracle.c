/*
 * oracle.c -- plain, slow, fp64 CPU oracle of the Mixture-of-Experts layer of a
 * prefill step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent reference that the
 * HIP path is checked against.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load it; the library under
 * expert_layer_amd/ never does, and the two share no code, header, table or
 * helper.
 *
 * What is computed, and where the pages say so:
 *  - "ASAP: A DiSaggregated and Asynchronous Inference System for MoE Prefill",
 *    section 3.4.2 (Bubble-Free Kernel Dispatching): the MoE kernel is a grouped
 *    matrix multiplication whose left operand is the hidden states and whose
 *    right operand is the expert weights of the layer.
 *  - same page, Table 1 and Table 2: K experts chosen per token out of E_total,
 *    hidden size H; the dispatch buffers carry expert IDs per token, token
 *    counts per expert, and the per-(token, choice) expert results that are
 *    combined back.
 *  - "Memory-Compute Disaggregation ... AFD Architecture Analysis", section 3
 *    (Data-Flow Closed Loop): the FFN side of an MoE model performs gated
 *    routing plus expert computation and returns the layer output.
 * The pages never write the formulas.  The concrete layer (softmax or sigmoid
 * scoring, group-limited top-k, renormalisation and scaling, SwiGLU experts, a
 * shared expert, fp8 block scales) is the plain textbook definition of the
 * layer that the workload statement names; every reading taken where the
 * pages are silent is listed in the design notes of the repository.
 *
 * Conventions.
 *  - Every operand is widened exactly to double (bf16, fp32 and e4m3 * fp32
 *    scale are all exact in double) and every sum is accumulated in double in
 *    the natural index order.  Parallel loops (OpenMP) only split independent
 *    outputs; no summation is reordered.
 *  - Matrices are [out][in] row-major: w_router [E][H], w_gate/w_up [E][I][H],
 *    w_down [E][H][I].
 *  - dtype codes: 0 = fp32, 1 = bf16 (uint16 bit patterns), 2 = OCP e4m3
 *    (uint8 codes: bias 7, max 448, S.1111.111 is NaN, no infinities).
 *  - Where a floating-point value decides an integer (the top-k choice, an
 *    e4m3 code) the decision is taken on fp32 values, the precision the GPU
 *    kernels use.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_E4M3 2

/* Threads an OpenMP loop of the oracle runs on (for reporting). */
int orc_threads(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------- formats */

/* bf16 is the upper half of an IEEE binary32 word. */
double orc_bf16_to_f64(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit float E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent field 0 is subnormal (m/8 * 2^-6); the all-ones
 * exponent+mantissa pattern is NaN; there are no infinities. */
double orc_e4m3_to_f64(uint8_t c) {
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    double v;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Round a double to the nearest e4m3 value, ties to the code with an even
 * mantissa, saturating to +-448.  Positive codes 0..126 are increasing in
 * value, so a binary search over them finds the two neighbours. */
uint8_t orc_e4m3_rne_sat(double v) {
    int neg = v < 0.0;
    double a = neg ? -v : v;
    uint8_t code;
    if (isnan(v)) return 0x7F;
    if (a >= 448.0) {
        code = 0x7E;
    } else {
        int lo = 0, hi = 126; /* decode(lo) <= a < decode(hi) */
        while (hi - lo > 1) {
            int mid = (lo + hi) / 2;
            if (orc_e4m3_to_f64((uint8_t)mid) <= a) lo = mid;
            else hi = mid;
        }
        double dl = a - orc_e4m3_to_f64((uint8_t)lo);
        double dh = orc_e4m3_to_f64((uint8_t)hi) - a;
        if (dl < dh) code = (uint8_t)lo;
        else if (dh < dl) code = (uint8_t)hi;
        else code = (uint8_t)((lo & 1) == 0 ? lo : hi);
    }
    if (neg && code != 0) code |= 0x80;
    return code;
}

/* Round a double to bf16, nearest-even.  The value is first rounded to fp32
 * (nearest-even, the C default), then fp32 to bf16: the rounding decision is
 * taken on the fp32 value, the precision in which the kernels hold it. */
uint16_t orc_bf16_rne(double v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static double ld(int dtype, const void *p, size_t i) {
    switch (dtype) {
    case ORC_F32: return (double)((const float *)p)[i];
    case ORC_BF16: return orc_bf16_to_f64(((const uint16_t *)p)[i]);
    default: return orc_e4m3_to_f64(((const uint8_t *)p)[i]);
    }
}

/* ------------------------------------------------------ router (logits) */

/* logits[t][e] = fp32( sum_h x[t][h] * w_router[e][h] ), summed in double. */
void orc_router_logits(int64_t T, int64_t H, int64_t E, int x_dtype, const void *x,
                       int w_dtype, const void *w_router, float *logits) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int64_t h = 0; h < H; ++h)
                acc += ld(x_dtype, x, (size_t)(t * H + h)) *
                       ld(w_dtype, w_router, (size_t)(e * H + h));
            logits[t * E + e] = (float)acc;
        }
    }
}

/* ------------------------------------------------------ gating (top-k) */

#define ORC_SOFTMAX 0
#define ORC_SIGMOID 1
#define ORC_GROUP_TOP2_SUM 0
#define ORC_GROUP_MAX 1

/* Per-token scoring, group limit, top-k and weights.
 *
 *  softmax router: z_e = fp32(l_e + b_e) (the bias is a logit bias),
 *                  p = softmax(z); raw score r_e = p_e; selection key c_e = z_e,
 *                  which orders the experts exactly as p does (exp is strictly
 *                  increasing) and is the same fp32 number on every side that
 *                  starts from the same logits.
 *  sigmoid router: s_e = 1 / (1 + exp(-l_e)); raw score r_e = s_e,
 *                  selection key c_e = s_e + b_e (the bias steers selection
 *                  only).
 *  keys are rounded to fp32 before any comparison.
 *  group limit (n_groups > 1): group g holds experts [g*E/G, (g+1)*E/G); its
 *                  score is the sum of its two largest keys (TOP2_SUM, summed
 *                  as an fp32 addition) or its largest key (MAX); the
 *                  topk_groups best groups are kept, ties to the lower group
 *                  index; the experts of the other groups cannot be chosen.
 *  top-k:          the k allowed experts with the largest keys, ordered by
 *                  key descending, ties to the lower expert index.
 *  weights:        w_j = r_{e_j} / sum_j' r_{e_j'} if renormalize, else r_{e_j};
 *                  then w_j *= routed_scale.
 * Returns 0, or -1 on an argument error. */
int orc_route_select(int64_t T, int E, int k, int score_fn, int n_groups, int topk_groups,
                     int group_score, int renormalize, double routed_scale,
                     const float *logits, const float *bias, int32_t *topk_ids,
                     float *topk_w) {
    if (E <= 0 || k <= 0 || k > E || n_groups <= 0 || E % n_groups != 0 ||
        topk_groups <= 0 || topk_groups > n_groups ||
        (int64_t)k > (int64_t)topk_groups * (E / n_groups))
        return -1;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t t = 0; t < T; ++t) {
        double *raw = (double *)malloc(sizeof(double) * (size_t)E);
        float *key = (float *)malloc(sizeof(float) * (size_t)E);
        char *allowed = (char *)malloc((size_t)E);
        char *taken = (char *)malloc((size_t)E);
        float *gscore = (float *)malloc(sizeof(float) * (size_t)n_groups);
        char *gkept = (char *)malloc((size_t)n_groups);
        if (!raw || !key || !allowed || !taken || !gscore || !gkept) {
            bad = 1;
        } else {
            const float *l = logits + t * E;
            if (score_fn == ORC_SOFTMAX) {
                double zmax = -INFINITY;
                for (int e = 0; e < E; ++e) {
                    double z = (double)(float)((double)l[e] + (bias ? (double)bias[e] : 0.0));
                    if (z > zmax) zmax = z;
                }
                double sum = 0.0;
                for (int e = 0; e < E; ++e) {
                    double z = (double)(float)((double)l[e] + (bias ? (double)bias[e] : 0.0));
                    raw[e] = exp(z - zmax);
                    sum += raw[e];
                }
                for (int e = 0; e < E; ++e) {
                    raw[e] /= sum;
                    key[e] = (float)((double)l[e] + (bias ? (double)bias[e] : 0.0));
                }
            } else {
                for (int e = 0; e < E; ++e) {
                    raw[e] = 1.0 / (1.0 + exp(-(double)l[e]));
                    key[e] = (float)(raw[e] + (bias ? (double)bias[e] : 0.0));
                }
            }
            /* group limit */
            int gs = E / n_groups;
            for (int g = 0; g < n_groups; ++g) {
                float best = -INFINITY, second = -INFINITY;
                for (int e = g * gs; e < (g + 1) * gs; ++e) {
                    if (key[e] > best) {
                        second = best;
                        best = key[e];
                    } else if (key[e] > second) {
                        second = key[e];
                    }
                }
                if (group_score == ORC_GROUP_MAX || gs == 1)
                    gscore[g] = best;
                else
                    gscore[g] = (float)((double)best + (double)second);
                gkept[g] = 0;
            }
            for (int r = 0; r < topk_groups; ++r) {
                int bg = -1;
                for (int g = 0; g < n_groups; ++g)
                    if (!gkept[g] && (bg < 0 || gscore[g] > gscore[bg])) bg = g;
                gkept[bg] = 1;
            }
            for (int e = 0; e < E; ++e) {
                allowed[e] = gkept[e / gs];
                taken[e] = 0;
            }
            /* top-k: repeatedly take the largest remaining key, lower index on ties */
            double rsum = 0.0;
            for (int j = 0; j < k; ++j) {
                int be = -1;
                for (int e = 0; e < E; ++e)
                    if (allowed[e] && !taken[e] && (be < 0 || key[e] > key[be])) be = e;
                taken[be] = 1;
                topk_ids[t * k + j] = be;
                rsum += raw[be];
            }
            for (int j = 0; j < k; ++j) {
                double r = raw[topk_ids[t * k + j]];
                double w = renormalize ? r / rsum : r;
                topk_w[t * k + j] = (float)(w * routed_scale);
            }
        }
        free(raw);
        free(key);
        free(allowed);
        free(taken);
        free(gscore);
        free(gkept);
    }
    return bad ? -1 : 0;
}

/* Per-token decision margins, for the input generator's acceptance test:
 * margin[t] = min( key_(k) - key_(k+1) among allowed experts,
 *                  gscore_(topk_groups) - gscore_(topk_groups+1) ),
 * computed in double from the same definitions as orc_route_select (no fp32
 * rounding), +inf where a gap does not exist. */
int orc_route_margin(int64_t T, int E, int k, int score_fn, int n_groups, int topk_groups,
                     int group_score, const float *logits, const float *bias, double *margin) {
    if (E <= 0 || k <= 0 || k > E || n_groups <= 0 || E % n_groups != 0 ||
        topk_groups <= 0 || topk_groups > n_groups)
        return -1;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t t = 0; t < T; ++t) {
        double *key = (double *)malloc(sizeof(double) * (size_t)E);
        double *gscore = (double *)malloc(sizeof(double) * (size_t)n_groups);
        char *used = (char *)malloc((size_t)(E > n_groups ? E : n_groups));
        if (!key || !gscore || !used) {
            bad = 1;
        } else {
            const float *l = logits + t * E;
            if (score_fn == ORC_SOFTMAX) {
                for (int e = 0; e < E; ++e) key[e] = (double)l[e] + (bias ? (double)bias[e] : 0.0);
            } else {
                for (int e = 0; e < E; ++e)
                    key[e] = 1.0 / (1.0 + exp(-(double)l[e])) + (bias ? (double)bias[e] : 0.0);
            }
            int gs = E / n_groups;
            double m = INFINITY;
            for (int g = 0; g < n_groups; ++g) {
                double best = -INFINITY, second = -INFINITY;
                for (int e = g * gs; e < (g + 1) * gs; ++e) {
                    if (key[e] > best) {
                        second = best;
                        best = key[e];
                    } else if (key[e] > second) {
                        second = key[e];
                    }
                }
                gscore[g] = (group_score == ORC_GROUP_MAX || gs == 1) ? best : best + second;
            }
            /* sorted group scores: gap between the topk_groups-th and the next */
            memset(used, 0, (size_t)n_groups);
            double prev = 0.0;
            for (int r = 0; r < n_groups && r <= topk_groups; ++r) {
                int bg = -1;
                for (int g = 0; g < n_groups; ++g)
                    if (!used[g] && (bg < 0 || gscore[g] > gscore[bg])) bg = g;
                used[bg] = 1;
                if (r == topk_groups) {
                    double gap = prev - gscore[bg];
                    if (gap < m) m = gap;
                } else {
                    prev = gscore[bg];
                }
            }
            /* experts of kept groups: used[g] marks exactly the topk_groups best */
            char *kept = (char *)malloc((size_t)n_groups);
            if (!kept) {
                bad = 1;
            } else {
                memset(kept, 0, (size_t)n_groups);
                memset(used, 0, (size_t)n_groups);
                for (int r = 0; r < topk_groups; ++r) {
                    int bg = -1;
                    for (int g = 0; g < n_groups; ++g)
                        if (!used[g] && (bg < 0 || gscore[g] > gscore[bg])) bg = g;
                    used[bg] = 1;
                    kept[bg] = 1;
                }
                char *taken = (char *)calloc((size_t)E, 1);
                if (!taken) {
                    bad = 1;
                } else {
                    double kth = 0.0;
                    for (int j = 0; j <= k; ++j) {
                        int be = -1;
                        for (int e = 0; e < E; ++e)
                            if (kept[e / gs] && !taken[e] && (be < 0 || key[e] > key[be])) be = e;
                        if (be < 0) break;
                        taken[be] = 1;
                        if (j == k) {
                            double gap = kth - key[be];
                            if (gap < m) m = gap;
                        } else {
                            kth = key[be];
                        }
                    }
                    free(taken);
                }
                free(kept);
            }
            margin[t] = m;
        }
        free(key);
        free(gscore);
        free(used);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------- dispatch */

/* Counting sort of the (token, choice) pairs by expert.
 *   counts[e]          = #{(t, j) : ids[t][j] == e}
 *   offsets[e]         = sum_{e' < e} counts[e']                  (E + 1 entries)
 *   padded_offsets[e]  = sum_{e' < e} ceil(counts[e'] / m_tile) * m_tile
 *   inside expert e the rows are in ascending token order (a token picks an
 *   expert at most once):  row(t, j) = padded_offsets[e] + #{t' < t : e in ids[t']}
 *   row_src[row]       = t * k + j, and -1 for padding rows (rows_cap entries;
 *                        entries past padded_offsets[E] are set to -1 too)
 *   tok_row[t * k + j] = row(t, j).
 * Returns 0, or -1 if an id is out of range or rows_cap is too small. */
int orc_dispatch(int64_t T, int k, int E, int m_tile, const int32_t *ids, int64_t rows_cap,
                 int32_t *counts, int32_t *offsets, int32_t *padded_offsets,
                 int32_t *row_src, int32_t *tok_row) {
    if (m_tile <= 0) return -1;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t i = 0; i < T * k; ++i) {
        if (ids[i] < 0 || ids[i] >= E) return -1;
        counts[ids[i]] += 1;
    }
    offsets[0] = 0;
    padded_offsets[0] = 0;
    for (int e = 0; e < E; ++e) {
        offsets[e + 1] = offsets[e] + counts[e];
        padded_offsets[e + 1] =
            padded_offsets[e] + ((counts[e] + m_tile - 1) / m_tile) * m_tile;
    }
    if ((int64_t)padded_offsets[E] > rows_cap) return -1;
    for (int64_t r = 0; r < rows_cap; ++r) row_src[r] = -1;
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!cursor) return -1;
    for (int e = 0; e < E; ++e) cursor[e] = padded_offsets[e];
    for (int64_t t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int e = ids[t * k + j];
            int32_t row = cursor[e]++;
            row_src[row] = (int32_t)(t * k + j);
            tok_row[t * k + j] = row;
        }
    }
    free(cursor);
    return 0;
}

/* ----------------------------------------------------------- expert FFN */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One SwiGLU expert applied to n rows:
 *   g_i = sum_h x[r][h] * w_gate[i][h],   u_i = sum_h x[r][h] * w_up[i][h]
 *   a_i = silu(g_i) * u_i,                silu(z) = z / (1 + e^-z)
 *   y[r][h] = sum_i a_i * w_down[h][i]
 * h_bf16 = 1 stores the intermediate activation a in bf16 (nearest-even, the
 * decision taken on its fp32 value) before the down projection: in a layer
 * whose activations are bf16, a is one of them.  h_bf16 = 0 keeps a exact,
 * which is the definition for fp32 layers and the reference for measuring
 * what the bf16 storage itself costs. */
void orc_expert_ffn(int64_t n, int64_t H, int64_t I, int x_dtype, const void *x_rows,
                    int w_dtype, const void *w_gate, const void *w_up, const void *w_down,
                    int h_bf16, double *y) {
    /* The loops run over the outputs (a weight row at a time, widened once and
     * applied to every row); each sum still runs over its index in order. */
    double *X = (double *)malloc(sizeof(double) * (size_t)(n * H + 1));
    double *A = (double *)malloc(sizeof(double) * (size_t)(n * I + 1));
    if (X && A) {
        for (int64_t e = 0; e < n * H; ++e) X[e] = ld(x_dtype, x_rows, (size_t)e);
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t i = 0; i < I; ++i) {
            double *wg = (double *)malloc(sizeof(double) * (size_t)H);
            double *wu = (double *)malloc(sizeof(double) * (size_t)H);
            if (wg && wu) {
                for (int64_t h = 0; h < H; ++h) {
                    wg[h] = ld(w_dtype, w_gate, (size_t)(i * H + h));
                    wu[h] = ld(w_dtype, w_up, (size_t)(i * H + h));
                }
                for (int64_t r = 0; r < n; ++r) {
                    const double *xr = X + r * H;
                    double g = 0.0, u = 0.0;
                    for (int64_t h = 0; h < H; ++h) {
                        g += xr[h] * wg[h];
                        u += xr[h] * wu[h];
                    }
                    double a = silu(g) * u;
                    if (h_bf16) a = orc_bf16_to_f64(orc_bf16_rne(a));
                    A[r * I + i] = a;
                }
            }
            free(wg);
            free(wu);
        }
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t h = 0; h < H; ++h) {
            double *wd = (double *)malloc(sizeof(double) * (size_t)I);
            if (wd) {
                for (int64_t i = 0; i < I; ++i) wd[i] = ld(w_dtype, w_down, (size_t)(h * I + i));
                for (int64_t r = 0; r < n; ++r) {
                    const double *a = A + r * I;
                    double acc = 0.0;
                    for (int64_t i = 0; i < I; ++i) acc += a[i] * wd[i];
                    y[r * H + h] = acc;
                }
            }
            free(wd);
        }
    }
    free(X);
    free(A);
}

/* The requantisation of the fp8 intermediate, one row a [I] at a time (see
 * orc_expert_ffn_fp8): per 128-column block, s = fp32(max |fp32(a_i)|) / 448
 * (1 for a zero block), a_i <- e4m3(e4m3_rne_sat(fp32(fp32(a_i) / s))) * s. */
static void requant_row_e4m3(int64_t I, double *a) {
    for (int64_t b = 0; b < I / 128; ++b) {
        float amax = 0.0f;
        for (int64_t i = b * 128; i < (b + 1) * 128; ++i) {
            float v = fabsf((float)a[i]);
            if (v > amax) amax = v;
        }
        float s = amax > 0.0f ? amax / 448.0f : 1.0f;
        for (int64_t i = b * 128; i < (b + 1) * 128; ++i) {
            float q = (float)a[i] / s;
            a[i] = orc_e4m3_to_f64(orc_e4m3_rne_sat((double)q)) * (double)s;
        }
    }
}

/* One SwiGLU expert on fp8 operands with block scales.
 *   x[r][h]      = e4m3(xq[r][h]) * xs[r][h / 128]          (1 x 128 per-row scales)
 *   W[o][c]      = e4m3(wq[o][c]) * ws[o / 128][c / 128]    (128 x 128 block scales)
 *   g, u, a as in orc_expert_ffn, in double.
 * The intermediate a is carried to the down projection as fp8 with one scale
 * per row and 128-column block (this step is part of the definition of the
 * fp8 layer):
 *   a32_i   = fp32(a_i)
 *   amax    = max_i |a32_i| over the block
 *   s       = amax / 448 as an fp32 division  (s = 1 when amax == 0)
 *   q_i     = e4m3_rne_sat( fp32(a32_i / s) )               (fp32 division)
 *   a'_i    = e4m3(q_i) * s
 *   y[r][h] = sum_i a'_i * Wd[h][i].
 * a_out (NULL allowed) receives a [n][I] before the requantisation. */
void orc_expert_ffn_fp8(int64_t n, int64_t H, int64_t I, const uint8_t *xq, const float *xs,
                        const uint8_t *wg, const float *sg, const uint8_t *wu, const float *su,
                        const uint8_t *wd, const float *sd, double *y, double *a_out) {
    int64_t HB = H / 128, IB = I / 128;
    /* loops over the outputs, as in orc_expert_ffn; each sum in index order */
    double *X = (double *)malloc(sizeof(double) * (size_t)(n * H + 1));
    double *A = (double *)malloc(sizeof(double) * (size_t)(n * I + 1));
    if (X && A) {
        for (int64_t r = 0; r < n; ++r)
            for (int64_t h = 0; h < H; ++h)
                X[r * H + h] = orc_e4m3_to_f64(xq[r * H + h]) * (double)xs[r * HB + h / 128];
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t i = 0; i < I; ++i) {
            double *wgr = (double *)malloc(sizeof(double) * (size_t)H);
            double *wur = (double *)malloc(sizeof(double) * (size_t)H);
            if (wgr && wur) {
                for (int64_t h = 0; h < H; ++h) {
                    wgr[h] = orc_e4m3_to_f64(wg[i * H + h]) * (double)sg[(i / 128) * HB + h / 128];
                    wur[h] = orc_e4m3_to_f64(wu[i * H + h]) * (double)su[(i / 128) * HB + h / 128];
                }
                for (int64_t r = 0; r < n; ++r) {
                    const double *xr = X + r * H;
                    double g = 0.0, u = 0.0;
                    for (int64_t h = 0; h < H; ++h) {
                        g += xr[h] * wgr[h];
                        u += xr[h] * wur[h];
                    }
                    A[r * I + i] = silu(g) * u;
                }
            }
            free(wgr);
            free(wur);
        }
        if (a_out) memcpy(a_out, A, sizeof(double) * (size_t)(n * I));
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < n; ++r) requant_row_e4m3(I, A + r * I);
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t h = 0; h < H; ++h) {
            double *wdr = (double *)malloc(sizeof(double) * (size_t)I);
            double *sdr = (double *)malloc(sizeof(double) * (size_t)I);
            if (wdr && sdr) {
                for (int64_t i = 0; i < I; ++i) {
                    wdr[i] = orc_e4m3_to_f64(wd[h * I + i]);
                    sdr[i] = (double)sd[(h / 128) * IB + i / 128];
                }
                for (int64_t r = 0; r < n; ++r) {
                    const double *a = A + r * I;
                    double acc = 0.0;
                    for (int64_t i = 0; i < I; ++i) acc += a[i] * wdr[i] * sdr[i];
                    y[r * H + h] = acc;
                }
            }
            free(wdr);
            free(sdr);
        }
    }
    free(X);
    free(A);
}

/* ------------------------------------------------------- MXFP4 weights
 * The low-precision expert weights of the DWDP page (appendix A4: the MoE
 * weights of its DeepSeek-R1 checkpoint are 4-bit floats with block scales)
 * in the OCP Microscaling (MX) v1.0 form that gfx950's scaled MFMA reads:
 * FP4 E2M1 elements, one E8M0 scale per 32 consecutive elements of a row.
 *   E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0;
 *         exponent 0: (-1)^s * m / 2;  else (-1)^s * 2^(e - 1) * (1 + m / 2).
 *   E8M0: 2^(code - 127); code 255 is NaN.
 * A matrix [rows][K] is stored as packed codes [rows][K / 2] (element k in
 * byte k / 2, the low nibble for even k) and scales [rows][K / 32]. */
double orc_e2m1_to_f64(uint8_t c) {
    double sign = (c & 0x8) ? -1.0 : 1.0;
    int e = (c >> 1) & 0x3, m = c & 0x1;
    if (e == 0) return sign * 0.5 * (double)m;
    return sign * ldexp(1.0 + 0.5 * (double)m, e - 1);
}

double orc_e8m0_to_f64(uint8_t c) { return c == 255 ? NAN : ldexp(1.0, (int)c - 127); }

/* Dequantised MXFP4 matrix: out[r][k] = e2m1(code of (r, k)) * e8m0(scale[r][k / 32]). */
void orc_mxfp4_dequant(int64_t rows, int64_t K, const uint8_t *codes, const uint8_t *scales, double *out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t b = codes[r * (K / 2) + k / 2];
            uint8_t c = (k & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 0xF);
            out[r * K + k] = orc_e2m1_to_f64(c) * orc_e8m0_to_f64(scales[r * (K / 32) + k / 32]);
        }
}

/* One SwiGLU expert on e4m3 rows (1 x 128 fp32 scales, as orc_expert_ffn_fp8)
 * with MXFP4 weights: the same steps as orc_expert_ffn_fp8 -- fp64 sums, the
 * intermediate requantised per row and 128 columns to e4m3 -- with each weight
 * the dequantised MXFP4 value above.  Gate/up [I][H], down [H][I]. */
void orc_expert_ffn_mxfp4(int64_t n, int64_t H, int64_t I, const uint8_t *xq, const float *xs,
                          const uint8_t *wg, const uint8_t *sg, const uint8_t *wu, const uint8_t *su,
                          const uint8_t *wd, const uint8_t *sd, double *y, double *a_out) {
    int64_t HB = H / 128;
    double *Wg = (double *)malloc(sizeof(double) * (size_t)(I * H));
    double *Wu = (double *)malloc(sizeof(double) * (size_t)(I * H));
    double *Wd = (double *)malloc(sizeof(double) * (size_t)(H * I));
    double *X = (double *)malloc(sizeof(double) * (size_t)(n * H + 1));
    double *A = (double *)malloc(sizeof(double) * (size_t)(n * I + 1));
    if (Wg && Wu && Wd && X && A) {
        orc_mxfp4_dequant(I, H, wg, sg, Wg);
        orc_mxfp4_dequant(I, H, wu, su, Wu);
        orc_mxfp4_dequant(H, I, wd, sd, Wd);
        for (int64_t r = 0; r < n; ++r)
            for (int64_t h = 0; h < H; ++h)
                X[r * H + h] = orc_e4m3_to_f64(xq[r * H + h]) * (double)xs[r * HB + h / 128];
        /* loops over the outputs, as in orc_expert_ffn; each sum in index order */
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t i = 0; i < I; ++i)
            for (int64_t r = 0; r < n; ++r) {
                const double *xr = X + r * H;
                double g = 0.0, u = 0.0;
                for (int64_t h = 0; h < H; ++h) {
                    g += xr[h] * Wg[i * H + h];
                    u += xr[h] * Wu[i * H + h];
                }
                A[r * I + i] = silu(g) * u;
            }
        if (a_out) memcpy(a_out, A, sizeof(double) * (size_t)(n * I));
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < n; ++r) requant_row_e4m3(I, A + r * I);
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t r = 0; r < n; ++r) {
                const double *a = A + r * I;
                double acc = 0.0;
                for (int64_t i = 0; i < I; ++i) acc += a[i] * Wd[h * I + i];
                y[r * H + h] = acc;
            }
    }
    free(Wg);
    free(Wu);
    free(Wd);
    free(X);
    free(A);
}

/* Rounds n doubles to bf16 (orc_bf16_rne) and widens them back: the stored
 * value of an activation a bf16 layer keeps in bf16. */
void orc_bf16_round_array(int64_t n, const double *in, double *out) {
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n; ++e) out[e] = orc_bf16_to_f64(orc_bf16_rne(in[e]));
}

/* -------------------------------------------------------------- combine */

/* out[t][h] = sum_{j < k} w[t][j] * y_rows[tok_row[t][j]][h]  (+ y_shared[t][h]) */
void orc_combine(int64_t T, int k, int64_t H, const double *y_rows, const int32_t *tok_row,
                 const float *topk_w, const double *y_shared, double *out) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                int64_t row = tok_row[t * k + j];
                acc += (double)topk_w[t * k + j] * y_rows[row * H + h];
            }
            if (y_shared) acc += y_shared[t * H + h];
            out[t * H + h] = acc;
        }
    }
}

/* ---------------------------------------------------------------- layer */

/* The whole layer on host buffers: logits -> gating -> dispatch -> experts ->
 * combine (+ shared expert).  Expert weights are [E][I][H] / [E][H][I] in
 * w_dtype; x and w_router in x_dtype.  Writes out [T][H] (double) and,
 * when non-NULL, logits [T][E], topk_ids [T][k] and topk_w [T][k].
 * Returns 0, or -1 on an argument or allocation error. */
int orc_layer(int64_t T, int64_t H, int E, int k, int64_t I, int score_fn, int n_groups,
              int topk_groups, int group_score, int renormalize, double routed_scale,
              int x_dtype, const void *x, const void *w_router, const float *bias,
              int w_dtype, const void *w_gate, const void *w_up, const void *w_down,
              int64_t I_shared, const void *sh_gate, const void *sh_up, const void *sh_down,
              int h_bf16, double *out, float *logits_out, int32_t *ids_out, float *w_out) {
    int rc = -1;
    size_t xs = x_dtype == ORC_F32 ? 4 : (x_dtype == ORC_BF16 ? 2 : 1);
    size_t ws = w_dtype == ORC_F32 ? 4 : (w_dtype == ORC_BF16 ? 2 : 1);
    float *logits = (float *)malloc(sizeof(float) * (size_t)(T * E + 1));
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T * k + 1));
    float *w = (float *)malloc(sizeof(float) * (size_t)(T * k + 1));
    int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int32_t *offs = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *poffs = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *row_src = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T * k + 1));
    int32_t *tok_row = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T * k + 1));
    double *y_rows = (double *)malloc(sizeof(double) * (size_t)(T * k * H + 1));
    double *y_sh = NULL;
    unsigned char *x_rows = (unsigned char *)malloc(xs * (size_t)(T * k * H + 1));
    if (!logits || !ids || !w || !counts || !offs || !poffs || !row_src || !tok_row ||
        !y_rows || !x_rows)
        goto done;
    orc_router_logits(T, H, E, x_dtype, x, x_dtype, w_router, logits);
    if (orc_route_select(T, E, k, score_fn, n_groups, topk_groups, group_score, renormalize,
                         routed_scale, logits, bias, ids, w) != 0)
        goto done;
    if (orc_dispatch(T, k, E, 1, ids, T * k, counts, offs, poffs, row_src, tok_row) != 0)
        goto done;
    /* expert e processes its rows [offs[e], offs[e+1]), gathered in order */
    for (int e = 0; e < E; ++e) {
        const unsigned char *wg = (const unsigned char *)w_gate + ws * (size_t)e * (size_t)(I * H);
        const unsigned char *wu = (const unsigned char *)w_up + ws * (size_t)e * (size_t)(I * H);
        const unsigned char *wd = (const unsigned char *)w_down + ws * (size_t)e * (size_t)(H * I);
        int64_t n = offs[e + 1] - offs[e];
        for (int64_t r = 0; r < n; ++r) {
            int64_t t = row_src[offs[e] + r] / k;
            memcpy(x_rows + xs * (size_t)(r * H), (const unsigned char *)x + xs * (size_t)(t * H),
                   xs * (size_t)H);
        }
        if (n > 0)
            orc_expert_ffn(n, H, I, x_dtype, x_rows, w_dtype, wg, wu, wd, h_bf16,
                           y_rows + (size_t)offs[e] * (size_t)H);
    }
    if (sh_gate) {
        y_sh = (double *)malloc(sizeof(double) * (size_t)(T * H + 1));
        if (!y_sh) goto done;
        orc_expert_ffn(T, H, I_shared, x_dtype, x, w_dtype, sh_gate, sh_up, sh_down, h_bf16,
                       y_sh);
    }
    orc_combine(T, k, H, y_rows, tok_row, w, y_sh, out);
    if (logits_out) memcpy(logits_out, logits, sizeof(float) * (size_t)(T * E));
    if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)(T * k));
    if (w_out) memcpy(w_out, w, sizeof(float) * (size_t)(T * k));
    rc = 0;
done:
    free(logits);
    free(ids);
    free(w);
    free(counts);
    free(offs);
    free(poffs);
    free(row_src);
    free(tok_row);
    free(y_rows);
    free(y_sh);
    free(x_rows);
    return rc;
}
