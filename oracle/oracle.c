/*
 * oracle.c -- plain CPU oracle of the Kimi-K2-style MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): loaded by the tests, the smoke
 * check and the CPU-baseline leg of the benchmark, never by the product.
 *
 * Double precision, plain loops, one token at a time.  Tokens are
 * independent (the MoEGate excerpt flattens [B, T, d] to rows), so the only
 * parallelism is an OpenMP loop over tokens; the arithmetic of each token
 * is the same whatever the thread count.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* Exact upcast of one stored element to double: fp32 directly, bf16 by
 * placing its 16 bits in the top half of an fp32 word. */
static double elem(const void *p, int32_t dtype, size_t i)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)p)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double sigmoid(double a) { return 1.0 / (1.0 + exp(-a)); }

/* OCP FP8 E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
 * 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities. */
static double fp8_e4m3(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7)
        return NAN;
    double v = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* E8M0 block scale: 2^(s - 127) (255 is NaN). */
static double e8m0(uint8_t s) { return s == 255 ? NAN : ldexp(1.0, (int)s - 127); }

/* Element (r, c) of a block-scaled FP8 matrix with `cols` columns. */
static double fp8_elem(const uint8_t *W, const uint8_t *S, int32_t cols,
                       int32_t r, int32_t c)
{
    return fp8_e4m3(W[(size_t)r * cols + c]) *
           e8m0(S[(size_t)(r / 128) * (cols / 128) + c / 128]);
}

/* A routed expert with block-scaled FP8 weights: the same SwiGLU as
 * swiglu() on the dequantised values. */
static void swiglu_fp8(int32_t din, int32_t F, const double *vin,
                       const uint8_t *Wg, const uint8_t *Sg, const uint8_t *Wu,
                       const uint8_t *Su, const uint8_t *Wd, const uint8_t *Sd,
                       double *h, double *y)
{
    for (int32_t f = 0; f < F; ++f) {
        double g = 0.0, u = 0.0;
        for (int32_t j = 0; j < din; ++j) {
            g += fp8_elem(Wg, Sg, din, f, j) * vin[j];
            u += fp8_elem(Wu, Su, din, f, j) * vin[j];
        }
        h[f] = g * sigmoid(g) * u;
    }
    for (int32_t o = 0; o < din; ++o) {
        double acc = 0.0;
        for (int32_t f = 0; f < F; ++f)
            acc += fp8_elem(Wd, Sd, F, o, f) * h[f];
        y[o] = acc;
    }
}

/* One token of the router [P3 four steps and MoEGate forward].
 * s_out (length E) receives sigmoid(z); sel (length K) the selected set in
 * ascending expert id; w (length K) the renormalised, scaled weights. */
static void route_one(int32_t d, int32_t E, int32_t K, int32_t x_dtype,
                      const void *x, size_t xrow, const float *W_r,
                      const float *b, float scale, double *s, double *v,
                      char *chosen, int32_t *sel, double *w, double *gap)
{
    /* step 1: z_e = sum_j x_j W_r[e, j]; step 2: s_e = sigmoid(z_e) */
    for (int32_t e = 0; e < E; ++e) {
        double z = 0.0;
        for (int32_t j = 0; j < d; ++j)
            z += elem(x, x_dtype, xrow + (size_t)j) * (double)W_r[(size_t)e * d + j];
        s[e] = sigmoid(z);
        /* step 3 uses the biased score; the bias only chooses */
        v[e] = s[e] + (double)b[e];
        chosen[e] = 0;
    }
    /* top-K of v: K rounds of "largest unchosen v"; scanning e upward with a
     * strict comparison sends ties to the lower expert index. */
    for (int32_t k = 0; k < K; ++k) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e)
            if (!chosen[e] && (best < 0 || v[e] > v[best]))
                best = e;
        chosen[best] = 1;
        sel[k] = best;
    }
    if (gap) {
        /* the last chosen is the K-th largest; compare with the best left */
        double vk = v[sel[K - 1]];
        double next = -INFINITY;
        for (int32_t e = 0; e < E; ++e)
            if (!chosen[e] && v[e] > next)
                next = v[e];
        *gap = (K == E) ? INFINITY : vk - next;
    }
    /* slots in ascending expert id (insertion sort of K values) */
    for (int32_t i = 1; i < K; ++i) {
        int32_t key = sel[i], j = i - 1;
        while (j >= 0 && sel[j] > key) {
            sel[j + 1] = sel[j];
            --j;
        }
        sel[j + 1] = key;
    }
    /* step 4: gather the UNBIASED scores, divide by their sum + 1e-20, then
     * multiply by the routed scaling factor */
    double den = 0.0;
    for (int32_t k = 0; k < K; ++k)
        den += s[sel[k]];
    den += 1e-20;
    for (int32_t k = 0; k < K; ++k)
        w[k] = (s[sel[k]] / den) * (double)scale;
}

int oracle_router(int32_t T, int32_t d, int32_t E, int32_t K, int32_t x_dtype,
                  const void *x, const float *W_r, const float *b, float scale,
                  int32_t *topk_idx, double *topk_w, double *gap,
                  double *scores, int32_t nthreads)
{
    if (T < 0 || d <= 0 || E <= 0 || K < 1 || K > E)
        return ORACLE_ERR_SHAPE;
    if (x_dtype != ORACLE_F32 && x_dtype != ORACLE_BF16)
        return ORACLE_ERR_SHAPE;
    if (T > 0 && (!x || !W_r || !b || !topk_idx || !topk_w))
        return ORACLE_ERR_NULL;
    int nt = nthreads > 0 ? nthreads : 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int32_t t = 0; t < T; ++t) {
        double *s = (double *)malloc(sizeof(double) * (size_t)E);
        double *v = (double *)malloc(sizeof(double) * (size_t)E);
        char *chosen = (char *)malloc((size_t)E);
        double g = 0.0;
        route_one(d, E, K, x_dtype, x, (size_t)t * d, W_r, b, scale, s, v,
                  chosen, topk_idx + (size_t)t * K, topk_w + (size_t)t * K,
                  &g);
        if (gap)
            gap[t] = g;
        if (scores)
            memcpy(scores + (size_t)t * E, s, sizeof(double) * (size_t)E);
        free(s);
        free(v);
        free(chosen);
    }
    return ORACLE_OK;
}

/* One token of the group-limited router [P3 MoEGate forward, the noaux_tc
 * branch; P3 "one group here" for K2].  Same steps 1, 2 and 4 as
 * route_one; step 3 becomes:
 *   - the E experts form n_group contiguous groups of E / n_group;
 *   - a group's score is the sum of its two largest biased scores v;
 *   - the topk_group groups of largest score are kept (ties toward the
 *     lower group index: the excerpt's unsorted topk leaves them open);
 *   - every expert outside the kept groups takes the value 0.0 (the
 *     excerpt's masked_fill(..., 0.0), not minus infinity), the others keep v;
 *   - the K experts of largest such value are selected (ties toward the
 *     lower expert index).
 * gap: v'_(K) - v'_(K+1) of the masked values; group_gap: the kept groups'
 * smallest score minus the largest dropped one (+inf when all are kept). */
static void route_one_grouped(int32_t d, int32_t E, int32_t K, int32_t n_group,
                              int32_t topk_group, int32_t x_dtype,
                              const void *x, size_t xrow, const float *W_r,
                              const float *b, float scale, double *s,
                              double *v, double *gs, char *gkeep, char *chosen,
                              int32_t *sel, double *w, double *gap,
                              double *group_gap)
{
    const int32_t per = E / n_group;
    for (int32_t e = 0; e < E; ++e) {
        double z = 0.0;
        for (int32_t j = 0; j < d; ++j)
            z += elem(x, x_dtype, xrow + (size_t)j) * (double)W_r[(size_t)e * d + j];
        s[e] = sigmoid(z);
        v[e] = s[e] + (double)b[e];
        chosen[e] = 0;
    }
    /* group scores: the two largest v of each group, summed */
    for (int32_t g = 0; g < n_group; ++g) {
        double m1 = -INFINITY, m2 = -INFINITY;
        for (int32_t e = g * per; e < (g + 1) * per; ++e) {
            if (v[e] > m1) {
                m2 = m1;
                m1 = v[e];
            } else if (v[e] > m2) {
                m2 = v[e];
            }
        }
        gs[g] = m1 + m2;
        gkeep[g] = 0;
    }
    /* keep topk_group groups: rounds of "largest unkept score", scanning g
     * upward with a strict comparison (ties toward the lower group index) */
    double last_kept = INFINITY;
    for (int32_t k = 0; k < topk_group; ++k) {
        int32_t best = -1;
        for (int32_t g = 0; g < n_group; ++g)
            if (!gkeep[g] && (best < 0 || gs[g] > gs[best]))
                best = g;
        gkeep[best] = 1;
        last_kept = gs[best];
    }
    if (group_gap) {
        double next = -INFINITY;
        for (int32_t g = 0; g < n_group; ++g)
            if (!gkeep[g] && gs[g] > next)
                next = gs[g];
        *group_gap = (topk_group == n_group) ? INFINITY : last_kept - next;
    }
    /* experts of dropped groups take 0.0 */
    for (int32_t e = 0; e < E; ++e)
        if (!gkeep[e / per])
            v[e] = 0.0;
    for (int32_t k = 0; k < K; ++k) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e)
            if (!chosen[e] && (best < 0 || v[e] > v[best]))
                best = e;
        chosen[best] = 1;
        sel[k] = best;
    }
    if (gap) {
        double vk = v[sel[K - 1]];
        double next = -INFINITY;
        for (int32_t e = 0; e < E; ++e)
            if (!chosen[e] && v[e] > next)
                next = v[e];
        *gap = (K == E) ? INFINITY : vk - next;
    }
    for (int32_t i = 1; i < K; ++i) {
        int32_t key = sel[i], j = i - 1;
        while (j >= 0 && sel[j] > key) {
            sel[j + 1] = sel[j];
            --j;
        }
        sel[j + 1] = key;
    }
    double den = 0.0;
    for (int32_t k = 0; k < K; ++k)
        den += s[sel[k]];
    den += 1e-20;
    for (int32_t k = 0; k < K; ++k)
        w[k] = (s[sel[k]] / den) * (double)scale;
}

int oracle_router_grouped(int32_t T, int32_t d, int32_t E, int32_t K,
                          int32_t n_group, int32_t topk_group, int32_t x_dtype,
                          const void *x, const float *W_r, const float *b,
                          float scale, int32_t *topk_idx, double *topk_w,
                          double *gap, double *group_gap, double *scores,
                          int32_t nthreads)
{
    if (T < 0 || d <= 0 || E <= 0 || K < 1 || K > E || n_group < 1 ||
        E % n_group != 0 || topk_group < 1 || topk_group > n_group ||
        (n_group > 1 && E / n_group < 2))
        return ORACLE_ERR_SHAPE;
    if (x_dtype != ORACLE_F32 && x_dtype != ORACLE_BF16)
        return ORACLE_ERR_SHAPE;
    if (T > 0 && (!x || !W_r || !b || !topk_idx || !topk_w))
        return ORACLE_ERR_NULL;
    int nt = nthreads > 0 ? nthreads : 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int32_t t = 0; t < T; ++t) {
        double *s = (double *)malloc(sizeof(double) * (size_t)E);
        double *v = (double *)malloc(sizeof(double) * (size_t)E);
        double *gs = (double *)malloc(sizeof(double) * (size_t)n_group);
        char *gkeep = (char *)malloc((size_t)n_group);
        char *chosen = (char *)malloc((size_t)E);
        double g = 0.0, gg = 0.0;
        route_one_grouped(d, E, K, n_group, topk_group, x_dtype, x,
                          (size_t)t * d, W_r, b, scale, s, v, gs, gkeep, chosen,
                          topk_idx + (size_t)t * K, topk_w + (size_t)t * K, &g,
                          &gg);
        if (gap)
            gap[t] = g;
        if (group_gap)
            group_gap[t] = gg;
        if (scores)
            memcpy(scores + (size_t)t * E, s, sizeof(double) * (size_t)E);
        free(s);
        free(v);
        free(gs);
        free(gkeep);
        free(chosen);
    }
    return ORACLE_OK;
}

int oracle_dispatch(int32_t T, int32_t E, int32_t K, const int32_t *topk_idx,
                    int32_t *counts, int32_t *offsets, int32_t *sorted_token,
                    int32_t *pos)
{
    if (T < 0 || E <= 0 || K < 1)
        return ORACLE_ERR_SHAPE;
    if (!counts || !offsets || (T > 0 && (!topk_idx || !sorted_token || !pos)))
        return ORACLE_ERR_NULL;
    for (int64_t a = 0; a < (int64_t)T * K; ++a)
        if (topk_idx[a] < 0 || topk_idx[a] >= E)
            return ORACLE_ERR_SHAPE;
    /* histogram */
    for (int32_t e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t a = 0; a < (int64_t)T * K; ++a)
        counts[topk_idx[a]] += 1;
    /* exclusive scan */
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    /* stable placement: visiting tokens in ascending order fills each
     * expert's segment in ascending token order */
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    for (int32_t e = 0; e < E; ++e)
        cursor[e] = offsets[e];
    for (int32_t t = 0; t < T; ++t)
        for (int32_t k = 0; k < K; ++k) {
            int32_t e = topk_idx[(size_t)t * K + k];
            int32_t p = cursor[e]++;
            sorted_token[p] = t;
            pos[(size_t)t * K + k] = p;
        }
    free(cursor);
    return ORACLE_OK;
}

/* y[o] = sum_f Wd[o*ldd + col0 + f] * h[f],
 * h[f] = silu(sum_j Wg[(row0+f)*din + j] v[j]) * (sum_j Wu[(row0+f)*din + j] v[j])
 * The SwiGLU expert of the llm-arch-kb entry (three matrices of
 * d_model x d_ff each); matrices in [out, in] layout like the router. */
static void swiglu(int32_t din, int32_t F, int32_t dout, const double *vin,
                   int32_t wdt, const void *Wg, const void *Wu, size_t row0,
                   const void *Wd, size_t ldd, size_t col0, double *h,
                   double *y)
{
    for (int32_t f = 0; f < F; ++f) {
        double g = 0.0, u = 0.0;
        size_t base = (row0 + (size_t)f) * (size_t)din;
        for (int32_t j = 0; j < din; ++j) {
            g += elem(Wg, wdt, base + (size_t)j) * vin[j];
            u += elem(Wu, wdt, base + (size_t)j) * vin[j];
        }
        h[f] = g * sigmoid(g) * u;
    }
    for (int32_t o = 0; o < dout; ++o) {
        double acc = 0.0;
        for (int32_t f = 0; f < F; ++f)
            acc += elem(Wd, wdt, (size_t)o * ldd + col0 + (size_t)f) * h[f];
        y[o] = acc;
    }
}

/* out = A v for A [rows, cols] stored row-major. */
static void matvec(int32_t rows, int32_t cols, const void *A, int32_t dt,
                   const double *v, double *out)
{
    for (int32_t r = 0; r < rows; ++r) {
        double acc = 0.0;
        for (int32_t c = 0; c < cols; ++c)
            acc += elem(A, dt, (size_t)r * cols + c) * v[c];
        out[r] = acc;
    }
}

static int check_layer(const oracle_layer *L)
{
    if (!L)
        return ORACLE_ERR_NULL;
    if (L->d <= 0 || L->E <= 0 || L->K < 1 || L->K > L->E || L->F <= 0 ||
        L->n_shared < 0 || L->d_latent < 0 ||
        (L->n_shared > 0 && L->F_shared <= 0))
        return ORACLE_ERR_SHAPE;
    if ((L->act_dtype != ORACLE_F32 && L->act_dtype != ORACLE_BF16) ||
        (L->w_dtype != ORACLE_F32 && L->w_dtype != ORACLE_BF16 && L->w_dtype != ORACLE_FP8))
        return ORACLE_ERR_SHAPE;
    if (L->w_dtype == ORACLE_FP8) {
        int32_t din = L->d_latent ? L->d_latent : L->d;
        if ((L->sw_dtype != ORACLE_F32 && L->sw_dtype != ORACLE_BF16) || L->F % 128 || din % 128)
            return ORACLE_ERR_SHAPE;
        if (!L->W_gate_scale || !L->W_up_scale || !L->W_down_scale)
            return ORACLE_ERR_NULL;
    }
    if (!L->W_gate || !L->W_up || !L->W_down)
        return ORACLE_ERR_NULL;
    if (L->n_shared > 0 && (!L->Ws_gate || !L->Ws_up || !L->Ws_down))
        return ORACLE_ERR_NULL;
    if (L->d_latent > 0 && (!L->W_lat_down || !L->W_lat_up))
        return ORACLE_ERR_NULL;
    return ORACLE_OK;
}

int oracle_forward_given_routing(const oracle_layer *L, int32_t T,
                                 const void *x, const int32_t *topk_idx,
                                 const double *topk_w, double *out,
                                 int32_t nthreads)
{
    int rc = check_layer(L);
    if (rc)
        return rc;
    if (T < 0)
        return ORACLE_ERR_SHAPE;
    if (T == 0)
        return ORACLE_OK;
    if (!x || !topk_idx || !topk_w || !out)
        return ORACLE_ERR_NULL;
    const int32_t d = L->d, K = L->K, F = L->F;
    const int32_t din = L->d_latent ? L->d_latent : d;
    /* every selected expert must be supplied */
    for (int64_t a = 0; a < (int64_t)T * K; ++a) {
        int32_t e = topk_idx[a];
        if (e < 0 || e >= L->E)
            return ORACLE_ERR_SHAPE;
        if (!L->W_gate[e] || !L->W_up[e] || !L->W_down[e])
            return ORACLE_ERR_NULL;
        if (L->w_dtype == ORACLE_FP8 &&
            (!L->W_gate_scale[e] || !L->W_up_scale[e] || !L->W_down_scale[e]))
            return ORACLE_ERR_NULL;
    }
    /* dtype of the shared experts and latent maps */
    const int32_t sdt = L->w_dtype == ORACLE_FP8 ? L->sw_dtype : L->w_dtype;
    const int32_t Fs_all = L->n_shared * L->F_shared;
    const int32_t hmax = F > L->F_shared ? F : L->F_shared;
    int nt = nthreads > 0 ? nthreads : 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int32_t t = 0; t < T; ++t) {
        double *xd = (double *)malloc(sizeof(double) * (size_t)d);
        double *xin = (double *)malloc(sizeof(double) * (size_t)din);
        double *routed_in = (double *)malloc(sizeof(double) * (size_t)din);
        double *y = (double *)malloc(sizeof(double) * (size_t)(din > d ? din : d));
        double *h = (double *)malloc(sizeof(double) * (size_t)hmax);
        double *o = out + (size_t)t * d;
        for (int32_t j = 0; j < d; ++j)
            xd[j] = elem(x, L->act_dtype, (size_t)t * d + j);
        /* routed experts' input: x, or its latent compression [P4] */
        if (L->d_latent)
            matvec(din, d, L->W_lat_down, sdt, xd, xin);
        else
            memcpy(xin, xd, sizeof(double) * (size_t)d);
        /* weighted sum of the selected experts, in slot order [P1 sec. 3] */
        for (int32_t j = 0; j < din; ++j)
            routed_in[j] = 0.0;
        for (int32_t k = 0; k < K; ++k) {
            int32_t e = topk_idx[(size_t)t * K + k];
            if (L->w_dtype == ORACLE_FP8)
                swiglu_fp8(din, F, xin, (const uint8_t *)L->W_gate[e], L->W_gate_scale[e],
                           (const uint8_t *)L->W_up[e], L->W_up_scale[e],
                           (const uint8_t *)L->W_down[e], L->W_down_scale[e], h, y);
            else
                swiglu(din, F, din, xin, L->w_dtype, L->W_gate[e], L->W_up[e], 0,
                       L->W_down[e], (size_t)F, 0, h, y);
            double wk = topk_w[(size_t)t * K + k];
            for (int32_t j = 0; j < din; ++j)
                routed_in[j] += wk * y[j];
        }
        /* back to the model width [P4]; identity in the K2 form */
        if (L->d_latent)
            matvec(d, din, L->W_lat_up, sdt, routed_in, o);
        else
            memcpy(o, routed_in, sizeof(double) * (size_t)d);
        /* always-on shared experts, unweighted [P1 sec. 3; P4] */
        for (int32_t sidx = 0; sidx < L->n_shared; ++sidx) {
            swiglu(d, L->F_shared, d, xd, sdt, L->Ws_gate, L->Ws_up,
                   (size_t)sidx * L->F_shared, L->Ws_down, (size_t)Fs_all,
                   (size_t)sidx * L->F_shared, h, y);
            for (int32_t j = 0; j < d; ++j)
                o[j] += y[j];
        }
        free(xd);
        free(xin);
        free(routed_in);
        free(y);
        free(h);
    }
    return ORACLE_OK;
}

int oracle_fp8_dequant(int32_t rows, int32_t cols, const uint8_t *codes,
                       const uint8_t *scales, double *out)
{
    if (rows <= 0 || cols <= 0 || rows % 128 || cols % 128)
        return ORACLE_ERR_SHAPE;
    if (!codes || !scales || !out)
        return ORACLE_ERR_NULL;
    for (int32_t r = 0; r < rows; ++r)
        for (int32_t c = 0; c < cols; ++c)
            out[(size_t)r * cols + c] = fp8_elem(codes, scales, cols, r, c);
    return ORACLE_OK;
}

int oracle_forward(const oracle_layer *L, int32_t T, const void *x,
                   double *out, int32_t *topk_idx, double *topk_w,
                   double *gap, int32_t nthreads)
{
    int rc = check_layer(L);
    if (rc)
        return rc;
    if (T < 0)
        return ORACLE_ERR_SHAPE;
    if (T == 0)
        return ORACLE_OK;
    if (!x || !out || !L->W_r || !L->b)
        return ORACLE_ERR_NULL;
    int32_t *idx = topk_idx ? topk_idx
                            : (int32_t *)malloc(sizeof(int32_t) * (size_t)T * L->K);
    double *w = topk_w ? topk_w
                       : (double *)malloc(sizeof(double) * (size_t)T * L->K);
    rc = oracle_router(T, L->d, L->E, L->K, L->act_dtype, x, L->W_r, L->b,
                       L->scale, idx, w, gap, NULL, nthreads);
    if (!rc)
        rc = oracle_forward_given_routing(L, T, x, idx, w, out, nthreads);
    if (!topk_idx)
        free(idx);
    if (!topk_w)
        free(w);
    return rc;
}

/* Aux-loss-free bias update [P1: the bias follows DeepSeek V3's schedule,
 * gamma = 1e-3, sign-only; P4: the bias is a load-adjustment term].  With
 * the batch's per-expert selection counts c_e and their mean
 * cbar = sum(c) / E, an expert above the mean is made less attractive and
 * one below it more: b_e <- b_e + gamma * sgn(cbar - c_e), sgn(0) = 0.  The
 * comparison is taken exactly as sum(c) - E c_e in integers; the new bias is
 * the fp32 rounding of the exact sum (the bias is an fp32 tensor). */
int oracle_bias_update(int32_t E, const int32_t *counts, const float *b_in,
                       float gamma, float *b_out)
{
    if (E <= 0)
        return ORACLE_ERR_SHAPE;
    if (!counts || !b_in || !b_out)
        return ORACLE_ERR_NULL;
    int64_t total = 0;
    for (int32_t e = 0; e < E; ++e)
        total += counts[e];
    for (int32_t e = 0; e < E; ++e) {
        int64_t diff = total - (int64_t)E * counts[e];
        double sg = diff > 0 ? 1.0 : (diff < 0 ? -1.0 : 0.0);
        b_out[e] = (float)((double)b_in[e] + (double)gamma * sg);
    }
    return ORACLE_OK;
}

static int cmp_desc(const void *a, const void *b)
{
    double x = *(const double *)a, y = *(const double *)b;
    return (x < y) - (x > y);
}

/* Quantile Balancing [P4, the load-balancing paragraph: a quantile of the
 * router scores gives each expert's selection bias, namely the score at
 * which that expert reaches its target load].  Reading:
 * over the batch, s[t, e] = sigmoid(x_t . W_r[e]) (the unbiased router
 * scores, as in oracle_router); every expert's target is the mean load
 * n = max(1, floor(T K / E)) tokens; its threshold theta_e is the n-th
 * largest of s[., e] (the expert would take exactly n tokens if it took
 * those scoring at least theta_e); the bias puts every threshold on a common
 * level: b_e = mean(theta) - theta_e, so the test s + b >= mean(theta) is
 * s >= theta_e for each expert.  A common shift of b leaves every top-K
 * unchanged, the mean keeps sum(b) = 0.  theta [E] (nullable) returns the
 * thresholds.  Requires T >= 1. */
int oracle_bias_quantile(int32_t T, int32_t d, int32_t E, int32_t K,
                         int32_t x_dtype, const void *x, const float *W_r,
                         double *b_out, double *theta, int32_t nthreads)
{
    if (T < 1 || d <= 0 || E <= 0 || K < 1 || K > E)
        return ORACLE_ERR_SHAPE;
    if (x_dtype != ORACLE_F32 && x_dtype != ORACLE_BF16)
        return ORACLE_ERR_SHAPE;
    if (!x || !W_r || !b_out)
        return ORACLE_ERR_NULL;
    int64_t n = ((int64_t)T * K) / E;
    if (n < 1)
        n = 1;
    double *th = (double *)malloc(sizeof(double) * (size_t)E);
    int nt = nthreads > 0 ? nthreads : 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int32_t e = 0; e < E; ++e) {
        double *col = (double *)malloc(sizeof(double) * (size_t)T);
        for (int32_t t = 0; t < T; ++t) {
            double z = 0.0;
            for (int32_t j = 0; j < d; ++j)
                z += elem(x, x_dtype, (size_t)t * d + (size_t)j) * (double)W_r[(size_t)e * d + j];
            col[t] = sigmoid(z);
        }
        qsort(col, (size_t)T, sizeof(double), cmp_desc);
        th[e] = col[n - 1];
        free(col);
    }
    double mean = 0.0;
    for (int32_t e = 0; e < E; ++e)
        mean += th[e];
    mean /= (double)E;
    for (int32_t e = 0; e < E; ++e) {
        b_out[e] = mean - th[e];
        if (theta)
            theta[e] = th[e];
    }
    free(th);
    return ORACLE_OK;
}

