/*
 * oracle.h -- plain CPU oracle of the Kimi-K2-style MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library; neither includes the other.
 *
 * Everything is evaluated in double precision on the exact (upcast) input
 * values, with plain loops and no blocking, fusion or reordering beyond what
 * the layer's definition states.  Sources (page title and section):
 *   [P3] OpenModelAtlas, "Kimi K2 · Router": the four steps
 *        z = x W_r, s = sigmoid(z), E_sel = [i in top_8(s + b)],
 *        G_i = 2.827 * s_i E_sel_i / sum_j s_j E_sel_j; the MoEGate code
 *        excerpt (fp32 logits, sigmoid, bias only for choice, gather of the
 *        unbiased scores, sum + 1e-20, then the routed scaling factor).
 *   [P1] llm-arch-kb, "Kimi K2 MoE", section 2 (top-K of the biased gate,
 *        weights from the unbiased gate over the selected set, sigmoid not
 *        softmax, SwiGLU experts with 3 matrices) and section 3 (the layer
 *        returns shared_expert(x) + the weighted routed outputs).
 *   [P4] lilting.ch, "Kimi K3's router picks 16 of 896 experts", the K3
 *        table and the Stable LatentMoE paragraph (routed experts act on a
 *        3584-wide compression of x, their combined output is projected
 *        back to 7168, two shared experts act on x itself).
 *   [P3] also states that the released checkpoint stores its weights in
 *        FP8 with block scales; it gives neither the element format nor the
 *        block shape nor the scale encoding.  This oracle's reading: OCP
 *        E4M3FN codes, one power-of-two scale (E8M0 exponent) per 128 x 128
 *        block, applied to the routed experts only.
 * Readings where the pages are silent (slot order, tie-break, SwiGLU form,
 * latent maps, shared-expert stacking, the FP8 format) are stated at each
 * function.
 *
 * Error behaviour: every function returns ORACLE_OK (0) or an error code;
 * argument checks run before any output is written, except that
 * oracle_forward may have written the routing when the expert step then
 * finds a selected expert missing.  All pointers are host pointers owned by
 * the caller.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_FP8 = 2 };
enum { ORACLE_OK = 0, ORACLE_ERR_NULL = 1, ORACLE_ERR_SHAPE = 2 };

typedef struct {
    int32_t d;          /* model dimension                                     */
    int32_t E;          /* routed experts                                      */
    int32_t K;          /* experts per token                                   */
    int32_t F;          /* routed intermediate size                            */
    int32_t n_shared;   /* always-on shared experts                            */
    int32_t F_shared;   /* intermediate size of each shared expert             */
    int32_t d_latent;   /* 0: experts act on x; else on W_lat_down x           */
    int32_t act_dtype;  /* ORACLE_F32 or ORACLE_BF16 (bf16 given as raw bits) */
    int32_t w_dtype;    /* dtype of expert, shared and latent weights          */
    float   scale;      /* routed scaling factor (2.827 for K2)                */
    const float *W_r;   /* [E, d]                                              */
    const float *b;     /* [E]   selection-only bias                          */
    /* Routed experts, one pointer per expert (NULL = not supplied; an error
     * only if a token selects it).  d_in = d_latent ? d_latent : d.
     * W_gate[e], W_up[e]: [F, d_in];  W_down[e]: [d_in, F].                  */
    const void *const *W_gate;
    const void *const *W_up;
    const void *const *W_down;
    /* Shared experts stacked: expert s owns rows [s*F_shared, (s+1)*F_shared)
     * of Ws_gate/Ws_up ([n_shared*F_shared, d]) and the same columns of
     * Ws_down ([d, n_shared*F_shared]).                                       */
    const void *Ws_gate;
    const void *Ws_up;
    const void *Ws_down;
    const void *W_lat_down;  /* [d_latent, d] */
    const void *W_lat_up;    /* [d, d_latent] */
    /* w_dtype == ORACLE_FP8 (block-scaled routed experts): W_gate[e] etc.
     * hold OCP FP8 E4M3FN codes (bias 7, max 448, 0x7F / 0xFF NaN), and
     * W_*_scale[e] one E8M0 code per 128 x 128 block of that matrix
     * (row-major over blocks: [rows/128, cols/128]); element (r, c) is
     * code(r, c) * 2^(scale[r/128][c/128] - 127).  The shared experts and
     * the latent maps then have dtype sw_dtype.  Otherwise these fields are
     * unused and shared / latent weights have dtype w_dtype.              */
    int32_t sw_dtype;
    const uint8_t *const *W_gate_scale;
    const uint8_t *const *W_up_scale;
    const uint8_t *const *W_down_scale;
} oracle_layer;

/* Router [P3 four steps; P3 MoEGate forward; P1 section 2].
 * x: [T, d] of x_dtype.  W_r [E, d], b [E] fp32.
 * Outputs: topk_idx [T, K] int32 -- the selected set in ascending expert id;
 *          topk_w [T, K] -- w_i = (s_i / (sum_S s + 1e-20)) * scale;
 *          gap [T] (nullable) -- v_(K) - v_(K+1) of v = s + b (+inf if K == E);
 *          scores [T, E] (nullable) -- s = sigmoid(z).
 * Selection: the K largest v, ties toward the lower expert index.          */
int oracle_router(int32_t T, int32_t d, int32_t E, int32_t K, int32_t x_dtype,
                  const void *x, const float *W_r, const float *b, float scale,
                  int32_t *topk_idx, double *topk_w, double *gap,
                  double *scores, int32_t nthreads);

/* Dispatch: counts [E], offsets [E+1] (exclusive scan, offsets[E] = T*K),
 * sorted_token [T*K] (for e ascending, every token t that selected e, in
 * ascending t), pos [T, K] (position of assignment (t, slot k) in
 * sorted_token).                                                             */
/* Group-limited router [P3 MoEGate forward, noaux_tc branch].  As
 * oracle_router, except for the choice: experts form n_group contiguous
 * groups; a group scores the sum of its two largest v = s + b; the
 * topk_group best groups are kept (ties toward the lower group index);
 * experts of the other groups take the value 0.0; the K largest values are
 * selected (ties toward the lower expert index).  n_group = 1 (or
 * topk_group = n_group) is oracle_router.  Requires E % n_group == 0,
 * 1 <= topk_group <= n_group and, for n_group > 1, at least 2 experts per
 * group.  group_gap [T] (nullable): smallest kept group score minus the
 * largest dropped one (+inf if all groups are kept).                        */
int oracle_router_grouped(int32_t T, int32_t d, int32_t E, int32_t K,
                          int32_t n_group, int32_t topk_group, int32_t x_dtype,
                          const void *x, const float *W_r, const float *b,
                          float scale, int32_t *topk_idx, double *topk_w,
                          double *gap, double *group_gap, double *scores,
                          int32_t nthreads);

/* Aux-loss-free bias update after a batch [P1 sign-only, gamma = 1e-3;
 * P4 load-adjustment bias]: b_out[e] = fp32(b_in[e] + gamma * sgn(cbar - c_e))
 * with c the per-expert selection counts and cbar their mean (sgn(0) = 0,
 * compared exactly as sum(c) - E c_e).  b_out may equal b_in.              */
int oracle_bias_update(int32_t E, const int32_t *counts, const float *b_in,
                       float gamma, float *b_out);

/* Quantile Balancing [P4 load-balancing paragraph], this reading: with
 * s = sigmoid(x W_r^T) over the batch and the mean load
 * n = max(1, floor(T K / E)), theta_e = the n-th largest s[., e] and
 * b_out[e] = mean(theta) - theta_e (sum zero).  theta [E] nullable.        */
int oracle_bias_quantile(int32_t T, int32_t d, int32_t E, int32_t K,
                         int32_t x_dtype, const void *x, const float *W_r,
                         double *b_out, double *theta, int32_t nthreads);

int oracle_dispatch(int32_t T, int32_t E, int32_t K, const int32_t *topk_idx,
                    int32_t *counts, int32_t *offsets, int32_t *sorted_token,
                    int32_t *pos);

/* Block-scaled FP8 matrix -> doubles [P3 checkpoint note; the format is
 * this oracle's reading]: out[r*cols + c] = e4m3fn(codes[r*cols + c]) *
 * 2^(scales[(r/128)*(cols/128) + c/128] - 127).  rows and cols must be
 * positive multiples of 128.  NaN codes (0x7F, 0xFF) and scale 255 give NaN. */
int oracle_fp8_dequant(int32_t rows, int32_t cols, const uint8_t *codes,
                       const uint8_t *scales, double *out);

/* Expert part of the layer for a given routing [P1 sections 2 and 3; P4]:
 *   out[t] = sum_s f_s(x[t]) + U( sum_k topk_w[t,k] * f_{idx[t,k]}(L(x[t])) )
 * with f(v) = W_down (silu(W_gate v) * (W_up v)), silu(a) = a*sigmoid(a),
 * L = W_lat_down and U = W_lat_up in the latent form, identity otherwise.
 * out: [T, d] double.                                                        */
int oracle_forward_given_routing(const oracle_layer *L, int32_t T,
                                 const void *x, const int32_t *topk_idx,
                                 const double *topk_w, double *out,
                                 int32_t nthreads);

/* Whole layer: oracle_router, then oracle_forward_given_routing.
 * topk_idx, topk_w, gap may be NULL.                                         */
int oracle_forward(const oracle_layer *L, int32_t T, const void *x,
                   double *out, int32_t *topk_idx, double *topk_w,
                   double *gap, int32_t nthreads);

#ifdef __cplusplus
}
#endif
#endif
