/*
 * moe.h -- C ABI of the MI355X (gfx950) Kimi-K2-style MoE layer forward.
 *
 * The layer (sources by page title and section):
 *   Router -- OpenModelAtlas "Kimi K2 · Router", the four steps and the
 *   MoEGate excerpt:  z = x W_r^T (fp32),  s = sigmoid(z),
 *   S = top_K(s + b) (the bias only chooses),  w_i = scale * s_i /
 *   (sum_{j in S} s_j + 1e-20) for i in S.
 *   Experts -- llm-arch-kb "Kimi K2 MoE" sections 2 and 3: SwiGLU experts
 *   f(v) = W_down (silu(W_gate v) * (W_up v)); the layer returns the
 *   always-on shared expert(s) plus sum_{i in S} w_i f_i(x).
 *   Latent form -- lilting.ch "Kimi K3's router picks 16 of 896 experts",
 *   the K3 table and the Stable LatentMoE paragraph: routed experts act on
 *   x_lat = W_lat_down x, their weighted sum is mapped back by W_lat_up,
 *   the shared experts act on x.
 * Readings where the pages leave a choice open:
 *   - ties in s + b go to the lower expert index;
 *   - the K slots of a token are written in ascending expert id;
 *   - dispatch is dropless (every token reaches exactly K experts);
 *   - several shared experts are stacked along their intermediate axis
 *     (their outputs are summed, unweighted);
 *   - intermediate activations (H = silu(g)*u, expert outputs, x_lat and
 *     the latent weighted sum) are rounded to the activation dtype; all
 *     products accumulate in fp32; the output is rounded once (RNE).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller, row-major,
 *     16-byte aligned.  The library never allocates, frees or retains memory;
 *     scratch lives in the caller's workspace (see moe_workspace_size), or,
 *     for moe_forward_noalloc only, in a fixed array the library holds.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work on it and return without synchronising; results are
 *     ready when the stream reaches them.  Concurrent calls need distinct
 *     workspaces.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     an error nothing is enqueued and no output is touched.  A failed
 *     kernel launch returns MOE_ERR_HIP; faults inside kernels surface at
 *     the caller's next synchronisation.
 *   - Limits: 1 <= K <= min(E, 16); E <= 1024; d, F, F_shared and d_latent
 *     are positive multiples of 64; 0 <= n_shared <= 8; T*K < 2^31.
 *   - T == 0 is a no-op: the data pointers may then be NULL (empty tensors);
 *     non-NULL expert_counts / expert_offsets are zero-filled.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* MOE_FP8_E4M3 is a weight dtype only: OCP FP8 E4M3FN codes (sign, 4
 * exponent bits with bias 7, 3 mantissa bits; 0x7F and 0xFF are NaN, no
 * infinities) with one E8M0 scale per 128 x 128 block (see
 * moe_expert_weights).                                                      */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL                    */
    MOE_ERR_SHAPE = 2,       /* a size is out of range                        */
    MOE_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned              */
    MOE_ERR_WORKSPACE = 4,   /* workspace smaller than moe_workspace_size()   */
    MOE_ERR_UNSUPPORTED = 5, /* a dtype combination the library does not run  */
    MOE_ERR_HIP = 6,         /* a HIP launch failed                           */
    MOE_ERR_SCRATCH = 7      /* moe_forward_noalloc: the layer needs more     */
                             /* scratch than MOE_NOALLOC_SCRATCH_BYTES        */
} moe_status;

typedef struct {
    int32_t T;         /* tokens: batch x positions flattened                 */
    int32_t d;         /* model dimension (7168 for K2 and K3)                */
    int32_t E;         /* routed experts (384 for K2, 896 for K3)             */
    int32_t K;         /* experts per token (8 for K2, 16 for K3)             */
    int32_t F;         /* routed-expert intermediate size                     */
    int32_t n_shared;  /* always-on shared experts (1 for K2, 2 for K3)       */
    int32_t F_shared;  /* intermediate size of EACH shared expert             */
    int32_t d_latent;  /* 0 = experts act on x; else the latent width (3584)  */
    float scale;       /* routed scaling factor (2.827 for K2)                */
    int32_t act_dtype; /* moe_dtype of x, out and the intermediates           */
    int32_t w_dtype;   /* moe_dtype of expert, shared and latent weights;     */
                       /* equal to act_dtype (W_r and b are always fp32), or  */
                       /* MOE_FP8_E4M3: routed experts in block-scaled FP8,   */
                       /* shared and latent weights bf16 (act_dtype bf16,     */
                       /* MOE_LAYOUT_FRAG16; d_in and F multiples of 128 and  */
                       /* at most 8192)                                       */
    int32_t w_layout;  /* moe_weight_layout of those weights (bf16 and FP8    */
                       /* may be, and FP8 must be, MOE_LAYOUT_FRAG16; fp32    */
                       /* must be MOE_LAYOUT_ROWS)                            */
    int32_t n_group;   /* group-limited choice: expert groups (0 or 1: none)  */
    int32_t topk_group;/* groups kept per token when n_group > 1              */
} moe_layer_desc;

/* Storage of the expert, shared and latent weight matrices.
 *   MOE_LAYOUT_ROWS: row-major [rows, cols] (nn.Linear [out, in]).
 *   MOE_LAYOUT_FRAG16, bf16 matrices: each [rows, cols] matrix as
 *     (rows/16) x (cols/32) blocks of 16 rows x 32 columns, block (i, j) at
 *     element offset (i * (cols/32) + j) * 512; inside a block, element
 *     (r, c) at ((c / 8) * 16 + r) * 8 + c % 8.  A block is then exactly
 *     the B operand of one v_mfma_f32_16x16x32_bf16 in lane order (lane l
 *     holds row l % 16, columns 8 (l / 16) .. 8 (l / 16) + 7), so the GEMMs
 *     read weights as whole 1 KiB blocks.
 *   MOE_LAYOUT_FRAG16, FP8 matrices (the routed experts under
 *     MOE_FP8_E4M3): (rows/16) x (cols/64) blocks of 16 rows x 64 columns,
 *     block (i, j) at byte (i * (cols/64) + j) * 1024; inside a block,
 *     element (r, c) at byte (((c % 32) / 8) * 16 + r) * 16 + (c / 32) * 8
 *     + c % 8, so lane l's 16 bytes hold the codes of the two bf16 operands
 *     (columns 0-31 and 32-63) that lane feeds.
 *   Stacked matrices (W_gate etc.) keep their per-expert stride rows * cols
 *   elements; the sizes of all buffers are those of the row-major layout.
 *   moe_pack_weights converts.                                              */
typedef enum { MOE_LAYOUT_ROWS = 0, MOE_LAYOUT_FRAG16 = 1 } moe_weight_layout;

/* Expert weights, nn.Linear layout [out, in]; d_in = d_latent ? d_latent : d.
 *   W_gate, W_up [E, F, d_in];  W_down [E, d_in, F]
 *   Ws_gate, Ws_up [n_shared*F_shared, d];  Ws_down [d, n_shared*F_shared]
 *     (shared expert s owns rows/columns [s*F_shared, (s+1)*F_shared))
 *   W_lat_down [d_latent, d];  W_lat_up [d, d_latent]  (NULL if d_latent == 0)
 * Shared pointers may be NULL when n_shared == 0.
 * Block scales of FP8 routed experts (OpenModelAtlas "Kimi K2 · Router": the
 * released weights are FP8 with block scales; the block shape and scale
 * encoding are this library's reading), used only when w_dtype is
 * MOE_FP8_E4M3:
 *   W_gate_scale, W_up_scale [E, F/128, d_in/128];  W_down_scale
 *   [E, d_in/128, F/128], uint8 E8M0 exponents s (row-major over blocks,
 *   not repacked), so that element (r, c) of a matrix is
 *   code(r, c) * 2^(s[r/128][c/128] - 127).  The product is rounded to
 *   bf16 before the MFMA; it is exact (3 mantissa bits) while it lies in
 *   bf16's normal range.  s = 255 (NaN in E8M0) is not supported.           */
typedef struct {
    const void *W_gate, *W_up, *W_down;
    const void *Ws_gate, *Ws_up, *Ws_down;
    const void *W_lat_down, *W_lat_up;
    const uint8_t *W_gate_scale, *W_up_scale, *W_down_scale;
} moe_expert_weights;

/* Bytes of device workspace moe_router (for_forward = 0) or moe_forward
 * (for_forward != 0) needs for this descriptor; 0 if the descriptor is
 * invalid.  Host-only; touches no device.                                    */
size_t moe_workspace_size(const moe_layer_desc *desc, int for_forward);

/* Router [router card, four steps and MoEGate excerpt].
 *   x [T, d] (act_dtype), W_r [E, d] fp32, b [E] fp32
 *   -> topk_idx [T, K] int32 (ascending expert id within each token),
 *      topk_w [T, K] fp32, expert_counts [E] int32 (nullable: tokens per
 *      expert).
 * With n_group > 1 (the excerpt's group-limited branch): the experts form
 * n_group contiguous groups, a group scores the sum of its two largest
 * s + b, the topk_group best groups are kept (ties toward the lower group
 * index) and the experts of the other groups compete with the value 0.0
 * (the excerpt's masked_fill) in the top-K.  Requires n_group <= 64,
 * E % n_group == 0, E / n_group >= 2 and 1 <= topk_group <= n_group.        */
moe_status moe_router(const moe_layer_desc *desc, const void *x,
                      const float *W_r, const float *b, int32_t *topk_idx,
                      float *topk_w, int32_t *expert_counts, void *workspace,
                      size_t workspace_bytes, void *stream);

/* Stage boundaries of moe_forward, for timing: when `stage_events` is not
 * NULL it points to MOE_NUM_STAGE_EVENTS hipEvent_t handles (created by the
 * caller; a NULL entry is skipped) that are recorded on `stream`:
 *   [MOE_EV_START]    before the first kernel
 *   [MOE_EV_ROUTER]   after the router (logits, top-K gate)
 *   [MOE_EV_DISPATCH] after histogram, scan and permutation
 *   [MOE_EV_LATENT]   after x_lat = x W_lat_down^T (same point as the
 *                     previous event in the K2 form)
 *   [MOE_EV_UP]       after the gate/up projection with SwiGLU (one kernel)
 *   [MOE_EV_DOWN]     after the down projection (one kernel)
 *   [MOE_EV_END]      after the combine (and latent up-projection)          */
enum {
    MOE_EV_START = 0,
    MOE_EV_ROUTER = 1,
    MOE_EV_DISPATCH = 2,
    MOE_EV_LATENT = 3,
    MOE_EV_UP = 4,
    MOE_EV_DOWN = 5,
    MOE_EV_END = 6,
    MOE_NUM_STAGE_EVENTS = 7
};

/* Whole layer [router card; llm-arch-kb K2 MoE sections 2-3; K3 essay].
 *   x [T, d], W_r [E, d], b [E], weights as above -> out [T, d] (act_dtype).
 * Optional outputs (each nullable), for inspection and parity checks:
 *   topk_idx [T, K], topk_w [T, K], expert_counts [E],
 *   expert_offsets [E + 1] (exclusive scan of the counts),
 *   sorted_token [T*K]: for e ascending, the tokens routed to e, ascending.  */
moe_status moe_forward(const moe_layer_desc *desc, const void *x,
                       const float *W_r, const float *b,
                       const moe_expert_weights *weights, void *out,
                       int32_t *topk_idx, float *topk_w,
                       int32_t *expert_counts, int32_t *expert_offsets,
                       int32_t *sorted_token, void *workspace,
                       size_t workspace_bytes, void *stream,
                       void *const *stage_events);

/* One GPU's share of an expert-parallel layer [K3 essay, load-imbalance
 * paragraph: the work of the tokens routed to an expert falls on the GPU
 * that holds it; the routed sum of llm-arch-kb K2 MoE section 3, split by
 * expert].  The layer has E_total routed experts; this call holds
 * experts e0 .. e0 + desc->E - 1 and applies them to the tokens of x with
 * the routing a moe_router call over all E_total experts returned:
 *   out[t] = shared(x_t) + sum over the k with e0 <= topk_idx[t,k] < e0 + E
 *            of topk_w[t,k] * expert_{topk_idx[t,k]}(x_t)
 * (the shared term only when desc->n_shared > 0; latent form: the sum is
 * taken in latent space, then mapped up together with the shared experts,
 * as in moe_forward).  Summing the outputs of slices that cover all
 * E_total experts, one of them with the shared experts, gives the whole
 * layer up to rounding; the slice [0, E_total) with the shared experts is
 * moe_forward after its router, bit for bit.
 *   desc: the layer with E = the slice's expert count; K (at most
 *         min(E_total, 16)), shapes and dtypes as for moe_forward (n_group,
 *         topk_group and scale are not used: the routing is given).
 *   weights: the slice's experts only (W_gate [E, F, din] ... in the
 *         descriptor's layout), plus the shared and latent matrices as
 *         moe_forward takes them.
 *   topk_idx [T, K] int32, topk_w [T, K] fp32: any expert id; ids outside
 *         the slice are skipped.
 *   expert_counts [E], expert_offsets [E + 1], sorted_token [T*K]: as for
 *         moe_forward over the slice's local experts 0 .. E - 1 (nullable).
 *   workspace: at least moe_slice_workspace_size(desc, e0, E_total) bytes.
 * MOE_ERR_SHAPE when e0 < 0, E_total outside 1 .. 1024 or e0 + E >
 * E_total; the other errors as for moe_forward, all before anything is
 * enqueued.                                                                 */
size_t moe_slice_workspace_size(const moe_layer_desc *desc, int32_t e0,
                                int32_t E_total);
moe_status moe_forward_slice(const moe_layer_desc *desc,
                             const moe_expert_weights *weights, const void *x,
                             const int32_t *topk_idx, const float *topk_w,
                             int32_t e0, int32_t E_total, void *out,
                             int32_t *expert_counts, int32_t *expert_offsets,
                             int32_t *sorted_token, void *workspace,
                             size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * whole layer exactly as moe_forward (same arguments, kernels and results),
 * but its scratch is a fixed array of MOE_NOALLOC_SCRATCH_BYTES (128 MiB)
 * that the library holds on each GPU it runs on until the process ends, so
 * no workspace is passed and nothing is allocated.  Enough for the K2 layer
 * up to T = 512 tokens and the K3 latent layer at T = 256; a descriptor
 * needing more (moe_workspace_size(desc, 1) > MOE_NOALLOC_SCRATCH_BYTES)
 * returns MOE_ERR_SCRATCH with nothing enqueued.  The array of the current
 * device is used (its address is resolved on the first call on that
 * device), so `stream` must belong to the current device.  All calls on one
 * GPU share that array and it keeps the last call's contents (no call reads
 * a byte of it that the same call did not write first): calls that overlap
 * in time on one GPU -- on different streams, or from several threads --
 * race on it and must be serialised by the caller.                         */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
moe_status moe_forward_noalloc(const moe_layer_desc *desc, const void *x,
                               const float *W_r, const float *b,
                               const moe_expert_weights *weights, void *out,
                               int32_t *topk_idx, float *topk_w,
                               int32_t *expert_counts, int32_t *expert_offsets,
                               int32_t *sorted_token, void *stream);

/* Aux-loss-free bias update after a batch [llm-arch-kb "Kimi K2 MoE"
 * section 2: the selection bias follows DeepSeek V3's schedule, sign only,
 * gamma = 1e-3; lilting.ch K3 essay: a per-expert load-adjustment bias].
 * expert_counts [E] int32 are the batch's selections per expert (as
 * moe_router / moe_forward return them, or summed over several batches);
 * b [E] fp32 is updated in place:
 *   b[e] += gamma * sgn(mean(expert_counts) - expert_counts[e])
 * with sgn(0) = 0 and the comparison taken exactly (sum(c) - E c_e), so an
 * expert above the mean load becomes less likely to be chosen.  Only E of
 * the descriptor is used.                                                    */
moe_status moe_bias_update(const moe_layer_desc *desc,
                           const int32_t *expert_counts, float *b,
                           float gamma, void *stream);

/* Quantile Balancing [lilting.ch K3 essay, the load-balancing paragraph:
 * each expert's selection bias comes from a quantile of the router scores,
 * namely the score theta_e at which expert e gets its target load].
 * This library's reading: over the batch x [T, d], s = sigmoid(x W_r^T)
 * (the unbiased scores, computed as in moe_router); every expert's target
 * is the mean load n = max(1, floor(T K / E)); theta_e = the n-th largest
 * s[., e]; the bias is written as
 *   b[e] = mean(theta) - theta_e        (b [E] fp32, output only)
 * so that s + b >= mean(theta) is s >= theta_e for every expert.  Uses
 * T, d, E, K and act_dtype of the descriptor; 1 <= T <= 32768; workspace of
 * at least moe_workspace_size(desc, 0) bytes.  Training-time work: the
 * pages fix the bias at inference.                                           */
moe_status moe_bias_quantile(const moe_layer_desc *desc, const void *x,
                             const float *W_r, float *b, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Rewrite row-major weights into MOE_LAYOUT_FRAG16 (a pure permutation of
 * each matrix; done once, e.g. when a model is loaded).  Every non-NULL
 * matrix of `src` (row-major, shapes from `desc`, whose w_layout is
 * ignored) is written to the same member of `dst`, which must then be
 * non-NULL, 16-byte aligned, of the same size and not overlap it.
 * Requires w_dtype MOE_BF16, or MOE_FP8_E4M3 (routed matrices as FP8 codes,
 * shared and latent ones bf16; the block scales are not touched and keep
 * their layout).  Shapes are checked as for moe_forward on the packed
 * result.  Enqueued on `stream` like the other calls.                       */
moe_status moe_pack_weights(const moe_layer_desc *desc,
                            const moe_expert_weights *src,
                            const moe_expert_weights *dst, void *stream);

/* Static text for a status code.                                            */
const char *moe_status_str(moe_status status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
