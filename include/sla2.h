/*
 * sla2.h — C ABI of libsla2.so: the SLA2 forward (and its backward) on one AMD MI355X (gfx950).
 *
 * SLA2 is sparse-linear attention with a learned block router. The four steps
 * follow the computation-flow paragraph (steps 1-4) of the summary page
 * "SLA2: Sparse-Linear Attention with Learnable Routing and QAT"
 * (paper.rainbus.top), with K smoothing and the per-key-block precompute of
 * §7 (implementation notes 1 and 2) of "SLA2: Sparse-Linear Attention v2 for
 * Diffusion Transformers" (zhaifeiyue.github.io):
 *
 *   router   pool Q (128-row blocks) and K (64-row blocks), project with
 *            proj_q / proj_k, P_c = row softmax(A B^T / sqrt d), hard Top-k
 *            -> block mask M_c and ascending per-row block lists (step 1)
 *   sparse   FlashAttention-style attention over the kept block pairs with
 *            INT8 Q, K and FP8 (OCP E4M3) P, V (step 2)
 *   linear   phi = softmax over d; h_j = phi(K_j)^T V_j, z_j; O_l from the
 *            dropped blocks, O_l = phi(Q) H / (phi(Q) Z) (step 3)
 *   combine  O = alpha * O_s + (1 - alpha) * O_l, alpha per query block (step 4)
 *
 * Conventions shared by every entry point
 *   Layout     Q, K, V: contiguous [B, H, N, d] in shape->dtype. proj_q, proj_k:
 *              fp32 [H, d, d] row-major, applied as x @ W (W[in][out]), no bias.
 *              alpha: fp32 [H, N/128], used as given (expected in [0, 1]).
 *              Outputs O, O_s, O_l: fp32 [B, H, N, d]. Masks: uint8 0/1
 *              [B, H, N/128, N/64]. Block lists: int32, ascending.
 *   Shapes     d == 128; N a positive multiple of 128, N <= 262144; B, H >= 1;
 *              B*H <= 65535. Otherwise SLA2_ERR_BAD_SHAPE.
 *   Kept count kb = sla2_blocks_kept(N/64, keep_frac) key blocks per query
 *              block; keep_frac must lie in (0, 1].
 *   Pointers   Every array pointer is caller-owned DEVICE memory, 16-byte aligned
 *              (SLA2_ERR_MISALIGNED otherwise). The library allocates no device
 *              memory and keeps no pointer after a call returns; buffers must stay alive
 *              until the stream has executed the work.
 *   Workspace  Caller-provided device scratch of sla2_workspace_bytes(shape, entry,
 *              keep_frac) bytes for the entry point it is passed to (each entry
 *              point asks only for what its kernels use).
 *   Streams    `stream` is a hipStream_t (NULL = the default stream). Every kernel
 *              of a call is enqueued on it, in order; no call creates streams or
 *              events, synchronises or copies device -> host (except
 *              sla2_workspace_status, which says so).
 *   Errors     Arguments are validated on the host before anything is enqueued;
 *              on error nothing is written. A failed launch returns SLA2_ERR_HIP.
 *              No C++ exception crosses this interface. Calls are re-entrant and
 *              hold no state between calls (the library caches only the device's
 *              architecture check); concurrent calls must use distinct workspaces.
 *              The attention kernel synchronises its wavefronts with bounded
 *              waits; if one ever gives up, it sets an error word in the workspace
 *              (read by sla2_workspace_status) instead of hanging.
 *   Debug      Environment SLA2_DEBUG_SYNC=1 synchronises and checks after every
 *              kernel, including the workspace's error word (slow; for debugging).
 */
#ifndef SLA2_H
#define SLA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The status, dtype, quantisation and entry types are plain 32-bit integers with named values
 * (not C enum types), so that any value a caller passes is well defined on the C++ side: an
 * out-of-range value is rejected with SLA2_ERR_BAD_DTYPE / SLA2_ERR_BAD_ARGUMENT, or gives 0 from
 * sla2_workspace_bytes and "unknown status" from sla2_status_string. */
typedef int32_t sla2_status;
enum {
    SLA2_OK = 0,
    SLA2_ERR_NULL_POINTER = 1,
    SLA2_ERR_BAD_SHAPE = 2,
    SLA2_ERR_BAD_DTYPE = 3,
    SLA2_ERR_MISALIGNED = 4,
    SLA2_ERR_BAD_ARGUMENT = 5,
    SLA2_ERR_WORKSPACE_TOO_SMALL = 6,
    SLA2_ERR_UNSUPPORTED_DEVICE = 7,
    SLA2_ERR_HIP = 8,
    SLA2_ERR_WAIT_TIMEOUT = 9
};

/* element type of Q, K, V */
typedef int32_t sla2_dtype;
enum { SLA2_FP32 = 0, SLA2_BF16 = 1 };

/* operand precision of the sparse branch (step 2 of the summary page's computation
 * flow quantises Q, K and P, V before the products; Eq. 9 and Eq. 11 of §4 of the
 * second page hold exactly only without quantisation):
 *   SLA2_QUANT_NONE    the unquantised branch: S = Q K_s^T / sqrt(d) and P V with
 *                      fp32 operands (fp32 MFMA, fp32 softmax); the reference form, not
 *                      the fast one. The code and scale taps are not written.
 *   SLA2_QUANT_I8_FP8  the low-bit branch: INT8 Q, K per block, OCP E4M3 P, V. */
typedef int32_t sla2_quant;
enum { SLA2_QUANT_NONE = 0, SLA2_QUANT_I8_FP8 = 1 };

/* the entry point a workspace is sized for (sla2_workspace_bytes) */
typedef int32_t sla2_entry;
enum {
    SLA2_ENTRY_ROUTER = 0,
    SLA2_ENTRY_ROUTER_SOFT = 1,
    SLA2_ENTRY_LINEAR_PRECOMPUTE = 2,
    SLA2_ENTRY_FORWARD = 3,
    SLA2_ENTRY_FORWARD_WITH_MASK = 4,
    SLA2_ENTRY_FORWARD_SLA1 = 5,
    SLA2_ENTRY_BACKWARD = 6,
    SLA2_ENTRY_ROUTER_GRAD = 7
};

typedef struct {
    int32_t B, H, N, d;
    sla2_dtype dtype;
} sla2_shape;

/* Optional debug outputs of sla2_forward / sla2_forward_with_mask; pass NULL for
 * the struct or for any member to skip it. Layouts in standard row order. */
typedef struct {
    float   *O_s;       /* [B,H,N,d] sparse-branch output (0 for a query block with no kept block) */
    float   *O_l;       /* [B,H,N,d] linear-branch output (0 for a query block with no dropped block) */
    int8_t  *q_codes;   /* [B,H,N,d] INT8 codes of Q, one scale per 128-row block */
    int8_t  *k_codes;   /* [B,H,N,d] INT8 codes of K_s = K - colmean(K), one scale per 64-row block */
    uint8_t *v_codes;   /* [B,H,N,d] E4M3 codes of V, one scale per 64-row block */
    float   *s_q;       /* [B,H,N/128] */
    float   *s_k;       /* [B,H,N/64] */
    float   *s_v;       /* [B,H,N/64] */
    float   *k_colmean; /* [B,H,d] colmean(K) rounded to fp32 */
    /* NULL, or SLA2_MAX_STAGES + 1 caller-created hipEvent_t handles: element 0 is
     * recorded on the stream before the first kernel and element s + 1 after kernel s,
     * so consecutive pairs time each kernel. Kernel order of sla2_forward: pool
     * (block sums, INT8 Q), colmean, project, score_topk, kv_prep (INT8 K_s, E4M3 V,
     * phi(K_s), z_j, h_j), linear_total, attn (sparse branch, linear branch and
     * combine); of sla2_forward_with_mask: pool, colmean, mask_to_list, kv_prep,
     * linear_total, attn. Unused trailing events are not recorded. */
    void   **stage_events;
} sla2_taps;

#define SLA2_MAX_STAGES 9

/* Kept key blocks per query block: max(1, floor(keep_frac * n_key_blocks + 1e-9)),
 * capped at n_key_blocks (the "top k%" of step 1). Host only; returns -1 when
 * n_key_blocks < 1 or keep_frac is not in (0, 1]. */
int32_t sla2_blocks_kept(int32_t n_key_blocks, float keep_frac);

/* Device workspace, in bytes, that `entry` needs for this shape. keep_frac matters
 * only for SLA2_ENTRY_FORWARD, SLA2_ENTRY_FORWARD_SLA1 and SLA2_ENTRY_ROUTER_GRAD (their block lists hold
 * kb = sla2_blocks_kept(N/64, keep_frac) entries per row); other entries ignore it.
 * Returns 0 for an invalid shape, entry or keep_frac. A workspace sized for one entry
 * serves any call of that entry with the same shape and a kept count no larger. */
size_t sla2_workspace_bytes(const sla2_shape *shape, sla2_entry entry, float keep_frac);

/* Error word of a workspace after the work enqueued on `stream` so far: SYNCHRONISES
 * `stream` and copies 4 bytes device -> host. SLA2_ERR_WAIT_TIMEOUT if a bounded wait
 * inside the attention kernel of the last forward call that used this workspace gave up
 * (its output is then unreliable), SLA2_OK otherwise. Meaningful only after a call of
 * sla2_forward, sla2_forward_with_mask or sla2_forward_sla1 on this workspace (each clears
 * the word before its attention kernel); the word is the workspace's first 4 bytes.
 * SLA2_ERR_NULL_POINTER, SLA2_ERR_MISALIGNED or SLA2_ERR_WORKSPACE_TOO_SMALL (< 256 bytes)
 * for a bad workspace, SLA2_ERR_HIP if the copy fails. */
sla2_status sla2_workspace_status(const void *workspace, size_t workspace_bytes, void *stream);

/* Static English text for a status code. */
const char *sla2_status_string(sla2_status status);

/* Step 1 only (the learned router).
 *   mask   [B,H,N/128,N/64] uint8 M_c, or NULL
 *   blocks [B,H,N/128,kb] int32 kept key-block indices, ascending (required)
 *   scores [B,H,N/128,N/64] fp32 P_c, or NULL
 * The projections and logits are fp32 (MFMA; fp64 block sums and colmean); ranking is by
 * the fp32 logit, exact, equal logits to the lower block index. */
sla2_status sla2_router(const sla2_shape *shape, const void *Q, const void *K,
                        const float *proj_q, const float *proj_k, float keep_frac,
                        uint8_t *mask, int32_t *blocks, float *scores,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Step 1 with SoftTop-k, the training-time router ("SLA2: Sparse-Linear Attention v2 for
 * Diffusion Transformers", §4 Eq. 17 and its six-checks item 3; summary page, step 1):
 *   soft_mask [B,H,N/128,N/64] fp32 sigma(P_c / tau + lambda_i) (required)
 *   lambda    [B,H,N/128] fp32 lambda_i (or NULL)
 *   stage_events  NULL, or 5 caller-created hipEvent_t handles recorded on the stream
 *             before the first kernel and after each of pool, colmean, project and
 *             score_soft (the SoftTop-k pass), so consecutive pairs time each kernel
 * P_c as in sla2_router (fp32 logits, fp64 softmax). lambda_i makes every row sum to kb =
 * sla2_blocks_kept(N/64, keep_frac), so the mask tends to the hard Top-k mask as tau -> 0;
 * it is found in fp32 by 16 safeguarded Newton steps inside the bracket [L - max x,
 * L - min x], x = P_c / tau, L = log(kb / (N/64 - kb)) (the pages' binary search, with
 * Newton steps where they stay in the bracket). kb = N/64 gives a mask of ones and
 * lambda = +inf. Deterministic (fixed-order reductions). tau must be
 * finite and > 0 with 1/tau finite (SLA2_ERR_BAD_ARGUMENT otherwise). */
sla2_status sla2_router_soft(const sla2_shape *shape, const void *Q, const void *K,
                             const float *proj_q, const float *proj_k, float keep_frac,
                             float tau, float *soft_mask, float *lambda, void **stage_events,
                             void *workspace, size_t workspace_bytes, void *stream);

/* The linear branch's per-key-block precompute (step 3; §7 note 2) on the smoothed
 * K_s = K - colmean(K):
 *   k_colmean [B,H,d] fp32 (required)
 *   h         [B,H,N/64,d,d] fp32 h_j = phi(K_s,j)^T V_j (or NULL)
 *   z         [B,H,N/64,d] fp32 column sums of phi(K_s,j) (or NULL)
 *   h_total   [B,H,d,d] fp32 sum over j of h_j (required)
 *   z_total   [B,H,d] fp32 sum over j of z_j (required)
 * phi(K_s) is rounded to bf16 for the matrix product; sums are fp32. */
sla2_status sla2_linear_precompute(const sla2_shape *shape, const void *K, const void *V,
                                   float *k_colmean, float *h, float *z,
                                   float *h_total, float *z_total,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* Sets up the current device for the library: checks that it is a gfx950, raises the
 * scoring kernel's LDS limit, and takes the device address of the static scratch of
 * sla2_router_noalloc. The first call of any entry point on a device does this by itself;
 * call it once per device beforehand where that first call must not load code or take
 * addresses (graph capture, allocation-free loops). SLA2_ERR_UNSUPPORTED_DEVICE on another
 * GPU, SLA2_ERR_HIP if a HIP call fails. */
sla2_status sla2_init_device(void);

/* Bytes of the static device scratch of sla2_router_noalloc (one copy per GPU, held until
 * the process ends): enough for the router at B*H = 12, N = 32768 (14 MB). */
#define SLA2_NOALLOC_SCRATCH_BYTES (32u << 20)

/* sla2_router for callers that cannot allocate device memory or pass a workspace (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the same kernels
 * and results as sla2_router, with the workspace in a file-scope device array of
 * SLA2_NOALLOC_SCRATCH_BYTES per GPU instead of caller memory. No allocation of any kind, no
 * copy. Shapes whose router workspace (sla2_workspace_bytes(shape, SLA2_ENTRY_ROUTER, ...))
 * exceeds the scratch return SLA2_ERR_WORKSPACE_TOO_SMALL before anything is enqueued; other
 * arguments and errors as sla2_router. Every call on one GPU shares that GPU's scratch, which
 * keeps the last call's contents (each call overwrites every region it reads before reading
 * it): calls that overlap on one GPU (different streams or threads, or an earlier call's work
 * still pending on another stream) race. Call sla2_init_device first where even the device's
 * one-time set-up must happen beforehand. */
sla2_status sla2_router_noalloc(const sla2_shape *shape, const void *Q, const void *K,
                                const float *proj_q, const float *proj_k, float keep_frac,
                                uint8_t *mask, int32_t *blocks, float *scores, void *stream);

/* The whole forward: router, sparse branch, linear branch and combine.
 *   O [B,H,N,d] fp32 (required); taps optional (NULL). */
sla2_status sla2_forward(const sla2_shape *shape, const void *Q, const void *K, const void *V,
                         const float *proj_q, const float *proj_k, const float *alpha,
                         float keep_frac, sla2_quant quant, float *O, const sla2_taps *taps,
                         void *workspace, size_t workspace_bytes, void *stream);

/* The earlier SLA formulation, as a comparison workload ("SLA2: Sparse-Linear Attention
 * v2 for Diffusion Transformers", §2 Q2 before/after table): the heuristic router
 * softmax(Qbar Kbar^T / sqrt(d)) -> Top-k (the learnable router with proj = I), the same
 * sparse and linear branches, and the mix O = O_s + O_l Wo without alpha.
 *   proj_o [H,d,d] fp32 Wo, applied as x @ Wo (required)
 *   O      [B,H,N,d] fp32 output (required)
 *   O_l    [B,H,N,d] fp32 the linear branch output, written on the way (required)
 *   stage_events  NULL, or 10 caller-created hipEvent_t handles recorded on the stream
 *          before the first kernel and after each of pool, colmean, project (identity),
 *          score_topk, fill (alpha = 1), kv_prep, linear_total, attn and sla1_mix (O += O_l Wo)
 * O_l Wo is an fp32 matrix product (fp32 MFMA). Same validation as sla2_forward. */
sla2_status sla2_forward_sla1(const sla2_shape *shape, const void *Q, const void *K,
                              const void *V, const float *proj_o, float keep_frac,
                              sla2_quant quant, float *O, float *O_l, void **stage_events,
                              void *workspace, size_t workspace_bytes, void *stream);

/* The forward with a caller-supplied block mask instead of the router. Any 0/1
 * pattern is accepted (any byte != 0 counts as 1): a row with no kept block gets
 * O_s = 0, a row with no dropped block gets O_l = 0. */
sla2_status sla2_forward_with_mask(const sla2_shape *shape, const void *Q, const void *K,
                                   const void *V, const uint8_t *mask, const float *alpha,
                                   sla2_quant quant, float *O, const sla2_taps *taps,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* The backward pass ("SLA2: Sparse-Linear Attention v2 for Diffusion Transformers": §3 table
 * and §4 six checks item 4, low-bit forward with a 16-bit backward, the straight-through
 * estimator; §7 note 3, the gradient derived by hand with the linear branch's dH_i, dZ_i
 * formed first). It returns the gradients of sum(dO * O) for the UNQUANTISED forward
 *   O = alpha O_s + (1 - alpha) O_l,  O_s = softmax over the kept keys of Q K_s^T / sqrt(d) V,
 *   O_l = phi(Q) H_i / (phi(Q) Z_i) over the dropped key blocks,  K_s = K - colmean(K),
 * with the block mask held fixed (the hard Top-k router has no gradient).
 *   mask   [B,H,N/128,N/64] uint8, the forward's block mask (any byte != 0 counts as 1)
 *   alpha  [H,N/128] fp32, as in the forward
 *   dO     [B,H,N,d] fp32, the gradient of the loss with respect to O
 *   dQ, dK, dV  [B,H,N,d] fp32 outputs (overwritten)
 *   dalpha [B,H,N/128] fp32 output: per batch and head; sum over B for alpha's gradient
 *   stage_events  NULL, or 15 caller-created hipEvent_t handles recorded on the stream before
 *          the first kernel and after each of pool (K sums), colmean, kv_prep, linear_total,
 *          mask_to_list, key_lists (mask transposed: the query blocks keeping each key block),
 *          key_plan (long key lists cut into work items of at most C query blocks),
 *          bwd_prep (bf16 copies of Q, K_s, V and alpha dO), bwd_lin_q (linear branch per
 *          query block),
 *          dh_total, bwd_q (sparse branch per query block: dQ, log-sum-exp, D),
 *          bwd_kv_extra (work items past the first of each key list: partial sums),
 *          bwd_kv (per key block: first work item, the partials, the linear part: dK_s, dV)
 *          and dk_center (dK = dK_s - colmean(dK_s))
 * Precision: Q, K_s, V, P, dS, dO_s = alpha dO, phi(Q), phi(K_s), H_i, dH_i and dh_j enter
 * the matrix products as bf16 (fp32 accumulation); softmax statistics, row sums and the
 * outputs are fp32. A query block with no kept block gets no sparse gradient and one with no
 * dropped block no linear gradient (their branch output is 0 in the forward). Deterministic. */
sla2_status sla2_backward(const sla2_shape *shape, const void *Q, const void *K, const void *V,
                          const uint8_t *mask, const float *alpha, const float *dO, float *dQ,
                          float *dK, float *dV, float *dalpha, void **stage_events,
                          void *workspace, size_t workspace_bytes, void *stream);

/* Stage-1 alpha fit, the alpha part ("SLA2: Sparse-Linear Attention v2 for Diffusion
 * Transformers", §4 six checks item 5: alpha is fitted with an MSE loss against full attention;
 * §3 mixing, §4 check 2: alpha in [0, 1]). With the router (the block mask) fixed the output is
 * affine in alpha, so the MSE of each (head, query block) over its 128 rows, d columns and all B
 * batches is minimised by
 *   alpha[h][i] = clip(<O_full - O_l, O_s - O_l> / |O_s - O_l|^2, 0, 1)   (1 where O_s = O_l).
 *   O_full [B,H,N,d] fp32, the full-attention target (e.g. sla2_forward at keep_frac = 1)
 *   O_s, O_l [B,H,N,d] fp32, the branch outputs under the mask (sla2_taps.O_s, O_l)
 *   alpha  [H,N/128] fp32 output
 * shape->dtype is not used (all four arrays are fp32). fp64 accumulation, fixed order
 * (deterministic). No workspace. The router part of stage 1 is sla2_router_grad. */
sla2_status sla2_fit_alpha(const sla2_shape *shape, const float *O_full, const float *O_s,
                           const float *O_l, float *alpha, void *stream);

/* Stage-1 router gradient: the router part of the first training stage ("SLA2: Sparse-Linear
 * Attention with Learnable Routing and QAT", summary page, novelty paragraph: router and alpha
 * are first fitted against full attention, and SoftTop-k replaces Top-k in training so that
 * the router gets gradients; "SLA2: Sparse-Linear Attention v2 for Diffusion Transformers",
 * §4 Eq. 17 (SoftTop-k), §5 training table, stage 1). For
 *   L = sum over b, h, rows, columns of (O - O_full)^2
 * it returns L per head and dL/dproj_q, dL/dproj_k under these readings (the pages leave
 * them open): the forward is the UNQUANTISED forward with the hard Top-k mask (stage 1 comes
 * before the quantisation-aware stage); the mask enters through the relaxation that weights
 * key block j's exponentials in the sparse branch by M_ij and its h_j, z_j in the linear
 * branch by 1 - M_ij (the forward itself at a 0/1 mask); dL/dM at the hard mask is passed
 * straight through to the SoftTop-k mask sigma(P_c / tau + lambda_i) (kept count kb, lambda_i
 * held to the row-sum constraint), then through P_c = softmax((Qbar Wq)(Kbar_s Wk)^T / sqrt(d)).
 *   O_full  [B,H,N,d] fp32, the full-attention target
 *   keep_frac, tau  as in sla2_router_soft (kb = sla2_blocks_kept(N/64, keep_frac))
 *   dproj_q, dproj_k  [H,d,d] fp32 outputs (summed over the batch; overwritten)
 *   loss    [H] fp64 output (summed over the batch)
 *   mask_grad  NULL, or [B,H,N/128,N/64] fp32 output: dL/dM_ij at the hard mask
 * Cost: a dense pass over every (query block, key block) pair, three 128 x 64 x 128 products
 * each (S, delta V^T and phi(Q) phi(K_s)^T) with f16 operands (delta = 2 (O - O_full) scaled by
 * a power of two per row) and fp32 accumulation; the router part in fp32 with fp64 sums for
 * dproj_q, dproj_k and the loss. Deterministic. Workspace: SLA2_ENTRY_ROUTER_GRAD. */
sla2_status sla2_router_grad(const sla2_shape *shape, const void *Q, const void *K, const void *V,
                             const float *proj_q, const float *proj_k, const float *alpha,
                             float keep_frac, float tau, const float *O_full, float *dproj_q,
                             float *dproj_k, double *loss, float *mask_grad, void *workspace,
                             size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SLA2_H */
