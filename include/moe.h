/*
 * moe.h -- C ABI of libmoe, the MI355X (gfx950) MoE expert block.
 *
 * The block, as the pages state the problem: a flat batch of token hidden
 * states goes through an fp32 router and a per-token top-k; the selected
 * (token, expert) rows are sorted by expert; each expert runs its SwiGLU FFN as
 * one grouped matmul over its contiguous rows; the rows come back to their
 * token in the same order, weighted by the top-k probabilities, and are summed
 * ("Halo's 2.8x over TRL is not a kernel, and its own benchmark proves it",
 * section "Where the gap actually is", EP token-routing figure and the EP
 * forward path described under it).  The backward computes the matching
 * activation, expert-weight and router gradients, with the routing adjoint
 * written as gathers, free of atomic adds ("Halo: Frontier-Lab Training for
 * Everyone", section "Some of the hard problems along the way").
 *
 * Conventions for every entry point:
 *  - Status: returns MOE_OK (0) or a negative MOE_ERR_*.  Arguments are
 *    validated on the host before anything is launched; an invalid call
 *    launches nothing and writes nothing.  moe_last_error() gives a message
 *    for the calling thread's last failure.
 *  - Memory: every tensor argument is a caller-owned DEVICE pointer (current
 *    HIP device), row-major and contiguous, 16-byte aligned.  The library
 *    never allocates device memory in these calls; scratch comes from the
 *    caller through a workspace pointer sized by the matching *_workspace_size
 *    query.
 *  - Streams: `stream` is a hipStream_t (NULL = the null stream).  Every call
 *    is asynchronous on that stream and makes no device-to-host copy; per
 *    expert counts and offsets stay on the device.
 *  - dtype: MOE_BF16 or MOE_F32 selects the storage type of activations and
 *    expert weights (x, w_r, w_gu, w_down, x_perm, gu, h, y_perm, y, dy, ...).
 *    Routing tensors are always fp32 / int32; weight and router gradients are
 *    always fp32.  MOE_F32 covers the forward path and the copy-type backward
 *    steps; moe_grouped_ffn_bwd and moe_router_logits_bwd need MOE_BF16.
 *  - Shapes: T >= 0 tokens, d = d_model, f = d_ff, E experts, k = top-k;
 *    1 <= k <= E <= 1024, k <= 32; d and f positive multiples of 8;
 *    R = T*k routed rows, R < 2^31.  Element offsets are computed in 64 bits.
 *  - Determinism: no floating-point atomics anywhere; repeated calls on the
 *    same inputs give bitwise identical results.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK               0
#define MOE_ERR_INVALID_ARG (-1)   /* null pointer, bad size, misalignment */
#define MOE_ERR_UNSUPPORTED (-2)   /* dtype / shape outside the supported set */
#define MOE_ERR_WORKSPACE   (-3)   /* workspace missing or too small */
#define MOE_ERR_HIP         (-4)   /* HIP launch or runtime error */

#define MOE_F32  0
#define MOE_BF16 1

/* Library version (major*10000 + minor*100 + patch). */
int moe_version(void);
/* Static description of a status code. */
const char *moe_strerror(int status);
/* Message for the calling thread's last failed call ("" if none). */
const char *moe_last_error(void);

/* ---------------------------------------------------------------- router */

/*
 * Router logits in fp32.  The pages fix the precision ("fp32 router logits" in
 * the EP forward path, section "Where the gap actually is"; `fp32_router:
 * true` in the recipe of section "The small-hardware end").  The summation
 * order is fixed as part of the definition so that top-k decisions are
 * reproducible bit for bit:
 *   logits[t,e] = ((fma chain over c = 0..d-1 of x[t,c]*w_r[e,c], from +0)
 *                  + bias[e]) + logit_add[t,e]
 * x: [T,d] (dtype), w_r: [E,d] (dtype), bias: [E] fp32 or NULL,
 * logit_add: [T,E] fp32 or NULL (additive noise), logits: [T,E] fp32 (out).
 */
int moe_router_logits(const void *x, const void *w_r, const float *bias,
                      const float *logit_add, int dtype, int64_t T, int d, int E,
                      float *logits, void *stream);

/*
 * Per-token top-k and the combine weights (the "per-token top-k router" and
 * "weighted by the top-k probabilities" of the EP token-routing figure).
 * topk_idx[t,0..k-1]: the k largest logits of token t, by value descending;
 * equal values go to the lower expert id (-0 equals +0); a NaN ranks below
 * every number (NaNs among themselves by lower id) and +-inf order as numbers,
 * so the selection is always defined.  topk_w[t,j] = softmax over the k
 * selected logits (NaN for every j when the selection holds a NaN or its
 * largest logit is +inf; finite logits are the intended use).
 * logits: [T,E] fp32; topk_idx: [T,k] int32 (out); topk_w: [T,k] fp32 (out).
 */
int moe_route(const float *logits, int64_t T, int E, int k,
              int32_t *topk_idx, float *topk_w, void *stream);

/* ---------------------------------------------------------------- permute */

size_t moe_permute_workspace_size(int64_t T, int E, int k);

/*
 * Sorts the selected (token, expert) slots by expert -- the single-GPU core of
 * the EP dispatch, which hands each expert its tokens "sorted by expert" (EP
 * token-routing figure).  Slot s = t*k + j.  Rows are expert-major; inside an
 * expert, slots keep ascending order.  Outputs:
 *   counts[E], offsets[E+1] (offsets[0]=0, offsets[E]=R), slot_to_row[R],
 *   row_to_slot[R] (int32);
 *   x_perm[r] = x[row_to_slot[r] / k]   (exact copy; x may be NULL to skip),
 *   w_perm[r] = topk_w[row_to_slot[r]]  (topk_w and w_perm may be NULL).
 * topk_idx entries must lie in [0,E) and a token's k entries must be distinct.
 * ws: device workspace of at least moe_permute_workspace_size(T,E,k) bytes.
 */
int moe_permute(const void *x, const int32_t *topk_idx, const float *topk_w, int dtype,
                int64_t T, int d, int E, int k,
                int32_t *counts, int32_t *offsets, int32_t *slot_to_row, int32_t *row_to_slot,
                void *x_perm, float *w_perm, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- experts */

size_t moe_grouped_ffn_workspace_size(int64_t R, int E, int d, int f, int dtype);

/*
 * Grouped SwiGLU expert FFN over rows sorted by expert ("grouped GEMM and
 * fused SwiGLU", "Halo: Frontier-Lab Training for Everyone", section "Novel
 * model integration example"; experts stored as single 3-D weight tensors,
 * section "One trainer architecture, one parallelism stack").  For each
 * expert e and each of its rows r in [offsets[e], offsets[e+1]):
 *   [g | u] = x_perm[r] . w_gu[e]^T        (gate rows 0..f-1, up rows f..2f-1)
 *   gu[r]   = store([g | u])                (store = dtype rounding)
 *   h[r]    = store(silu(gu_g) * gu_u),  silu(v) = v / (1 + exp(-v))
 *   y_perm[r] = store(row_scale[r] * (h[r] . w_down[e]^T))   (row_scale NULL = 1)
 * fp32 accumulation.  Experts with no rows are skipped.
 * x_perm: [R,d]; w_gu: [E,2f,d]; w_down: [E,d,f]; row_scale: [R] fp32 or NULL;
 * gu: [R,2f] (out, or NULL if not needed for a backward); h: [R,f] (out);
 * y_perm: [R,d] (out).  offsets: [E+1] int32 on the device, offsets[E] = R.
 */
int moe_grouped_ffn_fwd(const void *x_perm, const int32_t *offsets, int E, int64_t R,
                        int d, int f, const void *w_gu, const void *w_down,
                        const float *row_scale, int dtype, void *gu, void *h, void *y_perm,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * moe_grouped_ffn_fwd without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results (bit for bit), errors and
 * conventions as moe_grouped_ffn_fwd minus ws / ws_bytes.  Its scratch -- the
 * forward's two tile-start tables with their tile counters -- lives in a
 * static device array of 8704 bytes (enough for E <= 1024; a larger need
 * returns MOE_ERR_UNSUPPORTED), one copy per device, held until the process
 * ends; its address is taken once per device on that device's first call.
 * The call allocates nothing and clears what it needs itself, in stream
 * order.  Every call on one device shares that array: calls that may run
 * concurrently on one device (different streams, or threads) race and must
 * be serialised by the caller.
 */
int moe_grouped_ffn_fwd_noalloc(const void *x_perm, const int32_t *offsets, int E, int64_t R,
                                int d, int f, const void *w_gu, const void *w_down,
                                const float *row_scale, int dtype, void *gu, void *h,
                                void *y_perm, void *stream);

/*
 * Backward of moe_grouped_ffn_fwd (expert weights receive gradients: the
 * "expert gradient all-to-all" that LoRA skips, section "One trainer
 * architecture, one parallelism stack", is the exchange of these).  Per row r
 * of expert e, with w = row_scale[r] (1 if NULL):
 *   Gd          = dy_perm[r] . w_down[e]                      (fp32)
 *   d_row_scale[r] = sum_c h[r,c] * Gd[c]                      (fp32)
 *   dH = w*Gd;  s = sigmoid(g);  dg = dH*u*s*(1 + g*(1-s));  du = dH*g*s
 *   dgu[r]      = store([dg | du])
 *   dx_perm[r]  = store(dgu[r] . w_gu[e])
 *   dw_down[e]  = sum_r store(w*dy_perm[r])^T (x) h[r]          (fp32, [E,d,f])
 *   dw_gu[e]    = sum_r dgu[r]^T (x) x_perm[r]                  (fp32, [E,2f,d])
 * (g, u = the stored gu; experts with no rows get exactly zero dw.)
 * Inputs: x_perm [R,d], gu [R,2f], h [R,f] (saved by the forward), dy_perm [R,d].
 * Outputs: dgu [R,2f], dx_perm [R,d], dw_gu, dw_down, d_row_scale [R] (or NULL).
 * dtype must be MOE_BF16.
 */
int moe_grouped_ffn_bwd(const void *x_perm, const void *gu, const void *h,
                        const int32_t *offsets, int E, int64_t R, int d, int f,
                        const void *w_gu, const void *w_down, const float *row_scale,
                        const void *dy_perm, int dtype, void *dgu, void *dx_perm,
                        float *dw_gu, float *dw_down, float *d_row_scale,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * The grouped FFN with the row permutation folded into the GEMM operand
 * loads: the tokens go to their experts as one grouped matmul over the rows
 * sorted by expert ("Halo's 2.8x over TRL is not a kernel, and its own
 * benchmark proves it", section "Where the gap actually is"), and the sorted
 * rows are read from the token-major tensors where the GEMMs load them, so
 * x_perm and dy_perm are never stored.  Row r of the expert-sorted order is
 * token row_to_slot[r] / k (row_to_slot from moe_permute, which then needs no
 * x / x_perm).
 *
 * moe_grouped_ffn_fwd_gather: the results of moe_grouped_ffn_fwd with
 *   x_perm[r] = x[row_to_slot[r] / k]; x: [T,d] bf16, R = T*k.
 * moe_grouped_ffn_bwd_gather: the results of moe_grouped_ffn_bwd with that
 *   x_perm and dy_perm[r] = dy[row_to_slot[r] / k]; dy: [T,d] bf16;
 *   slot_to_row: [R], the inverse of row_to_slot (moe_permute writes both;
 *   S = w * dY_perm is formed from dY in token order through it).  x_perm:
 *   [R,d] or NULL; when given (the forward's permuted rows), the dW_gu GEMM
 *   reads it instead of gathering X, and x may be NULL.
 * Every other argument, output and the workspace
 * (moe_grouped_ffn_workspace_size(T*k, E, d, f, MOE_BF16)) are those of the
 * plain calls; bf16 only.  Limits (else MOE_ERR_UNSUPPORTED): k <= 32,
 * T*d < 2^30, T*k*k < 2^32.  row_to_slot must hold a permutation of
 * 0..T*k-1 and slot_to_row its inverse (as moe_permute writes them); other
 * values are not checked and index outside x, dy and the outputs.
 */
int moe_grouped_ffn_fwd_gather(const void *x, int64_t T, const int32_t *row_to_slot, int k,
                               const int32_t *offsets, int E, int d, int f,
                               const void *w_gu, const void *w_down, const float *row_scale,
                               void *gu, void *h, void *y_perm,
                               void *ws, size_t ws_bytes, void *stream);
int moe_grouped_ffn_bwd_gather(const void *x, const void *x_perm, const void *dy, int64_t T,
                               const int32_t *row_to_slot, const int32_t *slot_to_row, int k,
                               const void *gu, const void *h,
                               const int32_t *offsets, int E, int d, int f,
                               const void *w_gu, const void *w_down, const float *row_scale,
                               void *dgu, void *dx_perm, float *dw_gu, float *dw_down,
                               float *d_row_scale, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- combine */

/*
 * Returns each row to its token and sums ("the same rows in the same order",
 * EP token-routing figure; the weights were applied by the down projection):
 *   y[t] = store(sum over j = 0..k-1, ascending, of y_perm[slot_to_row[t*k+j]])
 * with an fp32 running sum.  y_perm: [R,d]; slot_to_row: [R]; y: [T,d] (out).
 */
int moe_combine(const void *y_perm, const int32_t *slot_to_row, int dtype,
                int64_t T, int d, int k, void *y, void *stream);

/*
 * Adjoint of moe_combine: a copy of each token's gradient to its k rows,
 *   dy_perm[slot_to_row[t*k+j]] = dy[t].
 * The combine returns each expert output row to its token ("Halo's 2.8x over
 * TRL is not a kernel, and its own benchmark proves it", section "Where the
 * gap actually is", EP token-routing figure); its adjoint is written as this
 * copy through the forward's own map, a gather with no atomic adds ("Halo:
 * Frontier-Lab Training for Everyone", section "Some of the hard problems
 * along the way", on the atomic-free routing backward).  dy: [T,d] (dtype);
 * slot_to_row: [T*k] int32 from moe_permute; dy_perm: [T*k,d] (out, every row
 * written once).  Errors as moe_combine.
 */
int moe_combine_bwd(const void *dy, const int32_t *slot_to_row, int dtype,
                    int64_t T, int d, int k, void *dy_perm, void *stream);

/*
 * Adjoint of the row permutation, as a gather (no atomic adds; "Halo:
 * Frontier-Lab Training for Everyone", section "Some of the hard problems
 * along the way"):
 *   dx[t] = store(sum over j ascending of dx_perm[slot_to_row[t*k+j]] + dx_add[t])
 * with an fp32 running sum; dx_add: [T,d] fp32 or NULL (the router's share).
 */
int moe_permute_bwd(const void *dx_perm, const int32_t *slot_to_row, const float *dx_add,
                    int dtype, int64_t T, int d, int k, void *dx, void *stream);

/* ---------------------------------------------------------------- grouped LoRA */

/*
 * LoRA on the fused expert weights with the experts frozen ("Halo:
 * Frontier-Lab Training for Everyone", section "One trainer architecture, one
 * parallelism stack": a grouped LoRA that adapts the 3-D expert tensors
 * directly, so the frozen experts need no gradients).  Per expert e, rank r,
 * scale s: W_gu[e] + s B_gu[e] A_gu[e] and W_down[e] + s B_dn[e] A_dn[e] with
 * a_gu [E,r,d], b_gu [E,2f,r] (gate rows then up rows), a_dn [E,r,f],
 * b_dn [E,d,r], all bf16, caller-owned device memory.  r is a multiple of 16,
 * 16 <= r <= 64; dtype must be MOE_BF16; other shapes, errors and conventions
 * as moe_grouped_ffn_fwd / _bwd.  Stored intermediates (bf16, [R,r]):
 *   z_gu = store(s X_perm A_gu^T),  z_dn = store(s H A_dn^T)      (forward outputs)
 * forward:  GU = store(X_perm W_gu^T + z_gu B_gu^T) (one fp32 accumulation:
 *           the rank-r product is one more K stage of the grouped GEMM),
 *           H = store(silu(g) u),  Y_perm = store(w (H W_down^T + z_dn B_dn^T)).
 * backward: u_dn = store(s dY_perm B_dn);  Gd = dY_perm W_down + u_dn A_dn
 *           feeds the dSwiGLU epilogue and d_row_scale as in moe_grouped_ffn_bwd;
 *           u_gu = store(s dGU B_gu);  dX_perm = store(dGU W_gu + u_gu A_gu);
 *           dB_gu = dGU^T z_gu [E,2f,r], dA_gu = u_gu^T X_perm [E,r,d],
 *           dB_dn = S^T z_dn [E,d,r] (S = store(w dY_perm)),
 *           dA_dn = store(w u_dn)^T H [E,r,f]; fp32, fully written (zeros for
 *           empty experts).  No expert weight gradients are formed.
 * ws: moe_grouped_ffn_lora_workspace_size(R,E,d,f,r) bytes for either call.
 */
size_t moe_grouped_ffn_lora_workspace_size(int64_t R, int E, int d, int f, int r);
int moe_grouped_ffn_fwd_lora(const void *x_perm, const int32_t *offsets, int E, int64_t R, int d,
                             int f, const void *w_gu, const void *w_down, const float *row_scale,
                             const void *a_gu, const void *b_gu, const void *a_dn,
                             const void *b_dn, int r, float scale, int dtype, void *z_gu,
                             void *z_dn, void *gu, void *h, void *y_perm, void *ws,
                             size_t ws_bytes, void *stream);
int moe_grouped_ffn_bwd_lora(const void *x_perm, const void *gu, const void *h,
                             const int32_t *offsets, int E, int64_t R, int d, int f,
                             const void *w_gu, const void *w_down, const float *row_scale,
                             const void *dy_perm, const void *a_gu, const void *b_gu,
                             const void *a_dn, const void *b_dn, int r, float scale,
                             const void *z_gu, const void *z_dn, int dtype, void *dgu,
                             void *dx_perm, float *d_row_scale, float *da_gu, float *db_gu,
                             float *da_dn, float *db_dn, void *ws, size_t ws_bytes,
                             void *stream);

/*
 * Where moe_grouped_ffn_bwd_lora leaves its stored rank-r rows in the
 * workspace `ws` it was given (same R, E, d, f, r): u_dn = store(s dY_perm
 * B_dn), uw_dn = store(w u_dn) (written only when row_scale was given) and
 * u_gu = store(s dGU B_gu), each [R,r] bf16 row-major.  The values are those
 * of the last backward call on that workspace, in stream order.  For
 * inspection and tests; the pointers alias ws and are not to be freed.
 * Errors: NULL pointers or r not in {16,32,48,64}: MOE_ERR_INVALID_ARG;
 * ws_bytes below moe_grouped_ffn_lora_workspace_size: MOE_ERR_WORKSPACE.
 */
int moe_grouped_ffn_lora_bwd_saved(const void *ws, size_t ws_bytes, int64_t R, int E, int d,
                                   int f, int r, const void **u_dn, const void **uw_dn,
                                   const void **u_gu);

/*
 * moe_permute_bwd with the router's share of the token gradient formed in the
 * same pass instead of read from memory:
 *   dx[t] = store(sum_{j asc} fp32(dx_perm[slot_to_row[t*k+j]]) + r[t]),
 *   r[t,:] = d_logits[t,:] . w_r  (fp32 fma chain over e ascending from +0,
 *            entries with d_logits == 0 skipped),
 * bit for bit what moe_router_logits_bwd's dx_router followed by
 * moe_permute_bwd gives, without storing dx_router ([T,d] fp32).  Same
 * pass as B6 of the backward; the router term is B8's dX (the router linear
 * map's adjoint, "fp32 router logits" in "Halo's 2.8x over TRL is not a
 * kernel, and its own benchmark proves it", section "Where the gap actually
 * is").  d_logits: [T,E] fp32; w_r: [E,d] (dtype); 1 <= E <= 1024; other
 * arguments and errors as moe_permute_bwd.
 */
int moe_permute_bwd_router(const void *dx_perm, const int32_t *slot_to_row, const float *d_logits,
                           const void *w_r, int dtype, int64_t T, int d, int E, int k, void *dx,
                           void *stream);

/* ---------------------------------------------------------------- router bwd */

/*
 * Adjoint of the softmax over the selected logits.  The routers are trained:
 * they receive the gradient of the loss through the combine weights (the
 * TorchTurbo page, "inclusionAI open-sources TorchTurbo, a SuperNode-native
 * post-training engine", section "Adapter": the routers apply the gradient of
 * the auxiliary loss, so they carry gradients), and the combine weights are
 * the top-k probabilities of the fp32 router ("Halo's 2.8x over TRL is not a
 * kernel, and its own benchmark proves it", section "Where the gap actually
 * is", EP token-routing figure).  With g_j =
 * d_row_scale[slot_to_row[t*k+j]] (the gradient of the loss with respect to
 * topk_w[t,j]):
 *   d_topk_w[t,j] = g_j                         (d_topk_w may be NULL)
 *   d_logits[t,topk_idx[t,j]] = w_j * (g_j - sum_i w_i g_i), 0 elsewhere.
 * All fp32; d_logits: [T,E] (out, fully written).  topk_idx / topk_w: [T,k]
 * from moe_route; d_row_scale: [T*k] from moe_grouped_ffn_bwd; slot_to_row:
 * [T*k] from moe_permute.  Invalid sizes or NULL required pointers:
 * MOE_ERR_INVALID_ARG, nothing launched.
 */
int moe_route_bwd(const int32_t *topk_idx, const float *topk_w, const float *d_row_scale,
                  const int32_t *slot_to_row, int64_t T, int E, int k,
                  float *d_topk_w, float *d_logits, void *stream);

size_t moe_router_logits_bwd_workspace_size(int64_t T, int d, int E);

/*
 * Adjoint of the router linear map that forms the fp32 router logits ("fp32
 * router logits" in the EP forward path, "Halo's 2.8x over TRL is not a
 * kernel, and its own benchmark proves it", section "Where the gap actually
 * is"; the routers are trained, the TorchTurbo page, section "Adapter").  Bias
 * and added noise carry no gradient:
 *   dx_router = d_logits . w_r    ([T,d] fp32, or NULL to skip)
 *   dw_r      = d_logits^T . x    ([E,d] fp32, or NULL to skip)
 * fp32 accumulation in a fixed order: dx_router as an fma chain over e
 * ascending (zero entries skipped), dw_r as per-chunk partials over 256-token
 * chunks summed in chunk order.  x: [T,d], w_r: [E,d] (dtype); d_logits:
 * [T,E] fp32.  dtype must be MOE_BF16.  ws:
 * moe_router_logits_bwd_workspace_size(T,d,E) bytes (MOE_ERR_WORKSPACE if
 * smaller).
 */
int moe_router_logits_bwd(const void *x, const void *w_r, const float *d_logits, int dtype,
                          int64_t T, int d, int E, float *dx_router, float *dw_r,
                          void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- router variants */

/*
 * The pages name three router features without giving formulas: balancing
 * through a bias on expert selection for a model family without a router
 * auxiliary loss ("Halo's 2.8x over TRL is not a kernel, and its own benchmark
 * proves it", section "The small-hardware end": the LFM2 config,
 * `moe_balancing: bias_update`, and the paragraph after it); a router
 * load-balancing auxiliary loss with a per-run coefficient whose gradient the
 * routers apply and whose unscaled and scaled values they report (the
 * TorchTurbo page, "inclusionAI open-sources TorchTurbo, a SuperNode-native
 * post-training engine", section "Adapter", ms-swift DPO); and MoE statistics
 * that ignore the right-padded tail of a batch, the valid prefix being n_valid
 * tokens (same TorchTurbo page, section "Model", sequence-parallel input
 * contract).  The formulas below are the plainest readings.
 */

/*
 * Top-k on the selection score fp32(logits[t,e] + sel_bias[e]) (by value
 * descending, equal scores to the lower expert id, as moe_route); topk_w[t,j]
 * is the softmax over the k selected logits WITHOUT the bias, so the bias only
 * steers which experts are chosen.  sel_bias: [E] fp32, not NULL (moe_route
 * is the unbiased call).  Other arguments and errors as moe_route; moe_route_bwd
 * is the adjoint with respect to the logits (the bias gets no gradient).
 */
int moe_route_biased(const float *logits, const float *sel_bias, int64_t T, int E, int k,
                     int32_t *topk_idx, float *topk_w, void *stream);

size_t moe_expert_load_workspace_size(int64_t T, int E, int k);

/*
 * Expert load over the valid prefix: load[e] = number of slots (t, j) with
 * t < n_valid and topk_idx[t,j] = e (ids outside [0,E) are not counted).
 * 0 <= n_valid <= T, else MOE_ERR_INVALID_ARG.  topk_idx: [T,k] int32;
 * load: [E] int32 (out, fully written; all zero when n_valid = 0).  Exact and
 * deterministic (per-block integer histograms summed in block order).
 * ws: moe_expert_load_workspace_size(T,E,k) bytes.
 */
int moe_expert_load(const int32_t *topk_idx, int64_t T, int64_t n_valid, int E, int k,
                    int32_t *load, void *ws, size_t ws_bytes, void *stream);

/*
 * Selection-bias balancing step, in place:
 *   sel_bias[e] += rate * sign(n_valid*k/E - load[e])
 * (under-loaded experts are raised, over-loaded lowered, an expert exactly at
 * the mean load is unchanged; the sign is decided exactly in integers; one fp32
 * add per expert).  load from moe_expert_load with the same n_valid.  rate must
 * be finite and >= 0.  load: [E] int32; sel_bias: [E] fp32 (in/out).
 */
int moe_bias_update(const int32_t *load, int64_t n_valid, int E, int k, float rate,
                    float *sel_bias, void *stream);

size_t moe_aux_loss_workspace_size(int64_t T, int E);

/*
 * Load-balancing auxiliary loss over the valid prefix (n = n_valid):
 *   p[t,:] = softmax(logits[t,:]) over all E experts (fp32),
 *   P_e = (1/n) sum_{t<n} p[t,e],  f_e = load[e] / (n k),
 *   aux = E * sum_e f_e P_e  (= 1 for balanced load and uniform p),
 *   aux_out[0] = aux, aux_out[1] = coeff * aux.
 * If d_logits is not NULL the gradient of coeff*aux with respect to the logits
 * is ADDED to it (the load is a count and carries none):
 *   d_logits[t,e] += p[t,e] (g_e - sum_e' p[t,e'] g_e'),  g_e = coeff E load[e] / (n^2 k),
 * for t < n; rows t >= n are not touched.  n = 0 writes aux_out = {0, 0} and
 * touches nothing else.  logits: [T,E] fp32; load: [E] int32 from moe_expert_load
 * with the same n_valid; aux_out: [2] fp32 (out); d_logits: [T,E] fp32 (in/out)
 * or NULL; coeff must be finite.  Deterministic: per-block partial sums
 * combined in a fixed order.  ws: moe_aux_loss_workspace_size(T,E) bytes.
 */
int moe_aux_loss(const float *logits, const int32_t *load, int64_t T, int64_t n_valid, int E,
                 int k, float coeff, float *aux_out, float *d_logits, void *ws, size_t ws_bytes,
                 void *stream);

/* ---------------------------------------------------------------- timing */

/*
 * Per-kernel timing for measurement.  While enabled, every kernel launch is
 * bracketed by a pair of HIP events on its own stream.  moe_timing_query
 * waits for the recorded events and returns, for launches recorded under
 * `name` (NULL = all), the summed duration in milliseconds and the launch
 * count.  moe_timing_reset drops all records.  Off by default.  Launch names:
 * router_logits, route_topk, permute_hist, permute_scan, permute_place,
 * permute_rows, tile_prefix, gg_fwd_gate_up_swiglu, gg_fwd_down_scale,
 * combine, combine_bwd, gg_bwd_dh_dswiglu, drs_reduce, gg_bwd_dx,
 * gg_bwd_dw_down, gg_bwd_dw_gate_up, route_bwd, router_dx, router_dw_partial,
 * router_dw_reduce, router_dw_zero, permute_bwd, ffn_gu_f32, ffn_down_f32,
 * route_topk_biased, expert_load, expert_load_reduce, bias_update, aux_loss,
 * aux_loss_final, lora_proj, lora_transpose, lora_grad,
 * gg_fwd_gate_up_swiglu_gather, gg_bwd_dh_dswiglu_gather, row_scale,
 * gg_bwd_dw_gate_up_gather.
 */
int moe_timing_enable(int on);
int moe_timing_reset(void);
int moe_timing_query(const char *name, double *total_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
