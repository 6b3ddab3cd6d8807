/*
 * moe.h -- C ABI of the MI355X (gfx950) library for the forward pass of one
 * DeepSeekMoE-style mixture-of-experts FFN layer: a softmax top-k router over
 * N_r fine-grained routed SwiGLU experts plus N_s always-on shared SwiGLU
 * experts fused into one MLP of width N_s*f.
 *
 * What the layer computes (sources: "Shared Expert" page on DeepSeek-V3, How
 * it works, eq. 12 without its residual term, and the SwiGLU definition;
 * Official code: MoE.forward returns shared + routed on the flattened (T, d)
 * batch; "What is an 'expert', really?", glossary and panel 2: a linear
 * router scores the experts, softmax makes blend weights, the top-k are kept):
 *
 *   l[t,e]  = u[t,:] . w_router[e,:] (+ router_bias[e])
 *   p[t,:]  = softmax over all N_r experts of l[t,:]
 *   S_t     = the k largest l[t,e] (ties to the lower e), slots in descending order
 *   out[t]  = FFN_shared(u[t]) + sum_{j<k} p[t,S_t[j]] * FFN_{S_t[j]}(u[t])
 *   FFN(x)  = W2 (SiLU(W1 x) * W3 x),   SiLU(z) = z * sigmoid(z)
 *
 * The kept gates are NOT renormalised; the shared MLP enters with coefficient
 * exactly 1; moe_layer_forward adds no residual and applies no normalisation
 * (u arrives already RMS-normalised).  moe_block_forward is the pre-norm block
 * around it: u = RMSNorm(x), out = x + layer(u).
 *
 * Every token goes to all k of its experts unless moe_dims.capacity sets a
 * seat limit per expert: then each expert keeps the first `capacity` of its
 * (token, slot) pairs in token order and the rest are dropped (they contribute
 * nothing; the shared MLP still runs on every token).  Source: "What is an
 * 'expert', really?", glossary: capacity factor / token dropping.
 *
 * Dense layers: n_routed == 0 (with top_k == 0) describes the dense prefix
 * layers' feed-forward block ("Shared and fine-grained experts", Developer
 * level: the first three DeepSeek-V3 layers stay dense, width 18432; "Shared
 * Expert", Official code: the same SwiGLU as the shared MLP).  Only the MLP of
 * width d_ff_shared (> 0) runs, through the shared-group kernels:
 *   out[t] = W2s (SiLU(W1s u[t]) * W3s u[t]);  d_ff, w_router, w1, w3, w2 are ignored.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked (host).  Every array is dense,
 *     row-major, 16-byte aligned.  Weights use the [out, in] layout:
 *       w_router [N_r, d]; w1, w3 [N_r, f, d]; w2 [N_r, d, f];
 *       w1s, w3s [f_s, d]; w2s [d, f_s]; router_bias [N_r] fp32.
 *   - The caller owns every buffer, including the workspace `ws` (size from
 *     moe_workspace_size).  The library allocates and frees nothing and keeps
 *     no state between calls; calls on different streams with different
 *     workspaces may run concurrently.
 *   - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL =
 *     the default stream).  No call copies device data to the host, except
 *     moe_read_diagnostics, which synchronises the stream.
 *   - Arguments are validated on the host before any HIP call.  A failing
 *     call returns a non-zero moe_status, enqueues nothing, and leaves a
 *     message in moe_last_error().  T == 0 is a valid no-op.
 *   - Faults inside a kernel surface at the caller's next synchronisation.
 *
 * Limits: 1 <= top_k <= 16; 1 <= n_routed <= 1024; top_k <= n_routed (or
 * n_routed == top_k == 0 for a dense layer); capacity >= 0; with n_group > 1:
 * n_group <= 64, n_routed % n_group == 0, 1 <= topk_group <= n_group and
 * topk_group * (n_routed / n_group) >= top_k;
 * d_model and d_ff (and d_ff_shared when non-zero) multiples of 64;
 * 64 <= d_model <= 32768; T <= 4194304 (2^22) and T * top_k < 2^31.  On the
 * bf16 prefill path every matrix the expert GEMMs read (u, the [T*k, f] and
 * [T, f_s] hidden activations, each expert's weight matrix) must be under
 * 4 GiB.  On every path each kernel dispatch must stay under 2^32 work-items
 * (the dispatch packet's 32-bit grid size); the expert-FFN launches of the
 * chosen path are checked for this before anything is enqueued.  Token batches
 * past these limits are rejected with MOE_ERR_UNSUPPORTED and must be split.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_VALUE = 1, /* null pointer, negative T, top_k > n_routed, misaligned pointer */
  MOE_ERR_UNSUPPORTED = 2,   /* a size or dtype outside the limits above */
  MOE_ERR_WORKSPACE = 3,     /* ws_bytes smaller than moe_workspace_size() */
  MOE_ERR_HIP = 4            /* a HIP launch or runtime call failed; text in moe_last_error() */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Layer shape.  dtype applies to u and to every weight (the router bias is
 * always fp32).  bf16 inputs are multiplied on bf16 matrix cores with fp32
 * accumulation; fp32 inputs use fp32 arithmetic throughout. */
typedef struct moe_dims {
  int32_t d_model;     /* d */
  int32_t n_routed;    /* N_r */
  int32_t d_ff;        /* f, width of one routed expert */
  int32_t d_ff_shared; /* f_s = N_s * f, width of the fused shared MLP; 0 = no shared expert */
  int32_t top_k;       /* k */
  int32_t dtype;       /* moe_dtype of u and the weights */
  int32_t out_dtype;   /* moe_dtype of `out` (MOE_F32 recommended) */
  int32_t capacity;    /* seats per routed expert per call; 0 = no limit.  A caller
                          with a capacity factor cf uses ceil(cf * T * top_k / n_routed). */
  int32_t n_group;     /* group-limited routing: experts form n_group contiguous groups
                          (0 or 1 = no groups) ... */
  int32_t topk_group;  /* ... of which each token keeps topk_group (see moe_router_topk) */
} moe_dims;

/* Device pointers to the layer's weights (layouts above).  router_bias may be
 * NULL (no bias); w1s, w3s, w2s must be NULL exactly when d_ff_shared == 0. */
typedef struct moe_weights {
  const void *w_router;
  const float *router_bias;
  const void *w1, *w3, *w2;
  const void *w1s, *w3s, *w2s;
} moe_weights;

/* Path choice and optional stage timing.
 *   path: 0 = automatic (decode path when T*top_k <= 2*n_routed and T <= 256,
 *         else prefill), 1 = prefill (tiled grouped GEMMs), 2 = decode
 *         (weight-streaming kernels over the experts that received tokens).
 *   events (host array of n_events hipEvent_t, may be NULL): when non-NULL the
 *   library records events[i] on `stream` at stage boundaries, in this order:
 *   0 start, 1 after router logits, 2 after top-k, 3 after permutation,
 *   4 after gate/up, 5 after down, 6 after combine (moe_layer_forward; for a
 *   dense layer 1-3 mark the same point), or 0 start, 1 after RMSNorm, then
 *   2..7 as 1..6 above (moe_block_forward), or 0 start, 1 after gate/up,
 *   2 after down (moe_expert_ffn).  Boundaries beyond n_events are not
 *   recorded.
 *   The automatic choice for a dense layer is the decode path when T <= 256. */
typedef struct moe_options {
  int32_t path;
  int32_t n_events;
  void **events;
} moe_options;

/* Diagnostics written by the kernels into the workspace header. */
typedef struct moe_diag {
  uint32_t flags;           /* bit 0: a top-k comparison could not be settled exactly
                               bit 1: topk_idx held an index outside [0, N_r) (skipped)
                               bit 2: topk_idx held a duplicate expert in one row */
  uint32_t tokens_exact;    /* tokens with a top-k comparison the first-level bound left open */
  uint32_t exact_keys;      /* exact fixed-point logits evaluated (comparisons fp64 left open) */
  uint32_t refinements;     /* fp64 logit recomputation passes */
} moe_diag;

/* Workspace needed by every call below for this shape and token count (host out). */
moe_status moe_workspace_size(const moe_dims *dims, int64_t T, size_t *bytes);

/* Router: logits, softmax over all N_r experts, per-token top-k (n_routed >= 1).
 * Writes topk_idx [T, k] int32 (slot 0 = largest logit; ties to the lower
 * expert index; the selection and slot order equal those of the exact real
 * logits of the stored inputs) and topk_w [T, k] fp32 = the full-softmax
 * probability of each kept expert.
 * With n_group > 1 and topk_group < n_group the top-k is group-limited: the
 * experts form n_group contiguous groups of n_routed / n_group, a group scores
 * its best expert's logit, each token keeps its topk_group best groups (ties to
 * the lower group) and its k experts are the top-k of those groups' experts;
 * the gates stay full-softmax probabilities.
 * Source: "What is an 'expert', really?" (glossary: router, top-k, softmax;
 * panel 2) and "Shared Expert" (How it works: the N_r centroids); node-limited
 * routing: "Shared and fine-grained experts" (Developer level, 'Why not go
 * finer still'; Researcher level, Systems limits: n_group 8, topk_group 4; the
 * group score is not on the pages). */
moe_status moe_router_topk(const moe_dims *dims, int64_t T, const void *u, const void *w_router,
                           const float *router_bias, int32_t *topk_idx, float *topk_w,
                           void *ws, size_t ws_bytes, void *stream);

/* Permutation: group the T*k (token, slot) pairs by expert.
 * counts [N_r] = pairs kept per expert; offsets [N_r+1] exclusive prefix of
 * counts (offsets[N_r] = T*k without a capacity); row_token [T*k]: rows
 * offsets[e]..offsets[e+1]-1 hold the tokens that chose e in ascending token
 * order; token_row [T, k]: the row of token t's slot j, or -1 when the pair was
 * dropped for capacity.  With dims->capacity = C > 0, counts[e] = min(pairs, C)
 * and expert e keeps its first C pairs in token order; row_token entries
 * past offsets[N_r] are then left unwritten.  Deterministic and
 * bit-exact.  Each row of topk_idx must hold k distinct experts in [0, N_r);
 * violations set moe_diag.flags.  Needs n_routed >= 1.
 * Source: "Shared Expert" (How it works: scatter-sum of routed outputs);
 * "What is an 'expert', really?" (glossary: capacity factor / token dropping). */
moe_status moe_permute(const moe_dims *dims, int64_t T, const int32_t *topk_idx, int32_t *counts,
                       int32_t *offsets, int32_t *row_token, int32_t *token_row,
                       void *ws, size_t ws_bytes, void *stream);

/* Expert FFNs: y_rows[r,:] = FFN_e(u[row_token[r],:]) for every row r of every
 * expert group e (fp32 [T*k, d]), and y_shared[t,:] = shared MLP of u[t,:]
 * (fp32 [T, d]) when the layer has shared experts (else y_shared must be NULL).
 * counts/offsets/row_token are moe_permute's outputs.
 * Source: "Shared Expert" (How it works: SwiGLU; Official code: fused shared
 * MLP of width N_s*f on the full batch); "Shared and fine-grained experts"
 * (Researcher level, Systems limits: grouped GEMM over many small experts).
 * Dense layer (n_routed == 0): only y_shared is written; counts, offsets,
 * row_token and y_rows are ignored and may be NULL. */
moe_status moe_expert_ffn(const moe_dims *dims, int64_t T, const void *u, const moe_weights *w,
                          const int32_t *counts, const int32_t *offsets, const int32_t *row_token,
                          float *y_rows, float *y_shared, const moe_options *opts,
                          void *ws, size_t ws_bytes, void *stream);

/* Combine: out[t,:] = y_shared[t,:] + sum_{j=0..k-1} topk_w[t,j] * y_rows[token_row[t,j],:],
 * accumulated in fp32 in exactly this order (y_shared NULL: start from 0;
 * slots with token_row -1 skipped), written as out_dtype.  Dense layer
 * (top_k == 0): out = y_shared converted; y_rows, topk_w, token_row ignored.
 * Source: "Shared Expert" (How it works: shared output added to the
 * scatter-sum of routed outputs; Watch-outs: coefficient 1). */
moe_status moe_combine(const moe_dims *dims, int64_t T, const float *y_rows, const float *y_shared,
                       const float *topk_w, const int32_t *token_row, void *out, void *stream);

/* The whole layer: router, permutation, expert FFNs, combine; `out` [T, d] in
 * out_dtype receives shared + routed (no residual).  Intermediates live in ws. */
moe_status moe_layer_forward(const moe_dims *dims, int64_t T, const void *u, const moe_weights *w,
                             void *out, const moe_options *opts, void *ws, size_t ws_bytes,
                             void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer as moe_layer_forward, computing the same result bit for bit, with the
 * workspace taken from a library-owned device array of MOE_STATIC_WS_BYTES
 * (64 MiB) instead of a `ws` argument.  The caller still passes u, the
 * weights and out.  Nothing is allocated or freed by the call: the array is
 * part of the library's code object, one per device, held by each device the
 * library runs on until the process ends; its device address is looked up
 * once per device on the first call made with that device current (the
 * current device must be the one `stream` belongs to).  A call whose
 * workspace (moe_workspace_size) exceeds MOE_STATIC_WS_BYTES is rejected with
 * MOE_ERR_WORKSPACE before anything is enqueued; at the DeepSeek-V3 shape this
 * covers decode batches (T = 64 needs about 27 MB).  Every call on one device
 * shares that device's array and leaves its contents behind for the next:
 * calls that overlap on one device (two streams, two threads) race and must
 * be serialised by the caller.  Intermediates that must start cleared are
 * cleared by the call's own kernels, so no call depends on what the previous
 * one left. */
#define MOE_STATIC_WS_BYTES (64 << 20)
moe_status moe_layer_forward_static(const moe_dims *dims, int64_t T, const void *u, const moe_weights *w,
                                    void *out, const moe_options *opts, void *stream);

/* RMSNorm of the residual stream: u[t,:] = x[t,:] / sqrt(mean_c x[t,c]^2 + eps) * norm_weight[:].
 * x and u are [T, d_model] in dims->dtype; norm_weight [d_model] is fp32.
 * The mean of squares, the scale and the products are evaluated in fp64 and
 * rounded once to dims->dtype (to nearest, ties to even), so u matches the
 * exact normalisation rounded once, except for a value within an fp64 ulp of
 * a rounding midpoint.  eps >= 0.  u may not alias x.  Only dims->d_model and
 * dims->dtype are read.
 * Source: "Shared Expert" (How it works: the FFN input is already
 * RMS-normalised; Watch-outs: the shared experts sit behind ffn_norm). */
moe_status moe_rmsnorm(const moe_dims *dims, int64_t T, const void *x, const float *norm_weight, double eps,
                       void *u, void *stream);

/* Pre-norm block: u = RMSNorm(x) (as moe_rmsnorm, kept in ws), then the layer
 * on u (as moe_layer_forward), then out[t,:] = x[t,:] + layer(u)[t,:], the
 * residual added in fp32 after the layer's own fp32 sum, written as
 * out_dtype.  x [T, d_model] in dtype; out may not alias x.  Works for dense
 * layers (n_routed == 0) too.
 * Source: "Shared Expert" (How it works: eq. 12's residual is added at block
 * level, x = x + ffn(ffn_norm(x)); MoE.forward returns shared + routed only). */
moe_status moe_block_forward(const moe_dims *dims, int64_t T, const void *x, const float *norm_weight, double eps,
                             const moe_weights *w, void *out, const moe_options *opts, void *ws, size_t ws_bytes,
                             void *stream);

/* Copy the diagnostics of the last call that used `ws` to *diag (host);
 * synchronises `stream`.  Intended for tests. */
moe_status moe_read_diagnostics(const void *ws, moe_diag *diag, void *stream);

/* Message of the last failing call on this thread (library-owned storage). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
