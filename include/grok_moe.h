/*
 * grok_moe.h -- C ABI of the MI355X (gfx950) forward pass of one Grok-1 mixture-of-experts FFN layer.
 *
 * The layer (pages cited by title and section):
 *   - Router: logits = x . gate^T (a Dense layer from d_model to the E experts), softmax over all E experts,
 *     then the top-2 experts per token; the call returns the top-k gates and their indices
 *     ("Grok-1: 314B Total Parameters, 25B Active Per Token (MoE Explained)", section "Expert Routing Details").
 *   - Expert: y = (GELU(x W1) (*) (x Wv)) W2, 8 experts of which 2 are active per token
 *     ("A functional bridge between openai/grok and xai-org/grok-1", the architecture diagram).
 *   - Combine: the layer output is the sum over the selected experts of the expert output times that
 *     expert's router probability ("... (MoE Explained)", section "How MoE Works in Practice").
 *   - Shapes: d_model 6144, d_ff 32768, 8 experts, top-2; router gate [8, 6144]
 *     ("Grok-1-BF16", section "Verification"); int8 weights with bf16 scales, scale broadcast over the
 *     grouped axis, JAX [in, out] layout ("Grok-1-BF16", section "Conversion Details").
 *
 * Conventions for every entry point:
 *   - All tensors are row-major and contiguous.  Tensor pointers are DEVICE pointers (HBM of the current HIP
 *     device), 16-byte aligned, owned by the caller, and must stay valid until the enqueued work completes.
 *   - `stream` is the hipStream_t the work is enqueued on (NULL = the legacy default stream).  Every call only
 *     ENQUEUES work and returns without synchronising; results are visible after the stream reaches that point.
 *   - Argument errors are detected on the host before anything is enqueued: the call returns a negative
 *     status, enqueues nothing and writes nothing.  A failed kernel launch returns GROK_MOE_EHIP.
 *   - The library allocates no memory and, apart from the scratch array of grok_moe_forward_noalloc (below), keeps
 *     no mutable global state: calls on different streams with distinct workspaces may run concurrently.
 *   - Weight layout, unless an entry point takes a grok_moe_layout: [E, in, out], W1 and Wv [E, d, f], W2 [E, f, d].
 *     int8 scales, unless an entry point takes a scale layout: [E, 1, f] for W1 and Wv, [E, 1, d] for W2 (one bf16
 *     scale per expert and output channel).
 *   - Supported shapes: k == 2, 2 <= E <= 64, d * f < 2^31.  bf16 and int8 layers need d and f to be multiples
 *     of 256; the fp32 layer needs multiples of 64.  T may be any value in [0, 2^24] (T == 0 enqueues nothing).
 *     Other shapes return GROK_MOE_EUNSUPPORTED; they are never padded silently.
 *   - Passes: the bf16 and int8 layers run at most P = min((2^31 - 1) / (2 d), (2^31 - 1) / (4 f)) tokens per
 *     pass (their tiled kernels address x and h with 32-bit offsets; P = 16383 at d = 6144, f = 32768).  The
 *     whole-layer entry points split a larger T into ceil(T / P) passes of near-equal size over consecutive tokens,
 *     each routed, binned and computed on its own (tokens are independent; expert_counts are summed); the step
 *     entry points grok_moe_expert_up / grok_moe_expert_down take at most P tokens (else EUNSUPPORTED).
 */
#ifndef GROK_MOE_H
#define GROK_MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of a layer.
 *   GROK_MOE_F32 : x, router_w, W1, Wv, W2 float32.  h (the GELU product) is kept in float32.
 *   GROK_MOE_BF16: x, router_w, W1, Wv, W2 bfloat16 (raw 16-bit patterns).  h is rounded once to bf16.
 *   GROK_MOE_W8  : x, router_w bfloat16; W1, Wv, W2 int8 with bf16 scales s1, sv, s2; h rounded to bf16.
 * Accumulation is fp32 in every expert matrix product; the router accumulates in fp64. */
typedef enum { GROK_MOE_F32 = 0, GROK_MOE_BF16 = 1, GROK_MOE_W8 = 2 } grok_moe_dtype;

/* Storage of the expert weights (page "Grok-1-BF16", section "Conversion Details": the checkpoint stores them in
 * JAX's [in, out] convention and the conversion transposes them to PyTorch's [out, in]):
 *   GROK_MOE_IN_OUT: W1, Wv [E, d, f], W2 [E, f, d];
 *   GROK_MOE_OUT_IN: W1, Wv [E, f, d], W2 [E, d, f].
 * The result is bit-identical for both on the same weights: the kernels multiply the same operands in the same
 * order. */
typedef enum { GROK_MOE_IN_OUT = 0, GROK_MOE_OUT_IN = 1 } grok_moe_layout;

enum {
  GROK_MOE_OK = 0,
  GROK_MOE_EINVAL = -1,       /* NULL or misaligned pointer, negative size, unknown dtype or layout */
  GROK_MOE_EUNSUPPORTED = -2, /* valid but unsupported shape (k != 2, E outside [2,64], d/f granularity or
                                 size, more than one pass of tokens in an expert step, scale groups) */
  GROK_MOE_EWORKSPACE = -3,   /* workspace smaller than grok_moe_workspace_size() */
  GROK_MOE_EHIP = -4,         /* a HIP launch failed */
  GROK_MOE_ESCRATCH = -5      /* grok_moe_forward_noalloc: the batch needs more than GROK_MOE_SCRATCH_BYTES */
};

/* Human-readable text of a status code (static storage; never NULL). */
const char* grok_moe_strerror(int status);

/* Bytes of device workspace grok_moe_forward() / grok_moe_forward_ex() need for this shape (0 if the shape is
 * invalid or T == 0).  The workspace holds routing results, the token permutation, h [k*T, f] and the partial
 * expert outputs of one pass (T tokens, or the larger pass size if T needs several passes). */
size_t grok_moe_workspace_size(int64_t T, int64_t d, int64_t f, int E, int k, grok_moe_dtype dtype);

/* The whole layer, with the arguments of the layer's statement grok_moe_forward(x, router_w, w1, wv, w2,
 * [int8 scales], T, d, f, E, k, out) followed by optional outputs: router -> token binning -> fused
 * up-projection with GELU product -> down-projection -> gate-weighted combine, all on `stream`.
 * Router: "... (MoE Explained)", section "Expert Routing Details" (softmax over all E, top-2; gates and indices
 * returned); experts: "A functional bridge ...", architecture diagram; combine: "... (MoE Explained)", section
 * "How MoE Works in Practice"; int8 form: "Grok-1-BF16", section "Conversion Details".
 *   x          [T, d]     f32 | bf16
 *   router_w   [E, d]     f32 | bf16 (the gate weight, [out, in])
 *   w1, wv     [E, d, f]  f32 | bf16 | int8
 *   w2         [E, f, d]  f32 | bf16 | int8
 *   s1, sv     [E, 1, f]  bf16, s2 [E, 1, d] bf16: int8 scales (GROK_MOE_W8 only; must be NULL otherwise)
 *   out        [T, d]     f32, overwritten: out[t] = p[t,0] * y_{e0}(x_t) + p[t,1] * y_{e1}(x_t)
 *   router_bias [E] f32 or NULL: added to the logits before the softmax
 *   topk_idx   [T, k] int32 or NULL (out): selected experts, descending logit, lower index first on ties
 *   topk_p     [T, k] f32 or NULL (out): their softmax probabilities over all E experts (not renormalised)
 *   expert_counts [E] int32 or NULL (out): number of tokens routed to each expert
 *   workspace  device buffer of at least grok_moe_workspace_size() bytes, 256-byte aligned, not shared
 *              with another call in flight.
 * Results are deterministic: identical inputs give bit-identical outputs (no floating-point atomics). */
int grok_moe_forward(const void* x, const void* router_w, const void* w1, const void* wv, const void* w2,
                     const void* s1, const void* sv, const void* s2,
                     int64_t T, int64_t d, int64_t f, int E, int k, grok_moe_dtype dtype,
                     float* out, const float* router_bias, int32_t* topk_idx, float* topk_p,
                     int32_t* expert_counts, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- int8 scale layouts ---------------------------------------------------------------------------------------
 * Page "Grok-1-BF16", section "Conversion Details": int8 weights times bf16 scales with grouped broadcasting,
 * scale shapes (1,N), (8,N), (8,1,N) and (8,8,N).  Where an entry point takes (scale_experts, groups), a scale
 * tensor is [scale_experts, groups, out]:
 *   W[e, k, n] = q[e, k, n] * s[scale_experts == 1 ? 0 : e, k / (in / groups), n]
 * with scale_experts = E (one tensor per expert) or 1 (shared by all experts), and `groups` contiguous groups of
 * in/groups input rows.  (8,1,N) and (8,N) are scale_experts = 8, groups = 1 (the layout of grok_moe_forward);
 * (1,N) is scale_experts = 1, groups = 1; (8,8,N) is scale_experts = 8, groups = 8.
 *   s1, sv  [scale_experts, groups_up, f]   bf16, groups_up divides d and d / groups_up is a multiple of 64
 *   s2      [scale_experts, groups_down, d] bf16, groups_down divides f and f / groups_down is a multiple of 64
 * Other group counts return GROK_MOE_EUNSUPPORTED; scale_experts other than 1 or E, or a group count < 1,
 * GROK_MOE_EINVAL.  A zero scale is allowed (its group contributes nothing).  Accumulation is fp32; with more
 * than one group the kernels keep each column's accumulator in units of the current group's scale (one fp32
 * rounding per group boundary), so non-zero scales of one column must not differ by more than ~1e30 in ratio.
 * scale_experts and the group counts are ignored unless dtype is GROK_MOE_W8. */

/* The whole layer in its general form: as grok_moe_forward, with the weights stored as weight_layout says and
 * int8 scales of layout [scale_experts, groups_up, f] (s1, sv) and [scale_experts, groups_down, d] (s2).
 * Workspace: grok_moe_workspace_size(). */
int grok_moe_forward_ex(const void* x, const void* router_w, const void* w1, const void* wv, const void* w2,
                        const void* s1, const void* sv, const void* s2, grok_moe_layout weight_layout,
                        int scale_experts, int groups_up, int groups_down, int64_t T, int64_t d, int64_t f, int E,
                        int k, grok_moe_dtype dtype, float* out, const float* router_bias, int32_t* topk_idx,
                        float* topk_p, int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* ---- The steps of the layer, one entry point each (grok_moe_forward_ex enqueues exactly these). -------------
 * A "slot" is one (token, selected expert) assignment; there are k*T of them, grouped by expert in ascending
 * expert order and, within an expert, in ascending token order. */

/* Router ("... (MoE Explained)", section "Expert Routing Details"): gate GEMV with fp64 accumulation, softmax
 * over all E, top-2 with the lower-index tie-break.  x [T,d], router_w [E,d] (f32 if dtype == GROK_MOE_F32,
 * else bf16); router_bias [E] f32 or NULL.  Writes topk_idx [T,k] int32 and topk_p [T,k] f32 (both required). */
int grok_moe_route(const void* x, const void* router_w, const float* router_bias, int64_t T, int64_t d, int E,
                   int k, grok_moe_dtype dtype, int32_t* topk_idx, float* topk_p, hipStream_t stream);

/* Token binning (the dispatch of each token to its selected experts, "... (MoE Explained)", section
 * "How MoE Works in Practice"): histogram of topk_idx [T,k], exclusive prefix sum, stable permutation.
 * Writes counts [E], offsets [E+1] (offsets[e] = first slot of expert e, offsets[E] = k*T),
 * perm [k*T] (slot -> token) and inv [T,k] ((token, j) -> slot).  topk_idx entries must lie in [0, E). */
int grok_moe_bin(const int32_t* topk_idx, int64_t T, int E, int k, int32_t* counts, int32_t* offsets,
                 int32_t* perm, int32_t* inv, hipStream_t stream);

/* Fused up-projection ("A functional bridge ...", architecture diagram; int8 form per "Grok-1-BF16",
 * section "Conversion Details"): for every slot s of expert e with token t = perm[s],
 *   a = x[t] . W1[e] (* s1),  b = x[t] . Wv[e] (* sv),  h[s] = GELU_erf(a) * b,
 * fp32 accumulation; h [k*T, f] is bf16 (rounded once, to nearest even) or f32 for GROK_MOE_F32.
 * counts/offsets/perm are grok_moe_bin's outputs; weights stored as weight_layout says; s1, sv of layout
 * [scale_experts, groups_up, f] (int8 only, else NULL). */
int grok_moe_expert_up(const void* x, const void* w1, const void* wv, const void* s1, const void* sv,
                       grok_moe_layout weight_layout, int scale_experts, int groups_up, const int32_t* counts,
                       const int32_t* offsets, const int32_t* perm, int64_t T, int64_t d, int64_t f, int E, int k,
                       grok_moe_dtype dtype, void* h, hipStream_t stream);

/* Number of partial sums grok_moe_expert_down() splits the f axis into for this shape (>= 1; for a T of
 * several passes, that of the first pass). */
int grok_moe_down_splits(int64_t T, int64_t d, int64_t f, int E, int k, grok_moe_dtype dtype);

/* Down-projection (the third matrix of "A functional bridge ...", architecture diagram):
 * y[p, s] = sum over the p-th chunk of f of h[s] . W2[e] (* s2), fp32, for every slot s of expert e.
 * y is [splits, k*T, d] f32 with splits = grok_moe_down_splits(...) (passed back in `splits` as a check; a
 * different value returns GROK_MOE_EINVAL).  Only the sum over p is specified; the chunks are near-equal ranges
 * of f (for the weight-streaming batches, boundaries at multiples of 128 rows).  W2 stored as weight_layout says;
 * s2 of layout [scale_experts, groups_down, d] (int8 only, else NULL). */
int grok_moe_expert_down(const void* h, const void* w2, const void* s2, grok_moe_layout weight_layout,
                         int scale_experts, int groups_down, const int32_t* counts, const int32_t* offsets,
                         int64_t T, int64_t d, int64_t f, int E, int k, grok_moe_dtype dtype, int splits, float* y,
                         hipStream_t stream);

/* Gate-weighted combine ("... (MoE Explained)", section "How MoE Works in Practice"):
 * out[t] = sum_j topk_p[t,j] * (sum_p y[p, inv[t,j]]), the partials summed in ascending p. out [T,d] f32. */
int grok_moe_combine(const float* y, int splits, const float* topk_p, const int32_t* inv, int64_t T, int64_t d,
                     int k, float* out, hipStream_t stream);

/* ---- The MoE part of a Grok-1 layer with its two norms and the residual ------------------------------------
 * Page "Grok-1-BF16", section "Architecture" (four norms per layer: pre-attention, post-attention, pre-MoE,
 * post-MoE) and section "Verification" (pre_moe_norm.scale and post_moe_norm.scale of shape [6144] around
 * moe_block); page "... (MoE Explained)", section "Why JAX Instead of PyTorch" (x = x + moe(norm(x))):
 *   xn  = RMSNorm(x; pre_scale),  out = x + RMSNorm(MoE(xn); post_scale),
 *   RMSNorm(v; g) = v / sqrt(mean(v^2) + eps) * g over the d axis.
 * eps is not on the pages (any eps >= 0).  pre_scale, post_scale [d] are in the activation type (f32 for
 * GROK_MOE_F32, bf16 otherwise).  xn is stored once rounded to the activation type (bf16 round-to-nearest-even
 * from a float64 evaluation) and is what the router and the experts see; the post-norm and the residual add are
 * evaluated in float64 and written as fp32. */

/* Workspace of grok_moe_block_forward (the layer's workspace plus xn). */
size_t grok_moe_block_workspace_size(int64_t T, int64_t d, int64_t f, int E, int k, grok_moe_dtype dtype);

/* The block: the arguments and conventions of grok_moe_forward_ex plus pre_scale, post_scale and eps; out [T,d]
 * fp32 = x + RMSNorm(MoE(RMSNorm(x; pre_scale)); post_scale).  Routing outputs refer to the normed input. */
int grok_moe_block_forward(const void* x, const void* pre_scale, const void* post_scale, double eps,
                           const void* router_w, const void* w1, const void* wv, const void* w2, const void* s1,
                           const void* sv, const void* s2, grok_moe_layout weight_layout, int scale_experts,
                           int groups_up, int groups_down, int64_t T, int64_t d, int64_t f, int E, int k,
                           grok_moe_dtype dtype, float* out, const float* router_bias, int32_t* topk_idx,
                           float* topk_p, int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Step: pre-MoE RMSNorm fused with the router (the norm of "Grok-1-BF16", section "Verification", in front of
 * the router of "... (MoE Explained)", section "Expert Routing Details").  Writes xn [T,d] (activation type),
 * topk_idx, topk_p. */
int grok_moe_route_norm(const void* x, const void* pre_scale, double eps, const void* router_w,
                        const float* router_bias, int64_t T, int64_t d, int E, int k, grok_moe_dtype dtype, void* xn,
                        int32_t* topk_idx, float* topk_p, hipStream_t stream);

/* Step: combine fused with the post-MoE RMSNorm and the residual add (x is the block input [T,d]); the combine of
 * "... (MoE Explained)", section "How MoE Works in Practice", then the post-MoE norm of "Grok-1-BF16", section
 * "Verification". */
int grok_moe_combine_norm(const float* y, int splits, const float* topk_p, const int32_t* inv, const void* x,
                          const void* post_scale, double eps, int64_t T, int64_t d, int k, grok_moe_dtype dtype,
                          float* out, hipStream_t stream);

/* ---- For callers that cannot allocate ------------------------------------------------------------------------
 * Code under HIP graph capture, tight serving loops, or harnesses that forbid hipMalloc cannot provide a workspace
 * from an allocation.  grok_moe_forward_noalloc is grok_moe_forward with the workspace taken from a static device
 * array of GROK_MOE_SCRATCH_BYTES bytes inside the library (one copy on each GPU the library runs on, held until
 * the process ends; its device address is looked up once per device, on the first call with that device current).
 * The call allocates nothing.  It runs on the CURRENT device (`stream` must belong to it).  A batch whose workspace,
 * grok_moe_workspace_size(T, d, f, E, k, dtype), exceeds GROK_MOE_SCRATCH_BYTES is rejected with
 * GROK_MOE_ESCRATCH before anything is enqueued (at d = 6144, f = 32768: up to 292 tokens in bf16, 372 with int8
 * weights).  No part of
 * the array has to start at zero: every call writes what it reads.  All calls on one GPU share its array, so calls
 * that overlap on one GPU (on different streams, or from different threads without ordering) RACE and give wrong
 * results; order them on one stream.  Arguments, results and errors are otherwise those of grok_moe_forward, and
 * the output is bit-identical to it. */
#define GROK_MOE_SCRATCH_BYTES ((size_t)64 << 20)

int grok_moe_forward_noalloc(const void* x, const void* router_w, const void* w1, const void* wv, const void* w2,
                             const void* s1, const void* sv, const void* s2, int64_t T, int64_t d, int64_t f, int E,
                             int k, grok_moe_dtype dtype, float* out, const float* router_bias, int32_t* topk_idx,
                             float* topk_p, int32_t* expert_counts, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GROK_MOE_H */
