/*
 * moe.h -- C ABI of the routed Mixture-of-Experts SwiGLU feed-forward layer
 * (forward pass) for AMD Instinct MI355X (gfx950).
 *
 * The layer (page "MoE Model Architectures", Mixtral 8x7B sections "Sparse
 * MoE Block" and "Expert FFN"; DeepSeek-V3 section "DeepSeekMoE
 * Architecture"):
 *     logits = x W_g (+ b)                      router gate
 *     p      = softmax(logits)                  over the E experts
 *     (idx, w) = top_k(p), w /= sum(w)          renormalisation optional
 *     out[t] = sum_j w[t,j] * FFN_{idx[t,j]}(x[t])  (+ FFN_shared(x[t]))
 *     FFN_e(v) = (silu(v W_gate[e]) * (v W_up[e])) W_down[e]
 *
 * Conventions shared by every entry point
 *  - All data pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates device memory, never frees, and never synchronises the
 *    host: every call only enqueues kernels on `stream` and returns.  Scratch
 *    memory comes from the caller's workspace (`ws`, `ws_bytes`), sized by
 *    moe_workspace_size() (moe_forward_noalloc uses a fixed per-GPU array of
 *    the library instead).  All buffers sized by routing use their worst case
 *    (T*k rows), so no count is ever read back to the host; calls can be
 *    captured into a HIP graph.
 *  - Arrays are dense and row-major.  x is [T, d]; W_g is [d, E]; expert
 *    weights are input-major: W_gate, W_up are [E, d, f] and W_down is
 *    [E, f, d] (the transpose of a torch nn.Linear weight).
 *  - Arguments are validated on the host before any HIP call.  A failing
 *    call returns a status code and enqueues nothing; moe_last_error()
 *    describes the failure (thread-local text).
 *  - T == 0 is valid and enqueues nothing.
 *  - Results are bitwise deterministic run to run: no floating-point atomics.
 *  - Calls on the same stream are ordered; calls that share a workspace must
 *    not run concurrently on different streams.
 *  - Layers of 64 or more expert groups (experts + shared) run part of the
 *    grouped GEMMs on a second stream that the library creates once per host
 *    thread and GPU (default priority, kept until the process ends); it
 *    joins back into `stream` through events before the call's next kernel,
 *    so ordering, graph capture and determinism are as for one stream.
 *    moe_forward_noalloc keeps every launch on `stream`.
 *
 * Conventions fixed here where the pages are silent:
 *  - Router logits are rounded to fp32 once from an fp64 sum (+ bias), and
 *    experts are selected on those fp32 logits, larger first, equal logits
 *    ordered by the lower expert index.  Softmax weights are fp32.
 *  - Capacity (capacity_factor > 0): C = max(1, ceil(cf * T * k / E)); an
 *    assignment a = t*k + j is kept when fewer than C earlier assignments
 *    (smaller a) went to the same expert.  Dropped assignments contribute
 *    nothing and the kept weights are not renormalised again.
 *    capacity_factor == 0 means uncapped (page "Faster writing: run only the
 *    chosen experts; uncap the large profile", the profile change to 0).
 *  - expert offsets have E + 1 entries with a leading 0 (the GPU-computed form
 *    in "Current Bug: CuTeDSLMoERunner produces wrong output", root-cause
 *    section); rows of one expert are kept in ascending assignment order.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size or flag   */
  MOE_ERR_UNSUPPORTED = 2,   /* valid request this library does not handle */
  MOE_ERR_WORKSPACE = 3,     /* ws too small (see moe_workspace_size)        */
  MOE_ERR_HIP = 4            /* a kernel launch failed                      */
} moe_status;

/* FP8 = OCP e4m3fn codes with per-output-channel fp32 scales.  MXFP8 = OCP
 * Microscaling: e4m3fn codes with one E8M0 scale byte (value 2^(byte - 127))
 * per 32 consecutive values along the reduction axis; the layer quantises its
 * activations to the same format on the fly (page "Current Bug:
 * CuTeDSLMoERunner produces wrong output", "Root Cause: scale_a layout doesn't
 * match expert_offsets": a grouped MoE on block-scaled activations and
 * weights, NVFP4 there).  MXFP4 = the same block scales with OCP E2M1 weight
 * codes (0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives; scale exponent
 * floor(log2 max|block|) - 2), two codes per byte, element 2j in the low
 * nibble; the activations are MXFP8 as above. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2, MOE_MXFP8 = 3, MOE_MXFP4 = 4 } moe_dtype;

typedef enum {
  MOE_PATH_AUTO = 0,         /* fused decode for T <= 8, grouped otherwise        */
  MOE_PATH_GROUPED = 1,      /* permute + grouped GEMMs + combine at any T        */
  MOE_PATH_FUSED_DECODE = 2  /* T <= 8 only; larger T returns UNSUPPORTED         */
} moe_path;

#define MOE_FUSED_DECODE_MAX_T 8

/* Who chooses.  Token choice ("MoE Model Architectures", Mixtral "Sparse MoE
 * Block"): every token takes its top_k experts.  Expert choice (same page,
 * Design Patterns, Pattern 3 "Expert Choice Routing"): every expert takes the
 * C tokens with the largest full-softmax score (fp32, ties -> lower token
 * index), C = max(1, min(T, ceil(cf * T * top_k / E))) with cf =
 * capacity_factor (1 when 0); a token's output is the sum over the experts
 * that chose it, in ascending expert order, of its score (divided by the sum
 * of those scores when renormalize = 1) times the expert output, plus the
 * shared expert.  Expert choice runs through moe_forward only (grouped path,
 * T <= MOE_EXPERT_CHOICE_MAX_T); the token-choice stage calls moe_route,
 * moe_permute, moe_grouped_ffn and moe_combine return MOE_ERR_UNSUPPORTED for
 * it. */
typedef enum { MOE_ROUTING_TOKEN_CHOICE = 0, MOE_ROUTING_EXPERT_CHOICE = 1 } moe_routing;
#define MOE_EXPERT_CHOICE_MAX_T 8192

typedef struct {
  int32_t T;                 /* tokens, >= 0                                     */
  int32_t d;                 /* hidden size, multiple of 64                      */
  int32_t E;                 /* routed experts, 1..1023                          */
  int32_t top_k;             /* 1..min(E, 32)                                    */
  int32_t f;                 /* expert intermediate size, multiple of 64         */
  int32_t renormalize;       /* 0 | 1                                            */
  float capacity_factor;     /* 0 => uncapped; else > 0 and finite               */
  int32_t act_dtype;         /* x, W_g, out: MOE_F32 | MOE_BF16                  */
  int32_t w_dtype;           /* experts: F32 (act F32) | BF16, FP8_E4M3, MXFP8 or
                                MXFP4 (act BF16; MXFP8 and MXFP4 need d, f
                                multiples of 128 and run on the grouped path at
                                every T)                                       */
  int32_t has_shared;        /* 0 | 1: one always-on shared expert, weight 1     */
  int32_t path;              /* moe_path                                         */
  int32_t routing;           /* moe_routing (0 = token choice, the default)      */
} moe_desc;

typedef struct {
  const void* W_g;           /* [d, E] act dtype                                  */
  const float* router_bias;  /* [E] fp32 or NULL; added to the logits           */
  const void* W_gate;        /* [E, d, f] w dtype                                 */
  const void* W_up;          /* [E, d, f]                                         */
  const void* W_down;        /* [E, f, d]                                         */
  const float* s_gate;       /* FP8 only: [E, f] per-output-channel scale, else NULL */
  const float* s_up;         /* FP8 only: [E, f]                                  */
  const float* s_down;       /* FP8 only: [E, d]                                  */
  const void* Ws_gate;       /* shared expert [d, f] (has_shared) else NULL       */
  const void* Ws_up;         /* [d, f]                                            */
  const void* Ws_down;       /* [f, d]                                            */
  const float* ss_gate;      /* FP8 shared scales [f], [f], [d] else NULL         */
  const float* ss_up;
  const float* ss_down;
  /* MXFP8 and MXFP4 only (else NULL).  The codes in W_gate, W_up, W_down (and
   * the shared Ws_*) are then OUTPUT-major, K contiguous: W_gate, W_up
   * [E, f, d], W_down [E, d, f] (a torch nn.Linear weight's own layout; for
   * MXFP4 in bytes [E, f, d/2] and [E, d, f/2], two codes per byte); these are
   * their E8M0 scales, one byte per 32 consecutive K values: */
  const uint8_t* mx_gate;    /* [E, f, d/32]                                       */
  const uint8_t* mx_up;      /* [E, f, d/32]                                       */
  const uint8_t* mx_down;    /* [E, d, f/32]                                       */
  const uint8_t* mxs_gate;   /* shared expert [f, d/32], [f, d/32], [d, f/32]      */
  const uint8_t* mxs_up;
  const uint8_t* mxs_down;
} moe_weights;

/* Optional outputs of moe_forward.  The router telemetry fields follow
 * "MoE Model Architectures", Switch Transformers "Load Balancing Loss" (E times
 * the sum over experts of the mean router probability times the fraction of
 * tokens routed there) and DeepSeek-V3 "Auxiliary-Loss-Free Load Balancing"
 * (the per-expert load a router bias steers).  With k slots per token the
 * fraction for expert e is d_routed[e] / T.  Requesting any telemetry field
 * adds one small launch (T <= 64) or three; the router logits they read live
 * in the workspace.  All fields are computed with fixed summation orders
 * (bitwise reproducible).
 * Nothing is written when T == 0. */
typedef struct {
  int32_t path_taken;        /* out: MOE_PATH_GROUPED or MOE_PATH_FUSED_DECODE    */
  int32_t* d_n_dropped;      /* device [1] or NULL: dropped assignments           */
  int32_t* d_counts;         /* device [E] or NULL: kept assignments per expert   */
  hipEvent_t ev_begin;       /* NULL or an event recorded on `stream` just before */
  hipEvent_t ev_end;         /* ... and just after the dominant expert-FFN kernel */
  int32_t* d_routed;         /* device [E] or NULL: assignments choosing each
                                expert, before any capacity limit                 */
  float* d_prob_mean;        /* device [E] or NULL: mean over tokens of the full
                                softmax probability (fp64 sums, fp32 result)      */
  float* d_lb_loss;          /* device [1] or NULL: E * sum_e prob_mean[e] *
                                routed[e] / T                                     */
} moe_stats;

/* Bytes of workspace every entry point below needs for `desc` (the maximum
 * over entry points).  Returns 0 when desc is invalid. */
size_t moe_workspace_size(const moe_desc* desc);

/* Per-expert capacity C for desc, or -1 when uncapped / desc invalid.  With
 * expert-choice routing, the number of tokens every expert takes. */
int32_t moe_capacity(const moe_desc* desc);

/* Router: logits, softmax, top-k and (optional) renormalisation.
 * Pages: "MoE Model Architectures", "Sparse MoE Block" (gate, softmax, topk,
 * divide by the top-k sum), "Auxiliary-Loss-Free Load Balancing" (bias);
 * "perf(moe): route granite-4.0-h single-token MoE through the fused kernel"
 * (fp32 softmax scores already equal the renormalised top-k softmax).
 *   x        [T, d] act dtype
 *   topk_idx [T, k] int32 out: slot 0 holds the largest logit
 *   topk_w   [T, k] fp32 out: softmax weights of the chosen experts
 *   logits   [T, E] fp32 out, or NULL
 * For T > 8 the workspace (moe_workspace_size) must be passed.  For T <= 8 it
 * may be NULL; when passed, routers with d * E > 65536 use it to spread the
 * logit dot products over many work-groups (NULL: one work-group). */
moe_status moe_route(const moe_desc* desc, const void* x, const moe_weights* w,
                     int32_t* topk_idx, float* topk_w, float* logits,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Token-to-expert permutation with capacity dropping.
 * Pages: "Sparse MoE Block" (per-expert gather in token order, empty experts
 * skipped); "Current Bug: CuTeDSLMoERunner produces wrong output" (expert
 * offsets); "Top-1 Routing" (expert capacity, overflow dropped).
 *   topk_idx      [T, k] int32 in, values in [0, E)
 *   counts        [E]      kept assignments per expert
 *   offsets       [E + 1]  exclusive prefix of counts, offsets[0] = 0
 *   sorted_assign [T * k]  kept assignment ids a = t*k + j, expert-major,
 *                          ascending a inside an expert; entries from
 *                          offsets[E] on are set to -1
 *   inv_perm      [T * k]  row of a in sorted_assign, or -1 if dropped
 *   n_dropped     [1]      number of dropped assignments */
moe_status moe_permute(const moe_desc* desc, const int32_t* topk_idx,
                       int32_t* counts, int32_t* offsets, int32_t* sorted_assign,
                       int32_t* inv_perm, int32_t* n_dropped,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* Grouped SwiGLU expert FFN over the permuted rows; only experts with rows
 * do work.  Pages: "Expert FFN" (w2(silu(w1 x) * w3 x)); "Faster writing: run
 * only the chosen experts" (touch only chosen experts' weights).
 *   sorted_assign, offsets  as produced by moe_permute (may come from elsewhere)
 *   y_sorted  [T*k (+ T when has_shared), d] fp32 out: row r < offsets[E] is
 *             FFN_e(x[sorted_assign[r] / k]) for the expert e owning row r;
 *             rows T*k + t hold the shared expert's FFN(x[t]); other rows are
 *             left untouched. */
moe_status moe_grouped_ffn(const moe_desc* desc, const void* x, const moe_weights* w,
                           const int32_t* sorted_assign, const int32_t* offsets,
                           float* y_sorted, void* ws, size_t ws_bytes, hipStream_t stream);

/* Weighted combine: out[t] = sum_{j kept} topk_w[t,j] * y_sorted[inv_perm[t*k+j]]
 * (+ y_sorted[T*k + t] with has_shared), summed in slot order in fp32 and
 * rounded once to the act dtype.  Pages: "Sparse MoE Block" (weighted
 * index_add), "Design Patterns" (shared + routed). */
moe_status moe_combine(const moe_desc* desc, const float* y_sorted, const int32_t* inv_perm,
                       const float* topk_w, void* out, hipStream_t stream);

/* Whole layer: route -> (permute -> grouped FFN -> combine) or, for T <= 8,
 * route -> fused decode (streams only the chosen experts' weights; page
 * "perf(moe): route granite-4.0-h single-token MoE through the fused
 * kernel").  out [T, d] act dtype.  stats may be NULL.
 * Expert-choice routing (desc->routing): route -> per-expert token selection
 * -> grouped FFN -> combine; stats->d_counts receives C per expert,
 * stats->d_n_dropped the number of tokens no expert chose; the telemetry
 * fields are token-choice statistics and are declined (MOE_ERR_UNSUPPORTED). */
moe_status moe_forward(const moe_desc* desc, const void* x, const moe_weights* w, void* out,
                       moe_stats* stats, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, results and path choice as
 * moe_forward; its scratch is a fixed array of MOE_NOALLOC_SCRATCH_BYTES
 * inside the library, one copy per GPU, held until the process ends.  The
 * first call on a device looks up that device's copy (with the device
 * current).  Layers whose moe_workspace_size() exceeds the array return
 * MOE_ERR_UNSUPPORTED and enqueue nothing.  Every call on one GPU uses the
 * same array, which keeps the previous call's contents (none of which a call
 * relies on): calls that overlap in time on one GPU, from different streams
 * or threads, race and must be serialised by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
moe_status moe_forward_noalloc(const moe_desc* desc, const void* x, const moe_weights* w, void* out,
                               moe_stats* stats, hipStream_t stream);

/* Gradients produced by moe_backward (fp32, dense, row-major, caller-owned
 * device memory).  Every field below is fully written by each call. */
typedef struct {
  float* dx;                 /* [T, d]                                            */
  float* dW_g;               /* [d, E] router weight                              */
  float* d_bias;             /* [E] router bias, or NULL (not computed)           */
  float* dW_gate;            /* [E, d, f]                                         */
  float* dW_up;              /* [E, d, f]                                         */
  float* dW_down;            /* [E, f, d]                                         */
  float* dWs_gate;           /* shared expert [d, f], [d, f], [f, d] (has_shared) */
  float* dWs_up;
  float* dWs_down;
  hipEvent_t ev_begin;       /* NULL or recorded just before the dX GEMM         */
  hipEvent_t ev_end;         /* ... and just after it                             */
} moe_grads;

/* Bytes of workspace moe_backward needs for desc (0 when desc is invalid or
 * not supported by the backward). */
size_t moe_backward_workspace_size(const moe_desc* desc);

/* Backward of moe_forward for layers with bf16 activations and bf16, fp8,
 * MXFP8 or MXFP4 weights, and for fp32 layers, token-choice or expert-choice
 * routing: given dout = dL/dout [T, d] (act dtype), the gradients of L with
 * respect to x, the router weight and bias, and every expert's (and the shared
 * expert's) three matrices.  The expert selection (top-k, capacity) is held
 * fixed: gradients flow through the routing weights (the softmax and its
 * renormalisation over the chosen experts) and through the chosen experts'
 * SwiGLU FFNs; dropped assignments carry no gradient; experts that received no
 * token get zero gradients.  Expert choice ("MoE Model Architectures", Design
 * Patterns, Pattern 3): the tokens each expert took are held fixed; a token's
 * routing gradient runs over the experts that took it (the full softmax, or
 * its renormalisation over those experts), and a token no expert took gets
 * only the shared expert's gradient.  The routing and the expert activations
 * are recomputed from x (nothing is kept from the forward).  fp8 weights: the
 * gradients are with respect to the weights' values (e4m3 code x channel
 * scale; the scales get none), and the GEMMs run on those values rounded once
 * to bf16, kept in the workspace.  MXFP8 / MXFP4 weights: the same, with the
 * values exact in bf16; the forward's MXFP8 quantisation of the expert inputs
 * and of the activated rows is recomputed and differentiated as the identity
 * (straight through).  fp32 layers compute every intermediate in fp32 (SIMT
 * FMA; no bf16 rounding).  Weight gradients are summed over each expert's
 * tokens in a fixed order without atomics: results are bitwise reproducible.
 * Pages: "Testing using claude to graft ETHOS onto modded-nanogpt base", "Key
 * Implementation Details" (a backward that recomputes the forward values and
 * accumulates each weight gradient over the tokens that chose the expert);
 * "Faster writing: run only the chosen experts; uncap the large profile",
 * "Test plan" (slot gradients of the chosen-experts dispatch).
 *   x, dout  [T, d] act dtype;  w as for moe_forward;  grads as documented above
 *   ws       moe_backward_workspace_size(desc) bytes, 256-byte aligned
 * Returns MOE_ERR_UNSUPPORTED for dtype pairs the forward declines.
 * T == 0 writes zero weight gradients. */
moe_status moe_backward(const moe_desc* desc, const void* x, const moe_weights* w, const void* dout,
                        const moe_grads* grads, void* ws, size_t ws_bytes, hipStream_t stream);

/* OCP MXFP8 quantisation of a row-major [rows, cols] matrix along its rows:
 * for every 32 consecutive values of a row, with m their largest magnitude,
 * the scale exponent is s = floor(log2 m) - 8 clamped to [-127, 127] (an
 * all-zero block takes -127), scales[b] = s + 127, and each value v becomes
 * the e4m3fn code nearest to v / 2^s (ties to the even code, magnitudes above
 * 448 saturated to 448, the sign kept for values that round to zero).  The
 * layer applies exactly this to x (and, inside its kernels, to the SwiGLU
 * activations) when w_dtype is MOE_MXFP8; weights may be prepared with it.
 *   in      [rows, cols] device, in_dtype MOE_F32 | MOE_BF16, 16-byte aligned
 *   codes   [rows, cols] uint8 out;  scales [rows, cols/32] uint8 out
 *   cols    multiple of 32; rows >= 0 (0 enqueues nothing)
 * Page: "Current Bug: CuTeDSLMoERunner produces wrong output", "Root Cause:
 * scale_a layout doesn't match expert_offsets" (per-token activation scale
 * factors of a block-scaled grouped MoE). */
moe_status moe_quantize_mxfp8(const void* in, int32_t in_dtype, int64_t rows, int32_t cols,
                              uint8_t* codes, uint8_t* scales, hipStream_t stream);

const char* moe_status_string(moe_status s);
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
