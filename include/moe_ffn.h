/*
 * moe_ffn.h -- C ABI of the MI355X (gfx950) MoE FFN layer forward.
 *
 * The layer is the Mixture-of-Experts feed-forward block of DFlash/DSpark
 * draft models:
 *   Router (score -> select -> routing_weights), permutation of the (token, k)
 *   slots by expert, grouped SwiGLU expert GEMMs (gate_up, optional clamp,
 *   down), weighted combine, optional (sigmoid-gated) shared expert.
 *
 * Pages cited (title and section):
 *   [SF1033]   SpecForge PR #1033 "MoE FFN for DFlash-family drafts: the
 *              module" -- "Router" section, the score / select /
 *              routing_weights table; commit note on the 1e-20 epsilon.
 *   [SF1073]   SpecForge PR #1073 "MoE drafts: DeepSeek-V4.1's own DSpark
 *              draft (stacked on #1035)" -- commit notes on the fp32
 *              expert_bias (selection only), on select receiving the shifted
 *              scores, on the DeepSeek-V4 family (sqrt-softplus scores,
 *              route_scale, clamped SwiGLU, one ungated shared expert), on the
 *              V4.1 converter (FP4 experts: two e2m1 codes per byte, low
 *              nibble first, one e8m0 scale per 32 inputs; w1/w3 fused into
 *              gate_up_proj, w2 into down_proj); on the load balancing
 *              (int64 tokens_per_expert over kept slots, moe/step_balance,
 *              update_expert_bias as one DeepSeek-V3 sign step).
 *   [SGL48763] sglang PR #48763 "[Feat] dflash: Serve MoE FFN drafts for
 *              DFlash and DSpark" -- commit notes on the DraftMoE forward
 *              (fp32 router logits, sigmoid-gated shared expert, a rank with
 *              no tokens routes an empty top-k) and on the CUDA fixes (shared
 *              expert must see the unmodified input; int32 expert ids).
 *   [SF941]    SpecForge PR #941 "feat(serving): SGLang draft classes for the
 *              Qwen3.8-27B DSpark MoE drafter (SGLang FusedMoE path) + tuned
 *              fused-MoE configs" -- "What" (fp32 router logits with the
 *              optional router bias; sigmoid-gated shared expert).
 *   [MI143]    MoE-Infinity PR #143 "feat(dflash): converge DFlash spec-decode
 *              stack -> dev (supersedes #140)" -- commit note on the resident
 *              gpt-oss MXFP4 experts (output-major [E,N,K/2] codes and
 *              [E,N,K/32] scales, used without a transpose; expert biases).
 *
 * Conventions (all entry points)
 *   - Every tensor pointer is a DEVICE pointer to contiguous row-major memory
 *     owned by the caller; the library never allocates, frees or copies to
 *     the host inside moe_route / moe_ffn_forward.  Scratch memory is the
 *     caller's `workspace`, sized by moe_workspace_bytes.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously and stream-ordered; there is no
 *     device->host synchronisation, so a call can be captured in a HIP graph.
 *   - The return value reports argument validation and launch errors only;
 *     a fault inside a kernel surfaces at the caller's next synchronisation.
 *     On a non-OK status nothing has been enqueued, and moe_last_error()
 *     gives a thread-local description.
 *   - Results are bitwise reproducible from call to call (no floating-point
 *     atomics; fixed reduction orders).
 *   - Calls that share a workspace must not overlap in time (same stream, or
 *     ordered by events).
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_FFN_ABI_VERSION 3

/* Symbols of the shared library are exported explicitly. */
#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

/* Limits of the kernels (checked by moe_validate). */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16
#define MOE_MAX_GROUPS 64

/* Storage formats. */
enum moe_dtype {
  MOE_DTYPE_F32 = 0,   /* IEEE binary32                                        */
  MOE_DTYPE_BF16 = 1,  /* bfloat16 (upper half of binary32)                    */
  MOE_DTYPE_MXFP4 = 2  /* OCP MX FP4: E2M1 codes + E8M0 scale per 32 inputs;
                          routed expert weights only                           */
};

/* Router score functions ([SF1033] Router table, row score; [SF1073]
 * DeepSeek-V4 family commit note). */
enum moe_score_fn {
  MOE_SCORE_SOFTMAX = 0,      /* softmax over the E logits                     */
  MOE_SCORE_SIGMOID = 1,      /* 1 / (1 + exp(-logit))                         */
  MOE_SCORE_SQRTSOFTPLUS = 2  /* sqrt(log(1 + exp(logit)))                      */
};

/* SwiGLU activation of the experts (routed and shared), on the clamped
 * pre-activations g' = min(g, L), u' = min(max(u, -L), L) (L = swiglu_limit):
 *   MOE_ACT_SWIGLU      h = silu(g') * u'                  ([SGL48763] DraftMLP
 *                       commit note; [SF1073] DeepSeek-V4 family: clamped SwiGLU)
 *   MOE_ACT_SWIGLU_OAI  h = g' * sigmoid(1.702 g') * (u' + 1): gpt-oss's
 *                       "swigluoai", named in [SGL48763]'s DraftMLP commit note
 *                       but defined on no page; the form gpt-oss publishes. */
enum moe_activation {
  MOE_ACT_SWIGLU = 0,
  MOE_ACT_SWIGLU_OAI = 1
};
#define MOE_SWIGLU_OAI_ALPHA 1.702f

/* How the MXFP4 experts' gate_up product is computed where experts hold
 * hundreds of rows (the large-tile kernels; elsewhere the decode path runs):
 *   MOE_MX_DECODE        codes decoded to bf16 (exact), bf16 matrix cores
 *   MOE_MX_BLOCK_SCALED  codes fed as they are to gfx950's block-scaled
 *                        matrix cores (E2M1 x E4M3 with E8M0 scales per 32
 *                        inputs), the bf16 activations split into two MXFP8
 *                        terms hi + lo per 32-input block, scale 2^(floor(
 *                        log2 max|x|) - 7); hi + lo equals x up to remainders
 *                        below the smallest E4M3 subnormal of their block.
 *                        Taken when H is a multiple of 64, H <= 4096 and the
 *                        gate_up scale array starts on 16 bytes; otherwise,
 *                        and for the down product, the decode path runs.
 * The four-bit code layout and scales are those of [SF1073] / [MI143]. */
enum moe_mx_gemm {
  MOE_MX_DECODE = 0,
  MOE_MX_BLOCK_SCALED = 1
};

/* Status codes. */
enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,      /* a value or pointer is invalid                  */
  MOE_ERR_UNSUPPORTED = -2,  /* valid, but outside what the kernels implement  */
  MOE_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required     */
  MOE_ERR_HIP = -4           /* a HIP runtime call failed                      */
};

/*
 * Layer configuration (plain values, host memory).
 *
 *   T  tokens (T = 0 is legal: a rank with no tokens routes an empty top-k,
 *      [SGL48763] DraftMoE forward commit note)
 *   H  hidden size; E experts; I expert intermediate size; K experts per token
 *   act_dtype  format of x, the router gate, the shared expert and `out`:
 *              MOE_DTYPE_F32 or MOE_DTYPE_BF16
 *   w_dtype    format of the routed experts: MOE_DTYPE_F32 (requires f32
 *              activations), MOE_DTYPE_BF16 or MOE_DTYPE_MXFP4 (both require
 *              bf16 activations)
 *   score_fn   enum moe_score_fn
 *   n_group, topk_group  group-limited selection ([SF1033] Router table, row
 *              select: DeepSeek-V3's group-limited top-k): experts are split
 *              into n_group equal contiguous groups, the topk_group groups
 *              with the largest sum of their two largest selection values are
 *              kept, top-K is taken over the kept experts.  1, 1 = plain top-K.
 *   norm_topk_prob  1: renormalise the K gathered scores by their sum
 *              (+1e-20); 0: use them as they are ([SF1033] Router table, row
 *              routing_weights).
 *   route_scale  multiplies every routed weight (routed_scaling_factor);
 *              never the shared expert.
 *   swiglu_limit  clamp of the SwiGLU activation of routed AND shared
 *              experts: h = silu(min(g, L)) * min(max(u, -L), L).  +INFINITY
 *              disables the clamp ([SF1073] DeepSeek-V4 family commit note).
 *   shared_I   intermediate size of the shared expert; 0 = none.
 *   shared_gated  1: the shared expert is scaled by sigmoid(x . sh_gate)
 *              ([SGL48763], [SF941]); 0: ungated ([SF1073]).
 *   activation enum moe_activation, for routed and shared experts alike.
 *              Both kinds take w_gate_up's gate rows first, then its up rows
 *              (a checkpoint that interleaves them is de-interleaved once when
 *              the weights are laid out).
 *   mx_gemm    enum moe_mx_gemm (MXFP4 experts only; ignored otherwise).
 */
typedef struct moe_config {
  int32_t T, H, E, I, K;
  int32_t act_dtype;
  int32_t w_dtype;
  int32_t score_fn;
  int32_t n_group;
  int32_t topk_group;
  int32_t norm_topk_prob;
  float route_scale;
  float swiglu_limit;
  int32_t shared_I;
  int32_t shared_gated;
  int32_t activation;
  int32_t mx_gemm;
} moe_config;

/*
 * Weights of the layer (device pointers; NULL = absent where allowed).
 *
 *   gate_w       [E, H] act_dtype: the router's linear gate.
 *   router_bias  [E] f32, nullable: added to the fp32 logits (moves selection
 *                AND weights; the logit-bias variant, [SF941] "What").
 *   expert_bias  [E] f32, nullable: added to the scores for selection only;
 *                the weights are gathered from the unshifted scores
 *                ([SF1073] expert-bias and select commit notes).
 *   w_gate_up    F32/BF16: [E, 2I, H]; rows [0, I) are the gate projection,
 *                rows [I, 2I) the up projection of each expert (the stacked
 *                gate_up_proj of [SF1073], output-major like nn.Linear).
 *                MXFP4: uint8 codes [E, 2I, H/2], input 2j in the low nibble
 *                of byte j, input 2j+1 in the high nibble ([SF1073], [MI143]).
 *   w_down       F32/BF16: [E, H, I].  MXFP4: uint8 codes [E, H, I/2].
 *   w_gate_up_scale  MXFP4 only: uint8 E8M0 [E, 2I, H/32], scale of inputs
 *                32j..32j+31 is 2^(s-127).
 *   w_down_scale MXFP4 only: uint8 E8M0 [E, H, I/32].
 *   b_gate_up    [E, 2I] act_dtype, nullable: per-expert bias added to the
 *                gate/up pre-activations (gpt-oss-style experts, [MI143]).
 *   b_down       [E, H] act_dtype, nullable: per-expert bias of the down
 *                projection.
 *   sh_gate_up   [2*shared_I, H] act_dtype (same row split as w_gate_up).
 *   sh_down      [H, shared_I] act_dtype.
 *   sh_gate      [H] act_dtype: required iff shared_gated.
 */
typedef struct moe_weights {
  const void *gate_w;
  const float *router_bias;
  const float *expert_bias;
  const void *w_gate_up;
  const void *w_down;
  const uint8_t *w_gate_up_scale;
  const uint8_t *w_down_scale;
  const void *b_gate_up;
  const void *b_down;
  const void *sh_gate_up;
  const void *sh_down;
  const void *sh_gate;
} moe_weights;

/*
 * Checks a configuration without touching any GPU.  Returns MOE_OK,
 * MOE_ERR_INVALID (T < 0; H, E, I or K <= 0; K > E; n_group < 1; E not a
 * multiple of n_group; topk_group outside [1, n_group]; group size < 2 with
 * n_group > 1; K > topk_group * E / n_group; unknown dtype or score_fn;
 * route_scale not finite; swiglu_limit NaN or negative; shared_I < 0;
 * unknown activation) or
 * MOE_ERR_UNSUPPORTED (E > MOE_MAX_EXPERTS, K > MOE_MAX_TOPK,
 * n_group > MOE_MAX_GROUPS, H, I or shared_I not a multiple of 32, a dtype
 * pairing other than f32/f32, bf16/bf16, bf16/mxfp4).
 */
MOE_API int moe_validate(const moe_config *cfg);

/* Bytes of device workspace moe_route / moe_ffn_forward need for `cfg`
 * (written to *bytes).  Host only; validates cfg first. */
MOE_API int moe_workspace_bytes(const moe_config *cfg, size_t *bytes);

/*
 * Router only ([SF1033] "Router" section: forward returns scores, indices,
 * weights):
 *   x        [T, H] act_dtype
 *   gate_w, router_bias, expert_bias  as in moe_weights
 *   scores   [T, E] f32 out: the UNSHIFTED scores (softmax / sigmoid /
 *            sqrt-softplus of the fp32 logits)
 *   indices  [T, K] int32 out: the selected experts, largest selection value
 *            first, equal values to the lower expert id
 *   weights  [T, K] f32 out: routing weights in the order of `indices`
 *   counts   [E] int32 out, nullable: slots routed to each expert
 * All of scores, indices, weights are required.
 */
MOE_API int moe_route(const moe_config *cfg, const void *x, const void *gate_w,
              const float *router_bias, const float *expert_bias, float *scores,
              int32_t *indices, float *weights, int32_t *counts, void *workspace,
              size_t workspace_bytes, void *stream);

/*
 * Whole layer forward:
 *   out[t] = sum_k weights[t,k] * expert_{indices[t,k]}(x[t])
 *            + gamma_t * shared(x[t])
 * with expert_e(x) = down_e(swiglu_L(gate_up_e(x) [+ b_gate_up_e])) [+ b_down_e]
 * and gamma_t = sigmoid(x[t] . sh_gate) (gated) or 1 (ungated).
 *   x     [T, H] act_dtype, not modified
 *   out   [T, H] act_dtype; must not overlap x (the shared expert reads the
 *         unmodified input, [SGL48763] CUDA-fix commit note)
 *   scores, indices, weights, counts: as in moe_route, each nullable (the
 *         router results then stay in the workspace).
 * Accumulation is fp32 throughout; with bf16 activations the SwiGLU output is
 * rounded to bf16 before the down projection and `out` is rounded once.
 */
MOE_API int moe_ffn_forward(const moe_config *cfg, const void *x, const moe_weights *w,
                    void *out, float *scores, int32_t *indices, float *weights,
                    int32_t *counts, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * Forward without allocation, for callers that cannot allocate device memory
 * or pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The same layer as moe_ffn_forward, with
 * the same arguments except the workspace: its scratch memory is a fixed
 * array of MOE_NOALLOC_SCRATCH_BYTES that the library holds in device memory,
 * one per GPU it runs on, until the process ends.
 *   - Returns MOE_ERR_WORKSPACE (with moe_last_error() text) when cfg needs
 *     more scratch than that (moe_workspace_bytes(cfg) > the maximum; at
 *     T = 72 every workload of this layer family fits; larger batches use
 *     moe_ffn_forward).
 *   - Calls no allocating routine (no hipMalloc / hipFree); the first call on
 *     a device looks up that device's copy of the array.
 *   - Every call on one GPU uses that GPU's one array: calls that overlap in
 *     time on one GPU (different streams, threads or processes sharing a
 *     context) race and give undefined results; order them on one stream.
 *     Nothing in the array needs to start at zero, so the contents left by
 *     an earlier call do not matter.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

MOE_API int moe_ffn_forward_noalloc(const moe_config *cfg, const void *x, const moe_weights *w,
                                    void *out, float *scores, int32_t *indices, float *weights,
                                    int32_t *counts, void *stream);

/*
 * Load-balancing state ([SF1073] commit notes on tokens_per_expert, on
 * MoEBalancing and on update_expert_bias).
 *
 * moe_balance_count adds one forward's kept slots to the running counts:
 *   tokens_per_expert[e] += #{(t, k) : indices[t,k] = e and token_mask[t] != 0}
 *   indices            [T, K] int32 (e.g. the `indices` output of a forward);
 *                      ids outside [0, E) are not counted
 *   token_mask         [T] uint8, nullable (NULL keeps every token): the
 *                      per-token kept flag (moe_token_mask)
 *   tokens_per_expert  [E] int64, accumulated in place (integer adds; the
 *                      result does not depend on their order)
 * T = 0 enqueues nothing.  MOE_ERR_INVALID for T < 0, K or E <= 0, a NULL or
 * misaligned pointer; MOE_ERR_UNSUPPORTED for E > MOE_MAX_EXPERTS.
 */
MOE_API int moe_balance_count(const int32_t *indices, const uint8_t *token_mask, int32_t T,
                              int32_t K, int32_t E, int64_t *tokens_per_expert, void *stream);

/*
 * moe_balance_update ends a balancing step on the pooled counts c = the
 * current tokens_per_expert [E]:
 *   step_balance[0] = E * max(c) / sum(c) as fp32 (evaluated in fp64; 1 when
 *                     sum(c) = 0): 1 for a uniform load, E / K when the load
 *                     has collapsed onto K experts; nullable
 *   expert_bias[e] += rate * (s_e - sum(s) / E), s_e = sign(sum(c) - E * c_e)
 *                     (the DeepSeek-V3 sign step: underloaded experts go up,
 *                     overloaded ones down; the delta has zero mean); fp32 in
 *                     that order, no fused multiply-add; skipped when
 *                     bias_update_rate is 0 (a loaded bias stays fixed), and
 *                     expert_bias may then be NULL
 *   tokens_per_expert[e] = 0 afterwards.
 * Pooling counts across ranks (an all-reduce) is the caller's, before this
 * call.  MOE_ERR_INVALID for E <= 0, a non-finite rate, a NULL or misaligned
 * required pointer; MOE_ERR_UNSUPPORTED for E > MOE_MAX_EXPERTS.
 */
MOE_API int moe_balance_update(int64_t *tokens_per_expert, float *expert_bias, int32_t E,
                               float bias_update_rate, float *step_balance, void *stream);

/*
 * Backward of the layer ([SF1033] "Router" section: forward returns scores,
 * indices, weights, and the MoE FFN trains; [SF1073] commit note on the V4.1
 * port: the output and every gradient are compared; the expert bias shifts
 * the picks, never the weights).
 *
 * Gradients of sum(out * dout) for the forward of `cfg` at (x, w), with the
 * selection held at the forward's `indices` (it is piecewise constant; the
 * selection-only expert_bias gets no gradient) and the routing weights taken
 * from the forward's unshifted `scores`:
 *   x, w     as in moe_ffn_forward (w_dtype f32 or bf16; MXFP4 experts are
 *            MOE_ERR_UNSUPPORTED here)
 *   dout     [T, H] act_dtype
 *   scores   [T, E] f32, indices [T, K] int32: the forward's outputs
 *   g        gradient outputs, all f32, overwritten (not accumulated):
 *            dx [T,H] (when T > 0), dgate [E,H], dw_gate_up [E,2I,H],
 *            dw_down [E,H,I] required; drouter_bias [E] iff w->router_bias; db_gate_up
 *            [E,2I] and db_down [E,H] iff the expert biases are given;
 *            dsh_gate_up [2Is,H], dsh_down [H,Is] iff a shared expert;
 *            dsh_gate [H] iff it is gated.  Experts with no slot get zeros.
 * Arithmetic is fp32 (inputs widened exactly), fixed summation orders: the
 * result is bitwise reproducible.  Workspace: moe_backward_workspace_bytes.
 */
typedef struct {
  float *dx;
  float *dgate;
  float *drouter_bias;
  float *dw_gate_up;
  float *dw_down;
  float *db_gate_up;
  float *db_down;
  float *dsh_gate_up;
  float *dsh_down;
  float *dsh_gate;
} moe_grads;

MOE_API int moe_backward_workspace_bytes(const moe_config *cfg, size_t *bytes);

MOE_API int moe_ffn_backward(const moe_config *cfg, const void *x, const moe_weights *w,
                             const void *dout, const float *scores, const int32_t *indices,
                             const moe_grads *g, void *workspace, size_t workspace_bytes,
                             void *stream);

/* Static text for a status code. */
MOE_API const char *moe_status_string(int status);

/* Thread-local description of the last non-OK status on this thread
 * ("" if none). */
MOE_API const char *moe_last_error(void);

/*
 * Measurement hook.  Stages of moe_ffn_forward, in launch order: */
enum moe_stage {
  MOE_STAGE_ROUTER_LOGITS = 0,   /* fp32 router logits                         */
  MOE_STAGE_ROUTER_SELECT = 1,   /* score, select, routing weights             */
  MOE_STAGE_PERMUTE = 2,         /* counts, offsets, slot <-> row maps         */
  MOE_STAGE_GATE_UP = 3,         /* routed gate_up GEMM + SwiGLU               */
  MOE_STAGE_SHARED_GATE_UP = 4,  /* shared-expert gate_up GEMM + SwiGLU; no
                                    kernel of its own (an empty interval)
                                    where its items run in the routed gate_up
                                    launch: bf16 weights and activations,
                                    T < 256                                   */
  MOE_STAGE_DOWN = 5,            /* routed down GEMM                           */
  MOE_STAGE_SHARED_DOWN = 6,     /* shared-expert down GEMM                    */
  MOE_STAGE_COMBINE = 7,         /* weighted combine (+ shared expert)         */
  MOE_NUM_STAGES = 8
};
/*
 * Arms (stage >= 0) or disarms (stage < 0) event recording on the calling
 * thread: the i-th subsequent moe_ffn_forward call on this thread records
 * start_events[i % n_events] and stop_events[i % n_events] around the stage.
 * Stages whose work is one kernel (MOE_STAGE_PERMUTE .. MOE_STAGE_COMBINE)
 * hand the pair to that kernel's launch (hipExtLaunchKernelGGL), so the GPU
 * records them at the kernel's own start and end; a stage that launches no
 * kernel in a call records the pair back to back.  The router stages record
 * them on the stream just before and after their kernels.  The events are
 * hipEvent_t handles (passed as void*) created and owned by the caller; the
 * arrays must stay valid while armed.  Arming resets the call counter.
 */
MOE_API int moe_profile_stage(int stage, void *const *start_events, void *const *stop_events,
                              int n_events);

/* MOE_FFN_ABI_VERSION of the built library. */
MOE_API int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
