/*
 * moe_decode.h -- C ABI of the decode-time quantized-expert MoE block for
 * AMD Instinct MI355X (gfx950).
 *
 * One decode step of one MoE layer is three calls on one HIP stream:
 *
 *   moe_route_topk   router: top-k experts per token and their weights
 *   moe_expert_plan  cohort plan: slots grouped by expert, distinct experts
 *   moe_decode_step  expert block: fused gate+up, SiLU*up, down projection,
 *                    weighted combine over k per token
 *
 * The pages this follows describe the problem, not an API: a router yields
 * per-token (expert, score) slots and is one named part of the decode cost
 * next to the expert gather and the combine (page "perf(moe): attribute the
 * MoE decode gap at the M = 1 expert gather", Proposed Solution, step 2);
 * routed experts are gathered once per (token, k) slot at M = 1 (same page,
 * Problem / Background); page "perf(moe): batched decode scales 1.55x
 * against 3.25x on dense" proposes a token dimension with a sum over k per
 * token and deduplicating expert ids across the cohort so that each expert
 * plane is read once per step (Proposed Solution), keeps n_tokens a runtime
 * extent that must not re-specialise kernels, asks that unsupported
 * configurations decline rather than fail, and that shapes be validated
 * before dispatch (Implementation Notes).
 *
 * Conventions for every entry point:
 *   - Every array pointer is a DEVICE pointer unless stated otherwise; the
 *     caller owns all memory.  The library allocates nothing and keeps no
 *     per-call state.
 *   - Calls are asynchronous on `hip_stream` (a hipStream_t; NULL = the
 *     default stream).  No call synchronises the host with the device.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     bad argument returns MOE_ERR_INVALID_ARG, a shape or mode with no
 *     kernel returns MOE_ERR_UNSUPPORTED (the caller falls back), a short
 *     workspace returns MOE_ERR_WORKSPACE; nothing aborts.  A failed launch
 *     returns MOE_ERR_DEVICE.
 *   - Expert ids inside device arrays cannot be checked on the host.  The
 *     kernels never read or write out of bounds on a bad id: the planner
 *     leaves such slots out of every list and the combine writes NaN for
 *     a token that holds one.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_WORKSPACE = 3,
    MOE_ERR_DEVICE = 4
} moe_status;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype;

/* Storage of the down projection (see moe_layer_t and moe_pack_down). */
typedef enum { MOE_DOWN_ROWS = 0, MOE_DOWN_COLS = 1 } moe_down_layout;

/* Gated activation of the expert MLP (see moe_layer_t). */
typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_GEGLU = 1 } moe_activation;

/* Limits enforced by validation. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOP_K 16
/* Tokens per call of the expert entry points (one row of combine
 * workgroups per token). */
#define MOE_MAX_TOKENS 65535

/*
 * One MoE layer: stacked expert weights, affine, groups along the input
 * dimension ("4-bit group 64" checkpoints; page "perf(moe): batched decode
 * scales 1.55x against 3.25x on dense", Current Behavior).
 *
 *   w = scale * q + bias,  q in 0 .. 2^bits - 1
 *
 * `bits` (gate and up) and `down_bits` (down) are 4, 6 or 8, `group_size`
 * (all three) 32, 64 or 128: the fused kernel is templated on bits and
 * group size, and 4-bit gate/up with 6-bit down must keep working (same
 * page, Implementation Notes).  A weight matrix is stored as
 * [expert][out][in*bits/32] uint32 words, each row a little-endian bit
 * stream: element c sits in stream bits c*bits .. c*bits+bits-1, stream bit
 * j being bit j % 32 of word j / 32 (at 4 bits: element 8*w+i in nibble i
 * of word w, lowest nibble first).  Scales and biases are fp16 bit
 * patterns, [expert][out][in/group_size].
 *   gate, up : out = dff,    in = hidden
 *   down     : out = hidden, in = dff
 * Each projection picks its kernels by its own width: 4-bit gate and up in
 * groups of 64 run the specialised gate+up kernels (MFMA for large
 * batches), 4-bit down in groups of 64 the specialised down kernels (either
 * down layout); a projection of any other width or group size runs the
 * generic row kernels, and a down projection on them needs MOE_DOWN_ROWS.
 * Every `*_q` pointer must be 16-byte aligned, every scale/bias pointer
 * 4-byte aligned.  The struct itself lives in host memory; the pointers it
 * holds are device pointers.
 *
 * `down_layout` selects how the down projection is stored:
 *   MOE_DOWN_ROWS  as above: down_q [E][hidden][dff/8], scales [E][hidden][dff/64]
 *   MOE_DOWN_COLS  the same bytes regrouped by moe_pack_down so that one
 *                  16-byte chunk (32 consecutive dff inputs) of 64
 *                  consecutive hidden rows is contiguous:
 *                  down_q [E][dff/32][hidden] 16-byte chunks,
 *                  scales and biases [E][dff/64][hidden].
 *                  Needs hidden % 64 == 0 and dff % 128 == 0.
 *
 * `expert_scale` (optional, NULL = none) is one fp32 factor per expert that
 * multiplies the gate and up pre-activations (the expert-scale sidecars of
 * page "perf(moe): attribute ...", Problem / Background).  `clamp_limit`
 * (0 = none) clips gate and up pre-activations to [-L, L] after the sidecar
 * and before SiLU*up (the clamp stage named on the same page).
 *
 * `activation` is MOE_ACT_SWIGLU (h = silu(g) * u) or MOE_ACT_GEGLU
 * (h = gelu(g) * u with the tanh form 0.5 g (1 + tanh(sqrt(2/pi)
 * (g + 0.044715 g^3)))), the GeGLU variant of the fused kernel that page
 * "perf(moe): batched decode scales 1.55x against 3.25x on dense" lists
 * among its kernels (Implementation Notes); the pages give no GELU formula,
 * the tanh form is the one of the gemma checkpoints that kernel serves.
 * `down_scale` (optional, NULL = none) is one fp32 factor per expert that
 * multiplies that expert's down-projection output y before the weighted
 * combine: the second of the "both sidecars" that page "perf(moe):
 * attribute ..." names (Problem / Background), which it does not define
 * further.
 *
 * Field order: the fields through expert_scale are those of the plain
 * 4-bit layer, in that order; the extensions follow, and all-zero
 * extensions mean the plain layer (rows-layout down, no down scale,
 * SwiGLU, down projection as wide as gate and up), so a caller that only
 * knows the plain fields and zero-fills the rest gets the plain layer.
 */
typedef struct {
    int32_t hidden;      /* H, multiple of 64 */
    int32_t dff;         /* expert intermediate size F, multiple of 64 */
    int32_t n_experts;   /* E, 1..MOE_MAX_EXPERTS */
    int32_t top_k;       /* k, 1..min(E, MOE_MAX_TOP_K) */
    int32_t bits;        /* 4, 6 or 8 (gate and up) */
    int32_t group_size;  /* 32, 64 or 128; divides hidden and dff */
    int32_t act_dtype;   /* moe_dtype of x, residual and out (int32, as wide as
                            the enum, so that any value is defined to read) */
    float clamp_limit;   /* >= 0; 0 disables the clamp */
    const uint32_t *gate_q, *up_q;
    const uint16_t *gate_s, *gate_b, *up_s, *up_b;
    const uint32_t *down_q;
    const uint16_t *down_s, *down_b;
    const float *expert_scale; /* [E] or NULL */
    /* extensions; zero = the plain layer */
    int32_t down_layout;       /* moe_down_layout */
    const float *down_scale;   /* [E] or NULL */
    int32_t activation;        /* moe_activation */
    int32_t down_bits;         /* 4, 6 or 8 (down projection); 0 = bits */
} moe_layer_t;

/*
 * Cohort plan of one step (all device arrays, int32, caller-allocated):
 *   counts[E]            slots routed to each expert
 *   offsets[E+1]         exclusive prefix sum of counts
 *   sorted_slots[B*k]    slot ids s = t*k + j grouped by expert, ascending
 *                        expert, ascending slot within an expert
 *   unique_experts[E]    distinct experts in ascending order, -1 after
 *   n_unique[1]          number of distinct experts
 *   work[E][4]           one 16-byte record per distinct expert u, in the
 *                        order of unique_experts: {expert, offsets[expert],
 *                        counts[expert], first slot of that expert}; after
 *                        the last distinct expert {-1, B*k, 0, 0}.  The
 *                        expert kernels read only this record before they
 *                        stream an expert's weights.  16-byte aligned.
 *                        Appended after the five plain arrays; it is
 *                        required (a plan without it is refused with
 *                        MOE_ERR_INVALID_ARG).
 */
typedef struct {
    int32_t *counts, *offsets, *sorted_slots, *unique_experts, *n_unique;
    int32_t *work;
} moe_plan_t;

/*
 * Router.  logits fp32 [n_tokens][n_experts] (finite) -> topk_idx int32
 * [n_tokens][top_k] in descending logit order, ties to the lower expert
 * id, and topk_w fp32 [n_tokens][top_k], the softmax of the kept logits
 * (equal to softmax over all experts, top-k, renormalise).
 * n_tokens == 0 returns MOE_OK without a launch.
 */
moe_status moe_route_topk(const float *logits, int32_t n_tokens, int32_t n_experts,
                          int32_t top_k, int32_t *topk_idx, float *topk_w,
                          void *hip_stream);

/*
 * Cohort planner: a stable counting sort of the n_tokens*top_k slots by
 * expert id and the list of distinct experts, so that each expert's
 * weights are streamed once per step for all the tokens routed to it.
 * Reads topk_idx int32 [n_tokens][top_k]; writes every array of `plan`
 * (a host struct of device pointers).  n_tokens == 0 writes an empty plan.
 */
moe_status moe_expert_plan(const int32_t *topk_idx, int32_t n_tokens, int32_t n_experts,
                           int32_t top_k, const moe_plan_t *plan, void *hip_stream);

/*
 * Router and planner of one step in a single launch (one workgroup, one
 * wave per token) when n_tokens <= 16; larger batches run the two kernels of
 * moe_route_topk and moe_expert_plan.  Same arguments and results as those
 * two calls.
 */
moe_status moe_route_plan(const float *logits, int32_t n_tokens, int32_t n_experts, int32_t top_k,
                          int32_t *topk_idx, float *topk_w, const moe_plan_t *plan,
                          void *hip_stream);

/*
 * Router projection, the step in front of the router: logits[t][e] =
 * sum_h x[t][h] * w_router[e][h] (the pages name the router as one of the
 * per-token decode costs: page "perf(moe): attribute the MoE decode gap at
 * the M = 1 expert gather", Proposed Solution step 2).
 *   x         [n_tokens][hidden], act_dtype (bf16 or fp32), 16-byte aligned
 *   w_router  bf16 bits [n_experts][hidden], 16-byte aligned
 *   logits    fp32 [n_tokens][n_experts], the router's input
 * Products exact, fp32 accumulation in a fixed order (a token's logits do
 * not depend on the rest of the batch).  MOE_ERR_UNSUPPORTED when hidden has
 * no lane geometry (hidden/8 must be a power of two up to 64 times 1..8),
 * n_experts > MOE_MAX_EXPERTS or n_tokens > MOE_MAX_TOKENS; n_tokens == 0
 * launches nothing.  Asynchronous on hip_stream.
 */
moe_status moe_router_logits(const void *x, int32_t n_tokens, int32_t hidden, moe_dtype act_dtype,
                             const uint16_t *w_router, int32_t n_experts, float *logits, void *hip_stream);

/* Bytes of device workspace moe_decode_step needs for up to max_tokens
 * tokens of this layer's shape (0 if the layer is invalid). */
size_t moe_workspace_size(const moe_layer_t *layer, int32_t max_tokens);

/*
 * Expert block of one step.
 *   x         [n_tokens][hidden], act_dtype
 *   topk_idx  int32 [n_tokens][top_k], topk_w fp32 [n_tokens][top_k]
 *   plan      the plan of topk_idx (host struct of device pointers)
 *   out       [n_tokens][hidden] act_dtype; must not alias x
 *   workspace device memory of at least moe_workspace_size(layer, n_tokens)
 *             bytes, 256-byte aligned; its contents need no initialisation
 *
 *   g = Wg[e] x_t, u = Wu[e] x_t   (fp32 accumulation)
 *   g, u *= expert_scale[e]        (if given)
 *   g, u = clip(g, u, -L, L)       (if clamp_limit > 0)
 *   h = silu(g) * u                (gelu(g) * u for MOE_ACT_GEGLU;
 *                                   fp32, never rounded)
 *   y = Wd[e] h                    (fp32)
 *   y *= down_scale[e]             (if given)
 *   o_t = sum_{j<k} topk_w[t][j] * y_{t,j}, in j order, rounded once to
 *         act_dtype (round to nearest even)
 *   out_t = o_t
 *
 * The fp32 partials with one final rounding follow page "perf(moe):
 * batched decode scales 1.55x against 3.25x on dense", Implementation
 * Notes.  Repeated calls are bitwise equal.  Batch invariance: below 16
 * tokens a token's result depends only on that token (bitwise the same
 * whatever else is in the batch).  From 16 tokens up, an expert that holds
 * 3 or more of the batch's tokens runs on the MFMA kernels, and from 128
 * tokens up every expert runs on the MFMA tile kernels; they add the same
 * exact fp32 products in another order, so a token routed to such an
 * expert may differ from its single-token result by fp32 rounding only
 * (relative L2 within 5e-4 of each other, both within the output
 * tolerance of the fp64 definition).  Between 16 and 127 tokens, tokens
 * whose experts all hold fewer than 3 tokens stay bitwise equal.
 */
moe_status moe_decode_step(const moe_layer_t *layer, const void *x, int32_t n_tokens,
                           const int32_t *topk_idx, const float *topk_w, const moe_plan_t *plan,
                           void *out, void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * moe_decode_step with the residual add of a layer stack fused into the
 * combine's store: out_t = act(residual_t + act(o_t)), i.e. the block's
 * output rounded to act_dtype as moe_decode_step stores it, added to the
 * residual in fp32 and rounded again (the layer stack runs every MoE
 * layer on every decode tick, page "perf(moe):
 * attribute the MoE decode gap at the M = 1 expert gather", Problem /
 * Background).  residual is [n_tokens][hidden] act_dtype or NULL (then
 * exactly moe_decode_step); out must not alias x or residual.
 */
moe_status moe_decode_step_residual(const moe_layer_t *layer, const void *x, int32_t n_tokens,
                                    const int32_t *topk_idx, const float *topk_w,
                                    const moe_plan_t *plan, const void *residual, void *out,
                                    void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * One layer step from router logits: moe_route_plan, then moe_decode_step,
 * with the same checks and results; topk_idx, topk_w and the plan are
 * outputs here (the plan as moe_route_plan writes it).
 *   logits  fp32 [n_tokens][n_experts], device
 * The pages split a decoded token's MoE time into router, expert GEMV and
 * combine (page "perf(moe): attribute the MoE decode gap at the M = 1
 * expert gather", Proposed Solution); at a few tokens each of those is a
 * short, latency-bound kernel.  So a batch of up to 8 tokens (with at most
 * 256 experts and n_tokens * top_k <= 64) takes two launches
 * instead of three or more: the gate+up workgroups select their own expert
 * from the logits and, with more than one token, deduplicate among
 * themselves so each distinct expert's gate and up rows are streamed once
 * for every token routed to it (one block also writes topk_idx, topk_w and
 * the plan); then one kernel does the down projection and the combine,
 * token by token.  Results are bitwise those of the longer path.
 */
moe_status moe_decode_layer(const moe_layer_t *layer, const float *logits, const void *x,
                            int32_t n_tokens, int32_t *topk_idx, float *topk_w,
                            const moe_plan_t *plan, const void *residual, void *out,
                            void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * The first half of moe_decode_layer: routes, plans and writes h into the
 * workspace (one launch for up to 8 tokens, else moe_route_plan and the
 * gate+up kernels); moe_expert_down_combine with the same workspace, plan,
 * topk_idx and topk_w is the second half.  Same checks as moe_decode_layer
 * (out and residual aside).
 */
moe_status moe_route_gate_up(const moe_layer_t *layer, const float *logits, const void *x,
                             int32_t n_tokens, int32_t *topk_idx, float *topk_w,
                             const moe_plan_t *plan, void *workspace, size_t workspace_bytes,
                             void *hip_stream);

/*
 * The two halves of moe_decode_step, for callers that instrument or overlap
 * the stages (the pages' fused decode kernel is likewise a gate/up kernel
 * followed by a down kernel: page "perf(moe): batched decode scales 1.55x
 * against 3.25x on dense", Current Behavior).  Same arguments, checks and
 * results as moe_decode_step; enqueue moe_expert_gate_up first, then
 * moe_expert_down_combine with the same workspace, on one stream.
 *   moe_expert_gate_up       writes h = silu(g) * u per slot into the workspace
 *   moe_expert_down_combine  reads h, writes out
 */
moe_status moe_expert_gate_up(const moe_layer_t *layer, const void *x, int32_t n_tokens,
                              const moe_plan_t *plan, void *workspace, size_t workspace_bytes,
                              void *hip_stream);
moe_status moe_expert_down_combine(const moe_layer_t *layer, int32_t n_tokens,
                                   const int32_t *topk_idx, const float *topk_w,
                                   const moe_plan_t *plan, const void *residual, void *out,
                                   void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * moe_decode_layer for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, checks and results as moe_decode_layer
 * (bitwise), without the workspace: the h and y intermediates live in a
 * device array of MOE_STATIC_SCRATCH_BYTES that the library reserves per
 * GPU when it is loaded and holds until the process ends.
 *   - MOE_ERR_WORKSPACE when moe_workspace_size(layer, n_tokens) exceeds
 *     MOE_STATIC_SCRATCH_BYTES (8 MiB: up to 93 tokens of the 2048 x 768
 *     top-8 layer).
 *   - hip_stream must belong to the current device (else
 *     MOE_ERR_INVALID_ARG).  The first call on a device looks up the
 *     array's device address; make that call outside graph capture.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (nothing in it needs clearing: each step writes h
 *     and y before reading them).  Calls that may overlap on one GPU (other
 *     streams, other host threads) race on it: serialise them.
 * Calls no hipMalloc, hipFree or other allocating routine.
 */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)8 << 20)
moe_status moe_decode_layer_static(const moe_layer_t *layer, const float *logits, const void *x,
                                   int32_t n_tokens, int32_t *topk_idx, float *topk_w,
                                   const moe_plan_t *plan, const void *residual, void *out,
                                   void *hip_stream);

/*
 * Regroup a layer's down projection from MOE_DOWN_ROWS (as stored by the
 * pages' 4-bit checkpoints) to MOE_DOWN_COLS, the layout the decode kernels
 * read fastest: a wave then reads 64 consecutive output rows with one
 * coalesced 1 KiB load per 32 inputs.  A one-time, load-time step; pure byte
 * movement, nothing is re-quantised.  `layer` describes the source
 * (down_layout must be MOE_DOWN_ROWS; 4-bit weights in groups of 64 only,
 * other formats return MOE_ERR_UNSUPPORTED); dst_q (16-byte aligned, E*hidden*dff/2
 * bytes), dst_s and dst_b (E*hidden*dff/64 fp16 each) are device buffers that
 * must not overlap the source.  Asynchronous on hip_stream.
 */
moe_status moe_pack_down(const moe_layer_t *layer, uint32_t *dst_q, uint16_t *dst_s, uint16_t *dst_b,
                         void *hip_stream);

/* Host-only check of a layer descriptor (no device access):
 * MOE_OK, MOE_ERR_INVALID_ARG or MOE_ERR_UNSUPPORTED. */
moe_status moe_layer_check(const moe_layer_t *layer);

/* Static description of a status code. */
const char *moe_status_str(moe_status status);

/* ABI version: bumped when a signature or struct changes (8: plain field
 * order of moe_layer_t, moe_decode_step without a residual,
 * moe_decode_step_residual). */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
