// Router and cohort planner kernels (gfx950) and their C-ABI entry points.
//
// Router: one wavefront per token.  Each lane holds E/64 logits; top-k is k
// rounds of a wave-wide maximum of 32-bit order-preserving keys whose six
// exchange steps are DPP quad permutes and row mirrors inside 16-lane rows
// and v_permlane16/32_swap across rows; ties on the logit go to the lower
// expert id through ballots of the lanes holding the maximum.  The winner
// of round j is known to every lane, so the softmax denominator of the kept
// logits accumulates in j order without any further exchange.  The router
// is the first of the three named parts of the per-token MoE cost (page
// "perf(moe): attribute the MoE decode gap at the M = 1 expert gather",
// Proposed Solution step 2).
//
// Planner: one workgroup.  Up to 64 slots, one wave does it all without a
// barrier (ballot-ranked peers, one DPP wave scan).  Beyond that, an LDS
// histogram of expert ids, a block-wide exclusive scan into per-expert
// offsets and the list of distinct experts, then a stable scatter of slot
// ids into per-expert lists by one wave in slot order.  Both write one
// 16-byte work record per distinct expert.  This is the cross-cohort deduplication of page
// "perf(moe): batched decode scales 1.55x against 3.25x on dense" (Proposed
// Solution, second bullet): the expert kernels walk the distinct experts, so
// each expert's weights are read once per step whatever the number of
// (token, k) slots routed to it.
//
// moe_route_plan runs both in one workgroup when the batch is small, so the
// indices stay in LDS and one launch disappears from the step.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>

#include "device_util.h"
#include "moe_internal.h"
#include "route_device.h"

namespace moe {

template <int PER_LANE>
__global__ __launch_bounds__(kBlock) void route_topk_kernel(const float *__restrict__ logits,
                                                            int n_tokens, int n_experts, int top_k,
                                                            int *__restrict__ topk_idx,
                                                            float *__restrict__ topk_w) {
    const int t = blockIdx.x * (kBlock / kWave) + (threadIdx.x / kWave);
    if (t >= n_tokens) return;  // uniform per wave
    const int lane = threadIdx.x & (kWave - 1);
    int id;
    float w;
    if (route_token<PER_LANE>(logits + (size_t)t * n_experts, n_experts, top_k, &id, &w)) {
        topk_idx[(size_t)t * top_k + lane] = id;
        topk_w[(size_t)t * top_k + lane] = w;
    }
}

// Small plans (<= 64 slots) run on one wave; larger ones on NT threads:
// 256, or 1024 from kPlanWideSlots slots on (the scatter's waves each walk
// one range of the slots, so more waves shorten it).
constexpr int kPlanWideSlots = 1024;

template <int PER_LANE, int NT>
__global__ __launch_bounds__(NT) void expert_plan_kernel(const int *__restrict__ topk_idx, int n_slots,
                                                         int n_experts, PlanOut p) {
    if (n_slots <= kWave) {
        __shared__ int cnt[MOE_MAX_EXPERTS], off[MOE_MAX_EXPERTS], uix[MOE_MAX_EXPERTS];
        if (threadIdx.x < kWave) plan_wave_small<PER_LANE>(topk_idx, n_slots, n_experts, p, cnt, off, uix);
    } else {
        plan_block<NT>(topk_idx, n_slots, n_experts, p);
    }
}

// Router and planner in one workgroup: its waves (up to 16) route the
// tokens, the indices are kept in LDS (and written out), then one wave (up
// to 64 slots) or the whole block plans them.
constexpr int kRoutePlanThreads = 1024;

template <int PER_LANE>
__global__ __launch_bounds__(kRoutePlanThreads) void route_plan_kernel(const float *__restrict__ logits, int n_tokens,
                                                            int n_experts, int top_k,
                                                            int *__restrict__ topk_idx,
                                                            float *__restrict__ topk_w, PlanOut p) {
    __shared__ int idx_lds[kRoutePlanMaxSlots];
    const int lane = threadIdx.x & (kWave - 1);
    const int n_waves = blockDim.x / kWave;
    for (int t = threadIdx.x / kWave; t < n_tokens; t += n_waves) {  // one wave per token
        int id;
        float w;
        if (route_token<PER_LANE>(logits + (size_t)t * n_experts, n_experts, top_k, &id, &w)) {
            topk_idx[(size_t)t * top_k + lane] = id;
            topk_w[(size_t)t * top_k + lane] = w;
            idx_lds[t * top_k + lane] = id;
        }
    }
    __syncthreads();
    const int n_slots = n_tokens * top_k;
    if (n_slots <= kWave) {  // launched with one wave per token
        __shared__ int cnt[MOE_MAX_EXPERTS], off[MOE_MAX_EXPERTS], uix[MOE_MAX_EXPERTS];
        if (threadIdx.x < kWave) plan_wave_small<PER_LANE>(idx_lds, n_slots, n_experts, p, cnt, off, uix);
    } else {                 // launched with kRoutePlanThreads threads
        plan_block<kRoutePlanThreads>(idx_lds, n_slots, n_experts, p);
    }
}

static PlanOut plan_out(const moe_plan_t *plan) {
    return PlanOut{plan->counts, plan->offsets, plan->sorted_slots, plan->unique_experts,
                   plan->n_unique, (int4 *)plan->work};
}

}  // namespace moe

using namespace moe;

#define MOE_PER_LANE_SWITCH(P, STMT) \
    switch (P) {                     \
        case 1: { constexpr int PL = 1; STMT; } break;  \
        case 2: { constexpr int PL = 2; STMT; } break;  \
        case 4: { constexpr int PL = 4; STMT; } break;  \
        case 8: { constexpr int PL = 8; STMT; } break;  \
        default: { constexpr int PL = 16; STMT; } break; \
    }

extern "C" moe_status moe_route_topk(const float *logits, int32_t n_tokens, int32_t n_experts,
                                     int32_t top_k, int32_t *topk_idx, float *topk_w,
                                     void *hip_stream) {
    const moe_status st = check_route_args(logits, n_tokens, n_experts, top_k, topk_idx, topk_w);
    if (st != MOE_OK) return st;
    if (n_tokens == 0) return MOE_OK;
    hipStream_t stream = (hipStream_t)hip_stream;
    const dim3 grid((n_tokens + kBlock / kWave - 1) / (kBlock / kWave));
    MOE_PER_LANE_SWITCH(per_lane_bucket(n_experts),
                        hipLaunchKernelGGL(route_topk_kernel<PL>, grid, dim3(kBlock), 0, stream, logits,
                                           n_tokens, n_experts, top_k, topk_idx, topk_w))
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

extern "C" moe_status moe_expert_plan(const int32_t *topk_idx, int32_t n_tokens, int32_t n_experts,
                                      int32_t top_k, const moe_plan_t *plan, void *hip_stream) {
    const moe_status st = check_plan_args(topk_idx, n_tokens, n_experts, top_k, plan);
    if (st != MOE_OK) return st;
    hipStream_t stream = (hipStream_t)hip_stream;
    const int n_slots = n_tokens * top_k;
    if (n_slots >= kPlanWideSlots) {
        MOE_PER_LANE_SWITCH(per_lane_bucket(n_experts),
                            hipLaunchKernelGGL((expert_plan_kernel<PL, 1024>), dim3(1), dim3(1024), 0, stream,
                                               topk_idx, n_slots, n_experts, plan_out(plan)))
    } else {
        MOE_PER_LANE_SWITCH(per_lane_bucket(n_experts),
                            hipLaunchKernelGGL((expert_plan_kernel<PL, kBlock>), dim3(1),
                                               dim3(n_slots <= kWave ? kWave : kBlock), 0, stream, topk_idx, n_slots,
                                               n_experts, plan_out(plan)))
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

extern "C" moe_status moe_route_plan(const float *logits, int32_t n_tokens, int32_t n_experts,
                                     int32_t top_k, int32_t *topk_idx, float *topk_w,
                                     const moe_plan_t *plan, void *hip_stream) {
    moe_status st = check_route_args(logits, n_tokens, n_experts, top_k, topk_idx, topk_w);
    if (st != MOE_OK) return st;
    st = check_plan_args(topk_idx, n_tokens, n_experts, top_k, plan);
    if (st != MOE_OK) return st;
    hipStream_t stream = (hipStream_t)hip_stream;
    if ((int64_t)n_tokens * top_k > kRoutePlanMaxSlots || n_tokens > kRoutePlanMaxTokens) {
        // large batches: the two kernels, the same results
        st = moe_route_topk(logits, n_tokens, n_experts, top_k, topk_idx, topk_w, hip_stream);
        if (st != MOE_OK) return st;
        return moe_expert_plan(topk_idx, n_tokens, n_experts, top_k, plan, hip_stream);
    }
    // one wave per token (at most 16); the block planner takes all 1024 threads
    const int n_slots = n_tokens * top_k;
    const int max_waves = kRoutePlanThreads / kWave;
    const int threads = n_slots <= kWave ? kWave * (n_tokens < max_waves ? (n_tokens > 0 ? n_tokens : 1) : max_waves)
                                         : kRoutePlanThreads;
    MOE_PER_LANE_SWITCH(per_lane_bucket(n_experts),
                        hipLaunchKernelGGL(route_plan_kernel<PL>, dim3(1), dim3(threads), 0, stream, logits,
                                           n_tokens, n_experts, top_k, topk_idx, topk_w, plan_out(plan)))
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}
