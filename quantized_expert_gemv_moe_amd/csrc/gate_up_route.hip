// The few-token routing gate+up kernel and moe_route_gate_up (gfx950).
//
// Up to 8 tokens, a step's router, planner and gate+up run in one launch:
// block 0 routes and plans for the API's outputs while every other wave
// selects its own expert from the logits and streams that expert's rows;
// with more than one token the waves deduplicate among themselves so each
// distinct expert is read once.  Larger batches, or layers outside its
// limits, take moe_route_plan and the batched gate+up kernels.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>

#include "device_util.h"
#include "expert_device.h"
#include "gate_up_device.h"
#include "moe_internal.h"
#include "route_device.h"

namespace moe {

// A small batch (up to BW tokens), routed here, on a 1-D grid of BW-wave
// blocks.  Block 0 routes every token in full, one wave per token, and
// writes topk_idx, topk_w and the plan, exactly as moe_route_plan would.
// Every other wave computes rows of one (token t, rank j) pair's expert e,
// which it finds from the logits itself (j + 1 selection rounds) instead of
// waiting for a router launch and a plan.
//
// One token (no DEDUP): every wave is one item (t, j, row block) and runs
// the selection rounds itself; the low ranks' weight loads go out first.
//
// More tokens (DEDUP): the items deduplicate among themselves, so each
// distinct expert's rows are streamed once per step (the cohort dedup of
// page "perf(moe): batched decode scales 1.55x against 3.25x on dense",
// Proposed Solution).  A block holds BW row blocks of one (t, j) pair:
// wave t selects e and shares it through LDS; then wave n ranks e among
// token n's experts (the number the router places before it), which says
// whether token n holds e and as which slot.  If a lower token holds e, the
// pair of that token owns the rows and this block exits; the owner computes
// them for every token holding e, in token order, from one register copy
// of the weights.  Sharing the selection and the tests across the block
// keeps the per-wave VALU work at that of the one-token kernel; with many
// items in flight this kernel's time follows the VALU issue and the number
// of waves in flight (95 registers: five waves per SIMD).
//
// The arithmetic per row and token is gate_up_kernel's, so h is bitwise the
// same as on the batched path and the same for a token alone.
constexpr int kRouteMaxTokens = 8;

template <int LPR, int NV, int RI, bool XBF16, int PL, int BW, bool DEDUP>
__global__ __launch_bounds__(BW * kWave) void gate_up_route_kernel(
    GateUpArgs a, const float *__restrict__ logits, int *__restrict__ topk_idx, float *__restrict__ topk_w,
    PlanOut p, int row_blocks, int n_tokens) {
    constexpr int RPI = kWave / LPR;
    constexpr int ROWS_WG = RPI * RI;
    constexpr int EP = kWave * PL;  // experts covered by the router lanes (>= n_experts)
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int sl = lane % LPR;
    const int E = a.n_experts, k = a.top_k;
    if (blockIdx.x == 0) {
        __shared__ int idx_lds[kWave];  // n_tokens * top_k <= 64
        __shared__ int cnt[EP], off[EP], uix[EP];
        if (wave < n_tokens) {
            int id;
            float wt;
            if (route_token<PL>(logits + (size_t)wave * E, E, k, &id, &wt)) {
                topk_idx[wave * k + lane] = id;
                topk_w[wave * k + lane] = wt;
                idx_lds[wave * k + lane] = id;
            }
        }
        __syncthreads();
        if (wave == 0) plan_wave_small<PL>(idx_lds, n_tokens * k, E, p, cnt, off, uix);
        return;
    }
    if constexpr (!DEDUP) {
        const int item = (blockIdx.x - 1) * BW + wave;
        if (item >= n_tokens * k * row_blocks) return;
        const int rb = item % row_blocks, j = (item / row_blocks) % k, t = item / (row_blocks * k);
        const int row0 = rb * ROWS_WG + lane / LPR;
        uint4 xraw0[XBF16 ? NV : 1][4];
        if constexpr (XBF16) {
#pragma unroll
            for (int v = 0; v < NV; ++v)
                load_x32_bf16((const uint16_t *)a.x, (size_t)t * a.hidden, (v * LPR + sl) * 32, xraw0[v]);
        }
        const int e = route_rank<PL>(logits + (size_t)t * E, E, j);
        GateUpRows<RI, NV> w;
        load_gate_up_rows<LPR, NV, RI, XBF16>(a, e, row0, sl, w);
        const float sc = a.expert_scale ? a.expert_scale[e] : 1.f;
        GateUpX<LPR, NV, XBF16> x;
        load_gate_up_x<LPR, NV, XBF16>(a, t, sl, x, XBF16 ? xraw0 : nullptr);
        gate_up_token_rows<LPR, NV, RI, XBF16>(a, w, x, t * k + j, row0, sc, a.clamp_limit);
    } else {
        // block -> (pair (t, j), group of BW row blocks); wave -> row block
        const int rbb_n = (row_blocks + BW - 1) / BW;
        const int pair = (blockIdx.x - 1) / rbb_n;
        const int t = pair / k, j = pair - t * k;  // t < n_tokens <= BW by the grid
        const int rb = ((blockIdx.x - 1) - pair * rbb_n) * BW + wave;
        const int row0 = rb * ROWS_WG + lane / LPR;
        uint4 xraw0[XBF16 ? NV : 1][4];
        if constexpr (XBF16) {
#pragma unroll
            for (int v = 0; v < NV; ++v)
                load_x32_bf16((const uint16_t *)a.x, (size_t)t * a.hidden, (v * LPR + sl) * 32, xraw0[v]);
        }
        __shared__ int e_lds;
        __shared__ int rank_lds[BW];
        // wave n < n_tokens holds token n's order keys; wave t selects e
        uint32_t kw[PL];
        const int kn = wave < n_tokens ? wave : n_tokens - 1;
        route_keys<PL>(logits + (size_t)kn * E, E, kw);
        if (wave == t) {
            uint32_t own[PL];
#pragma unroll
            for (int q = 0; q < PL; ++q) own[q] = kw[q];
            int sel = 0;
            for (int r = 0; r <= j; ++r) {
                uint32_t best;
                sel = route_take<PL>(own, &best);
            }
            if (lane == 0) e_lds = sel;
        }
        __syncthreads();
        const int e = __builtin_amdgcn_readfirstlane(e_lds);
        if (wave < n_tokens) {
            const int r = route_rank_of<PL>(kw, e);
            if (lane == 0) rank_lds[wave] = r;
        }
        __syncthreads();
        if (rb >= row_blocks) return;
        // tokens holding e (a bit each) and the rank of e in each (4 bits each)
        uint32_t held = 0, ranks = 0;
        for (int n = 0; n < n_tokens; ++n) {
            const int r = rank_lds[n];
            if (r < k) {
                held |= 1u << n;
                ranks |= (uint32_t)r << (4 * n);
            }
        }
        if (held & ((1u << t) - 1u)) return;  // a lower token's pair owns e's rows
        GateUpRows<RI, NV> w;
        load_gate_up_rows<LPR, NV, RI, XBF16>(a, e, row0, sl, w);
        const float sc = a.expert_scale ? a.expert_scale[e] : 1.f;
        uint32_t more = held & ~((2u << t) - 1u);  // the higher tokens holding e
        GateUpX<LPR, NV, XBF16> x;
        load_gate_up_x<LPR, NV, XBF16>(a, t, sl, x, XBF16 ? xraw0 : nullptr);
        // the next token's activations go out before this token's rows are
        // computed (past the last token they repeat this one, unused)
        int tn = more ? __builtin_ctz(more) : t;
        uint4 xraw_n[XBF16 ? NV : 1][4];
        if constexpr (XBF16) {
#pragma unroll
            for (int v = 0; v < NV; ++v)
                load_x32_bf16((const uint16_t *)a.x, (size_t)tn * a.hidden, (v * LPR + sl) * 32, xraw_n[v]);
        }
        gate_up_token_rows<LPR, NV, RI, XBF16>(a, w, x, t * k + j, row0, sc, a.clamp_limit);
        while (more) {
            const int tc = tn;
            const int jc = (ranks >> (4 * tc)) & 15;
            more &= more - 1;
            // the weights as opaque values: the nibble unpacking then stays
            // inside the loop instead of being hoisted into ~128 registers
            // of loop-invariant bf16 pairs
            opaque_rows(w);
            load_gate_up_x<LPR, NV, XBF16>(a, tc, sl, x, XBF16 ? xraw_n : nullptr);
            tn = more ? __builtin_ctz(more) : tc;
            if constexpr (XBF16) {
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    load_x32_bf16((const uint16_t *)a.x, (size_t)tn * a.hidden, (v * LPR + sl) * 32, xraw_n[v]);
            }
            gate_up_token_rows<LPR, NV, RI, XBF16>(a, w, x, tc * k + jc, row0, sc, a.clamp_limit);
        }
    }
}

// The routing gate+up kernel of a one-token batch: a planner block, then
// row blocks x top_k.
template <int LPR, int NV>
static moe_status launch_gate_up_route(const GateUpArgs &a, bool bf16, int pl, const float *logits,
                                       int32_t *idx, float *w, const PlanOut &p, int n_tokens, hipStream_t s) {
    constexpr int RI = gate_up_ri<LPR, NV>();
    constexpr int rows = (kWave / LPR) * RI;
    const int row_blocks = (a.dff + rows - 1) / rows;
    const int items = n_tokens * a.top_k * row_blocks;
    // 4-wave blocks up to 4 tokens, 8-wave blocks beyond (measured best at
    // either end)
    const int bw = n_tokens <= 4 ? 4 : 8;
    // one token: items (t, j, row block) packed BW to a block; more tokens:
    // each block holds BW row blocks of one (t, j) pair
    const int blocks = n_tokens > 1 ? n_tokens * a.top_k * ((row_blocks + bw - 1) / bw) : (items + bw - 1) / bw;
    const dim3 grid(1 + blocks), block(bw * kWave);
#define MOE_GUR_D(PL, BW, D)                                                                                 \
    if (bf16)                                                                                                \
        hipLaunchKernelGGL((gate_up_route_kernel<LPR, NV, RI, true, PL, BW, D>), grid, block, 0, s, a, logits,  \
                           idx, w, p, row_blocks, n_tokens);                                                 \
    else                                                                                                     \
        hipLaunchKernelGGL((gate_up_route_kernel<LPR, NV, RI, false, PL, BW, D>), grid, block, 0, s, a, logits, \
                           idx, w, p, row_blocks, n_tokens);
#define MOE_GUR(PL, BW)            \
    if (n_tokens > 1) {            \
        MOE_GUR_D(PL, BW, true)    \
    } else {                       \
        MOE_GUR_D(PL, BW, false)   \
    }
    switch (pl * 10 + bw / 4) {
        case 11: MOE_GUR(1, 4) break;
        case 21: MOE_GUR(2, 4) break;
        case 41: MOE_GUR(4, 4) break;
        case 12: MOE_GUR(1, 8) break;
        case 22: MOE_GUR(2, 8) break;
        case 42: MOE_GUR(4, 8) break;
        default: return MOE_ERR_UNSUPPORTED;
    }
#undef MOE_GUR
#undef MOE_GUR_D
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_route_gate_up(const moe_layer_t *layer, const float *logits, const void *x,
                                        int32_t n_tokens, int32_t *topk_idx, float *topk_w,
                                        const moe_plan_t *plan, void *workspace, size_t workspace_bytes,
                                        void *hip_stream) {
    moe_status st = check_step(layer, n_tokens, plan, workspace, workspace_bytes);
    if (st != MOE_OK || n_tokens == 0) return st;
    if ((st = check_route_args(logits, n_tokens, layer->n_experts, layer->top_k, topk_idx, topk_w)) != MOE_OK)
        return st;
    if ((st = check_plan_args(topk_idx, n_tokens, layer->n_experts, layer->top_k, plan)) != MOE_OK) return st;
    if ((st = check_x(x)) != MOE_OK) return st;
    hipStream_t stream = (hipStream_t)hip_stream;
    const int pl = per_lane_bucket(layer->n_experts);
    if (!fast_gate_up(layer) || n_tokens > kRouteMaxTokens || pl > 4 || n_tokens * layer->top_k > kWave) {
        // router + planner launch, then the deduplicated gate+up
        st = moe_route_plan(logits, n_tokens, layer->n_experts, layer->top_k, topk_idx, topk_w, plan, hip_stream);
        if (st != MOE_OK) return st;
        st = enqueue_gate_up(layer, x, n_tokens, plan, workspace, stream);
    } else {  // a few tokens: one launch that routes for itself
        Geometry gu;
        pick_geometry_gate_up(layer->hidden, &gu);
        const Workspace ws = workspace_layout(layer, n_tokens);
        float *h = (float *)((char *)workspace + ws.h_off);
        const GateUpArgs ga{(const uint4 *)layer->gate_q, (const uint4 *)layer->up_q, layer->gate_s,
                            layer->gate_b, layer->up_s, layer->up_b, layer->expert_scale,
                            layer->clamp_limit, x, plan_view(plan), h, layer->hidden, layer->dff,
                            layer->n_experts, layer->top_k, n_tokens * layer->top_k, INT_MAX, layer->activation};
        const PlanOut po{plan->counts, plan->offsets, plan->sorted_slots, plan->unique_experts, plan->n_unique,
                         (int4 *)plan->work};
        MOE_GEOMETRY_SWITCH(gu, st, launch_gate_up_route, ga, layer->act_dtype == MOE_DTYPE_BF16, pl, logits,
                            topk_idx, topk_w, po, n_tokens, stream)
    }
    if (st != MOE_OK) return st;
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}
