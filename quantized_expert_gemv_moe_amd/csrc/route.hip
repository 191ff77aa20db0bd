// Router and cohort planner kernels (gfx950) and their C-ABI entry points.
//
// Router: one wavefront per token.  Each lane holds E/64 logits; top-k is k
// rounds of a wave-wide arg-max whose six exchange steps are DPP quad
// permutes and row mirrors inside 16-lane rows and v_permlane16/32_swap
// across rows (larger value first, lower expert id on ties).  The winner of
// round j is known to every lane, so the softmax denominator of the kept
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

namespace moe {

// ----------------------------------------------------------------- router

// A candidate is one 64-bit key: order-preserving bits of the logit in the
// high word (+0 and -0 made equal first) and the complement of the expert
// id in the low word, so the unsigned maximum is the larger logit and, on
// equal logits, the lower id.  Key 0 is "no candidate".
__device__ __forceinline__ unsigned long long route_key(float v, int id) {
    const uint32_t u = __float_as_uint(v + 0.0f);
    const uint32_t hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)hi << 32) | (uint32_t)~(uint32_t)id;
}
__device__ __forceinline__ float key_value(unsigned long long k) {
    const uint32_t hi = (uint32_t)(k >> 32);
    return __uint_as_float((hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi);
}
__device__ __forceinline__ int key_id(unsigned long long k) { return (int)~(uint32_t)k; }

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
    return a > b ? a : b;
}

template <int CTRL>
__device__ __forceinline__ unsigned long long dpp64(unsigned long long k) {
    const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)k, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(k >> 32), CTRL, 0xF, 0xF, false);
    return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Wave-wide maximum of the keys; every lane ends with the same key.
__device__ __forceinline__ unsigned long long wave_max_key(unsigned long long k) {
    k = umax64(k, dpp64<0xB1>(k));   // quad_perm [1,0,3,2]
    k = umax64(k, dpp64<0x4E>(k));   // quad_perm [2,3,0,1]
    k = umax64(k, dpp64<0x141>(k));  // row_half_mirror
    k = umax64(k, dpp64<0x140>(k));  // row_mirror: each lane holds its 16-lane row maximum
    {   // rows (0,1) and (2,3)
        const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)k, (uint32_t)k, false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(k >> 32), (uint32_t)(k >> 32), false, false);
        k = umax64(((unsigned long long)hi[0] << 32) | lo[0], ((unsigned long long)hi[1] << 32) | lo[1]);
    }
    {   // halves
        const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)k, (uint32_t)k, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(k >> 32), (uint32_t)(k >> 32), false, false);
        k = umax64(((unsigned long long)hi[0] << 32) | lo[0], ((unsigned long long)hi[1] << 32) | lo[1]);
    }
    return k;
}

// Top-k of one token's logits by the calling wave: k rounds of a wave-wide
// key maximum.  Lane j < top_k returns the j-th expert id in *id and its
// weight in *w (softmax of the kept logits relative to the largest, the
// denominator summed in j order); returns false for lanes j >= top_k.
template <int PER_LANE>
__device__ __forceinline__ bool route_token(const float *__restrict__ row, int n_experts, int top_k,
                                            int *id, float *w) {
    const int lane = threadIdx.x & (kWave - 1);
    unsigned long long key[PER_LANE];
#pragma unroll
    for (int q = 0; q < PER_LANE; ++q) {
        const int e = lane + kWave * q;
        key[q] = e < n_experts ? route_key(row[e], e) : 0ull;
    }
    unsigned long long mine = 0ull;
    for (int j = 0; j < top_k; ++j) {
        unsigned long long best = key[0];
#pragma unroll
        for (int q = 1; q < PER_LANE; ++q) best = umax64(best, key[q]);
        best = wave_max_key(best);
#pragma unroll
        for (int q = 0; q < PER_LANE; ++q) key[q] = key[q] == best ? 0ull : key[q];  // taken
        mine = lane == j ? best : mine;
    }
    const float v = key_value(mine);
    const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float ex = lane < top_k ? expf(v - v0) : 0.f;
    float den = 0.f;
    for (int j = 0; j < top_k; ++j) den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
    *id = key_id(mine);
    *w = ex / den;
    return lane < top_k;
}

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

// ---------------------------------------------------------------- planner

// Exclusive scan of one int per thread over the 256-thread block; returns
// this thread's prefix and writes the block total to *total.
__device__ __forceinline__ int block_exclusive_scan(int v, int *lds4, int *total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int inc = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += o;
    }
    if (lane == kWave - 1) lds4[wave] = inc;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kBlock / kWave; ++w) {
        const int s = lds4[w];
        if (w < wave) base += s;
        tot += s;
    }
    *total = tot;
    __syncthreads();
    return base + inc - v;
}

struct PlanOut {
    int *counts, *offsets, *sorted_slots, *unique_experts, *n_unique;
    int4 *work;
};

// The planner body for one 256-thread workgroup.  `idx` may live in global
// memory or in LDS.
__device__ __forceinline__ void plan_block(const int *idx, int n_slots, int n_experts, const PlanOut &p) {
    __shared__ int cnt[MOE_MAX_EXPERTS];
    __shared__ int cursor[MOE_MAX_EXPERTS];
    __shared__ int first_slot[MOE_MAX_EXPERTS];
    __shared__ int uniq[MOE_MAX_EXPERTS];
    __shared__ int lds4[kBlock / kWave];
    const int tid = threadIdx.x;
    const unsigned E = (unsigned)n_experts;

    for (int e = tid; e < n_experts; e += kBlock) {
        cnt[e] = 0;
        first_slot[e] = INT_MAX;
    }
    __syncthreads();
    for (int s = tid; s < n_slots; s += kBlock) {
        const int e = idx[s];
        if ((unsigned)e < E) {
            atomicAdd(&cnt[e], 1);          // integer: order-free
            atomicMin(&first_slot[e], s);
        }
    }
    __syncthreads();

    constexpr int PER = MOE_MAX_EXPERTS / kBlock;  // experts owned per thread
    int c[PER], nz = 0, sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = tid * PER + i;
        c[i] = e < n_experts ? cnt[e] : 0;
        sum += c[i];
        nz += c[i] > 0;
    }
    int total_slots, total_unique;
    int run = block_exclusive_scan(sum, lds4, &total_slots);
    int urun = block_exclusive_scan(nz, lds4, &total_unique);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = tid * PER + i;
        if (e < n_experts) {
            p.counts[e] = c[i];
            p.offsets[e] = run;
            cursor[e] = run;
            if (c[i] > 0) {
                p.unique_experts[urun] = e;
                p.work[urun] = make_int4(e, run, c[i], first_slot[e]);
                uniq[urun] = e;
                ++urun;
            }
        }
        run += c[i];
    }
    for (int u = total_unique + tid; u < n_experts; u += kBlock) {
        p.unique_experts[u] = -1;
        p.work[u] = make_int4(-1, total_slots, 0, 0);
    }
    if (tid == 0) {
        p.offsets[n_experts] = total_slots;
        p.n_unique[0] = total_unique;
    }
    __syncthreads();

    // stable scatter, one wave, 64 slots at a time in slot order
    if (tid < kWave) {
        const int lane = tid;
        const int id_bits = n_experts > 1 ? 32 - __clz(n_experts - 1) : 0;
        const unsigned long long below = (1ull << lane) - 1ull;
        for (int base = 0; base < n_slots; base += kWave) {
            const int s = base + lane;
            const int e = s < n_slots ? idx[s] : -1;
            const bool ok = s < n_slots && (unsigned)e < E;
            unsigned long long peers = __ballot(ok);
            for (int b = 0; b < id_bits; ++b) {
                const bool bit = ok && ((e >> b) & 1);
                const unsigned long long m = __ballot(bit);
                peers &= bit ? m : ~m;
            }
            if (ok) p.sorted_slots[cursor[e] + __popcll(peers & below)] = s;
            // every lane has read its cursor before the last peer moves it
            __builtin_amdgcn_wave_barrier();
            if (ok && lane == 63 - __clzll(peers)) cursor[e] += __popcll(peers);
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP: row shifts, then
// row broadcasts of lanes 15 and 31).  Lanes whose source is out of range
// add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_add_src(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v += dpp_add_src<0x111, 0xF>(v);  // row_shr:1
    v += dpp_add_src<0x112, 0xF>(v);  // row_shr:2
    v += dpp_add_src<0x114, 0xF>(v);  // row_shr:4
    v += dpp_add_src<0x118, 0xF>(v);  // row_shr:8
    v += dpp_add_src<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_add_src<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// Planner for at most 64 slots by a single wave, without barriers: lane s
// holds slot s.  Peer masks come from ballots over the expert-id bits; lane
// l owns experts l*P .. l*P+P-1 for counts, offsets and the distinct list,
// whose per-lane sums (count << 16 | nonzero) go through one wave scan.
// LDS operations of one wave complete in order, so values one lane writes
// are visible to the others at their next LDS read.
// `cnt`, `off`, `uix`: LDS scratch of n_experts ints each.
template <int P>  // experts owned per lane: P >= ceil(n_experts / 64)
__device__ __forceinline__ void plan_wave_small(const int *idx, int n_slots, int n_experts, const PlanOut &p,
                                                int *cnt, int *off, int *uix) {
    const int lane = threadIdx.x & (kWave - 1);
    const unsigned E = (unsigned)n_experts;
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int e = lane * P + q;
        if (e < n_experts) cnt[e] = 0;
    }
    const int id = lane < n_slots ? idx[lane] : -1;
    const bool ok = lane < n_slots && (unsigned)id < E;
    unsigned long long peers = __ballot(ok);
    const int id_bits = n_experts > 1 ? 32 - __clz(n_experts - 1) : 0;
    for (int b = 0; b < id_bits; ++b) {
        const bool bit = ok && ((id >> b) & 1);
        const unsigned long long m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & ((1ull << lane) - 1ull));
    const int n_peer = __popcll(peers);
    __builtin_amdgcn_wave_barrier();
    if (ok && rank == 0) cnt[id] = n_peer;  // the lowest peer lane is the expert's first slot
    __builtin_amdgcn_wave_barrier();
    int c[P], sum = 0;
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int e = lane * P + q;
        c[q] = e < n_experts ? cnt[e] : 0;
        sum += (c[q] << 16) + (c[q] > 0 ? 1 : 0);
    }
    const int inc = wave_inclusive_scan(sum);
    const int tot = __builtin_amdgcn_readlane(inc, kWave - 1);
    const int total_slots = tot >> 16, total_unique = tot & 0xFFFF;
    const int excl = inc - sum;  // both fields non-negative: no borrow between them
    int run = excl >> 16, urun = excl & 0xFFFF;
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int e = lane * P + q;
        if (e < n_experts) {
            p.counts[e] = c[q];
            p.offsets[e] = run;
            off[e] = run;
            if (c[q] > 0) {
                p.unique_experts[urun] = e;
                uix[e] = urun;
                ++urun;
            }
            run += c[q];
        }
    }
    __builtin_amdgcn_wave_barrier();
    if (ok) {
        const int base = off[id];
        p.sorted_slots[base + rank] = lane;
        if (rank == 0) p.work[uix[id]] = make_int4(id, base, n_peer, lane);
    }
    for (int u = total_unique + lane; u < n_experts; u += kWave) {
        p.unique_experts[u] = -1;
        p.work[u] = make_int4(-1, total_slots, 0, 0);
    }
    if (lane == 0) {
        p.offsets[n_experts] = total_slots;
        p.n_unique[0] = total_unique;
    }
}

// Small plans (<= 64 slots) run on one wave; larger ones on 256 threads.
template <int PER_LANE>
__global__ __launch_bounds__(kBlock) void expert_plan_kernel(const int *__restrict__ topk_idx, int n_slots,
                                                             int n_experts, PlanOut p) {
    if (n_slots <= kWave) {
        __shared__ int cnt[MOE_MAX_EXPERTS], off[MOE_MAX_EXPERTS], uix[MOE_MAX_EXPERTS];
        if (threadIdx.x < kWave) plan_wave_small<PER_LANE>(topk_idx, n_slots, n_experts, p, cnt, off, uix);
    } else {
        plan_block(topk_idx, n_slots, n_experts, p);
    }
}

// Router and planner in one workgroup: the four waves route the tokens, the
// indices are kept in LDS (and written out), then the block plans them.
template <int PER_LANE>
__global__ __launch_bounds__(kBlock) void route_plan_kernel(const float *__restrict__ logits, int n_tokens,
                                                            int n_experts, int top_k,
                                                            int *__restrict__ topk_idx,
                                                            float *__restrict__ topk_w, PlanOut p) {
    __shared__ int idx_lds[kRoutePlanMaxSlots];
    const int lane = threadIdx.x & (kWave - 1);
    const int n_waves = blockDim.x / kWave;
    for (int t = threadIdx.x / kWave; t < n_tokens; t += n_waves) {
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
    if (n_slots <= kWave) {  // launched with one wave per token, at most four
        __shared__ int cnt[MOE_MAX_EXPERTS], off[MOE_MAX_EXPERTS], uix[MOE_MAX_EXPERTS];
        if (threadIdx.x < kWave) plan_wave_small<PER_LANE>(idx_lds, n_slots, n_experts, p, cnt, off, uix);
    } else {                 // launched with 256 threads
        plan_block(idx_lds, n_slots, n_experts, p);
    }
}

static int per_lane_bucket(int n_experts) {
    const int per_lane = (n_experts + kWave - 1) / kWave;
    return per_lane <= 1 ? 1 : per_lane <= 2 ? 2 : per_lane <= 4 ? 4 : per_lane <= 8 ? 8 : 16;
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
    MOE_PER_LANE_SWITCH(per_lane_bucket(n_experts),
                        hipLaunchKernelGGL(expert_plan_kernel<PL>, dim3(1), dim3(n_slots <= kWave ? kWave : kBlock),
                                           0, stream, topk_idx, n_slots, n_experts, plan_out(plan)))
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
    // small batches: one wave per token (at most four); else a full block for the planner
    const int n_slots = n_tokens * top_k;
    const int threads = n_slots <= kWave ? kWave * (n_tokens < 4 ? (n_tokens > 0 ? n_tokens : 1) : 4) : kBlock;
    MOE_PER_LANE_SWITCH(per_lane_bucket(n_experts),
                        hipLaunchKernelGGL(route_plan_kernel<PL>, dim3(1), dim3(threads), 0, stream, logits,
                                           n_tokens, n_experts, top_k, topk_idx, topk_w, plan_out(plan)))
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}
