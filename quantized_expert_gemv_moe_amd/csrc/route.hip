// Router and cohort planner kernels (gfx950) and their C-ABI entry points.
//
// Router: one wavefront per token.  Each lane holds E/64 logits; top-k is k
// rounds of a wave-wide arg-max (butterfly shuffles, larger value first,
// lower expert id on ties), then the kept logits get softmax weights.  The
// router is the first of the three named parts of the per-token MoE cost
// (page "perf(moe): attribute the MoE decode gap at the M = 1 expert
// gather", Proposed Solution step 2).
//
// Planner: one workgroup.  An LDS histogram of expert ids, a block-wide
// exclusive scan into per-expert offsets and the list of distinct experts,
// then a stable scatter of slot ids into per-expert lists by one wave in
// slot order (ballot-based peer ranks).  This is the cross-cohort
// deduplication of page "perf(moe): batched decode scales 1.55x against
// 3.25x on dense" (Proposed Solution, second bullet): the expert kernels
// walk the distinct experts, so each expert's weights are read once per
// step whatever the number of (token, k) slots routed to it.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>

#include "device_util.h"
#include "moe_internal.h"

namespace moe {

// ----------------------------------------------------------------- router

template <int PER_LANE>
__global__ __launch_bounds__(kBlock) void route_topk_kernel(const float *__restrict__ logits,
                                                            int n_tokens, int n_experts, int top_k,
                                                            int *__restrict__ topk_idx,
                                                            float *__restrict__ topk_w) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * (kBlock / kWave) + (threadIdx.x / kWave);
    if (t >= n_tokens) return;  // uniform per wave

    const float *row = logits + (size_t)t * n_experts;
    float v[PER_LANE];
    uint32_t avail = 0;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const int e = lane + kWave * i;
        v[i] = e < n_experts ? row[e] : 0.f;
        if (e < n_experts) avail |= 1u << i;
    }

    int my_id = 0;       // lane j < k ends holding the j-th selection
    float my_val = 0.f;
    for (int j = 0; j < top_k; ++j) {
        // best remaining element of this lane: ids ascend with i, so a
        // strict comparison keeps the lower id on equal values
        float bv = 0.f;
        int bi = INT_MAX;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
            if (((avail >> i) & 1u) && (bi == INT_MAX || v[i] > bv)) {
                bv = v[i];
                bi = lane + kWave * i;
            }
        }
#pragma unroll
        for (int off = kWave / 2; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, kWave);
            const int oi = __shfl_xor(bi, off, kWave);
            const bool take = oi != INT_MAX &&
                              (bi == INT_MAX || ov > bv || (ov == bv && oi < bi));
            if (take) {
                bv = ov;
                bi = oi;
            }
        }
        if (lane == (bi & (kWave - 1))) avail &= ~(1u << (bi / kWave));
        if (lane == j) {
            my_id = bi;
            my_val = bv;
        }
    }

    // softmax over the kept logits, relative to the largest one
    const float l0 = __shfl(my_val, 0, kWave);
    const float ex = lane < top_k ? expf(my_val - l0) : 0.f;
    float den = 0.f;
    for (int j = 0; j < top_k; ++j) den += __shfl(ex, j, kWave);  // fixed j order
    if (lane < top_k) {
        topk_idx[(size_t)t * top_k + lane] = my_id;
        topk_w[(size_t)t * top_k + lane] = ex / den;
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

__global__ __launch_bounds__(kBlock) void expert_plan_kernel(const int *__restrict__ topk_idx,
                                                             int n_slots, int n_experts,
                                                             int *__restrict__ counts,
                                                             int *__restrict__ offsets,
                                                             int *__restrict__ sorted_slots,
                                                             int *__restrict__ unique_experts,
                                                             int *__restrict__ n_unique) {
    __shared__ int cnt[MOE_MAX_EXPERTS];
    __shared__ int cursor[MOE_MAX_EXPERTS];
    __shared__ int lds4[kBlock / kWave];
    const int tid = threadIdx.x;
    const unsigned E = (unsigned)n_experts;

    for (int e = tid; e < n_experts; e += kBlock) cnt[e] = 0;
    __syncthreads();
    for (int s = tid; s < n_slots; s += kBlock) {
        const int e = topk_idx[s];
        if ((unsigned)e < E) atomicAdd(&cnt[e], 1);  // integer: order-free
    }
    __syncthreads();

    // each thread owns PER consecutive experts
    constexpr int PER = MOE_MAX_EXPERTS / kBlock;
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
            counts[e] = c[i];
            offsets[e] = run;
            cursor[e] = run;
            if (c[i] > 0) unique_experts[urun++] = e;
        }
        run += c[i];
    }
    for (int e = total_unique + tid; e < n_experts; e += kBlock) unique_experts[e] = -1;
    if (tid == 0) {
        offsets[n_experts] = total_slots;
        n_unique[0] = total_unique;
    }
    __syncthreads();

    // stable scatter, one wave, 64 slots at a time in slot order
    if (tid < kWave) {
        const int lane = tid;
        const int id_bits = n_experts > 1 ? 32 - __clz(n_experts - 1) : 0;
        const unsigned long long below = (1ull << lane) - 1ull;
        for (int base = 0; base < n_slots; base += kWave) {
            const int s = base + lane;
            const int e = s < n_slots ? topk_idx[s] : -1;
            const bool ok = s < n_slots && (unsigned)e < E;
            unsigned long long peers = __ballot(ok);
            for (int b = 0; b < id_bits; ++b) {
                const bool bit = ok && ((e >> b) & 1);
                const unsigned long long m = __ballot(bit);
                peers &= bit ? m : ~m;
            }
            int pos = 0;
            if (ok) {
                pos = cursor[e] + __popcll(peers & below);
                sorted_slots[pos] = s;
            }
            // every lane has read its cursor before the last peer moves it
            __builtin_amdgcn_wave_barrier();
            if (ok && lane == 63 - __clzll(peers)) cursor[e] += __popcll(peers);
            __builtin_amdgcn_wave_barrier();
        }
    }
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_route_topk(const float *logits, int32_t n_tokens, int32_t n_experts,
                                     int32_t top_k, int32_t *topk_idx, float *topk_w,
                                     void *hip_stream) {
    const moe_status st = check_route_args(logits, n_tokens, n_experts, top_k, topk_idx, topk_w);
    if (st != MOE_OK) return st;
    if (n_tokens == 0) return MOE_OK;
    hipStream_t stream = (hipStream_t)hip_stream;
    const dim3 grid((n_tokens + kBlock / kWave - 1) / (kBlock / kWave));
    const int per_lane = (n_experts + kWave - 1) / kWave;
#define MOE_ROUTE_CASE(P)                                                                      \
    case P:                                                                                    \
        hipLaunchKernelGGL(route_topk_kernel<P>, grid, dim3(kBlock), 0, stream, logits,       \
                           n_tokens, n_experts, top_k, topk_idx, topk_w);                     \
        break;
    switch (per_lane <= 1 ? 1 : per_lane <= 2 ? 2 : per_lane <= 4 ? 4 : per_lane <= 8 ? 8 : 16) {
        MOE_ROUTE_CASE(1)
        MOE_ROUTE_CASE(2)
        MOE_ROUTE_CASE(4)
        MOE_ROUTE_CASE(8)
        MOE_ROUTE_CASE(16)
    }
#undef MOE_ROUTE_CASE
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

extern "C" moe_status moe_expert_plan(const int32_t *topk_idx, int32_t n_tokens, int32_t n_experts,
                                      int32_t top_k, const moe_plan_t *plan, void *hip_stream) {
    const moe_status st = check_plan_args(topk_idx, n_tokens, n_experts, top_k, plan);
    if (st != MOE_OK) return st;
    hipStream_t stream = (hipStream_t)hip_stream;
    hipLaunchKernelGGL(expert_plan_kernel, dim3(1), dim3(kBlock), 0, stream, topk_idx,
                       n_tokens * top_k, n_experts, plan->counts, plan->offsets,
                       plan->sorted_slots, plan->unique_experts, plan->n_unique);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}
