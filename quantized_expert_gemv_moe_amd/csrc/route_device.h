// Device code of the router and the cohort planner, shared by the route
// kernels and by the single-token expert kernel that routes for itself.
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>

#include "device_util.h"

namespace moe {

// ----------------------------------------------------------------- router

// Order-preserving bits of a logit (+0 and -0 made equal first): unsigned
// comparison of keys is comparison of the logits.  Every finite logit's key
// is nonzero, so 0 marks an expert already taken (or past n_experts).
__device__ __forceinline__ uint32_t route_key(float v) {
    const uint32_t u = __float_as_uint(v + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// Wave-wide maximum of one key per lane, as a wave-uniform value: four DPP
// steps give every lane its 16-lane row maximum, two permlane swaps mix the
// rows.
__device__ __forceinline__ uint32_t wave_max_key(uint32_t k) {
    k = max(k, dpp32<0xB1>(k));   // quad_perm [1,0,3,2]
    k = max(k, dpp32<0x4E>(k));   // quad_perm [2,3,0,1]
    k = max(k, dpp32<0x141>(k));  // row_half_mirror
    k = max(k, dpp32<0x140>(k));  // row_mirror
    {
        const auto r = __builtin_amdgcn_permlane16_swap(k, k, false, false);  // rows (0,1), (2,3)
        k = max(r[0], r[1]);
    }
    {
        const auto r = __builtin_amdgcn_permlane32_swap(k, k, false, false);  // halves
        k = max(r[0], r[1]);
    }
    return __builtin_amdgcn_readfirstlane(k);
}

// The order keys of one token's logits: lane l holds experts l, l + 64, ...
// All loads are in flight at once and stay in bounds.
template <int PER_LANE>
__device__ __forceinline__ void route_keys(const float *__restrict__ row, int n_experts, uint32_t *key) {
    const int lane = threadIdx.x & (kWave - 1);
    float lg[PER_LANE];
#pragma unroll
    for (int q = 0; q < PER_LANE; ++q) {
        const int e = lane + kWave * q;
        lg[q] = row[e < n_experts ? e : n_experts - 1];
    }
#pragma unroll
    for (int q = 0; q < PER_LANE; ++q) key[q] = lane + kWave * q < n_experts ? route_key(lg[q]) : 0u;
}

// One selection round: the wave-wide largest remaining key; among lanes
// holding it (equal logits) the lowest expert id wins, found from the
// ballots of equal keys in id order.  The winner is marked taken.  Returns
// its expert id and writes its key to *best (both wave-uniform).
template <int PER_LANE>
__device__ __forceinline__ int route_take(uint32_t *key, uint32_t *best) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t b = key[0];
#pragma unroll
    for (int q = 1; q < PER_LANE; ++q) b = max(b, key[q]);
    b = wave_max_key(b);
    int win = -1;
#pragma unroll
    for (int q = PER_LANE - 1; q >= 0; --q) {
        const unsigned long long m = __builtin_amdgcn_ballot_w64(key[q] == b);
        if (m) win = kWave * q + __builtin_ctzll(m);
    }
#pragma unroll
    for (int q = 0; q < PER_LANE; ++q) key[q] = (lane + kWave * q == win) ? 0u : key[q];
    *best = b;
    return win;
}

// Top-k of NT tokens at once from their order keys (route_keys): top_k
// selection rounds per token, the tokens' rounds interleaved so their
// dependent exchange chains overlap.  Lane j < top_k gets token n's j-th
// expert id in id[n] and its weight in w[n] (softmax of the kept logits
// relative to the largest, the denominator summed in j order).
template <int PER_LANE, int NT>
__device__ __forceinline__ void route_select(uint32_t (*key)[PER_LANE], int top_k, int *id, float *w) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t mine[NT];
    int mine_id[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        mine[n] = 0u;
        mine_id[n] = 0;
    }
    for (int j = 0; j < top_k; ++j) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            uint32_t best;
            const int win = route_take<PER_LANE>(key[n], &best);
            mine[n] = lane == j ? best : mine[n];
            mine_id[n] = lane == j ? win : mine_id[n];
        }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const float v = key_value(mine[n]);
        const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
        const float ex = lane < top_k ? expf(v - v0) : 0.f;
        float den = 0.f;
        for (int j = 0; j < top_k; ++j) den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
        id[n] = mine_id[n];
        w[n] = ex / den;
    }
}

// Top-k of one token's logits by the calling wave.  Lane j < top_k returns
// the j-th expert id in *id and its weight in *w; returns false for lanes
// j >= top_k.
template <int PER_LANE>
__device__ __forceinline__ bool route_token(const float *__restrict__ row, int n_experts, int top_k,
                                            int *id, float *w) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t key[1][PER_LANE];
    route_keys<PER_LANE>(row, n_experts, key[0]);
    route_select<PER_LANE, 1>(key, top_k, id, w);
    return lane < top_k;
}

// The expert of rank `rank` (0 = largest logit) alone: rank + 1 selection
// rounds.  (An MSB-first radix select over the 32 key bits, whose time does
// not grow with the rank, measured slower at top-8 of 128: 32 dependent
// ballot steps against 4.5 rounds on average.)
template <int PER_LANE>
__device__ __forceinline__ int route_rank(const float *__restrict__ row, int n_experts, int rank) {
    uint32_t key[PER_LANE];
    route_keys<PER_LANE>(row, n_experts, key);
    int win = 0;
    for (int j = 0; j <= rank; ++j) {
        uint32_t best;
        win = route_take<PER_LANE>(key, &best);
    }
    return win;
}

// Rank of expert e (wave-uniform, < n_experts) among one token's experts in
// the router's order -- descending logit, ties to the lower id -- from that
// token's order keys (route_keys): the number of experts placed before it.
// The token holds e among its top k exactly when this is below k, and then
// e is its expert of that rank: the same order route_take walks.
template <int PER_LANE>
__device__ __forceinline__ int route_rank_of(const uint32_t *key, int e) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t ke = 0;
#pragma unroll
    for (int q = 0; q < PER_LANE; ++q) {
        const uint32_t v = __builtin_amdgcn_readlane(key[q], e & (kWave - 1));
        ke = (q == (e >> 6)) ? v : ke;
    }
    int n = 0;
#pragma unroll
    for (int q = 0; q < PER_LANE; ++q) {
        const int id = lane + kWave * q;
        const bool before = key[q] > ke || (key[q] == ke && id < e);
        n += __popcll(__builtin_amdgcn_ballot_w64(before));
    }
    return n;
}

// ---------------------------------------------------------------- planner

// Exclusive scan of one int per thread over a block of NT threads; returns
// this thread's prefix and writes the block total to *total.  `lds` holds
// NT / 64 ints.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int *lds, int *total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int inc = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += o;
    }
    if (lane == kWave - 1) lds[wave] = inc;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        const int s = lds[w];
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

// The planner body for one workgroup of NT threads (256 or 1024).  `idx`
// may live in global memory or in LDS.  The slots are cut into one
// contiguous range per wave; every wave counts its range per expert, each
// wave's first position per expert follows from the expert's offset plus
// the counts of the waves before it, and then every wave scatters its own
// range in slot order (64 slots at a time), so the waves place their slots
// at once and the sort stays stable.
template <int NT>
__device__ __forceinline__ void plan_block(const int *idx, int n_slots, int n_experts, const PlanOut &p) {
    constexpr int NW = NT / kWave;
    __shared__ int cnt[MOE_MAX_EXPERTS];
    __shared__ int cntw[NW][MOE_MAX_EXPERTS];  // per wave: count, then first position
    __shared__ int first_slot[MOE_MAX_EXPERTS];
    __shared__ int lds_scan[NW];
    const int tid = threadIdx.x;
    const unsigned E = (unsigned)n_experts;
    const int span = n_slots > NW ? (n_slots + NW - 1) / NW : 1;  // slots per wave range

    for (int e = tid; e < n_experts; e += NT) {
        first_slot[e] = INT_MAX;
#pragma unroll
        for (int w = 0; w < NW; ++w) cntw[w][e] = 0;
    }
    __syncthreads();
    for (int s = tid; s < n_slots; s += NT) {
        const int e = idx[s];
        if ((unsigned)e < E) {
            atomicAdd(&cntw[s / span][e], 1);  // integer: order-free
            atomicMin(&first_slot[e], s);
        }
    }
    __syncthreads();
    for (int e = tid; e < n_experts; e += NT) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) c += cntw[w][e];
        cnt[e] = c;
    }
    __syncthreads();

    constexpr int PER = MOE_MAX_EXPERTS / NT;  // experts owned per thread
    int c[PER], nz = 0, sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = tid * PER + i;
        c[i] = e < n_experts ? cnt[e] : 0;
        sum += c[i];
        nz += c[i] > 0;
    }
    int total_slots, total_unique;
    int run = block_exclusive_scan<NT>(sum, lds_scan, &total_slots);
    int urun = block_exclusive_scan<NT>(nz, lds_scan, &total_unique);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = tid * PER + i;
        if (e < n_experts) {
            p.counts[e] = c[i];
            p.offsets[e] = run;
            int base = run;  // each wave's first position for e
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const int cw = cntw[w][e];
                cntw[w][e] = base;
                base += cw;
            }
            if (c[i] > 0) {
                p.unique_experts[urun] = e;
                p.work[urun] = make_int4(e, run, c[i], first_slot[e]);
                ++urun;
            }
        }
        run += c[i];
    }
    for (int u = total_unique + tid; u < n_experts; u += NT) {
        p.unique_experts[u] = -1;
        p.work[u] = make_int4(-1, total_slots, 0, 0);
    }
    if (tid == 0) {
        p.offsets[n_experts] = total_slots;
        p.n_unique[0] = total_unique;
    }
    __syncthreads();

    // stable scatter: wave w walks its range in slot order, 64 slots at a time
    {
        const int lane = tid & (kWave - 1);
        const int w = tid / kWave;
        int *cursor = cntw[w];
        const int id_bits = n_experts > 1 ? 32 - __clz(n_experts - 1) : 0;
        const unsigned long long below = (1ull << lane) - 1ull;
        const int end = (w + 1) * span < n_slots ? (w + 1) * span : n_slots;
        for (int base = w * span; base < end; base += kWave) {
            const int s = base + lane;
            const int e = s < end ? idx[s] : -1;
            const bool ok = s < end && (unsigned)e < E;
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

}  // namespace moe
