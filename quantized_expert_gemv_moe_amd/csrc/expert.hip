// Expert kernels of one decode step (gfx950) and moe_decode_step.
//
// The expert block the pages turn on is the SwitchGLU expert evaluated once
// per (token, k) slot at M = 1 (page "perf(moe): attribute the MoE decode
// gap at the M = 1 expert gather", Problem / Background), with the
// deepseek_v4 clamp stage and the inkling expert-scale sidecars named on
// the same page, and a token dimension whose outputs are summed over k per
// token with fp32 partials and one final rounding (page "perf(moe): batched
// decode scales 1.55x against 3.25x on dense", Proposed Solution and
// Implementation Notes).  Every kernel here walks the *distinct* experts of
// the plan, so an expert's weights are streamed from HBM once per step for
// all the tokens routed to it, and each workgroup keeps its weights in
// registers while it loops over those tokens.
//
//   gate_up : (distinct expert, block of dff rows) per one-wave workgroup.
//             A row is read as 16-byte chunks by LPR lanes (64 for hidden
//             2048..8192).  4-bit weights are unpacked in registers; bf16
//             activations go through v_dot2_f32_bf16 with the nibbles
//             turned into bf16 pairs of value 128 + q, the offset folded
//             back with the chunk's activation sum; fp32 activations use
//             exact fp32 FMAs.  The group bias is folded as bias * sum(x).
//             Gate and up share the activations; SiLU(g) * u is written as
//             fp32 h per slot.
//   down    : (distinct expert, block of hidden rows) per 4-wave workgroup.
//             h of the expert's slots and its per-group sums are staged in
//             LDS; exact fp32 FMAs (h is never rounded to bf16).
//   combine : out[t] = sum_j w[t][j] * y[t*k+j] in j order, one rounding.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>

#include <mutex>

#include "device_util.h"
#include "expert_device.h"
#include "gate_up_device.h"
#include "mfma_device.h"
#include "moe_internal.h"
#include "route_device.h"

namespace moe {

template <int LPR, int NV, int RI, bool XBF16>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(gate_up_waves_per_simd<LPR, NV, XBF16>())))
void gate_up_kernel(GateUpArgs a) {
    gate_up_valu_block<LPR, NV, RI, XBF16>(a, blockIdx.x, blockIdx.y);
}

// ----------------------------------------------------- gate+up, MFMA tiles

// Experts with many tokens: v_mfma_f32_16x16x32_bf16.  A workgroup of NW
// waves owns 16 * RT rows of the expert and all of hidden; wave w takes GW
// of the 64-groups.  Per group and 16-row tile, each lane holds two words
// of its row (16 nibbles) as bf16 pairs of value 1 + q / 16, in the nibble
// pairing of the dot2 path, and its token's activations in the same
// pairing; two MFMAs then sum exactly one group, so the group scale (times
// 16) and the folded bias (b - 16 s) * sum(x) apply per group after the
// MFMA.  Output lane l holds token l % 16 and rows 4 * (l / 16) .. + 3.  The
// waves' partial sums meet in LDS and are added in wave order; tokens go in
// tiles of 16.
constexpr int kMfmaTokens = 16;  // token tile

// 16-row tiles per MFMA gate+up workgroup: one from eight waves up (the
// workgroup's registers then leave room for two workgroups per CU), two below.
constexpr int mfma_row_tiles(int nw) { return nw >= 8 ? 1 : 2; }

// NW waves, GW 64-groups per wave (NW * GW = hidden / 64), RT 16-row tiles.
// Every weight load of a wave is issued before its first MFMA, and every
// activation load of a token tile before that tile's first MFMA.
// Elements 64g + 16kq .. + 15 of a token's activations for each of the
// wave's groups: the B operands of one token column.
template <int GW>
__device__ __forceinline__ void load_x_mfma(const GateUpArgs &a, int slot, bool live, int g0, int kq,
                                            uint4 (*xw)[2]) {
    const uint16_t *xr = (const uint16_t *)a.x + (size_t)(slot / a.top_k) * a.hidden;
#pragma unroll
    for (int gi = 0; gi < GW; ++gi) {
        // unconditional loads (the slot is valid either way), masked after:
        // a load under a branch would make the compiler wait for every load
        // in flight where the branch joins.  The mask is opaque to the
        // optimizer, which would otherwise move the loads into a branch.
        uint32_t mk = live ? 0xFFFFFFFFu : 0u;
        asm volatile("" : "+v"(mk));
        const gv4u_gptr xp = (gv4u_gptr)(xr + (g0 + gi) * kGroup + 16 * kq);
        const gv4u v0 = xp[0], v1 = xp[1];
        xw[gi][0] = make_uint4(v0.x & mk, v0.y & mk, v0.z & mk, v0.w & mk);
        xw[gi][1] = make_uint4(v1.x & mk, v1.y & mk, v1.z & mk, v1.w & mk);
    }
}

template <int NW, int GW, int RT>
__device__ __forceinline__ void gate_up_mfma_block(const GateUpArgs &a, int rb, int u, float *smem, int min_count) {
    constexpr int ROWS = 16 * RT;
    constexpr int G = NW * GW;
    Work wk;
    if (!plan_expert(a.plan, u, a.n_experts, a.n_slots, &wk)) return;
    if (wk.count < min_count) return;  // the expert belongs to the VALU kernel
    const int H = a.hidden, F = a.dff;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int r16 = lane & 15, kq = lane >> 4;
    const int row0 = rb * ROWS;
    const int g0 = wave * GW;
    // order of issue: the first token tile's slot lookup, the weights, then
    // the activations that need the slot (their wait covers the lookup alone)
    int slot = plan_slot(a.plan, wk, r16 < wk.count ? r16 : wk.count - 1, a.n_slots);
    __builtin_amdgcn_sched_barrier(0);

    // this wave's weights: words 2kq and 2kq+1 of each group, per row tile
    // (ordinary loads: the streaming hint measured ~1.5 % slower at 32 tokens)
    uint2 wgq[GW][RT], wuq[GW][RT];
    {
        const uint2 *gq = (const uint2 *)a.gate_q, *uq = (const uint2 *)a.up_q;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int row = row0 + 16 * t + r16;
            const size_t rb = ((size_t)wk.e * F + (row < F ? row : F - 1)) * (H / 16) + g0 * 4 + kq;
#pragma unroll
            for (int gi = 0; gi < GW; ++gi) {
                wgq[gi][t] = gq[rb + gi * 4];
                wuq[gi][t] = uq[rb + gi * 4];
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    slot = r16 < wk.count ? slot : 0;
    uint4 xw[GW][2];
    load_x_mfma<GW>(a, slot, r16 < wk.count, g0, kq, xw);
    // per [group][row]: 16 * scale, and bias - 16 * scale (the weights go
    // into the MFMA as 1 + q / 16)
    float *sg = smem, *bg = smem + G * ROWS, *su = smem + 2 * G * ROWS, *bu = smem + 3 * G * ROWS;
    float *part = smem + 4 * G * ROWS;  // [wave][lane][8 * RT]
    for (int i = threadIdx.x; i < ROWS * G; i += NW * kWave) {
        const int r = i / G, g = i - r * G;
        const int row = row0 + r < F ? row0 + r : F - 1;
        const size_t si = ((size_t)wk.e * F + row) * G + g;
        const float s1 = f16_bits_to_f32(a.gate_s[si]), s2 = f16_bits_to_f32(a.up_s[si]);
        sg[g * ROWS + r] = 16.f * s1;
        bg[g * ROWS + r] = fmaf(-16.f, s1, f16_bits_to_f32(a.gate_b[si]));
        su[g * ROWS + r] = 16.f * s2;
        bu[g * ROWS + r] = fmaf(-16.f, s2, f16_bits_to_f32(a.up_b[si]));
    }
    __syncthreads();
    const float sc = a.expert_scale ? a.expert_scale[wk.e] : 1.f;
    const float lim = a.clamp_limit;

    for (int t0 = 0; t0 < wk.count; t0 += kMfmaTokens) {
        const int nt = wk.count - t0 < kMfmaTokens ? wk.count - t0 : kMfmaTokens;
        const bool live = r16 < nt;  // this lane's token column
        if (t0 > 0) {
            slot = live ? plan_slot(a.plan, wk, t0 + r16, a.n_slots) : 0;
            load_x_mfma<GW>(a, slot, live, g0, kq, xw);
        }
        f32x4_t accg[RT], accu[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            accg[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            accu[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int gi = 0; gi < GW; ++gi) {
            const int g = g0 + gi;
            uint32_t xb[2][4];
            float xs = 0.f;
            x8_pairs(xw[gi][0], xb[0], &xs);
            x8_pairs(xw[gi][1], xb[1], &xs);
            xs = swap16_sum(xs, xs);  // add the four lanes of the token
            xs = swap32_sum(xs, xs);
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                uint32_t ag[2][4], au[2][4];
                q4_pairs16(wgq[gi][t].x, ag[0]);
                q4_pairs16(wgq[gi][t].y, ag[1]);
                q4_pairs16(wuq[gi][t].x, au[0]);
                q4_pairs16(wuq[gi][t].y, au[1]);
                f32x4_t dg = mfma16x16x32(ag[0], xb[0], f32x4_t{0.f, 0.f, 0.f, 0.f});
                dg = mfma16x16x32(ag[1], xb[1], dg);
                f32x4_t du = mfma16x16x32(au[0], xb[0], f32x4_t{0.f, 0.f, 0.f, 0.f});
                du = mfma16x16x32(au[1], xb[1], du);
                const float4 s1 = *(const float4 *)(sg + g * ROWS + 16 * t + 4 * kq);
                const float4 b1 = *(const float4 *)(bg + g * ROWS + 16 * t + 4 * kq);
                const float4 s2 = *(const float4 *)(su + g * ROWS + 16 * t + 4 * kq);
                const float4 b2 = *(const float4 *)(bu + g * ROWS + 16 * t + 4 * kq);
                accg[t][0] += fmaf(s1.x, dg[0], b1.x * xs);
                accg[t][1] += fmaf(s1.y, dg[1], b1.y * xs);
                accg[t][2] += fmaf(s1.z, dg[2], b1.z * xs);
                accg[t][3] += fmaf(s1.w, dg[3], b1.w * xs);
                accu[t][0] += fmaf(s2.x, du[0], b2.x * xs);
                accu[t][1] += fmaf(s2.y, du[1], b2.y * xs);
                accu[t][2] += fmaf(s2.z, du[2], b2.z * xs);
                accu[t][3] += fmaf(s2.w, du[3], b2.w * xs);
            }
        }
        float *mine = part + ((size_t)wave * kWave + lane) * (8 * RT);
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mine[t * 8 + i] = accg[t][i];
                mine[t * 8 + 4 + i] = accu[t][i];
            }
        __syncthreads();
        // add the partials in wave order and finish the rows: output o =
        // (row tile, row of the lane's four) goes to wave o % NW
        if (live) {
            for (int o = wave; o < 4 * RT; o += NW) {
                const int t = o / 4, i = o % 4;
                float g = 0.f, u = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    const float *pw = part + ((size_t)w * kWave + lane) * (8 * RT);
                    g += pw[t * 8 + i];
                    u += pw[t * 8 + 4 + i];
                }
                const int row = row0 + 16 * t + 4 * kq + i;
                if (row < F) a.h[(size_t)slot * F + row] = act_mul(g, u, sc, lim, a.activation);
            }
        }
        __syncthreads();
    }
}

// Workgroups of eight or more waves fit four waves per SIMD (two workgroups
// per CU at eight) in 128 registers; the compiler would otherwise size them
// for two waves per SIMD.
template <int NW>
constexpr int mfma_waves_per_simd() { return NW >= 8 ? 4 : 1; }

template <int NW, int GW, int RT>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(mfma_waves_per_simd<NW>())))
void gate_up_mfma_kernel(GateUpArgs a, int min_count) {
    extern __shared__ float smem[];
    gate_up_mfma_block<NW, GW, RT>(a, blockIdx.x, blockIdx.y, smem, min_count);
}

// Both gate+up variants in one launch: blocks [0, mfma_blocks) are MFMA
// workgroups (row block, distinct expert) for the experts with min_count or
// more tokens; every wave of the later blocks is one dot2 workgroup (row
// block, distinct expert) for the others.  The two kinds run side by side
// instead of one launch after the other.
template <int LPR, int NV, int RI, int NW, int GW, int RT>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(mfma_waves_per_simd<NW>())))
void gate_up_mixed_kernel(GateUpArgs a, int mfma_blocks, int rb_mfma,
                                                                   int rb_valu, int n_valu, int min_count) {
    extern __shared__ float smem[];
    const int b = blockIdx.x;
    if (b < mfma_blocks) {
        gate_up_mfma_block<NW, GW, RT>(a, b % rb_mfma, b / rb_mfma, smem, min_count);
        return;
    }
    const int vb = (b - mfma_blocks) * NW + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (vb >= n_valu) return;
    gate_up_valu_block<LPR, NV, RI, true>(a, vb % rb_valu, vb / rb_valu);
}

// ------------------------------------------------------------------- down

// Four waves per workgroup.  h of up to `slots_per_stage` slots and its
// sums per 64-group live in dynamic LDS: [S][F] floats, then [S][F/64].
template <int LPR, int NV, int RI>
__global__ __launch_bounds__(kBlock) void down_kernel(DownArgs a) {
    constexpr int RPI = kWave / LPR;
    constexpr int ROWS_WG = RPI * RI * (kBlock / kWave);
    extern __shared__ float lds[];
    Work wk;
    if (!plan_expert(a.plan, blockIdx.y, a.n_experts, a.n_slots, &wk)) return;
    const int e = wk.e, count = wk.count;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int sl = lane % LPR;
    const int row0 = blockIdx.x * ROWS_WG + wave * RPI * RI + lane / LPR;
    const int H = a.hidden, F = a.dff;
    const int qrow = F / 32, grow = F / kGroup;
    const int S = a.slots_per_stage;
    float *hl = lds;               // [S][F]
    float *gs = lds + (size_t)S * F;  // [S][F/64]

    uint4 wd[RI][NV];
    float sd[RI][NV], bd[RI][NV];
#pragma unroll
    for (int r = 0; r < RI; ++r) {
        const int row = row0 + r * RPI;
        const int rr = row < H ? row : H - 1;
        const size_t rq = ((size_t)e * H + rr) * qrow;
        const size_t rs = ((size_t)e * H + rr) * grow;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int ch = v * LPR + sl;
            wd[r][v] = load_stream(a.down_q + rq + ch);
            sd[r][v] = f16_bits_to_f32(a.down_s[rs + ch / 2]);
            // the bias of a group is applied once, by the lane holding its even chunk
            bd[r][v] = (ch & 1) ? 0.f : f16_bits_to_f32(a.down_b[rs + ch / 2]);
        }
    }

    for (int s0 = 0; s0 < count; s0 += S) {
        const int ns = count - s0 < S ? count - s0 : S;
        __syncthreads();  // previous stage fully consumed
        const int f4 = F / 4;
        for (int i = threadIdx.x; i < ns * f4; i += kBlock) {
            const int j = i / f4, c = i - j * f4;
            const int slot = plan_slot(a.plan, wk, s0 + j, a.n_slots);
            ((float4 *)(hl + (size_t)j * F))[c] = ((const float4 *)(a.h + (size_t)slot * F))[c];
        }
        __syncthreads();
        // per-group sums of h: two threads per group, 32 elements each
        for (int i = threadIdx.x; i < ns * grow * 2; i += kBlock) {
            const int j = i / (grow * 2), g = (i / 2) % grow, half = i & 1;
            const float *src = hl + (size_t)j * F + g * kGroup + half * 32;
            float s = 0.f;
#pragma unroll
            for (int c = 0; c < 32; ++c) s += src[c];
            s += dpp<kDppQuad1032>(s);  // partner thread holds the other half
            if (!half) gs[j * grow + g] = s;
        }
        __syncthreads();
        for (int j = 0; j < ns; ++j) {
            const int slot = plan_slot(a.plan, wk, s0 + j, a.n_slots);
            float hv[NV][32], hsum[NV];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int ch = v * LPR + sl;
                const float4 *p = (const float4 *)(hl + (size_t)j * F + ch * 32);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const float4 q = p[c];
                    hv[v][4 * c + 0] = q.x;
                    hv[v][4 * c + 1] = q.y;
                    hv[v][4 * c + 2] = q.z;
                    hv[v][4 * c + 3] = q.w;
                }
                hsum[v] = gs[j * grow + ch / 2];
            }
#pragma unroll
            for (int r = 0; r < RI; ++r) {
                float y = 0.f;
#pragma unroll
                for (int v = 0; v < NV; ++v) y += fmaf(sd[r][v], dot32_q4(wd[r][v], hv[v]), bd[r][v] * hsum[v]);
                y = seg_sum<LPR>(y);
                const int row = row0 + r * RPI;
                if (sl == 0 && row < H) a.y[(size_t)slot * H + row] = y;
            }
        }
    }
}

// -------------------------------------------------- down, column layout

// MOE_DOWN_COLS: lane = output row, so the 32 h values of a chunk are the
// same for the whole wave.  NW waves split dff, CPW chunks of 32 inputs
// each, and their partial sums meet in LDS, added in wave order.  Chunks are
// the outer loop and up to S slots the inner one: a chunk's 32 weights are
// converted once for all the expert's tokens.  Each wave fetches the 64-input
// groups its chunks fall in for every slot of a stage at once (one 256-byte
// load each, all in flight together), forms the group sums from them, and
// parks them in its own LDS rows, from which the chunk values are read back
// as broadcasts; nothing waits for memory inside the chunk loop.
// Slots per stage: two.  Most experts this kernel sees hold one or two
// tokens (from 16 tokens up the others go to the MFMA kernel), and every
// stage issues its loads for all S slots whether or not they are used
// (measured at 32 tokens: 93.6 us per step against 94.8 with four).
// Sixteen-wave workgroups (dff 1536 and 2048) have 128 registers per wave;
// with two slots per stage they spilled (dff 2048: 86 registers, 296 bytes
// per lane of scratch), so they take one.
template <int NW>
constexpr int down_cols_stage() { return NW >= 16 ? 1 : 2; }

template <int NW, int CPW>
__global__ __launch_bounds__(NW * kWave) void down_cols_kernel(const uint4 *__restrict__ q,
                                                               const uint16_t *__restrict__ sc,
                                                               const uint16_t *__restrict__ bi,
                                                               const float *__restrict__ h,
                                                               float *__restrict__ y, PlanView plan,
                                                               int hidden, int dff, int n_experts,
                                                               int n_slots, int max_count) {
    constexpr int S = down_cols_stage<NW>();
    constexpr int NG = CPW / 2 + 1;  // groups a wave's CPW chunks can touch
    __shared__ float part[NW][S][kWave];
    __shared__ float4 hw[NW][S][NG][kGroup / 4];  // each wave's groups of h
    Work wk;
    if (!plan_expert(plan, blockIdx.y, n_experts, n_slots, &wk)) return;
    if (wk.count > max_count) return;  // the MFMA kernel's expert
    const int lane = threadIdx.x & (kWave - 1);
    // wave index as a scalar: addresses built from it stay wave-uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int H = hidden, F = dff, C = F / 32, G = F / kGroup;
    const int m = blockIdx.x * kWave + lane;  // hidden % 64 == 0: always a row
    const int c0 = wave * CPW;
    const int g0 = c0 / 2;  // first group of the wave's chunks

    uint4 wq[CPW];
    float ws[CPW], wb[CPW];
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
        const int c = c0 + j;
        wq[j] = load_stream(q + ((size_t)wk.e * C + c) * H + m);
        const size_t gi = ((size_t)wk.e * G + c / 2) * H + m;
        ws[j] = f16_bits_to_f32(sc[gi]);
        // a group's bias is applied once, with the sum of its 64 inputs, by its even chunk
        wb[j] = (c & 1) ? 0.f : f16_bits_to_f32(bi[gi]);
    }

    for (int s0 = 0; s0 < wk.count; s0 += S) {
        const int ns = wk.count - s0 < S ? wk.count - s0 : S;
        // every (slot, group) load is unconditional: slots past the stage
        // repeat its last one and groups past dff its last group, unused
        float hv[S][NG];
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const float *hs = h + (size_t)plan_slot(plan, wk, s0 + (i < ns ? i : ns - 1), n_slots) * F;
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
                const int g = g0 + gg < G ? g0 + gg : G - 1;
                hv[i][gg] = hs[g * kGroup + lane];
            }
        }
        float gsum[S][NG];
#pragma unroll
        for (int i = 0; i < S; ++i)
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
                ((float *)hw[wave][i][gg])[lane] = hv[i][gg];
                gsum[i][gg] = wave_sum_all(hv[i][gg]);
            }
        float acc[S];
#pragma unroll
        for (int i = 0; i < S; ++i) acc[i] = 0.f;
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
            const int c = c0 + j, gg = c / 2 - g0;
            float wf[32];
            const uint32_t wd[4] = {wq[j].x, wq[j].y, wq[j].z, wq[j].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {  // element 8k + i = nibble i of word k
                const uint32_t lo = wd[k] & 0x0F0F0F0Fu, hi = (wd[k] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    wf[8 * k + 2 * b] = (float)((lo >> (8 * b)) & 0xFFu);
                    wf[8 * k + 2 * b + 1] = (float)((hi >> (8 * b)) & 0xFFu);
                }
            }
#pragma unroll
            for (int i = 0; i < S; ++i) {
                if (i >= ns) break;  // uniform
                const float gs = (c & 1) ? 0.f : gsum[i][gg];
                const float4 *hc4 = &hw[wave][i][gg][(c & 1) * 8];  // uniform address: broadcast reads
                float hc[32];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const float4 v = hc4[t];
                    hc[4 * t] = v.x;
                    hc[4 * t + 1] = v.y;
                    hc[4 * t + 2] = v.z;
                    hc[4 * t + 3] = v.w;
                }
                float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    d0 = fmaf(wf[t], hc[t], d0);
                    d1 = fmaf(wf[8 + t], hc[8 + t], d1);
                    d2 = fmaf(wf[16 + t], hc[16 + t], d2);
                    d3 = fmaf(wf[24 + t], hc[24 + t], d3);
                }
                acc[i] += fmaf(ws[j], (d0 + d1) + (d2 + d3), wb[j] * gs);
            }
        }
#pragma unroll
        for (int i = 0; i < S; ++i)
            if (i < ns) part[wave][i][lane] = acc[i];
        __syncthreads();
        for (int i = wave; i < ns; i += NW) {
            float v = part[0][i][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) v += part[w][i][lane];
            y[(size_t)plan_slot(plan, wk, s0 + i, n_slots) * H + m] = v;
        }
        __syncthreads();
    }
}

// ----------------------------------------------------- down, MFMA tiles

// Experts with many tokens, column layout: v_mfma_f32_16x16x32_bf16 with h
// carried exactly.  Each fp32 h is split into three bf16 parts by
// truncation, h = hi + mid + lo with every bit of h in exactly one part
// (the low 16 bits of each remainder are dropped into the next), so the
// three MFMAs per 32 inputs sum (1 + q / 16) * h with every product exact
// in fp32, as the fp32 FMA kernels do; only the order of the fp32
// additions differs.  Per 64-group the result D gives
//   y += 16 s * D + (b - 16 s) * sum(h over the group),
// the group sum taken from the fp32 h.  A workgroup of NW waves owns
// 16 * RT rows of the expert; wave w takes GW of the 64-groups; lane
// (r, kq) holds word kq of chunks 2g and 2g + 1 of row r of each 16-row
// tile (256 contiguous bytes per chunk and tile across the wave) and the h
// of token r in the same nibble pairing as gate+up's MFMA kernel.  Partial
// sums meet in LDS and are added in wave order; tokens go in tiles of 16.
template <int NW, int GW, int RT>
__global__ __launch_bounds__(NW * kWave) void down_mfma_kernel(const uint32_t *__restrict__ q,
                                                               const uint16_t *__restrict__ sc,
                                                               const uint16_t *__restrict__ bi,
                                                               const float *__restrict__ h,
                                                               float *__restrict__ y, PlanView plan,
                                                               int hidden, int n_experts, int n_slots,
                                                               int min_count) {
    constexpr int ROWS = 16 * RT;
    constexpr int G = NW * GW, C = 2 * G, F = C * 32;
    extern __shared__ float smem[];
    Work wk;
    if (!plan_expert(plan, blockIdx.y, n_experts, n_slots, &wk)) return;
    if (wk.count < min_count) return;  // the VALU kernel's expert
    const int H = hidden;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int r16 = lane & 15, kq = lane >> 4;
    const int m0 = blockIdx.x * ROWS;
    const int g0 = wave * GW;

    // h of the lane's token (8 values of chunk 2g and 8 of chunk 2g + 1 per
    // group); unconditional loads (a lane without a token reads slot 0's
    // row and zeroes it), so the first tile's go out with the weights
    float hv[GW][2][8];
    auto load_h = [&](int slot, bool live) {
        const float *hr = h + (size_t)slot * F;
#pragma unroll
        for (int gi = 0; gi < GW; ++gi)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const float4 *p4 = (const float4 *)(hr + (2 * (g0 + gi) + c2) * 32 + 8 * kq);
                const float4 lo = p4[0], hi = p4[1];
                hv[gi][c2][0] = lo.x; hv[gi][c2][1] = lo.y; hv[gi][c2][2] = lo.z; hv[gi][c2][3] = lo.w;
                hv[gi][c2][4] = hi.x; hv[gi][c2][5] = hi.y; hv[gi][c2][6] = hi.z; hv[gi][c2][7] = hi.w;
            }
#pragma unroll
        for (int gi = 0; gi < GW; ++gi)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                for (int i = 0; i < 8; ++i) hv[gi][c2][i] = live ? hv[gi][c2][i] : 0.f;
    };
    // order of issue: the first tile's slot lookup, the weights, then the h
    // that needs the slot (its wait then covers the lookup alone)
    int slot = plan_slot(plan, wk, r16 < wk.count ? r16 : wk.count - 1, n_slots);
    __builtin_amdgcn_sched_barrier(0);

    // this wave's weights: word kq of chunks 2g, 2g + 1 of each row tile
    // (ordinary loads, as in the MFMA gate+up kernel)
    uint32_t wa[GW][RT][2];
#pragma unroll
    for (int gi = 0; gi < GW; ++gi)
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const int c = 2 * (g0 + gi) + c2;
                wa[gi][t][c2] = q[(((size_t)wk.e * C + c) * H + m0 + 16 * t + r16) * 4 + kq];
            }
    __builtin_amdgcn_sched_barrier(0);
    slot = r16 < wk.count ? slot : 0;
    load_h(slot, r16 < wk.count);
    // per [group][row]: 16 * scale, and bias - 16 * scale (the weights go
    // into the MFMA as 1 + q / 16)
    float *ss = smem, *sb = smem + G * ROWS;
    float *part = smem + 2 * G * ROWS;  // [wave][lane][4 * RT]
    for (int i = threadIdx.x; i < ROWS * G; i += NW * kWave) {
        const int g = i / ROWS, r = i - g * ROWS;
        const size_t si = ((size_t)wk.e * G + g) * H + m0 + r;
        const float s1 = f16_bits_to_f32(sc[si]);
        ss[g * ROWS + r] = 16.f * s1;
        sb[g * ROWS + r] = fmaf(-16.f, s1, f16_bits_to_f32(bi[si]));
    }
    __syncthreads();

    for (int t0 = 0; t0 < wk.count; t0 += kMfmaTokens) {
        const int nt = wk.count - t0 < kMfmaTokens ? wk.count - t0 : kMfmaTokens;
        const bool live = r16 < nt;  // this lane's token column
        if (t0 > 0) {
            slot = live ? plan_slot(plan, wk, t0 + r16, n_slots) : 0;
            load_h(slot, live);
        }
        f32x4_t acc[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int gi = 0; gi < GW; ++gi) {
            const int g = g0 + gi;
            uint32_t hb[2][3][4];
            float hs = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                split3_pairs(hv[gi][c2], hb[c2]);
#pragma unroll
                for (int i = 0; i < 8; ++i) hs += hv[gi][c2][i];
            }
            hs = swap16_sum(hs, hs);  // add the four lanes of the token
            hs = swap32_sum(hs, hs);
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                f32x4_t d = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    uint32_t a[4];
                    q4_pairs16(wa[gi][t][c2], a);
                    d = mfma16x16x32(a, hb[c2][0], d);
                    d = mfma16x16x32(a, hb[c2][1], d);
                    d = mfma16x16x32(a, hb[c2][2], d);
                }
                const float4 s1 = *(const float4 *)(ss + g * ROWS + 16 * t + 4 * kq);
                const float4 b1 = *(const float4 *)(sb + g * ROWS + 16 * t + 4 * kq);
                acc[t][0] += fmaf(s1.x, d[0], b1.x * hs);
                acc[t][1] += fmaf(s1.y, d[1], b1.y * hs);
                acc[t][2] += fmaf(s1.z, d[2], b1.z * hs);
                acc[t][3] += fmaf(s1.w, d[3], b1.w * hs);
            }
        }
        float *mine = part + ((size_t)wave * kWave + lane) * (4 * RT);
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) mine[t * 4 + i] = acc[t][i];
        __syncthreads();
        // add the partials in wave order: output o = (row tile, row of the
        // lane's four) goes to wave o % NW
        if (live) {
            for (int o = wave; o < 4 * RT; o += NW) {
                const int t = o / 4, i = o % 4;
                float v = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) v += part[((size_t)w * kWave + lane) * (4 * RT) + t * 4 + i];
                y[(size_t)slot * H + m0 + 16 * t + 4 * kq + i] = v;
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- combine

// The output element from the fp32 sum o: one rounding to the output dtype;
// with a residual, act(residual + act(o)) in fp32 (NaN stays NaN).
template <bool BF16>
__device__ __forceinline__ void store_out(float o, const void *residual, void *out, size_t i) {
    if constexpr (BF16) {
        uint16_t r = f32_to_bf16_rne(o);
        if (residual) {
            const float sum = bf16_bits_to_f32(((const uint16_t *)residual)[i]) + bf16_bits_to_f32(r);
            r = f32_to_bf16_rne(sum);
        }
        ((uint16_t *)out)[i] = r;
    } else {
        if (residual) o = ((const float *)residual)[i] + o;
        ((float *)out)[i] = o;
    }
}

// The residual as fp32 (a bf16 value widens exactly), and the output from o
// and that value: the same arithmetic as store_out, with the residual read
// ahead by the caller.
template <bool BF16>
__device__ __forceinline__ float load_residual(const void *residual, size_t i) {
    if constexpr (BF16)
        return bf16_bits_to_f32(((const uint16_t *)residual)[i]);
    else
        return ((const float *)residual)[i];
}

template <bool BF16>
__device__ __forceinline__ void store_out_res(float o, bool has_res, float rv, void *out, size_t i) {
    if constexpr (BF16) {
        uint16_t r = f32_to_bf16_rne(o);
        if (has_res) r = f32_to_bf16_rne(rv + bf16_bits_to_f32(r));
        ((uint16_t *)out)[i] = r;
    } else {
        if (has_res) o = rv + o;
        ((float *)out)[i] = o;
    }
}

// out[t][m] = sum_j w[t][j] * (y[t * k + j][m] * dscale[e]): fp32 FMAs in j
// order, the down-projection sidecar (if any) applied to y as it enters
// the sum; a token with an invalid expert id gets NaN.  The loads of up to
// kCombineBatch slots go out together (ids, weights, y, then the sidecar
// entries the ids name) before any of them is used, and the residual's
// ahead of them all: one memory round trip per batch instead of one per
// slot.  Loads past top_k repeat its last slot and are not used; with no
// sidecar or residual the same loads read valid memory that is not used,
// so no load sits under a branch.
constexpr int kCombineBatch = 8;

template <bool BF16>
__global__ __launch_bounds__(kBlock) void combine_kernel(const float *__restrict__ y,
                                                         const int *__restrict__ topk_idx,
                                                         const float *__restrict__ topk_w,
                                                         const float *__restrict__ dscale,
                                                         const void *residual, void *out,
                                                         int hidden, int top_k, int n_experts) {
    constexpr int U = kCombineBatch;
    const int t = blockIdx.y;
    const int m = blockIdx.x * kBlock + threadIdx.x;
    if (m >= hidden) return;
    const size_t oi = (size_t)t * hidden + m;
    const bool has_res = residual != nullptr;
    const float rv = load_residual<BF16>(has_res ? residual : (const void *)y, has_res ? oi : (size_t)m);
    const float *dsrc = dscale ? dscale : topk_w;
    float acc = 0.f;
    bool bad = false;
    for (int j0 = 0; j0 < top_k; j0 += U) {
        int e[U];
        float w[U], v[U], ds[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int s = t * top_k + (j0 + i < top_k ? j0 + i : top_k - 1);
            e[i] = topk_idx[s];
            w[i] = topk_w[s];
            v[i] = y[(size_t)s * hidden + m];
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const bool ok = (unsigned)e[i] < (unsigned)n_experts;
            ds[i] = dsrc[dscale && ok ? e[i] : 0];
        }
        // every product formed, the sum taking the live ones (x * 1 is x)
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const bool invalid = (unsigned)e[i] >= (unsigned)n_experts;
            const bool live = j0 + i < top_k;
            const float x = v[i] * (dscale && !invalid ? ds[i] : 1.f);
            const float a = fmaf(w[i], x, acc);
            acc = live ? a : acc;
            bad |= live && invalid;
        }
    }
    if (bad) acc = __builtin_nanf("");
    store_out_res<BF16>(acc, has_res, rv, out, oi);
}

// ------------------------------------ down + combine, token by token

// For a token alone there is nothing to deduplicate, and for a handful
// little: workgroup (block of RW output rows, token t) takes all k of the
// token's experts, lane (j, r) = expert j, row r (RW = 64 / KP, KP = top_k
// rounded up to a power of two), and combines the k results in LDS, so no
// combine launch follows.  Waves split
// dff exactly as down_cols_kernel<NW, CPW> does and every sum is formed in
// the same order (chunk dot products, per-wave chunk sums, wave-ordered
// totals, group sums from the same wave reduction, then the j-ordered
// combine), so a token's output is bitwise that of the batched kernels.
constexpr int kHPad = 4;  // floats between the LDS rows of h (bank spread)

// Workgroups are dealt to the 8 XCDs round robin by id.  Give each XCD a
// contiguous range of blocks instead, so neighbouring row blocks, which
// share cache lines of the weights' scales and biases, share one L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_block(int b, int n) {
    if (n % kXcds) return b;
    return (b % kXcds) * (n / kXcds) + b / kXcds;
}

// Sixteen-wave workgroups with one row block and four chunks per wave fit
// 64 registers, so two workgroups share a CU (eight waves per SIMD); the
// other shapes would spill there and keep the compiler's choice.
template <int NW, int CPW, int RB>
constexpr int down_token_waves_per_simd() { return NW >= 16 && RB == 1 && CPW == 4 ? 8 : 1; }

template <int NW, int CPW, int KP, int RB, bool BF16>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(down_token_waves_per_simd<NW, CPW, RB>())))
void down_token_kernel(const uint4 *__restrict__ q,
                                                                const uint16_t *__restrict__ sc,
                                                                const uint16_t *__restrict__ bi,
                                                                const float *__restrict__ h,
                                                                const int *__restrict__ topk_idx,
                                                                const float *__restrict__ topk_w,
                                                                const float *__restrict__ dscale,
                                                                const void *residual, void *out,
                                                                int hidden, int dff, int n_experts, int top_k) {
    constexpr int RW = kWave / KP;
    constexpr int RWB = RW * RB;  // rows per workgroup: RB blocks of RW rows share the staged h
    // dff = 32 * NW * CPW (the geometry's own shape): compile-time strides
    constexpr int C = NW * CPW, F = 32 * C, G = C / 2, HS = F + kHPad;
    extern __shared__ float smem[];
    const int H = hidden;
    float *hl = smem;                        // [k][HS]       h of the token's slots
    float *gs = smem + top_k * HS;           // [k][G]        sums of h over each 64-group
    float *part = gs + top_k * G;            // [NW][RB][64]  per-wave sums
    float *sl = part + NW * RB * kWave;      // [2][k][G][RWB] scales, then biases
    const int t = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int j = lane / RW, r = lane % RW;
    const bool live = j < top_k;
    const int mb = xcd_block(blockIdx.x, gridDim.x) * RWB;
    // Every load ahead of the weights is unconditional (clamped indices, the
    // value selected afterwards): a load under a branch makes the compiler
    // wait for all loads in flight where the branch joins.
    const int jc = live ? j : top_k - 1;
    const int e_ld = topk_idx[t * top_k + jc];
    const float w_ld = topk_w[t * top_k + jc];
    const int e_raw = live ? e_ld : 0;
    const float wj = live ? w_ld : 0.f;  // read now, used by the combine
    const int c0 = wave * CPW;

    // h of the token's slots, staged below: wave w takes the (slot, group)
    // pairs w, w + NW, ... (at most MAXP of them).  These loads need no
    // expert id, so they go out first, behind only the id load itself, and
    // the weights' latency overlaps theirs.
    constexpr int MAXP = (KP * CPW + 1) / 2;  // k * G / NW <= KP * (NW * CPW / 2) / NW
    const float *ht = h + (size_t)t * top_k * F;
    const int n_pairs = top_k * G;
    float hv0[MAXP];
#pragma unroll
    for (int i = 0; i < MAXP; ++i) {
        const int p = wave + i * NW;
        const int pc = p < n_pairs ? p : n_pairs - 1;  // past the end: loaded, not used
        const int jp = pc / G, g = pc - jp * G;
        hv0[i] = ht[(size_t)jp * F + g * kGroup + lane];
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the h loads ahead of the dependent ones

    const int e = (unsigned)e_raw < (unsigned)n_experts ? e_raw : 0;  // invalid: NaN below
    // Scales and biases of the block's RWB rows, 4 rows (8 bytes) per load:
    // unit u = ((sb * k + expert) * G + group) * RWB/4 + quarter.  Loading them
    // per lane would touch one cache line per 16 bytes used.  They go out
    // before the weights, so converting them waits for them alone.
    constexpr int QPR = RWB / 4;  // RW >= 4 as top_k <= 16
    const int n_units = 2 * top_k * G * QPR;
    uint2 su[(2 * KP * G * QPR + NW * kWave - 1) / (NW * kWave)];
#pragma unroll
    for (int i = 0; i < (int)(sizeof(su) / sizeof(su[0])); ++i) {
        const int u = threadIdx.x + i * NW * kWave;
        const int uc = u < n_units ? u : n_units - 1;  // past the end: loaded, not used
        const int qq = uc % QPR, g = (uc / QPR) % G, jx = (uc / (QPR * G)) % top_k, sb = uc / (QPR * G * top_k);
        // expert of slot jx from lane (jx, 0), which holds it already: a
        // second load of topk_idx here would wait for every load before it
        // (vector loads retire in order)
        const int ex = __builtin_amdgcn_ds_bpermute(jx * RW * 4, e);
        const uint16_t *src = sb ? bi : sc;
        su[i] = *(const uint2 *)(src + ((size_t)ex * G + g) * H + mb + 4 * qq);
    }
    __builtin_amdgcn_sched_barrier(0);
    uint4 wq[RB][CPW];
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int jj = 0; jj < CPW; ++jj)
            wq[b][jj] = load_stream(q + ((size_t)e * C + (c0 + jj)) * H + mb + b * RW + r);
    // down-projection sidecar; without one, a load of topk_w[0] (used by no
    // one) keeps the load unconditional and in the global address space (a
    // generic-pointer load would wait for every load in flight)
    const float ds_ld = dscale ? dscale[e] : topk_w[0];
    const float dsj = (dscale && live) ? ds_ld : 1.f;
    // the residual of the output this lane stores (row block `wave`, if it
    // has one), read now rather than after the combine; without a
    // residual (or a row block) a valid word is read and not used
    const bool has_res = residual != nullptr;
    const int rb_res = wave < RB ? wave : 0;
    const float rv = load_residual<BF16>(has_res ? residual : (const void *)topk_w,
                                         has_res ? (size_t)t * H + mb + rb_res * RW + (lane < RW ? r : 0) : 0);
    __builtin_amdgcn_sched_barrier(0);

    // stage h and its group sums while the weights are in flight; a pair
    // past the end repeats the last pair's value and sum into the same LDS
    // words as the wave that owns it
#pragma unroll
    for (int i = 0; i < MAXP; ++i) {
        const int p = wave + i * NW;
        const int pc = p < n_pairs ? p : n_pairs - 1;
        const int jp = pc / G, g = pc - jp * G;
        hl[jp * HS + g * kGroup + lane] = hv0[i];
        const float sum = wave_sum_all(hv0[i]);
        if (lane == 0) gs[jp * G + g] = sum;
    }
#pragma unroll
    for (int i = 0; i < (int)(sizeof(su) / sizeof(su[0])); ++i) {
        const int u = threadIdx.x + i * NW * kWave;
        if (u < n_units) {
            float *d = sl + (size_t)u * 4;  // unit u covers rows 4 * (u % QPR) .. + 3
            const uint32_t w0 = su[i].x, w1 = su[i].y;
            d[0] = f16_bits_to_f32((uint16_t)w0);
            d[1] = f16_bits_to_f32((uint16_t)(w0 >> 16));
            d[2] = f16_bits_to_f32((uint16_t)w1);
            d[3] = f16_bits_to_f32((uint16_t)(w1 >> 16));
        }
    }
    __syncthreads();

    float acc[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[b] = 0.f;
    if (live) {
#pragma unroll
        for (int jj = 0; jj < CPW; ++jj) {
            const int c = c0 + jj, g = c / 2;
            const float gsum = (c & 1) ? 0.f : gs[j * G + g];
            const float4 *hc = (const float4 *)(hl + j * HS + c * 32);
            float hv[32];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 v = hc[i];
                hv[4 * i] = v.x;
                hv[4 * i + 1] = v.y;
                hv[4 * i + 2] = v.z;
                hv[4 * i + 3] = v.w;
            }
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                const float ws = sl[((size_t)j * G + g) * RWB + b * RW + r];
                const float wb = (c & 1) ? 0.f : sl[(((size_t)top_k + j) * G + g) * RWB + b * RW + r];
                float wf[32];
                const uint32_t wd[4] = {wq[b][jj].x, wq[b][jj].y, wq[b][jj].z, wq[b][jj].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t lo = wd[k] & 0x0F0F0F0Fu, hi = (wd[k] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                    for (int bb = 0; bb < 4; ++bb) {
                        wf[8 * k + 2 * bb] = (float)((lo >> (8 * bb)) & 0xFFu);
                        wf[8 * k + 2 * bb + 1] = (float)((hi >> (8 * bb)) & 0xFFu);
                    }
                }
                float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    d0 = fmaf(wf[i], hv[i], d0);
                    d1 = fmaf(wf[8 + i], hv[8 + i], d1);
                    d2 = fmaf(wf[16 + i], hv[16 + i], d2);
                    d3 = fmaf(wf[24 + i], hv[24 + i], d3);
                }
                acc[b] += fmaf(ws, (d0 + d1) + (d2 + d3), wb * gsum);
            }
        }
    }
    const bool bad = __builtin_amdgcn_ballot_w64(live && (unsigned)e_raw >= (unsigned)n_experts) != 0;
#pragma unroll
    for (int b = 0; b < RB; ++b) part[(wave * RB + b) * kWave + lane] = acc[b];
    __syncthreads();
    // wave w finishes row blocks w, w + NW, ...: lane (j, r) sums expert j's
    // partials for row r in wave order, then lanes r < RW combine in j order
    for (int b = wave; b < RB; b += NW) {
        float y = part[b * kWave + lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) y += part[(w * RB + b) * kWave + lane];
        part[b * kWave + lane] = y * dsj;  // LDS operations of one wave complete in order
        __builtin_amdgcn_wave_barrier();
        float o = 0.f;
        for (int jk = 0; jk < top_k; ++jk) {
            const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), jk * RW));
            o = fmaf(wk, part[b * kWave + jk * RW + r], o);
        }
        if (bad) o = __builtin_nanf("");
        if (lane < RW) {
            const size_t oi = (size_t)t * H + mb + b * RW + r;
            if (b == wave)
                store_out_res<BF16>(o, has_res, rv, out, oi);
            else
                store_out<BF16>(o, residual, out, oi);
        }
    }
}

// ------------------------------------------------------------ dispatching

template <int LPR, int NV>
static moe_status launch_gate_up(const GateUpArgs &a, bool bf16, int groups_y, hipStream_t s) {
    constexpr int RI = gate_up_ri<LPR, NV>();
    constexpr int rows = (kWave / LPR) * RI;
    const dim3 grid((a.dff + rows - 1) / rows, groups_y);
    if (bf16)
        hipLaunchKernelGGL((gate_up_kernel<LPR, NV, RI, true>), grid, dim3(kWave), 0, s, a);
    else
        hipLaunchKernelGGL((gate_up_kernel<LPR, NV, RI, false>), grid, dim3(kWave), 0, s, a);
    return MOE_OK;
}

template <int LPR, int NV>
static moe_status launch_down(DownArgs a, int groups_y, int max_count, hipStream_t s) {
    constexpr int RI = 1;
    constexpr int rows = (kWave / LPR) * RI * (kBlock / kWave);
    const size_t per_slot = down_rows_slot_bytes(a.dff);
    int S = (int)(kDownRowsLdsBytes / per_slot);
    if (S < 1) return MOE_ERR_UNSUPPORTED;
    if (S > max_count) S = max_count;
    a.slots_per_stage = S;
    const dim3 grid((a.hidden + rows - 1) / rows, groups_y);
    hipLaunchKernelGGL((down_kernel<LPR, NV, RI>), grid, dim3(kBlock), S * per_slot, s, a);
    return MOE_OK;
}

template <int NW, int CPW>
static void launch_down_cols_t(const moe_layer_t *L, const float *h, float *y, PlanView pv, int groups_y,
                               int n_slots, int max_count, hipStream_t s) {
    const dim3 grid(L->hidden / kWave, groups_y);
    hipLaunchKernelGGL((down_cols_kernel<NW, CPW>), grid, dim3(NW * kWave), 0, s, (const uint4 *)L->down_q,
                       L->down_s, L->down_b, h, y, pv, L->hidden, L->dff, L->n_experts, n_slots, max_count);
}

static moe_status launch_down_cols(const moe_layer_t *L, const float *h, float *y, PlanView pv, int groups_y,
                                   int n_slots, int max_count, hipStream_t s) {
    int nw, cpw;
    if (!pick_down_cols(L->dff, &nw, &cpw)) return MOE_ERR_UNSUPPORTED;
    switch (nw * 100 + cpw) {
#define MOE_DC(NW, CPW) \
    case NW * 100 + CPW: launch_down_cols_t<NW, CPW>(L, h, y, pv, groups_y, n_slots, max_count, s); break;
        MOE_DC(4, 1) MOE_DC(4, 3) MOE_DC(4, 5) MOE_DC(4, 7)
        MOE_DC(8, 1) MOE_DC(8, 2) MOE_DC(12, 2)
        MOE_DC(16, 2) MOE_DC(16, 3) MOE_DC(16, 4)
#undef MOE_DC
        default: return MOE_ERR_UNSUPPORTED;
    }
    return MOE_OK;
}

// Smallest power of two >= top_k (1..16).
static int pow2_at_least(int k) {
    int p = 1;
    while (p < k) p *= 2;
    return p;
}

// LDS budget of the token-major down kernel: what one workgroup may hold on
// the current device (160 KiB on gfx950; queried once per device, 64 KiB if
// the query fails); and the token counts from which the kernel takes two
// and four row blocks per workgroup.
constexpr int kTokenRb2 = 2, kTokenRb4 = 4;
static size_t down_token_lds_budget() {
    static std::mutex mu;
    static size_t budget[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 65536;
    std::lock_guard<std::mutex> lock(mu);
    if (!budget[dev]) {
        int v = 0;
        budget[dev] = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0
                          ? (size_t)v
                          : 65536;
    }
    return budget[dev];
}

static size_t down_token_lds(const moe_layer_t *L, int nw, int rb) {
    const int F = L->dff, G = F / kGroup, k = L->top_k;
    const int rw = kWave / pow2_at_least(k);
    return ((size_t)k * (F + kHPad) + (size_t)k * G + (size_t)nw * rb * kWave + (size_t)2 * k * G * rw * rb) *
           sizeof(float);
}

template <int NW, int CPW, int KP, int RB>
static void launch_down_token_rb(const moe_layer_t *L, int n_tokens, const float *h, const int32_t *idx,
                                 const float *w, const void *residual, void *out, size_t lds, hipStream_t s) {
    const dim3 grid(L->hidden / (kWave / KP * RB), n_tokens);
    const uint4 *q = (const uint4 *)L->down_q;
    if (L->act_dtype == MOE_DTYPE_BF16)
        hipLaunchKernelGGL((down_token_kernel<NW, CPW, KP, RB, true>), grid, dim3(NW * kWave), lds, s, q,
                           L->down_s, L->down_b, h, idx, w, L->down_scale, residual, out, L->hidden, L->dff,
                           L->n_experts, L->top_k);
    else
        hipLaunchKernelGGL((down_token_kernel<NW, CPW, KP, RB, false>), grid, dim3(NW * kWave), lds, s, q,
                           L->down_s, L->down_b, h, idx, w, L->down_scale, residual, out, L->hidden, L->dff,
                           L->n_experts, L->top_k);
}

template <int NW, int CPW, int KP>
static void launch_down_token_t(const moe_layer_t *L, int n_tokens, const float *h, const int32_t *idx,
                                const float *w, const void *residual, void *out, int rb, hipStream_t s) {
    const size_t lds = down_token_lds(L, NW, rb);
    if (rb == 4)
        launch_down_token_rb<NW, CPW, KP, 4>(L, n_tokens, h, idx, w, residual, out, lds, s);
    else if (rb == 2)
        launch_down_token_rb<NW, CPW, KP, 2>(L, n_tokens, h, idx, w, residual, out, lds, s);
    else
        launch_down_token_rb<NW, CPW, KP, 1>(L, n_tokens, h, idx, w, residual, out, lds, s);
}

template <int NW, int CPW>
static moe_status launch_down_token_k(const moe_layer_t *L, int n_tokens, const float *h, const int32_t *idx,
                                      const float *w, const void *residual, void *out, int rb,
                                      hipStream_t s) {
    switch (pow2_at_least(L->top_k)) {
        case 1: launch_down_token_t<NW, CPW, 1>(L, n_tokens, h, idx, w, residual, out, rb, s); break;
        case 2: launch_down_token_t<NW, CPW, 2>(L, n_tokens, h, idx, w, residual, out, rb, s); break;
        case 4: launch_down_token_t<NW, CPW, 4>(L, n_tokens, h, idx, w, residual, out, rb, s); break;
        case 8: launch_down_token_t<NW, CPW, 8>(L, n_tokens, h, idx, w, residual, out, rb, s); break;
        case 16: launch_down_token_t<NW, CPW, 16>(L, n_tokens, h, idx, w, residual, out, rb, s); break;
        default: return MOE_ERR_UNSUPPORTED;
    }
    return MOE_OK;
}

// Row blocks per workgroup of the token-major down kernel: one for a single
// token (the most workgroups, the shortest path), more as tokens add
// workgroups, so the staged h of a token serves more rows; bounded by the
// LDS budget and by hidden.  Sixteen-wave workgroups (dff 1536, 2048) spill
// at four row blocks; with four chunks per wave (dff 2048) they take two
// row blocks for one token, where a workgroup stages as many bytes of h as
// it reads of weights (wide layer, one token: 33.3 -> 29.5 us per step),
// and one from two tokens, two workgroups per CU (four tokens: 120.2 ->
// 117.3 us).
static int down_token_rb(const moe_layer_t *L, int n_tokens, int nw, int cpw) {
    const int rw = kWave / pow2_at_least(L->top_k);
    const int rb_max = nw >= 16 ? 2 : 4;
    int rb0 = n_tokens >= kTokenRb4 ? 4 : n_tokens >= kTokenRb2 ? 2 : 1;
    if (nw >= 16 && cpw == 4) rb0 = n_tokens == 1 ? 2 : 1;
    for (int rb = rb0 < rb_max ? rb0 : rb_max; rb > 1; rb /= 2)
        if (L->hidden % (rw * rb) == 0 && down_token_lds(L, nw, rb) <= down_token_lds_budget()) return rb;
    return 1;
}

// The token-major down + combine kernel, when the layer has column-layout
// down weights and its LDS fits; MOE_ERR_UNSUPPORTED otherwise (the caller
// then takes the deduplicated kernels).
static moe_status launch_down_token(const moe_layer_t *L, int n_tokens, const float *h, const int32_t *idx,
                                    const float *w, const void *residual, void *out, hipStream_t s) {
    int nw, cpw;
    if (L->down_layout != MOE_DOWN_COLS || !pick_down_cols(L->dff, &nw, &cpw)) return MOE_ERR_UNSUPPORTED;
    if (L->hidden % (kWave / pow2_at_least(L->top_k))) return MOE_ERR_UNSUPPORTED;
    if (down_token_lds(L, nw, 1) > down_token_lds_budget()) return MOE_ERR_UNSUPPORTED;
    const int rb = down_token_rb(L, n_tokens, nw, cpw);
    switch (nw * 100 + cpw) {
#define MOE_DT(NW, CPW) \
    case NW * 100 + CPW: return launch_down_token_k<NW, CPW>(L, n_tokens, h, idx, w, residual, out, rb, s);
        MOE_DT(4, 1) MOE_DT(4, 3) MOE_DT(4, 5) MOE_DT(4, 7)
        MOE_DT(8, 1) MOE_DT(8, 2) MOE_DT(12, 2)
        MOE_DT(16, 2) MOE_DT(16, 3) MOE_DT(16, 4)
#undef MOE_DT
        default: return MOE_ERR_UNSUPPORTED;
    }
}

static int groups_y_of(const moe_layer_t *layer, int n_tokens) {
    const int n_slots = n_tokens * layer->top_k;
    return n_slots < layer->n_experts ? n_slots : layer->n_experts;
}

// Experts with at least this many slots take the MFMA kernel (when the batch
// can have such experts at all and the layer suits it).
constexpr int kMfmaMinCount = 3;
// The MFMA kernels are launched only for batches of this many tokens or
// more.  Below, few experts reach kMfmaMinCount tokens, and the extra
// workgroups (one per row block and distinct expert, most of them finding
// no such expert) cost more than the dot2 kernels save: measured on the
// decode layer shape, 16 tokens is where Zipf-skewed routing starts to gain.
constexpr int kMfmaMinTokens = 16;
// 16-row tiles per workgroup: two, or one where a wave's registers would not
// hold two (more than eight waves, i.e. hidden above 2048).

// Waves (NW) and 64-groups per wave (GW) of the MFMA gate+up kernel for a
// hidden size; false when it has no instance.
static bool mfma_gate_up_shape(const moe_layer_t *layer, int *nw, int *gw) {
    if (layer->act_dtype != MOE_DTYPE_BF16 || layer->hidden % kGroup) return false;
    const int G = layer->hidden / kGroup;
    if (G % 4) return false;
    switch (G / 4) {  // the instantiated workgroup sizes (MOE_GUM below)
        case 1: case 2: case 4: case 6: case 8: case 12: case 16: break;
        default: return false;  // dot2 kernels at every batch size
    }
    *gw = 4;
    *nw = G / 4;
    return true;
}

static size_t mfma_gate_up_lds(const moe_layer_t *layer, int nw) {
    const int G = layer->hidden / kGroup, rt = mfma_row_tiles(nw), ROWS = 16 * rt;
    return ((size_t)4 * G * ROWS + (size_t)nw * kWave * 8 * rt) * sizeof(float);
}

template <int LPR, int NV, int NW, int GW>
static moe_status launch_gate_up_mixed_t(const moe_layer_t *layer, const GateUpArgs &ga, int groups_y,
                                         hipStream_t stream) {
    constexpr int RT = mfma_row_tiles(NW);
    constexpr int RI = gate_up_ri<LPR, NV>();
    const int rb_mfma = (layer->dff + 16 * RT - 1) / (16 * RT);
    const int rows_valu = (kWave / LPR) * RI;
    const int rb_valu = (layer->dff + rows_valu - 1) / rows_valu;
    const int n_valu = rb_valu * groups_y;
    const int mfma_blocks = rb_mfma * groups_y;
    const dim3 grid(mfma_blocks + (n_valu + NW - 1) / NW);
    hipLaunchKernelGGL((gate_up_mixed_kernel<LPR, NV, RI, NW, GW, RT>), grid, dim3(NW * kWave),
                       mfma_gate_up_lds(layer, NW), stream, ga, mfma_blocks, rb_mfma, rb_valu, n_valu, kMfmaMinCount);
    return MOE_OK;
}

// One launch for both gate+up variants, for the hidden sizes that have an
// instance (the dot2 geometry and the MFMA shape both follow from hidden):
// 256 to 2048.  Beyond, a 12- or 16-wave block cannot give the dot2 waves
// their registers, and the two variants go in two launches.
static moe_status launch_gate_up_mixed(const moe_layer_t *layer, const GateUpArgs &ga, const Geometry &gu, int nw,
                                       int gw, int groups_y, hipStream_t stream) {
    if (gw != 4) return MOE_ERR_UNSUPPORTED;
    const int key = (gu.lpr * 8 + gu.nv) * 100 + nw;
    switch (key) {
#define MOE_GMX(LPR, NV, NW) \
    case (LPR * 8 + NV) * 100 + NW: return launch_gate_up_mixed_t<LPR, NV, NW, 4>(layer, ga, groups_y, stream);
        MOE_GMX(2, 4, 1) MOE_GMX(4, 4, 2) MOE_GMX(8, 4, 4) MOE_GMX(16, 3, 6) MOE_GMX(64, 1, 8)
#undef MOE_GMX
        default: return MOE_ERR_UNSUPPORTED;
    }
}

moe_status enqueue_gate_up(const moe_layer_t *layer, const void *x, int n_tokens, const moe_plan_t *plan,
                           void *workspace, hipStream_t stream) {
    const Workspace ws = workspace_layout(layer, n_tokens);
    float *h = (float *)((char *)workspace + ws.h_off);
    if (!fast_gate_up(layer)) return launch_generic_gate_up(layer, x, n_tokens, plan, h, stream);
    if (n_tokens >= kTileMinTokens && tile_gate_up_ok(layer))
        return launch_gate_up_tile(layer, x, n_tokens, plan, h, stream);
    Geometry gu;
    pick_geometry_gate_up(layer->hidden, &gu);
    int nw = 0, gw = 0;
    const bool use_mfma = n_tokens >= kMfmaMinTokens && mfma_gate_up_shape(layer, &nw, &gw);
    GateUpArgs ga{(const uint4 *)layer->gate_q, (const uint4 *)layer->up_q, layer->gate_s,
                  layer->gate_b, layer->up_s, layer->up_b, layer->expert_scale,
                  layer->clamp_limit, x, plan_view(plan), h, layer->hidden, layer->dff,
                  layer->n_experts, layer->top_k, n_tokens * layer->top_k,
                  use_mfma ? kMfmaMinCount - 1 : INT_MAX, layer->activation};
    const bool bf16 = layer->act_dtype == MOE_DTYPE_BF16;
    const int groups_y = groups_y_of(layer, n_tokens);
    moe_status st;
    if (use_mfma) {  // both variants in one launch where an instance exists
        st = launch_gate_up_mixed(layer, ga, gu, nw, gw, groups_y, stream);
        if (st != MOE_ERR_UNSUPPORTED) return st;
    }
    MOE_GEOMETRY_SWITCH(gu, st, launch_gate_up, ga, bf16, groups_y, stream)
    if (st != MOE_OK || !use_mfma) return st;
    const int rows = 16 * mfma_row_tiles(nw);
    const dim3 grid((layer->dff + rows - 1) / rows, groups_y);
    const size_t lds = mfma_gate_up_lds(layer, nw);
    switch (nw * 100 + gw) {
#define MOE_GUM(NW, GW)                                                                                  \
    case NW * 100 + GW:                                                                                  \
        hipLaunchKernelGGL((gate_up_mfma_kernel<NW, GW, mfma_row_tiles(NW)>), grid, dim3(NW * kWave), lds, stream, \
                           ga, kMfmaMinCount);                                                           \
        break;
        MOE_GUM(1, 4) MOE_GUM(2, 4) MOE_GUM(4, 4) MOE_GUM(6, 4) MOE_GUM(8, 4) MOE_GUM(12, 4) MOE_GUM(16, 4)
#undef MOE_GUM
        default: return MOE_ERR_UNSUPPORTED;
    }
    return MOE_OK;
}

// Batches up to this many tokens take the token-major down + combine kernel
// (one row of workgroups per token): with so few slots deduplication saves
// little of the down projection's bytes, and the combine launch goes away
// (measured faster than the deduplicated kernels plus combine at 2, 4 and
// 8 tokens).
constexpr int kTokenMajorMaxTokens = 8;

// The MFMA down kernel: waves (NW) and 64-groups per wave (GW) for a dff,
// 16-row tiles per workgroup (two: measured against one, four and eight at
// 32 and 256 tokens, more workgroups in flight beat fewer h re-reads); false
// when it has no instance.
constexpr int kMfmaDownRowTiles = 2;
static bool mfma_down_shape(const moe_layer_t *layer, int *nw, int *gw) {
    if (layer->down_layout != MOE_DOWN_COLS || layer->dff % kGroup) return false;
    if (layer->hidden % (16 * kMfmaDownRowTiles)) return false;
    const int G = layer->dff / kGroup;
    // twelve groups (dff 768): one group per wave, twelve waves; 71
    // registers, so two workgroups share a CU, against 120 and one six-wave
    // workgroup's worth of waves per SIMD pair with two groups per wave
    // (32 tokens: Zipf 87.2 -> 85.3 us, random 149.6 -> 144.9 us per step)
    if (G == 12) {
        *nw = 12;
        *gw = 1;
        return true;
    }
    for (int n = 8; n >= 2; n -= 2)
        if (G % n == 0 && G / n <= 4) {
            *nw = n;
            *gw = G / n;
            return true;
        }
    return false;
}

static moe_status launch_down_mfma(const moe_layer_t *L, const float *h, float *y, PlanView pv, int groups_y,
                                   int n_slots, int nw, int gw, hipStream_t s) {
    constexpr int RT = kMfmaDownRowTiles;
    const int G = L->dff / kGroup;
    const size_t lds = ((size_t)2 * G * 16 * RT + (size_t)nw * kWave * 4 * RT) * sizeof(float);
    const dim3 grid(L->hidden / (16 * RT), groups_y);
    switch (nw * 100 + gw) {
#define MOE_DM(NW, GW)                                                                                        \
    case NW * 100 + GW:                                                                                       \
        hipLaunchKernelGGL((down_mfma_kernel<NW, GW, RT>), grid, dim3(NW * kWave), lds, s, L->down_q, L->down_s, \
                           L->down_b, h, y, pv, L->hidden, L->n_experts, n_slots, kMfmaMinCount);             \
        break;
        MOE_DM(2, 1) MOE_DM(2, 2) MOE_DM(2, 3) MOE_DM(2, 4)
        MOE_DM(4, 1) MOE_DM(4, 2) MOE_DM(4, 3) MOE_DM(4, 4)
        MOE_DM(6, 1) MOE_DM(6, 2) MOE_DM(6, 3) MOE_DM(6, 4)
        MOE_DM(8, 1) MOE_DM(8, 2) MOE_DM(8, 3) MOE_DM(8, 4) MOE_DM(12, 1)
#undef MOE_DM
        default: return MOE_ERR_UNSUPPORTED;
    }
    return MOE_OK;
}

static moe_status enqueue_down_combine(const moe_layer_t *layer, int n_tokens, const int32_t *topk_idx,
                                       const float *topk_w, const moe_plan_t *plan,
                                       const void *residual, void *out, void *workspace,
                                       hipStream_t stream) {
    const Workspace ws = workspace_layout(layer, n_tokens);
    const float *h = (const float *)((char *)workspace + ws.h_off);
    float *y = (float *)((char *)workspace + ws.y_off);
    moe_status st;
    const bool fast = fast_down(layer);
    if (fast && n_tokens <= kTokenMajorMaxTokens) {
        st = launch_down_token(layer, n_tokens, h, topk_idx, topk_w, residual, out, stream);
        if (st != MOE_ERR_UNSUPPORTED) return st;
    }
    if (!fast) {
        st = launch_generic_down(layer, n_tokens, plan, h, y, stream);
    } else if (n_tokens >= kTileMinTokens && tile_down_ok(layer)) {
        st = launch_down_tile(layer, n_tokens, plan, h, y, stream);
    } else if (layer->down_layout == MOE_DOWN_COLS) {
        int nw = 0, gw = 0;
        const bool mfma = n_tokens >= kMfmaMinTokens && mfma_down_shape(layer, &nw, &gw);
        const int gy = groups_y_of(layer, n_tokens), n_slots = n_tokens * layer->top_k;
        st = launch_down_cols(layer, h, y, plan_view(plan), gy, n_slots, mfma ? kMfmaMinCount - 1 : INT_MAX, stream);
        if (st == MOE_OK && mfma) st = launch_down_mfma(layer, h, y, plan_view(plan), gy, n_slots, nw, gw, stream);
    } else {
        Geometry gd;
        pick_geometry(layer->dff, &gd);
        DownArgs da{(const uint4 *)layer->down_q, layer->down_s, layer->down_b, h, plan_view(plan), y,
                    layer->hidden, layer->dff, layer->n_experts, n_tokens * layer->top_k, 1};
        MOE_GEOMETRY_SWITCH(gd, st, launch_down, da, groups_y_of(layer, n_tokens), n_tokens, stream)
    }
    if (st != MOE_OK) return st;
    const dim3 cgrid((layer->hidden + kBlock - 1) / kBlock, n_tokens);
    if (layer->act_dtype == MOE_DTYPE_BF16)
        hipLaunchKernelGGL(combine_kernel<true>, cgrid, dim3(kBlock), 0, stream, y, topk_idx, topk_w,
                           layer->down_scale, residual, out, layer->hidden, layer->top_k, layer->n_experts);
    else
        hipLaunchKernelGGL(combine_kernel<false>, cgrid, dim3(kBlock), 0, stream, y, topk_idx, topk_w,
                           layer->down_scale, residual, out, layer->hidden, layer->top_k, layer->n_experts);
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_expert_gate_up(const moe_layer_t *layer, const void *x, int32_t n_tokens,
                                         const moe_plan_t *plan, void *workspace,
                                         size_t workspace_bytes, void *hip_stream) {
    moe_status st = check_step(layer, n_tokens, plan, workspace, workspace_bytes);
    if (st != MOE_OK || n_tokens == 0) return st;
    if ((st = check_x(x)) != MOE_OK) return st;
    st = enqueue_gate_up(layer, x, n_tokens, plan, workspace, (hipStream_t)hip_stream);
    if (st != MOE_OK) return st;
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

extern "C" moe_status moe_expert_down_combine(const moe_layer_t *layer, int32_t n_tokens,
                                              const int32_t *topk_idx, const float *topk_w,
                                              const moe_plan_t *plan, const void *residual,
                                              void *out, void *workspace, size_t workspace_bytes,
                                              void *hip_stream) {
    moe_status st = check_step(layer, n_tokens, plan, workspace, workspace_bytes);
    if (st != MOE_OK || n_tokens == 0) return st;
    if ((st = check_out(nullptr, topk_idx, topk_w, residual, out)) != MOE_OK) return st;
    st = enqueue_down_combine(layer, n_tokens, topk_idx, topk_w, plan, residual, out, workspace,
                              (hipStream_t)hip_stream);
    if (st != MOE_OK) return st;
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

extern "C" moe_status moe_decode_step_residual(const moe_layer_t *layer, const void *x, int32_t n_tokens,
                                               const int32_t *topk_idx, const float *topk_w,
                                               const moe_plan_t *plan, const void *residual, void *out,
                                               void *workspace, size_t workspace_bytes, void *hip_stream) {
    moe_status st = check_step(layer, n_tokens, plan, workspace, workspace_bytes);
    if (st != MOE_OK || n_tokens == 0) return st;
    if ((st = check_x(x)) != MOE_OK) return st;
    if ((st = check_out(x, topk_idx, topk_w, residual, out)) != MOE_OK) return st;
    hipStream_t stream = (hipStream_t)hip_stream;
    st = enqueue_gate_up(layer, x, n_tokens, plan, workspace, stream);
    if (st != MOE_OK) return st;
    st = enqueue_down_combine(layer, n_tokens, topk_idx, topk_w, plan, residual, out, workspace, stream);
    if (st != MOE_OK) return st;
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

extern "C" moe_status moe_decode_step(const moe_layer_t *layer, const void *x, int32_t n_tokens,
                                      const int32_t *topk_idx, const float *topk_w, const moe_plan_t *plan,
                                      void *out, void *workspace, size_t workspace_bytes, void *hip_stream) {
    return moe_decode_step_residual(layer, x, n_tokens, topk_idx, topk_w, plan, nullptr, out, workspace,
                                    workspace_bytes, hip_stream);
}

extern "C" moe_status moe_decode_layer(const moe_layer_t *layer, const float *logits, const void *x,
                                       int32_t n_tokens, int32_t *topk_idx, float *topk_w,
                                       const moe_plan_t *plan, const void *residual, void *out,
                                       void *workspace, size_t workspace_bytes, void *hip_stream) {
    moe_status st = check_step(layer, n_tokens, plan, workspace, workspace_bytes);
    if (st != MOE_OK || n_tokens == 0) return st;
    if ((st = check_x(x)) != MOE_OK) return st;
    if ((st = check_out(x, topk_idx, topk_w, residual, out)) != MOE_OK) return st;
    st = moe_route_gate_up(layer, logits, x, n_tokens, topk_idx, topk_w, plan, workspace, workspace_bytes,
                           hip_stream);
    if (st != MOE_OK) return st;
    st = enqueue_down_combine(layer, n_tokens, topk_idx, topk_w, plan, residual, out, workspace,
                              (hipStream_t)hip_stream);
    if (st != MOE_OK) return st;
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

// ------------------------------------------- the allocation-free variant

// Device memory of moe_decode_layer_static: the h and y workspace of the
// step in one array per device, reserved when the library is loaded and
// held until the process ends.  In host code `scratch` only names the
// symbol; its device address comes from hipGetSymbolAddress, once per
// device, and is what the kernels get.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_dev[kMaxDevices];  // device address of `scratch` per device, once looked up
}  // namespace

// The scratch array's address on the device of `stream`, which must be the
// current device (the lookup answers for the current device).
static moe_status scratch_of(hipStream_t stream, void **ptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur < 0 || cur >= kMaxDevices) return MOE_ERR_DEVICE;
    if (stream) {
        hipDevice_t sd = -1;
        if (hipStreamGetDevice(stream, &sd) != hipSuccess) return MOE_ERR_INVALID_ARG;
        if (sd != cur) return MOE_ERR_INVALID_ARG;
    }
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[cur]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_DEVICE;
        scratch_dev[cur] = p;
    }
    *ptr = scratch_dev[cur];
    return MOE_OK;
}

extern "C" moe_status moe_decode_layer_static(const moe_layer_t *layer, const float *logits, const void *x,
                                              int32_t n_tokens, int32_t *topk_idx, float *topk_w,
                                              const moe_plan_t *plan, const void *residual, void *out,
                                              void *hip_stream) {
    moe_status st = check_layer(layer);
    if (st != MOE_OK) return st;
    if (n_tokens < 0) return MOE_ERR_INVALID_ARG;
    if (n_tokens > MOE_MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
    if (n_tokens == 0) return MOE_OK;
    if (workspace_layout(layer, n_tokens).total > MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    void *ws = nullptr;
    if ((st = scratch_of((hipStream_t)hip_stream, &ws)) != MOE_OK) return st;
    return moe_decode_layer(layer, logits, x, n_tokens, topk_idx, topk_w, plan, residual, out, ws,
                            MOE_STATIC_SCRATCH_BYTES, hip_stream);
}
