// Device code of the dot2 gate+up kernels shared by the batched kernels and
// the few-token kernel that routes for itself: argument records, the
// nibble dot products, activation loads, cross-lane sums and the per-row
// gate/up evaluation.  Both families evaluate a row the same way, so h is
// bitwise the same whichever kernel computes it.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_util.h"
#include "expert_device.h"

namespace moe {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

struct GateUpArgs {
    const uint4 *gate_q, *up_q;
    const uint16_t *gate_s, *gate_b, *up_s, *up_b;
    const float *expert_scale;
    float clamp_limit;
    const void *x;
    PlanView plan;
    float *h;
    int hidden, dff, n_experts, top_k, n_slots;
    int max_count;  // the VALU kernel leaves experts with more slots to the MFMA kernel
    int activation;  // moe_activation
};

struct DownArgs {
    const uint4 *down_q;
    const uint16_t *down_s, *down_b;
    const float *h;
    PlanView plan;
    float *y;
    int hidden, dff, n_experts, n_slots, slots_per_stage;
};

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Eight nibbles of `w` against eight bf16 activations given as the pairs
// xp[p] = (x[p], x[p + 4]).  Each nibble pair becomes a bf16 pair of value
// (128 + q[p], 128 + q[p + 4]) by masking into the mantissa of 128.0; the
// products are exact in fp32.
__device__ __forceinline__ float dot8_q4_bf16(uint32_t w, const uint32_t *xp, float acc) {
    // The mask in an SGPR and the 128.0 pair in a VGPR, opaque to constant
    // folding: then (w & M) | B is one v_and_or_b32 (gfx9's three-operand
    // encoding takes no literal, so with both as literals the compiler
    // emits a separate and + or per nibble pair).
    uint32_t M, B;
    asm("s_mov_b32 %0, 0xf000f" : "=s"(M));
    asm("v_mov_b32 %0, 0x43004300" : "=v"(B));
    acc = dot2_bf16((w & M) | B, xp[0], acc);
    acc = dot2_bf16(((w >> 4) & M) | B, xp[1], acc);
    acc = dot2_bf16(((w >> 8) & M) | B, xp[2], acc);
    acc = dot2_bf16(((w >> 12) & M) | B, xp[3], acc);
    return acc;
}

// sum_i (128 + q_i) x_i over the 32 weights of one 16-byte chunk.
__device__ __forceinline__ float dot32_q4_bf16(uint4 q, const uint32_t *xp) {
    const float a0 = dot8_q4_bf16(q.x, xp + 0, 0.f);
    const float a1 = dot8_q4_bf16(q.y, xp + 4, 0.f);
    const float a2 = dot8_q4_bf16(q.z, xp + 8, 0.f);
    const float a3 = dot8_q4_bf16(q.w, xp + 12, 0.f);
    return (a0 + a1) + (a2 + a3);
}

// 32 bf16 activations starting at element c0 of row xr, as loaded 16-byte
// words.
// The loads go through a global-address-space pointer: the activations
// reach the kernels inside argument structs, where the compiler cannot
// prove the address space, and a generic (flat) load makes every later
// wait for memory also wait for all loads in flight.
typedef uint32_t gv4u __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) gv4u *gv4u_gptr;
__device__ __forceinline__ void load_x32_bf16(const uint16_t *x, size_t xr, int c0, uint4 *raw) {
    const gv4u_gptr p = (gv4u_gptr)(x + xr + c0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const gv4u v = p[i];
        raw[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
}

// The 16 pairs used by dot8_q4_bf16 from the loaded words, and the sum of
// the 32 activations (dot2 against the pair (1, 1): exact products, fp32
// accumulation).
__device__ __forceinline__ float x32_pairs(const uint4 *raw, uint32_t *xp) {
    const uint32_t ones = 0x3F803F80u;  // bf16 (1.0, 1.0)
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 w = raw[i];  // elements 8i .. 8i+7 as (x0,x1),(x2,x3),(x4,x5),(x6,x7)
        xp[4 * i + 0] = (w.x & 0xFFFFu) | (w.z << 16);
        xp[4 * i + 1] = (w.x >> 16) | (w.z & 0xFFFF0000u);
        xp[4 * i + 2] = (w.y & 0xFFFFu) | (w.w << 16);
        xp[4 * i + 3] = (w.y >> 16) | (w.w & 0xFFFF0000u);
        s0 = dot2_bf16(w.x, ones, dot2_bf16(w.y, ones, s0));
        s1 = dot2_bf16(w.z, ones, dot2_bf16(w.w, ones, s1));
    }
    return s0 + s1;
}

// 32 fp32 activations starting at element c0 of row xr and their sum.
__device__ __forceinline__ float load_x32_f32(const float *x, size_t xr, int c0, float *dst) {
    const float4 *p = (const float4 *)(x + xr + c0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 w = p[i];
        dst[4 * i + 0] = w.x;
        dst[4 * i + 1] = w.y;
        dst[4 * i + 2] = w.z;
        dst[4 * i + 3] = w.w;
    }
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        s0 += dst[4 * i + 0];
        s1 += dst[4 * i + 1];
        s2 += dst[4 * i + 2];
        s3 += dst[4 * i + 3];
    }
    return (s0 + s1) + (s2 + s3);
}

// ------------------------------------------------------- cross-lane sums

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuad1032 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuad2301 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// Sum over aligned segments of LPR lanes; every lane of a segment gets the
// same value (each step adds the same two numbers on both partner lanes).
template <int LPR>
__device__ __forceinline__ float seg_sum(float v) {
    if constexpr (LPR >= 2) v += dpp<kDppQuad1032>(v);
    if constexpr (LPR >= 4) v += dpp<kDppQuad2301>(v);
    if constexpr (LPR >= 8) v += dpp<kDppHalfMirror>(v);
    if constexpr (LPR >= 16) v += dpp<kDppMirror>(v);
    if constexpr (LPR >= 32) v += __shfl_xor(v, 16, kWave);
    if constexpr (LPR >= 64) v += __shfl_xor(v, 32, kWave);
    return v;
}

// Sum of lo and hi 32-lane halves of a and b at once: lanes 0..31 return
// a[l] + a[l+32], lanes 32..63 return b[l-32] + b[l] (v_permlane32_swap).
__device__ __forceinline__ float swap32_sum(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Same on 16-lane rows: rows (0,1) of a go to row 0, of b to row 1, rows
// (2,3) of a to row 2, of b to row 3 (v_permlane16_swap).
__device__ __forceinline__ float swap16_sum(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave-wide sums of eight per-lane values at once.  Lane l returns the total
// of v[2 * (l >> 4) + ((l >> 3) & 1)]: lanes 16r..16r+7 hold v[2r] and lanes
// 16r+8..16r+15 hold v[2r+1].  ~23 VALU ops instead of 8 separate trees.
__device__ __forceinline__ float wave_sum8(const float *v) {
    const int lane = threadIdx.x & (kWave - 1);
    float w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = swap32_sum(v[i], v[i + 4]);
    // w[i]: lanes 0..31 partial of v[i], lanes 32..63 partial of v[i+4]
    const float z0 = swap16_sum(w[0], w[2]);  // rows: v0 v2 v4 v6
    const float z1 = swap16_sum(w[1], w[3]);  // rows: v1 v3 v5 v7
    const bool upper = lane & 8;
    const float t = upper ? z1 : z0;
    const float s = upper ? z0 : z1;
    float m = t + dpp<kDppMirror>(s);
    m += dpp<kDppHalfMirror>(m);
    m += dpp<kDppQuad2301>(m);
    m += dpp<kDppQuad1032>(m);
    return m;
}

// Wave-wide sum; every lane gets the same total.
__device__ __forceinline__ float wave_sum_all(float v) {
    v += dpp<kDppQuad1032>(v);
    v += dpp<kDppQuad2301>(v);
    v += dpp<kDppHalfMirror>(v);
    v += dpp<kDppMirror>(v);  // every lane: its 16-lane row total
    v = swap16_sum(v, v);     // rows (0,1) and (2,3)
    v = swap32_sum(v, v);     // halves
    return v;
}

// ---------------------------------------------------------------- gate+up

// A lane's share of RI rows of one expert: its NV 16-byte chunks of each
// gate and up row with their scales and biases (as fp32; with bf16
// activations the bias also carries the -128 * scale of the nibble trick).
template <int RI, int NV>
struct GateUpRows {
    uint4 wg[RI][NV], wu[RI][NV];
    // fp16 bits as loaded: converted (and, with bf16 activations, the bias
    // folded) where the rows are evaluated, so nothing issued right after
    // the loads has to wait for them
    uint16_t sg[RI][NV], bg[RI][NV], su[RI][NV], bu[RI][NV];
};

// Makes the compiler treat the weights as redefined here, so work derived
// from them (unpacked nibbles) is not hoisted out of a token loop.
template <int RI, int NV>
__device__ __forceinline__ void opaque_rows(GateUpRows<RI, NV> &w) {
#pragma unroll
    for (int r = 0; r < RI; ++r)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            asm volatile("" : "+v"(w.wg[r][v].x), "+v"(w.wg[r][v].y), "+v"(w.wg[r][v].z), "+v"(w.wg[r][v].w));
            asm volatile("" : "+v"(w.wu[r][v].x), "+v"(w.wu[r][v].y), "+v"(w.wu[r][v].z), "+v"(w.wu[r][v].w));
        }
}

template <int LPR, int NV, int RI, bool XBF16>
__device__ __forceinline__ void load_gate_up_rows(const GateUpArgs &a, int e, int row0, int sl,
                                                  GateUpRows<RI, NV> &w) {
    constexpr int RPI = kWave / LPR;
    const int H = a.hidden, F = a.dff;
    const int qrow = H / 32, grow = H / kGroup;
    // scales and biases first: converting them then waits for them alone,
    // while the weights (issued after) are still in flight
#pragma unroll
    for (int r = 0; r < RI; ++r) {
        const int row = row0 + r * RPI;
        const size_t rs = ((size_t)e * F + (row < F ? row : F - 1)) * grow;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int ch = v * LPR + sl;
            w.sg[r][v] = a.gate_s[rs + ch / 2];
            w.bg[r][v] = a.gate_b[rs + ch / 2];
            w.su[r][v] = a.up_s[rs + ch / 2];
            w.bu[r][v] = a.up_b[rs + ch / 2];
        }
    }
#pragma unroll
    for (int r = 0; r < RI; ++r) {
        const int row = row0 + r * RPI;
        const size_t rq = ((size_t)e * F + (row < F ? row : F - 1)) * qrow;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int ch = v * LPR + sl;
            w.wg[r][v] = load_stream(a.gate_q + rq + ch);
            w.wu[r][v] = load_stream(a.up_q + rq + ch);
        }
    }
}

// One token's activations for this lane's chunks: bf16 pairs (or fp32
// values) and the sum of each chunk's 32 activations.
template <int LPR, int NV, bool XBF16>
struct GateUpX {
    uint32_t xp[XBF16 ? NV : 1][XBF16 ? 16 : 1];
    float xf[XBF16 ? 1 : NV][XBF16 ? 1 : 32];
    float xs[NV];
};

template <int LPR, int NV, bool XBF16>
__device__ __forceinline__ void load_gate_up_x(const GateUpArgs &a, int token, int sl, GateUpX<LPR, NV, XBF16> &x,
                                               const uint4 (*pre)[4] = nullptr) {
    const size_t xr = (size_t)token * a.hidden;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int c0 = (v * LPR + sl) * 32;
        if constexpr (XBF16) {
            uint4 raw[4];
            if (pre) {
#pragma unroll
                for (int q = 0; q < 4; ++q) raw[q] = pre[v][q];
            } else {
                load_x32_bf16((const uint16_t *)a.x, xr, c0, raw);
            }
            x.xs[v] = x32_pairs(raw, x.xp[v]);
        } else {
            x.xs[v] = load_x32_f32((const float *)a.x, xr, c0, x.xf[v]);
        }
    }
}

// h = silu(g) * u of one token for the segment's RI rows, into slot `slot`.
template <int LPR, int NV, int RI, bool XBF16>
__device__ __forceinline__ void gate_up_token_rows(const GateUpArgs &a, const GateUpRows<RI, NV> &w,
                                                   const GateUpX<LPR, NV, XBF16> &x, int slot, int row0,
                                                   float sc, float lim) {
    constexpr int RPI = kWave / LPR;
    constexpr bool WAVE8 = (LPR == kWave && RI == 4);
    const int lane = threadIdx.x & (kWave - 1);
    const int sl = lane % LPR;
    const int F = a.dff;
    float part[2 * RI];
#pragma unroll
    for (int r = 0; r < RI; ++r) {
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float dg, du;
            if constexpr (XBF16) {
                dg = dot32_q4_bf16(w.wg[r][v], x.xp[v]);
                du = dot32_q4_bf16(w.wu[r][v], x.xp[v]);
            } else {
                dg = dot32_q4(w.wg[r][v], x.xf[v]);
                du = dot32_q4(w.wu[r][v], x.xf[v]);
            }
            const float sg = f16_bits_to_f32(w.sg[r][v]), su = f16_bits_to_f32(w.su[r][v]);
            float bg = f16_bits_to_f32(w.bg[r][v]), bu = f16_bits_to_f32(w.bu[r][v]);
            if constexpr (XBF16) {  // fold the +128 of the bf16 nibble trick into the bias
                bg = fmaf(-128.f, sg, bg);
                bu = fmaf(-128.f, su, bu);
            }
            g += fmaf(sg, dg, bg * x.xs[v]);
            u += fmaf(su, du, bu * x.xs[v]);
        }
        part[2 * r] = g;
        part[2 * r + 1] = u;
    }
    if constexpr (WAVE8) {
        const float tot = wave_sum8(part);
        const float other = dpp<kDppMirror>(tot);  // lane 16r reads lane 16r+15 (the u)
        const int r = lane >> 4;
        const int row = row0 + r * RPI;
        if ((lane & 15) == 0 && row < F) a.h[(size_t)slot * F + row] = act_mul(tot, other, sc, lim, a.activation);
    } else {
#pragma unroll
        for (int r = 0; r < RI; ++r) {
            const float g = seg_sum<LPR>(part[2 * r]);
            const float u = seg_sum<LPR>(part[2 * r + 1]);
            const int row = row0 + r * RPI;
            if (sl == 0 && row < F) a.h[(size_t)slot * F + row] = act_mul(g, u, sc, lim, a.activation);
        }
    }
}

// One wave: row block rb of distinct expert u.  LPR lanes per row, NV
// chunks per lane, RI rows per segment; TCH tokens' activations in
// registers at a time.
template <int LPR, int NV, int RI, bool XBF16>
__device__ __forceinline__ void gate_up_valu_block(const GateUpArgs &a, int rb, int u) {
    constexpr int RPI = kWave / LPR;  // rows per wave-wide pass
    constexpr int ROWS_WG = RPI * RI;
    constexpr int TCH = (XBF16 && NV == 1) ? 2 : 1;
    const int lane = threadIdx.x & (kWave - 1);
    const int sl = lane % LPR;
    Work wk;
    if (!plan_expert(a.plan, u, a.n_experts, a.n_slots, &wk)) return;
    if (wk.count > a.max_count) return;  // the MFMA kernel's expert
    const int e = wk.e, count = wk.count;
    const int row0 = rb * ROWS_WG + lane / LPR;

    // The first TCH tokens' activations go out ahead of the weights, and
    // each pass fetches the next TCH tokens' before it computes, so no
    // activation load waits behind the weights.  Loads are unconditional
    // (past the last token they repeat it, unused): a load under a branch
    // would make the compiler wait for every load in flight where it joins.
    int slot_n[TCH];
    uint4 raw_n[TCH][XBF16 ? NV : 1][4];
#pragma unroll
    for (int i = 0; i < TCH; ++i) {
        slot_n[i] = plan_slot(a.plan, wk, i < count ? i : count - 1, a.n_slots);
        if constexpr (XBF16) {
#pragma unroll
            for (int v = 0; v < NV; ++v)
                load_x32_bf16((const uint16_t *)a.x, (size_t)(slot_n[i] / a.top_k) * a.hidden,
                              (v * LPR + sl) * 32, raw_n[i][v]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    GateUpRows<RI, NV> w;
    load_gate_up_rows<LPR, NV, RI, XBF16>(a, e, row0, sl, w);
    const float sc = a.expert_scale ? a.expert_scale[e] : 1.f;
    const float lim = a.clamp_limit;
    __builtin_amdgcn_sched_barrier(0);

    for (int t0 = 0; t0 < count; t0 += TCH) {
        int slot[TCH];
        uint4 raw[TCH][XBF16 ? NV : 1][4];
#pragma unroll
        for (int i = 0; i < TCH; ++i) {
            slot[i] = slot_n[i];
#pragma unroll
            for (int v = 0; v < (XBF16 ? NV : 1); ++v)
#pragma unroll
                for (int q = 0; q < 4; ++q) raw[i][v][q] = raw_n[i][v][q];
        }
        if constexpr (XBF16) {
#pragma unroll
            for (int i = 0; i < TCH; ++i) {
                const int tn = t0 + TCH + i;
                slot_n[i] = plan_slot(a.plan, wk, tn < count ? tn : count - 1, a.n_slots);
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    load_x32_bf16((const uint16_t *)a.x, (size_t)(slot_n[i] / a.top_k) * a.hidden,
                                  (v * LPR + sl) * 32, raw_n[i][v]);
            }
        } else {
            slot_n[0] = plan_slot(a.plan, wk, t0 + 1 < count ? t0 + 1 : count - 1, a.n_slots);
        }
#pragma unroll
        for (int i = 0; i < TCH; ++i) {
            if (i > 0 && t0 + i >= count) break;  // uniform: the chunk's tail is empty
            GateUpX<LPR, NV, XBF16> x;
            load_gate_up_x<LPR, NV, XBF16>(a, slot[i] / a.top_k, sl, x, XBF16 ? raw[i] : nullptr);
            gate_up_token_rows<LPR, NV, RI, XBF16>(a, w, x, slot[i], row0, sc, lim);
        }
    }
}

// At least four waves per SIMD for the one-chunk bf16 rows (they fit in 128
// registers without spilling): left to itself the compiler sizes this
// one-wave kernel's registers for two, and a CU then holds too few waves to
// keep enough loads in flight.
template <int LPR, int NV, bool XBF16>
constexpr int gate_up_waves_per_simd() { return (NV == 1 && XBF16) ? 4 : 1; }

// Rows per lane segment of the gate+up kernels: four for the whole-wave rows
// (the 8-value transposed reduction), fewer when a lane holds many chunks.
// Both gate+up kernels take the same value, so they reduce in the same order.
template <int LPR, int NV>
constexpr int gate_up_ri() {
    return (LPR == kWave) ? (NV <= 2 ? 4 : 2) : (NV <= 2 ? 2 : 1);
}

}  // namespace moe
