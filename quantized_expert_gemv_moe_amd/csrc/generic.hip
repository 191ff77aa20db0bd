// Expert kernels for the weight formats other than 4-bit elements in groups
// of 64: 4-, 6- or 8-bit elements (gate/up and down each at its own width)
// in groups of 32, 64 or 128.  The pages template their fused kernel on bits
// and group size and require a 6-bit down projection (4-bit gate/up) to keep
// working (page "perf(moe): batched decode scales 1.55x against 3.25x on
// dense", Implementation Notes).
//
// Rows are little-endian bit streams: element c of a row sits in stream
// bits c*bits .. c*bits+bits-1, bit j of the stream being bit j % 32 of
// word j / 32.  A "unit" is 16 consecutive elements of a row, bits/2 whole
// words (4-bit: 2, 6-bit: 3, 8-bit: 4), and always lies inside one group.
//
// One kernel serves both GEMVs of the expert block, walking the plan's
// distinct experts like the 4-bit kernels:
//   gate+up : in = x [tokens][hidden], two matrices (gate, up), out = h
//             [slots][dff] after the sidecar, clamp and gated activation;
//   down    : in = h [slots][dff] fp32, one matrix, out = y [slots][hidden]
//             (the combine launch then applies router weights and the
//             down sidecar).
// A row is read by `lpr` lanes (a power of two), each holding UPL units,
// unit u of the row going to lane u % lpr, so a wave instruction reads
// lpr consecutive units.  All of a lane's weight words are loaded before
// any math; a unit is dequantised once (w = scale * code + bias in fp32)
// and then used for every slot of the stage (fp32 FMAs).  Segment sums by
// a butterfly of lane exchanges.
#include <hip/hip_runtime.h>

#include "device_util.h"
#include "expert_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kGenBlock = 256;  // four independent waves
constexpr int kGenStage = 8;    // slots per pass over a lane's units (half for gate+up)

struct GenericArgs {
    const uint32_t *q0, *q1;  // gate and up, or down (q1 unused)
    const uint16_t *s0, *b0, *s1, *b1;
    const float *expert_scale;
    float clamp_limit;
    int activation;
    const void *in;
    PlanView plan;
    float *out;
    int rows, K, n_experts, n_slots, top_k, lpr, group_shift;  // group = 16 << group_shift
};

// The words of one unit, nontemporal (each is read once per step).
template <int BITS>
__device__ __forceinline__ void load_unit(const uint32_t *p, uint32_t (&w)[BITS / 2]) {
    if constexpr (BITS == 8) {
        const uint4 v = load_stream((const uint4 *)p);
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
        w[3] = v.w;
    } else if constexpr (BITS == 4) {
        typedef uint32_t v2u __attribute__((ext_vector_type(2)));
        const v2u v = __builtin_nontemporal_load((const v2u *)p);
        w[0] = v.x;
        w[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < BITS / 2; ++i) w[i] = __builtin_nontemporal_load(p + i);
    }
}

// Element i (0..15) of a unit as a float (exact: codes are below 2^8).
template <int BITS>
__device__ __forceinline__ float unit_code(const uint32_t (&w)[BITS / 2], int i) {
    const int p = i * BITS, wi = p / 32, off = p % 32;
    uint32_t v = w[wi] >> off;
    if (off + BITS > 32) v |= w[wi + 1] << (32 - off);
    return (float)(v & ((1u << BITS) - 1u));
}

// 16 consecutive inputs as fp32.
template <bool BF16>
__device__ __forceinline__ void load_in16(const void *base, size_t at, float (&v)[16]) {
    if constexpr (BF16) {
        const uint4 *p = (const uint4 *)((const uint16_t *)base + at);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint4 r = p[h];
            const uint32_t d[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * h + 2 * j] = __uint_as_float(d[j] << 16);
                v[8 * h + 2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
            }
        }
    } else {
        const float4 *p = (const float4 *)((const float *)base + at);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const float4 r = p[h];
            v[4 * h] = r.x;
            v[4 * h + 1] = r.y;
            v[4 * h + 2] = r.z;
            v[4 * h + 3] = r.w;
        }
    }
}

template <int BITS, int UPL, bool GU, bool XBF16>
__global__ __launch_bounds__(kGenBlock) void generic_rows_kernel(GenericArgs a) {
    constexpr int WPU = BITS / 2;  // words per unit
    constexpr int NM = GU ? 2 : 1;
    constexpr int S = GU ? kGenStage / 2 : kGenStage;
    Work wk;
    if (!plan_expert(a.plan, blockIdx.y, a.n_experts, a.n_slots, &wk)) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int lpr = a.lpr;
    const int seg = lane & (lpr - 1);
    const int row = (blockIdx.x * (kGenBlock / kWave) + wave) * (kWave / lpr) + lane / lpr;
    const bool live = row < a.rows;
    const int r = live ? row : a.rows - 1;  // a spare lane reads a valid row and stores nothing
    const size_t row_words = (size_t)a.K * BITS / 32;
    const int groups = a.K >> (4 + a.group_shift);
    const size_t rq = ((size_t)wk.e * a.rows + r) * row_words;
    const size_t rs = ((size_t)wk.e * a.rows + r) * groups;

    uint32_t q[NM][UPL][WPU];
    float sc[NM][UPL], bi[NM][UPL];
#pragma unroll
    for (int k = 0; k < UPL; ++k) {
        const int u = seg + k * lpr;
        load_unit<BITS>(a.q0 + rq + (size_t)u * WPU, q[0][k]);
        if constexpr (GU) load_unit<BITS>(a.q1 + rq + (size_t)u * WPU, q[NM - 1][k]);
    }
#pragma unroll
    for (int k = 0; k < UPL; ++k) {
        const int g = (seg + k * lpr) >> a.group_shift;
        sc[0][k] = f16_bits_to_f32(a.s0[rs + g]);
        bi[0][k] = f16_bits_to_f32(a.b0[rs + g]);
        if constexpr (GU) {
            sc[NM - 1][k] = f16_bits_to_f32(a.s1[rs + g]);
            bi[NM - 1][k] = f16_bits_to_f32(a.b1[rs + g]);
        }
    }
    const float esc = (GU && a.expert_scale) ? a.expert_scale[wk.e] : 1.f;

    for (int s0 = 0; s0 < wk.count; s0 += S) {
        const int ns = wk.count - s0 < S ? wk.count - s0 : S;
        size_t src[S];
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const int slot = plan_slot(a.plan, wk, i < ns ? s0 + i : s0, a.n_slots);
            src[i] = (size_t)(GU ? slot / a.top_k : slot) * a.K;
        }
        float acc[NM][S];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int i = 0; i < S; ++i) acc[m][i] = 0.f;
#pragma unroll
        for (int k = 0; k < UPL; ++k) {
            float w[NM][16];
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int c = 0; c < 16; ++c) w[m][c] = fmaf(sc[m][k], unit_code<BITS>(q[m][k], c), bi[m][k]);
            const size_t at = (size_t)(seg + k * lpr) * 16;
#pragma unroll
            for (int i = 0; i < S; ++i) {
                if (i >= ns) break;  // wave-uniform
                float xv[16];
                load_in16<XBF16>(a.in, src[i] + at, xv);
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    float d0 = 0.f, d1 = 0.f;
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        d0 = fmaf(w[m][c], xv[c], d0);
                        d1 = fmaf(w[m][8 + c], xv[8 + c], d1);
                    }
                    acc[m][i] += d0 + d1;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < S; ++i) {
            if (i >= ns) break;
            float v[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                v[m] = acc[m][i];
                for (int off = lpr >> 1; off > 0; off >>= 1) v[m] += __shfl_xor(v[m], off);
            }
            if (seg == 0 && live) {
                const int slot = plan_slot(a.plan, wk, s0 + i, a.n_slots);
                a.out[(size_t)slot * a.rows + row] =
                    GU ? act_mul(v[0], v[NM - 1], esc, a.clamp_limit, a.activation) : v[0];
            }
        }
    }
}

// ------------------------------------------------------------- host side

static int group_shift_of(int group) { return group == 32 ? 1 : group == 64 ? 2 : 3; }

template <int BITS, bool GU, bool XBF16>
static moe_status launch_generic_bits(const GenericArgs &a, int upl, int groups_y, hipStream_t s) {
    const int rows_per_block = (kGenBlock / kWave) * (kWave / a.lpr);
    const dim3 grid((a.rows + rows_per_block - 1) / rows_per_block, groups_y), block(kGenBlock);
    switch (upl) {
#define MOE_GEN(U) \
    case U: hipLaunchKernelGGL((generic_rows_kernel<BITS, U, GU, XBF16>), grid, block, 0, s, a); return MOE_OK;
        MOE_GEN(1) MOE_GEN(2) MOE_GEN(3) MOE_GEN(4) MOE_GEN(6) MOE_GEN(8)
#undef MOE_GEN
        default: return MOE_ERR_UNSUPPORTED;
    }
}

template <bool GU, bool XBF16>
static moe_status launch_generic(const GenericArgs &a, int bits, int upl, int groups_y, hipStream_t s) {
    switch (bits) {
        case 4: return launch_generic_bits<4, GU, XBF16>(a, upl, groups_y, s);
        case 6: return launch_generic_bits<6, GU, XBF16>(a, upl, groups_y, s);
        case 8: return launch_generic_bits<8, GU, XBF16>(a, upl, groups_y, s);
        default: return MOE_ERR_UNSUPPORTED;
    }
}

static int generic_groups_y(const moe_layer_t *L, int n_tokens) {
    const int n_slots = n_tokens * L->top_k;
    return n_slots < L->n_experts ? n_slots : L->n_experts;
}

moe_status launch_generic_gate_up(const moe_layer_t *L, const void *x, int n_tokens, const moe_plan_t *plan,
                                  float *h, hipStream_t s) {
    int lpr = 0, upl = 0;
    if (!pick_generic(L->hidden, &lpr, &upl)) return MOE_ERR_UNSUPPORTED;
    const GenericArgs a{L->gate_q, L->up_q, L->gate_s, L->gate_b, L->up_s, L->up_b, L->expert_scale,
                        L->clamp_limit, L->activation, x, PlanView{(const int4 *)plan->work, plan->sorted_slots},
                        h, L->dff, L->hidden, L->n_experts, n_tokens * L->top_k, L->top_k, lpr,
                        group_shift_of(L->group_size)};
    const int gy = generic_groups_y(L, n_tokens);
    if (L->act_dtype == MOE_DTYPE_BF16) return launch_generic<true, true>(a, L->bits, upl, gy, s);
    return launch_generic<true, false>(a, L->bits, upl, gy, s);
}

moe_status launch_generic_down(const moe_layer_t *L, int n_tokens, const moe_plan_t *plan, const float *h,
                               float *y, hipStream_t s) {
    int lpr = 0, upl = 0;
    if (!pick_generic(L->dff, &lpr, &upl)) return MOE_ERR_UNSUPPORTED;
    const GenericArgs a{L->down_q, nullptr, L->down_s, L->down_b, nullptr, nullptr, nullptr,
                        0.f, MOE_ACT_SWIGLU, h, PlanView{(const int4 *)plan->work, plan->sorted_slots},
                        y, L->hidden, L->dff, L->n_experts, n_tokens * L->top_k, L->top_k, lpr,
                        group_shift_of(L->group_size)};
    return launch_generic<false, false>(a, down_bits_of(L), upl, generic_groups_y(L, n_tokens), s);
}

}  // namespace moe
