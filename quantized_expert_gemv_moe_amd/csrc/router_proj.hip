// Router projection (gfx950) and moe_router_logits: logits = x . Wr^T, the
// step in front of the router (page "perf(moe): attribute the MoE decode
// gap at the M = 1 expert gather", Proposed Solution step 2 names the
// router as one of the per-token costs).  Wr is a dense bf16 matrix
// [n_experts][hidden].
//
// One wave per RPI = 64 / LPR expert rows and tile of tokens: LPR lanes read
// a row as 16-byte chunks (8 bf16), NV chunks per lane, and apply them to
// the tile's tokens from registers.  With bf16 activations the products go
// through v_dot2_f32_bf16 (exact products, fp32 accumulation); with fp32
// activations the weights are widened and multiplied with exact fp32 FMAs.
// The lanes of a row are summed by a fixed tree of cross-lane VALU moves, so
// the sum order is fixed.
#include <hip/hip_runtime.h>

#include "device_util.h"
#include "gate_up_device.h"
#include "moe_internal.h"

namespace moe {

typedef __attribute__((ext_vector_type(2))) __bf16 rp_bf16x2_t;

__device__ __forceinline__ float rp_dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(rp_bf16x2_t, a), __builtin_bit_cast(rp_bf16x2_t, b),
                                           c, false);
}

// 8 bf16 weights (one chunk) times 8 fp32 activations, exact fp32 FMAs.
__device__ __forceinline__ float rp_dot8_f32(uint4 w, const float4 &x0, const float4 &x1, float acc) {
    acc = fmaf(__uint_as_float(w.x << 16), x0.x, acc);
    acc = fmaf(__uint_as_float(w.x & 0xFFFF0000u), x0.y, acc);
    acc = fmaf(__uint_as_float(w.y << 16), x0.z, acc);
    acc = fmaf(__uint_as_float(w.y & 0xFFFF0000u), x0.w, acc);
    acc = fmaf(__uint_as_float(w.z << 16), x1.x, acc);
    acc = fmaf(__uint_as_float(w.z & 0xFFFF0000u), x1.y, acc);
    acc = fmaf(__uint_as_float(w.w << 16), x1.z, acc);
    acc = fmaf(__uint_as_float(w.w & 0xFFFF0000u), x1.w, acc);
    return acc;
}

// Sum over aligned segments of LPR lanes, every lane of a segment with the
// same total: DPP quad swaps and mirrors inside 16-lane rows, then
// v_permlane16_swap and v_permlane32_swap across rows, all VALU (a shuffle
// through the LDS crossbar per step had made the sums the longest chain of
// a wave).
template <int LPR>
__device__ __forceinline__ float rp_seg_sum(float v) {
    if constexpr (LPR >= 2) v += dpp<kDppQuad1032>(v);
    if constexpr (LPR >= 4) v += dpp<kDppQuad2301>(v);
    if constexpr (LPR >= 8) v += dpp<kDppHalfMirror>(v);
    if constexpr (LPR >= 16) v += dpp<kDppMirror>(v);
    if constexpr (LPR >= 32) v = swap16_sum(v, v);
    if constexpr (LPR >= 64) v = swap32_sum(v, v);
    return v;
}

// Tokens per wave: a wave computes its rows for a tile of TT tokens, with
// every activation load of the tile issued together; tiles go to separate
// waves (grid y), so a batch spreads over many waves instead of one wave
// walking every token.  A token's sum is formed the same way in any tile.
// Up to 4 tokens per tile (2 for rows of more than 4 chunks per lane), never
// more than the batch.
template <int NV>
constexpr int router_tile_max() { return NV <= 4 ? 4 : 2; }

template <int LPR, int NV, bool XBF16, int TT>
__global__ __launch_bounds__(kWave) void router_logits_kernel(const void *__restrict__ x,
                                                              const uint4 *__restrict__ wr,
                                                              float *__restrict__ logits, int n_tokens,
                                                              int hidden, int n_experts) {
    constexpr int RPI = kWave / LPR;
    const int lane = threadIdx.x;
    const int sl = lane % LPR;
    const int row = blockIdx.x * RPI + lane / LPR;
    const int rr = row < n_experts ? row : n_experts - 1;
    const int K = hidden / 8;  // 16-byte chunks per row
    const int t0 = blockIdx.y * TT;
    uint4 w[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) w[v] = wr[(size_t)rr * K + v * LPR + sl];
    float acc[TT];
    if constexpr (XBF16) {
        uint4 xv[TT][NV];  // tokens past the batch repeat its last one (not stored)
#pragma unroll
        for (int i = 0; i < TT; ++i) {
            const int t = t0 + i < n_tokens ? t0 + i : n_tokens - 1;
#pragma unroll
            for (int v = 0; v < NV; ++v) xv[i][v] = ((const uint4 *)x)[(size_t)t * K + v * LPR + sl];
        }
#pragma unroll
        for (int i = 0; i < TT; ++i) {
            float a = 0.f;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                a = rp_dot2(w[v].x, xv[i][v].x, a);
                a = rp_dot2(w[v].y, xv[i][v].y, a);
                a = rp_dot2(w[v].z, xv[i][v].z, a);
                a = rp_dot2(w[v].w, xv[i][v].w, a);
            }
            acc[i] = a;
        }
    } else {
#pragma unroll
        for (int i = 0; i < TT; ++i) {
            const int t = t0 + i < n_tokens ? t0 + i : n_tokens - 1;
            float a = 0.f;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const float4 *xp = (const float4 *)x + ((size_t)t * K + v * LPR + sl) * 2;
                a = rp_dot8_f32(w[v], xp[0], xp[1], a);
            }
            acc[i] = a;
        }
    }
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        const float a = rp_seg_sum<LPR>(acc[i]);
        if (sl == 0 && row < n_experts && t0 + i < n_tokens) logits[(size_t)(t0 + i) * n_experts + row] = a;
    }
}

// Lanes per row (a power of two up to 64) and chunks per lane (1..8) for a
// row of `chunks` 16-byte chunks: the fewest chunks per lane that fit.
static bool pick_router_geometry(int chunks, int *lpr, int *nv) {
    for (int n = 1; n <= 8; ++n) {
        if (chunks % n) continue;
        const int l = chunks / n;
        if (l <= 64 && (l & (l - 1)) == 0) {
            *lpr = l;
            *nv = n;
            return true;
        }
    }
    return false;
}

template <int LPR, int NV>
static void launch_router(const void *x, const uint16_t *wr, float *logits, int n_tokens, int hidden,
                          int n_experts, bool bf16, hipStream_t s) {
    constexpr int RPI = kWave / LPR;
    const int tt = n_tokens >= router_tile_max<NV>() ? router_tile_max<NV>() : n_tokens >= 2 ? 2 : 1;
    const dim3 grid((n_experts + RPI - 1) / RPI, (n_tokens + tt - 1) / tt);
#define MOE_RPT(TT)                                                                                         \
    if (bf16)                                                                                               \
        hipLaunchKernelGGL((router_logits_kernel<LPR, NV, true, TT>), grid, dim3(kWave), 0, s, x,           \
                           (const uint4 *)wr, logits, n_tokens, hidden, n_experts);                         \
    else                                                                                                    \
        hipLaunchKernelGGL((router_logits_kernel<LPR, NV, false, TT>), grid, dim3(kWave), 0, s, x,          \
                           (const uint4 *)wr, logits, n_tokens, hidden, n_experts);
    if (tt == 1) {
        MOE_RPT(1)
    } else if (tt == 2 || router_tile_max<NV>() == 2) {
        MOE_RPT(2)
    } else {
        MOE_RPT(router_tile_max<NV>())
    }
#undef MOE_RPT
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_router_logits(const void *x, int32_t n_tokens, int32_t hidden, moe_dtype act_dtype,
                                        const uint16_t *w_router, int32_t n_experts, float *logits,
                                        void *hip_stream) {
    if (n_tokens < 0 || hidden <= 0 || n_experts <= 0) return MOE_ERR_INVALID_ARG;
    if (act_dtype != MOE_DTYPE_BF16 && act_dtype != MOE_DTYPE_F32) return MOE_ERR_INVALID_ARG;
    if (n_experts > MOE_MAX_EXPERTS || n_tokens > MOE_MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
    int lpr = 0, nv = 0;
    if (hidden % 8 || !pick_router_geometry(hidden / 8, &lpr, &nv)) return MOE_ERR_UNSUPPORTED;
    if (n_tokens == 0) return MOE_OK;
    if (!x || !w_router || !logits) return MOE_ERR_INVALID_ARG;
    if ((uintptr_t)x % 16 || (uintptr_t)w_router % 16 || (uintptr_t)logits % 4) return MOE_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)hip_stream;
    const bool bf16 = act_dtype == MOE_DTYPE_BF16;
    switch (lpr * 16 + nv) {
#define MOE_RP(L, N) \
    case L * 16 + N: launch_router<L, N>(x, w_router, logits, n_tokens, hidden, n_experts, bf16, s); break;
        MOE_RP(64, 1) MOE_RP(64, 2) MOE_RP(64, 3) MOE_RP(64, 4) MOE_RP(64, 5) MOE_RP(64, 6) MOE_RP(64, 7)
        MOE_RP(64, 8)
        MOE_RP(32, 1) MOE_RP(32, 3) MOE_RP(32, 5) MOE_RP(32, 7)
        MOE_RP(16, 1) MOE_RP(16, 3) MOE_RP(16, 5) MOE_RP(16, 7)
        MOE_RP(8, 1) MOE_RP(8, 3) MOE_RP(8, 5) MOE_RP(8, 7)
        MOE_RP(4, 1) MOE_RP(4, 3) MOE_RP(4, 5) MOE_RP(4, 7)
        MOE_RP(2, 1) MOE_RP(2, 3) MOE_RP(2, 5) MOE_RP(2, 7)
        MOE_RP(1, 1) MOE_RP(1, 3) MOE_RP(1, 5) MOE_RP(1, 7)
#undef MOE_RP
        default: return MOE_ERR_UNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}
