// Device helpers shared by the gfx950 kernels of the MoE decode library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;      // CDNA wavefront width
constexpr int kBlock = 256;    // four waves per workgroup
constexpr int kGroup = 64;     // quantisation group along the input dimension
// batches routed and planned by one workgroup in moe_route_plan: one wave
// per token (at 32 tokens the router kernel on many workgroups plus the
// planner measured faster than one workgroup routing two tokens per wave)
constexpr int kRoutePlanMaxTokens = 16;
constexpr int kRoutePlanMaxSlots = kRoutePlanMaxTokens * 16;  // top_k <= 16

// fp16 bit pattern -> fp32 (exact; v_cvt_f32_f16).
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// bf16 bit pattern (low 16 bits of `b`) -> fp32 (exact).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Sum over aligned segments of LPR lanes (LPR a power of two <= 64).  Every
// lane of a segment ends with the same value: each butterfly step adds the
// same two operands on both partner lanes, and fp32 addition commutes.
template <int LPR>
__device__ __forceinline__ float segment_sum(float v) {
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Eight 4-bit weights of one word times eight fp32 activations, accumulated
// in element order into `acc`.  Element i of the word is nibble i, lowest
// first: bytes of (w & 0x0F0F0F0F) hold elements 0, 2, 4, 6 and bytes of
// ((w >> 4) & 0x0F0F0F0F) hold elements 1, 3, 5, 7.
__device__ __forceinline__ float dot8_q4(uint32_t w, const float *x, float acc) {
    const uint32_t lo = w & 0x0F0F0F0Fu;
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
    acc = fmaf((float)(lo & 0xFFu), x[0], acc);
    acc = fmaf((float)(hi & 0xFFu), x[1], acc);
    acc = fmaf((float)((lo >> 8) & 0xFFu), x[2], acc);
    acc = fmaf((float)((hi >> 8) & 0xFFu), x[3], acc);
    acc = fmaf((float)((lo >> 16) & 0xFFu), x[4], acc);
    acc = fmaf((float)((hi >> 16) & 0xFFu), x[5], acc);
    acc = fmaf((float)(lo >> 24), x[6], acc);
    acc = fmaf((float)(hi >> 24), x[7], acc);
    return acc;
}

// Nibble dot over one 16-byte chunk (32 weights) against 32 activations:
// four independent word accumulators, summed in a fixed order.
__device__ __forceinline__ float dot32_q4(uint4 q, const float *x) {
    float a0 = dot8_q4(q.x, x + 0, 0.f);
    float a1 = dot8_q4(q.y, x + 8, 0.f);
    float a2 = dot8_q4(q.z, x + 16, 0.f);
    float a3 = dot8_q4(q.w, x + 24, 0.f);
    return (a0 + a1) + (a2 + a3);
}

}  // namespace moe
