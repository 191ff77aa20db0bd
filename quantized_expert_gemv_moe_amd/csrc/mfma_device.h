// Operand helpers of the MFMA expert kernels (gfx950,
// v_mfma_f32_16x16x32_bf16).
//
// The 4-bit weights enter an MFMA as bf16 values 1 + q / 16, which bf16
// holds exactly, and the activations as bf16, so every product is exact in
// fp32; the affine format w = s * q + b of the layer (page "perf(moe):
// batched decode scales 1.55x against 3.25x on dense", Current Behavior:
// 4-bit group 64) is restored per 64-group after the MFMA as
//   16 s * D + (b - 16 s) * sum(x over the group).
// Within one 32-bit weight word (8 nibbles) the inputs are paired as
// (p, p + 4), p = 0..3, on both operands, so one word and one 16-byte
// activation word give the eight bf16 K-values of one lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gate_up_device.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint32_t *a, const uint32_t *b, f32x4_t c) {
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
    const u32x4_t av = {a[0], a[1], a[2], a[3]};
    const u32x4_t bv = {b[0], b[1], b[2], b[3]};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                   __builtin_bit_cast(bf16x8_t, bv), c, 0, 0, 0);
}

// The nibble pairs of one word as bf16 values 1 + q / 16 (q in mantissa bits
// 3..6 of 1.0).  Against an offset of 128 + q, the term the group bias has
// to take back out is 16 times the nibble unit instead of 128 times, so the
// cancellation in the epilogue loses about eight times fewer bits of the
// fp32 accumulation.
__device__ __forceinline__ void q4_pairs16(uint32_t w, uint32_t *o) {
    uint32_t M, B;  // opaque, for v_and_or_b32 (it takes no literal on gfx9)
    asm("s_mov_b32 %0, 0x780078" : "=s"(M));
    asm("v_mov_b32 %0, 0x3f803f80" : "=v"(B));
    o[0] = ((w << 3) & M) | B;
    o[1] = ((w >> 1) & M) | B;
    o[2] = ((w >> 5) & M) | B;
    o[3] = ((w >> 9) & M) | B;
}

// Eight bf16 activations (one 16-byte word) as the pairs (x_p, x_{p+4}),
// and their sum added into *acc.
__device__ __forceinline__ void x8_pairs(uint4 w, uint32_t *o, float *acc) {
    const uint32_t ones = 0x3F803F80u;
    o[0] = (w.x & 0xFFFFu) | (w.z << 16);
    o[1] = (w.x >> 16) | (w.z & 0xFFFF0000u);
    o[2] = (w.y & 0xFFFFu) | (w.w << 16);
    o[3] = (w.y >> 16) | (w.w & 0xFFFF0000u);
    *acc = dot2_bf16(w.x, ones, dot2_bf16(w.y, ones, dot2_bf16(w.z, ones, dot2_bf16(w.w, ones, *acc))));
}

// Eight fp32 values as three bf16 parts each, paired as (v_p, v_{p+4}):
// o[part][p].  The parts are cut by truncation, v = hi + mid + lo, every bit
// of v in exactly one of them (the low 16 bits of each remainder go on to
// the next), so three MFMAs with the same weights sum (1 + q / 16) * v with
// every product exact in fp32.
__device__ __forceinline__ void split3_pairs(const float *v, uint32_t (*o)[4]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float a = v[p], b = v[p + 4];
        const uint32_t a1 = __float_as_uint(a) & 0xFFFF0000u, b1 = __float_as_uint(b) & 0xFFFF0000u;
        const float ar = a - __uint_as_float(a1), br = b - __uint_as_float(b1);
        const uint32_t a2 = __float_as_uint(ar) & 0xFFFF0000u, b2 = __float_as_uint(br) & 0xFFFF0000u;
        const float ar2 = ar - __uint_as_float(a2), br2 = br - __uint_as_float(b2);
        const uint32_t a3 = __float_as_uint(ar2) & 0xFFFF0000u, b3 = __float_as_uint(br2) & 0xFFFF0000u;
        o[0][p] = (a1 >> 16) | b1;
        o[1][p] = (a2 >> 16) | b2;
        o[2][p] = (a3 >> 16) | b3;
    }
}

}  // namespace moe
