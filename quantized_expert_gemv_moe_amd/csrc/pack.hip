// moe_pack_down: regroup a down projection from rows ([E][hidden][dff/8]
// words, the layout of the pages' 4-bit checkpoints) to columns of 16-byte
// chunks ([E][dff/32][hidden] chunks), and its fp16 scales and biases from
// [E][hidden][dff/64] to [E][dff/64][hidden].  Pure byte movement.
#include <hip/hip_runtime.h>

#include "device_util.h"
#include "moe_internal.h"

namespace moe {

// One destination element per thread, hidden row fastest (coalesced writes).
__global__ __launch_bounds__(kBlock) void pack_down_q_kernel(const uint4 *__restrict__ src,
                                                             uint4 *__restrict__ dst, int E, int H,
                                                             int C) {
    const size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
    const size_t total = (size_t)E * C * H;
    if (i >= total) return;
    const size_t m = i % H, c = (i / H) % C, e = i / ((size_t)H * C);
    dst[i] = src[(e * H + m) * C + c];
}

__global__ __launch_bounds__(kBlock) void pack_down_sb_kernel(const uint16_t *__restrict__ src_s,
                                                              const uint16_t *__restrict__ src_b,
                                                              uint16_t *__restrict__ dst_s,
                                                              uint16_t *__restrict__ dst_b, int E,
                                                              int H, int G) {
    const size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
    const size_t total = (size_t)E * G * H;
    if (i >= total) return;
    const size_t m = i % H, g = (i / H) % G, e = i / ((size_t)H * G);
    dst_s[i] = src_s[(e * H + m) * G + g];
    dst_b[i] = src_b[(e * H + m) * G + g];
}

static bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_pack_down(const moe_layer_t *layer, uint32_t *dst_q, uint16_t *dst_s,
                                    uint16_t *dst_b, void *hip_stream) {
    if (!layer) return MOE_ERR_INVALID_ARG;
    if (layer->down_layout != MOE_DOWN_ROWS) return MOE_ERR_INVALID_ARG;
    // the packed layer must be one the column kernels serve
    moe_layer_t packed = *layer;
    packed.down_layout = MOE_DOWN_COLS;
    moe_status st = check_layer(&packed);
    if (st != MOE_OK) return st;
    if (!dst_q || !dst_s || !dst_b || (uintptr_t)dst_q % 16 || (uintptr_t)dst_s % 4 || (uintptr_t)dst_b % 4)
        return MOE_ERR_INVALID_ARG;
    const int E = layer->n_experts, H = layer->hidden, F = layer->dff;
    const size_t nq = (size_t)E * H * F / 2, nsb = (size_t)E * H * (F / kGroup) * 2;
    const void *srcs[3] = {layer->down_q, layer->down_s, layer->down_b};
    const size_t ns[3] = {nq, nsb, nsb};
    const void *dsts[3] = {dst_q, dst_s, dst_b};
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            if (overlap(srcs[i], ns[i], dsts[j], ns[j])) return MOE_ERR_INVALID_ARG;
    if (overlap(dst_q, nq, dst_s, nsb) || overlap(dst_q, nq, dst_b, nsb) || overlap(dst_s, nsb, dst_b, nsb))
        return MOE_ERR_INVALID_ARG;
    hipStream_t stream = (hipStream_t)hip_stream;
    const int C = F / 32, G = F / kGroup;
    const size_t tq = (size_t)E * C * H, tsb = (size_t)E * G * H;
    hipLaunchKernelGGL(pack_down_q_kernel, dim3((unsigned)((tq + kBlock - 1) / kBlock)), dim3(kBlock), 0, stream,
                       (const uint4 *)layer->down_q, (uint4 *)dst_q, E, H, C);
    hipLaunchKernelGGL(pack_down_sb_kernel, dim3((unsigned)((tsb + kBlock - 1) / kBlock)), dim3(kBlock), 0,
                       stream, layer->down_s, layer->down_b, dst_s, dst_b, E, H, G);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}
