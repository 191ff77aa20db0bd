// Host-side helpers shared by the entry points (validation, geometry).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "moe_decode.h"

namespace moe {

// Lane geometry of a GEMV over K inputs: a row is read as K/32 16-byte
// chunks by `lpr` lanes (a power of two, 1..64), each lane taking `nv`
// chunks (1..4), chunk c of a row going to lane c % lpr.
struct Geometry {
    int lpr;
    int nv;
};
bool pick_geometry(int K, Geometry *g);
bool pick_geometry_gate_up(int K, Geometry *g);
// Waves per workgroup and 32-input chunks per wave of the column-layout down
// kernel; false when that layout has no kernel for this dff.
bool pick_down_cols(int dff, int *nw, int *cpw);

// Weight formats, per projection: gate and up in 4 bits and groups of 64
// take the specialised gate+up kernels (fast_gate_up), a down projection in
// 4 bits and groups of 64 the specialised down kernels (fast_down); any other
// width or group size takes the generic row kernels (rows layout only for
// down).  pick_generic gives their lanes per row and 16-input units per lane
// for rows of K inputs.
constexpr int kGenMaxUpl = 8;  // 16-input units per lane of the generic row kernels
bool fast_gate_up(const moe_layer_t *layer);
bool fast_down(const moe_layer_t *layer);
// Width of the down projection: down_bits, or bits when down_bits is 0.
inline int down_bits_of(const moe_layer_t *layer) { return layer->down_bits ? layer->down_bits : layer->bits; }
bool pick_generic(int K, int *lpr, int *upl);
moe_status launch_generic_gate_up(const moe_layer_t *layer, const void *x, int n_tokens,
                                  const moe_plan_t *plan, float *h, hipStream_t stream);
moe_status launch_generic_down(const moe_layer_t *layer, int n_tokens, const moe_plan_t *plan,
                               const float *h, float *y, hipStream_t stream);

// Validation without device access.
moe_status check_layer(const moe_layer_t *layer);
// Checks shared by the expert entry points: the layer, the token count, the
// plan's work records and the workspace; x (16-byte aligned); out, residual
// and routing arrays.
moe_status check_step(const moe_layer_t *layer, int32_t n_tokens, const moe_plan_t *plan, void *workspace,
                      size_t workspace_bytes);
moe_status check_x(const void *x);
moe_status check_out(const void *x, const int32_t *topk_idx, const float *topk_w, const void *residual,
                     const void *out);

// Tile kernels (tile.hip) for batches of kTileMinTokens tokens or more:
// every distinct expert's tokens in blocks of 64 on MFMA, the workgroup's
// waves splitting the output rows.  The *_ok checks say whether a layer
// has them; the launchers take checked arguments.
constexpr int kTileMinTokens = 128;
bool tile_gate_up_ok(const moe_layer_t *layer);
bool tile_down_ok(const moe_layer_t *layer);
moe_status launch_gate_up_tile(const moe_layer_t *layer, const void *x, int n_tokens, const moe_plan_t *plan,
                               float *h, hipStream_t stream);
moe_status launch_down_tile(const moe_layer_t *layer, int n_tokens, const moe_plan_t *plan, const float *h,
                            float *y, hipStream_t stream);

// Enqueues the deduplicated gate+up kernels of a planned batch (h into the
// workspace); the layer and arguments are already checked.
moe_status enqueue_gate_up(const moe_layer_t *layer, const void *x, int n_tokens, const moe_plan_t *plan,
                           void *workspace, hipStream_t stream);
moe_status check_route_args(const void *logits, int32_t n_tokens, int32_t n_experts,
                            int32_t top_k, const void *idx, const void *w);
moe_status check_plan_args(const void *idx, int32_t n_tokens, int32_t n_experts,
                           int32_t top_k, const moe_plan_t *plan);

// Workspace layout of moe_decode_step: h [slots][dff] fp32, then the
// per-slot expert outputs [slots][hidden] fp32, each 256-byte aligned.
struct Workspace {
    size_t h_off, y_off, total;
};
Workspace workspace_layout(const moe_layer_t *layer, int64_t max_tokens);

constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// LDS of the row-layout down kernel: h of at least one slot and its group
// sums must fit (dff <= 8064), else that layout has no kernel for the shape.
constexpr size_t kDownRowsLdsBytes = 32768;
constexpr size_t down_rows_slot_bytes(int dff) { return ((size_t)dff + dff / 64) * sizeof(float); }

// Logits per lane of the router's wave: the smallest of 1, 2, 4, 8, 16 that
// holds n_experts / 64.
inline int per_lane_bucket(int n_experts) {
    const int per_lane = (n_experts + 63) / 64;
    return per_lane <= 1 ? 1 : per_lane <= 2 ? 2 : per_lane <= 4 ? 4 : per_lane <= 8 ? 8 : 16;
}

// Every (lanes per row, chunks per lane) pair that the geometry pickers return.
#define MOE_GEOMETRY_SWITCH(G, RET, FN, ...)                           \
    switch ((G).lpr * 8 + (G).nv) {                                    \
        case 64 * 8 + 1: RET = FN<64, 1>(__VA_ARGS__); break;          \
        case 64 * 8 + 2: RET = FN<64, 2>(__VA_ARGS__); break;          \
        case 64 * 8 + 3: RET = FN<64, 3>(__VA_ARGS__); break;          \
        case 64 * 8 + 4: RET = FN<64, 4>(__VA_ARGS__); break;          \
        case 32 * 8 + 3: RET = FN<32, 3>(__VA_ARGS__); break;          \
        case 32 * 8 + 4: RET = FN<32, 4>(__VA_ARGS__); break;          \
        case 16 * 8 + 3: RET = FN<16, 3>(__VA_ARGS__); break;          \
        case 16 * 8 + 4: RET = FN<16, 4>(__VA_ARGS__); break;          \
        case 8 * 8 + 3: RET = FN<8, 3>(__VA_ARGS__); break;            \
        case 8 * 8 + 4: RET = FN<8, 4>(__VA_ARGS__); break;            \
        case 4 * 8 + 3: RET = FN<4, 3>(__VA_ARGS__); break;            \
        case 4 * 8 + 4: RET = FN<4, 4>(__VA_ARGS__); break;            \
        case 2 * 8 + 3: RET = FN<2, 3>(__VA_ARGS__); break;            \
        case 2 * 8 + 4: RET = FN<2, 4>(__VA_ARGS__); break;            \
        case 1 * 8 + 2: RET = FN<1, 2>(__VA_ARGS__); break;            \
        case 1 * 8 + 3: RET = FN<1, 3>(__VA_ARGS__); break;            \
        case 1 * 8 + 4: RET = FN<1, 4>(__VA_ARGS__); break;            \
        default: RET = MOE_ERR_UNSUPPORTED; break;                     \
    }

}  // namespace moe
