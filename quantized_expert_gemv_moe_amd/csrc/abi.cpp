// Host-only part of the C ABI: argument validation, workspace sizing and
// status strings.  Nothing here touches the device, so every check runs
// (and is tested) without a GPU.  Validating shapes before dispatch instead
// of failing inside a launch follows page "perf(moe): batched decode scales
// 1.55x against 3.25x on dense", Implementation Notes (error handling).
#include <stdint.h>

#include "moe_internal.h"

namespace moe {

static bool pow2_le64(int v) { return v >= 1 && v <= 64 && (v & (v - 1)) == 0; }

// Down projection (and any GEMV over K): fewest lanes per row, i.e. the most
// chunks per lane (nv <= 4) with lanes per row a power of two.
bool pick_geometry(int K, Geometry *g) {
    if (K <= 0 || K % 64) return false;
    const int kch = K / 32;
    for (int nv = 4; nv >= 1; --nv) {
        if (kch % nv == 0 && pow2_le64(kch / nv)) {
            g->lpr = kch / nv;
            g->nv = nv;
            return true;
        }
    }
    return false;
}

// Gate/up projection: a whole wave per row when the row is 64..256 chunks
// (one reduction per row serves both matrices and all tokens in registers),
// otherwise the generic choice.
bool pick_geometry_gate_up(int K, Geometry *g) {
    if (K <= 0 || K % 64) return false;
    const int kch = K / 32;
    if (kch % 64 == 0 && kch / 64 <= 4) {
        g->lpr = 64;
        g->nv = kch / 64;
        return true;
    }
    return pick_geometry(K, g);
}

// Column-layout down projection: NW waves split the dff/32 chunks, CPW
// chunks each; 16 waves when that leaves 2..4 chunks per wave, else 8, else 4.
bool pick_down_cols(int dff, int *nw, int *cpw) {
    if (dff <= 0 || dff % 128) return false;
    const int C = dff / 32;
    if (C % 16 == 0 && C / 16 >= 2 && C / 16 <= 4) *nw = 16;
    // 24 chunks (dff 768): twelve waves of two rather than eight of three;
    // the token-major kernel then fits 106 registers instead of 205 at four
    // row blocks and 61 instead of 125 at one (4 tokens 25.9 -> 25.0 us,
    // 8 tokens 48.6 -> 45.9 us, 32 tokens Zipf 89.5 -> 87.1 us, disjoint
    // 153.4 -> 136.1 us per step; one token within noise)
    else if (C == 24) *nw = 12;
    else if (C % 8 == 0 && C / 8 <= 2) *nw = 8;
    else *nw = 4;
    *cpw = C / *nw;
    return *cpw <= 7 && C % *nw == 0;
}

// Which kernels a projection takes: 4 bits in groups of 64 the specialised
// ones, any other width or group size the generic row kernels.
bool fast_gate_up(const moe_layer_t *L) { return L->bits == 4 && L->group_size == 64; }
bool fast_down(const moe_layer_t *L) { return down_bits_of(L) == 4 && L->group_size == 64; }

// Lanes per row and units per lane of the generic row kernels for rows of K
// inputs: the most lanes (a power of two up to a wave's 64) dividing K/16
// units with at most kGenMaxUpl units per lane, UPL one of the instantiated
// counts.
bool pick_generic(int K, int *lpr, int *upl) {
    if (K <= 0 || K % 16) return false;
    const int units = K / 16;
    for (int l = 64; l >= 1; l >>= 1) {
        if (units % l) continue;
        const int u = units / l;
        if (u > kGenMaxUpl) return false;
        if (u == 5 || u == 7) return false;
        *lpr = l;
        *upl = u;
        return true;
    }
    return false;
}

static bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

moe_status check_layer(const moe_layer_t *L) {
    if (!L) return MOE_ERR_INVALID_ARG;
    if (L->hidden <= 0 || L->dff <= 0 || L->n_experts < 1 || L->top_k < 1)
        return MOE_ERR_INVALID_ARG;
    if (L->n_experts > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
    if (L->top_k > L->n_experts) return MOE_ERR_INVALID_ARG;
    if (L->top_k > MOE_MAX_TOP_K) return MOE_ERR_UNSUPPORTED;
    for (int b : {L->bits, down_bits_of(L)})
        if (b != 4 && b != 6 && b != 8) return MOE_ERR_UNSUPPORTED;
    if (L->group_size != 32 && L->group_size != 64 && L->group_size != 128) return MOE_ERR_UNSUPPORTED;
    if (L->hidden % 64 || L->dff % 64) return MOE_ERR_UNSUPPORTED;
    if (L->hidden % L->group_size || L->dff % L->group_size) return MOE_ERR_UNSUPPORTED;
    if (L->act_dtype != MOE_DTYPE_F32 && L->act_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
    if (!(L->clamp_limit >= 0.0f) || L->clamp_limit > 3.0e38f) return MOE_ERR_INVALID_ARG;
    const void *q[3] = {L->gate_q, L->up_q, L->down_q};
    for (const void *p : q)
        if (!p || !aligned(p, 16)) return MOE_ERR_INVALID_ARG;
    const void *sb[6] = {L->gate_s, L->gate_b, L->up_s, L->up_b, L->down_s, L->down_b};
    for (const void *p : sb)
        if (!p || !aligned(p, 4)) return MOE_ERR_INVALID_ARG;
    if (L->expert_scale && !aligned(L->expert_scale, 4)) return MOE_ERR_INVALID_ARG;
    if (L->down_scale && !aligned(L->down_scale, 4)) return MOE_ERR_INVALID_ARG;
    if (L->activation != MOE_ACT_SWIGLU && L->activation != MOE_ACT_GEGLU) return MOE_ERR_INVALID_ARG;
    if (L->down_layout != MOE_DOWN_ROWS && L->down_layout != MOE_DOWN_COLS) return MOE_ERR_INVALID_ARG;
    // each projection by its own width: specialised kernels for 4-bit in
    // groups of 64, the generic row kernels otherwise
    Geometry g;
    int lpr, upl;
    if (fast_gate_up(L) ? !pick_geometry_gate_up(L->hidden, &g) : !pick_generic(L->hidden, &lpr, &upl))
        return MOE_ERR_UNSUPPORTED;
    if (!fast_down(L)) {
        if (L->down_layout != MOE_DOWN_ROWS) return MOE_ERR_UNSUPPORTED;
        return pick_generic(L->dff, &lpr, &upl) ? MOE_OK : MOE_ERR_UNSUPPORTED;
    }
    if (L->down_layout == MOE_DOWN_ROWS) {
        if (!pick_geometry(L->dff, &g)) return MOE_ERR_UNSUPPORTED;
        if (down_rows_slot_bytes(L->dff) > kDownRowsLdsBytes) return MOE_ERR_UNSUPPORTED;
    } else if (L->down_layout == MOE_DOWN_COLS) {
        int nw, cpw;
        if (!pick_down_cols(L->dff, &nw, &cpw)) return MOE_ERR_UNSUPPORTED;
    } else {
        return MOE_ERR_INVALID_ARG;
    }
    return MOE_OK;
}

moe_status check_route_args(const void *logits, int32_t n_tokens, int32_t n_experts,
                            int32_t top_k, const void *idx, const void *w) {
    if (n_tokens < 0 || n_experts < 1 || top_k < 1 || top_k > n_experts) return MOE_ERR_INVALID_ARG;
    if (n_experts > MOE_MAX_EXPERTS || top_k > MOE_MAX_TOP_K) return MOE_ERR_UNSUPPORTED;
    if (n_tokens > 0 && (!logits || !idx || !w)) return MOE_ERR_INVALID_ARG;
    if ((int64_t)n_tokens * top_k > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status check_plan_args(const void *idx, int32_t n_tokens, int32_t n_experts, int32_t top_k,
                           const moe_plan_t *plan) {
    if (n_tokens < 0 || n_experts < 1 || top_k < 1 || top_k > n_experts) return MOE_ERR_INVALID_ARG;
    if (n_experts > MOE_MAX_EXPERTS || top_k > MOE_MAX_TOP_K) return MOE_ERR_UNSUPPORTED;
    if (!plan || !plan->counts || !plan->offsets || !plan->unique_experts || !plan->n_unique ||
        !plan->work || (uintptr_t)plan->work % 16)
        return MOE_ERR_INVALID_ARG;
    if (n_tokens > 0 && (!idx || !plan->sorted_slots)) return MOE_ERR_INVALID_ARG;
    if ((int64_t)n_tokens * top_k > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// Host-side checks shared by the three expert entry points.
moe_status check_step(const moe_layer_t *layer, int32_t n_tokens, const moe_plan_t *plan,
                             void *workspace, size_t workspace_bytes) {
    moe_status st = check_layer(layer);
    if (st != MOE_OK) return st;
    if (n_tokens < 0) return MOE_ERR_INVALID_ARG;
    if (n_tokens > MOE_MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
    if (n_tokens == 0) return MOE_OK;
    if (!plan || !plan->work || !plan->sorted_slots || (uintptr_t)plan->work % 16)
        return MOE_ERR_INVALID_ARG;
    if (!workspace || (uintptr_t)workspace % 256) return MOE_ERR_INVALID_ARG;
    if (workspace_bytes < workspace_layout(layer, n_tokens).total) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

moe_status check_x(const void *x) {
    if (!x || (uintptr_t)x % 16) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

moe_status check_out(const void *x, const int32_t *topk_idx, const float *topk_w,
                            const void *residual, const void *out) {
    if (!topk_idx || !topk_w || !out) return MOE_ERR_INVALID_ARG;
    if (out == x || (residual && out == residual)) return MOE_ERR_INVALID_ARG;
    if ((uintptr_t)out % 4 || (residual && (uintptr_t)residual % 4)) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

Workspace workspace_layout(const moe_layer_t *L, int64_t max_tokens) {
    Workspace w{0, 0, 0};
    const size_t slots = (size_t)max_tokens * (size_t)L->top_k;
    w.h_off = 0;
    w.y_off = align256(slots * (size_t)L->dff * sizeof(float));
    w.total = w.y_off + align256(slots * (size_t)L->hidden * sizeof(float));
    return w;
}

}  // namespace moe

extern "C" {

size_t moe_workspace_size(const moe_layer_t *layer, int32_t max_tokens) {
    if (moe::check_layer(layer) != MOE_OK || max_tokens < 0) return 0;
    return moe::workspace_layout(layer, max_tokens).total;
}

moe_status moe_layer_check(const moe_layer_t *layer) { return moe::check_layer(layer); }

const char *moe_status_str(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported configuration (caller falls back)";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_DEVICE: return "device launch failed";
    }
    return "unknown status";
}

int32_t moe_abi_version(void) { return 8; }

}  // extern "C"
