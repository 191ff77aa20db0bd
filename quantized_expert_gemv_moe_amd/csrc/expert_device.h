// Device helpers shared by the expert kernels of every weight format: the
// plan records a workgroup walks, streaming weight loads, and the gated
// activation that turns gate and up pre-activations into h.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_decode.h"

namespace moe {

struct PlanView {
    const int4 *work;          // {expert, first, count, first slot} per distinct expert
    const int *sorted_slots;
};

// The work record of the workgroup's distinct expert (one 16-byte load);
// false past the last distinct expert or on a malformed record, so no kernel
// ever indexes out of bounds.
struct Work {
    int e, first, count, slot0;
};
__device__ __forceinline__ bool plan_expert(const PlanView &p, int u, int n_experts, int n_slots, Work *w) {
    const int4 r = p.work[u];
    if ((unsigned)r.x >= (unsigned)n_experts) return false;
    if (r.y < 0 || r.z < 1 || r.y > n_slots - r.z || (unsigned)r.w >= (unsigned)n_slots) return false;
    *w = Work{r.x, r.y, r.z, r.w};
    return true;
}

// Device view of a plan (host side).
inline PlanView plan_view(const moe_plan_t *plan) {
    return PlanView{(const int4 *)plan->work, plan->sorted_slots};
}

// Slot i of the expert's list (the first one comes with the record).
__device__ __forceinline__ int plan_slot(const PlanView &p, const Work &w, int i, int n_slots) {
    const int s = i == 0 ? w.slot0 : p.sorted_slots[w.first + i];
    return (unsigned)s < (unsigned)n_slots ? s : 0;  // malformed plan: stay in bounds
}

// Streaming 16-byte load of weights that are read once per step.
__device__ __forceinline__ uint4 load_stream(const uint4 *p) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_nontemporal_load((const v4u *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// h from the gate and up pre-activations: expert-scale sidecar, clamp, then
// SiLU(g) * u, or GELU(g) * u (tanh form) for the GeGLU variant.
__device__ __forceinline__ float act_mul(float g, float u, float sc, float lim, int activation) {
    g *= sc;
    u *= sc;
    if (lim > 0.f) {
        g = fminf(fmaxf(g, -lim), lim);
        u = fminf(fmaxf(u, -lim), lim);
    }
    if (activation == MOE_ACT_GEGLU)
        return 0.5f * g * (1.f + tanhf(0.7978845608028654f * (g + 0.044715f * g * g * g))) * u;
    return g / (1.f + expf(-g)) * u;
}

}  // namespace moe
