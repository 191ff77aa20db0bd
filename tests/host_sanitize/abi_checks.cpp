// Host validation of the C ABI (abi.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer: every check runs on ordinary, extreme and
// garbage arguments, and the statuses the ABI documents are asserted.  No
// device code is compiled or called.
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "moe_internal.h"

using namespace moe;

static int failures = 0;

#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            std::fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

static const uintptr_t kFake = 0x10000000;

static moe_layer_t base_layer() {
    moe_layer_t L;
    std::memset(&L, 0, sizeof L);
    L.hidden = 2048;
    L.dff = 768;
    L.n_experts = 128;
    L.top_k = 8;
    L.bits = 4;
    L.group_size = 64;
    L.act_dtype = MOE_DTYPE_BF16;
    L.gate_q = (const uint32_t *)(kFake + 0x000000);
    L.up_q = (const uint32_t *)(kFake + 0x100000);
    L.gate_s = (const uint16_t *)(kFake + 0x200000);
    L.gate_b = (const uint16_t *)(kFake + 0x300000);
    L.up_s = (const uint16_t *)(kFake + 0x400000);
    L.up_b = (const uint16_t *)(kFake + 0x500000);
    L.down_q = (const uint32_t *)(kFake + 0x600000);
    L.down_s = (const uint16_t *)(kFake + 0x700000);
    L.down_b = (const uint16_t *)(kFake + 0x800000);
    return L;
}

static const int32_t kInts[] = {INT32_MIN, INT32_MIN + 1, -65536, -64, -1, 0, 1, 2, 3, 4, 5, 6, 7, 8,
                                16, 17, 31, 32, 48, 63, 64, 65, 96, 127, 128, 129, 192, 256, 320, 704,
                                768, 1024, 1025, 1408, 2048, 4096, 6144, 8064, 8192, 16384, 65535,
                                65536, 1 << 20, INT32_MAX - 63, INT32_MAX - 1, INT32_MAX};

// Every int field of the layer through every value above: the checks must
// return a defined status without undefined behaviour, and accept only
// values they support.
static void sweep_layer_fields() {
    int32_t moe_layer_t::*fields[] = {&moe_layer_t::hidden, &moe_layer_t::dff, &moe_layer_t::n_experts,
                                      &moe_layer_t::top_k, &moe_layer_t::bits, &moe_layer_t::group_size,
                                      &moe_layer_t::down_layout, &moe_layer_t::activation,
                                      &moe_layer_t::down_bits};
    for (auto f : fields)
        for (int32_t v : kInts) {
            moe_layer_t L = base_layer();
            L.*f = v;
            const moe_status st = moe_layer_check(&L);
            EXPECT(st == MOE_OK || st == MOE_ERR_INVALID_ARG || st == MOE_ERR_UNSUPPORTED);
            const size_t ws = moe_workspace_size(&L, 32);
            EXPECT((st == MOE_OK) == (ws > 0));
        }
    for (int32_t v : kInts) {
        moe_layer_t L = base_layer();
        L.act_dtype = v & 7;
        const moe_status st = moe_layer_check(&L);
        EXPECT(st == ((v & 7) <= 1 ? MOE_OK : MOE_ERR_INVALID_ARG));
    }
    // pairs of shape fields, so that divisibility checks meet each other
    for (int32_t h : kInts)
        for (int32_t d : kInts) {
            moe_layer_t L = base_layer();
            L.hidden = h;
            L.dff = d;
            for (int layout : {MOE_DOWN_ROWS, MOE_DOWN_COLS})
                for (int g : {32, 64, 128}) {
                    L.down_layout = layout;
                    L.group_size = g;
                    const moe_status st = moe_layer_check(&L);
                    if (st == MOE_OK) EXPECT(h > 0 && d > 0 && h % g == 0 && d % g == 0);
                }
        }
}

static void clamp_limits() {
    const float vals[] = {0.0f, -0.0f, 1.0f, 10.0f, 3.0e38f, INFINITY, -1.0f, -INFINITY, NAN};
    const moe_status want[] = {MOE_OK, MOE_OK, MOE_OK, MOE_OK, MOE_OK, MOE_ERR_INVALID_ARG,
                               MOE_ERR_INVALID_ARG, MOE_ERR_INVALID_ARG, MOE_ERR_INVALID_ARG};
    for (size_t i = 0; i < sizeof vals / sizeof vals[0]; ++i) {
        moe_layer_t L = base_layer();
        L.clamp_limit = vals[i];
        EXPECT(moe_layer_check(&L) == want[i]);
    }
}

static void pointers() {
    EXPECT(moe_layer_check(nullptr) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_workspace_size(nullptr, 4) == 0);
    moe_layer_t L = base_layer();
    L.gate_q = nullptr;
    EXPECT(moe_layer_check(&L) == MOE_ERR_INVALID_ARG);
    L = base_layer();
    L.down_q = (const uint32_t *)(kFake + 8);  // not 16-byte aligned
    EXPECT(moe_layer_check(&L) == MOE_ERR_INVALID_ARG);
    L = base_layer();
    L.up_b = (const uint16_t *)(kFake + 2);  // not 4-byte aligned
    EXPECT(moe_layer_check(&L) == MOE_ERR_INVALID_ARG);
    L = base_layer();
    L.expert_scale = (const float *)(kFake + 1);
    EXPECT(moe_layer_check(&L) == MOE_ERR_INVALID_ARG);
    L = base_layer();
    L.down_scale = (const float *)(kFake + 0x900000);
    L.expert_scale = (const float *)(kFake + 0xA00000);
    EXPECT(moe_layer_check(&L) == MOE_OK);
}

static void workspace_sizes() {
    moe_layer_t L = base_layer();
    const size_t one = moe_workspace_size(&L, 1);
    EXPECT(one >= (size_t)8 * (768 + 2048) * 4 && one % 256 == 0);
    EXPECT(moe_workspace_size(&L, 0) == 0);
    EXPECT(moe_workspace_size(&L, -1) == 0);
    // the largest request stays a size_t product, far from wrapping
    const size_t big = moe_workspace_size(&L, INT32_MAX);
    EXPECT(big > one && big / one >= (size_t)INT32_MAX / 2);
    L.hidden = 8192;
    L.dff = 6144;
    L.top_k = 16;
    EXPECT(moe_workspace_size(&L, INT32_MAX) > big);
}

static void step_checks() {
    moe_layer_t L = base_layer();
    int32_t dummy[8];
    moe_plan_t plan = {dummy, dummy, dummy, dummy, dummy, (int32_t *)(kFake + 0xB00000)};
    void *ws = (void *)(kFake + 0xC00000);
    const size_t need = moe_workspace_size(&L, 4);
    for (int32_t n : kInts) {
        const moe_status st = check_step(&L, n, &plan, ws, need);
        if (n < 0) EXPECT(st == MOE_ERR_INVALID_ARG);
        else if (n > MOE_MAX_TOKENS) EXPECT(st == MOE_ERR_UNSUPPORTED);
        else if (n > 4) EXPECT(st == MOE_ERR_WORKSPACE);
        else EXPECT(st == MOE_OK);
    }
    EXPECT(check_step(&L, 4, nullptr, ws, need) == MOE_ERR_INVALID_ARG);
    EXPECT(check_step(&L, 0, nullptr, nullptr, 0) == MOE_OK);  // empty batch
    moe_plan_t bad = plan;
    bad.work = (int32_t *)(kFake + 4);
    EXPECT(check_step(&L, 4, &bad, ws, need) == MOE_ERR_INVALID_ARG);
    bad = plan;
    bad.work = nullptr;
    EXPECT(check_step(&L, 4, &bad, ws, need) == MOE_ERR_INVALID_ARG);
    EXPECT(check_step(&L, 4, &plan, (void *)(kFake + 0xC00010), need) == MOE_ERR_INVALID_ARG);
    EXPECT(check_step(&L, 4, &plan, ws, need - 1) == MOE_ERR_WORKSPACE);
    EXPECT(check_x(nullptr) == MOE_ERR_INVALID_ARG);
    EXPECT(check_x((void *)(kFake + 8)) == MOE_ERR_INVALID_ARG);
    EXPECT(check_x((void *)kFake) == MOE_OK);
    const void *x = (void *)kFake, *o = (void *)(kFake + 0x1000), *r = (void *)(kFake + 0x2000);
    EXPECT(check_out(x, dummy, (const float *)dummy, nullptr, o) == MOE_OK);
    EXPECT(check_out(x, dummy, (const float *)dummy, r, o) == MOE_OK);
    EXPECT(check_out(x, dummy, (const float *)dummy, r, x) == MOE_ERR_INVALID_ARG);
    EXPECT(check_out(x, dummy, (const float *)dummy, r, r) == MOE_ERR_INVALID_ARG);
    EXPECT(check_out(x, nullptr, (const float *)dummy, nullptr, o) == MOE_ERR_INVALID_ARG);
    EXPECT(check_out(x, dummy, (const float *)dummy, nullptr, (void *)(kFake + 0x1002)) == MOE_ERR_INVALID_ARG);
}

static void route_and_plan_checks() {
    int32_t dummy[8];
    moe_plan_t plan = {dummy, dummy, dummy, dummy, dummy, (int32_t *)(kFake + 0xB00000)};
    const void *p = (void *)kFake;
    for (int32_t n : kInts)
        for (int32_t e : kInts)
            for (int32_t k : {INT32_MIN, -1, 0, 1, 2, 8, 16, 17, INT32_MAX}) {
                const moe_status a = check_route_args(p, n, e, k, p, p);
                const moe_status b = check_plan_args(p, n, e, k, &plan);
                EXPECT(a == MOE_OK || a == MOE_ERR_INVALID_ARG || a == MOE_ERR_UNSUPPORTED);
                EXPECT(b == a);  // same shape rules, every pointer present
                if (a == MOE_OK) EXPECT(n >= 0 && e >= 1 && e <= MOE_MAX_EXPERTS && k >= 1 && k <= e &&
                                        k <= MOE_MAX_TOP_K && (int64_t)n * k <= INT32_MAX / 2);
            }
    EXPECT(check_route_args(nullptr, 1, 8, 2, p, p) == MOE_ERR_INVALID_ARG);
    EXPECT(check_route_args(nullptr, 0, 8, 2, nullptr, nullptr) == MOE_OK);
    EXPECT(check_plan_args(p, 1, 8, 2, nullptr) == MOE_ERR_INVALID_ARG);
    moe_plan_t nowork = plan;
    nowork.work = nullptr;
    EXPECT(check_plan_args(p, 1, 8, 2, &nowork) == MOE_ERR_INVALID_ARG);
}

static void geometry_pickers() {
    for (int K = -200; K <= 20000; ++K) {
        Geometry g{0, 0};
        if (pick_geometry(K, &g)) EXPECT(g.lpr >= 1 && g.lpr <= 64 && g.nv >= 1 && g.nv <= 4 && g.lpr * g.nv * 32 == K);
        if (pick_geometry_gate_up(K, &g)) EXPECT(g.lpr * g.nv * 32 == K);
        int a = 0, b = 0;
        if (pick_generic(K, &a, &b)) EXPECT(a * b * 16 == K && b <= kGenMaxUpl);
        if (pick_down_cols(K, &a, &b)) EXPECT(a * b * 32 == K);
    }
    for (int K : kInts) {
        Geometry g{0, 0};
        int a = 0, b = 0;
        (void)pick_geometry(K, &g);
        (void)pick_geometry_gate_up(K, &g);
        (void)pick_generic(K, &a, &b);
        (void)pick_down_cols(K, &a, &b);
        (void)per_lane_bucket(K < 0 ? 0 : K);
        (void)down_rows_slot_bytes(K);
    }
}

static void strings() {
    for (int s = MOE_OK; s <= MOE_ERR_DEVICE; ++s) EXPECT(std::strlen(moe_status_str((moe_status)s)) > 0);
    EXPECT(moe_abi_version() > 0);
}

int main() {
    sweep_layer_fields();
    clamp_limits();
    pointers();
    workspace_sizes();
    step_checks();
    route_and_plan_checks();
    geometry_pickers();
    strings();
    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("abi checks ok\n");
    return 0;
}
