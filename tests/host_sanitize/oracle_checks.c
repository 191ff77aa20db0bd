/* The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer: each
 * entry point runs on small synthetic layers of every supported width and
 * group size, both activation dtypes, both activations, with and without
 * sidecars and clamp, on empty, single and ragged batches, and on the
 * conversions' special values.  Memory and arithmetic faults abort the run;
 * a few invariants are asserted on the way (routing weights sum to one, the
 * plan sorts every slot, outputs are finite). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t hidden, dff, n_experts, top_k;
    int32_t x_is_bf16;
    double clamp_limit;
    const uint32_t *gate_q, *up_q, *down_q;
    const uint16_t *gate_s, *gate_b, *up_s, *up_b, *down_s, *down_b;
    const float *sidecar;
    int32_t activation;
    const float *down_sidecar;
    int32_t bits, down_bits, group_size;
} orc_layer;

double orc_f16_to_f64(uint16_t h);
double orc_bf16_to_f64(uint16_t b);
uint16_t orc_f64_to_bf16(double v);
void orc_dequant(const uint32_t *q, const uint16_t *s, const uint16_t *b, int rows, int cols, int bits,
                 int group, double *w);
int orc_route_topk(const float *logits, int n_tokens, int n_experts, int top_k, int32_t *idx, double *w);
int orc_plan(const int32_t *idx, int n_tokens, int n_experts, int top_k, int32_t *counts, int32_t *offsets,
             int32_t *sorted_slots, int32_t *unique, int32_t *n_unique);
int orc_decode_step(const orc_layer *L, const void *x, int n_tokens, const int32_t *idx, const double *w,
                    double *out, double *h_out, double *y_out);
void orc_round_bf16(const double *v, size_t n, uint16_t *out);
void orc_round_f32(const double *v, size_t n, float *out);
void orc_residual_bf16(const uint16_t *x, const double *out, size_t n, uint16_t *x_next);
int orc_router_logits(const void *x, int x_is_bf16, int n_tokens, int hidden, int n_experts,
                      const uint16_t *w_router, double *logits);

static int failures = 0;
#define EXPECT(c)                                                          \
    do {                                                                   \
        if (!(c)) {                                                        \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c);        \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 16);
}
static float uniform(void) { return (float)(next32() & 0xFFFFFF) / 16777216.0f; }

/* Exactly-sized buffers, so ASan sees any read past a matrix. */
static uint32_t *rand_words(size_t n) {
    uint32_t *p = malloc(n * sizeof *p);
    for (size_t i = 0; i < n; ++i) p[i] = next32();
    return p;
}
static uint16_t *fp16_vals(size_t n, uint16_t lo, uint16_t span) {
    uint16_t *p = malloc(n * sizeof *p);
    for (size_t i = 0; i < n; ++i) p[i] = (uint16_t)(lo + next32() % span);
    return p;
}

static void run_layer(int H, int F, int E, int k, int bits, int dbits, int G, int bf16, int act, int side,
                      double clamp) {
    orc_layer L;
    memset(&L, 0, sizeof L);
    L.hidden = H, L.dff = F, L.n_experts = E, L.top_k = k, L.x_is_bf16 = bf16, L.clamp_limit = clamp;
    L.bits = bits, L.down_bits = dbits, L.group_size = G, L.activation = act;
    const size_t gw = (size_t)E * F * H * bits / 32, dw = (size_t)E * H * F * dbits / 32;
    const size_t gs = (size_t)E * F * (H / G), ds = (size_t)E * H * (F / G);
    uint32_t *gq = rand_words(gw), *uq = rand_words(gw), *dq = rand_words(dw);
    /* scales around 2^-9..2^-8, biases small and of either sign */
    uint16_t *gsc = fp16_vals(gs, 0x1C00, 0x400), *usc = fp16_vals(gs, 0x1C00, 0x400);
    uint16_t *dsc = fp16_vals(ds, 0x1C00, 0x400);
    uint16_t *gb = fp16_vals(gs, 0x9C00, 0x400), *ub = fp16_vals(gs, 0x9C00, 0x400);
    uint16_t *db = fp16_vals(ds, 0x1C00, 0x400);
    float *sc = malloc((size_t)E * sizeof *sc), *dsd = malloc((size_t)E * sizeof *dsd);
    for (int e = 0; e < E; ++e) sc[e] = 0.5f + uniform(), dsd[e] = 0.25f + uniform();
    L.gate_q = gq, L.up_q = uq, L.down_q = dq, L.gate_s = gsc, L.gate_b = gb, L.up_s = usc, L.up_b = ub;
    L.down_s = dsc, L.down_b = db;
    L.sidecar = side ? sc : NULL;
    L.down_sidecar = side ? dsd : NULL;

    const int batches[] = {0, 1, 3};
    for (int bi = 0; bi < 3; ++bi) {
        const int B = batches[bi];
        const size_t nx = (size_t)(B ? B : 1) * H, ns = (size_t)(B ? B : 1) * k;
        void *x = malloc(nx * (bf16 ? 2 : 4));
        for (size_t i = 0; i < nx; ++i) {
            const float v = uniform() * 2.0f - 1.0f;
            if (bf16) {
                uint32_t u;
                memcpy(&u, &v, 4);
                ((uint16_t *)x)[i] = (uint16_t)(u >> 16);
            } else {
                ((float *)x)[i] = v;
            }
        }
        float *logits = malloc((size_t)(B ? B : 1) * E * sizeof *logits);
        for (size_t i = 0; i < (size_t)(B ? B : 1) * E; ++i) logits[i] = (float)(next32() % 7);  /* ties */
        int32_t *idx = malloc(ns * sizeof *idx);
        double *w = malloc(ns * sizeof *w);
        EXPECT(orc_route_topk(logits, B, E, k, idx, w) == 0);
        for (int t = 0; t < B; ++t) {
            double sum = 0;
            for (int j = 0; j < k; ++j) sum += w[t * k + j];
            EXPECT(fabs(sum - 1.0) < 1e-12);
        }
        int32_t *cnt = malloc((size_t)E * 4), *off = malloc((size_t)(E + 1) * 4), *srt = malloc(ns * 4);
        int32_t *uni = malloc((size_t)E * 4), nu = -1;
        EXPECT(orc_plan(idx, B, E, k, cnt, off, srt, uni, &nu) == 0);
        EXPECT(off[E] == B * k && nu >= (B ? 1 : 0) && nu <= E);
        double *out = malloc(nx * sizeof *out), *h = malloc(ns * F * sizeof *h), *y = malloc(ns * H * sizeof *y);
        EXPECT(orc_decode_step(&L, x, B, idx, w, out, h, y) == 0);
        for (size_t i = 0; i < (size_t)B * H; ++i) EXPECT(isfinite(out[i]));
        uint16_t *ob = malloc(nx * 2), *xn = malloc(nx * 2);
        float *of = malloc(nx * 4);
        orc_round_bf16(out, (size_t)B * H, ob);
        orc_round_f32(out, (size_t)B * H, of);
        if (bf16) orc_residual_bf16((const uint16_t *)x, out, (size_t)B * H, xn);
        uint16_t *wr = fp16_vals((size_t)E * H, 0x3C00, 0x100);  /* any bf16 bits will do */
        double *lg = malloc((size_t)(B ? B : 1) * E * sizeof *lg);
        EXPECT(orc_router_logits(x, bf16, B, H, E, wr, lg) == 0);
        /* a bad expert id is refused, not read */
        if (B) {
            idx[0] = E;
            EXPECT(orc_plan(idx, B, E, k, cnt, off, srt, uni, &nu) == -1);
            EXPECT(orc_decode_step(&L, x, B, idx, w, out, NULL, NULL) == -1);
            idx[0] = -1;
            EXPECT(orc_decode_step(&L, x, B, idx, w, out, NULL, NULL) == -1);
        }
        free(x), free(logits), free(idx), free(w), free(cnt), free(off), free(srt), free(uni);
        free(out), free(h), free(y), free(ob), free(xn), free(of), free(wr), free(lg);
    }
    /* dense copies of one expert's matrices, exactly sized */
    double *wd = malloc((size_t)F * H * sizeof *wd);
    orc_dequant(gq, gsc, gb, F, H, bits, G, wd);
    orc_dequant(dq, dsc, db, H, F, dbits, G, wd);
    free(wd);
    free(gq), free(uq), free(dq), free(gsc), free(usc), free(dsc), free(gb), free(ub), free(db);
    free(sc), free(dsd);
}

static void conversions(void) {
    for (uint32_t h = 0; h < 65536; ++h) {
        (void)orc_f16_to_f64((uint16_t)h);
        const double b = orc_bf16_to_f64((uint16_t)h);
        if (!isnan(b)) EXPECT(orc_f64_to_bf16(b) == (uint16_t)h);
    }
    EXPECT(orc_f64_to_bf16(0.0) == 0x0000 && orc_f64_to_bf16(-0.0) == 0x8000);
    EXPECT(orc_f64_to_bf16(INFINITY) == 0x7F80 && orc_f64_to_bf16(-INFINITY) == 0xFF80);
    EXPECT(orc_f64_to_bf16(NAN) == 0x7FC0);
    EXPECT(orc_f64_to_bf16(1e300) == 0x7F80 && orc_f64_to_bf16(-1e300) == 0xFF80);
    EXPECT(orc_f64_to_bf16(1e-320) == 0x0000 && orc_f64_to_bf16(-5e-324) == 0x8000);
    EXPECT(orc_f64_to_bf16(ldexp(1.0, -133)) == 0x0001);
    const double v[] = {1e300, -1e300, 1e-320, NAN, INFINITY};
    float f[5];
    uint16_t b[5];
    orc_round_f32(v, 5, f);
    orc_round_bf16(v, 5, b);
    EXPECT(isinf(f[0]) && isinf(f[1]) && f[2] == 0.0f && isnan(f[3]) && isinf(f[4]));
}

int main(void) {
    /* widths and groups of the layer format, 6 bits straddling words */
    const int widths[][3] = {{4, 4, 64}, {4, 6, 64}, {6, 6, 32}, {8, 8, 128}, {8, 4, 128}, {4, 4, 32}, {6, 8, 64}};
    for (int i = 0; i < 7; ++i)
        for (int bf16 = 0; bf16 < 2; ++bf16)
            run_layer(256, 128, 6, 2, widths[i][0], widths[i][1], widths[i][2], bf16, i & 1, i % 3 == 0,
                      i == 2 ? 0.5 : 0.0);
    run_layer(128, 64, 8, 8, 4, 4, 64, 1, 0, 1, 10.0);  /* k = E */
    run_layer(64, 64, 1, 1, 4, 4, 64, 0, 1, 0, 0.0);    /* one expert */
    conversions();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle checks ok\n");
    return 0;
}
