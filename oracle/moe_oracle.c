/*
 * moe_oracle.c -- plain CPU oracle of the decode-time quantized-expert MoE
 * block.  TEST INFRASTRUCTURE ONLY: it is loaded by the tests, by the smoke
 * check and by the benchmark's CPU-baseline leg, never by the product path.
 * It shares no header, helper, table or constant with the HIP library.
 *
 * What it computes is the plain definition, per (token, k) slot, in fp64,
 * with no deduplication, no blocking and no fusion:
 *
 *   route    : per token, order experts by logit (descending, ties to the
 *              lower id), keep top_k, weight w_j = softmax over the kept
 *              logits (softmax over all experts, top-k, renormalise).
 *              The pages name a "router" as one third of the per-token cost
 *              (page "perf(moe): attribute the MoE decode gap at the M = 1
 *              expert gather", Proposed Solution step 2; page "perf(moe):
 *              batched decode scales 1.55x against 3.25x on dense",
 *              Proposed Solution); the formula itself is a reading.
 *   plan     : stable counting sort of the slots by expert id and the list
 *              of distinct experts -- the cross-cohort dedup that page
 *              "perf(moe): batched decode scales ..." proposes (Proposed
 *              Solution, second bullet).
 *   expert   : SwitchGLU expert: g = Wg x, u = Wu x (affine 4-, 6- or 8-bit weights,
 *              groups of 64, dequantised exactly in fp64), optional
 *              per-expert scale sidecar on g and u, optional clamp of g and
 *              u to [-L, L], h = silu(g) * u, y = Wd h.  The gather of one
 *              expert per (token, k) slot is the M = 1 path of page
 *              "perf(moe): attribute ..." (Problem / Background); the clamp
 *              stage and the expert-scale sidecars are the deepseek_v4 and
 *              inkling features named there.
 *   combine  : out[t] = sum_{j<k} w_j * y_{t,j}, "sum over k per token"
 *              (page "perf(moe): batched decode scales ...", Proposed
 *              Solution, first bullet), kept in fp64 and rounded once
 *              (Implementation Notes: f32 partials with a single final
 *              rounding).
 *
 * Every pin of this file lives in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------ conversions */

/* IEEE binary16 bit pattern -> exact double. */
double orc_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1F;
    int man = h & 0x3FF;
    double v;
    if (ex == 0) {
        v = ldexp((double)man, -24);
    } else if (ex == 31) {
        v = man ? NAN : INFINITY;
    } else {
        v = ldexp((double)(man + 1024), ex - 25);
    }
    return sign ? -v : v;
}

/* bfloat16 bit pattern -> exact double (bf16 is the top half of an fp32). */
double orc_bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bfloat16 (ties to even), in one step from
 * the double (no intermediate fp32, so no double rounding). */
uint16_t orc_f64_to_bf16(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);               /* a = m * 2^e with m in [0.5, 1) */
    /* bf16 keeps 8 significant bits; its smallest spacing is 2^-133. */
    int lsb_exp = e - 8;
    if (lsb_exp < -133) lsb_exp = -133;
    double r = nearbyint(ldexp(a, -lsb_exp));   /* integer multiple of the lsb, ties to even */
    double q = ldexp(r, lsb_exp);
    if (q >= ldexp(1.0, 128)) return sign | 0x7F80; /* overflow -> inf */
    float f = (float)q;                /* exact: q has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

/* ------------------------------------------------------------ dequantise */

/* One weight of an affine `bits`-bit matrix, w = scale * q + bias with q
 * unsigned.  A row of `cols` elements is a little-endian bit stream of
 * cols * bits / 32 words (bit j of the stream is bit j % 32 of word j / 32);
 * element c occupies stream bits c*bits .. c*bits + bits - 1, lowest first,
 * so 4-bit elements sit in nibble c % 8 of word c / 8 and a 6-bit element
 * may straddle two words.  Scale and bias (fp16) per `group` consecutive
 * elements of a row.  The pages template the fused kernel on bits and group
 * size and name 4-bit gate/up with 6-bit down, which needs Dff divisible by
 * 16 (page "perf(moe): batched decode scales 1.55x against 3.25x on
 * dense", Implementation Notes); they give no packing, and this bit stream
 * is the plainest one that makes 16 six-bit elements fill whole words. */
static double orc_weight(const uint32_t *q, const uint16_t *s, const uint16_t *b,
                         int cols, int bits, int group, int r, int c) {
    const uint32_t *row = q + (size_t)r * ((size_t)cols * bits / 32);
    uint32_t v = 0;
    for (int i = 0; i < bits; ++i) {
        size_t p = (size_t)c * bits + i;
        v |= ((row[p / 32] >> (p % 32)) & 1u) << i;
    }
    size_t g = (size_t)r * (cols / group) + c / group;
    return orc_f16_to_f64(s[g]) * (double)v + orc_f16_to_f64(b[g]);
}

/* Dense fp64 copy of one [rows][cols] quantised matrix (used by tests). */
void orc_dequant(const uint32_t *q, const uint16_t *s, const uint16_t *b,
                 int rows, int cols, int bits, int group, double *w) {
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < cols; ++c)
            w[(size_t)r * cols + c] = orc_weight(q, s, b, cols, bits, group, r, c);
}

/* ----------------------------------------------------------------- route */

/* logits [n_tokens][n_experts] fp32 -> idx [n_tokens][top_k], w [..] fp64.
 * Returns 0, or -1 on bad sizes. */
int orc_route_topk(const float *logits, int n_tokens, int n_experts, int top_k,
                   int32_t *idx, double *w) {
    if (n_tokens < 0 || n_experts < 1 || top_k < 1 || top_k > n_experts) return -1;
    char *taken = (char *)malloc((size_t)n_experts);
    if (!taken) return -1;
    for (int t = 0; t < n_tokens; ++t) {
        const float *l = logits + (size_t)t * n_experts;
        memset(taken, 0, (size_t)n_experts);
        /* selection: k rounds of "largest remaining, lowest id on ties" */
        for (int j = 0; j < top_k; ++j) {
            int best = -1;
            for (int e = 0; e < n_experts; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            idx[(size_t)t * top_k + j] = best;
        }
        /* weights: softmax restricted to the kept logits */
        double l0 = (double)l[idx[(size_t)t * top_k]];
        double den = 0.0;
        for (int j = 0; j < top_k; ++j)
            den += exp((double)l[idx[(size_t)t * top_k + j]] - l0);
        for (int j = 0; j < top_k; ++j)
            w[(size_t)t * top_k + j] = exp((double)l[idx[(size_t)t * top_k + j]] - l0) / den;
    }
    free(taken);
    return 0;
}

/* ------------------------------------------------------------------ plan */

/* Stable counting sort of the n_tokens*top_k slots by expert id.
 * counts[E], offsets[E+1], sorted_slots[n_slots], unique[E] (ascending,
 * padded with -1), n_unique[1].  Returns 0, or -1 on an id out of range. */
int orc_plan(const int32_t *idx, int n_tokens, int n_experts, int top_k,
             int32_t *counts, int32_t *offsets, int32_t *sorted_slots,
             int32_t *unique, int32_t *n_unique) {
    int n_slots = n_tokens * top_k;
    for (int e = 0; e < n_experts; ++e) counts[e] = 0;
    for (int s = 0; s < n_slots; ++s) {
        if (idx[s] < 0 || idx[s] >= n_experts) return -1;
        counts[idx[s]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < n_experts; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_experts > 0 ? n_experts : 1));
    if (!cursor) return -1;
    for (int e = 0; e < n_experts; ++e) cursor[e] = offsets[e];
    for (int s = 0; s < n_slots; ++s) sorted_slots[cursor[idx[s]]++] = s;
    free(cursor);
    int nu = 0;
    for (int e = 0; e < n_experts; ++e)
        if (counts[e] > 0) unique[nu++] = e;
    for (int e = nu; e < n_experts; ++e) unique[e] = -1;
    *n_unique = nu;
    return 0;
}

/* ---------------------------------------------------------------- expert */

typedef struct {
    int32_t hidden, dff, n_experts, top_k;
    int32_t x_is_bf16;          /* 1: x holds bf16 bit patterns, 0: fp32 */
    double clamp_limit;         /* <= 0: no clamp */
    const uint32_t *gate_q, *up_q, *down_q;
    const uint16_t *gate_s, *gate_b, *up_s, *up_b, *down_s, *down_b;
    const float *sidecar;       /* [E] or NULL */
    int32_t activation;         /* 0: SwiGLU, 1: GeGLU (tanh-form GELU) */
    const float *down_sidecar;  /* [E] or NULL: y *= down_sidecar[e] */
    int32_t bits;               /* width of gate and up elements */
    int32_t down_bits;          /* width of down elements */
    int32_t group_size;         /* elements per scale/bias group, all three */
} orc_layer;

static double orc_x(const orc_layer *L, const void *x, int t, int c) {
    size_t i = (size_t)t * L->hidden + c;
    if (L->x_is_bf16) return orc_bf16_to_f64(((const uint16_t *)x)[i]);
    return (double)((const float *)x)[i];
}

static double orc_clip(double v, double lim) {
    if (v > lim) return lim;
    if (v < -lim) return -lim;
    return v;
}

/* GELU in the tanh form, 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))):
 * the GeGLU variant the pages list as a next family (page "perf(moe):
 * batched decode scales 1.55x against 3.25x on dense", Implementation
 * Notes) gives no formula; this is the form of the gemma checkpoints it
 * names. */
static double orc_gelu(double g) {
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * g * (1.0 + tanh(c * (g + 0.044715 * g * g * g)));
}

/* Intermediate h (length dff) of expert e for token t: SiLU(g) * u (or
 * GELU(g) * u) after the optional sidecar (first) and clamp (second). */
static void orc_expert_h(const orc_layer *L, const void *x, int t, int e, double *h) {
    const int H = L->hidden, F = L->dff, nb = L->bits, G = L->group_size;
    const size_t gq = (size_t)e * F * ((size_t)H * nb / 32), gs = (size_t)e * F * (H / G);
    for (int n = 0; n < F; ++n) {
        double g = 0.0, u = 0.0;
        for (int c = 0; c < H; ++c) {
            double xv = orc_x(L, x, t, c);
            g += orc_weight(L->gate_q + gq, L->gate_s + gs, L->gate_b + gs, H, nb, G, n, c) * xv;
            u += orc_weight(L->up_q + gq, L->up_s + gs, L->up_b + gs, H, nb, G, n, c) * xv;
        }
        if (L->sidecar) {
            double sc = (double)L->sidecar[e];
            g *= sc;
            u *= sc;
        }
        if (L->clamp_limit > 0.0) {
            g = orc_clip(g, L->clamp_limit);
            u = orc_clip(u, L->clamp_limit);
        }
        h[n] = (L->activation == 1 ? orc_gelu(g) : g / (1.0 + exp(-g))) * u;
    }
}

/* y (length hidden) = Wd[e] h. */
static void orc_expert_down(const orc_layer *L, int e, const double *h, double *y) {
    const int H = L->hidden, F = L->dff, nb = L->down_bits, G = L->group_size;
    const size_t dq = (size_t)e * H * ((size_t)F * nb / 32), ds = (size_t)e * H * (F / G);
    for (int m = 0; m < H; ++m) {
        double acc = 0.0;
        for (int n = 0; n < F; ++n)
            acc += orc_weight(L->down_q + dq, L->down_s + ds, L->down_b + ds, F, nb, G, m, n) * h[n];
        y[m] = L->down_sidecar ? acc * (double)L->down_sidecar[e] : acc;
    }
}

/* One decode step of the expert block.
 *   x    [n_tokens][hidden] (bf16 bits or fp32)
 *   idx  [n_tokens][top_k]  expert ids, w [n_tokens][top_k] fp64 weights
 *   out  [n_tokens][hidden] fp64, unrounded
 *   h_out (optional) [n_tokens*top_k][dff] fp64, the per-slot intermediate
 *   y_out (optional) [n_tokens*top_k][hidden] fp64, per-slot expert output
 * Slots run in parallel (OpenMP); each slot's arithmetic is sequential. */
int orc_decode_step(const orc_layer *L, const void *x, int n_tokens,
                    const int32_t *idx, const double *w, double *out,
                    double *h_out, double *y_out) {
    const int H = L->hidden, F = L->dff, k = L->top_k;
    const int G = L->group_size;
    if (n_tokens < 0 || k < 1 || G < 1 || H % G || F % G) return -1;
    if (L->bits < 1 || L->bits > 16 || L->down_bits < 1 || L->down_bits > 16) return -1;
    if ((H * L->bits) % 32 || (F * L->down_bits) % 32) return -1;
    const int n_slots = n_tokens * k;
    for (int s = 0; s < n_slots; ++s)
        if (idx[s] < 0 || idx[s] >= L->n_experts) return -1;
    double *hbuf = (double *)malloc(sizeof(double) * (size_t)(n_slots ? n_slots : 1) * F);
    double *ybuf = (double *)malloc(sizeof(double) * (size_t)(n_slots ? n_slots : 1) * H);
    if (!hbuf || !ybuf) {
        free(hbuf);
        free(ybuf);
        return -1;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int s = 0; s < n_slots; ++s) {
        int t = s / k;
        orc_expert_h(L, x, t, idx[s], hbuf + (size_t)s * F);
        orc_expert_down(L, idx[s], hbuf + (size_t)s * F, ybuf + (size_t)s * H);
    }
    for (int t = 0; t < n_tokens; ++t)
        for (int m = 0; m < H; ++m) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j)
                acc += w[(size_t)t * k + j] * ybuf[((size_t)t * k + j) * H + m];
            out[(size_t)t * H + m] = acc;
        }
    if (h_out) memcpy(h_out, hbuf, sizeof(double) * (size_t)n_slots * F);
    if (y_out) memcpy(y_out, ybuf, sizeof(double) * (size_t)n_slots * H);
    free(hbuf);
    free(ybuf);
    return 0;
}

/* Elementwise rounding helpers for the I/O dtypes. */
void orc_round_bf16(const double *v, size_t n, uint16_t *out) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_f64_to_bf16(v[i]);
}

void orc_round_f32(const double *v, size_t n, float *out) {
    for (size_t i = 0; i < n; ++i) out[i] = (float)v[i];
}

/* Residual step of the layer stack: x' = bf16(f32(x) + f32(bf16(out))).
 * x and x_next are bf16 bit patterns; out is the unrounded fp64 layer output. */
void orc_residual_bf16(const uint16_t *x, const double *out, size_t n, uint16_t *x_next) {
    for (size_t i = 0; i < n; ++i) {
        float a = (float)orc_bf16_to_f64(x[i]);
        float o = (float)orc_bf16_to_f64(orc_f64_to_bf16(out[i]));
        float sum = a + o;                 /* one fp32 addition, RNE */
        x_next[i] = orc_f64_to_bf16((double)sum);
    }
}

/* Router projection, the step in front of the router: logits[t][e] =
 * sum_h x[t][h] * Wr[e][h], with Wr a dense bf16 matrix [n_experts][hidden]
 * (one row per expert) and x bf16 or fp32 as in the expert block.  Products
 * and the sum in fp64 (exact products; the sum in h order).  The pages
 * name the router as one of the per-token decode costs (page "perf(moe):
 * attribute the MoE decode gap at the M = 1 expert gather", Proposed
 * Solution step 2) without its form; a dense linear map of the token's
 * hidden state to one logit per expert is the plain reading. */
int orc_router_logits(const void *x, int x_is_bf16, int n_tokens, int hidden, int n_experts,
                      const uint16_t *w_router, double *logits) {
    if (n_tokens < 0 || hidden <= 0 || n_experts <= 0) return 1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < n_tokens; ++t)
        for (int e = 0; e < n_experts; ++e) {
            double acc = 0.0;
            for (int c = 0; c < hidden; ++c) {
                const double xv = x_is_bf16 ? orc_bf16_to_f64(((const uint16_t *)x)[(size_t)t * hidden + c])
                                            : (double)((const float *)x)[(size_t)t * hidden + c];
                acc += xv * orc_bf16_to_f64(w_router[(size_t)e * hidden + c]);
            }
            logits[(size_t)t * n_experts + e] = acc;
        }
    return 0;
}
