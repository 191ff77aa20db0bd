// Tile kernels (gfx950) for batches with many tokens per expert: the
// prefill-sized end of the token dimension, where each distinct expert of
// the plan holds tens of tokens.  Page "perf(moe): batched decode scales
// 1.55x against 3.25x on dense" gives the expert block a token dimension
// that is a runtime extent and deduplicates experts across it (Proposed
// Solution); with 256 to 1024 tokens and top-8 of 128 experts every
// expert holds about B * 8 / 128 of them, and the block is a set of small
// GEMMs, one per distinct expert, on MFMA.
//
// Work is cut into tile items: (distinct expert u, block of up to 64 of
// its tokens), items in the plan's order of distinct experts, ceil(count /
// 64) of them per expert.  The items of one expert read its weights again,
// so the weights go through the caches with ordinary loads here (the
// streaming hint of the few-token kernels measured ~9 % slower).  A workgroup takes one item and one block of
// output rows; its eight waves split the rows, 16 * RT each, and each wave
// holds all 64 tokens (four 16-token tiles) of the item in its
// accumulators while it walks the whole input dimension, 64-group by
// 64-group.  The item's activations for a group are staged once in LDS for
// all the waves, already in MFMA operand form with their group sums (read
// and converted by every wave, the activations rather than the weights
// would bound the kernels); no partial sums cross waves.
//
// MFMA operands (v_mfma_f32_16x16x32_bf16, D = A B): A is 16 tokens by 32
// inputs, B is 32 inputs by 16 weight rows, so the output lane (token
// 4 kq + i, row r) holds one row of four tokens and the per-(row, group)
// scale and bias it needs are the lane's own B row's.  The weights go in
// as exact bf16 values 1 + q / 16; the activations as bf16 (gate+up) or
// as the three exact bf16 parts of fp32 h (down), so every product is
// exact and only fp32 additions round, as in the other kernels.
#include <hip/hip_runtime.h>
#include <limits.h>

#include <mutex>

#include "device_util.h"
#include "expert_device.h"
#include "gate_up_device.h"
#include "mfma_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kTileWaves = 8;                      // waves per workgroup; they split the rows
constexpr int kTileThreads = kTileWaves * kWave;
constexpr int kStageUnits = 64 * 8 / kTileThreads;   // (token, eighth of a group) units each thread stages
static_assert(kStageUnits * kTileThreads == 64 * 8, "the staging covers 64 tokens x 8 parts");
constexpr int kTileTokenTiles = 4;                 // 16-token tiles per item
constexpr int kTileTokens = 16 * kTileTokenTiles;  // tokens per item
constexpr int kTileGateUpRowTiles = 1;             // 16-row tiles per wave, gate+up
constexpr int kTileDownRowTiles = 2;               // 16-row tiles per wave, down
constexpr int kXcds = 8;                           // XCDs of the device; workgroups go round robin

// The workgroup's (tile item, row block).  Workgroup ids are dealt to the
// XCDs round robin, so the row blocks of one item are numbered to land on
// one XCD and read its activations through one L2.
struct TileIndex {
    int item, rb;
};
__device__ __forceinline__ TileIndex tile_index(int row_blocks) {
    const int L = blockIdx.x, x = L % kXcds, j = L / kXcds;
    return TileIndex{(j / row_blocks) * kXcds + x, j - (j / row_blocks) * row_blocks};
}

// Tile item `item` -> its distinct expert's work record and token block,
// or false past the last item.  Every wave runs this by itself: each lane
// counts the blocks of a contiguous run of records, a wave scan places the
// runs, and the lane whose run holds the item finds it.  Records past the
// last distinct expert are the plan's end records and count no blocks.
__device__ __forceinline__ bool tile_item(const PlanView &p, int item, int n_records, int n_experts, int n_slots,
                                          Work *w, int *tb) {
    const int lane = threadIdx.x & (kWave - 1);
    const int per = (n_records + kWave - 1) / kWave;
    const int u0 = lane * per;
    int mine = 0;
    for (int q = 0; q < per; ++q) {
        Work wk;
        if (u0 + q < n_records && plan_expert(p, u0 + q, n_experts, n_slots, &wk))
            mine += (wk.count + kTileTokens - 1) / kTileTokens;
    }
    int incl = mine;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int v = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += v;
    }
    const int excl = incl - mine;
    const unsigned long long hit = __ballot(item >= excl && item < incl);
    if (!hit) return false;
    const int src = __ffsll(hit) - 1;
    int fu = -1, fb = 0;
    if (lane == src) {
        int at = excl;
        for (int q = 0; q < per; ++q) {
            Work wk;
            if (u0 + q < n_records && plan_expert(p, u0 + q, n_experts, n_slots, &wk)) {
                const int nb = (wk.count + kTileTokens - 1) / kTileTokens;
                if (item < at + nb) {
                    fu = u0 + q;
                    fb = item - at;
                    break;
                }
                at += nb;
            }
        }
    }
    fu = __shfl(fu, src, kWave);
    fb = __shfl(fb, src, kWave);
    if (fu < 0 || !plan_expert(p, fu, n_experts, n_slots, w)) return false;
    *tb = fb;
    return true;
}

// ----------------------------------------------------------------- gate+up

// Staged operands of one 64-group, in LDS: the workgroup turns each
// token's inputs into MFMA A operands once (bf16 pairs of x; the three bf16
// parts of fp32 h) and sums them once, and every wave reads them ready:
//   x  [j][token][kq] 16 bytes: inputs 16 kq + 8 j .. + 7, as pairs
//   h  [c][part][token][kq] 16 bytes: inputs 32 c + 8 kq .. + 7, one part
//   sums [token] fp32, the token's group sum
// so a wave's read of one operand for a 16-token tile is 1 KiB in a row.
constexpr int kXStageBytes = 2 * 64 * 64 + 64 * 4;      // per buffer
constexpr int kHStageBytes = 2 * 3 * 64 * 64 + 64 * 4;  // per buffer
constexpr int kTileRing = 4;             // 64-groups of loads in flight per thread

// A compile-time slot number: the ring's registers are indexed only with
// these, so every index is a constant before the arrays are laid out.
template <int N>
struct Slot {
    static constexpr int value = N;
};

// h[slot][row] = act(g, u) for the item's tokens and the workgroup's rows.
// Wave w owns rows row_b + 16 RT w .. + 16 RT - 1.  Per 64-group the
// workgroup stages the item's activations in LDS (thread i converts 16
// bytes of token i / 8), and lane (r16, kq) of every wave reads inputs
// 16 kq .. 16 kq + 15 of its four tokens from there (A operands) and holds
// words 2 kq, 2 kq + 1 of the group for each of its rows (B operands of two
// MFMAs).  The loop runs in passes of four groups, the next pass's loads in
// flight during the current one.
template <int RT>
__global__ __launch_bounds__(kTileThreads) void gate_up_tile_kernel(GateUpArgs a, int n_records, int row_blocks) {
    constexpr int TT = kTileTokenTiles;
    constexpr int ROWS = kTileWaves * 16 * RT;
    extern __shared__ __align__(16) unsigned char lds[];
    const TileIndex ti = tile_index(row_blocks);
    Work wk;
    int tb;
    if (!tile_item(a.plan, ti.item, n_records, a.n_experts, a.n_slots, &wk, &tb)) return;
    const int H = a.hidden, F = a.dff, G = H / kGroup;
    uint32_t *sbl = (uint32_t *)lds;                          // [2][G][ROWS] (scale | bias << 16)
    unsigned char *xl = lds + (size_t)2 * G * ROWS * 4;       // [2 buffers][kXStageBytes]
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int r16 = lane & 15, kq = lane >> 4;
    const int t0 = tb * kTileTokens;
    const int nt = wk.count - t0 < kTileTokens ? wk.count - t0 : kTileTokens;
    const int ntt = (nt + 15) >> 4;  // live token tiles (wave-uniform)
    const int row_b = ti.rb * ROWS;
    const int row_w = row_b + wave * 16 * RT;

    // this thread's share of the activation tile: 16 bytes of tokens
    // tid / 8 + 64 u / kStageUnits (tokens past the item read the first
    // token's row; their rows of D are never stored)
    constexpr int U = kStageUnits;
    const int xp = tid & 7;
    const uint4 *xsrc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int xt = (tid >> 3) + u * (kTileThreads / 8);
        const int xslot = plan_slot(a.plan, wk, t0 + (xt < nt ? xt : 0), a.n_slots);
        xsrc[u] = (const uint4 *)((const uint16_t *)a.x + (size_t)(xslot / a.top_k) * H) + xp;
    }
    const uint2 *gq = (const uint2 *)a.gate_q, *uq = (const uint2 *)a.up_q;
    size_t woff[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int row = row_w + 16 * rt + r16;
        woff[rt] = ((size_t)wk.e * F + (row < F ? row : F - 1)) * (H / 16) + kq;
    }
    // Two register sets, each holding one pass of four 64-groups: the
    // current pass and the loads of the next.  A pass reads each of its
    // rows' 128 bytes (four groups, one cache line) with four loads issued
    // back to back, so every line is used whole while it is in L2.
    uint2 wq[2][RT][2][4];
    uint4 xq[2][4][U];
    auto load_pass = [&](auto set, int k) __attribute__((always_inline)) {
        constexpr int S = decltype(set)::value;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                wq[S][rt][0][j] = gq[woff[rt] + 4 * (4 * k + j)];
                wq[S][rt][1][j] = uq[woff[rt] + 4 * (4 * k + j)];
            }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int u = 0; u < U; ++u) xq[S][j][u] = xsrc[u][8 * (4 * k + j)];
    };
    // thread (token xt, part xp) holds inputs 8 xp .. 8 xp + 7 of the group:
    // MFMA j = xp & 1 of lane kq = xp >> 1; the eight parts of a token sit
    // in eight neighbouring lanes, which add their sums
    auto stage_x = [&](int buf, const uint4 (&v)[U]) __attribute__((always_inline)) {
        unsigned char *b = xl + (size_t)buf * kXStageBytes;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int xt = (tid >> 3) + u * (kTileThreads / 8);
            uint32_t o[4];
            float sum = 0.f;
            x8_pairs(v[u], o, &sum);
            sum = seg_sum<8>(sum);  // DPP within the token's eight lanes
            *(uint4 *)(b + (((xp & 1) * 64 + xt) * 4 + (xp >> 1)) * 16) = make_uint4(o[0], o[1], o[2], o[3]);
            if (xp == 0) *(float *)(b + 2 * 64 * 64 + 4 * xt) = sum;
        }
    };
    const int K = G / 4;  // passes
    load_pass(Slot<0>{}, 0);
    // the workgroup's gate/up scales and biases (its wait covers the first pass)
    for (int i = tid; i < ROWS * G; i += kTileThreads) {
        const int r = i / G, g = i - r * G;
        const int row = row_b + r < F ? row_b + r : F - 1;
        const size_t si = ((size_t)wk.e * F + row) * G + g;
        sbl[g * ROWS + r] = a.gate_s[si] | (uint32_t)a.gate_b[si] << 16;
        sbl[(G + g) * ROWS + r] = a.up_s[si] | (uint32_t)a.up_b[si] << 16;
    }
    stage_x(0, xq[0][0]);
    __syncthreads();

    f32x4_t acc[RT][TT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[rt][tt][0] = acc[rt][tt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // one pass: the next pass's loads go out first (past the last pass they
    // repeat it), then the four groups, each staging the next group's
    // activations into the other LDS buffer before its MFMAs
    // The MFMAs of one group for NT token tiles: every LDS read first, then
    // the MFMA chains (one copy per tile count, no branch between them).
    auto tiles = [&](auto ntiles, const unsigned char *xg, const uint32_t (&b)[RT][2][2][4],
                     const float (&s16)[RT][2], const float (&bp)[RT][2]) __attribute__((always_inline)) {
        constexpr int NT = decltype(ntiles)::value;
        uint4 A0[NT], A1[NT];
        float4 S4[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int tok = 16 * tt + r16;
            A0[tt] = *(const uint4 *)(xg + ((0 * 64 + tok) * 4 + kq) * 16);
            A1[tt] = *(const uint4 *)(xg + ((1 * 64 + tok) * 4 + kq) * 16);
            // the group sums of the D rows' tokens 16 tt + 4 kq .. + 3
            S4[tt] = *(const float4 *)(xg + 2 * 64 * 64 + 4 * (16 * tt + 4 * kq));
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const uint32_t xa[2][4] = {{A0[tt].x, A0[tt].y, A0[tt].z, A0[tt].w}, {A1[tt].x, A1[tt].y, A1[tt].z, A1[tt].w}};
            const float xs[4] = {S4[tt].x, S4[tt].y, S4[tt].z, S4[tt].w};
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    f32x4_t d = mfma16x16x32(xa[0], b[rt][m][0], f32x4_t{0.f, 0.f, 0.f, 0.f});
                    d = mfma16x16x32(xa[1], b[rt][m][1], d);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[rt][tt][m][i] = fmaf(bp[rt][m], xs[i], fmaf(s16[rt][m], d[i], acc[rt][tt][m][i]));
                }
        }
    };
    auto pass = [&](auto set, int k) __attribute__((always_inline)) {
        constexpr int S = decltype(set)::value;
        load_pass(Slot<1 - S>{}, k + 1 < K ? k + 1 : K - 1);
        // the pass's scales and biases, all four groups' at once
        uint32_t sbp[4][RT][2];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    sbp[j][rt][m] = sbl[(m * G + 4 * k + j) * ROWS + (row_w - row_b) + 16 * rt + r16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int g = 4 * k + j;
            stage_x((g + 1) & 1, j < 3 ? xq[S][j + 1 < 4 ? j + 1 : 3] : xq[1 - S][0]);
            uint32_t b[RT][2][2][4];
            float s16[RT][2], bp[RT][2];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    q4_pairs16(wq[S][rt][m][j].x, b[rt][m][0]);
                    q4_pairs16(wq[S][rt][m][j].y, b[rt][m][1]);
                    const uint32_t sb = sbp[j][rt][m];
                    const float sv = f16_bits_to_f32((uint16_t)(sb & 0xFFFFu));
                    s16[rt][m] = 16.f * sv;
                    bp[rt][m] = fmaf(-16.f, sv, f16_bits_to_f32((uint16_t)(sb >> 16)));
                }
            const unsigned char *xg = xl + (size_t)(g & 1) * kXStageBytes;
            // tiles past the live tokens hold the first token's activations;
            // their rows of D are never stored
            if (ntt >= 3)
                tiles(Slot<4>{}, xg, b, s16, bp);
            else if (ntt == 2)
                tiles(Slot<2>{}, xg, b, s16, bp);
            else
                tiles(Slot<1>{}, xg, b, s16, bp);
            __syncthreads();
        }
    };
    for (int k = 0; k < K; k += 2) {
        pass(Slot<0>{}, k);
        if (k + 1 < K) pass(Slot<1>{}, k + 1);
    }

    const float esc = a.expert_scale ? a.expert_scale[wk.e] : 1.f;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        if (tt >= ntt) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tk = tt * 16 + 4 * kq + i;
            if (tk >= nt) continue;
            const int slot = plan_slot(a.plan, wk, t0 + tk, a.n_slots);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int row = row_w + 16 * rt + r16;
                if (row < F)
                    a.h[(size_t)slot * F + row] =
                        act_mul(acc[rt][tt][0][i], acc[rt][tt][1][i], esc, a.clamp_limit, a.activation);
            }
        }
    }
}

// -------------------------------------------------------------------- down

// y[slot][row] = Wd[e][row] . h[slot] for the item's tokens and the
// workgroup's rows of hidden; column layout of the down projection (chunk
// c of row m holds inputs 32 c .. 32 c + 31, word kq inputs 32 c + 8 kq ..
// + 7).  Per 64-group (two chunks) the workgroup stages the item's h in
// LDS (thread i splits 32 bytes of token i / 8 into their three bf16
// parts); lane (r16, kq) reads inputs 32 c + 8 kq .. + 7 of its four
// tokens from there (A operands) and holds word kq of both chunks for each
// of its rows (B operands).  Each thread keeps the loads of the next
// kTileRing groups in flight (a ring of registers, slot = group %
// kTileRing; the loop is unrolled by the ring's length so every slot index
// is static).
template <int RT>
__global__ __launch_bounds__(kTileThreads) void down_tile_kernel(const uint32_t *__restrict__ q,
                                                                 const uint16_t *__restrict__ sc,
                                                                 const uint16_t *__restrict__ bi,
                                                                 const float *__restrict__ h, float *__restrict__ y,
                                                                 PlanView plan, int hidden, int dff, int n_experts,
                                                                 int n_slots, int n_records, int row_blocks) {
    constexpr int TT = kTileTokenTiles;
    constexpr int ROWS = kTileWaves * 16 * RT;
    constexpr int NR = kTileRing;
    extern __shared__ __align__(16) unsigned char lds[];
    const TileIndex ti = tile_index(row_blocks);
    Work wk;
    int tb;
    if (!tile_item(plan, ti.item, n_records, n_experts, n_slots, &wk, &tb)) return;
    const int H = hidden, F = dff, G = F / kGroup, C = F / 32;
    uint32_t *sbl = (uint32_t *)lds;                        // [G][ROWS] (scale | bias << 16)
    unsigned char *hl = lds + (size_t)G * ROWS * 4;         // [2 buffers][kHStageBytes]
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int r16 = lane & 15, kq = lane >> 4;
    const int t0 = tb * kTileTokens;
    const int nt = wk.count - t0 < kTileTokens ? wk.count - t0 : kTileTokens;
    const int ntt = (nt + 15) >> 4;
    const int row_b = ti.rb * ROWS;
    const int row_w = row_b + wave * 16 * RT;

    // this thread's share of the h tile: 32 bytes of tokens tid / 8 +
    // 64 u / kStageUnits
    constexpr int U = kStageUnits;
    const int hp = tid & 7;
    const float4 *hsrc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int ht = (tid >> 3) + u * (kTileThreads / 8);
        const int hslot = plan_slot(plan, wk, t0 + (ht < nt ? ht : 0), n_slots);
        hsrc[u] = (const float4 *)(h + (size_t)hslot * F) + 2 * hp;
    }
    size_t wbase[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int m = row_w + 16 * rt + r16;
        wbase[rt] = ((size_t)wk.e * C * H + (m < H ? m : H - 1)) * 4 + kq;
    }
    float4 hr[NR][U][2];
    uint32_t wr[NR][RT][2];
    auto load = [&](auto slot, int g) __attribute__((always_inline)) {
        constexpr int s = decltype(slot)::value;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2)
                wr[s][rt][c2] = q[wbase[rt] + (size_t)(2 * g + c2) * H * 4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            hr[s][u][0] = hsrc[u][16 * g];
            hr[s][u][1] = hsrc[u][16 * g + 1];
        }
    };
    // thread (token ht, part hp) holds inputs 8 hp .. 8 hp + 7 of the group:
    // chunk hp >> 2, lane kq = hp & 3; it writes their three bf16 parts
    auto stage_h = [&](int buf, const float4 (&hv)[U][2]) __attribute__((always_inline)) {
        unsigned char *b = hl + (size_t)buf * kHStageBytes;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ht = (tid >> 3) + u * (kTileThreads / 8);
            const float4 v0 = hv[u][0], v1 = hv[u][1];
            const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            uint32_t o[3][4];
            split3_pairs(v, o);
            float sum = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
            sum = seg_sum<8>(sum);  // DPP within the token's eight lanes
#pragma unroll
            for (int p = 0; p < 3; ++p)
                *(uint4 *)(b + ((((hp >> 2) * 3 + p) * 64 + ht) * 4 + (hp & 3)) * 16) =
                    make_uint4(o[p][0], o[p][1], o[p][2], o[p][3]);
            if (hp == 0) *(float *)(b + 2 * 3 * 64 * 64 + 4 * ht) = sum;
        }
    };
    load(Slot<0>{}, 0);
    load(Slot<1>{}, 1);
    load(Slot<2>{}, 2);
    load(Slot<3>{}, 3);
    for (int i = tid; i < ROWS * G; i += kTileThreads) {
        const int g = i / ROWS, r = i - g * ROWS;
        const int m = row_b + r < H ? row_b + r : H - 1;
        const size_t si = ((size_t)wk.e * G + g) * H + m;
        sbl[g * ROWS + r] = sc[si] | (uint32_t)bi[si] << 16;
    }
    stage_h(0, hr[0]);
    __syncthreads();

    f32x4_t acc[RT][TT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[rt][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // The MFMAs of one group for NT token tiles: every LDS read first, then
    // the MFMA chains (one copy per tile count, no branch between them).
    auto tiles = [&](auto ntiles, const unsigned char *hg, const uint32_t (&b)[RT][2][4], const float (&s16)[RT],
                     const float (&bp)[RT]) __attribute__((always_inline)) {
        constexpr int NT = decltype(ntiles)::value;
        uint4 A[NT][2][3];
        float4 S4[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int tok = 16 * tt + r16;
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                for (int p = 0; p < 3; ++p) A[tt][c2][p] = *(const uint4 *)(hg + (((c2 * 3 + p) * 64 + tok) * 4 + kq) * 16);
            S4[tt] = *(const float4 *)(hg + 2 * 3 * 64 * 64 + 4 * (16 * tt + 4 * kq));
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const float hs[4] = {S4[tt].x, S4[tt].y, S4[tt].z, S4[tt].w};
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                f32x4_t d = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                    for (int p = 0; p < 3; ++p) {
                        const uint32_t ha[4] = {A[tt][c2][p].x, A[tt][c2][p].y, A[tt][c2][p].z, A[tt][c2][p].w};
                        d = mfma16x16x32(ha, b[rt][c2], d);
                    }
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[rt][tt][i] = fmaf(bp[rt], hs[i], fmaf(s16[rt], d[i], acc[rt][tt][i]));
            }
        }
    };
    auto step = [&](auto slot, int g) __attribute__((always_inline)) {
        constexpr int s = decltype(slot)::value;
        stage_h((g + 1) & 1, hr[(s + 1) % NR]);
        uint32_t b[RT][2][4];
        float s16[RT], bp[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            q4_pairs16(wr[s][rt][0], b[rt][0]);
            q4_pairs16(wr[s][rt][1], b[rt][1]);
            const uint32_t sb = sbl[g * ROWS + (row_w - row_b) + 16 * rt + r16];
            const float sv = f16_bits_to_f32((uint16_t)(sb & 0xFFFFu));
            s16[rt] = 16.f * sv;
            bp[rt] = fmaf(-16.f, sv, f16_bits_to_f32((uint16_t)(sb >> 16)));
        }
        load(slot, g + NR < G ? g + NR : G - 1);
        const unsigned char *hg = hl + (size_t)(g & 1) * kHStageBytes;
        // tiles past the live tokens hold the first token's h; their rows
        // of D are never stored
        if (ntt >= 3)
            tiles(Slot<4>{}, hg, b, s16, bp);
        else if (ntt == 2)
            tiles(Slot<2>{}, hg, b, s16, bp);
        else
            tiles(Slot<1>{}, hg, b, s16, bp);
        __syncthreads();
    };
    for (int g4 = 0; g4 < G; g4 += NR) {
        step(Slot<0>{}, g4);
        step(Slot<1>{}, g4 + 1);
        step(Slot<2>{}, g4 + 2);
        step(Slot<3>{}, g4 + 3);
    }

#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        if (tt >= ntt) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tk = tt * 16 + 4 * kq + i;
            if (tk >= nt) continue;
            const int slot = plan_slot(plan, wk, t0 + tk, n_slots);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int m = row_w + 16 * rt + r16;
                if (m < H) y[(size_t)slot * H + m] = acc[rt][tt][i];
            }
        }
    }
}

// -------------------------------------------------------------- host side

// Tile items of a batch: at most one per distinct expert plus one per 64
// slots (sum over experts of ceil(count / 64) <= n_unique + n_slots / 64).
static int tile_items_max(const moe_layer_t *L, int n_tokens, int *n_records) {
    const int n_slots = n_tokens * L->top_k;
    *n_records = n_slots < L->n_experts ? n_slots : L->n_experts;
    return *n_records + (n_slots + kTileTokens - 1) / kTileTokens;
}

static int tile_grid(int items, int row_blocks) {
    return kXcds * row_blocks * ((items + kXcds - 1) / kXcds);
}

static size_t tile_lds_budget() {
    static std::mutex mu;
    static size_t budget[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 65536;
    std::lock_guard<std::mutex> lock(mu);
    if (!budget[dev]) {
        int v = 0;
        budget[dev] = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0
                          ? (size_t)v
                          : 65536;
    }
    return budget[dev];
}

// LDS of a workgroup: the scales and biases of its rows, and two buffers of
// the item's activations for one 64-group.
static size_t gate_up_tile_lds(const moe_layer_t *L) {
    const size_t rows = kTileWaves * 16 * kTileGateUpRowTiles;
    return (size_t)2 * (L->hidden / kGroup) * rows * sizeof(uint32_t) + (size_t)2 * kXStageBytes;
}

static size_t down_tile_lds(const moe_layer_t *L) {
    const size_t rows = kTileWaves * 16 * kTileDownRowTiles;
    return (size_t)(L->dff / kGroup) * rows * sizeof(uint32_t) + (size_t)2 * kHStageBytes;
}

// The loop over the input dimension is unrolled by the load ring's length,
// so the 64-groups must come in whole rings.
bool tile_gate_up_ok(const moe_layer_t *L) {
    return fast_gate_up(L) && L->act_dtype == MOE_DTYPE_BF16 && L->hidden % (kGroup * kTileRing) == 0 &&
           gate_up_tile_lds(L) <= tile_lds_budget();
}

bool tile_down_ok(const moe_layer_t *L) {
    return fast_down(L) && L->down_layout == MOE_DOWN_COLS && L->dff % (kGroup * kTileRing) == 0 &&
           down_tile_lds(L) <= tile_lds_budget();
}

moe_status launch_gate_up_tile(const moe_layer_t *L, const void *x, int n_tokens, const moe_plan_t *plan, float *h,
                               hipStream_t s) {
    constexpr int RT = kTileGateUpRowTiles;
    int n_records = 0;
    const int items = tile_items_max(L, n_tokens, &n_records);
    const int row_blocks = (L->dff + kTileWaves * 16 * RT - 1) / (kTileWaves * 16 * RT);
    const GateUpArgs ga{(const uint4 *)L->gate_q, (const uint4 *)L->up_q, L->gate_s, L->gate_b, L->up_s, L->up_b,
                        L->expert_scale, L->clamp_limit, x, plan_view(plan), h, L->hidden, L->dff,
                        L->n_experts, L->top_k, n_tokens * L->top_k, INT_MAX, L->activation};
    hipLaunchKernelGGL(gate_up_tile_kernel<RT>, dim3(tile_grid(items, row_blocks)), dim3(kTileThreads),
                       gate_up_tile_lds(L), s, ga, n_records, row_blocks);
    return MOE_OK;
}

moe_status launch_down_tile(const moe_layer_t *L, int n_tokens, const moe_plan_t *plan, const float *h, float *y,
                            hipStream_t s) {
    constexpr int RT = kTileDownRowTiles;
    int n_records = 0;
    const int items = tile_items_max(L, n_tokens, &n_records);
    const int row_blocks = (L->hidden + kTileWaves * 16 * RT - 1) / (kTileWaves * 16 * RT);
    hipLaunchKernelGGL(down_tile_kernel<RT>, dim3(tile_grid(items, row_blocks)), dim3(kTileThreads), down_tile_lds(L), s,
                       L->down_q, L->down_s, L->down_b, h, y, plan_view(plan), L->hidden, L->dff, L->n_experts,
                       n_tokens * L->top_k, n_records, row_blocks);
    return MOE_OK;
}

}  // namespace moe
