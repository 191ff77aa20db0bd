"""GPU parity of the HIP path against the oracle, through the C ABI.

Indices and the dedup plan bit-exact; router weights within 1e-6; outputs
within relative L2 2e-3 of the fp64 oracle (plus the tighter diagnostic
against the once-rounded oracle, see gpu_helpers).  Every workload shape at
its full size, the routing regimes, and the edge cases.
"""

import numpy as np
import pytest
import torch

import quantized_expert_gemv_moe_amd as moe
from gpu_helpers import (REL_L2_DIAG, REL_L2_GATE, DeviceRun, check_against_oracle, dev_x, host_bits, layer_for,
                         log, record, rel_l2)
from moe_workloads import SHAPES, Shape, make_layer, make_logits, make_router, make_x
from oracle import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    moe.lib()
    yield


# ------------------------------------------------------------------ router
ROUTER_CASES = [
    ("toy", 1, "normal"), ("decode", 1, "normal"), ("cohort", 4, "sharing"), ("cohort", 8, "sharing"),
    ("wide", 1, "normal"), ("wide", 4, "normal"), ("stack", 32, "zipf"), ("decode", 1000, "normal"),
]


@pytest.mark.parametrize("name,B,regime", ROUTER_CASES)
def test_router_matches_oracle(name, B, regime):
    sh = SHAPES[name]
    lg = make_logits(sh, B, regime=regime, seed=21)
    idx, w = moe.route_topk(torch.from_numpy(lg).cuda(), sh.top_k)
    ridx, rw = oracle.route_topk(lg, sh.top_k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(w.cpu().numpy() - rw).max() <= 1e-6
    assert np.allclose(w.sum(dim=1).cpu().numpy(), 1.0, atol=1e-6)


@pytest.mark.parametrize("E,k", [(8, 1), (8, 8), (64, 16), (1024, 16), (1024, 1), (100, 7), (1, 1)])
def test_router_shapes_and_ties(E, k):
    sh = Shape("r", 30, 64, 64, E, k, "f32")
    lg = make_logits(sh, 37, seed=E + k)
    lg[0] = 0.0                      # all tied: ids ascending
    lg[1, ::3] = 1.0                 # partial ties
    lg[2] = -lg[2]
    lg[3] = 0.0
    lg[3, ::2] = -0.0                # -0 and +0 tie: ids ascending
    idx, w = moe.route_topk(torch.from_numpy(lg).cuda(), k)
    ridx, rw = oracle.route_topk(lg, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(w.cpu().numpy() - rw).max() <= 1e-6
    assert idx.cpu().numpy()[0].tolist() == list(range(k))
    assert idx.cpu().numpy()[3].tolist() == list(range(k))
    if k == 1:
        assert np.all(w.cpu().numpy() == 1.0)


def test_router_empty_batch_is_a_no_op():
    idx = torch.full((0, 8), -5, dtype=torch.int32, device="cuda")
    w = torch.zeros((0, 8), dtype=torch.float32, device="cuda")
    moe.route_topk(torch.zeros((0, 128), device="cuda"), 8, idx, w)
    torch.cuda.synchronize()


# --------------------------------------------------------------------- plan
def plan_np(plan, n):
    return dict(counts=plan.counts.cpu().numpy(), offsets=plan.offsets.cpu().numpy(),
                sorted_slots=plan.sorted_slots[:n].cpu().numpy(),
                unique_experts=plan.unique_experts.cpu().numpy(), n_unique=int(plan.n_unique.item()),
                work=plan.work.cpu().numpy())


def check_plan(got, ref, n_slots):
    for key in ("counts", "offsets", "sorted_slots", "unique_experts"):
        assert np.array_equal(got[key], ref[key]), key
    assert got["n_unique"] == ref["n_unique"]
    # work records: {expert, offsets[e], counts[e], first slot of e}; then {-1, n, 0, 0}
    E = len(ref["counts"])
    want = np.zeros((E, 4), np.int64)
    want[:, 0], want[:, 1] = -1, n_slots
    for u in range(ref["n_unique"]):
        e = ref["unique_experts"][u]
        want[u] = (e, ref["offsets"][e], ref["counts"][e], ref["sorted_slots"][ref["offsets"][e]])
    assert np.array_equal(got["work"], want), "work records"


@pytest.mark.parametrize("E,k,B,kind", [
    (128, 8, 1, "router"), (128, 8, 4, "sharing"), (128, 8, 8, "disjoint"), (128, 8, 32, "zipf"),
    (256, 6, 4, "router"), (8, 2, 1, "router"), (128, 8, 1024, "random"), (1024, 16, 512, "random"),
    (3, 2, 100, "random"), (1, 1, 5, "random"), (128, 8, 16, "same"),
])
def test_plan_matches_oracle(E, k, B, kind):
    sh = Shape("p", 31, 64, 64, E, k, "f32")
    rng = np.random.default_rng(B * 7 + E)
    if kind == "random":  # any ids, repeats within a token allowed
        idx = rng.integers(0, E, (B, k)).astype(np.int32)
    else:
        regime = {"router": "normal"}.get(kind, kind)
        idx, _ = oracle.route_topk(make_logits(sh, B, regime=regime, seed=5), k)
    plan = moe.expert_plan(torch.from_numpy(idx).cuda(), E)
    check_plan(plan_np(plan, B * k), oracle.plan(idx, E), B * k)


@pytest.mark.parametrize("E,k,B,regime", [
    (128, 8, 1, "normal"), (8, 2, 1, "normal"), (128, 8, 4, "sharing"), (128, 8, 32, "zipf"),
    (256, 6, 4, "normal"), (1024, 16, 64, "normal"), (128, 8, 65, "normal"), (64, 16, 200, "normal"),
    (1, 1, 3, "normal"),
    # just past the fused kernel's 16 tokens (the router and planner kernels),
    # odd counts and tied logits
    (128, 8, 17, "normal"), (128, 8, 47, "zipf"), (64, 4, 33, "same"), (256, 6, 50, "sharing"),
])
def test_route_plan_matches_oracle(E, k, B, regime):
    """The fused router+planner (one workgroup up to 16 tokens, two kernels beyond)."""
    sh = Shape("rp", 33, 64, 64, E, k, "f32")
    lg = make_logits(sh, B, regime=regime, seed=E * k + B)
    idx, w, plan = moe.route_plan(torch.from_numpy(lg).cuda(), k)
    ridx, rw = oracle.route_topk(lg, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(w.cpu().numpy() - rw).max() <= 1e-6
    check_plan(plan_np(plan, B * k), oracle.plan(ridx, E), B * k)


def test_plan_empty_batch():
    plan = moe.Plan.allocate(16, 8)
    plan.counts.fill_(7)
    moe.expert_plan(torch.zeros((0, 4), dtype=torch.int32, device="cuda"), 16, plan)
    got = plan_np(plan, 0)
    assert got["n_unique"] == 0 and got["counts"].sum() == 0
    assert np.all(got["offsets"] == 0) and np.all(got["unique_experts"] == -1)
    assert np.all(got["work"][:, 0] == -1)


# ------------------------------------------------------- expert block parity
DECODE_CASES = [
    # (shape, B, regime, x scale)
    ("toy", 1, "normal", 1.0),
    ("toy", 3, "normal", 1.0),
    ("decode", 1, "normal", 1.0),
    ("cohort", 4, "sharing", 1.0),
    ("cohort", 8, "sharing", 1.0),
    ("cohort", 8, "normal", 1.0),
    ("cohort", 8, "disjoint", 1.0),
    ("cohort", 6, "same", 1.0),
    ("wide", 1, "normal", 1.0),
    ("wide", 4, "normal", 1.0),
    ("wide", 2, "normal", 8.0),     # forced clamp: ~37 % of gate values beyond 10
    ("stack", 32, "zipf", 1.0),
]


@pytest.mark.parametrize("layout", ["rows", "cols"])
@pytest.mark.parametrize("name,B,regime,xs", DECODE_CASES)
def test_decode_step_matches_oracle(name, B, regime, xs, layout):
    sh = SHAPES[name]
    log(f"[case] decode {name} B={B} {regime} x*{xs} down={layout}")
    lg = make_logits(sh, B, regime=regime, seed=3)
    L = layer_for(sh, lg, seed=3) if sh.n_experts > 8 else make_layer(sh, seed=3)
    x = make_x(sh, B, seed=3, scale=xs)
    run = DeviceRun(L, x, lg, cols=layout == "cols")
    check_against_oracle(L, x, lg, run, f"{name}/B{B}/{regime}/x{xs}/{layout}")
    if xs > 1.0:
        h64 = oracle.decode_step(L, x, *oracle.route_topk(lg, sh.top_k), want_h=True)[1]
        lim = 10.0 / (1 + np.exp(-10.0)) * 10.0
        assert np.isclose(np.abs(h64).max(), lim) and np.isclose(np.abs(run.h).max(), lim, rtol=1e-6)


@pytest.mark.parametrize("H,F,E,k,act", [
    (256, 128, 8, 8, "f32"),       # k = E
    (512, 192, 16, 1, "bf16"),     # k = 1; 4 lanes x 4 chunks per gate/up row, 2 x 3 per down row
    (1024, 1536, 32, 4, "bf16"),   # 8 x 4 chunks per gate/up row, 16 x 3 per down row
    (8192, 64, 4, 2, "bf16"),      # 4 chunks per lane in a whole-wave row; one lane per down row
    (128, 4096, 4, 3, "f32"),      # one lane per gate/up row; one slot per LDS stage in down
    (64, 64, 2, 2, "bf16"),        # smallest rows
])
def test_decode_step_other_shapes(H, F, E, k, act):
    sh = Shape(f"s{H}x{F}", 32, H, F, E, k, act)
    B = 5
    lg = make_logits(sh, B, seed=H + F)
    L = make_layer(sh, seed=H + F)
    x = make_x(sh, B, seed=H + F)
    run = DeviceRun(L, x, lg)
    check_against_oracle(L, x, lg, run, f"{H}x{F}x{E}x{k}/{act}")


@pytest.mark.parametrize("E,H,F", [(3, 128, 128), (2, 256, 768), (4, 64, 2048), (1, 128, 384)])
def test_pack_down_is_the_stated_byte_permutation(E, H, F):
    sh = Shape(f"pk{H}x{F}", 34, H, F, E, 1, "bf16")
    L = make_layer(sh, seed=F)
    dl = moe.DeviceLayer.from_host(L)
    pk = dl.pack_down()
    torch.cuda.synchronize()
    q = pk.tensors["down_q"].cpu().numpy().view(np.uint32).reshape(E, F // 32, H, 4)
    want = L.down_q.reshape(E, H, F // 32, 4).transpose(0, 2, 1, 3)
    assert np.array_equal(q, want)
    for n in ("down_s", "down_b"):
        got = pk.tensors[n].cpu().numpy().view(np.uint16).reshape(E, F // 64, H)
        assert np.array_equal(got, getattr(L, n).transpose(0, 2, 1))
    # the source is untouched and gate/up are shared
    assert np.array_equal(dl.tensors["down_q"].cpu().numpy().view(np.uint32), L.down_q)
    assert pk.tensors["gate_q"].data_ptr() == dl.tensors["gate_q"].data_ptr()


@pytest.mark.parametrize("H,F,E,k", [(512, 128, 8, 2), (256, 256, 4, 4), (128, 512, 4, 2), (256, 1536, 4, 2),
                                     (128, 640, 2, 1), (128, 896, 2, 2), (128, 384, 2, 2), (128, 1024, 2, 2),
                                     (256, 768, 1, 1)])
def test_decode_step_column_layout_geometries(H, F, E, k):
    """Every (waves, chunks per wave) pairing of the column-layout down kernel."""
    sh = Shape(f"c{H}x{F}", 35, H, F, E, k, "bf16")
    B = 9  # more slots than one LDS stage (8) for some experts; all 9 when E = 1
    lg = make_logits(sh, B, seed=H * F)
    L = make_layer(sh, seed=H * F)
    x = make_x(sh, B, seed=H * F)
    run = DeviceRun(L, x, lg, cols=True)
    check_against_oracle(L, x, lg, run, f"cols {H}x{F}x{E}x{k}")


@pytest.mark.parametrize("H,F,E,k,B,regime", [
    (2048, 768, 128, 8, 12, "same"),    # 12 waves, 2-slot stages: every expert holds all 12 tokens
    (2048, 768, 128, 8, 9, "sharing"),  # 12 waves x 2 chunks; stages of 1 or 2 slots
    (512, 2048, 16, 4, 10, "same"),     # 16 waves, 2-slot stages: five stages per expert
    (256, 1536, 8, 2, 11, "normal"),    # 16 waves x 3 chunks
    (128, 896, 8, 2, 13, "same"),       # 4 waves x 7 chunks: four groups per wave and slot
])
def test_column_down_in_stages(H, F, E, k, B, regime):
    """The column-layout down kernel between 9 and 15 tokens (no MFMA, no
    token-major kernel): every expert's slots in stages, each stage's h
    groups fetched at once and read back from per-wave LDS rows."""
    sh = Shape(f"c{H}x{F}", 41, H, F, E, k, "bf16")
    log(f"[case] column down stages {H}x{F}x{E}x{k} B={B} {regime}")
    lg = make_logits(sh, B, regime=regime, seed=F + B)
    L = layer_for(sh, lg, seed=F + B) if E > 8 else make_layer(sh, seed=F + B)
    x = make_x(sh, B, seed=F + B)
    run = DeviceRun(L, x, lg, cols=True)
    check_against_oracle(L, x, lg, run, f"cols stages {H}x{F}x{E}x{k} B{B} {regime}")


MFMA_SHAPES = [
    (256, 128, 2, 1, 20),     # one group per wave
    (512, 192, 12, 2, 16),    # experts with 0..7 tokens: both variants in one launch
    (2048, 768, 1, 1, 40),    # 40 tokens on one expert: three token tiles of 16
    (4096, 256, 2, 2, 16),    # the wide hidden size: the two variants in two launches
    (1024, 64, 8, 8, 16),     # k = E: every expert holds all 16 tokens
    (1536, 128, 8, 1, 17),    # one to five tokens per expert
    (768, 256, 4, 2, 16),     # 12 groups: no MFMA workgroup shape, dot2 for every expert
]


# dff 192 and 64 have no column-layout down kernel: rows only
@pytest.mark.parametrize("H,F,E,k,B,layout", [s + (lay,) for s in MFMA_SHAPES for lay in ("rows", "cols")
                                              if lay == "rows" or s[1] not in (192, 64)])
def test_gate_up_mfma_path(H, F, E, k, B, layout):
    """In batches of 16 or more tokens, experts with >= 3 tokens run the
    MFMA gate+up kernel (and, with column-layout down weights, the MFMA down
    kernel where it has a shape)."""
    sh = Shape(f"m{H}x{F}", 36, H, F, E, k, "bf16")
    lg = make_logits(sh, B, seed=H + B)
    L = make_layer(sh, seed=H + B)
    x = make_x(sh, B, seed=H + B)
    run = DeviceRun(L, x, lg, cols=layout == "cols")
    check_against_oracle(L, x, lg, run, f"mfma {H}x{F}x{E}x{k} B{B} {layout}")
    assert run.plan_np["counts"].max() >= 3


@pytest.mark.parametrize("H,F,E,k,B,act", [
    (256, 128, 4, 2, 16, "bf16"),    # 2 waves x 1 group
    (128, 256, 3, 2, 16, "f32"),     # 4 x 1, fp32 activations
    (192, 384, 4, 2, 17, "bf16"),    # 6 x 1
    (64, 512, 2, 1, 16, "bf16"),     # 8 x 1
    (2048, 768, 24, 4, 18, "bf16"),  # 6 x 2: the decode layer's dff; 0..8 tokens per expert
    (128, 1024, 2, 2, 16, "bf16"),   # 8 x 2
    (256, 1536, 3, 2, 16, "bf16"),   # 8 x 3
    (4096, 2048, 4, 2, 20, "bf16"),  # 8 x 4: the wide layer; 20 tokens on some experts (two token tiles)
])
def test_down_mfma_path(H, F, E, k, B, act):
    """Column-layout down projection of experts with >= 3 tokens on MFMA, h
    split exactly into three bf16 parts; every (waves, groups) instance."""
    sh = Shape(f"d{H}x{F}", 38, H, F, E, k, act)
    lg = make_logits(sh, B, seed=F + B)
    L = make_layer(sh, seed=F + B)
    x = make_x(sh, B, seed=F + B)
    log(f"[case] down mfma {H}x{F}x{E}x{k} B={B} {act}")
    run = DeviceRun(L, x, lg, cols=True)
    check_against_oracle(L, x, lg, run, f"down mfma {H}x{F}x{E}x{k} B{B} {act}")
    assert run.plan_np["counts"].max() >= 3


@pytest.mark.parametrize("layout", ["rows", "cols"])
@pytest.mark.parametrize("H,F,E,k,act", [
    (2048, 768, 128, 8, "bf16"),    # the single-token decode layer
    (4096, 2048, 256, 6, "bf16"),   # four logits per router lane, sidecar and clamp
    (256, 128, 8, 2, "f32"),
    (512, 256, 16, 1, "bf16"),      # k = 1
    (256, 256, 4, 4, "bf16"),       # k = E
    (128, 384, 512, 16, "bf16"),    # 512 experts: routed by the router launch instead
    (1024, 512, 64, 4, "f32"),      # GeGLU with a down-projection sidecar
])
@pytest.mark.parametrize("ties,B", [("none", 1), ("ties", 1), ("none", 2), ("ties", 4), ("none", 8)])
def test_decode_layer_few_tokens_is_bitwise_the_two_call_path(H, F, E, k, act, layout, ties, B):
    """moe_decode_layer at B = 1, 2, 4, 8 (gate+up routes for itself, each wave
    selecting only its own rank) against moe_route_plan + moe_decode_step:
    outputs, routing and plan identical, also with tied logits (ties go to
    the lower id; -0 equals +0)."""
    wide = (H, E) == (4096, 256)
    geglu = H == 1024
    sh = Shape(f"l{H}x{F}x{E}", 37, H, F, E, k, act, sidecar=wide, clamp=10.0 if wide else 0.0,
               activation="geglu" if geglu else "swiglu", down_sidecar=geglu)
    log(f"[case] decode_layer B={B} {H}x{F}x{E}x{k} {act} down={layout} {ties}")
    lg = make_logits(sh, B, seed=E + k)
    if ties == "ties":
        lg[:, ::3] = 1.5                 # a third of the experts tie at the top
        lg[:, 1::7] = 0.0
        lg[:, 2::14] = -0.0
    L = layer_for(sh, lg, seed=E + k)
    x = make_x(sh, B, seed=E + k)
    res = make_x(sh, B, seed=E + k + 1)
    dl = moe.DeviceLayer.from_host(L)
    if layout == "cols":
        dl = dl.pack_down()
    lgt = torch.from_numpy(lg).cuda()
    xt, rt = dev_x(x), dev_x(res)
    out1, idx1, w1, plan1 = moe.decode_layer(dl, xt, lgt, residual=rt)
    idx2, w2, plan2 = moe.route_plan(lgt, k)
    out2 = moe.decode_step(dl, xt, idx2, w2, plan2, residual=rt)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2) and torch.equal(w1, w2)
    for f in ("counts", "offsets", "unique_experts", "n_unique", "work"):
        assert torch.equal(getattr(plan1, f), getattr(plan2, f)), f
    assert torch.equal(plan1.sorted_slots[:B * k], plan2.sorted_slots[:B * k])
    assert np.array_equal(host_bits(out1), host_bits(out2))
    ridx, _ = oracle.route_topk(lg, k)
    assert np.array_equal(idx1.cpu().numpy(), ridx)


# ------------------------------------------- GeGLU and the down-projection sidecar
GEGLU_CASES = [
    # (shape, B, regime): B <= 8 routes inside gate+up and combines in the down
    # kernel; 12 runs the VALU kernels and the combine launch; 16 and 32 the
    # MFMA kernels where an expert holds >= 3 tokens
    ("decode", 1, "normal"),
    ("cohort", 4, "sharing"),
    ("cohort", 12, "sharing"),
    ("wide", 2, "normal"),
    ("wide", 16, "same"),
    ("stack", 32, "zipf"),
]


@pytest.mark.parametrize("layout", ["rows", "cols"])
@pytest.mark.parametrize("name,B,regime", GEGLU_CASES)
def test_geglu_with_down_sidecar_matches_oracle(name, B, regime, layout):
    """GeGLU (tanh-form GELU) and a per-expert scale of the down output, on
    every kernel path, against the oracle's fp64 GELU and scaling."""
    import dataclasses
    sh = dataclasses.replace(SHAPES[name], activation="geglu", down_sidecar=True)
    log(f"[case] geglu+down sidecar {name} B={B} {regime} down={layout}")
    lg = make_logits(sh, B, regime=regime, seed=11)
    L = layer_for(sh, lg, seed=11)
    assert L.activation == "geglu" and L.down_sidecar is not None
    x = make_x(sh, B, seed=11)
    run = DeviceRun(L, x, lg, cols=layout == "cols")
    check_against_oracle(L, x, lg, run, f"geglu {name}/B{B}/{regime}/{layout}")


@pytest.mark.parametrize("B", [1, 4, 12, 32])
def test_power_of_two_down_sidecar_scales_the_output_exactly(B):
    """A down sidecar of 2 (4 for every other expert) multiplies each y by a
    power of two: with fp32 activations and no residual, every output is
    then exactly the weighted sum of those scaled y, so a uniform 2 doubles
    the output bit for bit; the GeGLU h is untouched by it."""
    import dataclasses
    sh = dataclasses.replace(SHAPES["cohort"], act="f32", activation="geglu")
    lg = make_logits(sh, B, regime="sharing", seed=B)
    L = layer_for(sh, lg, seed=B)
    x = make_x(sh, B, seed=B)
    base = DeviceRun(L, x, lg, cols=True)
    L.down_sidecar = np.full(sh.n_experts, 2.0, np.float32)
    two = DeviceRun(L, x, lg, cols=True)
    assert np.array_equal(two.out, base.out * 2)
    assert np.array_equal(two.h, base.h)
    check_against_oracle(L, x, lg, two, f"down sidecar x2 B{B}")
    L.down_sidecar = np.where(np.arange(sh.n_experts) % 2, 4.0, 2.0).astype(np.float32)
    check_against_oracle(L, x, lg, DeviceRun(L, x, lg, cols=True), f"down sidecar 2/4 B{B}")


# ------------------------------------------- other widths and group sizes
WIDTH_FORMATS = [(8, 8, 64), (4, 6, 64), (6, 6, 32), (8, 4, 128), (4, 4, 32), (4, 4, 128), (6, 8, 128)]


@pytest.mark.parametrize("bits,down_bits,group", WIDTH_FORMATS)
@pytest.mark.parametrize("name,B,regime", [("decode", 1, "normal"), ("cohort", 4, "sharing"),
                                           ("cohort", 9, "same"), ("toy", 3, "normal")])
def test_other_widths_match_oracle(bits, down_bits, group, name, B, regime):
    """4/6/8-bit gate+up and down in groups of 32/64/128 (the generic row
    kernels): routing, plan, h and outputs against the oracle; the "same"
    routing puts 9 slots on each expert (several slot stages per pass)."""
    import dataclasses
    sh = dataclasses.replace(SHAPES[name], bits=bits, down_bits=down_bits, group_size=group)
    log(f"[case] widths {bits}/{down_bits} g{group} {name} B={B} {regime}")
    lg = make_logits(sh, B, regime=regime, seed=bits * 10 + down_bits)
    L = layer_for(sh, lg, seed=group) if sh.n_experts > 8 else make_layer(sh, seed=group)
    x = make_x(sh, B, seed=group)
    run = DeviceRun(L, x, lg)
    check_against_oracle(L, x, lg, run, f"w{bits}/{down_bits}g{group} {name} B{B} {regime}")


@pytest.mark.parametrize("bits,down_bits,group", [(8, 8, 128), (6, 4, 32)])
def test_other_widths_on_the_wide_layer_with_geglu_and_sidecars(bits, down_bits, group):
    """hidden 4096 (four units per lane), the expert-scale sidecar, clamp,
    GeGLU and a down sidecar through the generic kernels."""
    import dataclasses
    sh = dataclasses.replace(SHAPES["wide"], bits=bits, down_bits=down_bits, group_size=group,
                             activation="geglu", down_sidecar=True)
    log(f"[case] widths wide {bits}/{down_bits} g{group}")
    lg = make_logits(sh, 2, seed=7)
    L = layer_for(sh, lg, seed=7)
    x = make_x(sh, 2, seed=7, scale=4.0)  # some gate values beyond the clamp
    run = DeviceRun(L, x, lg)
    check_against_oracle(L, x, lg, run, f"wide w{bits}/{down_bits}g{group}")


@pytest.mark.parametrize("bits,down_bits,layout,B", [
    (8, 4, "cols", 1), (8, 4, "cols", 4), (8, 4, "cols", 12), (8, 4, "cols", 20), (8, 4, "rows", 8),
    (4, 8, "rows", 1), (4, 8, "rows", 8), (4, 8, "rows", 20),
])
def test_mixed_width_layers_take_each_projections_kernels(bits, down_bits, layout, B):
    """Group-64 layers with one projection in 4 bits: the 4-bit projection
    runs the specialised kernels (the routing gate+up kernel at few tokens,
    MFMA from 16 tokens, the token-major or column-layout down kernels), the
    other the generic row kernels; results against the oracle."""
    import dataclasses
    sh = dataclasses.replace(SHAPES["cohort"], bits=bits, down_bits=down_bits, group_size=64)
    log(f"[case] mixed widths {bits}/{down_bits} {layout} B={B}")
    lg = make_logits(sh, B, regime="sharing", seed=bits + B)
    L = layer_for(sh, lg, seed=bits + B)
    x = make_x(sh, B, seed=bits + B)
    run = DeviceRun(L, x, lg, cols=layout == "cols")
    check_against_oracle(L, x, lg, run, f"mixed {bits}/{down_bits} {layout} B{B}")


def test_other_widths_batch_invariance_and_entry_points():
    """A token alone equals the same token in a batch bit for bit; the
    two-call path equals moe_decode_layer; the column layout is refused."""
    import dataclasses
    sh = dataclasses.replace(SHAPES["cohort"], bits=4, down_bits=6, group_size=64)
    B = 6
    lg = make_logits(sh, B, regime="sharing", seed=4)
    L = layer_for(sh, lg, seed=4)
    x = make_x(sh, B, seed=4)
    dl = moe.DeviceLayer.from_host(L)
    a = DeviceRun(L, x, lg, dl=dl)
    for t in range(B):
        one = DeviceRun(L, x[t:t + 1], lg[t:t + 1], dl=dl)
        assert np.array_equal(one.out[0], a.out[t]), f"token {t}"
    lgt = torch.from_numpy(lg).cuda()
    idx2, w2, plan2 = moe.route_plan(lgt, sh.top_k)
    out2 = moe.decode_step(dl, dev_x(x), idx2, w2, plan2)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out2), a.out)
    with pytest.raises(moe.MoeError):
        dl.pack_down()


# ------------------------------------------------------- large batches
@pytest.mark.parametrize("B,layout", [(256, "rows"), (256, "cols"), (1024, "cols")])
def test_prefill_sized_batch_on_sampled_tokens(B, layout):
    """Prefill-sized batches (every expert holds tokens, 16 or 64 on
    average, in several MFMA token tiles): routing and plan checked whole,
    h and outputs of sampled tokens against the oracle run on those tokens
    alone (a token's result depends on that token only)."""
    sh = SHAPES["cohort"]
    log(f"[case] prefill B={B} down={layout}")
    lg = make_logits(sh, B, regime="normal", seed=B + 5)
    L = layer_for(sh, lg, seed=B + 5)
    x = make_x(sh, B, seed=B + 5)
    run = DeviceRun(L, x, lg, cols=layout == "cols")
    idx, w = oracle.route_topk(lg, sh.top_k)
    assert np.array_equal(run.idx, idx)
    assert float(np.abs(run.w - w).max()) <= 1e-6
    p = oracle.plan(idx, sh.n_experts)
    for k in ("counts", "offsets", "sorted_slots", "unique_experts"):
        assert np.array_equal(run.plan_np[k], p[k]), k
    assert p["counts"].min() >= 3, "every expert should take the MFMA kernels"
    rng = np.random.default_rng(B)
    toks = np.unique(np.concatenate([[0, B - 1], rng.choice(B, 14, replace=False)]))
    out64, h64 = oracle.decode_step(L, x[toks], idx[toks], w[toks], want_h=True)
    slots = (toks[:, None] * sh.top_k + np.arange(sh.top_k)[None, :]).ravel()
    eh = rel_l2(run.h[slots], h64)
    got = oracle.bf16_to_f64(run.out[toks])
    eo = rel_l2(got, out64)
    dg = rel_l2(got, oracle.bf16_to_f64(oracle.round_bf16(out64)))
    log(f"[parity] prefill B={B} {layout}: {len(toks)} tokens h_rel={eh:.3g} out_rel={eo:.3g} diag={dg:.3g}")
    record(f"prefill B{B} {layout}", h=eh, out=eo, diag=dg)
    assert eh <= 1e-5 and eo <= REL_L2_GATE and dg <= REL_L2_DIAG
    assert np.isfinite(oracle.bf16_to_f64(run.out)).all()


@pytest.mark.parametrize("H,F,E,k,B,regime,layout,act", [
    (256, 256, 8, 2, 128, "normal", "cols", "swiglu"),    # ~32 tokens per expert: one block of two tiles
    (256, 192, 8, 2, 300, "zipf", "rows", "swiglu"),      # skewed counts over several blocks; a ragged gate row block
    (192, 256, 8, 2, 300, "zipf", "cols", "swiglu"),      # a ragged down row block (hidden 192); gate+up on its own kernels
    (512, 256, 16, 4, 200, "normal", "rows", "swiglu"),   # rows-layout down keeps its own kernels
    (256, 256, 256, 8, 160, "normal", "cols", "swiglu"),  # 256 plan records (four per lane); ~5 tokens each
    (256, 256, 4, 1, 129, "same", "cols", "swiglu"),      # one expert holds all 129 tokens: blocks of 64, 64, 1
    (4096, 256, 4, 2, 128, "normal", "cols", "swiglu"),   # 64 groups of hidden: 128 KB of scales in LDS
    (1024, 512, 8, 2, 140, "normal", "cols", "geglu"),    # GeGLU, both sidecars and the clamp
    (256, 128, 8, 2, 130, "normal", "cols", "swiglu"),    # dff 128: no whole load ring, the earlier kernels
])
def test_tile_kernels_match_oracle(H, F, E, k, B, regime, layout, act):
    """Batches of 128 tokens or more run the tile kernels: every distinct
    expert's tokens in blocks of 64 on MFMA (gate+up always, down with the
    column layout).  Whole outputs against the oracle; three tokens alone
    against the batch (a different kernel, the same exact products)."""
    geglu = act == "geglu"
    sh = Shape(f"t{H}x{F}", 40, H, F, E, k, "bf16", sidecar=geglu, clamp=10.0 if geglu else 0.0,
               activation=act, down_sidecar=geglu)
    log(f"[case] tile {H}x{F}x{E}x{k} B={B} {regime} {layout} {act}")
    lg = make_logits(sh, B, regime=regime, seed=H + B)
    L = make_layer(sh, seed=H + B)
    x = make_x(sh, B, seed=H + B, scale=4.0 if geglu else 1.0)
    dl = moe.DeviceLayer.from_host(L)
    if layout == "cols":
        dl = dl.pack_down()
    run = DeviceRun(L, x, lg, dl=dl)
    check_against_oracle(L, x, lg, run, f"tile {H}x{F}x{E}x{k} B{B} {regime} {layout} {act}")
    counts = run.plan_np["counts"]
    log(f"[tile] counts min {counts[counts > 0].min()} max {counts.max()}")
    for t in (0, B // 2, B - 1):
        one = DeviceRun(L, x[t:t + 1], lg[t:t + 1], dl=dl)
        assert rel_l2(oracle.bf16_to_f64(one.out[0]), oracle.bf16_to_f64(run.out[t])) <= 5e-4


# --------------------------------------------------------------- invariants
@pytest.mark.parametrize("layout", ["rows", "cols"])
def test_determinism_batch_invariance_permutation_and_duplicates(layout):
    sh = SHAPES["cohort"]
    B = 8
    lg = make_logits(sh, B, regime="sharing", seed=9)
    x = make_x(sh, B, seed=9)
    dup_lg = np.repeat(lg[2:3], 4, axis=0)
    L = layer_for(sh, np.concatenate([lg, dup_lg]), seed=9)
    dl = moe.DeviceLayer.from_host(L)
    if layout == "cols":
        dl = dl.pack_down()
    a = DeviceRun(L, x, lg, dl=dl)
    b = DeviceRun(L, x, lg, dl=dl)
    assert np.array_equal(a.out, b.out), "run-to-run results differ"
    # A token's result is bitwise the same alone and in the batch when its
    # experts take the same kernel variant.  Batches under 16 tokens run the
    # VALU kernels only, so here every token must match bitwise (the shared
    # experts hold three tokens: in a batch of 16 they would go to MFMA).
    assert a.plan_np["counts"].max() >= 3
    for t in range(B):
        one = DeviceRun(L, x[t:t + 1], lg[t:t + 1], dl=dl)
        assert np.array_equal(one.out[0], a.out[t]), f"token {t} alone differs from the batch"
    perm = np.array([5, 2, 7, 0, 1, 6, 3, 4])
    p = DeviceRun(L, x[perm], lg[perm], dl=dl)
    assert np.array_equal(p.out, a.out[perm])
    d = DeviceRun(L, np.repeat(x[2:3], 4, axis=0), dup_lg, dl=dl)
    assert d.plan_np["n_unique"] == sh.top_k
    assert np.all(d.out == d.out[0:1])
    assert np.array_equal(d.out[0], a.out[2])


@pytest.mark.parametrize("layout", ["rows", "cols"])
def test_batch_invariance_across_the_mfma_switch(layout):
    """In a batch of 16, tokens whose experts all hold < 3 tokens stay
    bitwise equal to the token alone; the others (MFMA kernels) stay within
    the fp32 pipeline's error of it."""
    sh = SHAPES["cohort"]
    B = 16
    lg = make_logits(sh, B, regime="sharing", seed=21)
    x = make_x(sh, B, seed=21)
    L = layer_for(sh, lg, seed=21)
    dl = moe.DeviceLayer.from_host(L)
    if layout == "cols":
        dl = dl.pack_down()
    a = DeviceRun(L, x, lg, dl=dl)
    check_against_oracle(L, x, lg, a, f"cohort B16 sharing {layout}")
    counts = a.plan_np["counts"]
    n_mfma = 0
    for t in range(B):
        one = DeviceRun(L, x[t:t + 1], lg[t:t + 1], dl=dl)
        if counts[a.idx[t]].max() < 3:
            assert np.array_equal(one.out[0], a.out[t]), f"token {t} alone differs from the batch"
        else:
            n_mfma += 1
            assert rel_l2(oracle.bf16_to_f64(one.out[0]), oracle.bf16_to_f64(a.out[t])) <= 5e-4
    assert 0 < n_mfma < B


def test_batch_size_changes_between_calls_with_the_same_buffers():
    sh = SHAPES["cohort"]
    lgs = {B: make_logits(sh, B, seed=40 + B) for B in (4, 1, 8, 3)}
    L = layer_for(sh, np.concatenate(list(lgs.values())), seed=40)
    dl = moe.DeviceLayer.from_host(L)
    plan = moe.Plan.allocate(sh.n_experts, 8 * sh.top_k)
    ws = moe.alloc_workspace(dl, 8)
    for B, lg in lgs.items():
        x = make_x(sh, B, seed=40 + B)
        out, idx, w, _ = moe.decode_layer(dl, dev_x(x), torch.from_numpy(lg).cuda(), plan=plan, workspace=ws)
        ridx, rw = oracle.route_topk(lg, sh.top_k)
        ref = oracle.decode_step(L, x, ridx, rw)
        got = oracle.bf16_to_f64(host_bits(out))
        assert np.array_equal(idx.cpu().numpy(), ridx)
        assert rel_l2(got, ref) <= 2e-3, B


def test_residual_stack_of_layers():
    sh = SHAPES["stack"]
    B, n_layers = 32, 4
    lgs = [make_logits(sh, B, layer=l, regime="zipf", seed=11) for l in range(n_layers)]
    layers = [layer_for(sh, lgs[l], layer=l, seed=11) for l in range(n_layers)]
    x0 = make_x(sh, B, seed=11)
    # oracle: the mirrored stack, and the per-layer inputs it saw
    seen = []
    ref = oracle.run_stack(layers, x0, lgs, sh.top_k, hook=lambda l, x, i, w, o: seen.append(x.copy()))
    xt = dev_x(x0)
    for l in range(n_layers):
        dl = moe.DeviceLayer.from_host(layers[l])
        nxt = torch.empty_like(xt)
        moe.decode_layer(dl, xt, torch.from_numpy(lgs[l]).cuda(), residual=xt, out=nxt)
        # teacher-forced: the same layer from the oracle's own input
        tf = torch.empty_like(xt)
        moe.decode_layer(dl, dev_x(seen[l]), torch.from_numpy(lgs[l]).cuda(), residual=dev_x(seen[l]), out=tf)
        idx, w = oracle.route_topk(lgs[l], sh.top_k)
        o64 = oracle.decode_step(layers[l], seen[l], idx, w)
        want = oracle.bf16_to_f64(oracle.residual_bf16(seen[l], o64))
        e = rel_l2(oracle.bf16_to_f64(host_bits(tf)) - oracle.bf16_to_f64(seen[l]),
                   want - oracle.bf16_to_f64(seen[l]))
        log(f"[stack] layer {l}: residual-branch rel L2 {e:.3g}")
        assert e <= 2e-3
        xt = nxt
    got = oracle.bf16_to_f64(host_bits(xt))
    e = rel_l2(got, oracle.bf16_to_f64(ref))
    log(f"[stack] final x rel L2 {e:.3g}")
    assert e <= 2e-3


def _host_layer(sh, t, experts):
    """A host copy of a device layer (rows layout) holding only `experts`;
    the others keep poisoned scales, so a wrong gather cannot pass."""
    from moe_workloads.gen import _empty_layer

    L = _empty_layer(sh)
    for e in experts:
        for n in ("gate_q", "up_q", "down_q"):
            dst = getattr(L, n)
            dst[e] = t[n][e].cpu().numpy().view(np.uint32).reshape(dst.shape[1:])
        for n in ("gate_s", "gate_b", "up_s", "up_b", "down_s", "down_b"):
            dst = getattr(L, n)
            dst[e] = t[n][e].cpu().numpy().view(np.uint16).reshape(dst.shape[1:])
        L.materialised[e] = True
    return L


def _check_stack_chain(n_layers, B, from_x, seed):
    """Runs the chained all-MoE stack layer by layer and checks every layer:
    routing and plan bit-exact for all tokens (against the oracle's routing
    of the logits the layer used); the layer's expert output against the
    oracle on 4 sampled tokens, from the GPU chain's own input to that layer,
    so each layer is checked without error carried over from the ones
    before it; and the next layer's input bit-exact equal to
    bf16(x + bf16(out)) for every token.  With from_x each layer's logits are
    projected from its input (moe_router_logits) and checked against the
    oracle's projection first.  Weights are drawn on the device; only the
    experts the sampled tokens touch are copied for the oracle."""
    from moe_workloads import make_layer_device

    sh = SHAPES["stack"]
    k, E = sh.top_k, sh.n_experts
    rng = np.random.default_rng(seed)
    x = dev_x(make_x(sh, B, seed=seed))
    plan = moe.Plan.allocate(E, B * k)
    ws = None
    worst = 0.0
    for l in range(n_layers):
        if from_x:
            wr = make_router(sh, layer=l, seed=seed)
            lgt = moe.router_logits(x, torch.from_numpy(wr.view(np.int16)).cuda().view(torch.bfloat16))
            torch.cuda.synchronize()
            lg = lgt.cpu().numpy()
            xb = host_bits(x)
            ref = oracle.router_logits(xb, wr)
            mag = np.abs(oracle.bf16_to_f64(xb)) @ np.abs(oracle.bf16_to_f64(wr)).T
            assert np.all(np.abs(lg.astype(np.float64) - ref) <= 1e-5 * mag), f"layer {l}: router logits"
        else:
            lg = make_logits(sh, B, layer=l, regime="zipf", seed=seed)
            lgt = torch.from_numpy(lg).cuda()
        t = make_layer_device(sh, l, torch.device("cuda"), seed=seed)
        rows = moe.DeviceLayer.from_tensors(sh.hidden, sh.dff, E, k, sh.act, 0.0, t)
        dl = rows.pack_down()
        if ws is None:
            ws = moe.alloc_workspace(dl, B)
        out = torch.empty_like(x)
        nxt = torch.empty_like(x)
        _, idx, w, _ = moe.decode_layer(dl, x, lgt, plan=plan, workspace=ws, out=out)
        moe.decode_layer(dl, x, lgt, plan=plan, workspace=ws, out=nxt, residual=x)
        torch.cuda.synchronize()
        ridx, rw = oracle.route_topk(lg, k)
        assert np.array_equal(idx.cpu().numpy(), ridx), f"layer {l}: routing"
        assert float(np.abs(w.cpu().numpy() - rw).max()) <= 1e-6, f"layer {l}: router weights"
        p = oracle.plan(ridx, E)
        assert np.array_equal(plan.sorted_slots[:B * k].cpu().numpy(), p["sorted_slots"]), f"layer {l}: plan"
        assert np.array_equal(plan.counts.cpu().numpy(), p["counts"]), f"layer {l}: plan counts"
        xb, ob, nb = host_bits(x), host_bits(out), host_bits(nxt)
        # NaN bit patterns carry no value: compare them as one value
        canon = lambda a: np.where(np.isnan(oracle.bf16_to_f64(a)), np.uint16(0x7FC0), a)
        want = oracle.residual_bf16(xb, oracle.bf16_to_f64(ob))
        assert np.array_equal(canon(nb), canon(want)), f"layer {l}: residual"
        # Nothing normalises the residual stream between layers, so on these
        # N(0, 0.02) weights a few tokens' activations grow until they
        # overflow bf16 in the last layers.  Sample finite tokens for the
        # tolerance checks, and check that an overflowed token overflows in
        # the oracle too.
        fin = np.isfinite(oracle.bf16_to_f64(ob)).all(axis=1) & np.isfinite(oracle.bf16_to_f64(xb)).all(axis=1)
        S = np.sort(rng.choice(np.flatnonzero(fin), min(4, int(fin.sum())), replace=False))
        L = _host_layer(sh, t, np.unique(ridx[S]))
        o64 = oracle.decode_step(L, xb[S], ridx[S], rw[S])
        got = oracle.bf16_to_f64(ob[S])
        gate = rel_l2(got, o64)
        diag = rel_l2(got, oracle.bf16_to_f64(oracle.round_bf16(o64)))
        record(f"stack {'from x ' if from_x else ''}layer {l}", n_unique=int(p["n_unique"]), out=gate, diag=diag,
               overflowed_tokens=int(B - fin.sum()))
        assert gate <= REL_L2_GATE, f"layer {l}: output rel L2 {gate}"
        assert diag <= REL_L2_DIAG, f"layer {l}: diagnostic rel L2 {diag}"
        if not fin.all():
            v = int(np.flatnonzero(~fin)[0])
            Lv = _host_layer(sh, t, np.unique(ridx[v]))
            ov = oracle.round_bf16(oracle.decode_step(Lv, xb[v:v + 1], ridx[v:v + 1], rw[v:v + 1]))
            assert not np.isfinite(oracle.bf16_to_f64(ov)).all(), f"layer {l}: token {v} overflows on the GPU only"
        worst = max(worst, gate)
        x = nxt
        del t, rows, dl, L
    return worst


def test_48_layer_stack_step():
    """The 48-layer all-MoE step at B = 32 with Zipf(1.1) routing per layer,
    each layer reading the previous layer's output through the residual, as
    the benchmark runs it; every layer checked (see _check_stack_chain)."""
    worst = _check_stack_chain(48, 32, from_x=False, seed=48)
    log(f"[stack48] worst layer output rel L2 {worst:.3g}")


def test_stack_routed_from_x():
    """Eight chained layers at B = 32 whose routing starts from x: each
    layer's logits projected from its own input by moe_router_logits, as the
    benchmark's stack routed from x runs it."""
    worst = _check_stack_chain(8, 32, from_x=True, seed=49)
    log(f"[stack from x] worst layer output rel L2 {worst:.3g}")


def test_invalid_expert_id_gives_nan_for_that_token_only():
    sh = SHAPES["cohort"]
    B = 3
    lg = make_logits(sh, B, seed=12)
    L = layer_for(sh, lg, seed=12)
    dl = moe.DeviceLayer.from_host(L)
    idx, w = oracle.route_topk(lg, sh.top_k)
    bad = idx.copy()
    bad[1, 3] = 5000          # out of range: left out of the plan, NaN for token 1
    bad[2, 0] = -1
    it = torch.from_numpy(bad).cuda()
    # the planner leaves the two bad slots out of every list
    got = plan_np(moe.expert_plan(it, sh.n_experts), B * sh.top_k)
    assert got["counts"].sum() == B * sh.top_k - 2 and got["offsets"][-1] == B * sh.top_k - 2
    wt = torch.from_numpy(w.astype(np.float32)).cuda()
    plan = moe.expert_plan(it, sh.n_experts)
    x = make_x(sh, B, seed=12)
    out = moe.decode_step(dl, dev_x(x), it, wt, plan)
    got = oracle.bf16_to_f64(host_bits(out))
    assert np.isnan(got[1]).all() and np.isnan(got[2]).all()
    ref = oracle.decode_step(L, x[:1], idx[:1], w[:1])
    assert rel_l2(got[0], ref[0]) <= 2e-3


def test_empty_batch_decode_step_is_a_no_op():
    sh = SHAPES["toy"]
    L = make_layer(sh, seed=1)
    dl = moe.DeviceLayer.from_host(L)
    out = torch.full((0, sh.hidden), 3.0, device="cuda")
    plan = moe.Plan.allocate(sh.n_experts, 1)
    moe.decode_step(dl, torch.zeros((0, sh.hidden), device="cuda"), torch.zeros((0, 2), dtype=torch.int32, device="cuda"),
                    torch.zeros((0, 2), device="cuda"), plan, out=out, workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()


# -------------------------------------------------------- router projection
@pytest.mark.parametrize("H,E,B,act", [
    (2048, 128, 1, "bf16"),    # the decode layer: 64 lanes x 4 chunks per row
    (2048, 128, 32, "bf16"),
    (4096, 256, 4, "bf16"),    # 64 x 8
    (256, 8, 3, "f32"),        # the toy layer: 32 lanes x 1 chunk, fp32 activations
    (384, 37, 5, "bf16"),      # 16 x 3; E not a multiple of the rows per wave
    (8, 5, 2, "f32"),          # one chunk per row
    (3072, 64, 2, "f32"),      # 64 x 6
    (384, 37, 9, "bf16"),      # larger batches: a ragged last tile
    (256, 8, 8, "f32"),        # 32-lane segments summed across two rows
    (3072, 64, 8, "f32"),
    (4096, 256, 16, "bf16"),   # 64 x 8: 2-token tiles
    (2048, 100, 33, "bf16"),   # E not a multiple of 4; ragged tile
])
def test_router_logits_match_oracle(H, E, B, act):
    sh = Shape(f"rp{H}x{E}", 39, H, 64, E, 1, act)
    x = make_x(sh, B, seed=H + E)
    wr = make_router(sh, seed=H + E)
    xt = dev_x(x)
    wt = torch.from_numpy(wr.view(np.int16)).cuda().view(torch.bfloat16)
    got = moe.router_logits(xt, wt)
    torch.cuda.synchronize()
    ref = oracle.router_logits(x, wr)
    xf = oracle.bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)
    mag = np.abs(xf) @ np.abs(oracle.bf16_to_f64(wr)).T
    err = np.abs(got.cpu().numpy().astype(np.float64) - ref)
    log(f"[parity] router logits {H}x{E} B{B} {act}: max err/|x||w| = {(err / mag).max():.3g}")
    # exact products, fp32 sums of H terms: far below 1e-5 of sum |x w|; one
    # dropped or doubled term is ~1/H of it
    assert np.all(err <= 1e-5 * mag + 1e-30)
    again = moe.router_logits(xt, wt)
    one = moe.router_logits(xt[B - 1:B].contiguous(), wt)
    torch.cuda.synchronize()
    assert torch.equal(got, again)
    assert torch.equal(one[0], got[B - 1])  # a token's logits do not depend on the batch


@pytest.mark.parametrize("name,B", [("decode", 1), ("cohort", 8), ("stack", 32)])
def test_layer_routed_from_the_projection(name, B):
    """x -> moe_router_logits -> moe_decode_layer, against the oracle routing
    the same fp32 logits."""
    sh = SHAPES[name]
    x = make_x(sh, B, seed=40)
    wr = make_router(sh, seed=40)
    lg = moe.router_logits(dev_x(x), torch.from_numpy(wr.view(np.int16)).cuda().view(torch.bfloat16))
    torch.cuda.synchronize()
    lg_np = lg.cpu().numpy()
    L = layer_for(sh, lg_np, seed=40)
    run = DeviceRun(L, x, lg_np, cols=True)
    check_against_oracle(L, x, lg_np, run, f"projected {name} B{B}")
