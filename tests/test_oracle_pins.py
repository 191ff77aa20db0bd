"""Pins of the C oracle against things other than itself (CPU only).

Each test targets a mistake the oracle could plausibly make: a dropped bias
term, a wrong nibble or group index, a transposed operand, a wrong tie
order, the sidecar and clamp in the wrong order, double rounding, a wrong
combine weight.  The pages print no worked example, so the pins are the
independent numpy brute force (tests/bruteforce.py), closed forms,
invariants and exhaustive checks of the conversions.
"""

import hashlib
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import bruteforce as bf
from moe_workloads import SHAPES, Shape, make_layer, make_logits, make_router, make_x, quantize_affine4
from moe_workloads.gen import bf16_bits_from_f32, f32_from_bf16_bits
from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(H=128, F=64, E=4, k=2, act="f32", sidecar=False, clamp=0.0, cfg=90):
    return Shape(f"tiny{H}x{F}x{E}x{k}", cfg, H, F, E, k, act, sidecar=sidecar, clamp=clamp)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ------------------------------------------------------------- generators
def test_generator_is_deterministic():
    sh = SHAPES["toy"]
    a = make_layer(sh, layer=0, seed=3)
    b = make_layer(sh, layer=0, seed=3)
    c = make_layer(sh, layer=0, seed=4)
    for name in ("gate_q", "up_s", "down_b"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
        assert not np.array_equal(getattr(a, name), getattr(c, name))
    h = hashlib.sha256(a.gate_q.tobytes() + a.down_s.tobytes()).hexdigest()
    assert h == hashlib.sha256(b.gate_q.tobytes() + b.down_s.tobytes()).hexdigest()
    assert np.array_equal(make_x(sh, 3, seed=1), make_x(sh, 3, seed=1))
    assert np.array_equal(make_logits(sh, 3, seed=1), make_logits(sh, 3, seed=1))


def test_expert_bytes_do_not_depend_on_selection():
    sh = SHAPES["toy"]
    full = make_layer(sh, seed=5)
    part = make_layer(sh, experts=[2, 6], seed=5)
    for name in ("gate_q", "gate_s", "up_q", "down_q", "down_b"):
        assert np.array_equal(getattr(full, name)[[2, 6]], getattr(part, name)[[2, 6]])
    assert np.isnan(part.gate_s[0].view(np.float16).astype(np.float32)).all()


def test_quantizer_round_trip_error_is_within_half_step():
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    q, s, b = quantize_affine4(w)
    deq = bf.dequant_dense(q, s, b)
    step = np.repeat(s.view(np.float16).astype(np.float64), 64, axis=1)
    # fp16 rounding of scale and bias adds a little over half a step
    assert np.all(np.abs(deq - w) <= 0.5 * step + 1e-4)


# ------------------------------------------------------------- conversions
def test_f16_decode_exhaustive_against_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    ours = np.array([oracle.f16_to_f64(int(v)) for v in bits[::7]])
    r = ref[::7]
    finite = np.isfinite(r)
    assert np.array_equal(ours[finite], r[finite])
    assert np.array_equal(np.isnan(ours), np.isnan(r))


def test_bf16_rounding_is_single_step_ties_to_even():
    with open(os.path.join(GOLDEN, "bf16_rounding.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        v = float.fromhex(c["value"])
        assert oracle.f64_to_bf16(v) == int(c["bf16"], 16), c


def test_bf16_rounding_matches_fp32_path_off_ties():
    # For values exactly representable in fp32 no double rounding can occur,
    # so fp64 -> bf16 must equal the integer-trick fp32 -> bf16 rounding.
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ours = oracle.round_bf16(v.astype(np.float64))
    assert np.array_equal(ours, bf16_bits_from_f32(v))


# ----------------------------------------------------------------- dequant
def test_nibble_order_low_nibble_first():
    with open(os.path.join(GOLDEN, "nibble_order.json")) as f:
        fx = json.load(f)
    q = np.zeros((1, 8), np.uint32)
    q[0, : len(fx["words"])] = [int(w, 16) for w in fx["words"]]
    one, zero = np.uint16(0x3C00), np.uint16(0)
    s = np.full((1, 1), one, np.uint16)
    b = np.full((1, 1), zero, np.uint16)
    w = oracle.dequant(q, s, b)[0]
    assert list(w[: len(fx["elements"])].astype(int)) == fx["elements"]


def test_dequant_against_hex_digits_and_groups():
    rng = np.random.default_rng(2)
    rows, cols = 3, 256
    q = rng.integers(0, 2 ** 32, (rows, cols // 8), dtype=np.uint64).astype(np.uint32)
    s = np.float16(rng.uniform(0.001, 0.1, (rows, cols // 64))).view(np.uint16)
    b = np.float16(rng.uniform(-1, 1, (rows, cols // 64))).view(np.uint16)
    w = oracle.dequant(q, s, b)
    for r in range(rows):
        for c in range(0, cols, 5):
            digit = int(("%08x" % q[r, c // 8])[7 - (c % 8)], 16)
            exp = float(s[r, c // 64].view(np.float16)) * digit + float(b[r, c // 64].view(np.float16))
            assert w[r, c] == exp
    assert np.array_equal(w, bf.dequant_dense(q, s, b))


# ------------------------------------------------------------------- route
def test_route_k1_weight_is_one_and_argmax():
    lg = make_logits(SHAPES["decode"], 6, seed=3)
    idx, w = oracle.route_topk(lg, 1)
    assert np.array_equal(idx[:, 0], np.argmax(lg, axis=1))
    assert np.all(w == 1.0)


def test_route_k_equals_e_is_full_softmax():
    lg = make_logits(SHAPES["toy"], 5, seed=4)
    idx, w = oracle.route_topk(lg, 8)
    full = softmax(lg.astype(np.float64), axis=1)
    got = np.zeros_like(full)
    for t in range(5):
        got[t, idx[t]] = w[t]
    assert np.allclose(got, full, rtol=1e-14, atol=1e-16)


def test_route_ties_go_to_lower_id():
    lg = np.zeros((2, 8), np.float32)
    lg[1, [5, 2, 7]] = 1.0
    idx, w = oracle.route_topk(lg, 4)
    assert idx[0].tolist() == [0, 1, 2, 3]
    assert idx[1].tolist() == [2, 5, 7, 0]
    assert np.allclose(w[0], 0.25, rtol=0, atol=1e-16)


@pytest.mark.parametrize("E,k,B", [(8, 2, 3), (128, 8, 16), (256, 6, 4), (64, 16, 5)])
def test_route_against_bruteforce_and_invariants(E, k, B):
    sh = Shape("r", 91, 64, 64, E, k, "f32")
    lg = make_logits(sh, B, seed=E + k)
    idx, w = oracle.route_topk(lg, k)
    bidx, bw = bf.route(lg, k)
    assert np.array_equal(idx, bidx)
    assert np.allclose(w, bw, rtol=1e-13, atol=1e-16)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)
    for t in range(B):
        assert len(set(idx[t].tolist())) == k


# -------------------------------------------------------------------- plan
@pytest.mark.parametrize("regime,B", [("normal", 1), ("normal", 7), ("sharing", 8), ("disjoint", 4),
                                      ("same", 5), ("zipf", 32)])
def test_plan_against_bruteforce_and_invariants(regime, B):
    sh = SHAPES["decode"]
    idx, _ = oracle.route_topk(make_logits(sh, B, regime=regime, seed=11), sh.top_k)
    p = oracle.plan(idx, sh.n_experts)
    q = bf.plan(idx, sh.n_experts)
    for key in ("counts", "offsets", "sorted_slots", "unique_experts"):
        assert np.array_equal(p[key], q[key]), key
    assert p["n_unique"] == q["n_unique"]
    n = B * sh.top_k
    assert sorted(p["sorted_slots"].tolist()) == list(range(n))
    assert p["counts"].sum() == n and p["offsets"][-1] == n
    flat = idx.ravel()
    for e in range(sh.n_experts):
        lst = p["sorted_slots"][p["offsets"][e]:p["offsets"][e + 1]]
        assert np.all(flat[lst] == e) and np.all(np.diff(lst) > 0)
    assert p["n_unique"] <= min(sh.n_experts, n)
    if regime == "same":
        assert p["n_unique"] == sh.top_k
    if regime == "disjoint":
        assert p["n_unique"] == min(n, sh.n_experts)


def test_plan_empty_batch():
    p = oracle.plan(np.zeros((0, 8), np.int32), 16)
    assert p["n_unique"] == 0 and p["counts"].sum() == 0
    assert np.all(p["unique_experts"] == -1) and np.all(p["offsets"] == 0)


# ------------------------------------------------------------ expert block
CASES = [
    dict(H=64, F=64, E=1, k=1, act="f32", B=1),
    dict(H=128, F=64, E=2, k=1, act="bf16", B=2),
    dict(H=256, F=128, E=4, k=2, act="f32", B=3),
    dict(H=128, F=128, E=8, k=4, act="bf16", B=5),
    dict(H=256, F=64, E=16, k=4, act="bf16", B=2),
    dict(H=64, F=128, E=8, k=2, act="f32", B=1, sidecar=True, clamp=0.5),
    dict(H=128, F=64, E=4, k=3, act="bf16", B=4, sidecar=True, clamp=10.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "H{H}F{F}E{E}k{k}{act}B{B}".format(**c))
def test_decode_against_dense_bruteforce(case):
    sh = tiny(case["H"], case["F"], case["E"], case["k"], case["act"],
              case.get("sidecar", False), case.get("clamp", 0.0))
    L = make_layer(sh, seed=7)
    x = make_x(sh, case["B"], seed=7, scale=4.0 if case.get("clamp") == 0.5 else 1.0)
    lg = make_logits(sh, case["B"], seed=7)
    idx, w = oracle.route_topk(lg, sh.top_k)
    out = oracle.decode_step(L, x, idx, w)
    bidx, bw, bout = bf.moe_dense(L, x, lg)
    assert np.array_equal(idx, bidx)
    assert rel_l2(out, bout) <= 1e-12


def test_toy_config_against_bruteforce():
    sh = SHAPES["toy"]
    L = make_layer(sh, seed=0)
    x = make_x(sh, 1, seed=0)
    lg = make_logits(sh, 1, seed=0)
    idx, w = oracle.route_topk(lg, sh.top_k)
    out = oracle.decode_step(L, x, idx, w)
    _, _, bout = bf.moe_dense(L, x, lg)
    assert rel_l2(out, bout) <= 1e-12


def _onehot_layer(H=128, F=64, seed=0):
    """Gate weights random nibbles with s=1, b=0; up q=0, b=1 (u = sum x)."""
    sh = tiny(H, F, 1, 1, "f32", cfg=92)
    L = make_layer(sh, seed=seed)
    rng = np.random.default_rng(seed)
    L.gate_q[:] = rng.integers(0, 2 ** 32, L.gate_q.shape, dtype=np.uint64).astype(np.uint32)
    L.gate_s[:] = 0x3C00
    L.gate_b[:] = 0
    L.up_q[:] = 0
    L.up_s[:] = 0x3C00
    L.up_b[:] = 0x3C00
    return sh, L


def test_onehot_x_reads_the_right_nibble():
    sh, L = _onehot_layer()
    silu = lambda v: v / (1.0 + math.exp(-v))  # noqa: E731
    for c in (0, 1, 7, 8, 63, 64, 65, 127):
        x = np.zeros((1, sh.hidden), np.float32)
        x[0, c] = 1.0
        _, h = oracle.decode_step(L, x, np.zeros((1, 1), np.int32), np.ones((1, 1)), want_h=True)
        for n in range(sh.dff):
            digit = int(("%08x" % L.gate_q[0, n, c // 8])[7 - (c % 8)], 16)
            assert h[0, n] == silu(float(digit)) * 1.0, (c, n)


def test_zero_nibbles_give_bias_times_group_sums():
    sh = tiny(256, 64, 1, 1, "f32", cfg=93)
    L = make_layer(sh, seed=1)
    rng = np.random.default_rng(1)
    for q, s, b in ((L.gate_q, L.gate_s, L.gate_b), (L.up_q, L.up_s, L.up_b)):
        q[:] = 0
        s[:] = np.float16(rng.uniform(0.01, 0.1, s.shape)).view(np.uint16)
        b[:] = np.float16(rng.uniform(-0.5, 0.5, b.shape)).view(np.uint16)
    x = make_x(sh, 1, seed=1)
    _, h = oracle.decode_step(L, x, np.zeros((1, 1), np.int32), np.ones((1, 1)), want_h=True)
    X = x.astype(np.float64).reshape(4, 64).sum(axis=1)
    g = L.gate_b[0].view(np.float16).astype(np.float64) @ X
    u = L.up_b[0].view(np.float16).astype(np.float64) @ X
    ref = g / (1 + np.exp(-g)) * u
    assert np.allclose(h[0], ref, rtol=1e-13, atol=0)


def test_single_expert_is_plain_quantized_swiglu_mlp():
    sh = tiny(256, 128, 1, 1, "bf16", cfg=94)
    L = make_layer(sh, seed=2)
    x = make_x(sh, 3, seed=2)
    out = oracle.decode_step(L, x, np.zeros((3, 1), np.int32), np.ones((3, 1)))
    X = f32_from_bf16_bits(x).astype(np.float64)
    Wg = bf.dequant_dense(L.gate_q[0], L.gate_s[0], L.gate_b[0])
    Wu = bf.dequant_dense(L.up_q[0], L.up_s[0], L.up_b[0])
    Wd = bf.dequant_dense(L.down_q[0], L.down_s[0], L.down_b[0])
    g = np.dot(X, Wg.T)
    u = np.dot(X, Wu.T)
    ref = np.dot(g / (1 + np.exp(-g)) * u, Wd.T)
    assert rel_l2(out, ref) <= 1e-13


def test_sidecar_applies_before_clamp():
    # sigma = 2 must equal doubling gate/up scales and biases, bitwise, with
    # the clamp active; clamping first would give 2*clip(g) != clip(2g).
    sh = tiny(128, 64, 2, 1, "f32", sidecar=True, clamp=0.75, cfg=95)
    L = make_layer(sh, seed=3)
    L.sidecar = np.array([2.0, 2.0], np.float32)
    x = make_x(sh, 2, seed=3, scale=3.0)
    idx = np.array([[0], [1]], np.int32)
    w = np.ones((2, 1))
    a, ha = oracle.decode_step(L, x, idx, w, want_h=True)
    L2 = make_layer(sh, seed=3)
    L2.sidecar = None
    for arr in (L2.gate_s, L2.gate_b, L2.up_s, L2.up_b):
        arr[:] = (arr.view(np.float16) * np.float16(2)).view(np.uint16)
    b, hb = oracle.decode_step(L2, x, idx, w, want_h=True)
    assert np.array_equal(a, b)
    # the clamp really fires in this case
    g_lim = 0.75 / (1 + math.exp(-0.75)) * 0.75
    assert np.isclose(np.abs(ha).max(), g_lim, rtol=1e-15)


def test_forced_clamp_matches_bruteforce():
    sh = tiny(256, 64, 4, 2, "bf16", sidecar=True, clamp=10.0, cfg=96)
    L = make_layer(sh, seed=4, std=0.2)
    x = make_x(sh, 3, seed=4, scale=8.0)
    lg = make_logits(sh, 3, seed=4)
    idx, w = oracle.route_topk(lg, sh.top_k)
    out, h = oracle.decode_step(L, x, idx, w, want_h=True)
    _, _, bout = bf.moe_dense(L, x, lg)
    assert rel_l2(out, bout) <= 1e-12
    lim = 10.0 / (1 + math.exp(-10.0)) * 10.0
    assert np.abs(h).max() <= lim * (1 + 1e-15)
    assert np.isclose(np.abs(h).max(), lim, rtol=1e-15)  # clamp reached


def test_doubling_down_scale_and_bias_doubles_output_exactly():
    sh = tiny(128, 128, 4, 2, "bf16", cfg=97)
    L = make_layer(sh, seed=5)
    x = make_x(sh, 2, seed=5)
    idx, w = oracle.route_topk(make_logits(sh, 2, seed=5), 2)
    a = oracle.decode_step(L, x, idx, w)
    for arr in (L.down_s, L.down_b):
        arr[:] = (arr.view(np.float16) * np.float16(2)).view(np.uint16)
    b = oracle.decode_step(L, x, idx, w)
    assert np.array_equal(b, 2 * a)


def test_combine_weights_are_linear():
    sh = tiny(128, 64, 4, 2, "f32", cfg=98)
    L = make_layer(sh, seed=6)
    x = make_x(sh, 1, seed=6)
    idx = np.array([[1, 3]], np.int32)
    _, y = oracle.decode_step(L, x, idx, np.array([[0.25, 0.75]]), want_y=True)
    out = oracle.decode_step(L, x, idx, np.array([[0.25, 0.75]]))
    assert np.allclose(out[0], 0.25 * y[0] + 0.75 * y[1], rtol=1e-15, atol=1e-300)


# -------------------------------------------------------------- invariants
def test_batch_invariance_permutation_and_duplicates():
    sh = tiny(256, 128, 8, 2, "bf16", cfg=99)
    L = make_layer(sh, seed=8)
    x = make_x(sh, 5, seed=8)
    lg = make_logits(sh, 5, seed=8)
    idx, w = oracle.route_topk(lg, 2)
    full = oracle.decode_step(L, x, idx, w)
    for t in range(5):
        one = oracle.decode_step(L, x[t:t + 1], idx[t:t + 1], w[t:t + 1])
        assert np.array_equal(one[0], full[t])
    perm = np.array([3, 0, 4, 1, 2])
    pidx, pw = oracle.route_topk(lg[perm], 2)
    pout = oracle.decode_step(L, x[perm], pidx, pw)
    assert np.array_equal(pout, full[perm])
    dup = np.repeat(x[2:3], 4, axis=0)
    didx, dw = oracle.route_topk(np.repeat(lg[2:3], 4, axis=0), 2)
    assert oracle.plan(didx, 8)["n_unique"] == 2
    dout = oracle.decode_step(L, dup, didx, dw)
    assert np.all(dout == dout[0:1])


def test_expert_relabelling_invariance():
    sh = tiny(128, 64, 8, 3, "bf16", cfg=100)
    L = make_layer(sh, seed=9)
    x = make_x(sh, 3, seed=9)
    lg = make_logits(sh, 3, seed=9)
    idx, w = oracle.route_topk(lg, 3)
    ref = oracle.decode_step(L, x, idx, w)
    perm = np.random.default_rng(9).permutation(8)  # new id i holds old expert perm[i]
    for name in ("gate_q", "gate_s", "gate_b", "up_q", "up_s", "up_b", "down_q", "down_s", "down_b"):
        setattr(L, name, np.ascontiguousarray(getattr(L, name)[perm]))
    pidx, pw = oracle.route_topk(np.ascontiguousarray(lg[:, perm]), 3)
    assert np.array_equal(perm[pidx], idx)
    assert np.array_equal(oracle.decode_step(L, x, pidx, pw), ref)


def test_poisoned_expert_shows_up_as_nan():
    sh = tiny(128, 64, 4, 1, "f32", cfg=101)
    L = make_layer(sh, experts=[0, 1, 2], seed=10)
    x = make_x(sh, 1, seed=10)
    assert np.isfinite(oracle.decode_step(L, x, np.array([[1]], np.int32), np.ones((1, 1)))).all()
    assert np.isnan(oracle.decode_step(L, x, np.array([[3]], np.int32), np.ones((1, 1)))).all()


def test_output_rounding_error_is_what_bf16_allows():
    sh = SHAPES["toy"]
    L = make_layer(sh, seed=12)
    sh16 = Shape("toy16", 0, 256, 128, 8, 2, "bf16")
    L.shape = sh16
    x = make_x(sh16, 4, seed=12)
    idx, w = oracle.route_topk(make_logits(sh16, 4, seed=12), 2)
    out = oracle.decode_step(L, x, idx, w)
    r = rel_l2(oracle.bf16_to_f64(oracle.round_bf16(out)), out)
    # RNE to 8 significant bits: per element |err| <= 2^-9 relative
    assert 5e-4 < r < 2.26e-3
    err = np.abs(oracle.bf16_to_f64(oracle.round_bf16(out)) - out)
    assert np.all(err <= np.abs(out) * 2.0 ** -8)


def test_residual_step_mirrors_two_roundings():
    rng = np.random.default_rng(13)
    x = bf16_bits_from_f32(rng.standard_normal(4096).astype(np.float32))
    out = rng.standard_normal(4096) * 0.1
    nxt = oracle.residual_bf16(x, out)
    o16 = f32_from_bf16_bits(oracle.round_bf16(out))
    ref = bf16_bits_from_f32((f32_from_bf16_bits(x) + o16).astype(np.float32))
    assert np.array_equal(nxt, ref)


# ------------------------------------------------------ router projection
# Pins of oracle.router_logits (the step in front of the router): an
# independent numpy product, one-hot and single-entry closed forms, and the
# fp32 / bf16 activation paths agreeing on bf16-representable values.

def test_router_logits_match_an_independent_float64_product():
    sh = Shape("rp", 120, 384, 64, 40, 4, "bf16")
    x = make_x(sh, 5, seed=30)
    wr = make_router(sh, seed=30)
    got = oracle.router_logits(x, wr)
    ref = f32_from_bf16_bits(x).astype(np.float64) @ f32_from_bf16_bits(wr).astype(np.float64).T
    assert got.shape == (5, 40)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    assert 0.5 < got.std() < 2.0  # unit-scale logits by construction


def test_router_logits_one_hot_activation_reads_a_weight_column():
    sh = Shape("rp1", 121, 128, 64, 12, 2, "bf16")
    wr = make_router(sh, seed=31)
    x = np.zeros((3, 128), np.uint16)
    for t, c in enumerate((0, 77, 127)):
        x[t, c] = 0x3F80  # bf16 1.0
    got = oracle.router_logits(x, wr)
    for t, c in enumerate((0, 77, 127)):
        assert np.array_equal(got[t], f32_from_bf16_bits(wr[:, c]).astype(np.float64))


def test_router_logits_single_entry_rows_scale_one_activation():
    rng = np.random.default_rng(32)
    x = rng.standard_normal((4, 96)).astype(np.float32)
    wr = np.zeros((6, 96), np.uint16)
    cols = [3, 3, 50, 95, 0, 17]
    pows = [0, 1, -2, 3, -1, 2]
    for e, (c, p) in enumerate(zip(cols, pows)):
        wr[e, c] = bf16_bits_from_f32(np.array([2.0 ** p], np.float32))[0]
    got = oracle.router_logits(x, wr)
    for e, (c, p) in enumerate(zip(cols, pows)):
        assert np.array_equal(got[:, e], x[:, c].astype(np.float64) * 2.0 ** p)


def test_router_logits_fp32_and_bf16_activations_agree():
    sh = Shape("rp2", 122, 256, 64, 16, 2, "bf16")
    xb = make_x(sh, 3, seed=33)
    wr = make_router(sh, seed=33)
    assert np.array_equal(oracle.router_logits(xb, wr), oracle.router_logits(f32_from_bf16_bits(xb), wr))


# ---------------------------------------------- GeGLU and the down sidecar
# GeGLU reads GELU in the tanh form.  It is pinned without retyping it: it
# stays within 5e-4 of the exact x * Phi(x) (scipy's normal CDF), it is
# 0 at 0, and with the same weights its h differs from SwiGLU's exactly as
# GELU(g) / SiLU(g) does, per element.

def _geglu_layer(down_sidecar=False, activation="geglu", cfg=140):
    sh = Shape("gg", cfg, 128, 64, 3, 1, "f32", activation=activation, down_sidecar=down_sidecar)
    return sh, make_layer(sh, seed=41)


def test_geglu_h_is_the_normal_cdf_gelu_within_the_tanh_form_error():
    from scipy.special import ndtr
    sh, L = _geglu_layer()
    x = make_x(sh, 1, seed=41) * np.float32(40.0)  # spread g over about +-6
    idx = np.array([[1]], np.int32)
    _, h = oracle.decode_step(L, x, idx, np.ones((1, 1)), want_h=True)
    q = bf.dequant_dense(L.gate_q[1], L.gate_s[1], L.gate_b[1])
    uq = bf.dequant_dense(L.up_q[1], L.up_s[1], L.up_b[1])
    g = q @ x[0].astype(np.float64)
    u = uq @ x[0].astype(np.float64)
    assert np.abs(g).max() > 3.0
    exact = g * ndtr(g) * u
    assert np.all(np.abs(h[0] - exact) <= 5e-4 * np.abs(u) + 1e-15)
    assert np.abs(h[0] - exact).max() > 0  # the tanh form, not the exact one


def test_geglu_tanh_form_matches_an_independent_implementation():
    # PyTorch's own tanh-form GELU (fp64, CPU) pins both constants of the
    # form to rounding level: a wrong cubic coefficient or sqrt(2/pi) moves
    # h far more than 1e-12 of its largest value at |g| up to ~6.  (Deep in
    # the negative tail 1 + tanh cancels, and the two tanh implementations
    # leave different residues of order 1e-16 there.)
    import torch
    sh, L = _geglu_layer()
    x = make_x(sh, 1, seed=44) * np.float32(40.0)
    idx = np.array([[2]], np.int32)
    _, h = oracle.decode_step(L, x, idx, np.ones((1, 1)), want_h=True)
    g = bf.dequant_dense(L.gate_q[2], L.gate_s[2], L.gate_b[2]) @ x[0].astype(np.float64)
    u = bf.dequant_dense(L.up_q[2], L.up_s[2], L.up_b[2]) @ x[0].astype(np.float64)
    assert np.abs(g).max() > 3.0
    ref = torch.nn.functional.gelu(torch.from_numpy(g), approximate="tanh").numpy() * u
    assert np.allclose(h[0], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_geglu_and_swiglu_differ_only_in_the_gate_function():
    sh_g, Lg = _geglu_layer()
    _, Ls = _geglu_layer(activation="swiglu")
    x = make_x(sh_g, 2, seed=42)
    idx = np.array([[0], [2]], np.int32)
    _, hg = oracle.decode_step(Lg, x, idx, np.ones((2, 1)), want_h=True)
    _, hs = oracle.decode_step(Ls, x, idx, np.ones((2, 1)), want_h=True)
    for t, e in enumerate((0, 2)):
        g = bf.dequant_dense(Lg.gate_q[e], Lg.gate_s[e], Lg.gate_b[e]) @ x[t].astype(np.float64)
        silu = g / (1.0 + np.exp(-g))
        nz = np.abs(silu) > 1e-30
        # h_geglu / h_swiglu = gelu(g) / silu(g); both sides from the same u
        ratio = hg[t][nz] / hs[t][nz]
        from scipy.special import ndtr
        assert np.allclose(ratio, g[nz] * ndtr(g[nz]) / silu[nz], rtol=2e-2, atol=1e-3)


def test_down_sidecar_scales_each_expert_output():
    sh, L = _geglu_layer(down_sidecar=True, activation="swiglu")
    x = make_x(sh, 2, seed=43)
    idx = np.array([[0], [2]], np.int32)
    w = np.array([[1.0], [1.0]])
    L.down_sidecar = np.array([2.0, 0.5, 0.25], np.float32)
    out, y = oracle.decode_step(L, x, idx, w, want_y=True)
    dsc = L.down_sidecar
    L.down_sidecar = None
    out0, y0 = oracle.decode_step(L, x, idx, w, want_y=True)
    assert np.array_equal(y[0], 2.0 * y0[0]) and np.array_equal(y[1], 0.25 * y0[1])
    assert np.array_equal(out, np.stack([2.0 * out0[0], 0.25 * out0[1]]))
    assert dsc is not None


# ------------------------------------------------ other widths and group sizes
# Elements of `bits` bits in a little-endian bit stream per row, fp16 scale
# and bias per `group` inputs (page "perf(moe): batched decode scales 1.55x
# against 3.25x on dense", Implementation Notes: the fused kernel is
# templated on bits and group size; 4-bit gate/up with 6-bit down).
WIDTHS = [(4, 32), (4, 128), (6, 32), (6, 64), (6, 128), (8, 32), (8, 64), (8, 128)]


def _recode(q_words, bits_from, bits_to):
    """Re-pack a matrix's element codes at another width (codes must fit)."""
    codes = bf.unpack_bigint(q_words.reshape(-1, q_words.shape[-1]), bits_from).astype(np.uint32)
    assert codes.max(initial=0) < 2 ** bits_to
    from moe_workloads import pack_bits
    return pack_bits(codes, bits_to).reshape(*q_words.shape[:-1], -1)


@pytest.mark.parametrize("bits,group", WIDTHS)
def test_width_dequant_against_bigint_reading(bits, group):
    rng = np.random.default_rng(bits * 1000 + group)
    rows, cols = 3, 256
    q = rng.integers(0, 2 ** 32, (rows, cols * bits // 32), dtype=np.uint64).astype(np.uint32)
    s = np.float16(rng.uniform(0.001, 0.1, (rows, cols // group))).view(np.uint16)
    b = np.float16(rng.uniform(-1, 1, (rows, cols // group))).view(np.uint16)
    w = oracle.dequant(q, s, b, bits, group)
    assert np.array_equal(w, bf.dequant_dense(q, s, b, bits, group))
    # spot check against per-element integer arithmetic on the row's words
    for r in range(rows):
        big = sum(int(v) << (32 * i) for i, v in enumerate(q[r]))
        for c in range(0, cols, 7):
            code = (big >> (bits * c)) & ((1 << bits) - 1)
            exp = float(s[r, c // group].view(np.float16)) * code + float(b[r, c // group].view(np.float16))
            assert w[r, c] == exp


@pytest.mark.parametrize("c", range(16))
def test_six_bit_one_hot_elements_straddle_words(c):
    """Sixteen 6-bit elements fill three words; element c = 63 alone sets
    stream bits 6c..6c+5, which for c = 5 and 10 cross a word boundary."""
    big = 63 << (6 * c)
    q = np.array([[(big >> (32 * i)) & 0xFFFFFFFF for i in range(3)]], np.uint32)
    s = np.array([[0x3C00]], np.uint16)   # 1.0
    b = np.array([[0]], np.uint16)
    q = np.concatenate([q, np.zeros((1, 9), np.uint32)], axis=1)  # 64 elements, one group
    w = oracle.dequant(q, s, b, 6, 64)[0]
    want = np.zeros(64)
    want[c] = 63
    assert np.array_equal(w, want)
    if c in (5, 10):
        assert q[0, c * 6 // 32] != 0 and q[0, (c * 6 + 5) // 32] != 0


def _width_shape(bits, down_bits, group, act="f32", cfg=95):
    return Shape(f"w{bits}{down_bits}g{group}", cfg, 256, 128, 4, 2, act, bits=bits, down_bits=down_bits,
                 group_size=group)


@pytest.mark.parametrize("bits,down_bits,group", [(8, 8, 64), (4, 6, 64), (6, 6, 32), (8, 4, 128), (4, 4, 32)])
def test_width_layer_against_bruteforce(bits, down_bits, group):
    sh = _width_shape(bits, down_bits, group)
    L = make_layer(sh, seed=bits + down_bits)
    x = make_x(sh, 3, seed=1)
    lg = make_logits(sh, 3, seed=1)
    idx, w = oracle.route_topk(lg, sh.top_k)
    out = oracle.decode_step(L, x, idx, w)
    _, _, bout = bf.moe_dense(L, x, lg)
    assert rel_l2(out, bout) <= 1e-12


def test_four_bit_codes_recoded_at_six_and_eight_bits_give_the_same_output():
    """The same codes stored at another width are the same matrix: the
    oracle's output is bitwise unchanged, with gate/up and down recoded
    separately (so a swapped width of the two projections shows)."""
    sh4 = _width_shape(4, 4, 64, act="bf16")
    L4 = make_layer(sh4, seed=5)
    x = make_x(sh4, 3, seed=5)
    idx, w = oracle.route_topk(make_logits(sh4, 3, seed=5), sh4.top_k)
    ref = oracle.decode_step(L4, x, idx, w)
    for nb, nd in ((8, 4), (4, 6), (6, 8), (8, 8)):
        import dataclasses
        L = dataclasses.replace(L4, shape=dataclasses.replace(sh4, bits=nb, down_bits=nd))
        L.gate_q, L.up_q = _recode(L4.gate_q, 4, nb), _recode(L4.up_q, 4, nb)
        L.down_q = _recode(L4.down_q, 4, nd)
        assert np.array_equal(oracle.decode_step(L, x, idx, w), ref), (nb, nd)


def test_group_split_with_repeated_scales_gives_the_same_output():
    """A layer of groups of 128 equals the same codes with each group's scale
    and bias repeated over two groups of 64, and over four of 32."""
    import dataclasses
    sh = _width_shape(6, 8, 128)
    L = make_layer(sh, seed=7)
    x = make_x(sh, 2, seed=7)
    idx, w = oracle.route_topk(make_logits(sh, 2, seed=7), sh.top_k)
    ref = oracle.decode_step(L, x, idx, w)
    for g in (64, 32):
        r = 128 // g
        L2 = dataclasses.replace(L, shape=dataclasses.replace(sh, group_size=g))
        for n in ("gate_s", "gate_b", "up_s", "up_b", "down_s", "down_b"):
            setattr(L2, n, np.repeat(getattr(L, n), r, axis=-1))
        assert np.array_equal(oracle.decode_step(L2, x, idx, w), ref), g
    # and a different scale in one half-group does change the output
    L3 = dataclasses.replace(L, shape=dataclasses.replace(sh, group_size=64))
    for n in ("gate_s", "gate_b", "up_s", "up_b", "down_s", "down_b"):
        setattr(L3, n, np.repeat(getattr(L, n), 2, axis=-1))
    L3.down_s = L3.down_s.copy()
    L3.down_s[..., 1::2] = (L3.down_s[..., 1::2].view(np.float16) * np.float16(2)).view(np.uint16)
    assert not np.allclose(oracle.decode_step(L3, x, idx, w), ref)


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_top_code_reads_the_full_width(bits):
    """All-ones codes (2^bits - 1) with scale 1, bias 0 and x = 1: every
    gate/up pre-activation equals hidden * (2^bits - 1)."""
    sh = Shape("top", 96, 64, 64, 1, 1, "f32", bits=bits, down_bits=bits, group_size=32)
    L = make_layer(sh, seed=0)
    for n in ("gate", "up", "down"):
        getattr(L, n + "_q")[:] = 0xFFFFFFFF
        getattr(L, n + "_s")[:] = 0x3C00
        getattr(L, n + "_b")[:] = 0
    x = np.ones((1, 64), np.float32)
    _, h = oracle.decode_step(L, x, np.zeros((1, 1), np.int32), np.ones((1, 1)), want_h=True)
    g = 64.0 * (2 ** bits - 1)
    assert np.allclose(h, g / (1 + np.exp(-g)) * g, rtol=1e-15)


def test_workload_packer_and_torch_quantiser_agree_at_every_width():
    import torch
    from moe_workloads import quantize_affine
    from moe_workloads.gen import quantize_affine_torch
    rng = np.random.default_rng(3)
    for bits, group in WIDTHS + [(4, 64)]:
        w = (rng.standard_normal((2, 4, 256)) * 0.02).astype(np.float32)
        tq, ts, tb = quantize_affine_torch(torch.from_numpy(w), bits, group)
        for n in range(2):
            q, s, b = quantize_affine(w[n], bits, group)
            assert np.array_equal(tq[n].numpy().view(np.uint32), q)
            assert np.array_equal(ts[n].numpy().view(np.uint16), s)
            assert np.array_equal(tb[n].numpy().view(np.uint16), b)
            codes = bf.unpack_bigint(q, bits)
            assert codes.max() <= 2 ** bits - 1
