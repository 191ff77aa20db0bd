"""Helpers of the GPU parity tests: move seeded inputs to the device, run the
three C-ABI calls, bring results back as numpy, and compare with the oracle.
Inputs come from moe_workloads only; expected values come from oracle/ only.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import quantized_expert_gemv_moe_amd as moe
from moe_workloads import make_layer
from oracle import oracle

# Output gate: relative L2 against the unrounded fp64 oracle (fp32
# accumulation, bf16 I/O).
REL_L2_GATE = 2e-3
# Diagnostic: relative L2 against the oracle rounded once to bf16.  A
# faithful fp32 pipeline differs from it only where its ~2e-6 relative
# pre-rounding error crosses a bf16 rounding boundary: a fraction
# p ~ 2 * 2e-6 / 2^-8 ~ 1e-3 of the elements moves by one bf16 ulp (2^-8
# relative), so this distance is ~sqrt(p) * 2^-8 ~ 1.5e-4 on average and,
# the flips being few in a small output, up to ~3e-4.  Rounding h, the
# weights or the per-expert outputs to bf16 scores 2e-3 or more.  Largest
# seen over every case of the suite: 2.4e-4 (4 sampled tokens of one stack
# layer, where few flips weigh most); median 2.7e-5.
REL_L2_DIAG = 3e-4
# Intermediate h (fp32 on both sides): the bf16 nibble dot with its +128
# offset carries ~2e-6 relative error; exact fp32 paths ~1e-7.
REL_L2_H = 1e-5
# Router weights: fp32 exp/divide against fp64.
W_ABS = 1e-6


def record(tag: str, **vals):
    """Appends one case's figures to the JSON-lines file named by
    MOE_PARITY_LOG, if set (pytest keeps passing tests' prints to itself)."""
    import json
    import os

    path = os.environ.get("MOE_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": tag, **vals}) + "\n")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def dev_x(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return oracle.bf16_to_f64(a)
    return a.astype(np.float64)


class DeviceRun:
    """One layer step on the GPU through the C ABI, results as numpy."""

    def __init__(self, layer_np, x: np.ndarray, logits: np.ndarray, residual: np.ndarray = None,
                 dl=None, max_tokens=None, cols: bool = False):
        sh = layer_np.shape
        if dl is None:
            dl = moe.DeviceLayer.from_host(layer_np)
            if cols:
                dl = dl.pack_down()
        self.dl = dl
        B = x.shape[0]
        self.B = B
        mt = max(max_tokens or B, 1)
        self.plan = moe.Plan.allocate(sh.n_experts, mt * sh.top_k)
        self.ws = moe.alloc_workspace(self.dl, mt)
        lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
        xt = dev_x(x)
        res = None if residual is None else dev_x(residual)
        self.out_t, idx, w, _ = moe.decode_layer(self.dl, xt, lg, plan=self.plan, workspace=self.ws,
                                                 residual=res)
        torch.cuda.synchronize()
        self.idx = idx.cpu().numpy()
        self.w = w.cpu().numpy()
        self.out = host_bits(self.out_t)
        n = B * sh.top_k
        self.plan_np = dict(
            counts=self.plan.counts.cpu().numpy(), offsets=self.plan.offsets.cpu().numpy(),
            sorted_slots=self.plan.sorted_slots[:n].cpu().numpy(),
            unique_experts=self.plan.unique_experts.cpu().numpy(),
            n_unique=int(self.plan.n_unique.cpu().numpy()[0]), work=self.plan.work.cpu().numpy())
        # h sits at the start of the workspace: [slots][dff] fp32
        self.h = self.ws[: n * sh.dff * 4].view(torch.float32).view(n, sh.dff).cpu().numpy()


def layer_for(shape, logits, layer=0, seed=0, std=0.02):
    """Only the experts the routing selects are drawn; the rest are poisoned."""
    idx, _ = oracle.route_topk(logits, shape.top_k)
    return make_layer(shape, layer=layer, experts=np.unique(idx), seed=seed, std=std)


def check_against_oracle(L, x, logits, run: DeviceRun, tag: str, diag=True):
    sh = L.shape
    idx, w = oracle.route_topk(logits, sh.top_k)
    assert np.array_equal(run.idx, idx), f"{tag}: router indices differ"
    dw = float(np.abs(run.w - w).max()) if w.size else 0.0
    assert dw <= W_ABS, f"{tag}: router weights off by {dw}"
    p = oracle.plan(idx, sh.n_experts)
    for k in ("counts", "offsets", "sorted_slots", "unique_experts"):
        assert np.array_equal(run.plan_np[k], p[k]), f"{tag}: plan {k} differs"
    assert run.plan_np["n_unique"] == p["n_unique"]
    out64, h64 = oracle.decode_step(L, x, idx, w, want_h=True)
    eh = rel_l2(run.h, h64)
    got = as_f64(run.out)
    gate = rel_l2(got, out64)
    if run.out.dtype == np.uint16:
        ref16 = oracle.bf16_to_f64(oracle.round_bf16(out64))
    else:
        ref16 = oracle.round_f32(out64).astype(np.float64)
    dg = rel_l2(got, ref16)
    log(f"[parity] {tag}: n_unique={p['n_unique']} h_rel={eh:.3g} out_rel={gate:.3g} diag={dg:.3g}")
    record(tag, n_unique=int(p["n_unique"]), h=eh, out=gate, diag=dg)
    assert np.isfinite(got).all(), f"{tag}: non-finite output"
    assert eh <= REL_L2_H, f"{tag}: h rel L2 {eh}"
    assert gate <= REL_L2_GATE, f"{tag}: output rel L2 {gate}"
    if diag:
        assert dg <= REL_L2_DIAG, f"{tag}: diagnostic rel L2 {dg}"
    return dict(h=eh, out=gate, diag=dg)
