#!/usr/bin/env python3
"""Decode-step benchmark of the quantized-expert MoE block on one MI355X.

A step is one pass of the whole hot path over one batch, moe_decode_layer:
router, cohort planner, fused gate+up, down projection and combine.  For
up to 8 tokens that is two launches (a gate+up kernel that routes, plans
and deduplicates for itself, then down + combine); for larger batches,
moe_route_plan (or the router and planner kernels), the gate+up kernels and
the down and combine kernels.  The default workload is the single-token
decode layer (hidden 2048, dff 768, 128 experts, top-8, B = 1, affine int4
g64 weights, bf16 activations).  Steps rotate over R layer instances
resident in HBM (48 by default, 16.3 GB of weights, ~1 GB of distinct expert
bytes touched per rotation), so the 256 MB Infinity Cache cannot serve
repeated weight reads.  Every input is seeded synthetic data (moe_workloads);
the weights are drawn and quantised on the device.

Timed passes (HIP graphs, replayed; HIP events on the capturing stream):
  1. headline : exactly K steps after W warm-up steps -> steps/s, unique
     expert GB/s; then three more passes of K steps for the min-max spread
  2. kernels  : R launches of each half of the step alone (moe_route_gate_up,
     moe_expert_down_combine) -> the dominant kernel's (gate+up: two thirds
     of the bytes) average duration for the roofline entry
  3. calibration: a streaming read and a copy of 4 GiB, and the time per
     node of a graph of tiny kernels (the launch floor of a graph)
  4. ladder   : B = 4 / 8 (30 % sharing, random and disjoint routing), B =
     32 (Zipf 1.1, random, disjoint), prefill chunks of B = 256 / 1024, and
     the wide clamped layer (hidden 4096, dff 2048, 256 experts, top-6,
     sidecar, clamp 10) at B = 1 / 4 -> each three passes, min-max
  5. stack    : the 48-layer all-MoE step at B = 32 (Zipf 1.1 per layer),
     each layer's output fed to the next through the residual, one graph
  6. next rows: the router projection (moe_router_logits) alone, the step
     with the GeGLU activation and a down-projection sidecar, and the step
     at other weight widths (4-bit gate/up with 6-bit down; 8-bit)
The oracle (plain fp64 C, OpenMP) is timed on a bounded sample of the same
workload on the host's cores, at all cores and at one core, median of three
(rank 0, N = 1 only).

Prints ONE JSON line.  ``--gpus N`` with N > 1 exits: the library and its
benchmark run on one GPU (how the path would shard is described, not
implemented).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, 8 TB/s
BYTES_PER_WEIGHT = 0.5625  # 4 bits + fp16 scale and bias per 64 weights

WORKLOADS = {
    # name: (shape, B, routing regime, description)
    "decode": ("decode", 1, "normal",
               "single-token decode MoE layer: hidden 2048, dff 768, 128 experts, top_k 8, B=1"),
    "cohort2": ("cohort", 2, "sharing", "batched cohort, same layer, B=2, 30% of tokens share a top-8"),
    "cohort4": ("cohort", 4, "sharing", "batched cohort, same layer, B=4, 30% of tokens share a top-8"),
    "cohort8": ("cohort", 8, "sharing", "batched cohort, same layer, B=8, 30% of tokens share a top-8"),
    "stack32": ("stack", 32, "zipf", "one layer of the 48-layer stack, B=32, Zipf(1.1) expert popularity"),
    "prefill256": ("cohort", 256, "normal", "prefill chunk on the same layer, B=256, independent tokens"),
    "prefill1024": ("cohort", 1024, "normal", "prefill chunk on the same layer, B=1024, independent tokens"),
    "wide1": ("wide", 1, "normal",
              "wide clamped layer: hidden 4096, dff 2048, 256 experts, top_k 6, sidecar, clamp 10, B=1"),
    "wide4": ("wide", 4, "normal",
              "wide clamped layer: hidden 4096, dff 2048, 256 experts, top_k 6, sidecar, clamp 10, B=4"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=480)
    ap.add_argument("--warmup", type=int, default=480,
                    help="untimed steps before the timed ones (ten graph replays of the 48-layer rotation)")
    ap.add_argument("--workload", default="decode", choices=sorted(WORKLOADS))
    ap.add_argument("--regime", default=None,
                    help="routing regime override (normal, sharing, disjoint, zipf, same)")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the headline steps of the workload (for profiler runs)")
    ap.add_argument("--layers", type=int, default=0, help="rotation length (default: >= 1 GB touched)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ladder", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="oracle sample budget per pass (three passes at all cores, three at one)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


# -------------------------------------------------------------- the setup
class Rotation:
    """R layer instances on the device and, per slot, the step's inputs and
    plan buffers."""

    def __init__(self, moe, shape, B, regime, R, seed, layers=None):
        import torch
        from moe_workloads import make_layer_device, make_logits, make_x

        self.shape, self.B, self.R = shape, B, R
        dev = torch.device("cuda")
        if layers is None:
            t0 = time.time()
            layers = []
            for l in range(R):
                t = make_layer_device(shape, l, dev, seed=seed)
                rows = moe.DeviceLayer.from_tensors(shape.hidden, shape.dff, shape.n_experts,
                                                    shape.top_k, shape.act, shape.clamp, t)
                # load-time regrouping of the down projection (moe_pack_down)
                layers.append(rows.pack_down())
                del rows, t
            torch.cuda.synchronize()
            log(f"[bench] {R} layers of {shape.name} generated on device in {time.time() - t0:.1f}s")
        self.layers = layers
        self.logits = [torch.from_numpy(make_logits(shape, B, layer=l, regime=regime, seed=seed)).to(dev)
                       for l in range(R)]
        xs = [make_x(shape, B, layer=l, seed=seed) for l in range(R)]
        if shape.act == "bf16":
            self.x = [torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16) for x in xs]
        else:
            self.x = [torch.from_numpy(x).to(dev) for x in xs]
        k = shape.top_k
        self.idx = [torch.empty((B, k), dtype=torch.int32, device=dev) for _ in range(R)]
        self.w = [torch.empty((B, k), dtype=torch.float32, device=dev) for _ in range(R)]
        self.plans = [moe.Plan.allocate(shape.n_experts, B * k, device=dev) for _ in range(R)]
        self.ws = moe.alloc_workspace(layers[0], B, device=dev)
        self.out = [torch.empty_like(self.x[0]) for _ in range(R)]
        self.moe = moe

    def step(self, i):
        """One layer step from the router logits (moe_decode_layer)."""
        self.moe.decode_layer(self.layers[i], self.x[i], self.logits[i], self.plans[i], self.ws, self.out[i],
                              bufs={"idx": self.idx[i], "w": self.w[i]})

    def n_unique(self):
        return [int(p.n_unique.item()) for p in self.plans]


def capture(fn):
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # eager run on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, reps):
    """Replay a graph `reps` times between two events on the current stream."""
    import torch

    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3  # seconds


class StepTimer:
    """One rotation captured as a graph (plus a graph of the remainder of K
    steps); passes of exactly K steps timed between HIP events."""

    def __init__(self, rot):
        self.rot = rot
        R = rot.R
        self.g_all = capture(lambda: [rot.step(i) for i in range(R)])
        self.g_rem = {}

    def warm(self, W):
        for _ in range(max(1, math.ceil(W / self.rot.R))):
            self.g_all.replay()

    def time(self, K):
        """Seconds for exactly K steps, and the wall time around them."""
        import torch

        R = self.rot.R
        rem = K % R
        if rem and rem not in self.g_rem:
            self.g_rem[rem] = capture(lambda: [self.rot.step(i) for i in range(rem)])
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record()
        for _ in range(K // R):
            self.g_all.replay()
        if rem:
            self.g_rem[rem].replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / 1e3, time.perf_counter() - t0


def spread(values):
    v = sorted(values)
    return {"min": v[0], "median": v[len(v) // 2], "max": v[-1], "n": len(v)}


def run_steps(rot, K, W):
    """W warm-up steps, then exactly K timed steps."""
    st = StepTimer(rot)
    st.warm(W)
    return st.time(K)


def run_kernel_pass(rot, reps=4):
    """Each stage alone, R launches per graph on the slots' precomputed plans."""
    m = rot.moe
    R = rot.R
    stages = {
        # router + planner + gate/up: one launch for a single token
        "route_gate_up": lambda: [m.route_gate_up(rot.layers[i], rot.x[i], rot.logits[i], rot.idx[i], rot.w[i],
                                                  rot.plans[i], rot.ws) for i in range(R)],
        "down_combine": lambda: [m.expert_down_combine(rot.layers[i], rot.B, rot.idx[i], rot.w[i], rot.plans[i],
                                                       rot.out[i], rot.ws) for i in range(R)],
    }
    res = {}
    for name, fn in stages.items():
        g = capture(fn)
        g.replay()
        res[name] = time_graph(g, reps) / (reps * R)  # seconds per launch
    return res


def run_router_projection(rot, reps=4, batches=(1, 32)):
    """The router projection in front of the router (moe_router_logits),
    timed alone on R distinct bf16 weight matrices at each batch size; the
    stack routed from x runs it in front of every layer."""
    import torch
    from moe_workloads import make_x

    sh, R = rot.shape, rot.R
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    wr = [(torch.randn((sh.n_experts, sh.hidden), device="cuda", generator=gen) / math.sqrt(sh.hidden))
          .to(torch.bfloat16) for _ in range(R)]
    nbytes = sh.n_experts * sh.hidden * 2
    res = {"bytes_per_launch": nbytes}
    for B in batches:
        xb = make_x(sh, B, seed=77)
        x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16) if sh.act == "bf16" else \
            torch.from_numpy(xb).cuda()
        lg = [torch.empty((B, sh.n_experts), dtype=torch.float32, device="cuda") for _ in range(R)]
        g = capture(lambda: [rot.moe.router_logits(x, wr[i], lg[i]) for i in range(R)])
        g.replay()
        t = time_graph(g, reps) / (reps * R)
        res[f"B{B}"] = {"us": t * 1e6, "gbps": nbytes / t / 1e9}
    res["us"], res["gbps"] = res[f"B{batches[0]}"]["us"], res[f"B{batches[0]}"]["gbps"]
    return res


def run_geglu_down_sidecar(rot, regime, seed):
    """The same step on the same weights with the GeGLU activation and a
    per-expert down-projection sidecar (uniform in [0.5, 1.5)), timed like
    the headline steps over 2R steps."""
    import torch

    sh, R = rot.shape, rot.R
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4321)
    layers = []
    for l in rot.layers:
        t = dict(l.tensors)
        t["down_sidecar"] = 0.5 + torch.rand(sh.n_experts, device="cuda", generator=gen)
        act = "bf16" if l.act_dtype == rot.moe.MOE_DTYPE_BF16 else "f32"
        layers.append(rot.moe.DeviceLayer.from_tensors(l.hidden, l.dff, l.n_experts, l.top_k, act,
                                                       l.clamp_limit, t, down_layout=l.down_layout,
                                                       activation="geglu"))
    lr = Rotation(rot.moe, sh, rot.B, regime, R, seed, layers=layers)
    t, _ = run_steps(lr, 2 * R, R)
    return {"us_per_step": t / (2 * R) * 1e6, "steps_per_s": 2 * R / t}


def run_widths(moe, shape, regime, seed, R=16, K=None):
    """The single-token step at other weight widths (generic row kernels,
    rows layout): 4-bit gate/up with 6-bit down, and 8-bit everywhere, both
    in groups of 64, on R freshly drawn layers."""
    import dataclasses

    import torch
    from moe_workloads import make_layer_device

    res = {}
    for nb, nd, grp in ((4, 6, 64), (8, 8, 64)):
        sh = dataclasses.replace(shape, bits=nb, down_bits=nd, group_size=grp)
        layers = []
        for l in range(R):
            t = make_layer_device(sh, l, torch.device("cuda"), seed=seed)
            layers.append(moe.DeviceLayer.from_tensors(sh.hidden, sh.dff, sh.n_experts, sh.top_k, sh.act,
                                                       sh.clamp, t, bits=nb, down_bits=nd, group_size=grp))
            del t
        torch.cuda.synchronize()
        rot = Rotation(moe, sh, 1, regime, R, seed, layers=layers)
        k = K or 8 * R
        t, _ = run_steps(rot, k, R)
        st = t / k
        nu = float(np.mean(rot.n_unique()))
        per_expert = sh.hidden * sh.dff * (2 * (nb / 8 + 4 / grp) + (nd / 8 + 4 / grp))
        res[f"g{nb}u{nb}d{nd}_group{grp}"] = {"us_per_step": st * 1e6, "steps_per_s": 1 / st,
                                              "unique_bytes": nu * per_expert,
                                              "unique_gbps": nu * per_expert / st / 1e9}
        del rot, layers
        torch.cuda.empty_cache()
    return res


def unique_bytes(shape, n_unique):
    return n_unique * 3 * shape.hidden * shape.dff * BYTES_PER_WEIGHT


def gate_up_bytes(shape, n_unique):
    return n_unique * 2 * shape.hidden * shape.dff * BYTES_PER_WEIGHT


class StackChain:
    """The 48-layer all-MoE step: layer l reads x_l, adds its expert output to
    it (the residual) and writes x_{l+1}, which layer l+1 reads; B tokens,
    logits pre-generated per layer (Zipf 1.1 expert popularity)."""

    def __init__(self, moe, shape, layers, B, regime, seed, from_x=False):
        import torch
        from moe_workloads import make_logits, make_router, make_x

        dev = torch.device("cuda")
        self.moe, self.shape, self.B, self.layers = moe, shape, B, layers
        L = len(layers)
        self.routers = None
        if from_x:  # each layer's logits projected from its own input (moe_router_logits)
            self.routers = [torch.from_numpy(make_router(shape, layer=l, seed=seed).view(np.int16)).to(dev)
                            .view(torch.bfloat16) for l in range(L)]
            self.logits = [torch.empty((B, shape.n_experts), dtype=torch.float32, device=dev) for _ in range(L)]
        else:
            self.logits = [torch.from_numpy(make_logits(shape, B, layer=l, regime=regime, seed=seed)).to(dev)
                           for l in range(L)]
        x0 = make_x(shape, B, layer=0, seed=seed)
        self.xs = [torch.from_numpy(x0.view(np.int16)).to(dev).view(torch.bfloat16)]
        self.xs += [torch.empty_like(self.xs[0]) for _ in range(L)]
        k = shape.top_k
        self.plans = [moe.Plan.allocate(shape.n_experts, B * k, device=dev) for _ in range(L)]
        self.idx = torch.empty((B, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((B, k), dtype=torch.float32, device=dev)
        self.ws = moe.alloc_workspace(layers[0], B, device=dev)

    def step(self):
        for l, layer in enumerate(self.layers):
            if self.routers is not None:
                self.moe.router_logits(self.xs[l], self.routers[l], self.logits[l])
            self.moe.decode_layer(layer, self.xs[l], self.logits[l], self.plans[l], self.ws, self.xs[l + 1],
                                  residual=self.xs[l], bufs={"idx": self.idx, "w": self.w})

    def n_unique(self):
        return [int(p.n_unique.item()) for p in self.plans]


def run_stack_chain(moe, shape, layers, B, regime, seed, reps=5, passes=3, from_x=False):
    import torch

    sc = StackChain(moe, shape, layers, B, regime, seed, from_x=from_x)
    g = capture(sc.step)
    g.replay()
    torch.cuda.synchronize()
    ts = [time_graph(g, reps) / reps for _ in range(passes)]
    nu = sc.n_unique()
    ub = sum(unique_bytes(shape, n) for n in nu)
    sp = spread(ts)
    st = sp["median"]
    how = "routed from x by the router projection in front of each layer" if from_x else f"{regime} routing"
    return {"workload": f"{len(layers)}-layer all-MoE step, B={B}, {how}, residual between layers",
            "layers": len(layers), "B": B, "ms_per_step": st * 1e3,
            "ms_per_step_min": sp["min"] * 1e3, "ms_per_step_max": sp["max"] * 1e3, "passes": passes,
            "steps_per_s": 1 / st, "tokens_per_s": B / st, "unique_experts_per_layer": float(np.mean(nu)),
            "unique_bytes_per_step": ub, "unique_gbps": ub / st / 1e9, "hbm_frac": ub / st / 1e9 / HBM_PEAK_GBPS}


def calibration(n_bytes=4 << 30, reps=5):
    """Streaming read and copy of n_bytes, and the time per node of a graph
    of 100 one-element kernels (the launch floor of a graph node)."""
    import torch

    a = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    out = torch.empty((), dtype=torch.float32, device="cuda")

    def best(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        return min(ts)

    t_read = best(lambda: torch.sum(a, dim=0, out=out))
    t_copy = best(lambda: b.copy_(a))
    del a, b
    tiny = torch.zeros(1, device="cuda")
    g = capture(lambda: [tiny.add_(1.0) for _ in range(100)])
    g.replay()
    t_node = min(time_graph(g, 10) / 1000 for _ in range(3))
    torch.cuda.empty_cache()
    return {"stream_read_gbps": n_bytes / t_read / 1e9, "copy_gbps": 2 * n_bytes / t_copy / 1e9,
            "bytes": n_bytes, "graph_node_us": t_node * 1e6,
            "note": "read: torch.sum over 4 GiB fp32; copy: 4 GiB each way (read + write counted); "
                    "graph node: one-element add kernels, 100 per graph"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------ CPU oracle
def cpu_baseline(rot, budget_s):
    """The oracle as it stands, on a bounded sample of the same workload:
    the slots' logits and x, and the experts each slot routes to, copied to
    the host.  Times route + plan + expert block per step."""
    import torch
    from moe_workloads.gen import POISON_F16, Layer
    from oracle import oracle

    sh = rot.shape
    E, H, F = sh.n_experts, sh.hidden, sh.dff
    n_slots = min(rot.R, 8)
    samples = []
    for i in range(n_slots):
        lg = rot.logits[i].cpu().numpy()
        x = rot.x[i].view(torch.int16).cpu().numpy().view(np.uint16) if sh.act == "bf16" else rot.x[i].cpu().numpy()
        ids = np.unique(rot.idx[i].cpu().numpy())
        t = rot.layers[i].tensors
        L = Layer(shape=sh,
                  gate_q=np.zeros((E, F, H // 8), np.uint32), gate_s=np.full((E, F, H // 64), POISON_F16, np.uint16),
                  gate_b=np.full((E, F, H // 64), POISON_F16, np.uint16),
                  up_q=np.zeros((E, F, H // 8), np.uint32), up_s=np.full((E, F, H // 64), POISON_F16, np.uint16),
                  up_b=np.full((E, F, H // 64), POISON_F16, np.uint16),
                  down_q=np.zeros((E, H, F // 8), np.uint32), down_s=np.full((E, H, F // 64), POISON_F16, np.uint16),
                  down_b=np.full((E, H, F // 64), POISON_F16, np.uint16),
                  sidecar=None if t.get("sidecar") is None else t["sidecar"].cpu().numpy(), clamp=sh.clamp)
        cols = rot.layers[i].down_layout == rot.moe.MOE_DOWN_COLS
        for e in ids:
            for n in ("gate_q", "up_q"):
                getattr(L, n)[e] = t[n][e].cpu().numpy().view(np.uint32).reshape(F, H // 8)
            for n in ("gate_s", "gate_b", "up_s", "up_b"):
                getattr(L, n)[e] = t[n][e].cpu().numpy().view(np.uint16).reshape(F, H // 64)
            dq = t["down_q"][e].cpu().numpy().view(np.uint32)
            # the column layout (moe_pack_down) back to the rows the oracle reads
            L.down_q[e] = (dq.reshape(F // 32, H, 4).transpose(1, 0, 2).reshape(H, F // 8) if cols
                           else dq.reshape(H, F // 8))
            for n in ("down_s", "down_b"):
                v = t[n][e].cpu().numpy().view(np.uint16)
                getattr(L, n)[e] = v.reshape(F // 64, H).T if cols else v.reshape(H, F // 64)
        samples.append((L, x, lg))
    oracle.lib()

    def one_pass(budget):
        done, t0 = 0, time.perf_counter()
        while True:
            L, x, lg = samples[done % n_slots]
            idx, w = oracle.route_topk(lg, sh.top_k)
            oracle.plan(idx, E)
            oracle.decode_step(L, x, idx, w)
            done += 1
            el = time.perf_counter() - t0
            if (el >= budget and done >= 3) or done >= 2000:
                return done, el

    all_threads = oracle.set_threads(int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1))
    res = {}
    for label, threads in (("all", all_threads), ("one", 1)):
        used = oracle.set_threads(threads)
        one_pass(0.0)  # one untimed warm-up step
        runs = [one_pass(budget_s) for _ in range(3)]
        rates = sorted(d / el for d, el in runs)
        res[label] = {"value": rates[1], "min": rates[0], "max": rates[2], "cores": used,
                      "steps": [d for d, _ in runs], "seconds": [round(el, 2) for _, el in runs]}
    oracle.set_threads(all_threads)
    a_, o_ = res["all"], res["one"]
    model = cpu_model()
    return {"value": a_["value"], "unit": "steps/s", "cores": a_["cores"], "kind": "oracle",
            "sample": f"median of 3 passes of ~{budget_s:.0f} s each ({sum(a_['steps'])} steps in all) of the "
                      f"same workload over {n_slots} of its layer slots, at {a_['cores']} threads; fp64 per-slot "
                      "oracle, no dedup: a correctness baseline, not a tuned CPU kernel",
            "min": a_["min"], "max": a_["max"], "cpu_model": model,
            "one_core": {"value": o_["value"], "min": o_["min"], "max": o_["max"], "cores": 1,
                         "steps": o_["steps"], "seconds": o_["seconds"]}}


# ------------------------------------------------------------------ main
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_b1_traffic.json")


def counted_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    record (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's counts), or
    None when there is none for this workload or the kernel sources changed
    since the counters were taken."""
    import hashlib

    if workload != "decode" or not os.path.exists(TRAFFIC_RECORD):
        return None
    rec = json.load(open(TRAFFIC_RECORD))
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != rec["sources_sha256"] or kernel not in rec["kernels"]:
        return None
    return rec["kernels"][kernel]["traffic_bytes"]


TRACE_RECORD = os.path.join(ROOT, "profiles", "decode_b1_kernel_trace.md")


def traced_kernel_us(workload: str, kernel: str):
    """Average duration of `kernel` in the committed rocprofv3 kernel trace
    of this workload (the tracer's own clock, which stretches each
    dispatch), or None."""
    if workload != "decode" or not os.path.exists(TRACE_RECORD):
        return None
    for line in open(TRACE_RECORD):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 3 and cells[0] == f"`{kernel}`":
            try:
                return float(cells[2])
            except ValueError:
                return None
    return None


def copy_calibration():
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n, "copies": 3}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding is described, not implemented)", file=sys.stderr, flush=True)
        sys.exit(2)
    import torch

    import quantized_expert_gemv_moe_amd as moe
    from moe_workloads import SHAPES

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    moe.lib()
    if args.copy_calibration:
        copy_calibration()
        return

    shape_name, B, regime, desc = WORKLOADS[args.workload]
    if args.regime:
        regime = args.regime
        desc = f"{desc} ({regime} routing)"
    sh = SHAPES[shape_name]
    per_layer = sh.n_experts * 3 * sh.hidden * sh.dff * BYTES_PER_WEIGHT
    R = args.layers or max(8, min(48, int(math.ceil(16.3e9 / per_layer))))
    rot = Rotation(moe, sh, B, regime, R, args.seed)

    timer = StepTimer(rot)
    timer.warm(args.warmup)
    secs, wall = timer.time(args.steps)  # the headline: exactly K steps
    nu = rot.n_unique()
    avg_unique = float(np.mean(nu))
    ms = secs * 1e3 / args.steps
    steps_per_s = args.steps / secs
    ub = unique_bytes(sh, avg_unique)
    gbps = ub / (secs / args.steps) / 1e9
    passes = [timer.time(args.steps)[0] / args.steps * 1e6 for _ in range(3)]
    log(f"[bench] {args.workload}: {ms * 1e3:.2f} us/step, {steps_per_s:.0f} steps/s, "
        f"unique {ub / 1e6:.2f} MB/step -> {gbps:.0f} GB/s ({gbps / HBM_PEAK_GBPS:.1%} of peak); wall {wall:.2f}s; "
        f"three more passes {' '.join(f'{p:.2f}' for p in passes)} us/step")

    if args.headline_only:
        print(json.dumps({"workload": args.workload, "regime": regime, "us_per_step": ms * 1e3,
                          "us_per_step_passes": passes, "unique_experts": avg_unique, "unique_gbps": gbps}),
              flush=True)
        return

    kpasses = [run_kernel_pass(rot) for _ in range(3)]
    kt = {k: spread([kp[k] for kp in kpasses])["median"] for k in kpasses[0]}
    gu_bytes = gate_up_bytes(sh, avg_unique)
    dn_bytes = avg_unique * sh.hidden * sh.dff * BYTES_PER_WEIGHT
    kernels = {k: {"us": v * 1e6, "us_min": min(kp[k] for kp in kpasses) * 1e6,
                   "us_max": max(kp[k] for kp in kpasses) * 1e6} for k, v in kt.items()}
    kernels["route_gate_up"]["gbps"] = gu_bytes / kt["route_gate_up"] / 1e9
    kernels["down_combine"]["gbps"] = dn_bytes / kt["down_combine"] / 1e9
    log(f"[bench] kernels: " + ", ".join(f"{k} {v['us']:.2f} us" for k, v in kernels.items()))
    ach = gu_bytes / kt["route_gate_up"] / 1e9
    gu_kernel = ("gate_up_route_kernel<64, 1, 4, true, 2, 4, false>"
                 if B == 1 and sh.hidden == 2048 and sh.n_experts == 128
                 else "gate_up_route_kernel" if B <= 8 else "route_plan_kernel + gate_up kernels")
    traffic = counted_traffic(args.workload, gu_kernel)
    traced_us = traced_kernel_us(args.workload, gu_kernel)

    cal = calibration()
    log(f"[bench] calibration: streaming read {cal['stream_read_gbps']:.0f} GB/s, copy {cal['copy_gbps']:.0f} GB/s, "
        f"graph node {cal['graph_node_us']:.2f} us")

    rp = run_router_projection(rot)
    log(f"[bench] router projection (next row): B=1 {rp['B1']['us']:.2f} us per launch ({rp['B1']['gbps']:.0f} GB/s), "
        f"B=32 {rp['B32']['us']:.2f} us")

    gg = run_geglu_down_sidecar(rot, regime, args.seed)
    gg["step_time_vs_swiglu"] = gg["us_per_step"] / (ms * 1e3)
    log(f"[bench] GeGLU + down sidecar (next row): {gg['us_per_step']:.2f} us/step "
        f"({gg['step_time_vs_swiglu']:.3f}x the SwiGLU step)")

    widths = None
    if sh.name == "decode" and B == 1:
        widths = run_widths(moe, sh, regime, args.seed)
        for kname, v in widths.items():
            log(f"[bench] widths {kname} (next row): {v['us_per_step']:.2f} us/step, "
                f"{v['unique_gbps']:.0f} GB/s of unique expert bytes")

    t1 = secs / args.steps

    def rung(wl, rg, layers, R2):
        s2, b2, _, _ = WORKLOADS[wl]
        s2h = SHAPES[s2]
        lr = Rotation(moe, s2h, b2, rg, R2, args.seed, layers=layers)
        tm = StepTimer(lr)
        tm.warm(R2)
        k2 = 2 * R2
        sp = spread([tm.time(k2)[0] / k2 for _ in range(3)])
        st = sp["median"]
        nu2 = float(np.mean(lr.n_unique()))
        ub2 = unique_bytes(s2h, nu2)
        # multiply-adds actually required: 3 matrices of H x F per (token, k) slot
        tflops = 2.0 * b2 * s2h.top_k * 3 * s2h.hidden * s2h.dff / st / 1e12
        r = {"workload": wl, "B": b2, "routing": rg, "steps_per_s": 1.0 / st, "us_per_step": st * 1e6,
             "us_per_step_min": sp["min"] * 1e6, "us_per_step_max": sp["max"] * 1e6, "passes": sp["n"],
             "tokens_per_s": b2 / st, "unique_experts": nu2, "unique_bytes": ub2, "unique_gbps": ub2 / st / 1e9,
             "hbm_frac": ub2 / st / 1e9 / HBM_PEAK_GBPS, "expert_tflops": tflops}
        if s2h.hidden == sh.hidden and s2h.dff == sh.dff and s2h.n_experts == sh.n_experts:
            r["step_time_vs_B1"] = st / t1
        log(f"[bench] ladder {wl} ({rg}): {st * 1e6:.2f} us/step [{sp['min'] * 1e6:.2f}, {sp['max'] * 1e6:.2f}], "
            f"n_unique {nu2:.1f}, {ub2 / st / 1e9:.0f} GB/s ({ub2 / st / 1e9 / HBM_PEAK_GBPS:.1%}), "
            f"{tflops:.2f} TFLOP/s")
        del lr, tm
        return r

    ladder, wide, stack, stack_x = [], [], None, None
    if not args.no_ladder and sh.name in ("decode", "cohort", "stack"):
        for wl, rg in (("cohort4", "sharing"), ("cohort4", "normal"), ("cohort4", "disjoint"),
                       ("cohort8", "sharing"), ("cohort8", "normal"), ("cohort8", "disjoint"),
                       ("stack32", "zipf"), ("stack32", "normal"), ("stack32", "disjoint"),
                       ("prefill256", "normal"), ("prefill1024", "normal")):
            ladder.append(rung(wl, rg, rot.layers, R))
        n_stack = min(48, len(rot.layers))
        stack = run_stack_chain(moe, SHAPES["stack"], rot.layers[:n_stack], 32, "zipf", args.seed)
        log(f"[bench] stack: {stack['ms_per_step']:.3f} ms per {n_stack}-layer step at B=32 "
            f"[{stack['ms_per_step_min']:.3f}, {stack['ms_per_step_max']:.3f}], "
            f"{stack['tokens_per_s']:.0f} tokens/s, {stack['unique_gbps']:.0f} GB/s ({stack['hbm_frac']:.1%})")
        stack_x = run_stack_chain(moe, SHAPES["stack"], rot.layers[:n_stack], 32, "normal", args.seed, from_x=True)
        log(f"[bench] stack routed from x: {stack_x['ms_per_step']:.3f} ms per {n_stack}-layer step at B=32 "
            f"[{stack_x['ms_per_step_min']:.3f}, {stack_x['ms_per_step_max']:.3f}], n_unique "
            f"{stack_x['unique_experts_per_layer']:.1f}, {stack_x['unique_gbps']:.0f} GB/s ({stack_x['hbm_frac']:.1%})")
        # the wide clamped layer on its own rotation (3.6 GB per layer)
        wsh = SHAPES["wide"]
        wper = wsh.n_experts * 3 * wsh.hidden * wsh.dff * BYTES_PER_WEIGHT
        Rw = max(8, min(48, int(math.ceil(16.3e9 / wper))))
        wrot = Rotation(moe, wsh, 1, "normal", Rw, args.seed)
        for wl in ("wide1", "wide4"):
            wide.append(rung(wl, "normal", wrot.layers, Rw))
        del wrot
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(rot, args.cpu_seconds)
        log(f"[bench] oracle: {cpu['value']:.2f} steps/s on {cpu['cores']} threads "
            f"({cpu['one_core']['value']:.2f} on one), {cpu['cpu_model']}")

    line = {
        "metric": "MoE decode steps/s and unique-expert HBM GB/s (% of peak) at B=1/4/8/32",
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": desc, "hidden": sh.hidden, "dff": sh.dff, "n_experts": sh.n_experts,
                   "top_k": sh.top_k, "n_tokens": B, "routing": regime,
                   "weights": "affine int4, group 64, fp16 scale+bias; down projection packed by moe_pack_down",
                   "activations": sh.act,
                   "accumulation": "f32", "rotation_layers": R},
        "unique_gbps": gbps,
        "hbm_frac": gbps / HBM_PEAK_GBPS,
        "hbm_frac_of_stream_read": gbps / cal["stream_read_gbps"],
        "unique_experts_per_step": avg_unique,
        "passes_us_per_step": {"values": passes, **spread(passes)},
        "roofline": {"bound": "hbm", "kernel": gu_kernel, "achieved": ach, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS, "traffic": traffic,
                     "bytes_per_launch": gu_bytes, "us_per_launch": kt["route_gate_up"] * 1e6,
                     # the same kernel's average under the kernel tracer (committed
                     # profile of this workload): its clock includes the tracer's own
                     # per-dispatch cost and excludes the gap between graph nodes
                     "us_per_launch_traced": traced_us,
                     "frac_traced": (gu_bytes / traced_us / 1e3 / HBM_PEAK_GBPS) if traced_us else None},
        "kernels": kernels,
        "calibration": cal,
        "ladder": ladder,
        "stack48": stack,
        "stack48_from_x": stack_x,
        "wide": wide,
        "next_rows": {"router_projection": rp, "geglu_down_sidecar": gg, "widths": widths},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
