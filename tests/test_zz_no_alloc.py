"""moe_decode_layer_static (no workspace, the library's per-device scratch
array) against moe_decode_layer on the same inputs: routing, plan and
output bitwise equal, on two calls in a row with the second batch smaller,
and the output within the oracle's tolerance."""

import numpy as np
import pytest
import torch

import quantized_expert_gemv_moe_amd as moe
from gpu_helpers import DeviceRun, check_against_oracle, dev_x, host_bits, layer_for, log
from moe_workloads import SHAPES, make_logits, make_x

pytestmark = pytest.mark.gpu


def test_static_scratch_entry_point_matches_decode_layer():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sh = SHAPES["stack"]
    k, E = sh.top_k, sh.n_experts
    dl = None
    for B, regime, seed in ((32, "zipf", 11), (5, "sharing", 12)):
        log(f"[case] decode_layer_static B={B} {regime}")
        lg = make_logits(sh, B, regime=regime, seed=seed)
        L = layer_for(sh, lg, seed=seed)
        x = make_x(sh, B, seed=seed)
        dl = moe.DeviceLayer.from_host(L).pack_down()
        ref = DeviceRun(L, x, lg, dl=dl)  # moe_decode_layer with its workspace
        check_against_oracle(L, x, lg, ref, f"static reference B{B}")
        xt, lgt = dev_x(x), torch.from_numpy(lg).cuda()
        plan = moe.Plan.allocate(E, B * k)
        out = torch.empty_like(xt)
        idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
        w = torch.empty((B, k), dtype=torch.float32, device="cuda")
        moe.decode_layer_static(dl, xt, lgt, plan, out, idx, w)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), ref.out), f"B={B}: output differs from moe_decode_layer"
        assert np.array_equal(idx.cpu().numpy(), ref.idx)
        assert np.array_equal(w.cpu().numpy(), ref.w)
        n = B * k
        for name in ("counts", "offsets", "unique_experts"):
            assert np.array_equal(getattr(plan, name).cpu().numpy(), ref.plan_np[name]), name
        assert np.array_equal(plan.sorted_slots[:n].cpu().numpy(), ref.plan_np["sorted_slots"])
        assert int(plan.n_unique.item()) == ref.plan_np["n_unique"]
