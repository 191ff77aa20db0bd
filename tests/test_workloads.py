"""The seeded input recipes (CPU): the device-side quantiser used for
benchmark volumes agrees bit for bit with the host one, and the routing
regimes have the structure their recipes state."""

import math

import numpy as np
import torch

from moe_workloads import SHAPES, make_logits, quantize_affine4
from moe_workloads.gen import quantize_affine4_torch


def test_torch_quantiser_matches_numpy_bitwise():
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((3, 48, 256)) * 0.02).astype(np.float32)
    w[0, 0, :64] = 0.125  # a constant group: scale 0, every nibble 0
    q, s, b = quantize_affine4_torch(torch.from_numpy(w))
    for n in range(3):
        rq, rs, rb = quantize_affine4(w[n])
        assert np.array_equal(q[n].numpy().view(np.uint32), rq)
        assert np.array_equal(s[n].numpy().view(np.uint16), rs)
        assert np.array_equal(b[n].numpy().view(np.uint16), rb)
    assert q[0, 0, :8].abs().sum().item() == 0


def topk(lg, k):
    return np.argsort(-lg, axis=1, kind="stable")[:, :k]


def test_sharing_regime_gives_the_shared_set_to_30_percent_of_tokens():
    sh = SHAPES["cohort"]
    for B in (4, 8, 32):
        lg = make_logits(sh, B, regime="sharing", seed=B)
        sets = [frozenset(r) for r in topk(lg, sh.top_k)]
        common = max(set(sets), key=sets.count)
        assert sets.count(common) >= math.ceil(0.3 * B)


def test_zipf_regime_follows_the_rank_bias():
    sh = SHAPES["stack"]
    lg = make_logits(sh, 4096, regime="zipf", seed=1)
    counts = np.bincount(topk(lg, sh.top_k).ravel(), minlength=sh.n_experts)
    bias = lg.mean(axis=0)
    order = np.argsort(-bias)
    # the most biased experts are picked far more often than the least
    assert counts[order[:8]].sum() > 10 * counts[order[-32:]].sum()
    # bias differences follow -1.1 ln(rank) within sampling noise
    assert abs((bias[order[0]] - bias[order[1]]) - 1.1 * math.log(2)) < 0.1


def test_disjoint_and_same_regimes():
    sh = SHAPES["cohort"]
    d = topk(make_logits(sh, 8, regime="disjoint", seed=2), sh.top_k)
    assert len(np.unique(d)) == 64
    s = topk(make_logits(sh, 6, regime="same", seed=2), sh.top_k)
    assert all(set(r) == set(s[0]) for r in s)
