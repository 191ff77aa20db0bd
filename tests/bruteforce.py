"""Brute-force dense reference for tiny shapes (numpy, fp64).

Written independently of the C oracle, and differently on purpose:
  * weights are dequantised densely, nibbles taken byte by byte from a
    little-endian uint8 view (low nibble of byte 0 first), other widths read
    from the row turned into one Python integer (little-endian bytes), and
    scales decoded by numpy's own float16;
  * routing computes the full softmax over all experts, then a stable
    argsort of the negated logits, then renormalises the kept probabilities;
  * the combine runs a *dense* gate: every expert is evaluated for every
    token and weighted by its gate value, zero where it was not selected;
  * the plan is numpy's stable argsort, bincount and unique.
Only for tiny shapes: it evaluates all E experts for every token.
"""

from __future__ import annotations

import numpy as np


def unpack_bigint(q: np.ndarray, bits: int) -> np.ndarray:
    """q uint32 [..., words] -> element codes [..., words*32/bits]: each row
    read as one little-endian integer, element c = bits c*bits.. of it."""
    q = np.ascontiguousarray(q, dtype="<u4")
    lead, words = q.shape[:-1], q.shape[-1]
    cols = words * 32 // bits
    flat = q.reshape(-1, words)
    out = np.zeros((flat.shape[0], cols), np.float64)
    mask = (1 << bits) - 1
    for r in range(flat.shape[0]):
        big = int.from_bytes(flat[r].tobytes(), "little")
        for c in range(cols):
            out[r, c] = (big >> (c * bits)) & mask
    return out.reshape(*lead, cols)


def dequant_dense(q: np.ndarray, s: np.ndarray, b: np.ndarray, bits: int = 4, group: int = 64) -> np.ndarray:
    """q uint32 [..., rows, cols*bits/32]; s, b fp16 bits [..., rows, cols/group] -> fp64."""
    if bits == 4:
        by = np.ascontiguousarray(q, dtype="<u4").view(np.uint8)  # [..., rows, cols/2]
        lo = (by & 0x0F).astype(np.float64)
        hi = (by >> 4).astype(np.float64)
        codes = np.stack([lo, hi], axis=-1).reshape(*by.shape[:-1], by.shape[-1] * 2)
    else:
        codes = unpack_bigint(q, bits)
    sc = np.asarray(s, np.uint16).view(np.float16).astype(np.float64)
    bi = np.asarray(b, np.uint16).view(np.float16).astype(np.float64)
    sc = np.repeat(sc, group, axis=-1)
    bi = np.repeat(bi, group, axis=-1)
    return sc * codes + bi


def route(logits: np.ndarray, k: int):
    lg = np.asarray(logits, np.float64)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-np.asarray(logits, np.float32), axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(p, idx, axis=1)
    return idx, sel / sel.sum(axis=1, keepdims=True)


def plan(idx: np.ndarray, E: int):
    flat = np.asarray(idx, np.int64).ravel()
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    sorted_slots = np.argsort(flat, kind="stable").astype(np.int32)
    u = np.unique(flat).astype(np.int32)
    unique = np.full(E, -1, np.int32)
    unique[: len(u)] = u
    return dict(counts=counts, offsets=offsets, sorted_slots=sorted_slots,
                unique_experts=unique, n_unique=len(u))


def x_f64(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, np.float64)


def moe_dense(layer, x: np.ndarray, logits: np.ndarray):
    """Returns (idx, w, out fp64 [B,H]) with a dense gate over all experts."""
    sh = layer.shape
    E, k = sh.n_experts, sh.top_k
    idx, w = route(logits, k)
    B = idx.shape[0]
    gate = np.zeros((B, E))
    for t in range(B):
        gate[t, idx[t]] = w[t]
    X = x_f64(x)
    nb, nd, G = sh.bits, sh.down_bits, sh.group_size
    Wg = dequant_dense(layer.gate_q, layer.gate_s, layer.gate_b, nb, G)  # [E,F,H]
    Wu = dequant_dense(layer.up_q, layer.up_s, layer.up_b, nb, G)
    Wd = dequant_dense(layer.down_q, layer.down_s, layer.down_b, nd, G)  # [E,H,F]
    out = np.zeros((B, sh.hidden))
    for e in range(E):
        if not layer.materialised[e]:
            continue  # never selected in the tests that use poisoned layers
        g = X @ Wg[e].T
        u = X @ Wu[e].T
        if layer.sidecar is not None:
            g = g * float(layer.sidecar[e])
            u = u * float(layer.sidecar[e])
        if layer.clamp and layer.clamp > 0:
            g = np.clip(g, -layer.clamp, layer.clamp)
            u = np.clip(u, -layer.clamp, layer.clamp)
        h = g * (1.0 / (1.0 + np.exp(-g))) * u
        y = h @ Wd[e].T
        out += gate[:, e:e + 1] * y
    return idx, w, out
