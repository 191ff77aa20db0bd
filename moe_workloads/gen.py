"""Workload shapes and seeded generators (inputs only, none of the method).

Seeding: every array is drawn from
``numpy.random.default_rng(SeedSequence([seed, cfg, layer, stream, index]))``
with the streams 0 activations, 1 logits, 2 gate, 3 up, 4 down, 5 sidecar,
6 Zipf rank permutation, 7 sharing set, 8 router projection, 9 down
sidecar.  The same arguments always give the same bytes.

Weight storage (the layout both sides read):
  * ``*_q``  uint32 ``[E][rows][cols*bits/32]``: a row is a little-endian
    bit stream, element c in stream bits ``c*bits .. c*bits+bits-1`` (so at
    4 bits nibble i of word w holds element ``8*w + i``, lowest nibble
    first).  Rows are output features (gate/up: Dff rows of ``hidden``
    inputs; down: ``hidden`` rows of Dff inputs), so the product is
    ``x @ W.T`` per expert.  Gate and up use ``shape.bits``, down
    ``shape.down_bits``.
  * ``*_s``, ``*_b`` uint16 ``[E][rows][cols/group]``: fp16 bit patterns of
    the per-group scale and bias of ``shape.group_size`` consecutive inputs.
Unmaterialised experts carry NaN scales and biases ("poison"): any read of
them turns the result into NaN.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Iterable, Optional, Sequence

import numpy as np

GROUP = 64
POISON_F16 = np.uint16(0x7E00)  # fp16 quiet NaN

# streams of the seed sequence
S_X, S_LOGITS, S_GATE, S_UP, S_DOWN, S_SIDECAR, S_RANK, S_SHARE, S_ROUTER, S_DOWN_SIDECAR = range(10)


@dataclass(frozen=True)
class Shape:
    """One MoE layer shape.  ``act`` is the dtype of x and out."""

    name: str
    cfg: int  # seed id of the workload family
    hidden: int
    dff: int
    n_experts: int
    top_k: int
    act: str  # "f32" or "bf16"
    sidecar: bool = False
    clamp: float = 0.0
    activation: str = "swiglu"   # or "geglu"
    down_sidecar: bool = False   # a per-expert fp32 scale of the down output
    bits: int = 4                # width of the gate and up elements
    down_bits: int = 4           # width of the down elements
    group_size: int = 64         # inputs per scale/bias group


SHAPES: Dict[str, Shape] = {
    # toy layer, fp32 I/O
    "toy": Shape("toy", 0, 256, 128, 8, 2, "f32"),
    # single-token decode layer of the qwen3-30b-a3b-4bit shape
    "decode": Shape("decode", 1, 2048, 768, 128, 8, "bf16"),
    # batched cohort on the same layer shape (30 % of tokens share a top-k)
    "cohort": Shape("cohort", 2, 2048, 768, 128, 8, "bf16"),
    # 256-expert top-6 layer with a per-expert scale sidecar and a +-10 clamp
    "wide": Shape("wide", 3, 4096, 2048, 256, 6, "bf16", sidecar=True, clamp=10.0),
    # one layer of the 48-layer stack (Zipf 1.1 expert popularity)
    "stack": Shape("stack", 4, 2048, 768, 128, 8, "bf16"),
}


def rng_for(seed: int, cfg: int, layer: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg, layer, stream, index]))


# ----------------------------------------------------------------- bf16 bits
def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------- quantisation
def pack_bits(q: np.ndarray, bits: int) -> np.ndarray:
    """Unsigned ``q[rows, cols]`` (< 2^bits) -> uint32 words [rows, cols*bits/32],
    each row a little-endian bit stream with element c at bits c*bits.."""
    rows, cols = q.shape
    assert (cols * bits) % 32 == 0
    b = ((q.astype(np.uint32)[:, :, None] >> np.arange(bits, dtype=np.uint32)) & 1).astype(np.uint8)
    packed = np.packbits(b.reshape(rows, cols * bits), axis=1, bitorder="little")
    return np.ascontiguousarray(packed).view("<u4").astype(np.uint32)


def quantize_affine(w: np.ndarray, bits: int = 4, group: int = GROUP):
    """Quantise fp32 ``w[rows, cols]`` to affine ``bits``-bit, groups of
    ``group`` along cols.

    Per group, with n = 2^bits - 1: scale = fp16((max - min) / n), bias =
    fp16(min), q = clip(rint((w - bias) / scale), 0, n).  Returns (q_words
    uint32 [rows, cols*bits/32], scale bits uint16 [rows, cols/group], bias
    bits uint16).  Any deterministic quantiser gives valid inputs; both sides
    read the stored bytes only.
    """
    rows, cols = w.shape
    assert cols % group == 0
    n = float(2 ** bits - 1)
    g = w.reshape(rows, cols // group, group).astype(np.float32, copy=False)
    mn = g.min(axis=2)
    mx = g.max(axis=2)
    s16 = ((mx - mn) / np.float32(n)).astype(np.float16)
    b16 = mn.astype(np.float16)
    s = s16.astype(np.float32)[:, :, None]
    b = b16.astype(np.float32)[:, :, None]
    safe = np.where(s == 0, np.float32(1.0), s)
    q = np.rint((g - b) / safe)
    q *= (s != 0)
    np.clip(q, 0, n, out=q)
    q = q.astype(np.uint32).reshape(rows, cols)
    return pack_bits(q, bits), s16.view(np.uint16), b16.view(np.uint16)


def quantize_affine4(w: np.ndarray):
    """:func:`quantize_affine` at 4 bits, groups of 64."""
    return quantize_affine(w, 4, GROUP)


# -------------------------------------------------------------------- layer
@dataclass
class Layer:
    shape: Shape
    gate_q: np.ndarray
    gate_s: np.ndarray
    gate_b: np.ndarray
    up_q: np.ndarray
    up_s: np.ndarray
    up_b: np.ndarray
    down_q: np.ndarray
    down_s: np.ndarray
    down_b: np.ndarray
    sidecar: Optional[np.ndarray]  # fp32 [E] or None
    clamp: float
    materialised: np.ndarray = field(default=None)  # bool [E]
    activation: str = "swiglu"
    down_sidecar: Optional[np.ndarray] = None  # fp32 [E] or None


def _empty_layer(shape: Shape) -> Layer:
    E, H, F = shape.n_experts, shape.hidden, shape.dff
    G, nb, nd = shape.group_size, shape.bits, shape.down_bits
    assert H % G == 0 and F % G == 0 and (H * nb) % 32 == 0 and (F * nd) % 32 == 0
    return Layer(
        shape=shape,
        gate_q=np.zeros((E, F, H * nb // 32), np.uint32),
        gate_s=np.full((E, F, H // G), POISON_F16, np.uint16),
        gate_b=np.full((E, F, H // G), POISON_F16, np.uint16),
        up_q=np.zeros((E, F, H * nb // 32), np.uint32),
        up_s=np.full((E, F, H // G), POISON_F16, np.uint16),
        up_b=np.full((E, F, H // G), POISON_F16, np.uint16),
        down_q=np.zeros((E, H, F * nd // 32), np.uint32),
        down_s=np.full((E, H, F // G), POISON_F16, np.uint16),
        down_b=np.full((E, H, F // G), POISON_F16, np.uint16),
        sidecar=None,
        clamp=shape.clamp,
        materialised=np.zeros(E, bool),
        activation=shape.activation,
    )


def make_layer(shape: Shape, layer: int = 0, experts: Optional[Iterable[int]] = None,
               seed: int = 0, std: float = 0.02) -> Layer:
    """Quantised weights of one layer; N(0, std) before quantisation.

    Only the experts in ``experts`` (all when None) are drawn; the others
    are poisoned.  Expert e's bytes do not depend on which others are drawn.
    """
    E, H, F = shape.n_experts, shape.hidden, shape.dff
    L = _empty_layer(shape)
    ids = range(E) if experts is None else sorted(set(int(e) for e in experts))
    for e in ids:
        for stream, (qa, sa, ba, rows, cols, nb) in (
            (S_GATE, (L.gate_q, L.gate_s, L.gate_b, F, H, shape.bits)),
            (S_UP, (L.up_q, L.up_s, L.up_b, F, H, shape.bits)),
            (S_DOWN, (L.down_q, L.down_s, L.down_b, H, F, shape.down_bits)),
        ):
            w = rng_for(seed, shape.cfg, layer, stream, e).standard_normal((rows, cols), np.float32)
            w *= np.float32(std)
            q, s, b = quantize_affine(w, nb, shape.group_size)
            qa[e], sa[e], ba[e] = q, s, b
        L.materialised[e] = True
    if shape.sidecar:
        L.sidecar = rng_for(seed, shape.cfg, layer, S_SIDECAR).uniform(0.5, 1.5, E).astype(np.float32)
    if shape.down_sidecar:
        L.down_sidecar = rng_for(seed, shape.cfg, layer, S_DOWN_SIDECAR).uniform(0.5, 1.5, E).astype(np.float32)
    return L


# -------------------------------------------------------------- activations
def make_x(shape: Shape, n_tokens: int, layer: int = 0, seed: int = 0, scale: float = 1.0) -> np.ndarray:
    """x ~ N(0,1) * scale: fp32 array for fp32 I/O, else bf16 bit patterns."""
    x = rng_for(seed, shape.cfg, layer, S_X).standard_normal((n_tokens, shape.hidden), np.float32)
    x *= np.float32(scale)
    if shape.act == "f32":
        return x
    return bf16_bits_from_f32(x)


def make_router(shape: Shape, layer: int = 0, seed: int = 0) -> np.ndarray:
    """Router projection weights, bf16 bit patterns [E][hidden] drawn from
    N(0, 1/hidden), so that N(0,1) activations give logits of unit scale."""
    w = rng_for(seed, shape.cfg, layer, S_ROUTER).standard_normal((shape.n_experts, shape.hidden), np.float32)
    w *= np.float32(1.0 / np.sqrt(shape.hidden))
    return bf16_bits_from_f32(w)


# ------------------------------------------------------------------- logits
def make_logits(shape: Shape, n_tokens: int, layer: int = 0, regime: str = "normal",
                seed: int = 0, share_frac: float = 0.3, zipf_s: float = 1.1) -> np.ndarray:
    """Router logits ``[n_tokens, E]`` fp32.

    regimes:
      normal   - N(0,1)
      sharing  - ceil(share_frac*B) tokens at seeded positions get +8 on one
                 seeded set of top_k experts, which becomes exactly their top-k
      zipf     - N(0,1) + bias[e], bias[e] = -s*ln(rank(e)), rank from a
                 seeded permutation of the experts (rank 1 = most popular)
      disjoint - token t gets +8 on experts t*k .. t*k+k-1 (mod E): the
                 worst case for unique-expert traffic
      same     - every token carries the logits of token 0
    """
    E, k = shape.n_experts, shape.top_k
    z = rng_for(seed, shape.cfg, layer, S_LOGITS).standard_normal((n_tokens, E), np.float32)
    if regime == "normal":
        return z
    if regime == "sharing":
        r = rng_for(seed, shape.cfg, layer, S_SHARE)
        n_s = int(math.ceil(share_frac * n_tokens))
        toks = r.choice(n_tokens, size=n_s, replace=False) if n_tokens else np.zeros(0, int)
        S = r.choice(E, size=k, replace=False)
        z[np.ix_(toks, S)] += np.float32(8.0)
        rest = np.setdiff1d(np.arange(E), S)
        for t in toks:
            assert z[t, S].min() > z[t, rest].max(), "sharing set is not the token's top-k"
        return z
    if regime == "zipf":
        perm = rng_for(seed, shape.cfg, layer, S_RANK).permutation(E)
        rank = np.empty(E, np.float64)
        rank[perm] = np.arange(1, E + 1)
        bias = (-zipf_s * np.log(rank)).astype(np.float32)
        return (z + bias[None, :]).astype(np.float32)
    if regime == "disjoint":
        for t in range(n_tokens):
            ids = (np.arange(k) + t * k) % E
            z[t, ids] += np.float32(8.0)
        return z
    if regime == "same":
        z[:] = z[0:1]
        return z
    raise ValueError(f"unknown routing regime {regime!r}")


# ------------------------------------------------- device-side bulk weights
def quantize_affine_torch(w, bits: int = 4, group: int = GROUP):
    """:func:`quantize_affine` on a torch tensor ``w[n, rows, cols]`` (any
    device), bit-identical to the numpy version on the same fp32 values.
    Returns int32 words [n, rows, cols*bits/32] and int16 fp16-bit scale/bias."""
    import torch

    n, rows, cols = w.shape
    lv = float(2 ** bits - 1)
    grp = w.reshape(n, rows, cols // group, group)
    mn = grp.amin(dim=3)
    mx = grp.amax(dim=3)
    s16 = ((mx - mn) / lv).half()
    b16 = mn.half()
    s = s16.float().unsqueeze(3)
    b = b16.float().unsqueeze(3)
    safe = torch.where(s == 0, torch.ones_like(s), s)
    q = torch.round((grp - b) / safe) * (s != 0)
    q = q.clamp_(0, lv).to(torch.int64).view(n, rows, cols)
    # the row's bit stream, 32 bits per word, lowest first
    bit = torch.arange(bits, device=w.device, dtype=torch.int64)
    stream = ((q.unsqueeze(3) >> bit) & 1).view(n, rows, cols * bits // 32, 32)
    shifts = torch.arange(32, device=w.device, dtype=torch.int64)
    words = (stream << shifts).sum(dim=3)  # < 2^32, in int64
    words = torch.where(words >= 2 ** 31, words - 2 ** 32, words).to(torch.int32)
    return words, s16.view(torch.int16), b16.view(torch.int16)


def quantize_affine4_torch(w):
    """:func:`quantize_affine_torch` at 4 bits, groups of 64."""
    return quantize_affine_torch(w, 4, GROUP)


def make_layer_device(shape: Shape, layer: int, device, seed: int = 0, std: float = 0.02,
                      chunk_experts: int = 8):
    """Same recipe as :func:`make_layer` (N(0,std), affine quantisation at the
    shape's widths and group size) drawn with torch's generator on
    ``device``, for benchmark volumes (GBs of weights).

    The bytes differ from :func:`make_layer` (another random stream); the
    distribution and storage layout are the same.  Returns a dict of device
    tensors named like :class:`Layer`'s fields.
    """
    import torch

    E, H, F = shape.n_experts, shape.hidden, shape.dff
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([seed, shape.cfg, layer, 9]).generate_state(1)[0]))
    out = {}
    for name, rows, cols, nb in (("gate", F, H, shape.bits), ("up", F, H, shape.bits),
                                 ("down", H, F, shape.down_bits)):
        qs, ss, bs = [], [], []
        for e0 in range(0, E, chunk_experts):
            n = min(chunk_experts, E - e0)
            w = torch.randn((n, rows, cols), generator=g, device=device, dtype=torch.float32)
            w.mul_(std)
            q, s, b = quantize_affine_torch(w, nb, shape.group_size)
            qs.append(q)
            ss.append(s)
            bs.append(b)
            del w
        out[name + "_q"] = torch.cat(qs)
        out[name + "_s"] = torch.cat(ss)
        out[name + "_b"] = torch.cat(bs)
    if shape.sidecar:
        sc = rng_for(seed, shape.cfg, layer, S_SIDECAR).uniform(0.5, 1.5, E).astype(np.float32)
        out["sidecar"] = torch.from_numpy(sc).to(device)
    else:
        out["sidecar"] = None
    return out


def expert_ids_for(idx: np.ndarray) -> Sequence[int]:
    """Distinct expert ids present in a routing array (for making only those)."""
    return sorted(set(int(v) for v in np.asarray(idx).ravel()))
