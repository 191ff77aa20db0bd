"""Python access to the C oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE ONLY.  Importing, calling or linking anything under
``oracle/`` is reserved to the tests, the smoke check and the benchmark's
CPU-baseline leg; the product path (the HIP library and its binding) never
does, and this module never imports the product package.

``build()`` compiles the oracle with gcc (plain C11, fp64, OpenMP, no
fast-math, no FMA contraction) into ``oracle/_build/libmoe_oracle.so``.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libmoe_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call([
            "gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-fPIC", "-shared", "-Wall", "-o", tmp, SRC, "-lm",
        ])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Layer(C.Structure):
    _fields_ = [
        ("hidden", C.c_int32), ("dff", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32),
        ("x_is_bf16", C.c_int32), ("clamp_limit", C.c_double),
        ("gate_q", C.c_void_p), ("up_q", C.c_void_p), ("down_q", C.c_void_p),
        ("gate_s", C.c_void_p), ("gate_b", C.c_void_p), ("up_s", C.c_void_p), ("up_b", C.c_void_p),
        ("down_s", C.c_void_p), ("down_b", C.c_void_p),
        ("sidecar", C.c_void_p),
        ("activation", C.c_int32), ("down_sidecar", C.c_void_p),
        ("bits", C.c_int32), ("down_bits", C.c_int32), ("group_size", C.c_int32),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC):
            build(force=True)
        L = C.CDLL(LIB_PATH)
        vp, i32, sz = C.c_void_p, C.c_int, C.c_size_t
        L.orc_route_topk.argtypes = [vp, i32, i32, i32, vp, vp]
        L.orc_plan.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp]
        L.orc_decode_step.argtypes = [C.POINTER(_Layer), vp, i32, vp, vp, vp, vp, vp]
        L.orc_dequant.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp]
        L.orc_round_bf16.argtypes = [vp, sz, vp]
        L.orc_round_f32.argtypes = [vp, sz, vp]
        L.orc_residual_bf16.argtypes = [vp, vp, sz, vp]
        L.orc_f16_to_f64.argtypes = [C.c_uint16]
        L.orc_f16_to_f64.restype = C.c_double
        L.orc_f64_to_bf16.argtypes = [C.c_double]
        L.orc_f64_to_bf16.restype = C.c_uint16
        L.orc_router_logits.argtypes = [vp, i32, i32, i32, i32, vp, vp]
        for f in ("orc_route_topk", "orc_plan", "orc_decode_step", "orc_router_logits"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def set_threads(n: int) -> int:
    """OpenMP threads the oracle uses from now on (process-wide); returns
    the number in effect.  Only the CPU-baseline timing changes it."""
    lib()
    gomp = C.CDLL("libgomp.so.1")
    gomp.omp_set_num_threads(C.c_int(int(n)))
    gomp.omp_get_max_threads.restype = C.c_int
    return int(gomp.omp_get_max_threads())


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def route_topk(logits: np.ndarray, top_k: int):
    """Router: idx int32 [B,k] (descending logit, ties to lower id) and fp64 weights."""
    lg = _c(logits, np.float32)
    B, E = lg.shape
    idx = np.zeros((B, top_k), np.int32)
    w = np.zeros((B, top_k), np.float64)
    rc = lib().orc_route_topk(_p(lg), B, E, top_k, _p(idx), _p(w))
    if rc:
        raise ValueError("oracle route: bad sizes")
    return idx, w


def plan(idx: np.ndarray, n_experts: int):
    """Dedup plan: counts, offsets, sorted_slots, unique_experts, n_unique."""
    ix = _c(idx, np.int32)
    B, k = ix.shape
    counts = np.zeros(n_experts, np.int32)
    offsets = np.zeros(n_experts + 1, np.int32)
    sorted_slots = np.zeros(max(B * k, 1), np.int32)[: B * k]
    unique = np.zeros(n_experts, np.int32)
    nu = np.zeros(1, np.int32)
    rc = lib().orc_plan(_p(ix), B, n_experts, k, _p(counts), _p(offsets), _p(sorted_slots), _p(unique), _p(nu))
    if rc:
        raise ValueError("oracle plan: expert id out of range")
    return dict(counts=counts, offsets=offsets, sorted_slots=sorted_slots,
                unique_experts=unique, n_unique=int(nu[0]))


def _layer_struct(layer, x_is_bf16: bool, keep: list) -> _Layer:
    sh = layer.shape
    arrs = {}
    for name in ("gate_q", "up_q", "down_q"):
        arrs[name] = _c(getattr(layer, name), np.uint32)
    for name in ("gate_s", "gate_b", "up_s", "up_b", "down_s", "down_b"):
        arrs[name] = _c(getattr(layer, name), np.uint16)
    sc = None if layer.sidecar is None else _c(layer.sidecar, np.float32)
    dsc = getattr(layer, "down_sidecar", None)
    dsc = None if dsc is None else _c(dsc, np.float32)
    keep.extend(arrs.values())
    keep.extend(a for a in (sc, dsc) if a is not None)
    act = getattr(layer, "activation", "swiglu")
    if act not in ("swiglu", "geglu"):
        raise ValueError(f"oracle: unknown activation {act}")
    st = _Layer(hidden=sh.hidden, dff=sh.dff, n_experts=sh.n_experts, top_k=sh.top_k,
                x_is_bf16=1 if x_is_bf16 else 0, clamp_limit=float(layer.clamp or 0.0),
                sidecar=None if sc is None else sc.ctypes.data,
                activation=1 if act == "geglu" else 0,
                down_sidecar=None if dsc is None else dsc.ctypes.data,
                bits=getattr(sh, "bits", 4), down_bits=getattr(sh, "down_bits", 4),
                group_size=getattr(sh, "group_size", 64))
    for name, a in arrs.items():
        setattr(st, name, a.ctypes.data)
    return st


def decode_step(layer, x: np.ndarray, idx: np.ndarray, w: np.ndarray,
                want_h: bool = False, want_y: bool = False):
    """Expert block of one decode step in fp64.

    ``x``: fp32 [B,H] or bf16 bit patterns (uint16) [B,H].  Returns the
    unrounded fp64 output [B,H], plus h [B*k,F] and y [B*k,H] on request.
    """
    sh = layer.shape
    x_is_bf16 = x.dtype == np.uint16
    xc = _c(x, np.uint16 if x_is_bf16 else np.float32)
    ix = _c(idx, np.int32)
    ww = _c(w, np.float64)
    B = xc.shape[0]
    keep: list = []
    st = _layer_struct(layer, x_is_bf16, keep)
    out = np.zeros((B, sh.hidden), np.float64)
    h = np.zeros((B * sh.top_k, sh.dff), np.float64) if want_h else None
    y = np.zeros((B * sh.top_k, sh.hidden), np.float64) if want_y else None
    rc = lib().orc_decode_step(C.byref(st), _p(xc), B, _p(ix), _p(ww), _p(out),
                               None if h is None else _p(h), None if y is None else _p(y))
    if rc:
        raise ValueError("oracle decode_step: bad arguments")
    res = [out]
    if want_h:
        res.append(h)
    if want_y:
        res.append(y)
    return res[0] if len(res) == 1 else tuple(res)


def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """Router projection in fp64: x fp32 [B,H] or bf16 bits [B,H], w_router
    bf16 bits [E,H] -> logits [B,E] = x . Wr^T."""
    x_is_bf16 = x.dtype == np.uint16
    xc = _c(x, np.uint16 if x_is_bf16 else np.float32)
    wc = _c(w_router, np.uint16)
    B, H = xc.shape
    E, H2 = wc.shape
    if H != H2:
        raise ValueError("oracle router_logits: hidden sizes differ")
    out = np.zeros((B, E), np.float64)
    if lib().orc_router_logits(_p(xc), 1 if x_is_bf16 else 0, B, H, E, _p(wc), _p(out)):
        raise ValueError("oracle router_logits: bad sizes")
    return out


def dequant(q: np.ndarray, s: np.ndarray, b: np.ndarray, bits: int = 4, group: int = 64) -> np.ndarray:
    """Dense fp64 [rows, cols] of one quantised matrix (q uint32 [rows, words])."""
    qc, sc, bc = _c(q, np.uint32), _c(s, np.uint16), _c(b, np.uint16)
    rows, words = qc.shape
    if (words * 32) % bits:
        raise ValueError("oracle dequant: words do not hold whole elements")
    cols = words * 32 // bits
    if cols % group or sc.shape != (rows, cols // group) or bc.shape != sc.shape:
        raise ValueError("oracle dequant: scale/bias shape does not match the groups")
    out = np.zeros((rows, cols), np.float64)
    lib().orc_dequant(_p(qc), _p(sc), _p(bc), rows, cols, bits, group, _p(out))
    return out


def round_bf16(v: np.ndarray) -> np.ndarray:
    vc = _c(v, np.float64)
    out = np.zeros(vc.shape, np.uint16)
    lib().orc_round_bf16(_p(vc), vc.size, _p(out))
    return out


def round_f32(v: np.ndarray) -> np.ndarray:
    vc = _c(v, np.float64)
    out = np.zeros(vc.shape, np.float32)
    lib().orc_round_f32(_p(vc), vc.size, _p(out))
    return out


def residual_bf16(x_bits: np.ndarray, out64: np.ndarray) -> np.ndarray:
    xc = _c(x_bits, np.uint16)
    oc = _c(out64, np.float64)
    assert xc.shape == oc.shape
    nxt = np.zeros(xc.shape, np.uint16)
    lib().orc_residual_bf16(_p(xc), _p(oc), xc.size, _p(nxt))
    return nxt


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_to_f64(h: int) -> float:
    return lib().orc_f16_to_f64(int(h))


def f64_to_bf16(v: float) -> int:
    return lib().orc_f64_to_bf16(float(v))


def run_stack(layers, x0_bits: np.ndarray, logits_per_layer, top_k: int,
              hook: Optional[callable] = None):
    """The layer stack: per layer route -> expert block -> residual with the
    two bf16 roundings, x_{l+1} = bf16(f32(x_l) + f32(bf16(out_l))).
    ``hook(l, x_l, idx, w, out64)`` sees every layer.  Returns the final x."""
    x = _c(x0_bits, np.uint16)
    for l, (layer, lg) in enumerate(zip(layers, logits_per_layer)):
        idx, w = route_topk(lg, top_k)
        out = decode_step(layer, x, idx, w)
        if hook is not None:
            hook(l, x, idx, w, out)
        x = residual_bf16(x, out)
    return x
