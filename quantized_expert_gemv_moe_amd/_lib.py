"""ctypes binding of ``libmoe_decode.so`` (include/moe_decode.h).

Argument marshalling only: every step of the decode block runs in the HIP
kernels behind the C ABI.  torch is used for device memory and the current
HIP stream.  There is no fallback: if the library is not built, or a call
returns an error status, this module raises.
"""

from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch

from . import build as _build

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
MOE_DOWN_ROWS, MOE_DOWN_COLS = 0, 1
MOE_ACT_SWIGLU, MOE_ACT_GEGLU = 0, 1
_ACTIVATIONS = {"swiglu": MOE_ACT_SWIGLU, "geglu": MOE_ACT_GEGLU}
MOE_MAX_EXPERTS = 1024
MOE_MAX_TOP_K = 16
MOE_MAX_TOKENS = 65535
MOE_STATIC_SCRATCH_BYTES = 8 << 20


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


class LayerStruct(C.Structure):
    _fields_ = [
        ("hidden", C.c_int32), ("dff", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32),
        ("bits", C.c_int32), ("group_size", C.c_int32), ("act_dtype", C.c_int32),
        ("clamp_limit", C.c_float),
        ("gate_q", C.c_void_p), ("up_q", C.c_void_p),
        ("gate_s", C.c_void_p), ("gate_b", C.c_void_p), ("up_s", C.c_void_p), ("up_b", C.c_void_p),
        ("down_q", C.c_void_p), ("down_s", C.c_void_p), ("down_b", C.c_void_p),
        ("expert_scale", C.c_void_p),
        ("down_layout", C.c_int32), ("down_scale", C.c_void_p), ("activation", C.c_int32),
        ("down_bits", C.c_int32),
    ]


class PlanStruct(C.Structure):
    _fields_ = [("counts", C.c_void_p), ("offsets", C.c_void_p), ("sorted_slots", C.c_void_p),
                ("unique_experts", C.c_void_p), ("n_unique", C.c_void_p), ("work", C.c_void_p)]


_lib = None

EXPORTS = ("moe_router_logits", "moe_route_topk", "moe_expert_plan", "moe_route_plan", "moe_workspace_size",
           "moe_decode_step", "moe_decode_step_residual",
           "moe_decode_layer", "moe_decode_layer_static", "moe_route_gate_up", "moe_expert_gate_up", "moe_expert_down_combine", "moe_pack_down",
           "moe_layer_check", "moe_status_str", "moe_abi_version")


def library_path() -> str:
    return _build.LIB_PATH


def lib() -> C.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"HIP library {path} is not built; run __graft_entry__.build() "
                "or python -m quantized_expert_gemv_moe_amd.build")
        L = C.CDLL(path)
        vp, i32 = C.c_void_p, C.c_int32
        L.moe_router_logits.argtypes = [vp, i32, i32, C.c_int, vp, i32, vp, vp]
        L.moe_router_logits.restype = C.c_int
        L.moe_route_topk.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.moe_route_topk.restype = C.c_int
        L.moe_expert_plan.argtypes = [vp, i32, i32, i32, C.POINTER(PlanStruct), vp]
        L.moe_expert_plan.restype = C.c_int
        L.moe_route_plan.argtypes = [vp, i32, i32, i32, vp, vp, C.POINTER(PlanStruct), vp]
        L.moe_route_plan.restype = C.c_int
        L.moe_workspace_size.argtypes = [C.POINTER(LayerStruct), i32]
        L.moe_workspace_size.restype = C.c_size_t
        L.moe_decode_step.argtypes = [C.POINTER(LayerStruct), vp, i32, vp, vp, C.POINTER(PlanStruct),
                                      vp, vp, C.c_size_t, vp]
        L.moe_decode_step.restype = C.c_int
        L.moe_decode_step_residual.argtypes = [C.POINTER(LayerStruct), vp, i32, vp, vp, C.POINTER(PlanStruct),
                                               vp, vp, vp, C.c_size_t, vp]
        L.moe_decode_step_residual.restype = C.c_int
        L.moe_decode_layer.argtypes = [C.POINTER(LayerStruct), vp, vp, i32, vp, vp, C.POINTER(PlanStruct),
                                       vp, vp, vp, C.c_size_t, vp]
        L.moe_decode_layer.restype = C.c_int
        L.moe_decode_layer_static.argtypes = [C.POINTER(LayerStruct), vp, vp, i32, vp, vp, C.POINTER(PlanStruct),
                                              vp, vp, vp]
        L.moe_decode_layer_static.restype = C.c_int
        L.moe_route_gate_up.argtypes = [C.POINTER(LayerStruct), vp, vp, i32, vp, vp, C.POINTER(PlanStruct),
                                        vp, C.c_size_t, vp]
        L.moe_route_gate_up.restype = C.c_int
        L.moe_expert_gate_up.argtypes = [C.POINTER(LayerStruct), vp, i32, C.POINTER(PlanStruct), vp,
                                         C.c_size_t, vp]
        L.moe_expert_gate_up.restype = C.c_int
        L.moe_expert_down_combine.argtypes = [C.POINTER(LayerStruct), i32, vp, vp, C.POINTER(PlanStruct), vp,
                                              vp, vp, C.c_size_t, vp]
        L.moe_expert_down_combine.restype = C.c_int
        L.moe_pack_down.argtypes = [C.POINTER(LayerStruct), vp, vp, vp, vp]
        L.moe_pack_down.restype = C.c_int
        L.moe_layer_check.argtypes = [C.POINTER(LayerStruct)]
        L.moe_layer_check.restype = C.c_int
        L.moe_status_str.argtypes = [C.c_int]
        L.moe_status_str.restype = C.c_char_p
        L.moe_abi_version.argtypes = []
        L.moe_abi_version.restype = C.c_int32
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


# ------------------------------------------------------- argument checks
# The C ABI validates everything it can see on the host (shapes in the layer
# struct, alignment, workspace size); the extents and dtypes of the device
# buffers it is handed are the caller's contract.  These checks hold every
# tensor to that contract before the call, so a wrong-sized buffer raises
# here instead of reaching a kernel.
def _act_dtype(layer: "DeviceLayer"):
    return torch.bfloat16 if layer.act_dtype == MOE_DTYPE_BF16 else torch.float32


def _need(t: Optional[torch.Tensor], name: str, dtype, shape):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous {dtype} device tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")


def _check_x(layer: "DeviceLayer", x: torch.Tensor, name: str = "x") -> int:
    if x is None or x.dim() != 2:
        raise ValueError(f"{name} must be a [B, hidden] tensor")
    _need(x, name, _act_dtype(layer), (x.shape[0], layer.hidden))
    return x.shape[0]


def _check_routing(layer: "DeviceLayer", B: int, idx: torch.Tensor, w: torch.Tensor):
    _need(idx, "idx", torch.int32, (B, layer.top_k))
    _need(w, "w", torch.float32, (B, layer.top_k))


def _check_plan_buffers(plan: "Plan", n_experts: int, n_slots: int):
    E = n_experts
    if (plan.counts.numel() < E or plan.offsets.numel() < E + 1 or plan.unique_experts.numel() < E
            or plan.work.numel() < 4 * E or plan.sorted_slots.numel() < n_slots or plan.n_unique.numel() < 1):
        raise ValueError("plan buffers are too small for this layer and batch")
    for t in (plan.counts, plan.offsets, plan.sorted_slots, plan.unique_experts, plan.n_unique, plan.work):
        if t.dtype != torch.int32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("plan buffers must be contiguous int32 device tensors")


def _check_plan(layer: "DeviceLayer", plan: "Plan", B: int):
    _check_plan_buffers(plan, layer.n_experts, B * layer.top_k)


def _check_logits(logits: torch.Tensor):
    if (logits is None or logits.dtype != torch.float32 or logits.dim() != 2 or not logits.is_contiguous()
            or not logits.is_cuda):
        raise ValueError("logits must be a contiguous fp32 [B, E] device tensor")


def _check_out(layer: "DeviceLayer", B: int, out: torch.Tensor, residual: Optional[torch.Tensor]):
    _need(out, "out", _act_dtype(layer), (B, layer.hidden))
    if residual is not None:
        _need(residual, "residual", _act_dtype(layer), (B, layer.hidden))


def _check_workspace(layer: "DeviceLayer", B: int, workspace: torch.Tensor):
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    need = workspace_size(layer, B)
    have = workspace.numel() * workspace.element_size()
    if have < need:
        raise ValueError(f"workspace holds {have} bytes, {need} needed for {B} tokens")


# ------------------------------------------------------------------- layer
@dataclass
class DeviceLayer:
    """Device tensors of one layer plus the ABI descriptor pointing at them."""

    hidden: int
    dff: int
    n_experts: int
    top_k: int
    act_dtype: int
    clamp_limit: float
    tensors: dict
    struct: LayerStruct
    down_layout: int = MOE_DOWN_ROWS
    activation: str = "swiglu"
    bits: int = 4
    down_bits: int = 4
    group_size: int = 64

    @staticmethod
    def from_tensors(hidden, dff, n_experts, top_k, act: str, clamp_limit: float, tensors: dict,
                     down_layout: int = MOE_DOWN_ROWS, activation: str = "swiglu", bits: int = 4,
                     down_bits: int = 4, group_size: int = 64):
        """``tensors``: gate_q/up_q/down_q (int32 or uint32 words), *_s/*_b (fp16 bits as
        int16/uint16), optional 'sidecar' (fp32 [E], on gate and up) and 'down_sidecar'
        (fp32 [E], on the down output); all on the same device.  ``activation`` is
        "swiglu" or "geglu"; ``bits`` (gate/up) and ``down_bits`` are 4, 6 or 8,
        ``group_size`` 32, 64 or 128."""
        if activation not in _ACTIVATIONS:
            raise ValueError(f"activation must be one of {sorted(_ACTIVATIONS)}")
        t = {k: v for k, v in tensors.items() if v is not None}
        for k, v in t.items():
            if not v.is_contiguous():
                raise ValueError(f"{k} must be contiguous")
        st = LayerStruct(hidden=hidden, dff=dff, n_experts=n_experts, top_k=top_k, bits=bits,
                         group_size=group_size, act_dtype=MOE_DTYPE_BF16 if act == "bf16" else MOE_DTYPE_F32,
                         clamp_limit=float(clamp_limit), down_layout=down_layout,
                         activation=_ACTIVATIONS[activation], down_bits=down_bits)
        for name in ("gate_q", "up_q", "down_q", "gate_s", "gate_b", "up_s", "up_b", "down_s", "down_b"):
            setattr(st, name, t[name].data_ptr())
        sc = t.get("sidecar")
        st.expert_scale = None if sc is None else sc.data_ptr()
        ds = t.get("down_sidecar")
        st.down_scale = None if ds is None else ds.data_ptr()
        return DeviceLayer(hidden, dff, n_experts, top_k, st.act_dtype, float(clamp_limit), t, st, down_layout,
                           activation, bits, down_bits, group_size)

    def pack_down(self, stream=None, free_rows: bool = False) -> "DeviceLayer":
        """A copy of this layer whose down projection is regrouped to MOE_DOWN_COLS
        (moe_pack_down); gate/up and the sidecars are shared."""
        if self.down_layout != MOE_DOWN_ROWS:
            raise ValueError("the down projection is already packed")
        t = dict(self.tensors)
        q = torch.empty_like(t["down_q"])
        s = torch.empty_like(t["down_s"])
        b = torch.empty_like(t["down_b"])
        _check(lib().moe_pack_down(C.byref(self.struct), _ptr(q), _ptr(s), _ptr(b), _stream(stream)),
               "moe_pack_down")
        if free_rows:
            torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
        t["down_q"], t["down_s"], t["down_b"] = q, s, b
        act = "bf16" if self.act_dtype == MOE_DTYPE_BF16 else "f32"
        return DeviceLayer.from_tensors(self.hidden, self.dff, self.n_experts, self.top_k, act, self.clamp_limit,
                                        t, down_layout=MOE_DOWN_COLS, activation=self.activation, bits=self.bits,
                                        down_bits=self.down_bits, group_size=self.group_size)

    @staticmethod
    def from_host(layer, device="cuda"):
        """Copy a ``moe_workloads.Layer`` (numpy) to the device."""
        import numpy as np

        def dev(a, dt):
            return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)

        sh = layer.shape
        t = {}
        for n in ("gate_q", "up_q", "down_q"):
            t[n] = dev(getattr(layer, n), np.int32)
        for n in ("gate_s", "gate_b", "up_s", "up_b", "down_s", "down_b"):
            t[n] = dev(getattr(layer, n), np.int16)
        t["sidecar"] = None if layer.sidecar is None else dev(layer.sidecar.astype(np.float32), np.float32)
        t["down_sidecar"] = (None if layer.down_sidecar is None
                             else dev(layer.down_sidecar.astype(np.float32), np.float32))
        return DeviceLayer.from_tensors(sh.hidden, sh.dff, sh.n_experts, sh.top_k, sh.act,
                                        layer.clamp or 0.0, t, activation=layer.activation, bits=sh.bits,
                                        down_bits=sh.down_bits, group_size=sh.group_size)

    def check(self) -> int:
        return lib().moe_layer_check(C.byref(self.struct))


# -------------------------------------------------------------------- plan
@dataclass
class Plan:
    counts: torch.Tensor
    offsets: torch.Tensor
    sorted_slots: torch.Tensor
    unique_experts: torch.Tensor
    n_unique: torch.Tensor
    work: torch.Tensor
    struct: PlanStruct

    @staticmethod
    def allocate(n_experts: int, max_slots: int, device="cuda") -> "Plan":
        i32 = dict(dtype=torch.int32, device=device)
        p = [torch.empty(n_experts, **i32), torch.empty(n_experts + 1, **i32),
             torch.empty(max(max_slots, 1), **i32), torch.empty(n_experts, **i32), torch.empty(1, **i32),
             torch.empty((n_experts, 4), **i32)]
        st = PlanStruct(*[x.data_ptr() for x in p])
        return Plan(*p, st)


# ------------------------------------------------------------- entry points
def router_logits(x: torch.Tensor, w_router: torch.Tensor, logits: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """moe_router_logits: x [B,H] (bf16 or fp32), w_router bf16 [E,H] -> fp32 logits [B,E]."""
    if x.dim() != 2 or not x.is_contiguous() or x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("x must be a contiguous bf16 or fp32 [B, H] tensor")
    if w_router.dim() != 2 or not w_router.is_contiguous() or w_router.dtype != torch.bfloat16:
        raise ValueError("w_router must be a contiguous bf16 [E, H] tensor")
    B, H = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != H:
        raise ValueError("x and w_router disagree on hidden")
    if logits is None:
        logits = torch.empty((B, E), dtype=torch.float32, device=x.device)
    act = MOE_DTYPE_BF16 if x.dtype == torch.bfloat16 else MOE_DTYPE_F32
    _check(lib().moe_router_logits(_ptr(x), B, H, act, _ptr(w_router), E, _ptr(logits), _stream(stream)),
           "moe_router_logits")
    return logits


def route_topk(logits: torch.Tensor, top_k: int, idx: Optional[torch.Tensor] = None,
               w: Optional[torch.Tensor] = None, stream=None):
    """moe_route_topk: fp32 logits [B,E] -> (int32 idx [B,k], fp32 w [B,k])."""
    _check_logits(logits)
    B, E = logits.shape
    if idx is None:
        idx = torch.empty((B, top_k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((B, top_k), dtype=torch.float32, device=logits.device)
    _need(idx, "idx", torch.int32, (B, top_k))
    _need(w, "w", torch.float32, (B, top_k))
    _check(lib().moe_route_topk(_ptr(logits), B, E, top_k, _ptr(idx), _ptr(w), _stream(stream)),
           "moe_route_topk")
    return idx, w


def expert_plan(idx: torch.Tensor, n_experts: int, plan: Optional[Plan] = None, stream=None) -> Plan:
    """moe_expert_plan over int32 idx [B,k]."""
    if idx.dtype != torch.int32 or idx.dim() != 2 or not idx.is_contiguous() or not idx.is_cuda:
        raise ValueError("idx must be a contiguous int32 [B, k] device tensor")
    B, k = idx.shape
    if plan is None:
        plan = Plan.allocate(n_experts, B * k, device=idx.device)
    _check_plan_buffers(plan, n_experts, B * k)
    _check(lib().moe_expert_plan(_ptr(idx), B, n_experts, k, C.byref(plan.struct), _stream(stream)),
           "moe_expert_plan")
    return plan


def route_plan(logits: torch.Tensor, top_k: int, plan: Optional[Plan] = None, idx: Optional[torch.Tensor] = None,
               w: Optional[torch.Tensor] = None, stream=None):
    """moe_route_plan: router and planner in one launch; returns (idx, w, plan)."""
    _check_logits(logits)
    B, E = logits.shape
    if idx is None:
        idx = torch.empty((B, top_k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((B, top_k), dtype=torch.float32, device=logits.device)
    if plan is None:
        plan = Plan.allocate(E, B * top_k, device=logits.device)
    _need(idx, "idx", torch.int32, (B, top_k))
    _need(w, "w", torch.float32, (B, top_k))
    _check_plan_buffers(plan, E, B * top_k)
    _check(lib().moe_route_plan(_ptr(logits), B, E, top_k, _ptr(idx), _ptr(w), C.byref(plan.struct),
                                _stream(stream)), "moe_route_plan")
    return idx, w, plan


def workspace_size(layer: DeviceLayer, max_tokens: int) -> int:
    return int(lib().moe_workspace_size(C.byref(layer.struct), int(max_tokens)))


def alloc_workspace(layer: DeviceLayer, max_tokens: int, device="cuda") -> torch.Tensor:
    n = workspace_size(layer, max_tokens)
    if n == 0 and max_tokens > 0:
        raise MoeError(layer.check() or MOE_ERR_INVALID_ARG, "moe_workspace_size")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def decode_step(layer: DeviceLayer, x: torch.Tensor, idx: torch.Tensor, w: torch.Tensor, plan: Plan,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                residual: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """moe_decode_step: x [B,H] (bf16 or fp32 per the layer) -> out [B,H];
    with a residual, moe_decode_step_residual (out = residual + the block)."""
    B = _check_x(layer, x)
    _check_routing(layer, B, idx, w)
    _check_plan(layer, plan, B)
    if out is None:
        out = torch.empty_like(x)
    _check_out(layer, B, out, residual)
    if workspace is None:
        workspace = alloc_workspace(layer, B, device=x.device)
    _check_workspace(layer, B, workspace)
    if residual is None:
        _check(lib().moe_decode_step(C.byref(layer.struct), _ptr(x), B, _ptr(idx), _ptr(w), C.byref(plan.struct),
                                     _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)),
               "moe_decode_step")
    else:
        _check(lib().moe_decode_step_residual(C.byref(layer.struct), _ptr(x), B, _ptr(idx), _ptr(w),
                                              C.byref(plan.struct), _ptr(residual), _ptr(out), _ptr(workspace),
                                              workspace.numel(), _stream(stream)), "moe_decode_step_residual")
    return out


def route_gate_up(layer: DeviceLayer, x: torch.Tensor, logits: torch.Tensor, idx: torch.Tensor, w: torch.Tensor,
                  plan: Plan, workspace: torch.Tensor, stream=None):
    """moe_route_gate_up: first half of decode_layer (routing, plan, h into the workspace)."""
    B = _check_x(layer, x)
    _need(logits, "logits", torch.float32, (B, layer.n_experts))
    _check_routing(layer, B, idx, w)
    _check_plan(layer, plan, B)
    _check_workspace(layer, B, workspace)
    _check(lib().moe_route_gate_up(C.byref(layer.struct), _ptr(logits), _ptr(x), x.shape[0], _ptr(idx), _ptr(w),
                                   C.byref(plan.struct), _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_route_gate_up")
    return idx, w, plan


def expert_gate_up(layer: DeviceLayer, x: torch.Tensor, plan: Plan, workspace: torch.Tensor, stream=None):
    """moe_expert_gate_up: first half of decode_step (h into the workspace)."""
    B = _check_x(layer, x)
    _check_plan(layer, plan, B)
    _check_workspace(layer, B, workspace)
    _check(lib().moe_expert_gate_up(C.byref(layer.struct), _ptr(x), x.shape[0], C.byref(plan.struct),
                                    _ptr(workspace), workspace.numel(), _stream(stream)), "moe_expert_gate_up")


def expert_down_combine(layer: DeviceLayer, n_tokens: int, idx: torch.Tensor, w: torch.Tensor, plan: Plan,
                        out: torch.Tensor, workspace: torch.Tensor, residual: Optional[torch.Tensor] = None,
                        stream=None):
    """moe_expert_down_combine: second half of decode_step."""
    B = int(n_tokens)
    _check_routing(layer, B, idx, w)
    _check_plan(layer, plan, B)
    _check_out(layer, B, out, residual)
    _check_workspace(layer, B, workspace)
    _check(lib().moe_expert_down_combine(C.byref(layer.struct), n_tokens, _ptr(idx), _ptr(w), C.byref(plan.struct),
                                         _ptr(residual), _ptr(out), _ptr(workspace), workspace.numel(),
                                         _stream(stream)), "moe_expert_down_combine")
    return out


def decode_layer(layer: DeviceLayer, x: torch.Tensor, logits: torch.Tensor, plan: Optional[Plan] = None,
                 workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 residual: Optional[torch.Tensor] = None, bufs: Optional[dict] = None, stream=None):
    """moe_decode_layer: one layer step from router logits (router, planner,
    expert block); returns (out, idx, w, plan)."""
    B = _check_x(layer, x)
    E = layer.n_experts
    _need(logits, "logits", torch.float32, (B, E))
    bufs = bufs or {}
    k = layer.top_k
    idx = bufs.get("idx")
    w = bufs.get("w")
    if idx is None:
        idx = torch.empty((B, k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((B, k), dtype=torch.float32, device=logits.device)
    if plan is None:
        plan = Plan.allocate(E, B * k, device=logits.device)
    _check_routing(layer, B, idx, w)
    _check_plan(layer, plan, B)
    if out is None:
        out = torch.empty_like(x)
    _check_out(layer, B, out, residual)
    if workspace is None:
        workspace = alloc_workspace(layer, B, device=x.device)
    _check_workspace(layer, B, workspace)
    _check(lib().moe_decode_layer(C.byref(layer.struct), _ptr(logits), _ptr(x), B, _ptr(idx), _ptr(w),
                                  C.byref(plan.struct), _ptr(residual), _ptr(out), _ptr(workspace),
                                  workspace.numel(), _stream(stream)), "moe_decode_layer")
    return out, idx, w, plan


def decode_layer_static(layer: DeviceLayer, x: torch.Tensor, logits: torch.Tensor, plan: Plan, out: torch.Tensor,
                        idx: torch.Tensor, w: torch.Tensor, residual: Optional[torch.Tensor] = None, stream=None):
    """moe_decode_layer_static: moe_decode_layer without a workspace (the library's
    per-device scratch array holds h and y).  Every buffer is the caller's:
    nothing is allocated here either."""
    B = _check_x(layer, x)
    _need(logits, "logits", torch.float32, (B, layer.n_experts))
    _check_routing(layer, B, idx, w)
    _check_plan(layer, plan, B)
    _check_out(layer, B, out, residual)
    _check(lib().moe_decode_layer_static(C.byref(layer.struct), _ptr(logits), _ptr(x), B, _ptr(idx), _ptr(w),
                                         C.byref(plan.struct), _ptr(residual), _ptr(out), _stream(stream)),
           "moe_decode_layer_static")
    return out
