"""The C ABI on the host (no GPU): exports, status codes, validation, sizing.

Every call here returns before anything is enqueued, so no device is touched:
invalid arguments are rejected on the host, and n_tokens == 0 returns
without a launch.
"""

import ctypes as C
import os
import re

import pytest

import quantized_expert_gemv_moe_amd as moe
from quantized_expert_gemv_moe_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_decode.h")

FAKE = 0x7F0000000000  # aligned, never dereferenced by host validation


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = moe.lib()
    declared = header_functions()
    assert set(declared) == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    assert L.moe_abi_version() == 8


def test_status_strings():
    for s in range(5):
        assert moe.status_str(s)
    assert "unsupported" in moe.status_str(moe.MOE_ERR_UNSUPPORTED)
    assert moe.status_str(99) == "unknown status"


def layer(**kw):
    st = _lib.LayerStruct(hidden=2048, dff=768, n_experts=128, top_k=8, bits=4, group_size=64,
                          act_dtype=moe.MOE_DTYPE_BF16, clamp_limit=0.0, down_bits=4)
    for i, n in enumerate(("gate_q", "up_q", "down_q", "gate_s", "gate_b", "up_s", "up_b", "down_s", "down_b")):
        setattr(st, n, FAKE + 0x100000 * i)
    st.expert_scale = None
    for k, v in kw.items():
        setattr(st, k, v)
    return st


def check(**kw):
    return moe.lib().moe_layer_check(C.byref(layer(**kw)))


def test_layer_check_accepts_the_workload_shapes():
    assert check() == moe.MOE_OK
    assert check(down_layout=moe.MOE_DOWN_COLS) == moe.MOE_OK
    assert check(hidden=4096, dff=2048, n_experts=256, top_k=6, down_layout=moe.MOE_DOWN_COLS) == moe.MOE_OK
    assert check(hidden=256, dff=128, n_experts=8, top_k=2, act_dtype=moe.MOE_DTYPE_F32) == moe.MOE_OK
    assert check(hidden=4096, dff=2048, n_experts=256, top_k=6, clamp_limit=10.0,
                 expert_scale=FAKE + 0x9000000) == moe.MOE_OK
    assert check(activation=moe.MOE_ACT_GEGLU, down_scale=FAKE + 0xA000000) == moe.MOE_OK
    # other widths and group sizes: the generic row kernels (rows layout)
    for bits, down_bits, group in ((8, 8, 64), (4, 6, 64), (6, 6, 32), (8, 4, 128), (4, 4, 32), (4, 4, 128)):
        assert check(bits=bits, down_bits=down_bits, group_size=group) == moe.MOE_OK
    assert check(hidden=4096, dff=2048, bits=6, down_bits=8, group_size=128) == moe.MOE_OK
    # each projection by its own width: a 4-bit group-64 down projection keeps
    # the column layout under generic gate+up kernels
    assert check(bits=8, down_layout=moe.MOE_DOWN_COLS) == moe.MOE_OK
    assert check(bits=6, hidden=4096, dff=2048, down_layout=moe.MOE_DOWN_COLS) == moe.MOE_OK
    # the largest dff the row-layout down kernel stages in LDS
    assert check(dff=6144) == moe.MOE_OK
    # a generic (8-bit) down projection has no such limit
    assert check(dff=8192, down_bits=8) == moe.MOE_OK


def test_zero_extensions_mean_the_plain_layer():
    # down_bits 0 takes gate/up's width: an 8-bit layer then has an 8-bit
    # (generic, rows-only) down projection, which refuses the column layout
    assert check(down_bits=0) == moe.MOE_OK
    assert check(bits=8, down_bits=0) == moe.MOE_OK
    assert check(bits=8, down_bits=0, down_layout=moe.MOE_DOWN_COLS) == moe.MOE_ERR_UNSUPPORTED
    assert check(bits=4, down_bits=0, down_layout=moe.MOE_DOWN_COLS) == moe.MOE_OK
    assert check(bits=3, down_bits=0) == moe.MOE_ERR_UNSUPPORTED


PLAIN_STRUCT = r"""
#include <stddef.h>
#include <stdio.h>
#include "moe_decode.h"
/* the plain 4-bit layer, field for field, as a caller that knows no
   extension declares it */
typedef struct {
    int32_t hidden, dff, n_experts, top_k, bits, group_size;
    moe_dtype act_dtype;
    float clamp_limit;
    const uint32_t *gate_q, *up_q;
    const uint16_t *gate_s, *gate_b, *up_s, *up_b;
    const uint32_t *down_q;
    const uint16_t *down_s, *down_b;
    const float *expert_scale;
} plain_layer;
typedef struct { int32_t *counts, *offsets, *sorted_slots, *unique_experts, *n_unique; } plain_plan;
#define F(S, P, f) printf("%s %s %zu %zu\n", #S, #f, offsetof(S, f), offsetof(P, f));
#define G(S, f) printf("%s %s %zu -\n", #S, #f, offsetof(S, f));
int main(void) {
    F(moe_layer_t, plain_layer, hidden) F(moe_layer_t, plain_layer, dff) F(moe_layer_t, plain_layer, n_experts)
    F(moe_layer_t, plain_layer, top_k) F(moe_layer_t, plain_layer, bits) F(moe_layer_t, plain_layer, group_size)
    F(moe_layer_t, plain_layer, act_dtype) F(moe_layer_t, plain_layer, clamp_limit)
    F(moe_layer_t, plain_layer, gate_q) F(moe_layer_t, plain_layer, up_q) F(moe_layer_t, plain_layer, gate_s)
    F(moe_layer_t, plain_layer, gate_b) F(moe_layer_t, plain_layer, up_s) F(moe_layer_t, plain_layer, up_b)
    F(moe_layer_t, plain_layer, down_q) F(moe_layer_t, plain_layer, down_s) F(moe_layer_t, plain_layer, down_b)
    F(moe_layer_t, plain_layer, expert_scale)
    G(moe_layer_t, down_layout) G(moe_layer_t, down_scale) G(moe_layer_t, activation) G(moe_layer_t, down_bits)
    F(moe_plan_t, plain_plan, counts) F(moe_plan_t, plain_plan, offsets) F(moe_plan_t, plain_plan, sorted_slots)
    F(moe_plan_t, plain_plan, unique_experts) F(moe_plan_t, plain_plan, n_unique) G(moe_plan_t, work)
    printf("sizeof %zu %zu %zu\n", sizeof(moe_layer_t), sizeof(plain_layer), sizeof(moe_plan_t));
    return 0;
}
"""


def test_struct_layout_matches_the_header_and_keeps_the_plain_prefix(tmp_path):
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "layout.c"
    src.write_text(PLAIN_STRUCT)
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run([cc, "-std=c11", "-Wall", "-Werror", "-I", inc, str(src), "-o", str(exe)], check=True)
    lines = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    py = {"moe_layer_t": _lib.LayerStruct, "moe_plan_t": _lib.PlanStruct}
    seen = 0
    for ln in lines:
        parts = ln.split()
        if not parts:
            continue
        if parts[0] == "sizeof":
            assert int(parts[1]) == C.sizeof(_lib.LayerStruct) and int(parts[3]) == C.sizeof(_lib.PlanStruct)
            assert int(parts[2]) < int(parts[1])
            continue
        struct, field, off, plain = parts
        assert getattr(py[struct], field).offset == int(off), (struct, field)
        if plain != "-":
            assert int(plain) == int(off), (struct, field)  # a plain caller's struct is a prefix
        seen += 1
    assert seen == len(_lib.LayerStruct._fields_) + len(_lib.PlanStruct._fields_)


@pytest.mark.parametrize("kw,want", [
    (dict(bits=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(bits=5), moe.MOE_ERR_UNSUPPORTED),
    (dict(down_bits=3), moe.MOE_ERR_UNSUPPORTED),
    (dict(group_size=16), moe.MOE_ERR_UNSUPPORTED),
    (dict(group_size=48), moe.MOE_ERR_UNSUPPORTED),
    (dict(dff=704, group_size=128), moe.MOE_ERR_UNSUPPORTED),          # group does not divide dff
    (dict(down_bits=8, down_layout=moe.MOE_DOWN_COLS), moe.MOE_ERR_UNSUPPORTED),  # generic down: rows only
    (dict(group_size=32, down_layout=moe.MOE_DOWN_COLS), moe.MOE_ERR_UNSUPPORTED),
    (dict(group_size=32, hidden=320 * 4, dff=320), moe.MOE_ERR_UNSUPPORTED),   # 20 units: no lane split
    (dict(bits=8, hidden=16384), moe.MOE_ERR_UNSUPPORTED),             # 1024 units: over 8 per lane
    (dict(hidden=2000), moe.MOE_ERR_UNSUPPORTED),
    (dict(dff=1408), moe.MOE_ERR_UNSUPPORTED),      # 44 chunks: no lane geometry
    (dict(n_experts=2048), moe.MOE_ERR_UNSUPPORTED),
    (dict(top_k=17, n_experts=64), moe.MOE_ERR_UNSUPPORTED),
    (dict(top_k=9, n_experts=8), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(hidden=0), moe.MOE_ERR_INVALID_ARG),
    (dict(act_dtype=7), moe.MOE_ERR_INVALID_ARG),
    (dict(clamp_limit=-1.0), moe.MOE_ERR_INVALID_ARG),
    (dict(clamp_limit=float("nan")), moe.MOE_ERR_INVALID_ARG),
    (dict(gate_q=None), moe.MOE_ERR_INVALID_ARG),
    (dict(down_q=FAKE + 8), moe.MOE_ERR_INVALID_ARG),  # not 16-byte aligned
    (dict(up_s=FAKE + 2), moe.MOE_ERR_INVALID_ARG),
    (dict(down_layout=5), moe.MOE_ERR_INVALID_ARG),
    (dict(activation=2), moe.MOE_ERR_INVALID_ARG),
    (dict(activation=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(down_scale=FAKE + 2), moe.MOE_ERR_INVALID_ARG),   # not 4-byte aligned
    (dict(dff=1152, down_layout=moe.MOE_DOWN_COLS), moe.MOE_ERR_UNSUPPORTED),  # 36 chunks: no column kernel
    (dict(dff=192, down_layout=moe.MOE_DOWN_COLS), moe.MOE_ERR_UNSUPPORTED),   # dff % 128 != 0
    # the row-layout down kernel stages one slot's h (and group sums) in
    # 32 KiB of LDS: dff 8192 has a lane geometry but no room there, so the
    # layer is refused before anything is enqueued (not after gate+up ran)
    (dict(dff=8192), moe.MOE_ERR_UNSUPPORTED),
])
def test_layer_check_rejects(kw, want):
    assert check(**kw) == want


def test_workspace_size():
    L = moe.lib()
    st = layer()
    # h [slots][dff] fp32 + y [slots][hidden] fp32, each 256-aligned
    assert L.moe_workspace_size(C.byref(st), 1) == 8 * 768 * 4 + 8 * 2048 * 4
    assert L.moe_workspace_size(C.byref(st), 32) == 256 * 768 * 4 + 256 * 2048 * 4
    assert L.moe_workspace_size(C.byref(st), 0) == 0
    assert L.moe_workspace_size(C.byref(layer(bits=3)), 4) == 0
    assert L.moe_workspace_size(None, 4) == 0


def test_route_validation_before_any_launch():
    L = moe.lib()
    f = L.moe_route_topk
    assert f(FAKE, 1, 128, 0, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 1, 8, 9, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, -1, 8, 2, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(None, 1, 8, 2, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 1, 2048, 8, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert f(FAKE, 1, 64, 32, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert f(None, 0, 8, 2, None, None, None) == moe.MOE_OK  # empty batch, no launch


def test_plan_validation_before_any_launch():
    L = moe.lib()
    p = _lib.PlanStruct(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    f = L.moe_expert_plan
    assert f(FAKE, 1, 128, 8, None, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 1, 8, 9, C.byref(p), None) == moe.MOE_ERR_INVALID_ARG
    assert f(None, 1, 8, 2, C.byref(p), None) == moe.MOE_ERR_INVALID_ARG
    bad = _lib.PlanStruct(FAKE, None, FAKE, FAKE, FAKE, FAKE)
    assert f(FAKE, 1, 8, 2, C.byref(bad), None) == moe.MOE_ERR_INVALID_ARG
    nowork = _lib.PlanStruct(FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert f(FAKE, 1, 8, 2, C.byref(nowork), None) == moe.MOE_ERR_INVALID_ARG
    unaligned = _lib.PlanStruct(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4)
    assert f(FAKE, 1, 8, 2, C.byref(unaligned), None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 1, 4096, 2, C.byref(p), None) == moe.MOE_ERR_UNSUPPORTED
    g = L.moe_route_plan
    assert g(FAKE, 1, 8, 9, FAKE, FAKE, C.byref(p), None) == moe.MOE_ERR_INVALID_ARG
    assert g(None, 1, 8, 2, FAKE, FAKE, C.byref(p), None) == moe.MOE_ERR_INVALID_ARG
    assert g(FAKE, 1, 8, 2, FAKE, FAKE, C.byref(nowork), None) == moe.MOE_ERR_INVALID_ARG
    assert g(FAKE, 1, 2048, 2, FAKE, FAKE, C.byref(p), None) == moe.MOE_ERR_UNSUPPORTED


def test_decode_step_validation_before_any_launch():
    L = moe.lib()
    st = layer()
    p = _lib.PlanStruct(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    ws_need = L.moe_workspace_size(C.byref(st), 4)
    f = L.moe_decode_step_residual
    X, O, W = FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000

    def call(lay=st, x=X, n=4, plan=p, res=None, out=O, ws=W, wsb=ws_need):
        return f(C.byref(lay), x, n, FAKE, FAKE, C.byref(plan) if plan is not None else None,
                 res, out, ws, wsb, None)

    def plain(lay=st, x=X, n=4, plan=p, out=O, ws=W, wsb=ws_need):
        return L.moe_decode_step(C.byref(lay), x, n, FAKE, FAKE, C.byref(plan) if plan is not None else None,
                                 out, ws, wsb, None)

    # the plain call takes out where the residual variant takes the residual
    assert plain(n=0) == moe.MOE_OK
    assert plain(out=X) == moe.MOE_ERR_INVALID_ARG
    assert plain(out=None) == moe.MOE_ERR_INVALID_ARG
    assert plain(wsb=ws_need - 1) == moe.MOE_ERR_WORKSPACE
    assert plain(lay=layer(bits=2)) == moe.MOE_ERR_UNSUPPORTED

    assert call(n=0) == moe.MOE_OK  # empty batch: nothing launched
    assert call(lay=layer(bits=2)) == moe.MOE_ERR_UNSUPPORTED
    assert call(n=-1) == moe.MOE_ERR_INVALID_ARG
    assert call(n=65536) == moe.MOE_ERR_UNSUPPORTED        # beyond MOE_MAX_TOKENS
    assert call(x=None) == moe.MOE_ERR_INVALID_ARG
    assert call(out=X) == moe.MOE_ERR_INVALID_ARG          # out aliases x
    assert call(res=O) == moe.MOE_ERR_INVALID_ARG          # out aliases residual
    assert call(x=X + 2) == moe.MOE_ERR_INVALID_ARG        # x not 16-byte aligned
    assert call(ws=W + 16) == moe.MOE_ERR_INVALID_ARG      # workspace not 256-aligned
    assert call(ws=None) == moe.MOE_ERR_INVALID_ARG
    assert call(wsb=ws_need - 1) == moe.MOE_ERR_WORKSPACE
    assert call(plan=None) == moe.MOE_ERR_INVALID_ARG
    assert call(plan=_lib.PlanStruct(FAKE, FAKE, None, FAKE, FAKE, FAKE)) == moe.MOE_ERR_INVALID_ARG
    assert call(plan=_lib.PlanStruct(FAKE, FAKE, FAKE, FAKE, FAKE, None)) == moe.MOE_ERR_INVALID_ARG


def test_decode_layer_validation_before_any_launch():
    L = moe.lib()
    st = layer()
    p = _lib.PlanStruct(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    ws_need = L.moe_workspace_size(C.byref(st), 1)
    f = L.moe_decode_layer
    G, X, O, W, I, WT = (FAKE + 0x5000000, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000,
                         FAKE + 0x6000000, FAKE + 0x7000000)

    def call(lay=st, lg=G, x=X, n=1, idx=I, wt=WT, plan=p, res=None, out=O, ws=W, wsb=ws_need):
        return f(C.byref(lay), lg, x, n, idx, wt, C.byref(plan) if plan is not None else None,
                 res, out, ws, wsb, None)

    assert call(n=0) == moe.MOE_OK  # empty batch: nothing launched
    assert call(lg=None) == moe.MOE_ERR_INVALID_ARG
    assert call(idx=None) == moe.MOE_ERR_INVALID_ARG
    assert call(wt=None) == moe.MOE_ERR_INVALID_ARG
    assert call(x=None) == moe.MOE_ERR_INVALID_ARG
    assert call(out=X) == moe.MOE_ERR_INVALID_ARG
    assert call(lay=layer(bits=3)) == moe.MOE_ERR_UNSUPPORTED
    assert call(wsb=ws_need - 1) == moe.MOE_ERR_WORKSPACE
    assert call(plan=None) == moe.MOE_ERR_INVALID_ARG
    assert call(plan=_lib.PlanStruct(None, FAKE, FAKE, FAKE, FAKE, FAKE)) == moe.MOE_ERR_INVALID_ARG
    assert call(plan=_lib.PlanStruct(FAKE, FAKE, FAKE, FAKE, None, FAKE)) == moe.MOE_ERR_INVALID_ARG
    g = L.moe_route_gate_up
    assert g(C.byref(st), G, X, 0, I, WT, C.byref(p), W, ws_need, None) == moe.MOE_OK
    assert g(C.byref(st), None, X, 1, I, WT, C.byref(p), W, ws_need, None) == moe.MOE_ERR_INVALID_ARG
    assert g(C.byref(st), G, None, 1, I, WT, C.byref(p), W, ws_need, None) == moe.MOE_ERR_INVALID_ARG
    assert g(C.byref(st), G, X, 1, I, WT, C.byref(p), W, ws_need - 1, None) == moe.MOE_ERR_WORKSPACE
    assert g(C.byref(layer(group_size=48)), G, X, 1, I, WT, C.byref(p), W, ws_need, None) == \
        moe.MOE_ERR_UNSUPPORTED


def test_pack_down_validation_before_any_launch():
    L = moe.lib()
    f = L.moe_pack_down
    D = FAKE + 0x40000000
    assert f(C.byref(layer(down_layout=moe.MOE_DOWN_COLS)), D, D + 0x10000000, D + 0x20000000, None) == \
        moe.MOE_ERR_INVALID_ARG                                                  # already packed
    assert f(C.byref(layer(dff=1152)), D, D + 0x10000000, D + 0x20000000, None) == moe.MOE_ERR_UNSUPPORTED
    assert f(C.byref(layer()), None, D + 0x10000000, D + 0x20000000, None) == moe.MOE_ERR_INVALID_ARG
    assert f(C.byref(layer()), D + 4, D + 0x10000000, D + 0x20000000, None) == moe.MOE_ERR_INVALID_ARG
    src = layer()
    # destination overlapping the source down weights
    assert f(C.byref(src), src.down_q, D + 0x10000000, D + 0x20000000, None) == moe.MOE_ERR_INVALID_ARG
    # overlapping destinations
    assert f(C.byref(src), D, D + 16, D + 0x20000000, None) == moe.MOE_ERR_INVALID_ARG


def test_router_logits_validation_before_any_launch():
    f = moe.lib().moe_router_logits
    X, W, O = FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000
    BF, F32 = moe.MOE_DTYPE_BF16, moe.MOE_DTYPE_F32
    assert f(X, 0, 2048, BF, W, 128, O, None) == moe.MOE_OK       # empty batch
    assert f(X, -1, 2048, BF, W, 128, O, None) == moe.MOE_ERR_INVALID_ARG
    assert f(X, 1, 2048, 5, W, 128, O, None) == moe.MOE_ERR_INVALID_ARG
    assert f(None, 1, 2048, BF, W, 128, O, None) == moe.MOE_ERR_INVALID_ARG
    assert f(X, 1, 2048, BF, None, 128, O, None) == moe.MOE_ERR_INVALID_ARG
    assert f(X, 1, 2048, BF, W, 128, None, None) == moe.MOE_ERR_INVALID_ARG
    assert f(X + 8, 1, 2048, BF, W, 128, O, None) == moe.MOE_ERR_INVALID_ARG
    assert f(X, 1, 2048, F32, W + 4, 128, O, None) == moe.MOE_ERR_INVALID_ARG
    assert f(X, 1, 2044, BF, W, 128, O, None) == moe.MOE_ERR_UNSUPPORTED  # hidden % 8
    assert f(X, 1, 8 * 9 * 64, BF, W, 128, O, None) == moe.MOE_ERR_UNSUPPORTED  # 576 chunks: no geometry
    assert f(X, 1, 2048, BF, W, 2048, O, None) == moe.MOE_ERR_UNSUPPORTED  # > MOE_MAX_EXPERTS


def test_binding_raises_on_error_status():
    with pytest.raises(moe.MoeError) as ei:
        _lib._check(moe.MOE_ERR_UNSUPPORTED, "probe")
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED


def test_binding_requires_the_built_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


def test_static_entry_point_refuses_what_its_scratch_cannot_hold():
    """moe_decode_layer_static checks the layer and the size on the host,
    before it looks up its device array: no device is touched here."""
    L = moe.lib()
    st = layer()
    p = moe.PlanStruct(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    f = L.moe_decode_layer_static
    X, LG, I, WT, O = FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000, FAKE + 0x4000000, FAKE + 0x5000000
    per_token = 8 * 768 * 4 + 8 * 2048 * 4  # h and y of the 2048 x 768 top-8 layer
    fits = moe.MOE_STATIC_SCRATCH_BYTES // per_token
    assert fits == 93
    assert f(C.byref(st), LG, X, fits + 1, I, WT, C.byref(p), None, O, None) == moe.MOE_ERR_WORKSPACE
    assert f(C.byref(st), LG, X, 0, I, WT, C.byref(p), None, O, None) == moe.MOE_OK  # no launch
    assert f(C.byref(st), LG, X, -1, I, WT, C.byref(p), None, O, None) == moe.MOE_ERR_INVALID_ARG
    assert f(C.byref(layer(top_k=0)), LG, X, 1, I, WT, C.byref(p), None, O, None) == moe.MOE_ERR_INVALID_ARG



def test_routing_wrappers_check_buffers_before_the_library():
    """The routing wrappers refuse host tensors, mis-shaped index/weight
    buffers and plans too small for the batch before anything reaches the
    library (a wrong size would otherwise become an out-of-bounds write)."""
    import torch

    with pytest.raises(ValueError, match="device"):
        moe.route_topk(torch.zeros((2, 128)), 8)
    with pytest.raises(ValueError, match="device"):
        moe.route_plan(torch.zeros((2, 128)), 8)
    with pytest.raises(ValueError, match="device"):
        moe.expert_plan(torch.zeros((2, 8), dtype=torch.int32), 128)
    # a plan allocated for fewer slots than the batch holds
    small = moe.Plan(*[torch.zeros(n, dtype=torch.int32) for n in (128, 129, 4, 128, 1)],
                     torch.zeros((128, 4), dtype=torch.int32), None)
    with pytest.raises(ValueError, match="too small"):
        _lib._check_plan_buffers(small, 128, 16)
