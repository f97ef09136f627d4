"""Host-side tests of the C ABI (no GPU): the library loads, exports every
symbol include/moe.h declares, sizes workspaces, and rejects bad arguments
before enqueuing anything (so no HIP call is reached)."""
import ctypes
import os
import re

import pytest

import top_routing_dispatch_amd as M
import workloads as W
from top_routing_dispatch_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char\*)\s+(moe_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 10
    L = M.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(B.EXPORTED)


def test_status_strings():
    L = M.lib()
    for st in range(5):
        assert L.moe_status_string(st).decode().startswith("MOE_")


def test_capacity_matches_formula():
    assert M.moe_capacity(W.SWITCH) == (80, 8192)                  # 1.25 * 8192 * 1 / 128
    cap, rows = M.moe_capacity(W.DEEPSEEKV3)
    assert cap == 2**31 - 1 and rows == 8192 * 8                    # dropless
    c = W.MoEConfig("c", 10, 8, 4, 1, 8, capacity_factor=1.5)       # 3.75 -> 4
    assert M.moe_capacity(c) == (4, 10)
    c = W.MoEConfig("c", 10, 8, 4, 2, 8, capacity_factor=0.01)      # ceil(0.05) = 1
    assert M.moe_capacity(c) == (1, 4)


def test_capacity_agrees_with_oracle():
    from oracle import moe_oracle as O
    for cf in (0.3, 0.75, 1.0, 1.1, 1.25, 1.7, 2.0):
        for T, k, E in ((8192, 1, 128), (777, 8, 64), (10, 3, 7)):
            c = W.MoEConfig("c", T, 8, E, k, 8, capacity_factor=cf)
            assert M.moe_capacity(c)[0] == O.capacity(cf, T, k, E), (cf, T, k, E)


def test_workspace_sizes_cover_buffers():
    c = W.DEEPSEEKV3
    layer = M.moe_workspace_size(c, M.MOE_OP_LAYER)
    A = 8192 * 8
    assert layer >= A * 7168 * 2 + A * 2048 * 2        # y_perm + hidden
    assert M.moe_workspace_size(c, M.MOE_OP_ROUTE) >= 8192 * 256 * 4
    for op in range(6):
        assert M.moe_workspace_size(c, op) % 256 == 0


@pytest.mark.parametrize("field,value,status", [
    ("top_k", 0, M.MOE_ERR_INVALID_ARGUMENT),
    ("top_k", 5, M.MOE_ERR_INVALID_ARGUMENT),          # k > E
    ("num_experts", 2000, M.MOE_ERR_UNSUPPORTED),
    ("d_model", 30, M.MOE_ERR_UNSUPPORTED),            # bf16 rows must be 16-byte multiples
    ("scoring", 7, M.MOE_ERR_INVALID_ARGUMENT),
    ("num_tokens", -1, M.MOE_ERR_INVALID_ARGUMENT),
    ("router_dtype", W.BF16, None),
])
def test_config_validation(field, value, status):
    cfg = W.MoEConfig("v", 16, 64, 4, 2, 32).replace(**{field: value})
    if field == "router_dtype":
        cfg = cfg.replace(act_dtype=W.F32)            # f32 activations with bf16 router: unsupported
        status = M.MOE_ERR_UNSUPPORTED
    with pytest.raises(M.MoEError) as ei:
        M.moe_workspace_size(cfg, M.MOE_OP_LAYER)
    assert ei.value.status == status


def _raw(fn, *args):
    return getattr(M.lib(), fn)(*args)


def test_null_and_misaligned_pointers_rejected_before_launch():
    cfg = W.MoEConfig("v", 16, 64, 4, 2, 32)
    c = B.make_config(cfg)
    p = ctypes.c_void_p(0x100000)           # aligned, never dereferenced: validation fails first
    mis = ctypes.c_void_p(0x100004)
    ws_n = M.moe_workspace_size(cfg, M.MOE_OP_ROUTE)
    # missing outputs
    assert _raw("moe_route", ctypes.byref(c), p, p, None, None, p, None, p, ws_n, None) == M.MOE_ERR_INVALID_ARGUMENT
    # misaligned input
    assert _raw("moe_route", ctypes.byref(c), mis, p, None, p, p, None, p, ws_n, None) == M.MOE_ERR_INVALID_ARGUMENT
    # workspace too small
    assert _raw("moe_route", ctypes.byref(c), p, p, None, p, p, None, p, ws_n - 256, None) == \
        M.MOE_ERR_WORKSPACE_TOO_SMALL
    # permute: x without x_perm
    assert _raw("moe_permute", ctypes.byref(c), p, p, p, p, p, p, None, p, 1 << 20, None) == \
        M.MOE_ERR_INVALID_ARGUMENT
    # expert ffn: bad activation / group count
    assert _raw("moe_expert_ffn", ctypes.byref(c), 4, 32, 9, 8, p, None, p, p, p, p, p, 1 << 20, None) == \
        M.MOE_ERR_INVALID_ARGUMENT
    assert _raw("moe_expert_ffn", ctypes.byref(c), 0, 32, 0, 8, p, None, p, p, p, p, p, 1 << 20, None) == \
        M.MOE_ERR_INVALID_ARGUMENT
    # layer: missing weights struct
    assert _raw("moe_layer_forward", ctypes.byref(c), None, p, p, None, None, None, ctypes.c_float(0.01), None,
                None, p, 1 << 30, None) == M.MOE_ERR_INVALID_ARGUMENT
    # layer: shared experts declared but weights missing
    cs = B.make_config(cfg.replace(num_shared=1, d_ff_shared=16))
    w = B.moe_weights(p.value, None, p.value, p.value, None, None)
    assert _raw("moe_layer_forward", ctypes.byref(cs), ctypes.byref(w), p, p, None, None, None, ctypes.c_float(0.01),
                None, None, p, 1 << 30, None) == M.MOE_ERR_INVALID_ARGUMENT
    # null config
    assert _raw("moe_combine", None, p, p, p, None, p, None) == M.MOE_ERR_INVALID_ARGUMENT


def test_ep_layout_arguments_rejected_before_launch():
    p = ctypes.c_void_p(0x100000)           # never dereferenced: validation fails first
    bad = M.MOE_ERR_INVALID_ARGUMENT
    # experts not divisible by ranks, zero ranks, more ranks than experts, null outputs
    assert _raw("moe_ep_send_layout", 10, 4, p, p, p, None) == bad
    assert _raw("moe_ep_send_layout", 8, 0, p, p, p, None) == bad
    assert _raw("moe_ep_send_layout", 4, 8, p, p, p, None) == bad
    assert _raw("moe_ep_send_layout", 8, 2, p, None, p, None) == bad
    assert _raw("moe_ep_send_layout", 2048, 2, p, p, p, None) == M.MOE_ERR_UNSUPPORTED
    # receive layout: zero ranks / experts, negative capacity, missing gather
    assert _raw("moe_ep_recv_layout", 0, 4, p, 16, p, p, None) == bad
    assert _raw("moe_ep_recv_layout", 2, 0, p, 16, p, p, None) == bad
    assert _raw("moe_ep_recv_layout", 2, 4, p, -1, p, p, None) == bad
    assert _raw("moe_ep_recv_layout", 2, 4, p, 16, p, None, None) == bad
    assert _raw("moe_ep_recv_layout", 2, 4, None, 16, p, p, None) == bad


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


def _tiny_layer_args(cfg, dev="cpu"):
    import torch
    T, D, E, k, F = cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.top_k, cfg.d_ff
    act = torch.bfloat16
    w = dict(w_router=torch.zeros(E, D, dtype=act), sel_bias=None, w13=torch.zeros(E, 2 * F, D, dtype=act),
             w2=torch.zeros(E, D, F, dtype=act), ws13=None, ws2=None)
    x = torch.zeros(T, D, dtype=act)
    y = torch.zeros(T, D, dtype=act)
    ws = torch.zeros(M.moe_workspace_size(cfg, M.MOE_OP_LAYER), dtype=torch.uint8)
    return w, x, y, ws


def test_binding_rejects_host_tensors_before_the_call():
    cfg = W.MoEConfig("v", 16, 64, 4, 2, 32)
    w, x, y, ws = _tiny_layer_args(cfg)
    with pytest.raises(ValueError, match="must be on the GPU"):
        M.moe_layer_forward(cfg, w, x, y, ws=ws)


@pytest.mark.parametrize("bad", ["dtype", "short", "transposed", "missing_weight", "short_ws", "idx_dtype"])
def test_binding_checks_types_and_sizes(monkeypatch, bad):
    """With the device check stubbed out (no GPU here), every other host check
    must still reject a bad argument before the library is called."""
    import torch
    monkeypatch.setattr(B, "_on_device", lambda t: True)
    called = []
    monkeypatch.setattr(B, "_check", lambda fn, st: called.append(fn))
    cfg = W.MoEConfig("v", 16, 64, 4, 2, 32)
    w, x, y, ws = _tiny_layer_args(cfg)
    idx = torch.zeros(16, 2, dtype=torch.int32)
    if bad == "dtype":
        x = x.float()
    elif bad == "short":
        y = y[:-1]
    elif bad == "transposed":
        x = torch.zeros(64, 16, dtype=torch.bfloat16).t()
    elif bad == "missing_weight":
        w["w2"] = None
    elif bad == "short_ws":
        ws = ws[:-256]
    elif bad == "idx_dtype":
        idx = idx.long()
    with pytest.raises(ValueError):
        M.moe_layer_forward(cfg, w, x, y, topk_idx=idx, ws=ws)
    assert set(called) <= {"moe_workspace_size", "moe_capacity"}      # host-side size queries only


def test_oversized_operands_rejected_before_launch():
    """A DeepSeek-V3-shaped layer at T = 131,072: the permuted rows
    [T k, D] bf16 alone are 15 GB, past the 32-bit byte offsets the kernels
    address operands with, so every call rejects the configuration up front
    (the largest T that fits at this shape is 37,430)."""
    big = W.DEEPSEEKV3.replace(num_tokens=131072)
    for op in (M.MOE_OP_ROUTE, M.MOE_OP_LAYER, M.MOE_OP_EXPERT_FFN, M.MOE_OP_LAYER_BACKWARD):
        with pytest.raises(M.MoEError) as ei:
            M.moe_workspace_size(big, op)
        assert ei.value.status == M.MOE_ERR_UNSUPPORTED
    c = B.make_config(big)
    p = ctypes.c_void_p(0x100000)           # never dereferenced: validation fails first
    w = B.moe_weights(p.value, p.value, p.value, p.value, p.value, p.value)
    assert _raw("moe_layer_forward", ctypes.byref(c), ctypes.byref(w), p, p, None, None, None, ctypes.c_float(0.01),
                None, None, p, 1 << 62, None) == M.MOE_ERR_UNSUPPORTED
    assert M.moe_capacity(W.DEEPSEEKV3.replace(num_tokens=37430))[1] == 37430 * 8
    with pytest.raises(M.MoEError):
        M.moe_capacity(W.DEEPSEEKV3.replace(num_tokens=37431))
    # x alone past the limit: a wide token matrix with top-1
    wide = W.MoEConfig("wide", 300000, 7168, 8, 1, 64)
    with pytest.raises(M.MoEError):
        M.moe_workspace_size(wide, M.MOE_OP_ROUTE)


def test_layer_stages_pick_the_one_workgroup_kernel_for_small_batches(monkeypatch):
    """moe_layer_stages is host-side: the fused kernel for batches with little
    work, the staged kernels otherwise, MOE_FUSED overriding the choice where
    the batch fits one workgroup."""
    staged = ["router_logits", "route_select", "permute", "expert_gate_up", "expert_down", "combine",
              "load_stats"]
    assert M.moe_layer_stages(W.TINY) == ["fused_layer"]
    assert M.moe_layer_stages(W.MIXTRAL) == staged
    assert M.moe_layer_stages(W.DEEPSEEKV3) == staged[:5] + ["shared_gate_up", "shared_down"] + staged[5:]
    assert M.moe_layer_stages(W.TINY.replace(num_tokens=0)) == ["permute", "load_stats"]
    wide = W.MoEConfig("wide", 16, 512, 8, 2, 512)
    assert "fused_layer" not in M.moe_layer_stages(wide)            # fits, but too much work for one CU
    too_big = [W.TINY.replace(num_tokens=257), W.TINY.replace(num_experts=65, top_k=2),
               W.MoEConfig("k9", 16, 32, 16, 9, 16), W.TINY.replace(d_ff=8192),
               W.TINY.replace(num_tokens=256, num_experts=64)]   # the last two past the LDS
    try:
        monkeypatch.setenv("MOE_FUSED", "1")
        M.moe_reload_tuning()
        assert M.moe_layer_stages(wide) == ["fused_layer"]
        for c in too_big:
            assert "fused_layer" not in M.moe_layer_stages(c), c
        monkeypatch.setenv("MOE_FUSED", "0")
        M.moe_reload_tuning()
        assert M.moe_layer_stages(W.TINY) == staged
    finally:
        monkeypatch.delenv("MOE_FUSED")
        M.moe_reload_tuning()
    with pytest.raises(M.MoEError):
        M.moe_layer_stages(W.TINY.replace(top_k=5))
