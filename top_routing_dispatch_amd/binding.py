"""ctypes binding of the C ABI in include/moe.h.

Argument marshalling only: every function here turns torch tensors into device
pointers, passes the current HIP stream and raises on a non-OK status.  All
computation happens in the HIP kernels of libmoe_hip.so.  There is no fallback:
if the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_hip.so")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_SOFTMAX_TOPK, MOE_TOPK_SOFTMAX, MOE_SIGMOID_BIAS = 0, 1, 2
MOE_SWIGLU, MOE_GELU = 0, 1
(MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_EXPERT_FFN, MOE_OP_SHARED_FFN,
 MOE_OP_LOAD_STATS, MOE_OP_LAYER, MOE_OP_EXPERT_CHOICE, MOE_OP_LAYER_BACKWARD) = range(8)

EXPORTED = ("moe_capacity", "moe_workspace_size", "moe_route", "moe_permute", "moe_expert_ffn",
            "moe_combine", "moe_load_stats", "moe_layer_forward", "moe_layer_forward_timed",
            "moe_layer_backward", "moe_expert_choice_capacity", "moe_expert_choice_forward", "moe_ep_send_layout",
            "moe_ep_recv_layout",
            "moe_status_string", "moe_last_error")
STAGES = ("router_logits", "route_select", "permute", "expert_gate_up", "expert_down", "shared_gate_up",
          "shared_down", "combine", "load_stats")


class moe_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_tokens", "d_model", "num_experts", "top_k", "d_ff", "num_shared", "d_ff_shared",
        "scoring", "renormalize", "activation", "act_dtype", "router_dtype")] + [
        ("capacity_factor", ctypes.c_float)]


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_router", "sel_bias", "w13", "w2", "ws13", "ws2")]


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        super().__init__(f"{fn} failed: {_status_name(status)}{(' (' + detail + ')') if detail else ''}")


_lib = None


def _status_name(st: int) -> str:
    try:
        return lib().moe_status_string(st).decode()
    except Exception:  # pragma: no cover - only used while formatting an error
        return str(st)


def lib() -> ctypes.CDLL:
    """Load libmoe_hip.so (built in-tree by build.py); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with top_routing_dispatch_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        cfgp = ctypes.POINTER(moe_config)
        sig = {
            "moe_capacity": [cfgp, ctypes.POINTER(i32), ctypes.POINTER(i32)],
            "moe_workspace_size": [cfgp, i32, ctypes.POINTER(sz)],
            "moe_route": [cfgp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "moe_permute": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "moe_expert_ffn": [cfgp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "moe_combine": [cfgp, vp, vp, vp, vp, vp, vp],
            "moe_load_stats": [cfgp, vp, vp, f32, vp, vp, vp, vp, vp, vp, sz, vp],
            "moe_layer_forward": [cfgp, ctypes.POINTER(moe_weights), vp, vp, vp, vp, vp, f32, vp, vp, vp, sz, vp],
            "moe_layer_forward_timed": [cfgp, ctypes.POINTER(moe_weights), vp, vp, vp, vp, vp, f32, vp, vp, vp, sz,
                                        vp, ctypes.POINTER(vp)],
            "moe_layer_backward": [cfgp, ctypes.POINTER(moe_weights), vp, vp, f32, vp, vp, vp, vp, vp, vp, vp, sz,
                                   vp],
            "moe_expert_choice_capacity": [cfgp, ctypes.POINTER(i32)],
            "moe_expert_choice_forward": [cfgp, ctypes.POINTER(moe_weights), vp, vp, vp, vp, vp, vp, sz, vp,
                                          ctypes.POINTER(vp)],
            "moe_ep_send_layout": [i32, i32, vp, vp, vp, vp],
            "moe_ep_recv_layout": [i32, i32, vp, i32, vp, vp, vp],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def make_config(cfg) -> moe_config:
    """moe_config from any object carrying the same field names."""
    c = moe_config()
    for name, _ in moe_config._fields_:
        setattr(c, name, getattr(cfg, name))
    return c


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, st: int):
    if st != MOE_OK:
        detail = lib().moe_last_error().decode() if st == MOE_ERR_HIP else ""
        raise MoEError(fn, st, detail)


def moe_capacity(cfg):
    c = make_config(cfg)
    cap, rows = ctypes.c_int32(), ctypes.c_int32()
    _check("moe_capacity", lib().moe_capacity(ctypes.byref(c), ctypes.byref(cap), ctypes.byref(rows)))
    return cap.value, rows.value


def moe_workspace_size(cfg, op: int) -> int:
    c = make_config(cfg)
    n = ctypes.c_size_t()
    _check("moe_workspace_size", lib().moe_workspace_size(ctypes.byref(c), op, ctypes.byref(n)))
    return n.value


def workspace(cfg, op: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(moe_workspace_size(cfg, op), 256), dtype=torch.uint8, device=device)


def moe_route(cfg, x, w_router, sel_bias, topk_idx, topk_w, probs, ws, stream=None):
    c = make_config(cfg)
    _check("moe_route", lib().moe_route(ctypes.byref(c), _ptr(x), _ptr(w_router), _ptr(sel_bias), _ptr(topk_idx),
                                        _ptr(topk_w), _ptr(probs), _ptr(ws), ws.numel() if ws is not None else 0,
                                        _stream(stream)))


def moe_permute(cfg, topk_idx, x, counts, offsets, row_of, token_of_row, x_perm, ws, stream=None):
    c = make_config(cfg)
    _check("moe_permute", lib().moe_permute(ctypes.byref(c), _ptr(topk_idx), _ptr(x), _ptr(counts), _ptr(offsets),
                                            _ptr(row_of), _ptr(token_of_row), _ptr(x_perm), _ptr(ws),
                                            ws.numel() if ws is not None else 0, _stream(stream)))


def moe_expert_ffn(cfg, num_groups, d_ff, activation, max_rows, x_in, gather_rows, offsets, w13, w2, y_out, ws,
                   stream=None):
    c = make_config(cfg)
    _check("moe_expert_ffn", lib().moe_expert_ffn(ctypes.byref(c), num_groups, d_ff, activation, max_rows, _ptr(x_in),
                                                  _ptr(gather_rows), _ptr(offsets), _ptr(w13), _ptr(w2), _ptr(y_out),
                                                  _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def moe_combine(cfg, y_perm, row_of, topk_w, y_shared, y, stream=None):
    c = make_config(cfg)
    _check("moe_combine", lib().moe_combine(ctypes.byref(c), _ptr(y_perm), _ptr(row_of), _ptr(topk_w),
                                            _ptr(y_shared), _ptr(y), _stream(stream)))


def moe_load_stats(cfg, counts, probs, alpha, f, P, aux_loss, imbalance, dropped, ws, stream=None):
    c = make_config(cfg)
    _check("moe_load_stats", lib().moe_load_stats(ctypes.byref(c), _ptr(counts), _ptr(probs), float(alpha), _ptr(f),
                                                  _ptr(P), _ptr(aux_loss), _ptr(imbalance), _ptr(dropped), _ptr(ws),
                                                  ws.numel() if ws is not None else 0, _stream(stream)))


def moe_layer_forward(cfg, weights: dict, x, y, topk_idx=None, topk_w=None, counts=None, alpha=0.01, stats=None,
                      dropped=None, ws=None, stream=None):
    c = make_config(cfg)
    w = moe_weights()
    for name, _ in moe_weights._fields_:
        t = weights.get(name)
        setattr(w, name, None if t is None else t.data_ptr())
    _check("moe_layer_forward", lib().moe_layer_forward(
        ctypes.byref(c), ctypes.byref(w), _ptr(x), _ptr(y), _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
        float(alpha), _ptr(stats), _ptr(dropped), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def moe_layer_forward_timed(cfg, weights: dict, x, y, topk_idx=None, topk_w=None, counts=None, alpha=0.01,
                            stats=None, dropped=None, ws=None, stage_events=None, stream=None):
    """stage_events: list of 2 * len(STAGES) torch.cuda.Event (enable_timing=True)
    already recorded once (so that their HIP handles exist), or None entries."""
    c = make_config(cfg)
    w = moe_weights()
    for name, _ in moe_weights._fields_:
        t = weights.get(name)
        setattr(w, name, None if t is None else t.data_ptr())
    n = 2 * len(STAGES)
    arr = (ctypes.c_void_p * n)()
    if stage_events is not None:
        for i, ev in enumerate(stage_events):
            arr[i] = None if ev is None else ev.cuda_event
    _check("moe_layer_forward_timed", lib().moe_layer_forward_timed(
        ctypes.byref(c), ctypes.byref(w), _ptr(x), _ptr(y), _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
        float(alpha), _ptr(stats), _ptr(dropped), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream),
        arr))


def moe_layer_backward(cfg, weights: dict, x, dy, alpha, dx, dw_router, dw13, dw2, dws13=None, dws2=None, ws=None,
                       stream=None):
    """Gradients of <dy, y> + alpha-weighted balance loss, the routing fixed."""
    c = make_config(cfg)
    w = moe_weights()
    for name, _ in moe_weights._fields_:
        t = weights.get(name)
        setattr(w, name, None if t is None else t.data_ptr())
    _check("moe_layer_backward", lib().moe_layer_backward(
        ctypes.byref(c), ctypes.byref(w), _ptr(x), _ptr(dy), float(alpha), _ptr(dx), _ptr(dw_router), _ptr(dw13),
        _ptr(dw2), _ptr(dws13), _ptr(dws2), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def moe_expert_choice_capacity(cfg) -> int:
    c = make_config(cfg)
    cap = ctypes.c_int32()
    _check("moe_expert_choice_capacity", lib().moe_expert_choice_capacity(ctypes.byref(c), ctypes.byref(cap)))
    return cap.value


def moe_expert_choice_forward(cfg, weights: dict, x, y, token_of_row=None, row_w=None, unselected=None, ws=None,
                              stage_events=None, stream=None):
    """Expert-choice layer forward; stage_events as for moe_layer_forward_timed."""
    c = make_config(cfg)
    w = moe_weights()
    for name, _ in moe_weights._fields_:
        t = weights.get(name)
        setattr(w, name, None if t is None else t.data_ptr())
    arr = None
    if stage_events is not None:
        arr = (ctypes.c_void_p * (2 * len(STAGES)))()
        for i, ev in enumerate(stage_events):
            arr[i] = None if ev is None else ev.cuda_event
    _check("moe_expert_choice_forward", lib().moe_expert_choice_forward(
        ctypes.byref(c), ctypes.byref(w), _ptr(x), _ptr(y), _ptr(token_of_row), _ptr(row_w), _ptr(unselected),
        _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream), arr))


def moe_ep_send_layout(num_experts, num_ranks, offsets, send_counts, send_offsets, stream=None):
    _check("moe_ep_send_layout", lib().moe_ep_send_layout(num_experts, num_ranks, _ptr(offsets), _ptr(send_counts),
                                                          _ptr(send_offsets), _stream(stream)))


def moe_ep_recv_layout(recv_counts, rows_cap, local_offsets, gather, stream=None):
    """recv_counts: [R, E_local] int32 device tensor."""
    R, El = recv_counts.shape
    _check("moe_ep_recv_layout", lib().moe_ep_recv_layout(R, El, _ptr(recv_counts), rows_cap, _ptr(local_offsets),
                                                          _ptr(gather), _stream(stream)))
