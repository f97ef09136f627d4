"""ctypes binding of the C ABI in include/moe.h.

Argument marshalling only: every function here turns torch tensors into device
pointers, passes the current HIP stream and raises on a non-OK status.  All
computation happens in the HIP kernels of libmoe_hip.so.  There is no fallback:
if the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; MOE_LIB_PATH names another build of the same sources
# (a tuning variant)
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(_PKG, "libmoe_hip.so")

(MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP,
 MOE_ERR_DEBUG_CHECK) = range(6)
MOE_F32, MOE_BF16 = 0, 1
MOE_SOFTMAX_TOPK, MOE_TOPK_SOFTMAX, MOE_SIGMOID_BIAS = 0, 1, 2
MOE_SWIGLU, MOE_GELU = 0, 1
(MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_EXPERT_FFN, MOE_OP_SHARED_FFN,
 MOE_OP_LOAD_STATS, MOE_OP_LAYER, MOE_OP_EXPERT_CHOICE, MOE_OP_LAYER_BACKWARD) = range(8)

EXPORTED = ("moe_capacity", "moe_workspace_size", "moe_route", "moe_permute", "moe_expert_ffn",
            "moe_combine", "moe_load_stats", "moe_layer_forward", "moe_layer_forward_timed", "moe_layer_forward_static",
            "moe_layer_backward", "moe_expert_choice_capacity", "moe_expert_choice_forward", "moe_ep_send_layout",
            "moe_ep_recv_layout", "moe_layer_stages", "moe_check_dispatch",
            "moe_reload_tuning", "moe_status_string", "moe_last_error")
STAGES = ("router_logits", "route_select", "permute", "expert_gate_up", "expert_down", "shared_gate_up",
          "shared_down", "combine", "load_stats", "fused_layer")


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
            "moe_layer_forward_static": [cfgp, ctypes.POINTER(moe_weights), vp, vp, vp, vp, vp, f32, vp, vp, vp],
            "moe_layer_backward": [cfgp, ctypes.POINTER(moe_weights), vp, vp, f32, vp, vp, vp, vp, vp, vp, vp, sz,
                                   vp],
            "moe_expert_choice_capacity": [cfgp, ctypes.POINTER(i32)],
            "moe_expert_choice_forward": [cfgp, ctypes.POINTER(moe_weights), vp, vp, vp, vp, vp, vp, sz, vp,
                                          ctypes.POINTER(vp)],
            "moe_ep_send_layout": [i32, i32, vp, vp, vp, vp],
            "moe_ep_recv_layout": [i32, i32, vp, i32, vp, vp, vp],
            "moe_layer_stages": [cfgp, ctypes.POINTER(i32)],
            "moe_check_dispatch": [cfgp, vp, vp, vp, vp, vp],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.moe_reload_tuning.argtypes = []
        L.moe_reload_tuning.restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def moe_reload_tuning():
    """Re-read the MOE_* tuning variables (the library reads them once); the
    workspace sizes cached here depend on them."""
    _check("moe_reload_tuning", lib().moe_reload_tuning())
    _workspace_size_cached.cache_clear()
    _layer_specs.cache_clear()


def _new_config(cfg) -> moe_config:
    c = moe_config()
    for name, _ in moe_config._fields_:
        setattr(c, name, getattr(cfg, name))
    return c


@functools.lru_cache(maxsize=512)
def _config_cached(cfg) -> moe_config:
    return _new_config(cfg)


def make_config(cfg) -> moe_config:
    """moe_config from any object carrying the same field names (one shared,
    read-only structure per hashable configuration: the library only reads
    it)."""
    try:
        return _config_cached(cfg)
    except TypeError:                    # not hashable
        return _new_config(cfg)


def _ptr(t: Optional[torch.Tensor]):
    """Device address of a tensor as a plain integer (ctypes converts it for
    the c_void_p parameters), or None."""
    return None if t is None else t.data_ptr()


_I32, _F32, _BYTES = "int32", "float32", "bytes"


def _elem(cfg, kind):
    """torch dtype an argument of `kind` must have: "act" / "router" follow the
    configuration's activation and router types."""
    if kind == "act":
        return torch.bfloat16 if cfg.act_dtype == MOE_BF16 else torch.float32
    if kind == "router":
        return torch.bfloat16 if cfg.router_dtype == MOE_BF16 else torch.float32
    return {_I32: torch.int32, _F32: torch.float32}[kind]


def _on_device(t: torch.Tensor) -> bool:
    return t.is_cuda


def _arg(fn: str, name: str, t, kind, numel: int, cfg=None, required: bool = False):
    """Host-side check of one tensor argument before its pointer crosses the C
    ABI (which cannot see sizes or types): a device tensor, dense, of the
    expected element type, holding at least `numel` elements (bytes for a
    workspace).  Raises ValueError instead of letting a kernel read or write
    past a buffer."""
    if t is None:
        if required:
            raise ValueError(f"{fn}: {name} is required")
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{fn}: {name} must be a torch.Tensor")
    if numel == 0 and t.numel() == 0:
        return                           # nothing is read or written through it
    if not _on_device(t):
        raise ValueError(f"{fn}: {name} must be on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{fn}: {name} must be contiguous")
    if kind == _BYTES:
        have = t.numel() * t.element_size()
    else:
        want = _elem(cfg, kind)
        if t.dtype != want:
            raise ValueError(f"{fn}: {name} must be {want} (got {t.dtype})")
        have = t.numel()
    if have < numel:
        raise ValueError(f"{fn}: {name} holds {have} {'bytes' if kind == _BYTES else 'elements'}, needs {numel}")


def _ws_bytes(ws) -> int:
    return 0 if ws is None else ws.numel() * ws.element_size()


def _rows_cap(cfg) -> int:
    return moe_capacity(cfg)[1]


def _check_weights(fn, cfg, weights: dict, need_experts: bool = True):
    T, D, E, F = cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.d_ff
    nF = (2 if cfg.activation == MOE_SWIGLU else 1) * F
    SF = cfg.num_shared * cfg.d_ff_shared
    _arg(fn, "w_router", weights.get("w_router"), "router", E * D, cfg, required=True)
    _arg(fn, "sel_bias", weights.get("sel_bias"), _F32, E, cfg)
    _arg(fn, "w13", weights.get("w13"), "act", E * nF * D, cfg, required=need_experts)
    _arg(fn, "w2", weights.get("w2"), "act", E * D * F, cfg, required=need_experts)
    _arg(fn, "ws13", weights.get("ws13"), "act", 2 * SF * D, cfg, required=SF > 0)
    _arg(fn, "ws2", weights.get("ws2"), "act", D * SF, cfg, required=SF > 0)


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, st: int):
    if st != MOE_OK:
        detail = (lib().moe_last_error().decode()
                  if st in (MOE_ERR_HIP, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_DEBUG_CHECK) else "")
        raise MoEError(fn, st, detail)


def moe_capacity(cfg):
    c = make_config(cfg)
    cap, rows = ctypes.c_int32(), ctypes.c_int32()
    _check("moe_capacity", lib().moe_capacity(ctypes.byref(c), ctypes.byref(cap), ctypes.byref(rows)))
    return cap.value, rows.value


def moe_layer_stages(cfg):
    """Names of the stages moe_layer_forward runs for `cfg` (every output asked
    for): the staged kernels, or "fused_layer" alone for small batches."""
    c = make_config(cfg)
    runs = (ctypes.c_int32 * len(STAGES))()
    _check("moe_layer_stages", lib().moe_layer_stages(ctypes.byref(c), runs))
    return [name for name, r in zip(STAGES, runs) if r]


def moe_check_dispatch(cfg, topk_idx, counts, offsets, row_of, token_of_row):
    """The host-side dispatch check on numpy int32 arrays (shapes as in
    moe_permute); raises MoEError(MOE_ERR_DEBUG_CHECK) naming the first bad
    entry."""
    import numpy as np
    arrs = [np.ascontiguousarray(a, dtype=np.int32) for a in (topk_idx, counts, offsets, row_of, token_of_row)]
    ptrs = [a.ctypes.data_as(ctypes.c_void_p) if a.size else None for a in arrs]
    c = make_config(cfg)
    _check("moe_check_dispatch", lib().moe_check_dispatch(ctypes.byref(c), *ptrs))


def _workspace_size(cfg, op: int) -> int:
    c = make_config(cfg)
    n = ctypes.c_size_t()
    _check("moe_workspace_size", lib().moe_workspace_size(ctypes.byref(c), op, ctypes.byref(n)))
    return n.value


@functools.lru_cache(maxsize=1024)
def _workspace_size_cached(cfg, op: int) -> int:
    return _workspace_size(cfg, op)


def moe_workspace_size(cfg, op: int) -> int:
    try:
        return _workspace_size_cached(cfg, op)
    except TypeError:                    # not hashable
        return _workspace_size(cfg, op)


def workspace(cfg, op: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(moe_workspace_size(cfg, op), 256), dtype=torch.uint8, device=device)


def moe_route(cfg, x, w_router, sel_bias, topk_idx, topk_w, probs, ws, stream=None):
    T, D, E, k = cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.top_k
    fn = "moe_route"
    _arg(fn, "x", x, "act", T * D, cfg, required=T > 0)
    _arg(fn, "w_router", w_router, "router", E * D, cfg, required=True)
    _arg(fn, "sel_bias", sel_bias, _F32, E, cfg)
    _arg(fn, "topk_idx", topk_idx, _I32, T * k, cfg, required=T > 0)
    _arg(fn, "topk_w", topk_w, _F32, T * k, cfg, required=T > 0)
    _arg(fn, "probs", probs, _F32, T * E, cfg)
    _arg(fn, "ws", ws, _BYTES, moe_workspace_size(cfg, MOE_OP_ROUTE), cfg, required=T > 0)
    c = make_config(cfg)
    _check("moe_route", lib().moe_route(ctypes.byref(c), _ptr(x), _ptr(w_router), _ptr(sel_bias), _ptr(topk_idx),
                                        _ptr(topk_w), _ptr(probs), _ptr(ws), _ws_bytes(ws),
                                        _stream(stream)))


def moe_permute(cfg, topk_idx, x, counts, offsets, row_of, token_of_row, x_perm, ws, stream=None):
    T, D, E, k = cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.top_k
    A = _rows_cap(cfg)
    fn = "moe_permute"
    _arg(fn, "topk_idx", topk_idx, _I32, T * k, cfg, required=T > 0)
    _arg(fn, "x", x, "act", T * D, cfg)
    _arg(fn, "counts", counts, _I32, E, cfg, required=True)
    _arg(fn, "offsets", offsets, _I32, E + 1, cfg, required=True)
    _arg(fn, "row_of", row_of, _I32, T * k, cfg, required=T > 0)
    _arg(fn, "token_of_row", token_of_row, _I32, A, cfg, required=A > 0)
    _arg(fn, "x_perm", x_perm, "act", A * D, cfg)
    _arg(fn, "ws", ws, _BYTES, moe_workspace_size(cfg, MOE_OP_PERMUTE), cfg, required=T > 0)
    c = make_config(cfg)
    _check("moe_permute", lib().moe_permute(ctypes.byref(c), _ptr(topk_idx), _ptr(x), _ptr(counts), _ptr(offsets),
                                            _ptr(row_of), _ptr(token_of_row), _ptr(x_perm), _ptr(ws),
                                            _ws_bytes(ws), _stream(stream)))


def moe_expert_ffn(cfg, num_groups, d_ff, activation, max_rows, x_in, gather_rows, offsets, w13, w2, y_out, ws,
                   stream=None):
    D = cfg.d_model
    nF = (2 if activation == MOE_SWIGLU else 1) * d_ff
    fn = "moe_expert_ffn"
    need = max_rows > 0
    # with a gather map the rows of x_in it names are the caller's to bound
    _arg(fn, "x_in", x_in, "act", D if gather_rows is not None else max_rows * D, cfg, required=need)
    if x_in is not None and x_in.numel() % D:
        raise ValueError(f"{fn}: x_in must hold whole rows of {D}")
    _arg(fn, "gather_rows", gather_rows, _I32, max_rows, cfg)
    _arg(fn, "offsets", offsets, _I32, num_groups + 1, cfg)
    _arg(fn, "w13", w13, "act", num_groups * nF * D, cfg, required=need)
    _arg(fn, "w2", w2, "act", num_groups * D * d_ff, cfg, required=need)
    _arg(fn, "y_out", y_out, "act", max_rows * D, cfg, required=need)
    c = make_config(cfg)
    _check("moe_expert_ffn", lib().moe_expert_ffn(ctypes.byref(c), num_groups, d_ff, activation, max_rows, _ptr(x_in),
                                                  _ptr(gather_rows), _ptr(offsets), _ptr(w13), _ptr(w2), _ptr(y_out),
                                                  _ptr(ws), _ws_bytes(ws), _stream(stream)))


def moe_combine(cfg, y_perm, row_of, topk_w, y_shared, y, stream=None):
    T, D, k = cfg.num_tokens, cfg.d_model, cfg.top_k
    fn = "moe_combine"
    # row_of (device data) names the rows of y_perm that are read: they are
    # the caller's to provide; here only whole rows are required
    _arg(fn, "y_perm", y_perm, "act", D if T > 0 and _rows_cap(cfg) > 0 else 0, cfg)
    if y_perm is not None and y_perm.numel() % D:
        raise ValueError(f"{fn}: y_perm must hold whole rows of {D}")
    _arg(fn, "row_of", row_of, _I32, T * k, cfg, required=T > 0)
    _arg(fn, "topk_w", topk_w, _F32, T * k, cfg, required=T > 0)
    _arg(fn, "y_shared", y_shared, "act", T * D, cfg)
    _arg(fn, "y", y, "act", T * D, cfg, required=T > 0)
    c = make_config(cfg)
    _check("moe_combine", lib().moe_combine(ctypes.byref(c), _ptr(y_perm), _ptr(row_of), _ptr(topk_w),
                                            _ptr(y_shared), _ptr(y), _stream(stream)))


def moe_load_stats(cfg, counts, probs, alpha, f, P, aux_loss, imbalance, dropped, ws, stream=None):
    T, E = cfg.num_tokens, cfg.num_experts
    fn = "moe_load_stats"
    _arg(fn, "counts", counts, _I32, E, cfg, required=True)
    _arg(fn, "probs", probs, _F32, T * E, cfg, required=T > 0)
    for name, t, n in (("f", f, E), ("P", P, E), ("aux_loss", aux_loss, 1), ("imbalance", imbalance, 1)):
        _arg(fn, name, t, _F32, n, cfg)
    _arg(fn, "dropped", dropped, _I32, 1, cfg)
    _arg(fn, "ws", ws, _BYTES, moe_workspace_size(cfg, MOE_OP_LOAD_STATS), cfg, required=T > 0)
    c = make_config(cfg)
    _check("moe_load_stats", lib().moe_load_stats(ctypes.byref(c), _ptr(counts), _ptr(probs), float(alpha), _ptr(f),
                                                  _ptr(P), _ptr(aux_loss), _ptr(imbalance), _ptr(dropped), _ptr(ws),
                                                  _ws_bytes(ws), _stream(stream)))


def _layer_specs_of(cfg, with_ws: bool):
    """(name, kind, numel, required) of every tensor argument of the layer
    forward, weights first."""
    T, D, E, k, F = cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.top_k, cfg.d_ff
    nF = (2 if cfg.activation == MOE_SWIGLU else 1) * F
    SF = cfg.num_shared * cfg.d_ff_shared
    specs = [("w_router", "router", E * D, True), ("sel_bias", _F32, E, False),
             ("w13", "act", E * nF * D, True), ("w2", "act", E * D * F, True),
             ("ws13", "act", 2 * SF * D, SF > 0), ("ws2", "act", D * SF, SF > 0),
             ("x", "act", T * D, T > 0), ("y", "act", T * D, T > 0),
             ("topk_idx", _I32, T * k, False), ("topk_w", _F32, T * k, False), ("counts", _I32, E, False),
             ("stats", _F32, 2 * E + 2, False), ("dropped", _I32, 1, False)]
    if with_ws:
        specs.append(("ws", _BYTES, moe_workspace_size(cfg, MOE_OP_LAYER), T > 0))
    return tuple((name, None if kind == _BYTES else _elem(cfg, kind), kind, n, req) for name, kind, n, req in specs)


@functools.lru_cache(maxsize=512)
def _layer_specs(cfg, with_ws: bool):
    return _layer_specs_of(cfg, with_ws)


def _check_layer_args(fn, cfg, weights, x, y, topk_idx, topk_w, counts, stats, dropped, ws):
    """The per-tensor checks of _arg on every argument of the layer forward,
    in one pass; the first argument that fails is re-checked by _arg for its
    message.  The specs (element types and sizes) are cached per hashable
    configuration."""
    with_ws = fn != "moe_layer_forward_static"
    try:
        specs = _layer_specs(cfg, with_ws)
    except TypeError:                    # not hashable
        specs = _layer_specs_of(cfg, with_ws)
    g = weights.get
    tensors = (g("w_router"), g("sel_bias"), g("w13"), g("w2"), g("ws13"), g("ws2"),
               x, y, topk_idx, topk_w, counts, stats, dropped, ws)
    on_device = _on_device
    for (name, dt, kind, numel, req), t in zip(specs, tensors):
        if t is None:
            if req:
                raise ValueError(f"{fn}: {name} is required")
            continue
        if isinstance(t, torch.Tensor):
            n_t = t.numel()
            if numel == 0 and n_t == 0:
                continue                 # nothing is read or written through it
            if (on_device(t) and t.is_contiguous() and
                    (n_t * t.element_size() >= numel if dt is None else (t.dtype is dt and n_t >= numel))):
                continue
        _arg(fn, name, t, kind, numel, cfg, required=req)
        raise ValueError(f"{fn}: {name} failed its check")


def moe_layer_forward(cfg, weights: dict, x, y, topk_idx=None, topk_w=None, counts=None, alpha=0.01, stats=None,
                      dropped=None, ws=None, stream=None):
    _check_layer_args("moe_layer_forward", cfg, weights, x, y, topk_idx, topk_w, counts, stats, dropped, ws)
    c = make_config(cfg)
    w = moe_weights()
    for name, _ in moe_weights._fields_:
        t = weights.get(name)
        setattr(w, name, None if t is None else t.data_ptr())
    _check("moe_layer_forward", lib().moe_layer_forward(
        ctypes.byref(c), ctypes.byref(w), _ptr(x), _ptr(y), _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
        float(alpha), _ptr(stats), _ptr(dropped), _ptr(ws), _ws_bytes(ws), _stream(stream)))


MOE_STATIC_SCRATCH_BYTES = 64 << 20


def moe_layer_forward_static(cfg, weights: dict, x, y, topk_idx=None, topk_w=None, counts=None, alpha=0.01,
                             stats=None, dropped=None, stream=None):
    """moe_layer_forward in the library's static device scratch: no workspace
    argument, nothing allocated (for callers that cannot allocate)."""
    _check_layer_args("moe_layer_forward_static", cfg, weights, x, y, topk_idx, topk_w, counts, stats, dropped, None)
    c = make_config(cfg)
    w = moe_weights()
    for name, _ in moe_weights._fields_:
        t = weights.get(name)
        setattr(w, name, None if t is None else t.data_ptr())
    _check("moe_layer_forward_static", lib().moe_layer_forward_static(
        ctypes.byref(c), ctypes.byref(w), _ptr(x), _ptr(y), _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
        float(alpha), _ptr(stats), _ptr(dropped), _stream(stream)))


def moe_layer_forward_timed(cfg, weights: dict, x, y, topk_idx=None, topk_w=None, counts=None, alpha=0.01,
                            stats=None, dropped=None, ws=None, stage_events=None, stream=None):
    """stage_events: list of 2 * len(STAGES) torch.cuda.Event (enable_timing=True)
    already recorded once (so that their HIP handles exist), or None entries."""
    _check_layer_args("moe_layer_forward_timed", cfg, weights, x, y, topk_idx, topk_w, counts, stats, dropped, ws)
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
    _check("moe_layer_forward_timed", lib().moe_layer_forward_timed(
        ctypes.byref(c), ctypes.byref(w), _ptr(x), _ptr(y), _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
        float(alpha), _ptr(stats), _ptr(dropped), _ptr(ws), _ws_bytes(ws), _stream(stream), arr))


def moe_layer_backward(cfg, weights: dict, x, dy, alpha, dx, dw_router, dw13, dw2, dws13=None, dws2=None, ws=None,
                       stream=None):
    """Gradients of <dy, y> + alpha-weighted balance loss, the routing fixed."""
    T, D, E, F = cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.d_ff
    nF = (2 if cfg.activation == MOE_SWIGLU else 1) * F
    SF = cfg.num_shared * cfg.d_ff_shared
    fn = "moe_layer_backward"
    _check_weights(fn, cfg, weights)
    for name, t in (("x", x), ("dy", dy), ("dx", dx)):
        _arg(fn, name, t, "act", T * D, cfg, required=T > 0)
    _arg(fn, "dw_router", dw_router, _F32, E * D, cfg, required=True)
    _arg(fn, "dw13", dw13, _F32, E * nF * D, cfg, required=True)
    _arg(fn, "dw2", dw2, _F32, E * D * F, cfg, required=True)
    _arg(fn, "dws13", dws13, _F32, 2 * SF * D, cfg, required=SF > 0)
    _arg(fn, "dws2", dws2, _F32, D * SF, cfg, required=SF > 0)
    _arg(fn, "ws", ws, _BYTES, moe_workspace_size(cfg, MOE_OP_LAYER_BACKWARD), cfg, required=T > 0)
    c = make_config(cfg)
    w = moe_weights()
    for name, _ in moe_weights._fields_:
        t = weights.get(name)
        setattr(w, name, None if t is None else t.data_ptr())
    _check("moe_layer_backward", lib().moe_layer_backward(
        ctypes.byref(c), ctypes.byref(w), _ptr(x), _ptr(dy), float(alpha), _ptr(dx), _ptr(dw_router), _ptr(dw13),
        _ptr(dw2), _ptr(dws13), _ptr(dws2), _ptr(ws), _ws_bytes(ws), _stream(stream)))


def moe_expert_choice_capacity(cfg) -> int:
    c = make_config(cfg)
    cap = ctypes.c_int32()
    _check("moe_expert_choice_capacity", lib().moe_expert_choice_capacity(ctypes.byref(c), ctypes.byref(cap)))
    return cap.value


def moe_expert_choice_forward(cfg, weights: dict, x, y, token_of_row=None, row_w=None, unselected=None, ws=None,
                              stage_events=None, stream=None):
    """Expert-choice layer forward; stage_events as for moe_layer_forward_timed."""
    T, D = cfg.num_tokens, cfg.d_model
    fn = "moe_expert_choice_forward"
    rows = cfg.num_experts * moe_expert_choice_capacity(cfg)
    _check_weights(fn, cfg, weights)
    _arg(fn, "x", x, "act", T * D, cfg, required=T > 0)
    _arg(fn, "y", y, "act", T * D, cfg, required=T > 0)
    _arg(fn, "token_of_row", token_of_row, _I32, rows, cfg)
    _arg(fn, "row_w", row_w, _F32, rows, cfg)
    _arg(fn, "unselected", unselected, _I32, 1, cfg)
    _arg(fn, "ws", ws, _BYTES, moe_workspace_size(cfg, MOE_OP_EXPERT_CHOICE), cfg, required=T > 0)
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
        _ptr(ws), _ws_bytes(ws), _stream(stream), arr))


class _Int32Only:
    act_dtype = router_dtype = MOE_F32


def moe_ep_send_layout(num_experts, num_ranks, offsets, send_counts, send_offsets, stream=None):
    fn = "moe_ep_send_layout"
    _arg(fn, "offsets", offsets, _I32, num_experts + 1, _Int32Only, required=True)
    _arg(fn, "send_counts", send_counts, _I32, max(num_ranks, 0), _Int32Only, required=True)
    _arg(fn, "send_offsets", send_offsets, _I32, max(num_ranks, 0) + 1, _Int32Only, required=True)
    _check("moe_ep_send_layout", lib().moe_ep_send_layout(num_experts, num_ranks, _ptr(offsets), _ptr(send_counts),
                                                          _ptr(send_offsets), _stream(stream)))


def moe_ep_recv_layout(recv_counts, rows_cap, local_offsets, gather, stream=None):
    """recv_counts: [R, E_local] int32 device tensor."""
    fn = "moe_ep_recv_layout"
    _arg(fn, "recv_counts", recv_counts, _I32, 1, _Int32Only, required=True)
    R, El = recv_counts.shape
    _arg(fn, "local_offsets", local_offsets, _I32, El + 1, _Int32Only, required=True)
    _arg(fn, "gather", gather, _I32, rows_cap, _Int32Only, required=rows_cap > 0)
    _check("moe_ep_recv_layout", lib().moe_ep_recv_layout(R, El, _ptr(recv_counts), rows_cap, _ptr(local_offsets),
                                                          _ptr(gather), _stream(stream)))
