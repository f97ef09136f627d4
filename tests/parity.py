"""Helpers of the GPU parity tests: run the oracle and the HIP path on the same
seeded inputs and compare them element by element.

Bars (from the layer's definition of equivalence):
  * expert ids, counts, permutation and drop decisions: bit-exact, except
    tokens whose k-th and (k+1)-th oracle scores are within 1e-6 relative
    (either choice is correct there; adjacent slots within 1e-6 may swap);
  * float32 outputs within 1e-5 relative; bfloat16 outputs within 2e-2 max
    relative error, where the error of an element is |gpu - ref| divided by
    max(|ref|, rms of that token's reference row).
"""
from __future__ import annotations

import numpy as np
import torch

import top_routing_dispatch_amd as M
import workloads as W
from oracle import moe_oracle as O
from workloads.torch_io import act_torch_dtype, device_weights, to_numpy, to_torch

F32_TOL = 1e-5
BF16_TOL = 2e-2
W_TOL = 1e-5


def out_tol(cfg) -> float:
    return BF16_TOL if cfg.act_dtype == W.BF16 else F32_TOL


def row_rel_err(y_gpu: np.ndarray, y_ref: np.ndarray) -> float:
    y_gpu = O.widen(y_gpu) if y_gpu.dtype == np.uint16 else y_gpu.astype(np.float64)
    if y_ref.size == 0:
        return 0.0
    rms = np.sqrt((y_ref ** 2).mean(axis=-1, keepdims=True))
    denom = np.maximum(np.abs(y_ref), rms)
    denom = np.where(denom == 0, 1.0, denom)
    return float((np.abs(y_gpu - y_ref) / denom).max())


def rel_err(a: np.ndarray, ref: np.ndarray) -> float:
    a = a.astype(np.float64)
    if ref.size == 0:
        return 0.0
    return float((np.abs(a - ref) / np.maximum(np.abs(ref), 1e-30)).max())


def oracle_forward(cfg, inp, sel_bias=None):
    b = inp.sel_bias if sel_bias is None else sel_bias
    return O.forward(cfg, inp.x, inp.w_router, b, lambda e: (inp.w13[e], inp.w2[e]), inp.shared)


def refinement_margin(s32: np.ndarray) -> np.ndarray:
    """Per-token logit margin within which the route kernel trusts its float32
    logits (tokens with keys closer than that are refined in float64)."""
    return np.ldexp(1.0 + np.abs(s32).max(axis=1), -16)


def route_differences(cfg, ref, idx_gpu: np.ndarray, sel_bias) -> np.ndarray:
    """Tokens whose GPU selection differs from the oracle's; asserts that every
    such token is a near-tie the oracle itself cannot decide (1e-6 relative)."""
    key = O.exemption_key(ref["logits"], cfg.scoring, sel_bias)
    bnd, swp = O.near_tie_mask(key, cfg.top_k)
    idx_ref = ref["idx"]
    diff = np.nonzero((idx_gpu != idx_ref).any(axis=1))[0]
    for t in diff:
        if bnd[t]:
            continue
        # same set, order differs only across near-tied adjacent slots
        assert sorted(idx_gpu[t].tolist()) == sorted(idx_ref[t].tolist()), (
            f"token {t}: gpu {idx_gpu[t].tolist()} vs oracle {idx_ref[t].tolist()} (not a near tie)")
        for j in range(cfg.top_k):
            if idx_gpu[t, j] != idx_ref[t, j]:
                assert (j < cfg.top_k - 1 and swp[t, j]) or (j > 0 and swp[t, j - 1]), (
                    f"token {t} slot {j}: gpu {idx_gpu[t].tolist()} vs oracle {idx_ref[t].tolist()}")
    return diff


class DeviceLayer:
    """The seeded workload on the GPU plus the library's workspaces."""

    def __init__(self, cfg, inp, sel_bias=None, device="cuda"):
        self.cfg, self.inp = cfg, inp
        self.dev = device
        self.x = to_torch(inp.x, device)
        self.weights = device_weights(inp, device)
        if sel_bias is not None:
            self.weights["sel_bias"] = to_torch(np.asarray(sel_bias, dtype=np.float32), device)
        self.cap, self.rows_cap = M.moe_capacity(cfg)

    def layer(self, alpha=None, ws=None):
        cfg, T, k, E = self.cfg, self.cfg.num_tokens, self.cfg.top_k, self.cfg.num_experts
        dev = self.dev
        y = torch.empty((T, cfg.d_model), dtype=act_torch_dtype(cfg), device=dev)
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        counts = torch.empty(E, dtype=torch.int32, device=dev)
        stats = torch.empty(2 * E + 2, dtype=torch.float32, device=dev)
        dropped = torch.empty(1, dtype=torch.int32, device=dev)
        if ws is None:
            ws = M.workspace(cfg, M.MOE_OP_LAYER, dev)
        M.moe_layer_forward(cfg, self.weights, self.x, y, idx, w, counts, cfg.alpha if alpha is None else alpha,
                            stats, dropped, ws)
        torch.cuda.synchronize()
        return dict(y=to_numpy(y), idx=to_numpy(idx), w=to_numpy(w), counts=to_numpy(counts),
                    stats=to_numpy(stats), dropped=int(to_numpy(dropped)[0]))

    def route(self, with_probs=True):
        cfg, T, k, E = self.cfg, self.cfg.num_tokens, self.cfg.top_k, self.cfg.num_experts
        idx = torch.empty((T, k), dtype=torch.int32, device=self.dev)
        w = torch.empty((T, k), dtype=torch.float32, device=self.dev)
        probs = torch.empty((T, E), dtype=torch.float32, device=self.dev) if with_probs else None
        ws = M.workspace(cfg, M.MOE_OP_ROUTE, self.dev)
        M.moe_route(cfg, self.x, self.weights["w_router"], self.weights["sel_bias"], idx, w, probs, ws)
        torch.cuda.synchronize()
        return dict(idx=to_numpy(idx), w=to_numpy(w), probs=None if probs is None else to_numpy(probs))


def check_layer(cfg, inp, ref, got, sel_bias=None):
    """Full-layer comparison: selection, counts, weights, outputs, statistics."""
    b = inp.sel_bias if sel_bias is None else sel_bias
    diff = route_differences(cfg, ref, got["idx"], b)
    same = np.setdiff1d(np.arange(cfg.num_tokens), diff)
    # counts: the oracle's, moved by the exempt tokens' (equally valid) choices
    counts = ref["counts"].copy()
    for t in diff:
        for e in ref["idx"][t]:
            counts[e] -= 1
        for e in got["idx"][t]:
            counts[e] += 1
    np.testing.assert_array_equal(got["counts"], counts)
    assert rel_err(got["w"][same], ref["w"][same]) <= W_TOL
    if len(diff) == 0:
        assert got["dropped"] == ref["dropped"]
        E = cfg.num_experts
        st = got["stats"]
        assert rel_err(st[:E], ref["f"]) <= W_TOL
        assert rel_err(st[E:2 * E], ref["P"]) <= W_TOL
        assert abs(st[2 * E] - ref["aux_loss"]) <= W_TOL * abs(ref["aux_loss"]) + 1e-12
        assert abs(st[2 * E + 1] - ref["imbalance"]) <= W_TOL * abs(ref["imbalance"])
        err = row_rel_err(got["y"], ref["y"])
    else:
        # tokens sharing a capacity-limited expert with a near-tie token may legitimately move;
        # compare the rest
        err = row_rel_err(got["y"][same], ref["y"][same]) if cfg.capacity_factor <= 0 else 0.0
    assert err <= out_tol(cfg), f"max relative error {err:.3e} > {out_tol(cfg)}"
    return diff, err


def ec_check_selection(ref, tor_gpu: np.ndarray, capacity: int) -> int:
    """Expert-choice choices of the GPU against the oracle's: per expert the
    same token set, except tokens whose probability is within 1e-6 relative
    of the expert's C-th largest (either choice is correct there); rows of an
    expert ascending.  Returns the number of experts with a near-tie exchange."""
    p = ref["probs"]
    T, E = p.shape
    C = capacity
    ties = 0
    for e in range(E):
        got = tor_gpu[e * C:(e + 1) * C]
        assert (np.diff(got) > 0).all(), f"expert {e}: rows not ascending"
        want = ref["token_of_row"][e * C:(e + 1) * C]
        if np.array_equal(got, want):
            continue
        col = p[:, e]
        v = np.sort(col)[::-1][C - 1]
        band = np.abs(col - v) <= 1e-6 * abs(v)
        sg, sw = set(got.tolist()), set(want.tolist())
        for t in sg ^ sw:
            assert band[t], f"expert {e}: token {t} chosen differently and not a near tie"
        ties += 1
    return ties


def ec_oracle_output(cfg, inp, tor: np.ndarray, capacity: int, expert_weights=None, rows=None):
    """Oracle layer output for a given expert-choice selection (the GPU's, so
    that near-tie exchanges do not matter): float64 probabilities as gates.
    rows: optional token subset to evaluate."""
    p = O.softmax(O.router_logits(inp.x, inp.w_router))
    T = cfg.num_tokens
    C = capacity
    ew = expert_weights or (lambda e: (inp.w13[e], inp.w2[e]))
    X = O.widen(inp.x)
    toks = np.arange(T) if rows is None else np.asarray(rows)
    pos = {int(t): i for i, t in enumerate(toks)}
    y = np.zeros((len(toks), X.shape[1]))
    for e in range(cfg.num_experts):
        sel = [int(t) for t in tor[e * C:(e + 1) * C] if int(t) in pos]
        if not sel:
            continue
        w13, w2 = ew(e)
        out = O.expert_apply(X[sel], w13, w2, cfg.activation, cfg.d_ff)
        for t, o in zip(sel, out):
            y[pos[t]] += p[t, e] * o
    if cfg.num_shared:
        y += O.shared_experts(inp.x[toks], inp.shared)
    return y
