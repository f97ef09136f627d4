"""Helpers of the GPU parity tests: run the oracle and the HIP path on the same
seeded inputs and compare them element by element.

Bars (from the layer's definition of equivalence):
  * expert ids, counts, permutation and drop decisions: bit-exact, except
    tokens whose k-th and (k+1)-th oracle scores are within 1e-6 relative
    (either choice is correct there; adjacent slots within 1e-6 may swap).
    At such a token the GPU's choice must itself be a correct top-k under that
    band; the oracle's steps after the selection (weights, counts, capacity,
    permutation, drops, statistics, experts, combine), which are pure
    functions of the chosen experts, are then re-run with the GPU's choice
    and every token is compared against that re-run, capacity configurations
    included;
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
REL_TIE = 1e-6     # near-tie band of the selection, relative to the k-th best key


def set_env(monkeypatch, name: str, value: str):
    """Set a MOE_* tuning variable for one test and make the library read it
    (it reads them once otherwise); conftest re-reads them after the test."""
    monkeypatch.setenv(name, value)
    M.moe_reload_tuning()


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


def _band(v) -> float:
    return REL_TIE * max(abs(float(v)), 1e-30)


def selection_error(key_row: np.ndarray, sel, k: int):
    """Why an ordered selection `sel` of one token is not a correct top-k of
    `key_row` under the near-tie rule, or None when it is.  Correct means: k
    distinct experts in range; none left out ranks above a chosen one by more
    than 1e-6 relative to the k-th best key (so the set can differ from the
    oracle's only across a near-tied selection boundary); and the slots are in
    descending key order up to the same relative band (adjacent near-tied
    slots may swap)."""
    E = key_row.shape[0]
    sel = [int(e) for e in sel]
    if len(sel) != k or len(set(sel)) != k or min(sel) < 0 or max(sel) >= E:
        return f"not {k} distinct experts in [0, {E})"
    qk = np.sort(key_row)[::-1][k - 1]
    chosen = key_row[sel]
    if k < E:
        rest = np.delete(key_row, sel)
        if rest.max() - chosen.min() >= _band(qk):
            return "an expert left out ranks above a chosen one by more than the tie band"
    for j in range(k - 1):
        a, b = chosen[j], chosen[j + 1]
        if b - a >= REL_TIE * max(abs(float(a)), abs(float(b)), 1e-30):
            return f"slots {j} and {j + 1} out of order beyond the tie band"
    return None


def route_differences(cfg, ref, idx_gpu: np.ndarray, sel_bias) -> np.ndarray:
    """Tokens whose GPU selection differs from the oracle's; asserts that every
    such token carries a selection that is itself correct under the near-tie
    rule, measured on the oracle's float64 key (exemption_key)."""
    key = O.exemption_key(ref["logits"], cfg.scoring, sel_bias)
    idx_ref = ref["idx"]
    diff = np.nonzero((idx_gpu != idx_ref).any(axis=1))[0]
    for t in diff:
        why = selection_error(key[t], idx_gpu[t], cfg.top_k)
        assert why is None, (f"token {t}: gpu {idx_gpu[t].tolist()} vs oracle {idx_ref[t].tolist()}: {why}")
    return diff


def rerun_on_choice(cfg, ref, idx_gpu: np.ndarray, diff: np.ndarray, alpha=None):
    """The oracle's steps after the selection, which are pure functions of the
    chosen experts, re-run with the GPU's (equally valid) choice at the exempt
    tokens `diff`: gate weights of the chosen experts, counts, capacity,
    permutation, drops and the load statistics.  Returns dict(idx, w, disp,
    stats)."""
    T, E, k = cfg.num_tokens, cfg.num_experts, cfg.top_k
    al = cfg.alpha if alpha is None else alpha
    if len(diff) == 0:
        idx, w = ref["idx"], ref["w"]
    else:
        idx = ref["idx"].copy()
        idx[diff] = idx_gpu[diff]
        w = ref["w"].copy()
        w[diff] = O.gate_weights(ref["logits"][diff], idx[diff], cfg.scoring, cfg.renormalize)
    if len(diff) == 0 and "row_of" in ref:
        disp = {key: ref[key] for key in ("counts", "kept", "offsets", "row_of", "token_of_row", "dropped")}
    else:
        disp = O.dispatch(idx, E, O.capacity(cfg.capacity_factor, T, k, E))
    st = O.load_stats(disp["counts"], ref["probs"], k, al, disp["kept"])
    return dict(idx=idx, w=w, disp=disp, stats=st)


def check_stats(cfg, st, got_stats: np.ndarray, got_dropped: int):
    E = cfg.num_experts
    assert got_dropped == st["dropped"], f"dropped {got_dropped} vs {st['dropped']}"
    assert rel_err(got_stats[:E], st["f"]) <= W_TOL
    assert rel_err(got_stats[E:2 * E], st["P"]) <= W_TOL
    assert abs(got_stats[2 * E] - st["aux_loss"]) <= W_TOL * abs(st["aux_loss"]) + 1e-12
    assert abs(got_stats[2 * E + 1] - st["imbalance"]) <= W_TOL * abs(st["imbalance"])


def layer_output_on_choice(cfg, inp, ref, ch):
    """y of the oracle's dispatch / experts / combine for the re-run choice."""
    if ch["idx"] is ref["idx"]:
        return ref["y"]
    Y = O.expert_outputs(inp.x, ch["disp"], lambda e: (inp.w13[e], inp.w2[e]), cfg.activation, cfg.d_ff,
                         cfg.num_experts)
    return O.combine(Y, ch["disp"], ch["w"], cfg.num_tokens, ref["y_shared"])


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


def check_layer(cfg, inp, ref, got, sel_bias=None, alpha=None):
    """Full-layer comparison: selection (near-tie exemption only), then counts,
    drops, weights, statistics and every token's output against the oracle
    re-run on the GPU's choice at the exempt tokens."""
    b = inp.sel_bias if sel_bias is None else sel_bias
    diff = route_differences(cfg, ref, got["idx"], b)
    ch = rerun_on_choice(cfg, ref, got["idx"], diff, alpha)
    np.testing.assert_array_equal(got["counts"], ch["disp"]["counts"])
    assert rel_err(got["w"], ch["w"]) <= W_TOL
    check_stats(cfg, ch["stats"], got["stats"], got["dropped"])
    err = row_rel_err(got["y"], layer_output_on_choice(cfg, inp, ref, ch))
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
