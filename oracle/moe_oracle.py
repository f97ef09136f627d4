"""Plain CPU oracle for the forward pass of a sparse Mixture-of-Experts FFN
layer with token-choice top-k routing.

TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the benchmark's
CPU-baseline leg import this module.  The library never calls it, and this
module imports nothing from the library: the two share no code.

Everything is float64 NumPy.  bfloat16 inputs (uint16 bit patterns) and
float32 inputs are widened exactly, and no intermediate is rounded back to a
narrower type.  The structure follows the pages' plain per-expert loop, step by
step; the steps and their sources:

  route        router logits s = W_g x              "Top-k 路由" page, 門控函式的數學形式 Step 1;
                                                    Tiny-MoE page ("从 Dense FFN 到 MoE") §4 Router
  scores       softmax / sigmoid + selection bias   "Top-k 路由" Step 2 note (a)/(b);
                                                    "别只比较 Top-k" page, Score / Select / Merge steps
  top-k        k best experts per token             Tiny-MoE §4 (top-k of the probabilities); "Top-K Routing (MoE)"
                                                    glossary, Implementation Router MoE
  weights      renormalised / k-way softmax / raw   same places
  dispatch     per-expert (token, slot) lists       Tiny-MoE §5 (torch.where, row-major order)
  capacity     C = CF * tokens/E * k, overflow drop "Top-k 路由" 容量因子 section;
                                                    "别只比较 Top-k" mechanism table (Switch overflow)
  experts      SwiGLU / GELU FFN                    Tiny-MoE §3
  shared       always-on experts, weight 1          "别只比较 Top-k" six-family table
  combine      index_add of weighted outputs        Tiny-MoE §6; "Top-k 路由" Step 3
  statistics   importance, load, alpha*E*sum f*P    "Top-k 路由" 負載均衡 section; Tiny-MoE §8;
                                                    "别只比较 Top-k" [9,4,2,1] assignment example
  expert       each expert takes its top-C tokens   "Top-k 路由" Token-Choice vs Expert-Choice table;
   choice                                           "MoE 路由算法" page, 数学机理 (2)
  backward     gradients with the routing held fixed  "Top-k 路由" 門控網路的梯度流 (note 3, 反向 line);
                                                    Tiny-MoE §9
  EP layouts   rows per destination rank, received "Top-k 路由" 通訊拓撲：All-to-All figure;
               rows in expert-major order           "别只比较 Top-k" 按目标专家发送 / two-All-to-All
                                                    dispatcher section

Readings taken where the pages are silent (each is also listed with its reason
in the design notes):
  * top-k ties go to the lower expert index; slots are ordered by descending
    score (sorted top-k order);
  * SOFTMAX_TOPK ranks on p = softmax(s); TOPK_SOFTMAX ranks on s, the
    pages' Top-k(s) (same order as p); SIGMOID_BIAS ranks on sigmoid(s) + b;
  * rows inside an expert are in ascending token order, experts in ascending
    id: the row-major coordinate order torch.where returns;
  * capacity C = ceil(CF * T * k / E), evaluated in float64 from the float32
    value of CF; the first C assignments of an expert in token order are kept,
    overflow contributes zero (the residual path carries the token) and the
    surviving weights are not renormalised;
  * load f_e counts routed assignments (before capacity) over T*k;
    importance P_e is the token mean of the full softmax (sigmoid: a / sum a);
  * shared experts add with weight 1 to every token.

Parity pins: every function here is checked by the tests against the pages'
worked examples, closed forms, brute force or an independent library routine.
"""
from __future__ import annotations

import math
from typing import Callable, Dict, Optional, Sequence

import numpy as np
from scipy.special import erf

SOFTMAX_TOPK, TOPK_SOFTMAX, SIGMOID_BIAS = 0, 1, 2
SWIGLU, GELU = 0, 1


# --------------------------------------------------------------------------
# exact widening of stored inputs
# --------------------------------------------------------------------------
def widen(a: np.ndarray) -> np.ndarray:
    """Exact float64 value of a stored tensor: uint16 arrays are bfloat16 bit
    patterns (value = the float32 whose upper half is those bits)."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# Gate: logits, scores, top-k, weights
# --------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """s = W_g x for every token: x [T, D], W_g [E, D] (nn.Linear [out, in])
    -> s [T, E].  "Top-k 路由" Step 1; Tiny-MoE §4 (nn.Linear, bias=False)."""
    return widen(x) @ widen(w_router).T


def softmax(s: np.ndarray) -> np.ndarray:
    """Row softmax over experts (Tiny-MoE §4 routing probabilities)."""
    z = np.exp(s - s.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def sigmoid(s: np.ndarray) -> np.ndarray:
    """Affinity a = 1 / (1 + exp(-s)) ("别只比较 Top-k", Score: sigmoid affinity)."""
    return 1.0 / (1.0 + np.exp(-s))


def selection_key(s: np.ndarray, scoring: int, sel_bias: Optional[np.ndarray]) -> np.ndarray:
    """The quantity top-k ranks on.
    SOFTMAX_TOPK: p = softmax(s)           (softmax first, then top-k; note (a))
    TOPK_SOFTMAX: s itself                 (top-k of the logits; Step 2, note (b))
    SIGMOID_BIAS: sigmoid(s) + b           (bias takes part in selection only)"""
    if scoring == SOFTMAX_TOPK:
        return softmax(s)
    if scoring == TOPK_SOFTMAX:
        return s.copy()
    if scoring == SIGMOID_BIAS:
        b = np.zeros(s.shape[-1]) if sel_bias is None else widen(sel_bias)
        return sigmoid(s) + b[None, :]
    raise ValueError(f"unknown scoring {scoring}")


def exemption_key(s: np.ndarray, scoring: int, sel_bias: Optional[np.ndarray]) -> np.ndarray:
    """Score on which the 1e-6 relative near-tie exemption is measured: the
    routing probability for both softmax modes (same order as s), the biased
    affinity for sigmoid."""
    if scoring == TOPK_SOFTMAX:
        return softmax(s)
    return selection_key(s, scoring, sel_bias)


def topk(q: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries per row, in descending order; equal
    values go to the lower index (stable sort of -q)."""
    order = np.argsort(-q, axis=-1, kind="stable")
    return order[:, :k].astype(np.int64)


def gate_weights(s: np.ndarray, idx: np.ndarray, scoring: int, renormalize: int) -> np.ndarray:
    """Combine weight of each selected (token, slot).
    SOFTMAX_TOPK: p_sel, divided by sum p_sel when renormalize (Tiny-MoE §4;
                  glossary TopKRouter); raw p_top1 for Switch ("Top-k 路由"
                  Step 2 note: Switch keeps the softmax value).
    TOPK_SOFTMAX: exp(s_i) / sum_{j in TopK} exp(s_j)  ("Top-k 路由" Step 2).
    SIGMOID_BIAS: a_sel / sum a_sel from the *unbiased* affinity
                  ("别只比较 Top-k", Merge step)."""
    rows = np.arange(s.shape[0])[:, None]
    if scoring == SOFTMAX_TOPK:
        p = softmax(s)[rows, idx]
        return p / p.sum(axis=-1, keepdims=True) if renormalize else p
    if scoring == TOPK_SOFTMAX:
        sel = s[rows, idx]
        z = np.exp(sel - sel.max(axis=-1, keepdims=True))
        return z / z.sum(axis=-1, keepdims=True)
    if scoring == SIGMOID_BIAS:
        a = sigmoid(s)[rows, idx]
        return a / a.sum(axis=-1, keepdims=True) if renormalize else a
    raise ValueError(f"unknown scoring {scoring}")


def importance_probs(s: np.ndarray, scoring: int) -> np.ndarray:
    """Per-token soft probability over all experts used for P_e: the full
    softmax (Tiny-MoE §8: importance is its token mean); for sigmoid scoring
    the affinities normalised to sum 1 per token."""
    if scoring == SIGMOID_BIAS:
        a = sigmoid(s)
        return a / a.sum(axis=-1, keepdims=True)
    return softmax(s)


def near_tie_mask(key: np.ndarray, k: int, rel: float = 1e-6):
    """(boundary, slot_swap): boundary[t] is True where the k-th and (k+1)-th
    best keys differ by less than `rel` relative (either selection is correct);
    slot_swap[t, j] is True where slots j and j+1 may swap for the same reason."""
    T, E = key.shape
    srt = -np.sort(-key, axis=-1)
    denom = lambda v: np.maximum(np.abs(v), 1e-30)
    if k < E:
        boundary = (srt[:, k - 1] - srt[:, k]) / denom(srt[:, k - 1]) < rel
    else:
        boundary = np.zeros(T, dtype=bool)
    if k > 1:
        slot_swap = (srt[:, : k - 1] - srt[:, 1:k]) / denom(srt[:, : k - 1]) < rel
    else:
        slot_swap = np.zeros((T, 0), dtype=bool)
    return boundary, slot_swap


def route(x, w_router, sel_bias, top_k: int, scoring: int, renormalize: int) -> Dict[str, np.ndarray]:
    s = router_logits(x, w_router)
    q = selection_key(s, scoring, sel_bias)
    idx = topk(q, top_k)
    w = gate_weights(s, idx, scoring, renormalize)
    return dict(logits=s, key=q, idx=idx, w=w, probs=importance_probs(s, scoring))


# --------------------------------------------------------------------------
# Dispatch: counts, capacity, permutation
# --------------------------------------------------------------------------
def capacity(capacity_factor: float, num_tokens: int, top_k: int, num_experts: int) -> Optional[int]:
    """Expert buffer C = ceil(CF * T * k / E) ("Top-k 路由" 容量因子: CF x tokens/N x k),
    evaluated in float64 from the float32 value of CF; None when dropless."""
    cf = float(np.float32(capacity_factor))
    if cf <= 0.0:
        return None
    return int(math.ceil(cf * float(num_tokens * top_k) / float(num_experts)))


def expert_counts(idx: np.ndarray, num_experts: int) -> np.ndarray:
    """Routed assignments per expert (before capacity)."""
    c = np.zeros(num_experts, dtype=np.int64)
    for e in idx.reshape(-1):
        c[e] += 1
    return c


def dispatch(idx: np.ndarray, num_experts: int, cap: Optional[int]) -> Dict[str, np.ndarray]:
    """Per-expert batches, Tiny-MoE §5: for each expert in ascending id,
    (token_indices, route_slots) = coordinates of idx == e in row-major order.
    With a capacity the first `cap` of them are kept, the rest dropped
    (row -1).  Kept rows are laid out expert after expert."""
    T, k = idx.shape
    counts = expert_counts(idx, num_experts)
    kept = counts.copy() if cap is None else np.minimum(counts, cap)
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    row_of = np.full((T, k), -1, dtype=np.int64)
    token_of_row = np.zeros(int(offsets[-1]), dtype=np.int64)
    for e in range(num_experts):
        toks, slots = np.nonzero(idx == e)
        n = int(kept[e])
        rows = offsets[e] + np.arange(n)
        row_of[toks[:n], slots[:n]] = rows
        token_of_row[rows] = toks[:n]
    return dict(counts=counts, kept=kept, offsets=offsets, row_of=row_of,
                token_of_row=token_of_row, dropped=int(counts.sum() - kept.sum()))


# --------------------------------------------------------------------------
# Experts
# --------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def gelu(z: np.ndarray) -> np.ndarray:
    """Exact (erf) GELU, nn.GELU's default form (Tiny-MoE §3 classic FFN)."""
    return z * 0.5 * (1.0 + erf(z / math.sqrt(2.0)))


def swiglu_expert(X, w_gate, w_up, w_down) -> np.ndarray:
    """down(silu(gate(X)) * up(X)), Tiny-MoE §3 SwiGLU (bias-free nn.Linear)."""
    X = widen(X)
    h = silu(X @ widen(w_gate).T) * (X @ widen(w_up).T)
    return h @ widen(w_down).T


def gelu_expert(X, w_in, w_out) -> np.ndarray:
    """W_out gelu(W_in X), the classic FFN of Tiny-MoE §3 without biases."""
    X = widen(X)
    return gelu(X @ widen(w_in).T) @ widen(w_out).T


def expert_apply(X, w13, w2, activation: int, d_ff: int) -> np.ndarray:
    """One routed expert.  w13 holds gate rows then up rows (SwiGLU) or the input
    projection (GELU); w2 is the output projection [D, F]."""
    if activation == SWIGLU:
        return swiglu_expert(X, w13[:d_ff], w13[d_ff:2 * d_ff], w2)
    if activation == GELU:
        return gelu_expert(X, w13[:d_ff], w2)
    raise ValueError(f"unknown activation {activation}")


def shared_experts(x, shared: Sequence) -> np.ndarray:
    """Always-on experts: sum over s of SwiGLU_s(x), weight 1, every token
    ("别只比较 Top-k" six-family table: shared direct path)."""
    X = widen(x)
    y = np.zeros_like(X)
    for g, u, d in shared:
        y += swiglu_expert(X, g, u, d)
    return y


def expert_outputs(x, disp, expert_weights: Callable[[int], tuple], activation: int,
                   d_ff: int, num_experts: int) -> np.ndarray:
    """Y [A_kept, D]: expert e applied to its batch x[token_of_row[off_e:off_e+1]]
    (Tiny-MoE §5: an expert's batch is its tokens' rows).  Expert weights are
    fetched lazily so only experts with rows are materialised."""
    X = widen(x)
    off, tor = disp["offsets"], disp["token_of_row"]
    Y = np.zeros((int(off[-1]), X.shape[1]))
    for e in range(num_experts):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            w13, w2 = expert_weights(e)
            Y[a:b] = expert_apply(X[tor[a:b]], w13, w2, activation, d_ff)
    return Y


def combine(Y: np.ndarray, disp, w: np.ndarray, num_tokens: int, y_shared=None) -> np.ndarray:
    """y_t = sum over kept (t, j) of w[t, j] * Y[row(t, j)]  (+ shared), an
    accumulating scatter like index_add (Tiny-MoE §6; "Top-k 路由" Step 3).
    Dropped assignments add nothing."""
    D = Y.shape[1] if Y.size else (y_shared.shape[1] if y_shared is not None else 0)
    y = np.zeros((num_tokens, D))
    row_of = disp["row_of"]
    toks, slots = np.nonzero(row_of >= 0)
    np.add.at(y, toks, w[toks, slots][:, None] * Y[row_of[toks, slots]])
    if y_shared is not None:
        y += y_shared
    return y


# --------------------------------------------------------------------------
# Load statistics and balance loss
# --------------------------------------------------------------------------
def load_stats(counts: np.ndarray, probs: np.ndarray, top_k: int, alpha: float,
               kept: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """f_e = share of routed assignments, P_e = mean soft probability,
    L = alpha * E * sum f_e P_e ("Top-k 路由" 負載均衡; Tiny-MoE §8),
    imbalance = max count / ideal mean T*k/E ("别只比较 Top-k" [9,4,2,1]
    example) and dropped = assignments over capacity."""
    counts = np.asarray(counts, dtype=np.float64)
    E = counts.shape[0]
    A = counts.sum()
    f = counts / A
    P = probs.mean(axis=0)
    L = alpha * E * float(np.sum(f * P))
    imbalance = counts.max() / (A / E)
    dropped = 0 if kept is None else int(counts.sum() - np.asarray(kept).sum())
    return dict(f=f, P=P, aux_loss=L, imbalance=imbalance, dropped=dropped)


def num_parameters_swiglu(d_model: int, d_ff: int) -> int:
    """Parameters of one bias-free SwiGLU expert: gate [F,D] + up [F,D] + down [D,F]."""
    shapes = [(d_ff, d_model), (d_ff, d_model), (d_model, d_ff)]
    return sum(a * b for a, b in shapes)


# --------------------------------------------------------------------------
# Backward pass
# --------------------------------------------------------------------------
def silu_grad(z: np.ndarray) -> np.ndarray:
    """d silu / dz = sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    sg = sigmoid(z)
    return sg * (1.0 + z * (1.0 - sg))


def gelu_grad(z: np.ndarray) -> np.ndarray:
    """d gelu / dz for the erf GELU: Phi(z) + z phi(z)."""
    return 0.5 * (1.0 + erf(z / math.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def gate_grad(s: np.ndarray, idx: np.ndarray, dw: np.ndarray, scoring: int, renormalize: int) -> np.ndarray:
    """d loss / d s from d loss / d w through the combine weights of the
    selected experts only (the selection itself is a constant: "Top-k 路由"
    page, 門控網路的梯度流, note 3 and the 反向 line; Tiny-MoE §9).  For each
    token, with g the weights' gradient on the selected experts:
      raw probability  (w = p_sel):        ds = p * (g~ - <g~, p>), g~ = g on selected, 0 elsewhere
      renormalised / k-way softmax:        ds_sel = w * (g - <g, w>), 0 elsewhere
      sigmoid, renormalised:               ds_sel = a(1-a) * (g - <g, w>) / sum_sel a
      sigmoid, raw:                        ds_sel = a(1-a) * g"""
    T, E = s.shape
    ds = np.zeros((T, E))
    for t in range(T):
        sel = idx[t]
        g = dw[t]
        if scoring == SOFTMAX_TOPK and not renormalize:
            p = softmax(s[t])
            gt = np.zeros(E)
            np.add.at(gt, sel, g)
            ds[t] = p * (gt - np.dot(gt, p))
        elif scoring in (SOFTMAX_TOPK, TOPK_SOFTMAX):
            w = gate_weights(s[t:t + 1], sel[None, :], scoring, 1)[0]
            np.add.at(ds[t], sel, w * (g - np.dot(g, w)))
        else:
            a = sigmoid(s[t, sel])
            if renormalize:
                w = a / a.sum()
                np.add.at(ds[t], sel, a * (1.0 - a) * (g - np.dot(g, w)) / a.sum())
            else:
                np.add.at(ds[t], sel, a * (1.0 - a) * g)
    return ds


def aux_loss_grad(s: np.ndarray, counts: np.ndarray, top_k: int, alpha: float, scoring: int) -> np.ndarray:
    """d L_aux / d s for L_aux = alpha E sum_e f_e P_e with the assignment
    shares f constant (they come from the discrete routing) and P_e the token
    mean of the soft probabilities ("Top-k 路由" 負載均衡; Tiny-MoE §8-§9:
    the soft importance carries the balance loss's gradient)."""
    T, E = s.shape
    f = np.asarray(counts, dtype=np.float64) / (T * top_k)
    c = alpha * E * f / T                      # d L_aux / d p_hat[t, e], every token
    if scoring == SIGMOID_BIAS:
        a = sigmoid(s)
        S = a.sum(axis=1, keepdims=True)
        inner = (c[None, :] - (a * c[None, :]).sum(axis=1, keepdims=True) / S) / S
        return inner * a * (1.0 - a)
    p = softmax(s)
    return p * (c[None, :] - (p * c[None, :]).sum(axis=1, keepdims=True))


def backward(cfg, x, w_router, sel_bias, expert_weights: Callable[[int], tuple], shared: Sequence,
             dy: np.ndarray, alpha: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Gradients of  <dy, y> + L_aux  (dy: the gradient of the loss with
    respect to the layer output; L_aux the balance loss with coefficient
    alpha) with respect to x, the router weight, every routed expert's w13 /
    w2 and the shared experts' weights, the routing decisions held fixed
    (Tiny-MoE §9: selected experts get the task gradient, the router gets it
    through the selected weights and the balance-loss gradient through the
    soft importance; indices, counts and capacity drops are constants).
    Returns float64 dx [T, D], dw_router [E, D], dw13 {e: [n_mat F, D]},
    dw2 {e: [D, F]}, dshared [(d_gate, d_up, d_down)], and the intermediates
    dlogits [T, E], dw [T, k]."""
    T, E, k, F = cfg.num_tokens, cfg.num_experts, cfg.top_k, cfg.d_ff
    al = cfg.alpha if alpha is None else alpha
    fw = forward(cfg, x, w_router, sel_bias, expert_weights, shared, alpha=al)
    X = widen(x)
    dY = widen(dy) if dy.dtype == np.uint16 else np.asarray(dy, dtype=np.float64)
    dx = np.zeros_like(X)
    row_of, tor, off = fw["row_of"], fw["token_of_row"], fw["offsets"]
    # combine: y_t = sum_j w[t, j] Y[row(t, j)]
    dw = np.zeros((T, k))
    dYp = np.zeros_like(fw["y_perm"])
    for t in range(T):
        for j in range(k):
            r = row_of[t, j]
            if r >= 0:
                dw[t, j] = np.dot(dY[t], fw["y_perm"][r])
                dYp[r] = fw["w"][t, j] * dY[t]
    dw13, dw2 = {}, {}
    for e in range(E):
        a_, b_ = int(off[e]), int(off[e + 1])
        if b_ == a_:
            continue
        w13, w2 = expert_weights(e)
        W13, W2 = widen(w13), widen(w2)
        Xe = X[tor[a_:b_]]
        dYe = dYp[a_:b_]
        if cfg.activation == SWIGLU:
            G, U = Xe @ W13[:F].T, Xe @ W13[F:].T
            S = silu(G)
            H = S * U
            dH = dYe @ W2
            dG = dH * U * silu_grad(G)
            dU = dH * S
            dw13[e] = np.concatenate([dG.T @ Xe, dU.T @ Xe], axis=0)
            dXe = dG @ W13[:F] + dU @ W13[F:]
        else:
            Z = Xe @ W13.T
            H = gelu(Z)
            dH = dYe @ W2
            dZ = dH * gelu_grad(Z)
            dw13[e] = dZ.T @ Xe
            dXe = dZ @ W13
        dw2[e] = dYe.T @ H
        np.add.at(dx, tor[a_:b_], dXe)
    dsh = []
    for g, u, d in shared:
        Wg, Wu, Wd = widen(g), widen(u), widen(d)
        G, U = X @ Wg.T, X @ Wu.T
        S = silu(G)
        H = S * U
        dH = dY @ Wd
        dG = dH * U * silu_grad(G)
        dU = dH * S
        dsh.append((dG.T @ X, dU.T @ X, dY.T @ H))
        dx += dG @ Wg + dU @ Wu
    s = fw["logits"]
    dlogits = gate_grad(s, fw["idx"], dw, cfg.scoring, cfg.renormalize)
    dlogits += aux_loss_grad(s, fw["counts"], k, al, cfg.scoring)
    Wr = widen(w_router)
    dx += dlogits @ Wr
    return dict(dx=dx, dw_router=dlogits.T @ X, dw13=dw13, dw2=dw2, dshared=dsh, dlogits=dlogits, dw=dw,
                forward=fw)


# --------------------------------------------------------------------------
# Expert-choice routing
# --------------------------------------------------------------------------
def expert_choice_capacity(capacity_factor: float, num_tokens: int, top_k: int, num_experts: int) -> int:
    """Tokens each expert takes: the buffer formula of the "Top-k 路由" page
    (容量因子: CF * tokens / N * k) with k the average number of experts per
    token and CF = 1 when none is given, rounded up, at most T."""
    cf = float(np.float32(capacity_factor)) if capacity_factor > 0 else 1.0
    c = math.ceil(cf * num_tokens * top_k / num_experts) if num_tokens > 0 else 0
    return min(c, num_tokens)


def expert_choice_route(x, w_router, capacity: int) -> Dict[str, np.ndarray]:
    """Expert choice ("Top-k 路由" page, Token-Choice vs Expert-Choice table:
    each expert picks its top-C tokens; "MoE 路由算法" page, 数学机理 (2)): the
    routing probabilities p = softmax(W_g x) over experts, then for every
    expert the C tokens with the largest p[:, e] (equal values: lower token
    index first).  The gate of a chosen (token, expert) is p[t, e].  Rows are
    laid out expert after expert, tokens ascending inside an expert (as the
    token-choice dispatch); every expert has exactly C rows."""
    s = router_logits(x, w_router)
    p = softmax(s)
    T, E = p.shape
    chosen = topk(p.T, capacity) if capacity > 0 else np.zeros((E, 0), dtype=np.int64)   # [E, C], by score
    token_of_row = np.concatenate([np.sort(chosen[e]) for e in range(E)]) if E else np.zeros(0, np.int64)
    expert_of_row = np.repeat(np.arange(E), capacity)
    row_w = p[token_of_row, expert_of_row] if token_of_row.size else np.zeros(0)
    offsets = np.arange(E + 1, dtype=np.int64) * capacity
    return dict(logits=s, probs=p, chosen=chosen, token_of_row=token_of_row.astype(np.int64),
                row_w=row_w, offsets=offsets)


def expert_choice_combine(Y: np.ndarray, token_of_row: np.ndarray, row_w: np.ndarray, num_tokens: int,
                          y_shared=None) -> np.ndarray:
    """y_t = sum over the rows of token t of row_w * Y[row] (+ shared): the
    index_add accumulation of the Tiny-MoE §6 combine.  A token no expert
    chose gets nothing from the routed experts (the residual path carries it:
    "MoE 路由算法" page, 深度剖析 ②)."""
    D = Y.shape[1] if Y.size else (y_shared.shape[1] if y_shared is not None else 0)
    y = np.zeros((num_tokens, D))
    if token_of_row.size:
        np.add.at(y, token_of_row, row_w[:, None] * Y)
    if y_shared is not None:
        y += y_shared
    return y


def expert_choice_forward(cfg, x, w_router, expert_weights: Callable[[int], tuple],
                          shared: Sequence = ()) -> Dict[str, np.ndarray]:
    """Expert-choice layer: route, the selected experts' FFN on their rows,
    shared experts, combine.  Returns the routing and y."""
    C = expert_choice_capacity(cfg.capacity_factor, cfg.num_tokens, cfg.top_k, cfg.num_experts)
    r = expert_choice_route(x, w_router, C)
    disp = dict(offsets=r["offsets"], token_of_row=r["token_of_row"])
    Y = expert_outputs(x, disp, expert_weights, cfg.activation, cfg.d_ff, cfg.num_experts)
    ys = shared_experts(x, shared) if len(shared) else None
    y = expert_choice_combine(Y, r["token_of_row"], r["row_w"], cfg.num_tokens, ys)
    unselected = int(cfg.num_tokens - np.unique(r["token_of_row"]).size)
    return dict(route=r, capacity=C, Y=Y, y=y, unselected=unselected)


# --------------------------------------------------------------------------
# Expert parallelism: the layouts around the two all-to-all exchanges
# --------------------------------------------------------------------------
def ep_send_layout(kept: np.ndarray, num_ranks: int) -> Dict[str, np.ndarray]:
    """Rows each rank sends in the dispatch all-to-all ("Top-k 路由" page,
    通訊拓撲：All-to-All figure: experts 0-3 on one device, 4-7 on the other;
    "别只比较 Top-k" page, 按目标专家发送: an assignment goes to the rank that
    owns its expert).  Experts sit on ranks in contiguous blocks of E / R, so
    rank r receives the kept rows of experts r*E/R .. (r+1)*E/R - 1; with the
    rows laid out expert after expert those are one contiguous run.
    Returns send_counts [R] and send_offsets [R+1] (exclusive prefix)."""
    E = len(kept)
    assert E % num_ranks == 0
    per = E // num_ranks
    counts = np.zeros(num_ranks, dtype=np.int64)
    for e in range(E):
        counts[e // per] += int(kept[e])
    offsets = np.zeros(num_ranks + 1, dtype=np.int64)
    for r in range(num_ranks):
        offsets[r + 1] = offsets[r] + counts[r]
    return dict(send_counts=counts, send_offsets=offsets)


def ep_recv_layout(recv_counts: np.ndarray) -> Dict[str, np.ndarray]:
    """Where the local experts' rows sit after the dispatch all-to-all, and the
    expert-major view the local grouped FFN reads.  recv_counts[r][e] = rows
    that source rank r sends for local expert e.  The received buffer holds
    the sources one after another, each source's rows expert after expert
    (the order of its own expert-major rows).  The local FFN takes the rows
    of local expert 0 first (from source 0, then source 1, ...), then those
    of expert 1, and so on.  Returns local_offsets [E_local+1] and gather
    [rows]: gather[j] = position in the received buffer of expert-major row j."""
    recv_counts = np.asarray(recv_counts, dtype=np.int64)
    R, El = recv_counts.shape
    # received position of the first row of each (source, expert) run
    src_start = np.zeros((R, El), dtype=np.int64)
    pos = 0
    for r in range(R):
        for e in range(El):
            src_start[r, e] = pos
            pos += recv_counts[r, e]
    local_offsets = np.zeros(El + 1, dtype=np.int64)
    gather = np.zeros(pos, dtype=np.int64)
    j = 0
    for e in range(El):
        local_offsets[e] = j
        for r in range(R):
            for i in range(int(recv_counts[r, e])):
                gather[j] = src_start[r, e] + i
                j += 1
    local_offsets[El] = j
    return dict(local_offsets=local_offsets, gather=gather)


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------
def forward(cfg, x, w_router, sel_bias, expert_weights: Callable[[int], tuple],
            shared: Sequence = (), alpha: Optional[float] = None) -> Dict[str, np.ndarray]:
    """MoE layer forward, returning every intermediate the library exposes.
    `cfg` carries the fields of the layer configuration; `expert_weights(e)`
    returns (w13, w2) of routed expert e."""
    T, E, k = cfg.num_tokens, cfg.num_experts, cfg.top_k
    r = route(x, w_router, sel_bias, k, cfg.scoring, cfg.renormalize)
    cap = capacity(cfg.capacity_factor, T, k, E)
    disp = dispatch(r["idx"], E, cap)
    Y = expert_outputs(x, disp, expert_weights, cfg.activation, cfg.d_ff, E)
    ys = shared_experts(x, shared) if len(shared) else None
    y = combine(Y, disp, r["w"], T, ys)
    st = load_stats(disp["counts"], r["probs"], k, cfg.alpha if alpha is None else alpha, disp["kept"])
    out = dict(r)
    out.update(disp)
    out.update(st)
    out.update(y_perm=Y, y_shared=ys, y=y, capacity=cap)
    return out
