"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test ties one oracle function to something other than itself: a worked
example printed on the pages (tests/golden/*.json, each citing its source),
a closed form, an invariant, brute force on tiny inputs, or an independent
library routine (CPU torch in float64).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# router / top-k / weights
# --------------------------------------------------------------------------
def test_router_worked_example():
    g = gold("router_worked_example.json")
    p = np.array([g["probabilities"]])
    s = np.log(p)                       # softmax(log p) = p exactly up to rounding
    q = O.selection_key(s, O.SOFTMAX_TOPK, None)
    np.testing.assert_allclose(q, p, rtol=1e-15)
    idx = O.topk(q, g["top_k"])
    assert idx.tolist() == [g["topk_indices"]]
    raw = O.gate_weights(s, idx, O.SOFTMAX_TOPK, renormalize=0)
    np.testing.assert_allclose(raw, [g["topk_weights"]], rtol=1e-14)
    ren = O.gate_weights(s, idx, O.SOFTMAX_TOPK, renormalize=1)
    np.testing.assert_allclose(ren, [g["renormalized"]], rtol=1e-14)
    # tie reading: 0.10 at experts 0 and 3 -> expert 0
    assert O.topk(q, 3).tolist() == [g["top3_indices"]]


def _brute_topk(qrow, k):
    """Max-sum subset of size k; among equal sums the lexicographically smallest
    index tuple; then slots ordered by (value desc, index asc)."""
    best, best_sum = None, None
    for comb in itertools.combinations(range(len(qrow)), k):
        ssum = sum(qrow[i] for i in comb)
        if best is None or ssum > best_sum or (ssum == best_sum and comb < best):
            best, best_sum = comb, ssum
    return sorted(best, key=lambda i: (-qrow[i], i))


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_random_and_ties(seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(20):
        T = int(rng.integers(1, 17))
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, min(E, 4) + 1))
        if seed % 2 == 0:
            q = rng.integers(0, 3, size=(T, E)).astype(np.float64)   # many exact ties, exact sums
        else:
            q = rng.standard_normal((T, E)).round(1)                   # ties after rounding
            q = np.round(q * 10).astype(np.float64)                    # integers: exact subset sums
        idx = O.topk(q, k)
        for t in range(T):
            assert idx[t].tolist() == _brute_topk(q[t].tolist(), k)


def test_topk_values_match_torch():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((50, 33))
    idx = O.topk(q, 5)
    vals = np.take_along_axis(q, idx, axis=1)
    tv, _ = torch.topk(torch.from_numpy(q), 5, dim=-1, sorted=True)
    np.testing.assert_array_equal(vals, tv.numpy())


def test_softmax_matches_torch_and_sums_to_one():
    rng = np.random.default_rng(8)
    s = rng.standard_normal((40, 17)) * 3
    p = O.softmax(s)
    np.testing.assert_allclose(p, torch.softmax(torch.from_numpy(s), -1).numpy(), rtol=1e-13, atol=0)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-14)


def test_renormalised_weights_sum_to_one():
    rng = np.random.default_rng(9)
    s = rng.standard_normal((64, 16))
    b = rng.uniform(-0.1, 0.1, 16)
    for scoring, ren in [(O.SOFTMAX_TOPK, 1), (O.TOPK_SOFTMAX, 0), (O.SIGMOID_BIAS, 1)]:
        idx = O.topk(O.selection_key(s, scoring, b), 4)
        w = O.gate_weights(s, idx, scoring, ren)
        np.testing.assert_allclose(w.sum(-1), 1.0, rtol=1e-14)
        assert (w > 0).all()


def test_topk_softmax_equals_renormalised_softmax_topk():
    """exp(s_i)/sum_K exp(s_j) = p_i / sum_K p_j: the two softmax orders agree once
    the selected probabilities are renormalised (closed form)."""
    rng = np.random.default_rng(10)
    s = rng.standard_normal((80, 12)) * 2
    i1 = O.topk(O.selection_key(s, O.TOPK_SOFTMAX, None), 3)
    i2 = O.topk(O.selection_key(s, O.SOFTMAX_TOPK, None), 3)
    np.testing.assert_array_equal(i1, i2)
    w1 = O.gate_weights(s, i1, O.TOPK_SOFTMAX, 0)
    w2 = O.gate_weights(s, i2, O.SOFTMAX_TOPK, 1)
    np.testing.assert_allclose(w1, w2, rtol=1e-13)
    # and TOPK_SOFTMAX's weight is the k-way softmax of the selected logits, checked with torch
    sel = np.take_along_axis(s, i1, 1)
    np.testing.assert_allclose(w1, torch.softmax(torch.from_numpy(sel), -1).numpy(), rtol=1e-13)


def test_switch_top1_weight_is_raw_probability():
    rng = np.random.default_rng(11)
    s = rng.standard_normal((100, 128)) * 0.5
    idx = O.topk(O.selection_key(s, O.SOFTMAX_TOPK, None), 1)
    w = O.gate_weights(s, idx, O.SOFTMAX_TOPK, renormalize=0)
    p = torch.softmax(torch.from_numpy(s), -1).numpy()
    np.testing.assert_allclose(w[:, 0], p.max(-1), rtol=1e-13)
    assert (w[:, 0] >= 1.0 / 128).all() and (w[:, 0] < 1).all()


def test_sigmoid_bias_selection_only():
    rng = np.random.default_rng(12)
    s = rng.standard_normal((60, 32))
    # b = 0: sigmoid is monotone, so selection = top-k of the logits
    i0 = O.topk(O.selection_key(s, O.SIGMOID_BIAS, np.zeros(32)), 8)
    np.testing.assert_array_equal(i0, O.topk(s, 8))
    # a large bias on a chosen set forces that set; the weights ignore the bias
    forced = np.array([3, 5, 7, 11, 13, 17, 19, 23])
    b = np.zeros(32)
    b[forced] = 10.0
    i1 = O.topk(O.selection_key(s, O.SIGMOID_BIAS, b), 8)
    assert all(sorted(r) == sorted(forced.tolist()) for r in i1.tolist())
    w = O.gate_weights(s, i1, O.SIGMOID_BIAS, 1)
    a = 1.0 / (1.0 + np.exp(-np.take_along_axis(s, i1, 1)))
    np.testing.assert_allclose(w, a / a.sum(1, keepdims=True), rtol=1e-14)
    # torch's sigmoid as an independent routine for the affinity
    np.testing.assert_allclose(O.sigmoid(s), torch.sigmoid(torch.from_numpy(s)).numpy(), rtol=1e-14)


def test_near_tie_mask():
    key = np.array([[0.5, 0.3, 0.3, 0.1],            # boundary tie at k=2
                    [0.4, 0.4, 0.1, 0.1],            # slot tie only
                    [0.5, 0.3, 0.3 - 1e-3, 0.1]])    # clear gap
    bnd, sw = O.near_tie_mask(key, 2)
    assert bnd.tolist() == [True, False, False]
    assert sw[:, 0].tolist() == [False, True, False]


# --------------------------------------------------------------------------
# exact widening of stored inputs
# --------------------------------------------------------------------------
def test_widen_every_bfloat16_pattern_matches_torch():
    """All 65,536 bfloat16 bit patterns against torch's own bfloat16 -> float64
    conversion (NaN patterns stay NaN, signed zeros and infinities keep their
    sign)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.widen(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127                      # exponent all ones, mantissa non-zero, both signs
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_widen_hand_values():
    """bfloat16 = sign, 8 exponent bits (bias 127), 7 mantissa bits."""
    cases = {0x3F80: 1.0, 0xC049: -3.140625, 0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126,
             0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127, 0x8000: -0.0, 0x7F80: math.inf, 0xFF80: -math.inf,
             0x3E80: 0.25, 0x4120: 10.0}
    bits = np.array(list(cases), dtype=np.uint16)
    got = O.widen(bits)
    for b, v, g in zip(cases, cases.values(), got):
        assert g == v and math.copysign(1.0, g) == math.copysign(1.0, v), hex(b)
    # float32 storage widens to the same value (no bit reinterpretation)
    f = np.array([1.5, -2.25e-30, 3.0e38], dtype=np.float32)
    np.testing.assert_array_equal(O.widen(f), torch.from_numpy(f).double().numpy())
    # a bfloat16 pattern is the upper half of the float32 it stands for
    f32 = np.array([1.0, -3.140625, 0.25], dtype=np.float32)
    np.testing.assert_array_equal(O.widen((f32.view(np.uint32) >> 16).astype(np.uint16)), f32.astype(np.float64))


# --------------------------------------------------------------------------
# near-tie exemption key
# --------------------------------------------------------------------------
def test_exemption_key_per_mode_matches_library_routines():
    """The score the 1e-6 exemption is measured on: the routing probability
    softmax(s) for both softmax modes, the biased affinity sigmoid(s) + b for
    sigmoid scoring (torch's float64 softmax / sigmoid as independent
    routines)."""
    rng = np.random.default_rng(31)
    s = rng.standard_normal((40, 16)) * 2
    b = rng.uniform(-0.1, 0.1, 16)
    p = torch.softmax(torch.from_numpy(s), -1).numpy()
    for scoring in (O.SOFTMAX_TOPK, O.TOPK_SOFTMAX):
        np.testing.assert_allclose(O.exemption_key(s, scoring, None), p, rtol=1e-13, atol=0)
    a = torch.sigmoid(torch.from_numpy(s)).numpy()
    np.testing.assert_allclose(O.exemption_key(s, O.SIGMOID_BIAS, b), a + b[None, :], rtol=1e-14, atol=0)
    np.testing.assert_allclose(O.exemption_key(s, O.SIGMOID_BIAS, None), a, rtol=1e-14, atol=0)


def test_exemption_key_orders_like_the_selection_key():
    """The exemption key ranks the experts exactly as the key top-k selects on
    (p is monotone in s), so exempt tokens are those whose selection boundary
    is close, in every mode."""
    rng = np.random.default_rng(32)
    s = rng.standard_normal((200, 24)) * 3
    b = rng.uniform(-0.1, 0.1, 24)
    for scoring in (O.SOFTMAX_TOPK, O.TOPK_SOFTMAX, O.SIGMOID_BIAS):
        bias = b if scoring == O.SIGMOID_BIAS else None
        np.testing.assert_array_equal(O.topk(O.exemption_key(s, scoring, bias), 6),
                                      O.topk(O.selection_key(s, scoring, bias), 6))


def test_topk_softmax_exemption_gap_is_the_logit_difference():
    """For top-k-then-softmax the ranking is on the logits, whose relative gap
    depends on where zero is; the exemption uses p instead, whose relative gap
    (p_i - p_j) / p_i = 1 - exp(-(s_i - s_j)) depends only on the logit
    difference (closed form), like the k-way softmax weights themselves."""
    rng = np.random.default_rng(33)
    s = rng.standard_normal((50, 8))
    key = O.exemption_key(s, O.TOPK_SOFTMAX, None)
    srt = -np.sort(-key, axis=1)
    ss = -np.sort(-s, axis=1)
    np.testing.assert_allclose((srt[:, 0] - srt[:, 1]) / srt[:, 0], -np.expm1(-(ss[:, 0] - ss[:, 1])), rtol=1e-9)
    # shifting every logit of a token leaves the exemption decision unchanged
    for c in (-50.0, 1e-3, 75.0):
        np.testing.assert_allclose(O.exemption_key(s + c, O.TOPK_SOFTMAX, None), key, rtol=1e-12)


@pytest.mark.parametrize("scoring", [O.SOFTMAX_TOPK, O.TOPK_SOFTMAX])
def test_softmax_modes_exempt_hand_built_near_ties(scoring):
    """k = 2; experts 1 and 2 straddle the boundary.  A logit gap of 4e-7 is a
    relative gap of about 4e-7 in p (exempt), 3e-6 is not; a gap of 4e-7
    between slots 1 and 2 only lets the slots swap.  Logits near zero show why
    the gap is not measured on s: 1e-9 against -1e-9 is a relative gap of 2 in
    s but a near tie in p."""
    s = np.array([[1.0, 0.5, 0.5 - 4e-7, 0.0],
                  [1.0, 0.5, 0.5 - 3e-6, 0.0],
                  [0.7, 0.7 - 4e-7, 0.2, 0.0],
                  [0.9, 1e-9, -1e-9, -0.5]])
    bnd, swp = O.near_tie_mask(O.exemption_key(s, scoring, None), 2)
    assert bnd.tolist() == [True, False, False, True]
    assert swp[:, 0].tolist() == [False, False, True, False]


def test_sigmoid_mode_exempts_near_ties_of_the_biased_affinity():
    """The sigmoid exemption is measured on a + b, the key that selects: two
    experts whose logits are far apart can tie once the bias is added, and the
    same logits with no bias are not a near tie."""
    a1, b1, b2 = 0.6, 0.0, -0.05
    a2 = a1 + b1 - b2 + 2e-7                          # a2 + b2 = a1 + b1 + 2e-7
    s = np.array([[3.0, math.log(a1 / (1 - a1)), math.log(a2 / (1 - a2)), -2.0]])
    b = np.array([0.0, b1, b2, 0.0])
    bnd, _ = O.near_tie_mask(O.exemption_key(s, O.SIGMOID_BIAS, b), 2)
    assert bnd.tolist() == [True]
    bnd0, _ = O.near_tie_mask(O.exemption_key(s, O.SIGMOID_BIAS, np.zeros(4)), 2)
    assert bnd0.tolist() == [False]


# --------------------------------------------------------------------------
# dispatch and capacity
# --------------------------------------------------------------------------
def test_dispatch_worked_example():
    g = gold("dispatch_worked_example.json")
    idx = np.array(g["topk_indices"])
    d = O.dispatch(idx, 4, None)
    e = g["expert"]
    rows = range(d["offsets"][e], d["offsets"][e + 1])
    toks = [int(d["token_of_row"][r]) for r in rows]
    assert toks == g["token_indices"]
    slots = [int(np.nonzero(d["row_of"][t] == r)[0][0]) for t, r in zip(toks, rows)]
    assert slots == g["route_slots"]
    assert d["counts"].tolist() == g["counts"]
    assert d["offsets"].tolist() == g["offsets"]
    assert d["token_of_row"].tolist() == g["token_of_row"]
    assert d["row_of"].tolist() == g["row_of"]
    c = g["capacity_2"]
    d2 = O.dispatch(idx, 4, 2)
    assert d2["counts"].tolist() == g["counts"]
    assert d2["kept"].tolist() == c["kept"]
    assert d2["offsets"].tolist() == c["offsets"]
    assert d2["row_of"].tolist() == c["row_of"]
    assert d2["token_of_row"].tolist() == c["token_of_row"]
    assert d2["dropped"] == c["dropped"]


@pytest.mark.parametrize("cap", [None, 1, 3, 7])
def test_dispatch_invariants(cap):
    rng = np.random.default_rng(13)
    T, E, k = 37, 9, 3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    d = O.dispatch(idx, E, cap)
    assert d["counts"].sum() == T * k
    # counts by an independent route: bincount
    np.testing.assert_array_equal(d["counts"], np.bincount(idx.ravel(), minlength=E))
    A = int(d["offsets"][-1])
    kept_rows = d["row_of"][d["row_of"] >= 0]
    assert sorted(kept_rows.tolist()) == list(range(A))          # bijection onto [0, A)
    for (t, j), r in np.ndenumerate(d["row_of"]):
        if r >= 0:
            assert d["token_of_row"][r] == t
            assert d["offsets"][idx[t, j]] <= r < d["offsets"][idx[t, j] + 1]
    for e in range(E):
        seg = d["token_of_row"][d["offsets"][e]:d["offsets"][e + 1]]
        assert (np.diff(seg) > 0).all()                            # ascending tokens
        allt = sorted(t for t in range(T) if e in idx[t])
        n = len(allt) if cap is None else min(cap, len(allt))
        assert seg.tolist() == allt[:n]                           # first C by token order kept
    assert d["dropped"] == T * k - A


def test_capacity_every_token_on_one_expert():
    T, E, C = 50, 4, 12
    idx = np.zeros((T, 1), dtype=np.int64)
    d = O.dispatch(idx, E, C)
    assert d["token_of_row"].tolist() == list(range(C))
    assert (d["row_of"][:C, 0] == np.arange(C)).all() and (d["row_of"][C:, 0] == -1).all()
    assert d["dropped"] == T - C


def test_capacity_formula():
    for c in gold("capacity_examples.json")["cases"]:
        assert O.capacity(c["capacity_factor"], c["num_tokens"], c["top_k"], c["num_experts"]) == c["capacity"]
    assert O.capacity(0.0, 10, 1, 2) is None


# --------------------------------------------------------------------------
# experts
# --------------------------------------------------------------------------
def test_parameter_counts():
    g = gold("parameter_counts.json")
    D, F, E, k = g["d_model"], g["d_ff"], g["num_experts"], g["top_k"]
    assert O.num_parameters_swiglu(D, F) == g["per_expert"]
    assert E * O.num_parameters_swiglu(D, F) == g["all_experts"]
    assert D * E == g["router"]
    assert D * E + k * O.num_parameters_swiglu(D, F) == g["active_per_token"]
    assert O.num_parameters_swiglu(D, g["dense_ff"]) == g["dense_swiglu"]
    # and the generated Tiny workload has exactly these shapes
    w13, w2 = W.make_expert(W.TINY, 0)
    assert w13.size + w2.size == g["per_expert"]


def test_activation_closed_forms():
    assert O.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(O.silu(np.array([1.0])), [1.0 / (1.0 + math.exp(-1.0))], rtol=1e-15)
    # Phi(1) = 0.8413447460685429 (standard normal CDF); gelu(1) = Phi(1)
    np.testing.assert_allclose(O.gelu(np.array([1.0])), [0.8413447460685429], rtol=1e-14)
    np.testing.assert_allclose(O.gelu(np.array([-1.0])), [-(1 - 0.8413447460685429)], rtol=1e-13)
    z = np.linspace(-8, 8, 101)
    tz = torch.from_numpy(z)
    np.testing.assert_allclose(O.gelu(z), torch.nn.functional.gelu(tz).numpy(), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(O.silu(z), torch.nn.functional.silu(tz).numpy(), rtol=1e-13, atol=1e-300)


def test_swiglu_expert_matches_torch_module():
    rng = np.random.default_rng(14)
    D, F = 24, 40
    x = rng.standard_normal((7, D))
    g, u, d = (rng.standard_normal(s) * 0.1 for s in [(F, D), (F, D), (D, F)])
    lin = lambda w: torch.nn.Linear(w.shape[1], w.shape[0], bias=False).double()
    G, U, Dn = lin(g), lin(u), lin(d)
    with torch.no_grad():
        G.weight.copy_(torch.from_numpy(g)); U.weight.copy_(torch.from_numpy(u)); Dn.weight.copy_(torch.from_numpy(d))
        tx = torch.from_numpy(x)
        ref = Dn(torch.nn.functional.silu(G(tx)) * U(tx)).numpy()
    np.testing.assert_allclose(O.swiglu_expert(x, g, u, d), ref, rtol=1e-12, atol=1e-15)
    w13 = np.concatenate([g, u])
    np.testing.assert_allclose(O.expert_apply(x, w13, d, O.SWIGLU, F), ref, rtol=1e-12, atol=1e-15)


def test_gelu_expert_matches_torch():
    rng = np.random.default_rng(15)
    D, F = 16, 20
    x = rng.standard_normal((5, D))
    wi, wo = rng.standard_normal((F, D)), rng.standard_normal((D, F)) * 0.1
    tx = torch.from_numpy(x)
    ref = (torch.nn.functional.gelu(tx @ torch.from_numpy(wi).T) @ torch.from_numpy(wo).T).numpy()
    np.testing.assert_allclose(O.expert_apply(x, wi, wo, O.GELU, F), ref, rtol=1e-12, atol=1e-15)


def test_shared_concatenation_equals_sum():
    """S shared experts summed == one expert of width S*F_s on the packed layout."""
    cfg = W.MoEConfig("t", 9, 16, 2, 1, 8, num_shared=3, d_ff_shared=12, act_dtype=W.F32, router_dtype=W.F32)
    shared = [W.make_shared_expert(cfg, i) for i in range(3)]
    ws13, ws2 = W.pack_shared(cfg, shared)
    x = W.make_tokens(cfg)
    ys = O.shared_experts(x, shared)
    SF = 3 * 12
    one = O.swiglu_expert(x, ws13[:SF], ws13[SF:], ws2)
    np.testing.assert_allclose(ys, one, rtol=1e-12, atol=1e-15)


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------
def _rand_experts(rng, E, D, F):
    return [(rng.standard_normal((2 * F, D)) * 0.3, rng.standard_normal((D, F)) * 0.3) for _ in range(E)]


def test_combine_worked_example():
    g = gold("combine_worked_example.json")
    rng = np.random.default_rng(16)
    T, D, F, E = 4, 6, 5, 4
    x = rng.standard_normal((T, D))
    ex = _rand_experts(rng, E, D, F)
    idx = np.array(g["topk_indices"])
    w = np.full(idx.shape, 0.5)
    w[g["token"]] = g["token0_weights"]
    d = O.dispatch(idx, E, None)
    Y = O.expert_outputs(x, d, lambda e: ex[e], O.SWIGLU, F, E)
    y = O.combine(Y, d, w, T)
    e2 = O.expert_apply(x[:1], *ex[2], O.SWIGLU, F)[0]
    e0 = O.expert_apply(x[:1], *ex[0], O.SWIGLU, F)[0]
    np.testing.assert_allclose(y[0], 0.75 * e2 + 0.25 * e0, rtol=1e-13, atol=1e-15)


def test_combine_accumulates_identical_experts():
    """Identical experts + renormalised weights give y = E(x) for any routing
    (an assigning combine would give only the last route's share)."""
    rng = np.random.default_rng(17)
    T, D, F, E, k = 20, 8, 6, 5, 2
    x = rng.standard_normal((T, D))
    one = _rand_experts(rng, 1, D, F)[0]
    s = rng.standard_normal((T, E))
    idx = O.topk(O.selection_key(s, O.SOFTMAX_TOPK, None), k)
    w = O.gate_weights(s, idx, O.SOFTMAX_TOPK, 1)
    d = O.dispatch(idx, E, None)
    Y = O.expert_outputs(x, d, lambda e: one, O.SWIGLU, F, E)
    y = O.combine(Y, d, w, T)
    np.testing.assert_allclose(y, O.expert_apply(x, *one, O.SWIGLU, F), rtol=1e-12, atol=1e-14)


def test_soft_routing_k_equals_e_is_dense_weighted_sum():
    """k = E routes every token to every expert: the layer is the dense
    weighted sum over all experts of softmax(s)_e * E_e(x) (soft routing)."""
    rng = np.random.default_rng(18)
    T, D, F, E = 11, 8, 6, 5
    x = rng.standard_normal((T, D))
    wr = rng.standard_normal((E, D))
    ex = _rand_experts(rng, E, D, F)
    cfg = W.MoEConfig("soft", T, D, E, E, F, act_dtype=W.F32, router_dtype=W.F32)
    out = O.forward(cfg, x, wr, None, lambda e: ex[e])
    p = torch.softmax(torch.from_numpy(x @ wr.T), -1).numpy()
    dense = np.zeros((T, D))
    for e in range(E):
        dense += p[:, e:e + 1] * O.expert_apply(x, *ex[e], O.SWIGLU, F)
    np.testing.assert_allclose(out["y"], dense, rtol=1e-12, atol=1e-14)


def test_dropped_assignment_contributes_zero():
    rng = np.random.default_rng(19)
    T, D, F, E = 6, 4, 3, 2
    x = rng.standard_normal((T, D))
    ex = _rand_experts(rng, E, D, F)
    idx = np.zeros((T, 1), dtype=np.int64)
    w = np.ones((T, 1))
    d = O.dispatch(idx, E, 2)
    Y = O.expert_outputs(x, d, lambda e: ex[e], O.SWIGLU, F, E)
    y = O.combine(Y, d, w, T)
    np.testing.assert_allclose(y[:2], O.expert_apply(x[:2], *ex[0], O.SWIGLU, F), rtol=1e-13)
    assert (y[2:] == 0).all()


# --------------------------------------------------------------------------
# load statistics
# --------------------------------------------------------------------------
def test_assignment_example_9_4_2_1():
    g = gold("load_examples.json")["assignment_example"]
    c = np.array(g["counts"])
    st = O.load_stats(c, np.full((4, 4), 0.25), 4, 0.01)
    assert c.sum() == g["total"] and c.sum() / 4 == g["ideal_mean"]
    assert st["imbalance"] == pytest.approx(g["imbalance_e0"], rel=1e-15)
    np.testing.assert_allclose(st["f"].sum(), 1.0)


def test_importance_vs_load_cases():
    g = gold("load_examples.json")["importance_vs_load"]
    for case in ("case_A", "case_B"):
        c = g[case]
        probs = np.array(c["probabilities"])
        s = np.log(probs)
        idx = O.topk(O.selection_key(s, O.SOFTMAX_TOPK, None), 1)
        assert idx.tolist() == c["topk_indices"]
        counts = O.expert_counts(idx, 2)
        st = O.load_stats(counts, O.importance_probs(s, O.SOFTMAX_TOPK), 1, alpha=1.0)
        np.testing.assert_allclose(st["P"], c["importance"], rtol=1e-14)
        np.testing.assert_allclose(st["f"], c["load"], rtol=1e-15)
        assert st["aux_loss"] == pytest.approx(c["loss_over_alpha"], rel=1e-14)


@pytest.mark.parametrize("E,k", [(4, 2), (8, 1), (64, 6)])
def test_uniform_routing_loss_equals_alpha(E, k):
    alpha = 0.01
    T = E * 3
    idx = np.array([[(t + j) % E for j in range(k)] for t in range(T)])   # every expert k*3 times
    counts = O.expert_counts(idx, E)
    assert (counts == counts[0]).all()
    probs = np.full((T, E), 1.0 / E)
    st = O.load_stats(counts, probs, k, alpha)
    assert st["aux_loss"] == pytest.approx(alpha, rel=1e-14)
    assert st["imbalance"] == pytest.approx(1.0, rel=1e-15)


def test_sigmoid_importance_sums_to_one():
    rng = np.random.default_rng(20)
    s = rng.standard_normal((30, 16))
    P = O.importance_probs(s, O.SIGMOID_BIAS)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=1e-14)
    a = 1 / (1 + np.exp(-s))
    np.testing.assert_allclose(P * a.sum(-1, keepdims=True), a, rtol=1e-14)


# --------------------------------------------------------------------------
# whole layer against a token-by-token evaluation (no dispatch, no permutation)
# --------------------------------------------------------------------------
def _per_token_reference(cfg, inp, out):
    X = O.widen(inp.x)
    y = np.zeros_like(X)
    for t in range(cfg.num_tokens):
        for j in range(cfg.top_k):
            if out["row_of"][t, j] < 0:
                continue
            e = int(out["idx"][t, j])
            y[t] += out["w"][t, j] * O.expert_apply(X[t:t + 1], inp.w13[e], inp.w2[e], cfg.activation, cfg.d_ff)[0]
        for g, u, d in inp.shared:
            y[t] += O.swiglu_expert(X[t:t + 1], g, u, d)[0]
    return y


@pytest.mark.parametrize("cfg", [
    W.TINY,
    W.TINY.replace(name="tiny_cap", capacity_factor=0.75),
    W.MoEConfig("tiny_shared_sigmoid", 40, 32, 8, 3, 24, num_shared=2, d_ff_shared=16,
                scoring=W.SIGMOID_BIAS, act_dtype=W.BF16, router_dtype=W.BF16, zipf_s=1.0),
    W.MoEConfig("tiny_gelu_switch", 48, 16, 6, 1, 20, scoring=W.SOFTMAX_TOPK, renormalize=0,
                activation=W.GELU, act_dtype=W.BF16, router_dtype=W.F32, capacity_factor=1.0),
    W.MoEConfig("tiny_topk_softmax", 32, 16, 8, 2, 12, scoring=W.TOPK_SOFTMAX),
], ids=lambda c: c.name)
def test_forward_matches_per_token_evaluation(cfg):
    inp = W.make_inputs(cfg)
    out = O.forward(cfg, inp.x, inp.w_router, inp.sel_bias, lambda e: (inp.w13[e], inp.w2[e]), inp.shared)
    assert out["counts"].sum() == cfg.num_tokens * cfg.top_k
    ref = _per_token_reference(cfg, inp, out)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-14)
    if cfg.capacity_factor <= 0:
        assert out["dropped"] == 0 and (out["row_of"] >= 0).all()
    else:
        assert out["dropped"] == int((out["row_of"] < 0).sum())


def test_tiny_workload_routes_every_assignment():
    cfg = W.TINY
    inp = W.make_inputs(cfg)
    out = O.forward(cfg, inp.x, inp.w_router, None, lambda e: (inp.w13[e], inp.w2[e]))
    assert out["counts"].sum() == 128                      # N * K = 64 * 2
    np.testing.assert_allclose(out["w"].sum(1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(out["P"].sum(), 1.0, rtol=1e-14)
    assert out["aux_loss"] > 0


# --------------------------------------------------------------------------
# expert-parallel layouts
# --------------------------------------------------------------------------
def _ep_exchange(rank_idx, num_experts, num_ranks):
    """CPU simulation of the dispatch all-to-all on top of the oracle's
    per-rank dispatch: returns, per destination rank, the received buffer as
    (source rank, token) pairs and the oracle's receive layout."""
    per = num_experts // num_ranks
    sends = []
    for idx in rank_idx:
        d = O.dispatch(np.asarray(idx), num_experts, None)
        lay = O.ep_send_layout(d["kept"], num_ranks)
        sends.append((d, lay))
    out = []
    for dst in range(num_ranks):
        received = []
        recv_counts = np.zeros((num_ranks, per), dtype=np.int64)
        for src, (d, lay) in enumerate(sends):
            lo, hi = lay["send_offsets"][dst], lay["send_offsets"][dst + 1]
            received += [(src, int(t)) for t in d["token_of_row"][lo:hi]]
            recv_counts[src] = d["kept"][dst * per:(dst + 1) * per]
        out.append((received, recv_counts, O.ep_recv_layout(recv_counts)))
    return sends, out


def test_ep_all_to_all_figure():
    g = gold("ep_all_to_all_figure.json")
    E, R = g["num_experts"], g["num_ranks"]
    sends, recvs = _ep_exchange([rk["topk_indices"] for rk in g["ranks"]], E, R)
    for rk, (d, lay), want in zip(g["ranks"], sends, g["send"]):
        np.testing.assert_array_equal(lay["send_counts"], want["send_counts"])
        np.testing.assert_array_equal(lay["send_offsets"], want["send_offsets"])
        assert [rk["tokens"][t] for t in d["token_of_row"]] == want["rows_in_order"]
    for (received, recv_counts, lay), want in zip(recvs, g["recv"]):
        names = [g["ranks"][s]["tokens"][t] for s, t in received]
        assert names == want["received"]
        np.testing.assert_array_equal(recv_counts, want["recv_counts"])
        np.testing.assert_array_equal(lay["local_offsets"], want["local_offsets"])
        np.testing.assert_array_equal(lay["gather"], want["gather"])
        assert [names[j] for j in lay["gather"]] == want["expert_rows"]


@pytest.mark.parametrize("R,E,k", [(2, 8, 2), (4, 16, 3), (8, 32, 1)])
def test_ep_layouts_brute_force(R, E, k):
    """After the simulated exchange, the rows the local FFN reads for each
    local expert are exactly the (source rank, token) assignments routed to
    that expert, sources in rank order and tokens ascending inside a source
    (found by scanning every rank's routing); every received row is read once."""
    rng = np.random.default_rng(R * 100 + E)
    rank_idx = []
    for r in range(R):
        T = int(rng.integers(0, 40))
        rank_idx.append(np.array([rng.choice(E, size=k, replace=False) for _ in range(T)],
                                 dtype=np.int64).reshape(T, k))
    sends, recvs = _ep_exchange(rank_idx, E, R)
    per = E // R
    for (d, lay), idx in zip(sends, rank_idx):
        assert lay["send_offsets"][-1] == idx.size        # dropless: every assignment is sent once
    for dst, (received, recv_counts, lay) in enumerate(recvs):
        gather = lay["gather"]
        assert sorted(gather.tolist()) == list(range(len(received)))
        for e in range(per):
            want = [(src, t) for src in range(R) for t in range(len(rank_idx[src]))
                    for j in range(k) if rank_idx[src][t, j] == dst * per + e]
            lo, hi = lay["local_offsets"][e], lay["local_offsets"][e + 1]
            assert [received[gather[i]] for i in range(lo, hi)] == want


def test_ep_dispatch_payload_worked_example():
    """"别只比较 Top-k" page, payload example: 8 tokens x Top-2 x hidden 4096 in
    bf16 is a 131,072-byte dispatch when every assignment leaves the rank."""
    rng = np.random.default_rng(7)
    E, R, T, k, D = 16, 2, 8, 2, 4096
    idx = np.array([rng.choice(np.arange(8, 16), size=k, replace=False) for _ in range(T)])   # all on rank 1
    d = O.dispatch(idx, E, None)
    lay = O.ep_send_layout(d["kept"], R)
    remote = int(lay["send_counts"][1])
    assert lay["send_counts"][0] == 0
    assert remote * D * 2 == 131072


# --------------------------------------------------------------------------
# expert-choice routing
# --------------------------------------------------------------------------
def test_expert_choice_capacity_is_the_buffer_formula():
    """C is the "Top-k 路由" 容量因子 buffer (the same worked cases as the
    token-choice capacity), CF = 1 when none is given, at most T."""
    for c in gold("capacity_examples.json")["cases"]:
        want = min(c["capacity"], c["num_tokens"])
        assert O.expert_choice_capacity(c["capacity_factor"], c["num_tokens"], c["top_k"], c["num_experts"]) == want
    assert O.expert_choice_capacity(0.0, 4096, 6, 64) == 384          # T k / E
    assert O.expert_choice_capacity(0.0, 3, 8, 2) == 3                # at most T


@pytest.mark.parametrize("seed", range(6))
def test_expert_choice_selection_brute_force(seed):
    """Every expert's chosen set is the C-subset of tokens with the largest
    total probability, equal totals going to the lexicographically smallest
    token set (enumerated over all subsets), with ties built in."""
    rng = np.random.default_rng(40 + seed)
    T, E, D = int(rng.integers(3, 8)), int(rng.integers(1, 5)), 6
    x = rng.standard_normal((T, D))
    wr = rng.standard_normal((E, D))
    if seed % 2 == 0 and T > 2:
        x[1] = x[0]                                                 # equal probabilities of tokens 0 and 1
    C = int(rng.integers(1, T + 1))
    r = O.expert_choice_route(x, wr, C)
    p = O.softmax(x @ wr.T)
    for e in range(E):
        best = None
        for sub in itertools.combinations(range(T), C):
            v = sum(p[t, e] for t in sub)
            if best is None or v > best[0] + 1e-15:
                best = (v, sub)
        assert tuple(sorted(r["chosen"][e])) == best[1]
        rows = r["token_of_row"][e * C:(e + 1) * C]
        assert list(rows) == sorted(rows)
        np.testing.assert_array_equal(r["row_w"][e * C:(e + 1) * C], p[rows, e])
    np.testing.assert_array_equal(r["offsets"], np.arange(E + 1) * C)


def test_expert_choice_single_expert_takes_the_first_tokens():
    """One expert: every probability is 1, all tied, so the expert takes
    tokens 0 .. C-1 with gate 1."""
    rng = np.random.default_rng(50)
    x = rng.standard_normal((9, 4))
    r = O.expert_choice_route(x, rng.standard_normal((1, 4)), 4)
    np.testing.assert_array_equal(r["token_of_row"], [0, 1, 2, 3])
    np.testing.assert_array_equal(r["row_w"], np.ones(4))


def test_expert_choice_every_token_is_dense_soft_routing():
    """C = T: every expert takes every token, so the layer is the dense
    probability-weighted sum over all experts (the soft-routing formula)."""
    rng = np.random.default_rng(51)
    T, D, F, E = 7, 8, 6, 4
    x = rng.standard_normal((T, D))
    wr = rng.standard_normal((E, D))
    ex = _rand_experts(rng, E, D, F)
    cfg = W.MoEConfig("ec_dense", T, D, E, E, F, act_dtype=W.F32, router_dtype=W.F32)
    out = O.expert_choice_forward(cfg, x, wr, lambda e: ex[e])
    assert out["capacity"] == T and out["unselected"] == 0
    p = torch.softmax(torch.from_numpy(x @ wr.T), -1).numpy()
    dense = np.zeros((T, D))
    for e in range(E):
        dense += p[:, e:e + 1] * O.expert_apply(x, *ex[e], O.SWIGLU, F)
    np.testing.assert_allclose(out["y"], dense, rtol=1e-12, atol=1e-14)


def test_expert_choice_unchosen_token_gets_only_the_shared_path():
    """Two experts that both prefer tokens 0 and 1 (C = 1): token 2 is chosen
    by neither, so its routed output is zero and only the shared expert
    reaches it; the chosen tokens get p * E(x)."""
    rng = np.random.default_rng(52)
    D, F = 4, 3
    wr = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0]])
    x = np.array([[4.0, 0, 0, 0], [0, 4.0, 0, 0], [0.1, 0.1, 0, 0]])
    ex = _rand_experts(rng, 2, D, F)
    sh = [tuple(rng.standard_normal(s) for s in ((F, D), (F, D), (D, F)))]
    cfg = W.MoEConfig("ec_unchosen", 3, D, 2, 1, F, act_dtype=W.F32, router_dtype=W.F32, capacity_factor=0.5)
    out = O.expert_choice_forward(cfg, x, wr, lambda e: ex[e], sh)
    assert out["capacity"] == 1 and out["unselected"] == 1
    np.testing.assert_array_equal(out["route"]["token_of_row"], [0, 1])
    ys = O.shared_experts(x, sh)
    np.testing.assert_allclose(out["y"][2], ys[2], rtol=1e-13)
    p = O.softmax(x @ wr.T)
    for t, e in ((0, 0), (1, 1)):
        want = p[t, e] * O.expert_apply(x[t:t + 1], *ex[e], O.SWIGLU, F)[0] + ys[t]
        np.testing.assert_allclose(out["y"][t], want, rtol=1e-12)


# --------------------------------------------------------------------------
# backward pass
# --------------------------------------------------------------------------
def _bw_case(name, T, D, E, k, F, **kw):
    return W.MoEConfig(name, T, D, E, k, F, act_dtype=W.F32, router_dtype=W.F32, **kw)


BW_CASES = [
    _bw_case("bw_switch_like", 24, 12, 6, 1, 10, scoring=O.SOFTMAX_TOPK, renormalize=0, activation=O.GELU,
             capacity_factor=1.0),
    _bw_case("bw_softmax_renorm_shared", 20, 10, 5, 2, 8, scoring=O.SOFTMAX_TOPK, renormalize=1, num_shared=2,
             d_ff_shared=6),
    _bw_case("bw_topk_softmax", 18, 8, 4, 2, 7, scoring=O.TOPK_SOFTMAX),
    _bw_case("bw_sigmoid_bias", 22, 9, 8, 3, 6, scoring=O.SIGMOID_BIAS, renormalize=1, num_shared=1, d_ff_shared=5),
    _bw_case("bw_sigmoid_raw_capacity", 16, 8, 4, 2, 6, scoring=O.SIGMOID_BIAS, renormalize=0, capacity_factor=0.75),
]


def _bw_inputs(cfg, seed):
    rng = np.random.default_rng(seed)
    T, D, E, F = cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.d_ff
    x = rng.standard_normal((T, D))
    wr = rng.standard_normal((E, D)) * 0.5
    b = rng.uniform(-0.1, 0.1, E) if cfg.scoring == O.SIGMOID_BIAS else None
    ex = [(rng.standard_normal((cfg.n_mat * F, D)) * 0.3, rng.standard_normal((D, F)) * 0.3) for _ in range(E)]
    sh = [tuple(rng.standard_normal(s) * 0.3 for s in ((cfg.d_ff_shared, D), (cfg.d_ff_shared, D),
                                                        (D, cfg.d_ff_shared))) for _ in range(cfg.num_shared)]
    dy = rng.standard_normal((T, D))
    return x, wr, b, ex, sh, dy


def _torch_grads(cfg, x, wr, ex, sh, dy, alpha, fw):
    """The same loss written with torch float64 operations, the routing
    decisions (indices, kept rows, counts) taken from the oracle's forward."""
    import torch.nn.functional as Fn
    tt = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    X, Wr = tt(x), tt(wr)
    W13 = [tt(a) for a, _ in ex]
    W2 = [tt(b) for _, b in ex]
    SH = [tuple(tt(m) for m in trip) for trip in sh]
    T, E, k, F = cfg.num_tokens, cfg.num_experts, cfg.top_k, cfg.d_ff
    s = X @ Wr.T
    idx = torch.tensor(fw["idx"])
    if cfg.scoring == O.SOFTMAX_TOPK:
        g = torch.softmax(s, -1).gather(1, idx)
        if cfg.renormalize:
            g = g / g.sum(1, keepdim=True)
    elif cfg.scoring == O.TOPK_SOFTMAX:
        g = torch.softmax(s.gather(1, idx), -1)
    else:
        a = torch.sigmoid(s).gather(1, idx)
        g = a / a.sum(1, keepdim=True) if cfg.renormalize else a
    y = torch.zeros((T, cfg.d_model), dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            if fw["row_of"][t, j] < 0:
                continue
            e = int(fw["idx"][t, j])
            xt = X[t:t + 1]
            if cfg.activation == O.SWIGLU:
                h = Fn.silu(xt @ W13[e][:F].T) * (xt @ W13[e][F:].T)
            else:
                h = Fn.gelu(xt @ W13[e].T)
            y[t] = y[t] + g[t, j] * (h @ W2[e].T)[0]
    for Wg, Wu, Wd in SH:
        y = y + (Fn.silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T
    if cfg.scoring == O.SIGMOID_BIAS:
        a = torch.sigmoid(s)
        ph = a / a.sum(1, keepdim=True)
    else:
        ph = torch.softmax(s, -1)
    f = torch.tensor(fw["counts"], dtype=torch.float64) / (T * k)
    loss = (torch.tensor(dy) * y).sum() + alpha * E * (f * ph.mean(0)).sum()
    loss.backward()
    return X.grad.numpy(), Wr.grad.numpy(), [w.grad for w in W13], [w.grad for w in W2], \
        [tuple(m.grad for m in trip) for trip in SH]


@pytest.mark.parametrize("cfg", BW_CASES, ids=lambda c: c.name)
def test_backward_matches_torch_autograd(cfg):
    """Every gradient of the oracle's backward against CPU torch autograd of
    the same loss (float64), the routing held fixed."""
    x, wr, b, ex, sh, dy = _bw_inputs(cfg, 7)
    alpha = 0.05
    g = O.backward(cfg, x, wr, b, lambda e: ex[e], sh, dy, alpha=alpha)
    gx, gwr, g13, g2, gsh = _torch_grads(cfg, x, wr, ex, sh, dy, alpha, g["forward"])
    np.testing.assert_allclose(g["dx"], gx, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dw_router"], gwr, rtol=1e-10, atol=1e-12)
    for e in range(cfg.num_experts):
        want13 = g13[e].numpy() if g13[e] is not None else np.zeros_like(ex[e][0])
        want2 = g2[e].numpy() if g2[e] is not None else np.zeros_like(ex[e][1])
        np.testing.assert_allclose(g["dw13"].get(e, np.zeros_like(ex[e][0])), want13, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(g["dw2"].get(e, np.zeros_like(ex[e][1])), want2, rtol=1e-10, atol=1e-12)
    for got, want in zip(g["dshared"], gsh):
        for a, b_ in zip(got, want):
            np.testing.assert_allclose(a, b_.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_finite_differences():
    """Central differences of the scalar loss <dy, y> + L_aux, computed with
    the oracle's forward, along random coordinates of x, the router weight and
    one expert's matrices (steps small enough that no routing decision moves)."""
    cfg = BW_CASES[1]
    x, wr, b, ex, sh, dy = _bw_inputs(cfg, 8)
    alpha = 0.05
    g = O.backward(cfg, x, wr, b, lambda e: ex[e], sh, dy, alpha=alpha)

    def loss(x_, wr_, ex_):
        fw = O.forward(cfg, x_, wr_, b, lambda e: ex_[e], sh, alpha=alpha)
        return float((dy * fw["y"]).sum() + fw["aux_loss"]), fw["idx"]

    base_idx = g["forward"]["idx"]
    rng = np.random.default_rng(3)
    h = 1e-6
    e0 = int(base_idx[0, 0])
    checks = [("x", tuple(rng.integers(0, s) for s in x.shape)), ("wr", tuple(rng.integers(0, s) for s in wr.shape)),
              ("w13", tuple(rng.integers(0, s) for s in ex[e0][0].shape)),
              ("w2", tuple(rng.integers(0, s) for s in ex[e0][1].shape))]
    for what, pos in checks:
        vals = []
        for sgn in (1, -1):
            x_, wr_, ex_ = x.copy(), wr.copy(), [(a.copy(), c.copy()) for a, c in ex]
            tgt = {"x": x_, "wr": wr_, "w13": ex_[e0][0], "w2": ex_[e0][1]}[what]
            tgt[pos] += sgn * h
            v, idx = loss(x_, wr_, ex_)
            assert np.array_equal(idx, base_idx)
            vals.append(v)
        fd = (vals[0] - vals[1]) / (2 * h)
        an = {"x": g["dx"], "wr": g["dw_router"], "w13": g["dw13"][e0], "w2": g["dw2"][e0]}[what][pos]
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (what, pos, fd, an)
