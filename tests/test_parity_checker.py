"""The GPU parity checker itself, on the CPU: synthetic "GPU" results built
from the oracle with one near-tied token's selection exchanged must pass, and
results with a plausible kernel mistake must fail.

Experts 2 and 3 get identical router rows, so their logits tie exactly for
every token (the oracle takes expert 2, the lower index); their expert weights
differ, so the choice changes the output.  With capacity, the exchanged
token's assignment can push another token of expert 3 over capacity, which
only a re-run of the dispatch on the GPU's choice (not a patch of the counts)
accounts for.
"""
import numpy as np
import pytest

import workloads as W
from oracle import moe_oracle as O
from parity import check_layer, oracle_forward, route_differences, selection_error

BASE = W.MoEConfig("checker", 48, 16, 6, 2, 12, act_dtype=W.F32, router_dtype=W.F32)


def _inputs(cfg):
    inp = W.make_inputs(cfg)
    inp.w_router[3] = inp.w_router[2]
    return inp


def _gpu_like(cfg, inp, ref, idx):
    """What a correct GPU layer would return for the selection `idx`: the
    oracle's own steps run on it, rounded to the GPU's output types."""
    s = ref["logits"]
    w = O.gate_weights(s, idx, cfg.scoring, cfg.renormalize)
    disp = O.dispatch(idx, cfg.num_experts, O.capacity(cfg.capacity_factor, cfg.num_tokens, cfg.top_k,
                                                      cfg.num_experts))
    Y = O.expert_outputs(inp.x, disp, lambda e: (inp.w13[e], inp.w2[e]), cfg.activation, cfg.d_ff, cfg.num_experts)
    y = O.combine(Y, disp, w, cfg.num_tokens, ref["y_shared"])
    st = O.load_stats(disp["counts"], ref["probs"], cfg.top_k, cfg.alpha, disp["kept"])
    stats = np.concatenate([st["f"], st["P"], [st["aux_loss"], st["imbalance"]]]).astype(np.float32)
    return dict(y=y.astype(np.float32), idx=idx.astype(np.int32), w=w.astype(np.float32),
                counts=disp["counts"].astype(np.int32), stats=stats, dropped=disp["dropped"])


def _tied_boundary_tokens(ref, k):
    """The first half of the tokens whose k-th choice is expert 2 with expert 3
    right behind (tied): exchanging only some of them moves the counts of
    experts 2 and 3 towards each other, which changes who is kept when one
    of them is over capacity."""
    toks = [t for t in range(ref["idx"].shape[0]) if ref["idx"][t, k - 1] == 2 and
            O.topk(ref["key"][t:t + 1], k + 1)[0, k] == 3]
    return toks[:(len(toks) + 1) // 2]


@pytest.mark.parametrize("cap", [0.0, 1.0])
def test_exchanged_near_tie_passes(cap):
    cfg = BASE.replace(capacity_factor=cap)
    inp = _inputs(cfg)
    ref = oracle_forward(cfg, inp)
    toks = _tied_boundary_tokens(ref, cfg.top_k)
    assert toks, "the construction must give a tied boundary"
    idx = ref["idx"].copy()
    idx[toks, cfg.top_k - 1] = 3
    got = _gpu_like(cfg, inp, ref, idx)
    if cap > 0:
        # the exchange must change who is kept somewhere, or the case tests nothing
        base = O.dispatch(ref["idx"], cfg.num_experts, O.capacity(cap, cfg.num_tokens, cfg.top_k, cfg.num_experts))
        assert not np.array_equal(got["counts"], base["counts"].astype(np.int32))
    diff, err = check_layer(cfg, inp, ref, got)
    assert sorted(diff.tolist()) == sorted(toks)
    assert err <= 1e-6


def test_exchange_at_a_clear_gap_fails():
    cfg = BASE
    inp = _inputs(cfg)
    ref = oracle_forward(cfg, inp)
    # a token whose k-th and (k+1)-th keys are far apart
    srt = -np.sort(-ref["key"], axis=1)
    t = int(np.argmax((srt[:, 1] - srt[:, 2]) / srt[:, 1]))
    idx = ref["idx"].copy()
    idx[t, 1] = O.topk(ref["key"][t:t + 1], 3)[0, 2]
    got = _gpu_like(cfg, inp, ref, idx)
    with pytest.raises(AssertionError, match="left out ranks above"):
        check_layer(cfg, inp, ref, got)


def test_slot_swap_at_a_clear_gap_fails():
    cfg = BASE
    inp = _inputs(cfg)
    ref = oracle_forward(cfg, inp)
    srt = -np.sort(-ref["key"], axis=1)
    t = int(np.argmax((srt[:, 0] - srt[:, 1]) / srt[:, 0]))
    idx = ref["idx"].copy()
    idx[t] = idx[t, ::-1]
    got = _gpu_like(cfg, inp, ref, idx)
    with pytest.raises(AssertionError, match="out of order"):
        check_layer(cfg, inp, ref, got)


def test_output_of_the_oracle_choice_at_an_exchanged_token_fails():
    """A GPU that reports the exchanged selection but computed the output of
    the other one (a combine reading the wrong rows) is caught, capacity
    configuration included."""
    cfg = BASE.replace(capacity_factor=1.0)
    inp = _inputs(cfg)
    ref = oracle_forward(cfg, inp)
    toks = _tied_boundary_tokens(ref, cfg.top_k)
    idx = ref["idx"].copy()
    idx[toks, cfg.top_k - 1] = 3
    got = _gpu_like(cfg, inp, ref, idx)
    got["y"] = ref["y"].astype(np.float32)
    with pytest.raises(AssertionError, match="max relative error"):
        check_layer(cfg, inp, ref, got)


def test_counts_patched_instead_of_rerun_fail():
    """With capacity, counts moved by the exchanged token alone are not what the
    re-run dispatch gives when the exchange changes who is kept: the drops
    differ too."""
    cfg = BASE.replace(capacity_factor=1.0)
    inp = _inputs(cfg)
    ref = oracle_forward(cfg, inp)
    toks = _tied_boundary_tokens(ref, cfg.top_k)
    idx = ref["idx"].copy()
    idx[toks, cfg.top_k - 1] = 3
    got = _gpu_like(cfg, inp, ref, idx)
    assert got["dropped"] != ref["dropped"], "the exchange must change the number of drops"
    got["dropped"] = ref["dropped"]
    with pytest.raises(AssertionError, match="dropped"):
        check_layer(cfg, inp, ref, got)


def test_wrong_weight_at_an_exchanged_token_fails():
    cfg = BASE
    inp = _inputs(cfg)
    ref = oracle_forward(cfg, inp)
    toks = _tied_boundary_tokens(ref, cfg.top_k)
    idx = ref["idx"].copy()
    idx[toks, cfg.top_k - 1] = 3
    got = _gpu_like(cfg, inp, ref, idx)
    got["w"][toks[0]] *= np.float32(1.001)
    with pytest.raises(AssertionError):
        check_layer(cfg, inp, ref, got)


def test_selection_error_rules():
    key = np.array([0.50, 0.30, 0.30 * (1 - 5e-7), 0.10, 0.30 * (1 - 5e-6)])
    assert selection_error(key, [0, 1], 2) is None
    assert selection_error(key, [0, 2], 2) is None               # boundary within the band
    assert "left out" in selection_error(key, [0, 4], 2)          # 5e-6 below the k-th: outside
    assert "out of order" in selection_error(key, [1, 0], 2)
    assert "distinct" in selection_error(key, [0, 0], 2)
    assert "distinct" in selection_error(key, [0, 5], 2)
    assert selection_error(key, [1, 2], 2) is not None            # drops the clear winner
    # k = E: every expert is chosen, only the order can be wrong
    assert selection_error(key[:2], [0, 1], 2) is None


def test_route_differences_reports_only_exempt_tokens():
    cfg = BASE
    inp = _inputs(cfg)
    ref = oracle_forward(cfg, inp)
    toks = _tied_boundary_tokens(ref, cfg.top_k)
    idx = ref["idx"].copy()
    assert len(route_differences(cfg, ref, idx, None)) == 0
    idx[toks, cfg.top_k - 1] = 3
    assert sorted(route_differences(cfg, ref, idx, None).tolist()) == sorted(toks)
