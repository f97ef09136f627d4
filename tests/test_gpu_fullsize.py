"""Full-size parity at the benchmark workloads (Switch, Mixtral, DeepSeekMoE,
DeepSeek-V3 shapes), in the launch configuration bench.py times
(moe_layer_forward on the whole batch):

  * expert selection of every token against the float64 oracle (near-tie
    exemption only; at an exempt token the oracle's later steps are re-run
    on the GPU's choice): weights, counts, drops and the load statistics of
    every token, and the full permutation of the oracle's own selection,
    bit-exact;
  * the float32 router logits the selection starts from, against float64:
    the error must sit far inside the margin that triggers the float64
    near-tie refinement;
  * layer outputs of the tokens of the first and last row of every active
    expert (so every expert and every tile class of the grouped GEMM
    launches is covered) plus a seeded random sample, each computed by the
    oracle expert by expert (only the experts the sample uses are widened).

The oracle widens every active expert's weights once (about 0.2 s each at
the DeepSeek-V3 shape), so these tests carry their own time limit.
"""
import numpy as np
import pytest
import torch

import top_routing_dispatch_amd as M
import workloads as W
from oracle import moe_oracle as O
from workloads.torch_io import act_torch_dtype, to_numpy, to_torch, upload_experts

from parity import (W_TOL, check_stats, ec_check_selection, ec_oracle_output, out_tol, refinement_margin, rel_err,
                    rerun_on_choice, route_differences, row_rel_err)

pytestmark = pytest.mark.gpu

SAMPLE = {"switch": 32, "mixtral": 12, "deepseekmoe": 24, "deepseekv3": 8}
DECODE_SAMPLE = 32

_EXPERTS = {}


def _experts(name):
    """Routed expert weights of a full-size workload on the device (and their
    host bytes), generated once per module run; other models are dropped."""
    if name not in _EXPERTS:
        _EXPERTS.clear()
        torch.cuda.empty_cache()
        _EXPERTS[name] = upload_experts(W.CONFIGS[name], "cuda", keep_host=True)
    return _EXPERTS[name]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["switch", "mixtral", "deepseekmoe", "deepseekv3"])
def test_full_size_layer(name):
    print(f"[full-size parity] {name}", flush=True)
    _check_full_weights(W.CONFIGS[name], SAMPLE[name])


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", W.DECODE_TOKENS)
@pytest.mark.parametrize("name", ["deepseekv3", "mixtral"])
def test_decode_full_size(name, T):
    """Decode-sized batches (the first T tokens of the workload) on the
    full-size Mixtral- and DeepSeek-V3-shaped weights, as bench.py times them:
    every routing decision, and the outputs of up to 32 tokens."""
    cfg = W.decode_config(W.CONFIGS[name], T)
    print(f"[decode full-size parity] {cfg.name}", flush=True)
    _check_full_weights(cfg, min(T, DECODE_SAMPLE))


def _check_full_weights(cfg, n_sample):
    T, E, k, D = cfg.num_tokens, cfg.num_experts, cfg.top_k, cfg.d_model
    dev = "cuda"
    inp = W.make_inputs(cfg, with_experts=False)
    w13, w2, host = _experts(W.base_name(cfg))
    weights = dict(w_router=to_torch(inp.w_router, dev), sel_bias=to_torch(inp.sel_bias, dev), w13=w13, w2=w2,
                   ws13=to_torch(inp.ws13, dev), ws2=to_torch(inp.ws2, dev))
    x = to_torch(inp.x, dev)

    # --- the benchmark's call
    y = torch.empty((T, D), dtype=act_torch_dtype(cfg), device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    stats = torch.empty(2 * E + 2, dtype=torch.float32, device=dev)
    dropped = torch.empty(1, dtype=torch.int32, device=dev)
    ws = M.workspace(cfg, M.MOE_OP_LAYER, dev)
    M.moe_layer_forward(cfg, weights, x, y, idx, tw, counts, cfg.alpha, stats, dropped, ws)
    # float32 logits as the route kernel sees them
    wsr = M.workspace(cfg, M.MOE_OP_ROUTE, dev)
    idx2 = torch.empty_like(idx)
    tw2 = torch.empty_like(tw)
    M.moe_route(cfg, x, weights["w_router"], weights["sel_bias"], idx2, tw2, None, wsr)
    torch.cuda.synchronize()
    s32 = wsr[: T * E * 4].view(torch.float32).reshape(T, E).cpu().numpy().astype(np.float64)

    # --- oracle routing of every token (float64)
    ref = O.route(inp.x, inp.w_router, inp.sel_bias, k, cfg.scoring, cfg.renormalize)
    err_s = np.abs(s32 - ref["logits"]).max(axis=1)
    margin = refinement_margin(s32)
    print(f"  float32 logit error max {err_s.max():.3e}; smallest margin/error {np.min(margin / np.maximum(err_s, 1e-30)):.1f}")
    assert (err_s * 16 < margin).all(), "float32 logits too far from exact for the refinement margin"

    gi, gw = to_numpy(idx), to_numpy(tw)
    np.testing.assert_array_equal(gi, to_numpy(idx2))
    diff = route_differences(cfg, ref, gi, inp.sel_bias)
    print(f"  near-tie tokens {len(diff)}")
    # the oracle's steps after the selection, re-run on the GPU's choice at the exempt tokens
    ch = rerun_on_choice(cfg, ref, gi, diff)
    disp = ch["disp"]
    assert rel_err(gw, ch["w"]) <= W_TOL
    np.testing.assert_array_equal(to_numpy(counts), disp["counts"])
    check_stats(cfg, ch["stats"], to_numpy(stats), int(to_numpy(dropped)[0]))

    # --- permutation of the oracle's selection, bit-exact at full size
    cap_c, rows_cap = M.moe_capacity(cfg)
    c2 = torch.empty(E, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_of = torch.empty((T, k), dtype=torch.int32, device=dev)
    tor = torch.empty(rows_cap, dtype=torch.int32, device=dev)
    M.moe_permute(cfg, to_torch(ref["idx"].astype(np.int32), dev), None, c2, off, row_of, tor, None,
                  M.workspace(cfg, M.MOE_OP_PERMUTE, dev))
    torch.cuda.synchronize()
    own = O.dispatch(ref["idx"], E, O.capacity(cfg.capacity_factor, T, k, E))
    A = int(own["offsets"][-1])
    np.testing.assert_array_equal(to_numpy(off), own["offsets"])
    np.testing.assert_array_equal(to_numpy(row_of), own["row_of"])
    np.testing.assert_array_equal(to_numpy(tor)[:A], own["token_of_row"])

    # --- sampled outputs, oracle expert by expert, on the re-run choice
    sample, why = coverage_sample(cfg, disp, n_sample)
    X = O.widen(inp.x[sample])
    y_ref = np.zeros((len(sample), D))
    users = {}
    for i, t in enumerate(sample):
        for j in range(k):
            if disp["row_of"][t, j] >= 0:
                users.setdefault(int(ch["idx"][t, j]), []).append((i, j))
    for e, lst in users.items():
        rows = [i for i, _ in lst]
        out = O.expert_apply(X[rows], host[e][0], host[e][1], cfg.activation, cfg.d_ff)
        for (i, j), o in zip(lst, out):
            y_ref[i] += ch["w"][sample[i], j] * o
    if cfg.num_shared:
        y_ref += O.shared_experts(inp.x[sample], inp.shared)
    active = int((disp["kept"] > 0).sum())
    print(f"  sampled {len(sample)} tokens over {len(users)} of {active} active experts ({why})")
    assert len(users) == active, "every active expert must have a sampled token"
    err = row_rel_err(to_numpy(y)[sample], y_ref)
    print(f"  max rel err {err:.3e}")
    assert err <= out_tol(cfg)


def coverage_sample(cfg, disp, n_extra, seed=1234):
    """Tokens whose outputs are checked: for every expert with kept rows, the
    token of its first and of its last row (the first and last m-tile of
    every group, so every tile class of the grouped GEMM launches is hit:
    deep tiles, shallow weight-streaming groups and the partial tiles at a
    group's end, among them the split last-round tiles), plus `n_extra`
    tokens drawn at random."""
    off, tor = disp["offsets"], disp["token_of_row"]
    must = set()
    for e in range(cfg.num_experts):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            must.add(int(tor[a]))
            must.add(int(tor[b - 1]))
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(cfg.num_tokens), np.fromiter(must, dtype=np.int64, count=len(must)))
    extra = rng.choice(rest, size=min(n_extra, len(rest)), replace=False) if len(rest) else []
    sample = np.sort(np.concatenate([np.fromiter(must, dtype=np.int64, count=len(must)),
                                     np.asarray(extra, dtype=np.int64)]))
    return sample, f"first and last row of every expert: {len(must)} tokens, {len(extra)} random"


@pytest.mark.parametrize("name", sorted(W.EP_CONFIGS))
def test_ep_local_share_full_size(name):
    """One GPU's share of the DeepSeek-V3-shaped layer on 8 ranks, as bench.py
    times it: the receive layout of 65,536 rows for 32 local experts
    (bit-exact against the oracle) and the local grouped FFN over the received
    rows in place, sampled rows against the oracle."""
    ep = W.EP_CONFIGS[name]
    cfg = W.CONFIGS[ep.base]
    El, D, F = ep.local_experts, cfg.d_model, cfg.d_ff
    print(f"[ep local share] {name}", flush=True)
    rc = W.ep_recv_counts(ep)
    total = int(rc.sum())
    xr = W.make_received_rows(ep, total)
    experts = {}
    w13 = torch.empty((El, 2 * F, D), dtype=torch.bfloat16, device="cuda")
    w2 = torch.empty((El, D, F), dtype=torch.bfloat16, device="cuda")
    for e, a, b in W.iter_experts(cfg, experts=range(ep.rank * El, (ep.rank + 1) * El), workers=16):
        w13[e - ep.rank * El].copy_(to_torch(a, "cpu"))
        w2[e - ep.rank * El].copy_(to_torch(b, "cpu"))
        experts[e - ep.rank * El] = (a, b)
    lo = torch.empty(El + 1, dtype=torch.int32, device="cuda")
    g = torch.empty(total, dtype=torch.int32, device="cuda")
    M.moe_ep_recv_layout(to_torch(rc, "cuda"), total, lo, g)
    y = torch.empty((total, D), dtype=torch.bfloat16, device="cuda")
    lcfg = cfg.replace(num_experts=El, num_tokens=total, top_k=1, num_shared=0, d_ff_shared=0)
    ws = M.workspace(lcfg, M.MOE_OP_EXPERT_FFN, "cuda")
    M.moe_expert_ffn(lcfg, El, F, cfg.activation, total, to_torch(xr, "cuda"), g, lo, w13, w2, y, ws)
    torch.cuda.synchronize()
    lay = O.ep_recv_layout(rc)
    np.testing.assert_array_equal(to_numpy(lo), lay["local_offsets"])
    np.testing.assert_array_equal(to_numpy(g), lay["gather"])
    rng = np.random.default_rng(4321)
    sample = np.sort(rng.choice(total, size=16, replace=False))
    got = to_numpy(y)[sample]
    ref = np.zeros((len(sample), D))
    for i, j in enumerate(sample):
        e = int(np.searchsorted(lay["local_offsets"], j, side="right") - 1)
        X = O.widen(xr[lay["gather"][j:j + 1]])
        ref[i] = O.expert_apply(X, experts[e][0], experts[e][1], cfg.activation, F)[0]
    err = row_rel_err(got, ref)
    print(f"  sampled {len(sample)} rows: max rel err {err:.3e}")
    assert err <= out_tol(cfg)


@pytest.mark.parametrize("name", ["deepseekv3_ec", "mixtral_ec", "deepseekmoe_ec"])
def test_expert_choice_full_size(name):
    """Expert-choice routing on the full-size workloads, as bench.py times it:
    every expert's chosen tokens against the float64 oracle (near ties of the
    C-th probability exempt), the gates, and 24 tokens' outputs."""
    cfg = W.EC_CONFIGS[name]
    T, E, D = cfg.num_tokens, cfg.num_experts, cfg.d_model
    print(f"[expert choice full-size] {name}", flush=True)
    C = M.moe_expert_choice_capacity(cfg)
    inp = W.make_inputs(cfg, with_experts=False)
    w13, w2, host = _experts(W.base_name(cfg))
    dev = "cuda"
    weights = dict(w_router=to_torch(inp.w_router, dev), w13=w13, w2=w2, ws13=to_torch(inp.ws13, dev),
                   ws2=to_torch(inp.ws2, dev))
    y = torch.empty((T, D), dtype=act_torch_dtype(cfg), device=dev)
    tor = torch.empty(E * C, dtype=torch.int32, device=dev)
    rw = torch.empty(E * C, dtype=torch.float32, device=dev)
    uns = torch.empty(1, dtype=torch.int32, device=dev)
    ws = M.workspace(cfg, M.MOE_OP_EXPERT_CHOICE, dev)
    M.moe_expert_choice_forward(cfg, weights, to_torch(inp.x, dev), y, tor, rw, uns, ws)
    torch.cuda.synchronize()
    ref = O.expert_choice_route(inp.x, inp.w_router, C)
    tg = to_numpy(tor).astype(np.int64)
    ties = ec_check_selection(ref, tg, C)
    gates = ref["probs"][tg, np.repeat(np.arange(E), C)]
    assert rel_err(to_numpy(rw), gates) <= W_TOL
    unsel = int(to_numpy(uns)[0])
    assert unsel == T - np.unique(tg).size
    print(f"  C={C}, experts with a near-tie exchange {ties}, tokens no expert took {unsel}")
    rng = np.random.default_rng(99)
    sample = np.sort(rng.choice(T, size=24, replace=False))
    y_ref = ec_oracle_output(cfg, inp, tg, C, expert_weights=lambda e: host[e], rows=sample)
    err = row_rel_err(to_numpy(y)[sample], y_ref)
    print(f"  sampled {len(sample)} tokens: max rel err {err:.3e}")
    assert err <= out_tol(cfg)
