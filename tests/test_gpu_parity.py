"""GPU parity: the HIP path through the C ABI against the CPU oracle, on seeded
inputs at sizes the oracle finishes in seconds (several tiles, ragged tails).
"""
import os

import numpy as np
import pytest
import torch

import top_routing_dispatch_amd as M
import workloads as W
from oracle import moe_oracle as O
from workloads.torch_io import act_torch_dtype, to_numpy, to_torch

from parity import (BF16_TOL, W_TOL, DeviceLayer, check_layer, ec_check_selection, ec_oracle_output, oracle_forward,
                    out_tol, refinement_margin, rel_err, rerun_on_choice, route_differences, row_rel_err, set_env)

pytestmark = pytest.mark.gpu

SMALL = [
    W.TINY,
    W.MoEConfig("switch_small", 700, 136, 16, 1, 200, scoring=W.SOFTMAX_TOPK, renormalize=0,
                activation=W.GELU, act_dtype=W.BF16, router_dtype=W.F32, capacity_factor=1.25),
    W.MoEConfig("mixtral_small", 520, 264, 8, 2, 328, scoring=W.TOPK_SOFTMAX, zipf_s=1.0),
    W.MoEConfig("deepseekmoe_small", 600, 200, 32, 6, 136, num_shared=2, d_ff_shared=72,
                scoring=W.SOFTMAX_TOPK, renormalize=1),
    W.MoEConfig("deepseekv3_small", 777, 320, 64, 8, 256, num_shared=1, d_ff_shared=128,
                scoring=W.SIGMOID_BIAS, renormalize=1, zipf_s=1.2),
    W.MoEConfig("fp32_shared_gelu", 150, 96, 12, 3, 100, num_shared=3, d_ff_shared=20,
                activation=W.GELU, act_dtype=W.F32, router_dtype=W.F32, capacity_factor=0.8),
    W.MoEConfig("bf16_x_f32_router_swiglu", 300, 64, 24, 4, 72, act_dtype=W.BF16, router_dtype=W.F32),
]

EDGE = [
    W.MoEConfig("one_token", 1, 64, 4, 2, 64),
    W.MoEConfig("one_expert", 130, 64, 1, 1, 48),
    W.MoEConfig("k_equals_e_soft", 90, 64, 8, 8, 40, renormalize=1),
    W.MoEConfig("mostly_empty_experts", 20, 72, 64, 2, 56, scoring=W.SIGMOID_BIAS),
    W.MoEConfig("max_experts_max_k", 70, 64, 1024, 32, 16, scoring=W.SOFTMAX_TOPK),
    W.MoEConfig("ragged_everything", 259, 8, 5, 3, 8, num_shared=1, d_ff_shared=8, capacity_factor=0.6),
    # three permutation tiles with the largest masks (E * 8 words of LDS) and
    # an expert count that is not a power of two (prefix scans over 1024 threads)
    W.MoEConfig("experts_1000_three_tiles", 600, 64, 1000, 8, 16, scoring=W.SOFTMAX_TOPK, capacity_factor=1.0),
]


@pytest.mark.parametrize("path", ["default", "staged"])
@pytest.mark.parametrize("cfg", SMALL + EDGE, ids=lambda c: c.name)
def test_layer_forward_matches_oracle(cfg, path, monkeypatch):
    """Every configuration on the path the library picks (the one-workgroup
    kernel for the smallest batches) and on the staged kernels."""
    if path == "staged":
        set_env(monkeypatch, "MOE_FUSED", "0")
    stages = M.moe_layer_stages(cfg)
    print(f"[layer parity] {cfg.name} {path}: {' '.join(stages)}", flush=True)
    assert ("fused_layer" in stages) == (path == "default" and cfg.name in FUSED_BY_DEFAULT)
    inp = W.make_inputs(cfg)
    ref = oracle_forward(cfg, inp)
    dl = DeviceLayer(cfg, inp)
    got = dl.layer()
    diff, err = check_layer(cfg, inp, ref, got)
    print(f"  max rel err {err:.3e}, near-tie tokens {len(diff)}")


# Batches that fit one workgroup, over the scoring rules, both activations,
# both element types, capacity drops and shared experts, up to the largest
# batch the fused kernel takes.
FUSED_SHAPES = [
    W.MoEConfig("fused_sigmoid_bias_shared", 64, 128, 16, 4, 64, num_shared=2, d_ff_shared=32,
                scoring=W.SIGMOID_BIAS, renormalize=1, zipf_s=1.2),
    W.MoEConfig("fused_topk_softmax_capacity", 96, 64, 8, 2, 80, scoring=W.TOPK_SOFTMAX, capacity_factor=0.75,
                zipf_s=1.0),
    W.MoEConfig("fused_f32_gelu_shared_capacity", 48, 96, 12, 3, 64, num_shared=3, d_ff_shared=16,
                activation=W.GELU, act_dtype=W.F32, router_dtype=W.F32, capacity_factor=0.8),
    W.MoEConfig("fused_switch_top1", 128, 64, 16, 1, 96, renormalize=0, activation=W.GELU, router_dtype=W.F32,
                capacity_factor=1.25),
    W.MoEConfig("fused_sigmoid_unnormalised_f32", 33, 40, 64, 6, 24, scoring=W.SIGMOID_BIAS, renormalize=0,
                act_dtype=W.F32, router_dtype=W.F32),
    W.MoEConfig("fused_k_equals_e", 40, 32, 4, 4, 16, act_dtype=W.F32, router_dtype=W.F32),
    W.MoEConfig("fused_most_tokens", 256, 32, 8, 2, 48, num_shared=1, d_ff_shared=32, capacity_factor=1.0),
    W.MoEConfig("fused_most_experts", 64, 32, 64, 6, 32, scoring=W.SIGMOID_BIAS, renormalize=1, zipf_s=1.2),
]
FUSED_BY_DEFAULT = {"tiny", "one_token", "one_expert", "k_equals_e_soft", "mostly_empty_experts"}


@pytest.mark.parametrize("cfg", FUSED_SHAPES, ids=lambda c: c.name)
def test_fused_layer_matches_oracle_and_staged_path(cfg, monkeypatch):
    """The one-workgroup layer against the oracle, and its routing decisions
    and statistics against the staged path's (selections equal away from
    near ties, counts and drops equal where the selections are).  MOE_FUSED=1
    takes the one-workgroup kernel for every batch that fits, also where the
    staged path is faster."""
    set_env(monkeypatch, "MOE_FUSED", "1")
    assert M.moe_layer_stages(cfg) == ["fused_layer"]
    print(f"[fused layer] {cfg.name}", flush=True)
    inp = W.make_inputs(cfg)
    ref = oracle_forward(cfg, inp)
    dl = DeviceLayer(cfg, inp)
    fused = dl.layer()
    diff, err = check_layer(cfg, inp, ref, fused)
    print(f"  fused: max rel err {err:.3e}, near-tie tokens {len(diff)}")
    set_env(monkeypatch, "MOE_FUSED", "0")
    assert "fused_layer" not in M.moe_layer_stages(cfg)
    staged = dl.layer()
    check_layer(cfg, inp, ref, staged)
    if (fused["idx"] == staged["idx"]).all():
        np.testing.assert_array_equal(fused["counts"], staged["counts"])
        assert fused["dropped"] == staged["dropped"]
        assert rel_err(fused["w"], staged["w"]) <= W_TOL
        assert row_rel_err(fused["y"], O.widen(staged["y"])) <= 2 * out_tol(cfg)


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_route_matches_oracle(cfg):
    print(f"[route parity] {cfg.name}", flush=True)
    inp = W.make_inputs(cfg, with_experts=False)
    ref = O.route(inp.x, inp.w_router, inp.sel_bias, cfg.top_k, cfg.scoring, cfg.renormalize)
    dl = DeviceLayer(cfg, inp)
    got = dl.route()
    diff = route_differences(cfg, ref, got["idx"], inp.sel_bias)
    assert rel_err(got["w"], rerun_on_choice(cfg, ref, got["idx"], diff)["w"]) <= W_TOL
    assert rel_err(got["probs"], ref["probs"]) <= W_TOL


def _permute_gpu(cfg, idx, x_host):
    T, k, E = cfg.num_tokens, cfg.top_k, cfg.num_experts
    cap, rows_cap = M.moe_capacity(cfg)
    dev = "cuda"
    idx_d = to_torch(idx.astype(np.int32), dev)
    x_d = to_torch(x_host, dev) if x_host is not None else None
    counts = torch.full((E,), -7, dtype=torch.int32, device=dev)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=dev)
    row_of = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    tor = torch.full((max(rows_cap, 1),), -7, dtype=torch.int32, device=dev)
    xp = None
    if x_d is not None:
        xp = torch.zeros((max(rows_cap, 1), cfg.d_model), dtype=act_torch_dtype(cfg), device=dev)
    ws = M.workspace(cfg, M.MOE_OP_PERMUTE, dev)
    M.moe_permute(cfg, idx_d, x_d, counts, offsets, row_of, tor, xp, ws)
    torch.cuda.synchronize()
    return (to_numpy(counts), to_numpy(offsets), to_numpy(row_of), to_numpy(tor)[:rows_cap],
            None if xp is None else to_numpy(xp)[:rows_cap])


@pytest.mark.parametrize("cfg", SMALL + EDGE[:4] + EDGE[-1:], ids=lambda c: c.name)
def test_permute_bit_exact(cfg):
    """Dispatch of the oracle's own selection: counts, offsets, permutation, drops
    and the gathered rows are bit-exact."""
    print(f"[permute parity] {cfg.name}", flush=True)
    inp = W.make_inputs(cfg, with_experts=False)
    ref = O.route(inp.x, inp.w_router, inp.sel_bias, cfg.top_k, cfg.scoring, cfg.renormalize)
    disp = O.dispatch(ref["idx"], cfg.num_experts, O.capacity(cfg.capacity_factor, cfg.num_tokens, cfg.top_k,
                                                              cfg.num_experts))
    counts, offsets, row_of, tor, xp = _permute_gpu(cfg, ref["idx"], inp.x)
    np.testing.assert_array_equal(counts, disp["counts"])
    np.testing.assert_array_equal(offsets, disp["offsets"])
    np.testing.assert_array_equal(row_of, disp["row_of"])
    A = int(disp["offsets"][-1])
    np.testing.assert_array_equal(tor[:A], disp["token_of_row"])
    assert (tor[A:] == -1).all()
    np.testing.assert_array_equal(xp[:A], inp.x[disp["token_of_row"]])


def test_permute_worked_example_and_capacity():
    """The Tiny-MoE dispatch example (4 tokens, top-2), dropless and with C = 2."""
    idx = np.array([[2, 0], [1, 2], [3, 0], [2, 1]])
    cfg = W.MoEConfig("ex", 4, 8, 4, 2, 8, act_dtype=W.F32, router_dtype=W.F32)
    counts, offsets, row_of, tor, _ = _permute_gpu(cfg, idx, None)
    assert counts.tolist() == [2, 2, 3, 1] and offsets.tolist() == [0, 2, 4, 7, 8]
    assert tor.tolist() == [0, 2, 1, 3, 0, 1, 3, 2]
    assert row_of.tolist() == [[4, 0], [2, 5], [7, 1], [6, 3]]
    cfg2 = cfg.replace(capacity_factor=1.0)          # C = ceil(1.0 * 4 * 2 / 4) = 2
    counts, offsets, row_of, tor, _ = _permute_gpu(cfg2, idx, None)
    assert offsets.tolist() == [0, 2, 4, 6, 7]
    assert row_of.tolist() == [[4, 0], [2, 5], [6, 1], [-1, 3]]
    assert tor.tolist() == [0, 2, 1, 3, 0, 1, 2, -1]      # A_cap = min(T*k, E*C) = 8 rows, 7 kept


def test_permute_every_token_on_one_expert_with_capacity():
    T, E = 1000, 8
    cfg = W.MoEConfig("one_hot", T, 8, E, 1, 8, act_dtype=W.F32, router_dtype=W.F32, capacity_factor=2.0)
    C = O.capacity(2.0, T, 1, E)     # 250
    idx = np.full((T, 1), 5)
    counts, offsets, row_of, tor, _ = _permute_gpu(cfg, idx, None)
    assert counts.tolist() == [0] * 5 + [T] + [0] * 2
    assert offsets[-1] == C
    assert tor.tolist() == list(range(C)) + [-1] * (T - C)
    assert (row_of[:C, 0] == np.arange(C)).all() and (row_of[C:, 0] == -1).all()


def test_permute_skips_repeated_and_out_of_range_ids():
    """Slots whose expert id is outside [0, E) or repeats an earlier slot of the
    same token are not dispatched (row -1, not counted); the other slots keep
    the order of the valid ones.  (Library behaviour for inputs moe_route never
    produces; the pages do not define them.)"""
    idx = np.array([[1, 1], [0, 4], [-1, 2], [2, 0], [3, 3]])
    cfg = W.MoEConfig("bad_ids", 5, 8, 4, 2, 8, act_dtype=W.F32, router_dtype=W.F32)
    counts, offsets, row_of, tor, _ = _permute_gpu(cfg, idx, None)
    # valid slots in (token, slot) order: (0,0)->1 (1,0)->0 (2,1)->2 (3,0)->2 (3,1)->0 (4,0)->3
    assert counts.tolist() == [2, 1, 2, 1]
    assert offsets.tolist() == [0, 2, 3, 5, 6]
    assert tor.tolist() == [1, 3, 0, 2, 3, 4, -1, -1, -1, -1]
    assert row_of.tolist() == [[2, -1], [0, -1], [-1, 3], [4, 1], [5, -1]]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_expert_ffn_matches_oracle(cfg):
    """Grouped expert FFN on the oracle's expert batches (x_perm, offsets)."""
    print(f"[expert ffn parity] {cfg.name}", flush=True)
    inp = W.make_inputs(cfg)
    ref = oracle_forward(cfg, inp)
    A = int(ref["offsets"][-1])
    dev = "cuda"
    xp = to_torch(inp.x[ref["token_of_row"]], dev) if A else torch.empty((0, cfg.d_model), device=dev)
    off = to_torch(ref["offsets"].astype(np.int32), dev)
    y = torch.zeros((max(A, 1), cfg.d_model), dtype=act_torch_dtype(cfg), device=dev)
    ws = torch.empty(max(M.moe_workspace_size(cfg, M.MOE_OP_EXPERT_FFN), 256), dtype=torch.uint8, device=dev)
    M.moe_expert_ffn(cfg, cfg.num_experts, cfg.d_ff, cfg.activation, A, xp, None, off,
                     to_torch(inp.w13, dev), to_torch(inp.w2, dev), y, ws)
    torch.cuda.synchronize()
    err = row_rel_err(to_numpy(y)[:A], ref["y_perm"])
    assert err <= out_tol(cfg), err
    if cfg.num_shared:
        ys = torch.zeros((cfg.num_tokens, cfg.d_model), dtype=act_torch_dtype(cfg), device=dev)
        ws2 = M.workspace(cfg, M.MOE_OP_SHARED_FFN, dev)
        M.moe_expert_ffn(cfg, 1, cfg.num_shared * cfg.d_ff_shared, W.SWIGLU, cfg.num_tokens, to_torch(inp.x, dev),
                         None, None, to_torch(inp.ws13, dev), to_torch(inp.ws2, dev), ys, ws2)
        torch.cuda.synchronize()
        err = row_rel_err(to_numpy(ys), ref["y_shared"])
        assert err <= out_tol(cfg), err


@pytest.mark.parametrize("cfg", [SMALL[0], SMALL[3]], ids=lambda c: c.name)
def test_expert_ffn_gathered_rows(cfg):
    """Same grouped FFN reading token rows through the permutation (gather_rows)."""
    inp = W.make_inputs(cfg)
    ref = oracle_forward(cfg, inp)
    A = int(ref["offsets"][-1])
    dev = "cuda"
    y = torch.zeros((A, cfg.d_model), dtype=act_torch_dtype(cfg), device=dev)
    ws = M.workspace(cfg, M.MOE_OP_EXPERT_FFN, dev)
    M.moe_expert_ffn(cfg, cfg.num_experts, cfg.d_ff, cfg.activation, A, to_torch(inp.x, dev),
                     to_torch(ref["token_of_row"].astype(np.int32), dev), to_torch(ref["offsets"].astype(np.int32), dev),
                     to_torch(inp.w13, dev), to_torch(inp.w2, dev), y, ws)
    torch.cuda.synchronize()
    assert row_rel_err(to_numpy(y), ref["y_perm"]) <= out_tol(cfg)


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_combine_matches_oracle(cfg):
    """Combine on oracle-supplied expert outputs (rounded to the activation type)."""
    inp = W.make_inputs(cfg)
    ref = oracle_forward(cfg, inp)
    dev = "cuda"
    enc = (lambda a: W.f32_to_bf16_bits(a.astype(np.float32))) if cfg.act_dtype == W.BF16 else \
        (lambda a: a.astype(np.float32))
    yp_h = enc(ref["y_perm"]) if ref["y_perm"].size else enc(np.zeros((1, cfg.d_model)))
    yp = to_torch(yp_h, dev)
    ys = to_torch(enc(ref["y_shared"]), dev) if ref["y_shared"] is not None else None
    y = torch.empty((cfg.num_tokens, cfg.d_model), dtype=act_torch_dtype(cfg), device=dev)
    M.moe_combine(cfg, yp, to_torch(ref["row_of"].astype(np.int32), dev), to_torch(ref["w"].astype(np.float32), dev),
                  ys, y)
    torch.cuda.synchronize()
    # expected from the same rounded operands, in float64
    Yr = O.widen(yp_h)
    ysr = O.widen(enc(ref["y_shared"])) if ref["y_shared"] is not None else None
    exp = O.combine(Yr[:int(ref["offsets"][-1])], ref, ref["w"].astype(np.float32).astype(np.float64),
                    cfg.num_tokens, ysr)
    assert row_rel_err(to_numpy(y), exp) <= out_tol(cfg)


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_load_stats_matches_oracle(cfg):
    inp = W.make_inputs(cfg, with_experts=False)
    r = O.route(inp.x, inp.w_router, inp.sel_bias, cfg.top_k, cfg.scoring, cfg.renormalize)
    cap = O.capacity(cfg.capacity_factor, cfg.num_tokens, cfg.top_k, cfg.num_experts)
    d = O.dispatch(r["idx"], cfg.num_experts, cap)
    st = O.load_stats(d["counts"], r["probs"], cfg.top_k, cfg.alpha, d["kept"])
    dev = "cuda"
    E = cfg.num_experts
    f = torch.empty(E, device=dev)
    P = torch.empty(E, device=dev)
    out = torch.empty(2, device=dev)
    dropped = torch.empty(1, dtype=torch.int32, device=dev)
    ws = M.workspace(cfg, M.MOE_OP_LOAD_STATS, dev)
    M.moe_load_stats(cfg, to_torch(d["counts"].astype(np.int32), dev), to_torch(r["probs"].astype(np.float32), dev),
                     cfg.alpha, f, P, out[0:1], out[1:2], dropped, ws)
    torch.cuda.synchronize()
    assert rel_err(to_numpy(f), st["f"]) <= W_TOL
    assert rel_err(to_numpy(P), st["P"]) <= W_TOL
    o = to_numpy(out)
    assert abs(o[0] - st["aux_loss"]) <= W_TOL * st["aux_loss"]
    assert abs(o[1] - st["imbalance"]) <= W_TOL * st["imbalance"]
    assert int(to_numpy(dropped)[0]) == st["dropped"]


def test_load_stats_worked_examples():
    """[9,4,2,1] -> imbalance 2.25; uniform routing -> loss = alpha."""
    dev = "cuda"
    cfg = W.MoEConfig("ex", 8, 8, 4, 2, 8, act_dtype=W.F32, router_dtype=W.F32)
    probs = torch.full((8, 4), 0.25, device=dev)
    f = torch.empty(4, device=dev); P = torch.empty(4, device=dev); o = torch.empty(2, device=dev)
    dr = torch.empty(1, dtype=torch.int32, device=dev)
    ws = M.workspace(cfg, M.MOE_OP_LOAD_STATS, dev)
    M.moe_load_stats(cfg, torch.tensor([9, 4, 2, 1], dtype=torch.int32, device=dev), probs, 0.01, f, P,
                     o[0:1], o[1:2], dr, ws)
    torch.cuda.synchronize()
    assert abs(o[1].item() - 2.25) < 1e-6
    M.moe_load_stats(cfg, torch.tensor([4, 4, 4, 4], dtype=torch.int32, device=dev), probs, 0.01, f, P,
                     o[0:1], o[1:2], dr, ws)
    torch.cuda.synchronize()
    assert abs(o[0].item() - 0.01) < 1e-8 and int(dr.item()) == 0


def test_forced_expert_with_capacity_drops_to_residual():
    """A huge selection bias sends every token to expert 3; with capacity C only
    the first C tokens get expert output, the rest get exactly zero (the
    residual carries them)."""
    cfg = W.MoEConfig("forced", 300, 64, 8, 1, 32, scoring=W.SIGMOID_BIAS, renormalize=0, capacity_factor=2.0)
    inp = W.make_inputs(cfg)
    b = np.zeros(8, dtype=np.float32)
    b[3] = 100.0
    ref = oracle_forward(cfg, inp, sel_bias=b)
    assert (ref["idx"][:, 0] == 3).all()
    C = O.capacity(2.0, 300, 1, 8)
    dl = DeviceLayer(cfg, inp, sel_bias=b)
    got = dl.layer()
    check_layer(cfg, inp, ref, got, sel_bias=b)
    y = O.widen(got["y"])
    assert (y[C:] == 0).all() and got["dropped"] == 300 - C


def test_empty_batch():
    cfg = W.MoEConfig("empty", 0, 64, 8, 2, 32)
    inp = W.make_inputs(cfg)
    dl = DeviceLayer(cfg, inp)
    got = dl.layer()
    assert got["y"].shape == (0, 64)
    assert (got["counts"] == 0).all() and got["dropped"] == 0


@pytest.mark.parametrize("cfg", [SMALL[2], SMALL[4], SMALL[1]], ids=lambda c: c.name)
def test_deterministic(cfg):
    inp = W.make_inputs(cfg)
    dl = DeviceLayer(cfg, inp)
    a, b = dl.layer(), dl.layer()
    for key in ("y", "idx", "w", "counts", "stats"):
        np.testing.assert_array_equal(a[key], b[key])


def test_near_tie_refinement_decides_in_double_precision():
    """Two experts whose logits differ by far less than float32 can resolve:
    the library must still pick the one the exact logits rank higher."""
    T, D, E = 64, 64, 16
    cfg = W.MoEConfig("ties", T, D, E, 2, 16, act_dtype=W.F32, router_dtype=W.F32, scoring=W.TOPK_SOFTMAX)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((T, D)).astype(np.float32)
    wr = (rng.standard_normal((E, D)) * 0.02).astype(np.float32)
    # expert 9 = expert 4 plus a tiny perturbation on one coordinate: logits of 4 and 9
    # differ by ~x[:, 0] * 2^-20, below float32 resolution of a D-long sum
    wr[4] = wr[2] * 3
    wr[9] = wr[4]
    wr[9, 0] = np.nextafter(wr[9, 0], np.float32(1.0))
    inp = W.HostInputs(cfg, x, wr, None, np.zeros((E, 32, D), np.float32), np.zeros((E, D, 16), np.float32),
                       [], None, None)
    ref = O.route(x, wr, None, 2, cfg.scoring, 0)
    dl = DeviceLayer(cfg, inp)
    got = dl.route()
    diff = route_differences(cfg, ref, got["idx"], None)
    # the exact logits of 4 and 9 are distinct (gap ~1e-9 relative: exempt by the 1e-6 rule),
    # yet the refinement orders them like the float64 oracle
    np.testing.assert_array_equal(got["idx"], ref["idx"])
    assert len(diff) == 0


V2_SHAPES = [
    W.MoEConfig("v2_swiglu_shared", 700, 256, 8, 2, 320, num_shared=1, d_ff_shared=128),
    W.MoEConfig("v2_gelu_capacity", 900, 192, 16, 1, 384, scoring=W.SOFTMAX_TOPK, renormalize=0,
                activation=W.GELU, router_dtype=W.F32, capacity_factor=1.25),
    W.MoEConfig("v2_sigmoid_many", 333, 128, 64, 6, 128, num_shared=2, d_ff_shared=64, scoring=W.SIGMOID_BIAS,
                zipf_s=1.2),
]


# -1: general kernel; 0-13: deep-tile kernel with 32- or 64-deep slices (9, 10:
# persistent tiles; 12, 13: slices staged in registers); 14-21: persistent
# weight-streaming kernel
GEMM_TILE_CONFIGS = range(-1, 22)
WS_CONFIGS = range(14, 22)


@pytest.mark.parametrize("gemm_cfg", [str(c) for c in GEMM_TILE_CONFIGS])
@pytest.mark.parametrize("cfg", V2_SHAPES, ids=lambda c: c.name)
def test_every_gemm_tile_config(cfg, gemm_cfg, monkeypatch):
    """Each tile configuration of the pipelined expert GEMM (K a multiple of 64)
    against the oracle, through the whole layer; -1 is the general kernel."""
    set_env(monkeypatch, "MOE_GEMM_CFG", gemm_cfg)
    print(f"[tile config {gemm_cfg}] {cfg.name}", flush=True)
    inp = W.make_inputs(cfg)
    ref = oracle_forward(cfg, inp)
    got = DeviceLayer(cfg, inp).layer()
    diff, err = check_layer(cfg, inp, ref, got)
    print(f"  max rel err {err:.3e}")


SPLIT_SHAPES = [
    # shallow (<= 64 rows) and deep groups side by side
    W.MoEConfig("split_sigmoid_zipf", 1500, 256, 32, 4, 192, num_shared=1, d_ff_shared=128,
                scoring=W.SIGMOID_BIAS, zipf_s=1.4),
    W.MoEConfig("split_softmax_ragged", 777, 320, 16, 2, 448, zipf_s=1.2),
]


@pytest.mark.parametrize("split", ["0", "1", "1-pers9", "1-rows128", "1-sh16-rows192"])
@pytest.mark.parametrize("cfg", SPLIT_SHAPES + V2_SHAPES, ids=lambda c: c.name)
def test_shallow_group_split(cfg, split, monkeypatch):
    """Expert FFN with shallow groups split off to the persistent
    weight-streaming kernel (1; rowsN: groups of up to N rows count as
    shallow, so that they take several of its 64-row tiles; 1-sh16: its
    64 x 256 configuration), to the persistent configuration 9 of the
    deep-tile kernel (1-pers9), and without the split (0), against the oracle."""
    set_env(monkeypatch, "MOE_GEMM_SPLIT", split[0])
    if split == "1-pers9":
        set_env(monkeypatch, "MOE_GEMM_SHCFG", "9")
    if split.startswith("1-sh"):
        set_env(monkeypatch, "MOE_GEMM_SHCFG", split[4:6])
    if "-rows" in split:
        set_env(monkeypatch, "MOE_SHALLOW_ROWS", split.split("-rows")[1])
    print(f"[split {split}] {cfg.name}", flush=True)
    inp = W.make_inputs(cfg)
    ref = oracle_forward(cfg, inp)
    counts = np.bincount(ref["idx"].ravel(), minlength=cfg.num_experts)
    print(f"  group rows: min {counts.min()} max {counts.max()}, <= 64: {(counts <= 64).sum()}")
    got = DeviceLayer(cfg, inp).layer()
    diff, err = check_layer(cfg, inp, ref, got)
    print(f"  max rel err {err:.3e}")


TAIL_SHAPES = [
    # down projections with K >= 4096 and fewer 256x256 tiles than CUs, so
    # that every tile runs in the split tail (K = 4096: eight units of 8
    # slices each; K = 4160 = 65 slices: one unit, as 65 has no even
    # divisor); the case with full rounds before the tail is the full-size
    # Mixtral-shaped layer; ragged N and ragged groups
    W.MoEConfig("tail_split_deep", 800, 512, 8, 2, 4096, zipf_s=0.5),
    W.MoEConfig("tail_split_ragged", 900, 448, 6, 2, 4160, zipf_s=1.0),
]


@pytest.mark.parametrize("parent", ["0", "13"])
@pytest.mark.parametrize("tail", ["0", "1"])
@pytest.mark.parametrize("cfg", TAIL_SHAPES, ids=lambda c: c.name)
def test_down_tail_split(cfg, tail, parent, monkeypatch):
    """The down projection on 256x256 tiles (DMA rings: 0; slices staged in
    registers: 13) with the tiles of its last, partial round split over the
    contraction (1) and without (0), against the oracle."""
    set_env(monkeypatch, "MOE_GEMM_CFG", parent)
    set_env(monkeypatch, "MOE_GEMM_TAIL", tail)
    print(f"[tail {tail} parent {parent}] {cfg.name}", flush=True)
    inp = W.make_inputs(cfg)
    ref = oracle_forward(cfg, inp)
    got = DeviceLayer(cfg, inp).layer()
    diff, err = check_layer(cfg, inp, ref, got)
    print(f"  max rel err {err:.3e}")


# Group sizes that give a 256-row tile every count of active 32-row blocks in
# either row half of its waves (1-4), waves that load no activation rows,
# empty groups and groups of several tiles.
STAGED_GROUPS = [0, 1, 31, 32, 33, 64, 65, 100, 128, 129, 200, 255, 0, 256, 257, 600]


@pytest.mark.parametrize("gather", [False, True], ids=["rows", "gathered"])
@pytest.mark.parametrize("activation", [W.SWIGLU, W.GELU], ids=["swiglu", "gelu"])
@pytest.mark.parametrize("D,F", [(64, 64), (128, 192), (384, 128), (256, 320)])
def test_staged_slices_bit_identical_to_dma_rings(D, F, activation, gather, monkeypatch):
    """The deep-tile configurations that stage slices in registers (12: four
    waves, 13: eight) reproduce the bits of configuration 0 (DMA rings), whose
    results the tile-configuration tests check against the oracle: each output
    is accumulated by the same MFMAs in the same order.  Contractions of 1, 2,
    3, 4, 5 and 6 slices of 64 cover the staged loop's prologue, steady part
    and tail."""
    dev = "cuda"
    G = len(STAGED_GROUPS)
    offs = np.concatenate([[0], np.cumsum(STAGED_GROUPS)]).astype(np.int32)
    rows = int(offs[-1])
    cfg = W.MoEConfig("staged_bits", rows, D, G, 1, F, activation=activation)
    print(f"[staged bits] D={D} F={F} act={activation} gather={gather} rows={rows}", flush=True)
    g = torch.Generator().manual_seed(7 * D + F + 1000 * activation)
    nF = (2 if activation == W.SWIGLU else 1) * F
    if gather:
        src = torch.randn(rows + 37, D, generator=g).to(torch.bfloat16)
        pick = torch.randperm(rows + 37, generator=g)[:rows].to(torch.int32)
        x_in, rows_in = src.to(dev), pick.to(dev)
    else:
        x_in, rows_in = torch.randn(rows, D, generator=g).to(torch.bfloat16).to(dev), None
    w13 = (torch.randn(G, nF, D, generator=g) * 0.05).to(torch.bfloat16).to(dev)
    w2 = (torch.randn(G, D, F, generator=g) * 0.05).to(torch.bfloat16).to(dev)
    off = torch.from_numpy(offs).to(dev)
    ws = M.workspace(cfg, M.MOE_OP_EXPERT_FFN, dev)
    outs = {}
    for c in ("0", "12", "13"):
        set_env(monkeypatch, "MOE_GEMM_CFG", c)
        y = torch.full((rows, D), float("nan"), dtype=torch.bfloat16, device=dev)
        M.moe_expert_ffn(cfg, G, F, activation, rows, x_in, rows_in, off, w13, w2, y, ws)
        torch.cuda.synchronize()
        outs[c] = y.cpu()
    assert torch.isfinite(outs["0"].float()).all()
    for c in ("12", "13"):
        same = outs[c].view(torch.int16) == outs["0"].view(torch.int16)
        assert bool(same.all()), f"config {c}: {int((~same).sum())} of {same.numel()} outputs differ"


WS_SHAPES = [
    # more tiles than workgroups of the persistent weight-streaming kernel, so
    # that its ring crosses tile boundaries: a 512-deep GELU contraction with
    # capacity (8 slices per tile) and a 192-deep SwiGLU one (3 slices per
    # tile: the loads run more than a whole tile ahead)
    W.MoEConfig("ws_gelu_many_tiles", 2048, 512, 128, 1, 2048, scoring=W.SOFTMAX_TOPK, renormalize=0,
                activation=W.GELU, router_dtype=W.F32, capacity_factor=1.25),
    W.MoEConfig("ws_swiglu_many_tiles", 1024, 192, 96, 2, 1536, zipf_s=1.0),
]


@pytest.mark.parametrize("gemm_cfg", ["default"] + [str(c) for c in WS_CONFIGS])
@pytest.mark.parametrize("cfg", WS_SHAPES, ids=lambda c: c.name)
def test_weight_streaming_many_tiles(cfg, gemm_cfg, monkeypatch):
    """The persistent weight-streaming GEMM (its configurations 14-21, and the
    default choice for these shallow groups) against the oracle with several
    tiles per workgroup."""
    if gemm_cfg != "default":
        set_env(monkeypatch, "MOE_GEMM_CFG", gemm_cfg)
    print(f"[ws {gemm_cfg}] {cfg.name}", flush=True)
    inp = W.make_inputs(cfg)
    ref = oracle_forward(cfg, inp)
    got = DeviceLayer(cfg, inp).layer()
    diff, err = check_layer(cfg, inp, ref, got)
    print(f"  max rel err {err:.3e}")


KSPLIT_SHAPES = [
    # many units per workgroup of the weight-streaming kernel, so that its ring
    # crosses unit boundaries (other contraction offsets): a GELU layer with
    # capacity (512- and 2048-deep contractions) and a SwiGLU one (256 / 1024)
    W.MoEConfig("ksplit_gelu_capacity", 2048, 512, 128, 1, 2048, scoring=W.SOFTMAX_TOPK, renormalize=0,
                activation=W.GELU, router_dtype=W.F32, capacity_factor=1.25),
    W.MoEConfig("ksplit_swiglu_shared", 1024, 256, 48, 2, 1024, num_shared=1, d_ff_shared=512, zipf_s=1.0),
]


@pytest.mark.parametrize("ks", ["2", "4", "8"])
@pytest.mark.parametrize("gemm_cfg", [str(c) for c in WS_CONFIGS])
@pytest.mark.parametrize("cfg", KSPLIT_SHAPES, ids=lambda c: c.name)
def test_contraction_split(cfg, gemm_cfg, ks, monkeypatch):
    """Every configuration of the weight-streaming GEMM with its contraction
    split in 2, 4 or 8 parts (float32 partial sums added by a second kernel;
    a launch whose contraction the forced split does not divide runs unsplit)
    against the oracle, shared expert included."""
    set_env(monkeypatch, "MOE_GEMM_CFG", gemm_cfg)
    set_env(monkeypatch, "MOE_GEMM_KSPLIT", ks)
    print(f"[ksplit {ks} cfg {gemm_cfg}] {cfg.name}", flush=True)
    inp = W.make_inputs(cfg)
    ref = oracle_forward(cfg, inp)
    got = DeviceLayer(cfg, inp).layer()
    diff, err = check_layer(cfg, inp, ref, got)
    print(f"  max rel err {err:.3e}")


DECODE_SHAPES = [
    # decode-sized batches with long contractions: every group is shallow and
    # the tiles are few, so both projections run on the weight-streaming
    # kernel with the contraction split (gate/up 4 and down 8 parts in the
    # first; the shared expert split in the second; GELU in the third)
    W.MoEConfig("decode_t1_e8", 1, 1024, 8, 2, 2048, scoring=W.TOPK_SOFTMAX, zipf_s=1.0),
    W.MoEConfig("decode_t3_shared", 3, 512, 64, 8, 512, num_shared=1, d_ff_shared=1024,
                scoring=W.SIGMOID_BIAS, zipf_s=1.2),
    W.MoEConfig("decode_t2_gelu", 2, 768, 16, 1, 3072, scoring=W.SOFTMAX_TOPK, renormalize=0,
                activation=W.GELU, router_dtype=W.F32),
    W.MoEConfig("decode_t8_e64", 8, 1024, 64, 6, 1024, num_shared=2, d_ff_shared=512, renormalize=1),
    # long rows: the combine spreads one token's row over two workgroups
    # (bf16 with a shared expert, bf16 top-1, float32)
    W.MoEConfig("decode_t5_wide", 5, 8192, 16, 4, 128, num_shared=1, d_ff_shared=128, renormalize=1),
    W.MoEConfig("decode_t3_wide_k1", 3, 9216, 8, 1, 128, renormalize=0),
    W.MoEConfig("decode_t2_f32_wide", 2, 4096, 4, 2, 64, act_dtype=W.F32, router_dtype=W.F32),
    # more rows than one shallow tile but no group above 48 (the token
    # count): every group shallow, on all CUs
    W.MoEConfig("decode_t48_rows384", 48, 1024, 32, 8, 1024, scoring=W.SIGMOID_BIAS, zipf_s=1.2),
    # a few groups above 64 rows among many small ones (12 rows per group on
    # average): the shallow groups beside the deep ones on 192 CUs
    W.MoEConfig("decode_t200_skewed", 200, 1024, 128, 8, 1024, zipf_s=1.3),
]


@pytest.mark.parametrize("ks", ["auto", "1"])
@pytest.mark.parametrize("cfg", DECODE_SHAPES, ids=lambda c: c.name)
def test_decode_shapes(cfg, ks, monkeypatch):
    """Decode-sized layers (1 to 8 tokens) against the oracle, with the
    automatic contraction split and without it."""
    if ks != "auto":
        set_env(monkeypatch, "MOE_GEMM_KSPLIT", ks)
    print(f"[decode ksplit {ks}] {cfg.name}", flush=True)
    inp = W.make_inputs(cfg)
    ref = oracle_forward(cfg, inp)
    got = DeviceLayer(cfg, inp).layer()
    diff, err = check_layer(cfg, inp, ref, got)
    print(f"  max rel err {err:.3e}")


ROUTER_SHAPES = [
    # the router kernels' range (E <= 256, D % 64 == 0): float32 and bf16
    # weights, ragged expert counts, row counts that are not multiples of 16 or 32;
    # E <= 64 goes to the kernel that splits the contraction over waves
    W.MoEConfig("router_e8_bf16w", 333, 4096, 8, 2, 64, scoring=W.TOPK_SOFTMAX, zipf_s=1.0),
    W.MoEConfig("router_e40_f32w", 250, 320, 40, 3, 64, scoring=W.SOFTMAX_TOPK, renormalize=1,
                router_dtype=W.F32),
    W.MoEConfig("router_e64_bf16w", 517, 2048, 64, 6, 64, scoring=W.SOFTMAX_TOPK, renormalize=1),
    W.MoEConfig("router_e16_f32w", 64, 128, 16, 1, 64, scoring=W.SOFTMAX_TOPK, renormalize=0,
                router_dtype=W.F32),
    W.MoEConfig("router_e128_f32w", 300, 256, 128, 2, 64, scoring=W.SOFTMAX_TOPK, renormalize=1,
                router_dtype=W.F32),
    W.MoEConfig("router_e200_bf16w", 257, 192, 200, 4, 64, scoring=W.SIGMOID_BIAS, zipf_s=1.2),
    W.MoEConfig("router_e256_f32w", 129, 512, 256, 8, 64, scoring=W.TOPK_SOFTMAX, router_dtype=W.F32),
    # few tokens, many experts: the experts split over workgroups by default
    W.MoEConfig("router_t1_e256_bf16w", 1, 7168, 256, 8, 64, scoring=W.SIGMOID_BIAS, zipf_s=1.2),
    W.MoEConfig("router_t5_e160_f32w", 5, 384, 160, 4, 64, scoring=W.SOFTMAX_TOPK, renormalize=1,
                router_dtype=W.F32),
    W.MoEConfig("router_t16_e8_bf16w", 16, 4096, 8, 2, 64, scoring=W.TOPK_SOFTMAX, zipf_s=1.0),
    W.MoEConfig("router_t3_e64_bf16w", 3, 2048, 64, 6, 64, scoring=W.SOFTMAX_TOPK, renormalize=1),
    W.MoEConfig("router_t9_e128_f32w", 9, 768, 128, 1, 64, scoring=W.SOFTMAX_TOPK, renormalize=0,
                router_dtype=W.F32),
    # more tokens than the expert split takes by default
    W.MoEConfig("router_t600_e256_bf16w", 600, 256, 256, 8, 64, scoring=W.SIGMOID_BIAS, zipf_s=1.2),
]


@pytest.mark.parametrize("kernel", ["1", "1-tiled", "1-split", "1-gemv", "0"])
@pytest.mark.parametrize("cfg", ROUTER_SHAPES, ids=lambda c: c.name)
def test_router_logits_and_selection(cfg, kernel, monkeypatch):
    """Router logits within the refinement margin of the float64 logits and the
    selection equal to the oracle's, with the router kernels (1: the default
    choice; 1-tiled / 1-split: for E > 64, every expert per workgroup / the
    experts split over workgroups; 1-gemv: one wave per expert, where the
    tokens fit) and the general GEMM path (0)."""
    set_env(monkeypatch, "MOE_ROUTER_KERNEL", kernel[0])
    if kernel != "1" and kernel[0] == "1":
        set_env(monkeypatch, "MOE_ROUTER_PATH", kernel[2:])
    print(f"[router {kernel}] {cfg.name}", flush=True)
    T, E, k = cfg.num_tokens, cfg.num_experts, cfg.top_k
    inp = W.make_inputs(cfg, with_experts=False)
    ref = O.route(inp.x, inp.w_router, inp.sel_bias, k, cfg.scoring, cfg.renormalize)
    x = to_torch(inp.x, "cuda")
    wr = to_torch(inp.w_router, "cuda")
    bias = to_torch(inp.sel_bias, "cuda") if inp.sel_bias is not None else None
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = M.workspace(cfg, M.MOE_OP_ROUTE, "cuda")
    M.moe_route(cfg, x, wr, bias, idx, tw, None, ws)
    torch.cuda.synchronize()
    s32 = ws[: T * E * 4].view(torch.float32).reshape(T, E).cpu().numpy().astype(np.float64)
    err = np.abs(s32 - ref["logits"]).max(axis=1)
    margin = refinement_margin(s32)
    print(f"  logit error max {err.max():.3e}; smallest margin/error {np.min(margin / np.maximum(err, 1e-30)):.1f}")
    assert (err * 16 < margin).all()
    gi = to_numpy(idx)
    diff = route_differences(cfg, ref, gi, inp.sel_bias)
    assert rel_err(to_numpy(tw), rerun_on_choice(cfg, ref, gi, diff)["w"]) <= W_TOL


GRAPH_SHAPES = [
    # Switch-like (capacity, GELU, weight-streaming GEMM) and one with shared
    # experts on the auxiliary stream and the deep-tile GEMM
    W.MoEConfig("graph_gelu_capacity", 900, 192, 16, 1, 384, scoring=W.SOFTMAX_TOPK, renormalize=0,
                activation=W.GELU, router_dtype=W.F32, capacity_factor=1.25),
    W.MoEConfig("graph_swiglu_shared", 700, 256, 8, 2, 320, num_shared=1, d_ff_shared=128),
    # the one-workgroup kernel
    W.TINY,
]


@pytest.mark.parametrize("cfg", GRAPH_SHAPES, ids=lambda c: c.name)
def test_layer_forward_graph_replay(cfg):
    """The layer forward captured in a HIP graph (its auxiliary-stream work
    joins the capture through the fork / join events) and replayed several
    times, with eager calls of the same layer in between: every replay equals
    the eager result bit for bit."""
    print(f"[graph replay] {cfg.name}", flush=True)
    inp = W.make_inputs(cfg)
    dl = DeviceLayer(cfg, inp)
    T, k, E = cfg.num_tokens, cfg.top_k, cfg.num_experts
    dev = "cuda"
    y = torch.empty((T, cfg.d_model), dtype=act_torch_dtype(cfg), device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    stats = torch.empty(2 * E + 2, dtype=torch.float32, device=dev)
    dropped = torch.empty(1, dtype=torch.int32, device=dev)
    ws = M.workspace(cfg, M.MOE_OP_LAYER, dev)

    def call():
        M.moe_layer_forward(cfg, dl.weights, dl.x, y, idx, w, counts, cfg.alpha, stats, dropped, ws)

    call()                                  # eager: reference, and one-time set-up outside the capture
    torch.cuda.synchronize()
    ref = [to_numpy(t).copy() for t in (y, idx, w, counts, stats)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(0); idx.fill_(-9); w.fill_(0); counts.fill_(-9); stats.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        got = [to_numpy(t) for t in (y, idx, w, counts, stats)]
        for r, a in zip(ref, got):
            np.testing.assert_array_equal(a, r)
        call()                              # eager work between the replays
        torch.cuda.synchronize()


# --------------------------------------------------------------------------
# expert-parallel layouts and the local expert FFN over received rows
# --------------------------------------------------------------------------
@pytest.mark.parametrize("R,E,T,k", [(2, 8, 300, 2), (4, 64, 777, 6), (8, 256, 513, 8), (1, 16, 50, 3)])
def test_ep_send_layout(R, E, T, k):
    """Per-rank send counts and offsets of the GPU permutation against the
    oracle's (sums of kept rows over each rank's experts), bit-exact."""
    print(f"[ep send] R={R} E={E} T={T} k={k}", flush=True)
    cfg = W.MoEConfig("ep_send", T, 64, E, k, 64, scoring=W.SIGMOID_BIAS, zipf_s=1.2)
    inp = W.make_inputs(cfg, with_experts=False)
    ref = O.route(inp.x, inp.w_router, inp.sel_bias, k, cfg.scoring, cfg.renormalize)
    idx = to_torch(ref["idx"].astype(np.int32), "cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    row_of = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tor = torch.empty(T * k, dtype=torch.int32, device="cuda")
    M.moe_permute(cfg, idx, None, counts, off, row_of, tor, None, M.workspace(cfg, M.MOE_OP_PERMUTE, "cuda"))
    sc = torch.empty(R, dtype=torch.int32, device="cuda")
    so = torch.empty(R + 1, dtype=torch.int32, device="cuda")
    M.moe_ep_send_layout(E, R, off, sc, so)
    torch.cuda.synchronize()
    want = O.ep_send_layout(O.dispatch(ref["idx"], E, None)["kept"], R)
    np.testing.assert_array_equal(to_numpy(sc), want["send_counts"])
    np.testing.assert_array_equal(to_numpy(so), want["send_offsets"])


def _recv_counts(R, El, seed, empty_frac=0.2, hi=40):
    rng = np.random.default_rng(seed)
    rc = rng.integers(0, hi, size=(R, El)).astype(np.int32)
    rc[rng.random((R, El)) < empty_frac] = 0
    return rc


@pytest.mark.parametrize("R,El,seed,extra", [(8, 32, 1, 0), (3, 5, 2, 17), (1, 1, 3, 0), (16, 64, 4, 5),
                                             (4, 4, 5, -1)])
def test_ep_recv_layout(R, El, seed, extra):
    """Local offsets and the gather map against the oracle, bit-exact; entries
    past the received total are -1 (extra > 0: spare capacity), and a
    capacity one short of the total (extra = -1) clamps the offsets and
    leaves the last row undescribed."""
    print(f"[ep recv] R={R} El={El} seed={seed} extra={extra}", flush=True)
    rc = _recv_counts(R, El, seed)
    if rc.sum() == 0:
        rc[0, 0] = 3
    want = O.ep_recv_layout(rc)
    total = int(rc.sum())
    cap = total + extra
    lo = torch.empty(El + 1, dtype=torch.int32, device="cuda")
    g = torch.full((max(cap, 1),), -7, dtype=torch.int32, device="cuda")
    M.moe_ep_recv_layout(to_torch(rc, "cuda"), cap, lo, g)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_numpy(lo), np.minimum(want["local_offsets"], cap))
    got = to_numpy(g)[:cap]
    n = min(cap, total)
    np.testing.assert_array_equal(got[:n], want["gather"][:n])
    assert (got[n:] == -1).all()


@pytest.mark.parametrize("activation", [W.SWIGLU, W.GELU])
def test_ep_local_ffn_over_received_rows(activation):
    """The local grouped FFN reading the received rows in place through the
    gather map (ragged counts, empty pairs) against the oracle, expert by
    expert on the oracle's expert-major rows."""
    print(f"[ep local ffn] activation={activation}", flush=True)
    R, El, D, F = 4, 6, 256, 320
    cfg = W.MoEConfig("ep_local", 64, D, El, 2, F, activation=activation)
    rc = _recv_counts(R, El, 11, hi=90)
    total = int(rc.sum())
    rng = np.random.default_rng(12)
    xr = W.f32_to_bf16_bits(rng.standard_normal((total, D), dtype=np.float32))
    experts = [W.make_expert(cfg, e) for e in range(El)]
    w13 = to_torch(np.stack([a for a, _ in experts]), "cuda")
    w2 = to_torch(np.stack([b for _, b in experts]), "cuda")
    lo = torch.empty(El + 1, dtype=torch.int32, device="cuda")
    g = torch.empty(total, dtype=torch.int32, device="cuda")
    M.moe_ep_recv_layout(to_torch(rc, "cuda"), total, lo, g)
    y = torch.empty((total, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(M.moe_workspace_size(cfg.replace(num_tokens=total, top_k=1), M.MOE_OP_EXPERT_FFN) + 256,
                     dtype=torch.uint8, device="cuda")
    M.moe_expert_ffn(cfg, El, F, activation, total, to_torch(xr, "cuda"), g, lo, w13, w2, y, ws)
    torch.cuda.synchronize()
    lay = O.ep_recv_layout(rc)
    got = to_numpy(y)
    errs = []
    for e in range(El):
        a, b = lay["local_offsets"][e], lay["local_offsets"][e + 1]
        if a == b:
            continue
        X = O.widen(xr[lay["gather"][a:b]])
        ref = O.expert_apply(X, experts[e][0], experts[e][1], activation, F)
        errs.append(row_rel_err(got[a:b], ref))
    err = max(errs)
    print(f"  max rel err {err:.3e}")
    assert err <= BF16_TOL


# --------------------------------------------------------------------------
# expert-choice routing
# --------------------------------------------------------------------------
EC_SHAPES = [
    W.MoEConfig("ec_swiglu", 700, 256, 8, 2, 320, zipf_s=1.0),
    W.MoEConfig("ec_many_experts_shared", 333, 128, 64, 6, 128, num_shared=2, d_ff_shared=64),
    W.MoEConfig("ec_gelu_f32_router", 500, 192, 16, 1, 256, activation=W.GELU, router_dtype=W.F32),
    W.MoEConfig("ec_fp32_shared", 150, 96, 12, 3, 100, num_shared=3, d_ff_shared=20, act_dtype=W.F32,
                router_dtype=W.F32),
    W.MoEConfig("ec_capacity_factor", 257, 64, 5, 2, 48, capacity_factor=1.5),
    W.MoEConfig("ec_every_token", 40, 64, 4, 4, 64),
    W.MoEConfig("ec_256_experts", 600, 64, 256, 8, 64, scoring=W.SIGMOID_BIAS, zipf_s=1.2),
    W.MoEConfig("ec_max_tokens", 8192, 64, 4, 1, 32),
    W.MoEConfig("ec_one_token", 1, 64, 8, 2, 64),
]


@pytest.mark.parametrize("cfg", EC_SHAPES, ids=lambda c: c.name)
def test_expert_choice_matches_oracle(cfg):
    """Expert-choice layer: every expert's chosen tokens bit-exact against
    the oracle (near ties of the C-th probability exempt), gates within 1e-5
    of the float64 probabilities, unchosen-token count, and the outputs against
    the oracle evaluated on the GPU's choices."""
    print(f"[expert choice] {cfg.name}", flush=True)
    T, E, D = cfg.num_tokens, cfg.num_experts, cfg.d_model
    C = M.moe_expert_choice_capacity(cfg)
    assert C == O.expert_choice_capacity(cfg.capacity_factor, T, cfg.top_k, E)
    inp = W.make_inputs(cfg)
    ref = O.expert_choice_route(inp.x, inp.w_router, C)
    dev = "cuda"
    weights = dict(w_router=to_torch(inp.w_router, dev), w13=to_torch(inp.w13, dev), w2=to_torch(inp.w2, dev),
                   ws13=to_torch(inp.ws13, dev), ws2=to_torch(inp.ws2, dev))
    x = to_torch(inp.x, dev)
    y = torch.empty((T, D), dtype=act_torch_dtype(cfg), device=dev)
    tor = torch.empty(E * C, dtype=torch.int32, device=dev)
    rw = torch.empty(E * C, dtype=torch.float32, device=dev)
    uns = torch.empty(1, dtype=torch.int32, device=dev)
    ws = M.workspace(cfg, M.MOE_OP_EXPERT_CHOICE, dev)
    M.moe_expert_choice_forward(cfg, weights, x, y, tor, rw, uns, ws)
    torch.cuda.synchronize()
    tg = to_numpy(tor).astype(np.int64)
    ties = ec_check_selection(ref, tg, C)
    print(f"  C={C}, experts with a near-tie exchange: {ties}")
    p = ref["probs"]
    gates = p[tg, np.repeat(np.arange(E), C)]
    assert rel_err(to_numpy(rw), gates) <= W_TOL
    assert int(to_numpy(uns)[0]) == T - np.unique(tg).size
    if ties == 0:
        assert int(to_numpy(uns)[0]) == O.expert_choice_forward(
            cfg, inp.x, inp.w_router, lambda e: (inp.w13[e], inp.w2[e]), inp.shared)["unselected"]
    y_ref = ec_oracle_output(cfg, inp, tg, C)
    err = row_rel_err(to_numpy(y), y_ref)
    print(f"  max rel err {err:.3e}")
    assert err <= out_tol(cfg)


def test_expert_choice_deterministic():
    cfg = EC_SHAPES[1]
    inp = W.make_inputs(cfg)
    dev = "cuda"
    weights = dict(w_router=to_torch(inp.w_router, dev), w13=to_torch(inp.w13, dev), w2=to_torch(inp.w2, dev),
                   ws13=to_torch(inp.ws13, dev), ws2=to_torch(inp.ws2, dev))
    x = to_torch(inp.x, dev)
    ws = M.workspace(cfg, M.MOE_OP_EXPERT_CHOICE, dev)
    outs = []
    for _ in range(3):
        y = torch.empty((cfg.num_tokens, cfg.d_model), dtype=torch.bfloat16, device=dev)
        M.moe_expert_choice_forward(cfg, weights, x, y, ws=ws)
        torch.cuda.synchronize()
        outs.append(to_numpy(y))
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


# --------------------------------------------------------------------------
# backward pass
# --------------------------------------------------------------------------
BW_SHAPES = [
    W.MoEConfig("bw_switch", 300, 128, 16, 1, 192, scoring=W.SOFTMAX_TOPK, renormalize=0, activation=W.GELU,
                router_dtype=W.F32, capacity_factor=1.25),
    W.MoEConfig("bw_mixtral", 256, 256, 8, 2, 320, scoring=W.TOPK_SOFTMAX, zipf_s=1.0),
    W.MoEConfig("bw_deepseekmoe", 200, 128, 32, 6, 128, num_shared=2, d_ff_shared=64, scoring=W.SOFTMAX_TOPK,
                renormalize=1),
    W.MoEConfig("bw_deepseekv3", 333, 192, 64, 8, 128, num_shared=1, d_ff_shared=128, scoring=W.SIGMOID_BIAS,
                renormalize=1, zipf_s=1.2),
    W.MoEConfig("bw_sigmoid_raw_capacity", 150, 64, 8, 2, 96, scoring=W.SIGMOID_BIAS, renormalize=0,
                capacity_factor=0.8),
    # E not a multiple of 4: the router gradients take the float32 path
    W.MoEConfig("bw_six_experts", 96, 64, 6, 2, 64, scoring=W.SOFTMAX_TOPK, renormalize=1),
]
# Gradient tolerance (none is stated for the backward): the forward's 2e-2
# covers a chain of three bf16 roundings (H, y_perm, y); the input gradient
# passes six (dy_perm, the recomputed G and U, dH, dG / dU, dx_perm, dx) and the
# weight gradients up to five, so the bar scales to 4e-2.
BW_TOL = 4e-2


def tensor_rel_err(g: np.ndarray, r: np.ndarray) -> float:
    """|gpu - ref| over max(|ref|, rms of the whole reference tensor): a
    weight gradient of an expert with few rows is (near) rank-one, so one of
    its rows can be a cancelling dot product whose own scale says nothing
    about the tensor's."""
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt((r ** 2).mean()))
    den = np.maximum(np.abs(r), rms if rms > 0 else 1.0)
    return float((np.abs(g.astype(np.float64) - r) / den).max())


@pytest.mark.parametrize("cfg", BW_SHAPES, ids=lambda c: c.name)
def test_layer_backward_matches_oracle(cfg):
    """Every gradient of moe_layer_backward (input, router, routed and shared
    expert weights) against the float64 oracle backward on the same routing:
    the input gradient row by row (each row is a token), each weight gradient
    against the scale of its whole tensor (bf16 intermediates, float32
    accumulation)."""
    print(f"[backward] {cfg.name}", flush=True)
    T, E, D, F, k = cfg.num_tokens, cfg.num_experts, cfg.d_model, cfg.d_ff, cfg.top_k
    alpha = 0.05
    inp = W.make_inputs(cfg)
    rng = np.random.default_rng(5)
    dy_h = W.f32_to_bf16_bits(rng.standard_normal((T, D), dtype=np.float32))
    ref = O.backward(cfg, inp.x, inp.w_router, inp.sel_bias, lambda e: (inp.w13[e], inp.w2[e]), inp.shared, dy_h,
                     alpha=alpha)
    dl = DeviceLayer(cfg, inp)
    got_route = dl.layer()
    assert np.array_equal(got_route["idx"], ref["forward"]["idx"]), "routing differs (near tie): pick another seed"
    dev = "cuda"
    nF = cfg.n_mat * F
    SF = cfg.num_shared * cfg.d_ff_shared
    dx = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    dwr = torch.empty((E, D), dtype=torch.float32, device=dev)
    dw13 = torch.empty((E, nF, D), dtype=torch.float32, device=dev)
    dw2 = torch.empty((E, D, F), dtype=torch.float32, device=dev)
    dws13 = torch.empty((2 * SF, D), dtype=torch.float32, device=dev) if SF else None
    dws2 = torch.empty((D, SF), dtype=torch.float32, device=dev) if SF else None
    ws = M.workspace(cfg, M.MOE_OP_LAYER_BACKWARD, dev)
    M.moe_layer_backward(cfg, dl.weights, dl.x, to_torch(dy_h, dev), alpha, dx, dwr, dw13, dw2, dws13, dws2, ws)
    torch.cuda.synchronize()
    errs = {"dx": row_rel_err(to_numpy(dx), ref["dx"]), "dw_router": tensor_rel_err(to_numpy(dwr), ref["dw_router"])}
    g13, g2 = to_numpy(dw13), to_numpy(dw2)
    e13 = e2 = 0.0
    for e in range(E):
        r13 = ref["dw13"].get(e, np.zeros((nF, D)))
        r2 = ref["dw2"].get(e, np.zeros((D, F)))
        if e in ref["dw13"]:
            e13 = max(e13, tensor_rel_err(g13[e], r13))
            e2 = max(e2, tensor_rel_err(g2[e], r2))
        else:
            assert (g13[e] == 0).all() and (g2[e] == 0).all(), f"expert {e} without rows has a gradient"
    errs["dw13"], errs["dw2"] = e13, e2
    if SF:
        rg = np.concatenate([np.concatenate([a for a, _, _ in ref["dshared"]], axis=0),
                             np.concatenate([b for _, b, _ in ref["dshared"]], axis=0)], axis=0)
        rd = np.concatenate([c for _, _, c in ref["dshared"]], axis=1)
        errs["dws13"] = tensor_rel_err(to_numpy(dws13), rg)
        errs["dws2"] = tensor_rel_err(to_numpy(dws2), rd)
    print("  " + ", ".join(f"{n} {v:.2e}" for n, v in errs.items()))
    for n, v in errs.items():
        assert v <= BW_TOL, f"{n}: {v:.3e}"


@pytest.mark.parametrize("cfg", [BW_SHAPES[1], BW_SHAPES[3]], ids=lambda c: c.name)
def test_weight_gradient_variants_identical(cfg):
    """The weight-gradient kernel's tile size (256x256 on eight waves or
    128x128 on four) and its LDS chunk permutation change where partial
    products are staged, not the order in which any output adds its rows:
    every gradient must be bit-identical across the variants (the narrow
    DeepSeek-V3-shaped case runs 128x128 by default, so forcing 256x256
    also covers partial tiles)."""
    print(f"[backward variants] {cfg.name}", flush=True)
    T, E, D, F = cfg.num_tokens, cfg.num_experts, cfg.d_model, cfg.d_ff
    inp = W.make_inputs(cfg)
    rng = np.random.default_rng(9)
    dy = to_torch(W.f32_to_bf16_bits(rng.standard_normal((T, D), dtype=np.float32)), "cuda")
    dl = DeviceLayer(cfg, inp)
    nF = cfg.n_mat * F
    SF = cfg.num_shared * cfg.d_ff_shared
    ws = M.workspace(cfg, M.MOE_OP_LAYER_BACKWARD, "cuda")

    def run(env):
        old = {k: os.environ.get(k) for k in env}
        os.environ.update(env)
        M.moe_reload_tuning()
        try:
            out = dict(dx=torch.empty((T, D), dtype=torch.bfloat16, device="cuda"),
                       dwr=torch.empty((E, D), dtype=torch.float32, device="cuda"),
                       dw13=torch.empty((E, nF, D), dtype=torch.float32, device="cuda"),
                       dw2=torch.empty((E, D, F), dtype=torch.float32, device="cuda"),
                       dws13=torch.empty((2 * SF, D), dtype=torch.float32, device="cuda") if SF else None,
                       dws2=torch.empty((D, SF), dtype=torch.float32, device="cuda") if SF else None)
            M.moe_layer_backward(cfg, dl.weights, dl.x, dy, 0.05, out["dx"], out["dwr"], out["dw13"], out["dw2"],
                                 out["dws13"], out["dws2"], ws)
            torch.cuda.synchronize()
            return {n: to_numpy(t) for n, t in out.items() if t is not None}
        finally:
            for k, v in old.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
            M.moe_reload_tuning()

    base = run({})
    for env in ({"MOE_WGRAD_SWZ": "0"}, {"MOE_WGRAD_SWZ": "1"}, {"MOE_WGRAD_TILE": "128"},
                {"MOE_WGRAD_TILE": "256"}):
        got = run(env)
        for n in base:
            assert np.array_equal(got[n].view(np.uint8), base[n].view(np.uint8)), f"{env}: {n} differs"


# --------------------------------------------------------------------------
# MOE_DEBUG: host-side checks of the dispatch tables
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [SMALL[1], SMALL[3], SMALL[5], EDGE[5]], ids=lambda c: c.name)
def test_debug_checks_pass_on_the_staged_path(cfg, monkeypatch):
    """With MOE_DEBUG=1 the staged layer and moe_permute check their tables
    on the host and still return the oracle's results."""
    set_env(monkeypatch, "MOE_DEBUG", "1")
    set_env(monkeypatch, "MOE_FUSED", "0")
    print(f"[debug checks] {cfg.name}", flush=True)
    inp = W.make_inputs(cfg)
    ref = oracle_forward(cfg, inp)
    dl = DeviceLayer(cfg, inp)
    check_layer(cfg, inp, ref, dl.layer())
    T, k, E = cfg.num_tokens, cfg.top_k, cfg.num_experts
    cap, rows_cap = M.moe_capacity(cfg)
    idx = to_torch(ref["idx"].astype(np.int32), "cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    row_of = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tor = torch.empty(rows_cap, dtype=torch.int32, device="cuda")
    ws = M.workspace(cfg, M.MOE_OP_PERMUTE, "cuda")
    M.moe_permute(cfg, idx, None, counts, offsets, row_of, tor, None, ws)
    torch.cuda.synchronize()


def test_debug_checks_reject_bad_tables_before_launch(monkeypatch):
    """MOE_DEBUG=1 turns caller tables out of range into MOE_ERR_DEBUG_CHECK
    before any launch.  Every buffer has room for the bad rows as well, so
    the call stays within its memory even if a check did not fire."""
    set_env(monkeypatch, "MOE_DEBUG", "1")
    cfg = W.MoEConfig("debug_tables", 64, 64, 4, 2, 32)
    dev = "cuda"
    G, F, D, rows, slack = 4, 32, 64, 128, 64
    x = torch.zeros(((rows + slack) * D,), dtype=torch.bfloat16, device=dev)
    y = torch.zeros(((rows + slack) * D,), dtype=torch.bfloat16, device=dev)
    w13 = torch.zeros((G * 2 * F * D,), dtype=torch.bfloat16, device=dev)
    w2 = torch.zeros((G * D * F,), dtype=torch.bfloat16, device=dev)
    need = M.moe_workspace_size(cfg.replace(num_tokens=(rows + slack) * 2), M.MOE_OP_EXPERT_FFN)
    ws = torch.empty(4 * need + (1 << 20), dtype=torch.uint8, device=dev)
    good = torch.tensor([0, 32, 64, 96, rows], dtype=torch.int32, device=dev)
    M.moe_expert_ffn(cfg, G, F, M.MOE_SWIGLU, rows, x, None, good, w13, w2, y, ws)
    torch.cuda.synchronize()
    past = torch.tensor([0, 32, 64, 96, rows + 16], dtype=torch.int32, device=dev)
    with pytest.raises(M.MoEError, match="exceeds max_rows") as e:
        M.moe_expert_ffn(cfg, G, F, M.MOE_SWIGLU, rows, x, None, past, w13, w2, y, ws)
    assert e.value.status == M.MOE_ERR_DEBUG_CHECK
    gather = torch.zeros(rows + slack, dtype=torch.int32, device=dev)
    gather[5] = -1
    x_after_one_row = x.view(rows + slack, D)[1:].reshape(-1)   # row -1 of it is still x's first row
    with pytest.raises(M.MoEError, match=r"gather_rows\[5\]"):
        M.moe_expert_ffn(cfg, G, F, M.MOE_SWIGLU, rows, x_after_one_row, gather, good, w13, w2, y, ws)
    T, k = cfg.num_tokens, cfg.top_k
    _, rows_cap = M.moe_capacity(cfg)
    y_perm = torch.zeros(((rows_cap + slack) * D,), dtype=torch.bfloat16, device=dev)
    row_of = torch.arange(T * k, dtype=torch.int32, device=dev).reshape(T, k)
    row_of[7, 1] = rows_cap + 3
    tw = torch.full((T, k), 0.5, dtype=torch.float32, device=dev)
    out = torch.zeros((T, D), dtype=torch.bfloat16, device=dev)
    with pytest.raises(M.MoEError, match=r"row_of\[15\]") as e:
        M.moe_combine(cfg, y_perm, row_of, tw, None, out)
    assert e.value.status == M.MOE_ERR_DEBUG_CHECK
    torch.cuda.synchronize()
