"""The host-side dispatch check (moe_check_dispatch, what MOE_DEBUG=1 runs on
copies of the device tables) on the CPU: tables built by the oracle's
dispatch ("从 Dense FFN 到 MoE" §5 batches, "Top-k 路由" 容量因子) pass, and
each kind of corruption is caught with a message naming the entry."""
import numpy as np
import pytest

import top_routing_dispatch_amd as M
import workloads as W
from oracle import moe_oracle as O


def _tables(cfg, idx):
    """counts, offsets, row_of and token_of_row [A_cap] (-1 past the kept
    rows) from the oracle's dispatch."""
    cap, rows_cap = M.moe_capacity(cfg)
    disp = O.dispatch(idx, cfg.num_experts, O.capacity(cfg.capacity_factor, cfg.num_tokens, cfg.top_k,
                                                       cfg.num_experts))
    tor = np.full(rows_cap, -1, dtype=np.int32)
    tor[: len(disp["token_of_row"])] = disp["token_of_row"]
    return dict(idx=idx.astype(np.int32), counts=disp["counts"].astype(np.int32),
                offsets=disp["offsets"].astype(np.int32), row_of=disp["row_of"].astype(np.int32), tor=tor)


def _random_idx(cfg, seed):
    """Distinct experts per token with a skew, like a router's choice."""
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, cfg.num_experts + 1) ** 1.1
    p /= p.sum()
    return np.stack([rng.choice(cfg.num_experts, cfg.top_k, replace=False, p=p) for _ in range(cfg.num_tokens)])


def _check(cfg, t):
    M.moe_check_dispatch(cfg, t["idx"], t["counts"], t["offsets"], t["row_of"], t["tor"])


CFGS = [W.MoEConfig("dropless", 97, 64, 12, 3, 32),
        W.MoEConfig("capacity", 120, 64, 8, 2, 32, capacity_factor=0.75),
        W.MoEConfig("top1_capacity", 64, 64, 4, 1, 32, capacity_factor=1.0)]


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_oracle_dispatch_passes(cfg):
    t = _tables(cfg, _random_idx(cfg, 1))
    if cfg.capacity_factor > 0:
        assert (t["row_of"] < 0).any(), "the case must drop assignments"
    _check(cfg, t)


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
@pytest.mark.parametrize("mistake", ["count", "offset", "row_swap", "row_past_end", "dropped_kept", "kept_dropped",
                                     "token", "tail_not_cleared"])
def test_corrupted_tables_fail(cfg, mistake):
    t = _tables(cfg, _random_idx(cfg, 2))
    kept = np.argwhere(t["row_of"] >= 0)
    if mistake == "count":
        t["counts"][3] += 1
        pat = "counts"
    elif mistake == "offset":
        t["offsets"][2] += 1
        pat = "offsets"
    elif mistake == "row_swap":
        (a, b), (c, d) = kept[0], kept[1]
        t["row_of"][a, b], t["row_of"][c, d] = t["row_of"][c, d], t["row_of"][a, b]
        pat = "row_of"
    elif mistake == "row_past_end":
        a, b = kept[-1]
        t["row_of"][a, b] = t["offsets"][-1]
        pat = "row_of"
    elif mistake == "dropped_kept":
        a, b = kept[0]
        t["row_of"][a, b] = -1
        pat = "row_of"
    elif mistake == "kept_dropped":
        drops = np.argwhere(t["row_of"] < 0)
        if len(drops) == 0:
            pytest.skip("dropless: nothing is dropped")
        a, b = drops[0]
        t["row_of"][a, b] = 0
        pat = "row_of"
    elif mistake == "token":
        t["tor"][0] = (t["tor"][0] + 1) % cfg.num_tokens
        pat = "token_of_row"
    else:
        if t["offsets"][-1] == len(t["tor"]):
            pytest.skip("every row is kept: no tail")
        t["tor"][-1] = 0
        pat = "token_of_row"
    with pytest.raises(M.MoEError, match=pat) as e:
        _check(cfg, t)
    assert e.value.status == M.MOE_ERR_DEBUG_CHECK


def test_invalid_and_repeated_ids_are_skipped():
    """Ids outside [0, E) and a repeat of an id an earlier slot of the token
    used are not dispatched: row -1, not counted (worked by hand)."""
    cfg = W.MoEConfig("hand", 4, 64, 3, 2, 32)
    idx = np.array([[0, 2], [2, 2], [-1, 1], [3, 0]], dtype=np.int32)
    counts = np.array([2, 1, 2], dtype=np.int32)              # e0: t0, t3; e1: t2; e2: t0, t1
    offsets = np.array([0, 2, 3, 5], dtype=np.int32)
    row_of = np.array([[0, 3], [4, -1], [-1, 2], [-1, 1]], dtype=np.int32)
    tor = np.array([0, 3, 2, 0, 1, -1, -1, -1], dtype=np.int32)
    M.moe_check_dispatch(cfg, idx, counts, offsets, row_of, tor)
    bad = row_of.copy()
    bad[1, 1] = 5                                              # the repeated id given a row
    with pytest.raises(M.MoEError, match=r"row_of\[1\]\[1\]"):
        M.moe_check_dispatch(cfg, idx, counts, offsets, bad, tor)
    with pytest.raises(M.MoEError, match=r"counts\[2\]"):
        M.moe_check_dispatch(cfg, idx, np.array([2, 1, 3], dtype=np.int32), offsets, row_of, tor)
