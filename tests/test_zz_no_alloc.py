"""The allocation-free layer forward (moe_layer_forward_static): it runs in the
library's static device scratch and must give what moe_layer_forward gives
with a caller-owned workspace, call after call on the same scratch (the
second call smaller than the first, so stale contents of the first call
would show), and reject shapes whose workspace exceeds the scratch before
launching anything."""
import numpy as np
import pytest
import torch

import top_routing_dispatch_amd as M
import workloads as W
from workloads.torch_io import act_torch_dtype, to_numpy

from parity import DeviceLayer, check_layer, oracle_forward

CALLS = [
    # larger first: shared expert, sigmoid + bias, skewed routing, ragged sizes
    W.MoEConfig("static_large", 700, 256, 16, 4, 320, num_shared=1, d_ff_shared=128, scoring=W.SIGMOID_BIAS,
                zipf_s=1.0),
    # then smaller: GELU, capacity drops, float32 router weight
    W.MoEConfig("static_small", 97, 128, 8, 2, 192, scoring=W.SOFTMAX_TOPK, renormalize=0, activation=W.GELU,
                router_dtype=W.F32, capacity_factor=1.0),
]


def _outputs(cfg, dev):
    T, E, k, D = cfg.num_tokens, cfg.num_experts, cfg.top_k, cfg.d_model
    return dict(y=torch.full((T, D), 7.0, dtype=act_torch_dtype(cfg), device=dev),
                idx=torch.full((T, k), -5, dtype=torch.int32, device=dev),
                w=torch.full((T, k), -1.0, dtype=torch.float32, device=dev),
                counts=torch.full((E,), -3, dtype=torch.int32, device=dev),
                stats=torch.full((2 * E + 2,), -1.0, dtype=torch.float32, device=dev),
                dropped=torch.full((1,), -9, dtype=torch.int32, device=dev))


@pytest.mark.gpu
def test_static_scratch_matches_workspace_forward_call_after_call():
    dev = "cuda"
    for cfg in CALLS:
        print(f"[static scratch] {cfg.name}", flush=True)
        assert M.moe_workspace_size(cfg, M.MOE_OP_LAYER) <= M.MOE_STATIC_SCRATCH_BYTES
        inp = W.make_inputs(cfg)
        dl = DeviceLayer(cfg, inp, device=dev)
        want = dl.layer()                                   # caller-owned workspace
        o = _outputs(cfg, dev)
        M.moe_layer_forward_static(cfg, dl.weights, dl.x, o["y"], o["idx"], o["w"], o["counts"], cfg.alpha,
                                   o["stats"], o["dropped"])
        torch.cuda.synchronize()
        got = {key: to_numpy(t) for key, t in o.items()}
        got["dropped"] = int(got["dropped"][0])
        for key in ("y", "idx", "w", "counts", "stats"):
            np.testing.assert_array_equal(got[key], want[key], err_msg=f"{cfg.name}: {key}")
        assert got["dropped"] == want["dropped"]
        diff, err = check_layer(cfg, inp, oracle_forward(cfg, inp), got)
        print(f"  identical to the workspace call; against the oracle: max rel err {err:.3e}, "
              f"near-tie tokens {len(diff)}")


def test_static_scratch_rejects_large_shapes_before_launch():
    """The DeepSeek-V3-shaped batch needs about 1.2 GB of workspace: rejected
    on the host (no GPU is touched) with both sizes in the message."""
    import ctypes
    from top_routing_dispatch_amd import binding as B
    c = B.make_config(W.DEEPSEEKV3)
    p = ctypes.c_void_p(0x100000)            # never dereferenced: the size check fails first
    w = B.moe_weights(p.value, p.value, p.value, p.value, p.value, p.value)
    st = M.lib().moe_layer_forward_static(ctypes.byref(c), ctypes.byref(w), p, p, None, None, None,
                                          ctypes.c_float(1e-4), None, None, None)
    assert st == M.MOE_ERR_WORKSPACE_TOO_SMALL
    msg = M.lib().moe_last_error().decode()
    assert "needs" in msg and str(M.MOE_STATIC_SCRATCH_BYTES) in msg
