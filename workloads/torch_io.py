"""Move seeded host workloads onto the GPU as torch tensors (input plumbing only)."""
from __future__ import annotations

import numpy as np
import torch

from . import BF16, HostInputs, MoEConfig, iter_experts


def to_torch(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy -> torch on `device`; uint16 arrays are bfloat16 bit patterns."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """torch -> numpy; bfloat16 comes back as uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def act_torch_dtype(cfg: MoEConfig):
    return torch.bfloat16 if cfg.act_dtype == BF16 else torch.float32


def device_weights(inp: HostInputs, device="cuda") -> dict:
    return dict(w_router=to_torch(inp.w_router, device), sel_bias=to_torch(inp.sel_bias, device),
                w13=to_torch(inp.w13, device), w2=to_torch(inp.w2, device),
                ws13=to_torch(inp.ws13, device), ws2=to_torch(inp.ws2, device))


def upload_experts(cfg: MoEConfig, device="cuda", keep_host: bool = False, workers: int = 16, progress=None):
    """Generate the routed expert weights expert by expert and copy them into
    device tensors w13 [E, n_mat*F, D], w2 [E, D, F] without holding all of them
    on the host (unless keep_host)."""
    dt = act_torch_dtype(cfg)
    w13 = torch.empty((cfg.num_experts, cfg.n_mat * cfg.d_ff, cfg.d_model), dtype=dt, device=device)
    w2 = torch.empty((cfg.num_experts, cfg.d_model, cfg.d_ff), dtype=dt, device=device)
    host = {} if keep_host else None
    for e, a, b in iter_experts(cfg, workers=workers):
        w13[e].copy_(to_torch(a, "cpu"))
        w2[e].copy_(to_torch(b, "cpu"))
        if keep_host:
            host[e] = (a, b)
        if progress is not None and (e + 1) % 32 == 0:
            progress(e + 1)
    return w13, w2, host
