"""Seeded synthetic workloads for the sparse-MoE layer forward.

This module only *makes inputs*: layer shapes, seeded random tensors and the
bfloat16 encoding of those tensors.  It holds none of the layer's arithmetic
(no routing, no scoring, no expert math), so both the CPU oracle and the GPU
path can consume exactly the same bytes without sharing any code of the method.

Shapes follow the model families that the pages tabulate:
  * the Tiny MoE walk-through ("从 Dense FFN 到 MoE", §3 expert, §4 Router: D=32,
    F=48, four experts, top-2);
  * Switch Transformer (top-1, capacity factor, "Top-k 路由" page, model table
    and 容量因子 section);
  * Mixtral 8x7B, DeepSeekMoE-16B and DeepSeek-V3 ("别只比较 Top-k" page,
    six-family table; "Top-K Routing (MoE)" glossary, parameter table).
Hidden sizes D and F of the four large shapes are the workload's own choice;
the pages give D and F only for the Tiny model.

Random streams: numpy PCG64 seeded through ``SeedSequence(seed).spawn``.  Child
streams, in order: 0 tokens x, 1 router weight, 2 skew permutation, 3 selection
bias, then one child per routed expert and one per shared expert (each of those
spawns gate / up / down grand-children so an expert can be regenerated alone).
Floating samples are drawn in float32; bfloat16 tensors are the
round-to-nearest-even encoding of those samples, kept as uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

# enum values mirror include/moe.h
SOFTMAX_TOPK, TOPK_SOFTMAX, SIGMOID_BIAS = 0, 1, 2
SWIGLU, GELU = 0, 1
F32, BF16 = 0, 1

WEIGHT_STD = 0.02   # "weights ~ N(0, 0.02)": read as standard deviation 0.02
BIAS_RANGE = 0.1    # selection bias ~ U(-0.1, 0.1)


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    num_tokens: int          # T
    d_model: int             # D
    num_experts: int         # E
    top_k: int               # k
    d_ff: int                # F
    num_shared: int = 0      # S
    d_ff_shared: int = 0     # F_s
    scoring: int = SOFTMAX_TOPK
    renormalize: int = 1
    activation: int = SWIGLU
    act_dtype: int = BF16
    router_dtype: int = BF16
    capacity_factor: float = 0.0     # <= 0 : dropless
    zipf_s: float = 0.0              # 0 : no skew
    alpha: float = 0.01              # balance-loss coefficient
    seed: int = 0

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)

    @property
    def n_mat(self) -> int:
        """Input-side matrices per expert: gate+up for SwiGLU, one for GELU."""
        return 2 if self.activation == SWIGLU else 1


TINY = MoEConfig("tiny", 64, 32, 4, 2, 48, scoring=SOFTMAX_TOPK, renormalize=1,
                 activation=SWIGLU, act_dtype=F32, router_dtype=F32)
SWITCH = MoEConfig("switch", 8192, 768, 128, 1, 3072, scoring=SOFTMAX_TOPK,
                   renormalize=0, activation=GELU, act_dtype=BF16,
                   router_dtype=F32, capacity_factor=1.25)
MIXTRAL = MoEConfig("mixtral", 4096, 4096, 8, 2, 14336, scoring=TOPK_SOFTMAX,
                    activation=SWIGLU, zipf_s=1.0)
DEEPSEEKMOE = MoEConfig("deepseekmoe", 4096, 2048, 64, 6, 1408, num_shared=2,
                        d_ff_shared=1408, scoring=SOFTMAX_TOPK, renormalize=1)
DEEPSEEKV3 = MoEConfig("deepseekv3", 8192, 7168, 256, 8, 2048, num_shared=1,
                       d_ff_shared=2048, scoring=SIGMOID_BIAS, renormalize=1,
                       zipf_s=1.2, alpha=1e-4)

CONFIGS = {c.name: c for c in (TINY, SWITCH, MIXTRAL, DEEPSEEKMOE, DEEPSEEKV3)}

# Decode-shaped batches: the first T tokens of a workload with its full-size
# weights (token generation runs the layer on a handful of tokens per step,
# where the expert matrices are read for very few rows each).
DECODE_TOKENS = (1, 8, 64, 256)
DECODE_SEP = "_decode_t"


def decode_config(cfg: MoEConfig, tokens: int) -> MoEConfig:
    return cfg.replace(name=f"{cfg.name}{DECODE_SEP}{tokens}", num_tokens=tokens)


def base_name(cfg: MoEConfig) -> str:
    """The workload whose weights a (decode-shaped or expert-choice)
    configuration uses."""
    name = cfg.name.split(DECODE_SEP)[0]
    return name[:-len("_ec")] if name.endswith("_ec") else name


DECODE_CONFIGS = {d.name: d for d in (decode_config(CONFIGS[n], t) for n in ("mixtral", "deepseekv3")
                                      for t in DECODE_TOKENS)}


# Expert-choice routing at the shapes of three workloads: the same tokens,
# weights and expert FFNs; each expert takes C = T k / E tokens (k read as the
# average experts per token; the scoring mode of the workload is not used).
EC_SUFFIX = "_ec"
EC_CONFIGS = {c.name + EC_SUFFIX: c.replace(name=c.name + EC_SUFFIX, capacity_factor=0.0)
              for c in (MIXTRAL, DEEPSEEKMOE, DEEPSEEKV3)}


@dataclasses.dataclass(frozen=True)
class EpShare:
    """One GPU's share of an expert-parallel layer: the experts of `rank` out
    of `ranks` contiguous blocks of the base workload's routed experts, and
    the rows the dispatch all-to-all delivers to it."""
    name: str
    base: str              # workload whose shapes and expert weights are used
    ranks: int
    rank: int
    rows_per_pair: int     # rows each source rank sends for each local expert

    @property
    def local_experts(self) -> int:
        return CONFIGS[self.base].num_experts // self.ranks


# DeepSeek-V3-shaped layer on 8 GPUs: 32 local experts; 8 ranks x 8192 tokens
# x top-8 assignments spread evenly give 2,048 rows per expert, 256 from each
# source rank (65,536 received rows).
EP_CONFIGS = {e.name: e for e in (EpShare("deepseekv3_ep8_local", "deepseekv3", 8, 0, 256),)}


def ep_recv_counts(ep: EpShare) -> np.ndarray:
    """Rows per (source rank, local expert): the even split of the recipe."""
    return np.full((ep.ranks, ep.local_experts), ep.rows_per_pair, dtype=np.int32)


def make_received_rows(ep: EpShare, n_rows: int) -> np.ndarray:
    """Received activation rows [n_rows, D] ~ N(0, 1) in bf16, from a stream
    of their own (the child after the base workload's expert streams)."""
    cfg = CONFIGS[ep.base]
    ss = np.random.SeedSequence(cfg.seed).spawn(4 + cfg.num_experts + cfg.num_shared + 1)[-1]
    return _encode(_normal(ss, (n_rows, cfg.d_model)), cfg.act_dtype)


# --------------------------------------------------------------------------
# bfloat16 encoding (input preparation only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16, returned as uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _encode(a: np.ndarray, dtype: int) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == BF16 else np.ascontiguousarray(a, dtype=np.float32)


# --------------------------------------------------------------------------
# stream layout
# --------------------------------------------------------------------------
def _streams(cfg: MoEConfig):
    root = np.random.SeedSequence(cfg.seed)
    return root.spawn(4 + cfg.num_experts + cfg.num_shared)


def _rng(ss) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


def _normal(ss, shape, std=1.0) -> np.ndarray:
    a = _rng(ss).standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if std != 1.0:
        a *= np.float32(std)
    return a


def zipf_channel(cfg: MoEConfig, perm: np.ndarray) -> np.ndarray:
    """Router-weight column on the constant input channel that realises a Zipf(s)
    preference over experts (input structure only): expert of preference rank r
    gets log-offset -s*ln(r+1), scaled by tau = sigma*sqrt(6)/pi so that the
    Gaussian noise logit of std sigma = 0.02*sqrt(D-1) acts like a Gumbel of
    scale tau."""
    sigma = WEIGHT_STD * math.sqrt(cfg.d_model - 1)
    tau = sigma * math.sqrt(6.0) / math.pi
    col = tau * (-cfg.zipf_s * np.log(perm.astype(np.float64) + 1.0))
    return col.astype(np.float32)


def make_tokens(cfg: MoEConfig) -> np.ndarray:
    s = _streams(cfg)
    x = _normal(s[0], (cfg.num_tokens, cfg.d_model))
    if cfg.zipf_s > 0:
        x[:, cfg.d_model - 1] = 1.0
    return _encode(x, cfg.act_dtype)


def make_router(cfg: MoEConfig) -> np.ndarray:
    s = _streams(cfg)
    w = _normal(s[1], (cfg.num_experts, cfg.d_model), WEIGHT_STD)
    if cfg.zipf_s > 0:
        perm = _rng(s[2]).permutation(cfg.num_experts)
        w[:, cfg.d_model - 1] = zipf_channel(cfg, perm)
    return _encode(w, cfg.router_dtype)


def make_bias(cfg: MoEConfig) -> Optional[np.ndarray]:
    if cfg.scoring != SIGMOID_BIAS:
        return None
    s = _streams(cfg)
    return _rng(s[3]).uniform(-BIAS_RANGE, BIAS_RANGE, cfg.num_experts).astype(np.float32)


def make_expert(cfg: MoEConfig, e: int):
    """Routed expert e: (w13 [n_mat*F, D], w2 [D, F]) in the activation dtype.
    SwiGLU: w13 rows 0..F-1 are the gate projection, F..2F-1 the up projection.
    GELU: w13 is the input projection [F, D]."""
    s = _streams(cfg)[4 + e].spawn(3)
    F, D = cfg.d_ff, cfg.d_model
    mats = [_normal(s[i], (F, D), WEIGHT_STD) for i in range(cfg.n_mat)]
    w13 = np.concatenate(mats, axis=0) if len(mats) > 1 else mats[0]
    w2 = _normal(s[2], (D, F), WEIGHT_STD)
    return _encode(w13, cfg.act_dtype), _encode(w2, cfg.act_dtype)


def make_shared_expert(cfg: MoEConfig, i: int):
    """Shared expert i: (gate [F_s, D], up [F_s, D], down [D, F_s])."""
    s = _streams(cfg)[4 + cfg.num_experts + i].spawn(3)
    Fs, D = cfg.d_ff_shared, cfg.d_model
    g = _normal(s[0], (Fs, D), WEIGHT_STD)
    u = _normal(s[1], (Fs, D), WEIGHT_STD)
    d = _normal(s[2], (D, Fs), WEIGHT_STD)
    return _encode(g, cfg.act_dtype), _encode(u, cfg.act_dtype), _encode(d, cfg.act_dtype)


def pack_shared(cfg: MoEConfig, shared):
    """Concatenate S shared SwiGLU experts into the one-expert layout the library
    takes: ws13 [2*S*F_s, D] = [gate_0; ...; gate_{S-1}; up_0; ...; up_{S-1}],
    ws2 [D, S*F_s] = [down_0 | ... | down_{S-1}] (a pure re-layout of bytes)."""
    if not shared:
        return None, None
    ws13 = np.concatenate([g for g, _, _ in shared] + [u for _, u, _ in shared], axis=0)
    ws2 = np.concatenate([d for _, _, d in shared], axis=1)
    return np.ascontiguousarray(ws13), np.ascontiguousarray(ws2)


def iter_experts(cfg: MoEConfig, experts=None, workers: int = 8):
    """Yield (e, w13, w2) for every routed expert, generating in a thread pool
    (numpy's generators release the GIL while filling arrays)."""
    ids = list(range(cfg.num_experts)) if experts is None else list(experts)
    with ThreadPoolExecutor(max(1, workers)) as ex:
        for e, (w13, w2) in zip(ids, ex.map(lambda i: make_expert(cfg, i), ids)):
            yield e, w13, w2


@dataclasses.dataclass
class HostInputs:
    cfg: MoEConfig
    x: np.ndarray
    w_router: np.ndarray
    sel_bias: Optional[np.ndarray]
    w13: Optional[np.ndarray]       # [E, n_mat*F, D] (None when not materialised)
    w2: Optional[np.ndarray]        # [E, D, F]
    shared: list                    # [(gate, up, down)] * S
    ws13: Optional[np.ndarray]
    ws2: Optional[np.ndarray]


def make_inputs(cfg: MoEConfig, with_experts: bool = True, workers: int = 8) -> HostInputs:
    """All layer inputs on the host.  With ``with_experts=False`` the routed
    expert weights are not materialised (regenerate them with make_expert)."""
    x = make_tokens(cfg)
    wr = make_router(cfg)
    b = make_bias(cfg)
    w13 = w2 = None
    if with_experts:
        dt = np.uint16 if cfg.act_dtype == BF16 else np.float32
        w13 = np.empty((cfg.num_experts, cfg.n_mat * cfg.d_ff, cfg.d_model), dtype=dt)
        w2 = np.empty((cfg.num_experts, cfg.d_model, cfg.d_ff), dtype=dt)
        for e, a, c in iter_experts(cfg, workers=workers):
            w13[e] = a
            w2[e] = c
    shared = [make_shared_expert(cfg, i) for i in range(cfg.num_shared)]
    ws13, ws2 = pack_shared(cfg, shared)
    return HostInputs(cfg, x, wr, b, w13, w2, shared, ws13, ws2)
