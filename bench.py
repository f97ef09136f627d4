"""Benchmark of the sparse-MoE layer forward on one MI355X.

One step = one moe_layer_forward over a batch of seeded synthetic tokens that
is already resident in HBM: router logits, scoring / top-k, permute, grouped
expert FFN (routed and shared), combine and the load statistics.

Prints ONE JSON line: MoE-layer tokens/s, the roofline of the dominant stage
(timed live with HIP events on the library's stream over the timed steps), the
per-stage breakdown of an untimed pass with every stage bracketed by events
(and of a second one with the MALL and L2 evicted before each pass), the
median / p10 / p90 of single steps' HIP-event times (an untimed run of the
same length), and the CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

# MI355X published peaks
HBM_GBPS = 8000.0
MFMA_BF16_TFLOPS = 2500.0
VALU_F32_TFLOPS = 157.3      # published float32 vector peak (packed FP32; the kernels use half of it, unpacked)

# Files whose change invalidates HBM-traffic counters taken earlier: the GEMM
# kernels, their launch planning and the synthetic workload recipe.
TRAFFIC_SOURCES = ("top_routing_dispatch_amd/csrc/common.h", "top_routing_dispatch_amd/csrc/gemm.hip",
                   "top_routing_dispatch_amd/csrc/gemm_v3.hip",
                   "top_routing_dispatch_amd/csrc/gemm_ws.hip", "top_routing_dispatch_amd/csrc/api.hip",
                   "workloads/__init__.py")

AUX_STAGES = ("shared_gate_up", "shared_down", "load_stats")   # on the library's auxiliary stream
DEFAULT_CPU_SAMPLE = {"tiny": 64, "switch": 8192, "mixtral": 1024, "deepseekmoe": 4096, "deepseekv3": 256}
CPU_MIN_SECONDS = 10.0       # the oracle's sample is repeated until this much time has passed


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def router_planes(cfg):
    """bf16 planes the router GEMM runs over: a float32 router weight with bf16
    tokens is split exactly into three bf16 planes (hi + mid + lo), each
    multiplied on the matrix cores."""
    return 3 if (cfg.router_dtype == W.F32 and cfg.act_dtype == W.BF16) else 1


def stage_work(cfg, stage, A, E_act, T):
    """Algorithmic (flops, bytes) of one launch of a stage; A = kept rows.
    The grouped GEMMs count the expert weights once, the rows they read and
    the rows they write back to token order (x in, y_perm out); the
    activation H between the two projections is an intermediate of the
    implementation, not of the method, and is left out (stage_h_bytes gives
    it)."""
    b = 2 if cfg.act_dtype == W.BF16 else 4
    br = 2 if cfg.router_dtype == W.BF16 else 4
    D, F, E, k = cfg.d_model, cfg.d_ff, cfg.num_experts, cfg.top_k
    nm = cfg.n_mat
    SF = cfg.num_shared * cfg.d_ff_shared
    if stage == "router_logits":
        return 2.0 * T * D * E * router_planes(cfg), T * D * b + E * D * br + T * E * 4
    if stage == "route_select":
        return 0.0, T * E * 4 * 2 + T * k * 8
    if stage == "permute":
        return 0.0, T * k * 4 * 3 + A * 4 + (E + 1) * 8
    if stage == "expert_gate_up":
        return 2.0 * A * D * F * nm, E_act * nm * F * D * b + A * D * b
    if stage == "expert_down":
        return 2.0 * A * F * D, E_act * D * F * b + A * D * b
    if stage == "expert_ffn":
        f1, b1 = stage_work(cfg, "expert_gate_up", A, E_act, T)
        f2, b2 = stage_work(cfg, "expert_down", A, E_act, T)
        return f1 + f2, b1 + b2
    if stage == "shared_gate_up":
        return 2.0 * T * D * 2 * SF, 2 * SF * D * b + T * D * b
    if stage == "shared_down":
        return 2.0 * T * SF * D, D * SF * b + T * D * b
    if stage == "combine":
        return 0.0, A * D * b + T * k * 8 + (T * D * b if SF else 0) + T * D * b
    if stage == "load_stats":
        return 0.0, T * E * 4 + E * 4
    if stage == "fused_layer":
        # x and the weights read once (routed experts with rows only), y and
        # the routing outputs written: what the one-workgroup layer must move
        parts = ("router_logits", "expert_ffn") + (("shared_gate_up", "shared_down") if SF else ())
        fl = sum(stage_work(cfg, p, A, E_act, T)[0] for p in parts)
        by = (T * D * b + E * D * br + E_act * (nm + 1) * F * D * b + 3 * SF * D * b + T * D * b
              + T * k * 8 + E * 4 + (2 * E + 2) * 4)
        return fl, by
    raise KeyError(stage)


def stage_h_bytes(cfg, stage, A, T):
    """Bytes of the activation H that a projection writes (gate/up) or reads
    (down) on top of stage_work's."""
    b = 2 if cfg.act_dtype == W.BF16 else 4
    SF = cfg.num_shared * cfg.d_ff_shared
    if stage in ("expert_gate_up", "expert_down"):
        return A * cfg.d_ff * b
    if stage == "expert_ffn":
        return 2 * A * cfg.d_ff * b
    if stage in ("shared_gate_up", "shared_down"):
        return T * SF * b
    return 0


def roofline_of(cfg, stage, flops, nbytes, ms):
    """The stage against its roof: the larger of its time at the compute peak
    (bf16 matrix cores; float32 vector units for the all-float32 layer) and
    its time at the HBM peak decides the bound."""
    t = ms * 1e-3
    gemm = flops > 0
    if gemm and cfg.act_dtype == W.F32:
        peak_f, unit_bound = VALU_F32_TFLOPS, "alu"
    else:
        peak_f, unit_bound = MFMA_BF16_TFLOPS, "mfma"
    if gemm and flops / max(nbytes, 1) > peak_f * 1e12 / (HBM_GBPS * 1e9):
        achieved = flops / t / 1e12
        return dict(bound=unit_bound, achieved=round(achieved, 2), peak=peak_f, unit="TFLOP/s",
                    frac=round(achieved / peak_f, 4))
    achieved = nbytes / t / 1e9
    return dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_GBPS, unit="GB/s",
                frac=round(achieved / HBM_GBPS, 4))


def targets_of(cfg, stage_ms, A, E_act, T):
    """The layer's stated targets at the measured stage times: router,
    selection, permutation and combine against the HBM peak, the routed
    expert GEMMs (gate/up + down) against the bf16 matrix-core peak."""
    out = {}
    for st in ("router_logits", "route_select", "permute", "combine"):
        if st in stage_ms:
            _, by = stage_work(cfg, st, A, E_act, T)
            out[st + "_hbm_frac"] = round(by / (stage_ms[st] * 1e-3) / 1e9 / HBM_GBPS, 4)
    if "expert_ffn" in stage_ms:
        fl = stage_work(cfg, "expert_ffn", A, E_act, T)[0]
        ms = stage_ms["expert_ffn"]
        out["expert_gemm_ms"] = round(ms, 4)
        out["expert_gemm_mfma_frac"] = round(fl / (ms * 1e-3) / 1e12 / MFMA_BF16_TFLOPS, 4)
    if "fused_layer" in stage_ms:
        out["fused_layer_us"] = round(stage_ms["fused_layer"] * 1e3, 2)
    return out


def sources_digest():
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_file(workload, stage):
    return os.path.join(ROOT, "profiles", f"{stage}_{workload}_hbm_traffic.md")


def measured_traffic(workload, stage):
    """HBM bytes per launch of `stage`'s kernel from the committed FETCH_SIZE /
    WRITE_SIZE summary, or None when there is none or the kernel sources have
    changed since the counters were taken."""
    path = traffic_file(workload, stage)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith(("#", "|", " ", "`")):
                key, val = ln.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("sources_digest") != sources_digest():
        log(f"[bench] {os.path.basename(path)} is stale (kernel sources changed): traffic = null")
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(mib, reps):
    """A plain streaming copy of known size (torch.neg on float32, out of place)
    for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "kernel": "torch.neg float32", "bytes_read": 4 * n,
                      "bytes_written": 4 * n, "launches": reps}), flush=True)


def copy_rate(mib=1024, reps=5):
    """Live rate of a plain streaming copy (torch.neg on float32, 1 GiB in and
    1 GiB out, HIP events on torch's stream): what this GPU's HBM delivers to
    a simple kernel, reported beside the published peak."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.neg(src, out=dst)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.neg(src, out=dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return dict(kernel="torch.neg float32, 1 GiB read + 1 GiB written", gbps=round(8 * n / (ms * 1e-3) / 1e9, 1))


def gpu_clocks():
    """The GPU's current clocks as rocm-smi reports them (card 0), or None when
    the tool is missing or fails: context for the roofline fractions, which
    use the published peaks."""
    import subprocess
    try:
        out = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=15)
        data = json.loads(out.stdout)
        card = data.get("card0") or next(iter(data.values()))
        return {k.strip(" :"): v for k, v in card.items() if "clock" in k.lower() or "clk" in k.lower()}
    except Exception:
        return None


def host_info():
    """Threads the oracle's BLAS uses, the BLAS library and the host CPU model
    (for the CPU baseline's record)."""
    cores, blas = 1, None
    try:
        import threadpoolctl
        info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if info:
            cores = max(i.get("num_threads", 1) for i in info)
            blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer')} threads)"
                             for i in info)
    except Exception:
        pass
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.lower().startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return dict(cores=int(cores), cpu_model=model, blas=blas, host_cpus=os.cpu_count())


def cpu_baseline(cfg, inp, sample_tokens, expert_choice=False):
    """The oracle as it stands, on the first `sample_tokens` tokens (expert
    choice: those tokens as a batch of their own, C recomputed for it)."""
    from oracle import moe_oracle as O
    hi = host_info()
    Ts = min(sample_tokens, cfg.num_tokens)
    scfg = cfg.replace(num_tokens=Ts)
    x = inp.x[:Ts]
    passes = 0
    t0 = time.perf_counter()
    while True:
        if expert_choice:
            O.expert_choice_forward(scfg, x, inp.w_router, lambda e: (inp.w13[e], inp.w2[e]), inp.shared)
        else:
            O.forward(scfg, x, inp.w_router, inp.sel_bias, lambda e: (inp.w13[e], inp.w2[e]), inp.shared)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= CPU_MIN_SECONDS:
            break
    return dict(value=round(Ts * passes / dt, 2), unit="tokens/s", cores=hi["cores"], kind="oracle",
                sample=f"first {Ts} of {cfg.num_tokens} tokens, all {cfg.num_experts} experts"
                       + (", capacity recomputed for the sample" if cfg.capacity_factor > 0 or expert_choice else "")
                       + f"; {passes} pass(es) in {dt:.1f} s",
                cpu_model=hi["cpu_model"], blas=hi["blas"], host_cpus=hi["host_cpus"])


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="deepseekv3",
                    choices=sorted(W.CONFIGS) + sorted(W.DECODE_CONFIGS) + sorted(W.EP_CONFIGS) + sorted(W.EC_CONFIGS),
                    help="workload; <model>_decode_t<T>: the first T tokens on that model's full-size weights; "
                         "<model>_ep8_local: one GPU's share of an 8-rank expert-parallel layer; "
                         "<model>_ec: the model's layer with expert-choice routing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time moe_layer_backward (forward recomputed inside) instead of the forward")
    ap.add_argument("--cpu-sample-tokens", type=int, default=None)
    ap.add_argument("--copy-calibration", type=int, default=None, metavar="MIB",
                    help="only run a plain copy of MIB MiB --steps times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return

    if args.config in W.EP_CONFIGS:
        run_ep_share(args, W.EP_CONFIGS[args.config])
        return
    if args.backward:
        run_backward(args, W.CONFIGS.get(args.config) or W.DECODE_CONFIGS[args.config])
        return

    import torch
    import top_routing_dispatch_amd as M
    from workloads.torch_io import act_torch_dtype, to_torch, upload_experts

    cfg = W.CONFIGS.get(args.config) or W.DECODE_CONFIGS.get(args.config) or W.EC_CONFIGS[args.config]
    ec = args.config in W.EC_CONFIGS
    dev = "cuda"
    torch.cuda.set_device(0)
    t_setup = time.perf_counter()
    inp = W.make_inputs(cfg, with_experts=False)
    x = to_torch(inp.x, dev)
    w13, w2, host = upload_experts(cfg, dev, keep_host=not args.no_cpu_baseline,
                                   progress=lambda n: log(f"[bench] generated {n}/{cfg.num_experts} experts"))
    if host is not None:
        inp.w13 = _Stack(host, 0)
        inp.w2 = _Stack(host, 1)
    weights = dict(w_router=to_torch(inp.w_router, dev), sel_bias=to_torch(inp.sel_bias, dev), w13=w13, w2=w2,
                   ws13=to_torch(inp.ws13, dev), ws2=to_torch(inp.ws2, dev))
    T, E, k = cfg.num_tokens, cfg.num_experts, cfg.top_k
    y = torch.empty((T, cfg.d_model), dtype=act_torch_dtype(cfg), device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    stats = torch.empty(2 * E + 2, dtype=torch.float32, device=dev)
    dropped = torch.empty(1, dtype=torch.int32, device=dev)
    ws = M.workspace(cfg, M.MOE_OP_EXPERT_CHOICE if ec else M.MOE_OP_LAYER, dev)
    if ec:
        C_ec = M.moe_expert_choice_capacity(cfg)
        tor_ec = torch.empty(E * C_ec, dtype=torch.int32, device=dev)
        rw_ec = torch.empty(E * C_ec, dtype=torch.float32, device=dev)
        uns_ec = torch.empty(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] {cfg.name}: setup {time.perf_counter() - t_setup:.1f} s, workspace {ws.numel() / 1e6:.1f} MB")

    nst = len(M.STAGES)

    UP, DOWN = M.STAGES.index("expert_gate_up"), M.STAGES.index("expert_down")

    def event_slots(stage):
        """Event slots (2 s = start, 2 s + 1 = stop) that time a stage; the
        routed expert FFN spans the gate/up start to the down stop (with the
        shallow expert groups on a second stream beside the deep ones, the
        split between the two projections is not a kernel boundary)."""
        if stage == "expert_ffn":
            return [2 * UP, 2 * DOWN + 1]
        si = M.STAGES.index(stage)
        return [2 * si, 2 * si + 1]

    def new_events(slots=None):
        """Events for the given event slots (all by default), None elsewhere."""
        evs = [None] * (2 * nst)
        for i in (range(2 * nst) if slots is None else slots):
            e = torch.cuda.Event(enable_timing=True)
            e.record()      # creates the HIP event handle
            evs[i] = e
        return evs

    def step(evs=None):
        if ec:
            M.moe_expert_choice_forward(cfg, weights, x, y, tor_ec, rw_ec, uns_ec, ws, stage_events=evs)
            return
        M.moe_layer_forward_timed(cfg, weights, x, y, idx, tw, counts, cfg.alpha, stats, dropped, ws,
                                  stage_events=evs)

    # stages that run (the others' events only hold their creation-time records)
    ran = set(M.STAGES) - {"permute", "load_stats", "fused_layer"} if ec else set(M.moe_layer_stages(cfg))
    if ec and cfg.num_shared == 0:
        ran -= {"shared_gate_up", "shared_down"}
    log(f"[bench] stages: {' '.join(s for s in M.STAGES if s in ran)}")

    def stage_times(events, stages):
        out = {}
        for si in stages:
            name = M.STAGES[si]
            if name not in ran:
                continue
            vals = [evs[2 * si].elapsed_time(evs[2 * si + 1]) for evs in events]
            if vals and max(vals) > 0:
                out[name] = float(np.mean(vals))
        if not ec and UP in stages and DOWN in stages and "expert_gate_up" in out and "expert_down" in out:
            a, b = event_slots("expert_ffn")
            out["expert_ffn"] = float(np.mean([evs[a].elapsed_time(evs[b]) for evs in events]))
        return out

    def span_ms(events, stage):
        a, b = event_slots(stage)
        return float(np.mean([evs[a].elapsed_time(evs[b]) for evs in events]))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Untimed breakdown pass: every stage bracketed by events, to find the
    # slowest stage.  The timed steps below record only that stage's two
    # events, so the per-step time carries no extra event packets.
    n_prof = max(1, min(args.steps, 10))
    prof_events = [new_events() for _ in range(n_prof)]
    torch.cuda.synchronize()
    for i in range(n_prof):
        step(prof_events[i])
    torch.cuda.synchronize()
    stage_ms = stage_times(prof_events, range(nst))
    # the dominant stage is the slowest one on the caller's stream: the
    # stages on the library's auxiliary stream (shared experts, load
    # statistics) run beside the routed path and their event spans include
    # the time they wait for the chip
    main_ms = {k: v for k, v in stage_ms.items() if k not in AUX_STAGES}
    if "expert_ffn" in main_ms:
        # the routed expert FFN is timed as one grouped-GEMM stage
        main_ms.pop("expert_gate_up")
        main_ms.pop("expert_down")
    dominant = max(main_ms or stage_ms, key=(main_ms or stage_ms).get)
    # The same stages with the caches cold: a 512 MB scratch read before each
    # pass evicts the 256 MB MALL and the L2s, so no stage reads what the
    # previous pass left there (a read, so that no dirty lines are left whose
    # write-back would fall on the first stage).
    n_cold = 5
    cold_events = [new_events() for _ in range(n_cold)]
    scratch = torch.ones(64 << 20, dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    for i in range(n_cold):
        scratch.sum()
        step(cold_events[i])
    torch.cuda.synchronize()
    stage_cold_ms = stage_times(cold_events, range(nst))
    del scratch
    events = [new_events(event_slots(dominant)) for _ in range(args.steps)]
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step")
    # the dominant stage's time over the timed steps (HIP events on the library's stream)
    dom_ms = span_ms(events, dominant)
    # the spread of single steps, from HIP events around each step of an
    # untimed run of the same length (kept out of the timed region above)
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for i in range(args.steps):
        step_ev[i][0].record()
        step()
        step_ev[i][1].record()
    torch.cuda.synchronize()
    per_step = np.array([a.elapsed_time(b) for a, b in step_ev])

    if ec:
        kept = np.full(E, C_ec)                         # every expert takes exactly C tokens
    else:
        c_host = counts.cpu().numpy()
        cap, rows_cap = M.moe_capacity(cfg)
        kept = np.minimum(c_host, cap)
    A = int(kept.sum())
    E_act = int((kept > 0).sum())
    stage_info = {}
    for name, ms in stage_ms.items():
        fl, by = stage_work(cfg, name, A, E_act, T)
        stage_info[name] = dict(ms=round(ms, 4), **roofline_of(cfg, name, fl, by, ms))
    fl, by = stage_work(cfg, dominant, A, E_act, T)
    roof = roofline_of(cfg, dominant, fl, by, dom_ms)
    roof["kernel"] = dominant
    roof["ms"] = round(dom_ms, 4)
    hb = stage_h_bytes(cfg, dominant, A, T)
    if hb:
        # the same stage with the activation H between the projections counted as traffic
        roof["with_h"] = dict(bytes=int(by + hb), gbps=round((by + hb) / (dom_ms * 1e-3) / 1e9, 1),
                              hbm_frac=round((by + hb) / (dom_ms * 1e-3) / 1e9 / HBM_GBPS, 4))
    if fl > 0:
        roof["mfma_frac" if cfg.act_dtype == W.BF16 else "alu_frac"] = round(
            fl / (dom_ms * 1e-3) / 1e12 / (MFMA_BF16_TFLOPS if cfg.act_dtype == W.BF16 else VALU_F32_TFLOPS), 4)
        roof["hbm_frac"] = round(by / (dom_ms * 1e-3) / 1e9 / HBM_GBPS, 4)
    roof["traffic"] = measured_traffic(cfg.name, dominant)
    if roof["bound"] == "hbm":
        ref = copy_rate()
        ref["achieved_over_copy"] = round(roof["achieved"] / ref["gbps"], 4)
        roof["copy_ref"] = ref
    roof["clocks"] = gpu_clocks()

    cpu = None
    if not args.no_cpu_baseline:
        n = args.cpu_sample_tokens or DEFAULT_CPU_SAMPLE.get(cfg.name, 64)
        log(f"[bench] timing the CPU oracle on {n} tokens")
        cpu = cpu_baseline(cfg, inp, n, expert_choice=ec)

    value = T / (ms_per_step * 1e-3)
    line = {
        "metric": "MoE-layer tokens/sec at 1 GPU; % HBM roofline (route/permute) and % MFMA peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.act_dtype == W.BF16 else "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": T, "d_model": cfg.d_model, "experts": E, "top_k": k,
                   "d_ff": cfg.d_ff, "shared": cfg.num_shared, "d_ff_shared": cfg.d_ff_shared,
                   "scoring": ["softmax_topk", "topk_softmax", "sigmoid_bias"][cfg.scoring],
                   "activation": ["swiglu", "gelu"][cfg.activation], "capacity_factor": cfg.capacity_factor,
                   "kept_rows": A, "active_experts": E_act, "max_expert_rows": int(kept.max()),
                   "routing": "expert_choice" if ec else "token_choice"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "step_ms": {q: round(float(np.percentile(per_step, p)), 4)
                    for q, p in (("median", 50), ("p10", 10), ("p90", 90))},
        "targets": targets_of(cfg, stage_ms, A, E_act, T),
        "stages": stage_info,
        "stages_cold_ms": {name: round(ms, 4) for name, ms in stage_cold_ms.items()},
    }
    print(json.dumps(line), flush=True)


def run_ep_share(args, ep):
    """One GPU's share of an expert-parallel layer: a step is the receive
    layout of the rows the dispatch all-to-all delivered plus the local grouped
    expert FFN reading them in place (the exchanges are not part of one GPU).
    Throughput is received rows per second."""
    import torch
    import top_routing_dispatch_amd as M
    from workloads.torch_io import to_torch

    cfg = W.CONFIGS[ep.base]
    El, D, F = ep.local_experts, cfg.d_model, cfg.d_ff
    dev = "cuda"
    torch.cuda.set_device(0)
    rc_host = W.ep_recv_counts(ep)
    total = int(rc_host.sum())
    xr_host = W.make_received_rows(ep, total)
    xr = to_torch(xr_host, dev)
    rc = to_torch(rc_host, dev)
    first = ep.rank * El
    w13 = torch.empty((El, cfg.n_mat * F, D), dtype=torch.bfloat16, device=dev)
    w2 = torch.empty((El, D, F), dtype=torch.bfloat16, device=dev)
    host = {}
    for e, a, b in W.iter_experts(cfg, experts=range(first, first + El), workers=16):
        w13[e - first].copy_(to_torch(a, "cpu"))
        w2[e - first].copy_(to_torch(b, "cpu"))
        host[e - first] = (a, b)
    lcfg = cfg.replace(num_experts=El, num_tokens=total, top_k=1, num_shared=0, d_ff_shared=0)
    lo = torch.empty(El + 1, dtype=torch.int32, device=dev)
    g = torch.empty(total, dtype=torch.int32, device=dev)
    y = torch.empty((total, D), dtype=torch.bfloat16, device=dev)
    ws = M.workspace(lcfg, M.MOE_OP_EXPERT_FFN, dev)

    def step():
        M.moe_ep_recv_layout(rc, total, lo, g)
        M.moe_expert_ffn(lcfg, El, F, cfg.activation, total, xr, g, lo, w13, w2, y, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    ev_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    flops = 2.0 * total * D * F * (cfg.n_mat + 1)
    roof = dict(bound="mfma", achieved=round(flops / (ev_ms * 1e-3) / 1e12, 2), peak=MFMA_BF16_TFLOPS,
                unit="TFLOP/s", frac=round(flops / (ev_ms * 1e-3) / 1e12 / MFMA_BF16_TFLOPS, 4),
                kernel="local expert FFN (gate/up + down)", ms=round(ev_ms, 4), traffic=None)
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import moe_oracle as O
        lay = O.ep_recv_layout(rc_host)
        n = args.cpu_sample_tokens or 128
        rows = lay["gather"][:n]                       # the first rows of local expert 0
        passes, t1 = 0, time.perf_counter()
        while True:
            O.expert_apply(O.widen(xr_host[rows]), host[0][0], host[0][1], cfg.activation, F)
            passes += 1
            if time.perf_counter() - t1 >= CPU_MIN_SECONDS:
                break
        dt = time.perf_counter() - t1
        hi = host_info()
        cpu = dict(value=round(n * passes / dt, 2), unit="rows/s", cores=hi["cores"], kind="oracle",
                   sample=f"{n} received rows of local expert 0; {passes} pass(es) in {dt:.1f} s",
                   cpu_model=hi["cpu_model"], blas=hi["blas"], host_cpus=hi["host_cpus"])
    line = {
        "metric": "MoE-layer tokens/sec at 1 GPU; % HBM roofline (route/permute) and % MFMA peak",
        "value": round(total / (ms_per_step * 1e-3), 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": ep.name, "base": ep.base, "ranks": ep.ranks, "rank": ep.rank, "local_experts": El,
                   "received_rows": total, "d_model": D, "d_ff": F},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def run_backward(args, cfg):
    """One step = moe_layer_backward over the batch: the forward recomputed in
    its workspace, then the gradients of x, the router and every expert weight."""
    import torch
    import top_routing_dispatch_amd as M
    from workloads.torch_io import to_torch, upload_experts

    dev = "cuda"
    torch.cuda.set_device(0)
    inp = W.make_inputs(cfg, with_experts=False)
    x = to_torch(inp.x, dev)
    w13, w2, _ = upload_experts(cfg, dev)
    weights = dict(w_router=to_torch(inp.w_router, dev), sel_bias=to_torch(inp.sel_bias, dev), w13=w13, w2=w2,
                   ws13=to_torch(inp.ws13, dev), ws2=to_torch(inp.ws2, dev))
    T, E, D, F, k = cfg.num_tokens, cfg.num_experts, cfg.d_model, cfg.d_ff, cfg.top_k
    nF, SF = cfg.n_mat * F, cfg.num_shared * cfg.d_ff_shared
    g = torch.Generator(device="cpu").manual_seed(1)
    dy = torch.randn((T, D), generator=g).to(torch.bfloat16).to(dev)
    dx = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    dwr = torch.empty((E, D), dtype=torch.float32, device=dev)
    dw13 = torch.empty((E, nF, D), dtype=torch.float32, device=dev)
    dw2 = torch.empty((E, D, F), dtype=torch.float32, device=dev)
    dws13 = torch.empty((2 * SF, D), dtype=torch.float32, device=dev) if SF else None
    dws2 = torch.empty((D, SF), dtype=torch.float32, device=dev) if SF else None
    ws = M.workspace(cfg, M.MOE_OP_LAYER_BACKWARD, dev)

    def step():
        M.moe_layer_backward(cfg, weights, x, dy, cfg.alpha, dx, dwr, dw13, dw2, dws13, dws2, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a_ev.record()
    for _ in range(args.steps):
        step()
    b_ev.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    A = T * k if cfg.capacity_factor <= 0 else M.moe_capacity(cfg)[1]
    # expert GEMM work of the call (forward recomputation included): forward
    # (n_mat + 1) products, gate/up recomputed (n_mat), dH (1), dX (n_mat),
    # dW2 (1), dW13 (n_mat); shared experts the same over T rows
    flops = 2.0 * A * D * F * (4 * cfg.n_mat + 3) + 2.0 * T * D * SF * (4 * 2 + 3)
    ev_ms = a_ev.elapsed_time(b_ev) / args.steps
    roof = dict(bound="mfma", achieved=round(flops / (ev_ms * 1e-3) / 1e12, 2), peak=MFMA_BF16_TFLOPS,
                unit="TFLOP/s", frac=round(flops / (ev_ms * 1e-3) / 1e12 / MFMA_BF16_TFLOPS, 4),
                kernel="layer backward (expert GEMM work, forward recomputation included)", ms=round(ev_ms, 4),
                traffic=None)
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import moe_oracle as O
        Ts = min(args.cpu_sample_tokens or 64, T)
        scfg = cfg.replace(num_tokens=Ts)
        dy_h = dy[:Ts].float().cpu().numpy()
        expert = lambda e: W.make_expert(cfg, e)
        passes, t1 = 0, time.perf_counter()
        while True:
            O.backward(scfg, inp.x[:Ts], inp.w_router, inp.sel_bias, expert, inp.shared, dy_h, alpha=cfg.alpha)
            passes += 1
            if time.perf_counter() - t1 >= CPU_MIN_SECONDS:
                break
        dt = time.perf_counter() - t1
        hi = host_info()
        cpu = dict(value=round(Ts * passes / dt, 2), unit="tokens/s", cores=hi["cores"], kind="oracle",
                   sample=f"backward of the first {Ts} of {T} tokens (forward recomputed, experts regenerated); "
                          f"{passes} pass(es) in {dt:.1f} s",
                   cpu_model=hi["cpu_model"], blas=hi["blas"], host_cpus=hi["host_cpus"])
    line = {
        "metric": "MoE-layer tokens/sec at 1 GPU; % HBM roofline (route/permute) and % MFMA peak",
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name + "_backward", "tokens": T, "d_model": D, "experts": E, "top_k": k,
                   "d_ff": F, "shared": cfg.num_shared, "d_ff_shared": cfg.d_ff_shared,
                   "expert_gemm_flops_per_step": flops},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


class _Stack:
    """Indexable view of per-expert host weights kept by upload_experts."""

    def __init__(self, host, i):
        self.host, self.i = host, i

    def __getitem__(self, e):
        return self.host[e][self.i]


if __name__ == "__main__":
    main()
