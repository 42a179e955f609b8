"""Benchmark of the TQP routed-expert layer on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
route -> permute -> expert FFNs -> combine -> adapter-only backward, at
T=8192 tokens, d=2048, E=460 experts, top-12, d_ff=768, int4 group-128 base,
rank-16 adapters, bf16 activations (the 8K-context, 460-expert, top-12
setting of "Reversible Foundations: Training a 120B Sparse MoE through
State-Preserving Scaling", abstract; hidden sizes are this library's).

Prints one JSON line.  `value` is tokens/s of the timed steps with every input
already resident in device memory.  `roofline` reports the gate/up expert GEMM
(the dominant kernel; one launch per tile class, timed together) against the
bf16 matrix-core peak, timed with HIP events on its own launch stream; `cpu_baseline` times the fp64 oracle on a bounded
sample of the same workload on this host's cores.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-extras]
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
sys.path.insert(0, ROOT)

from sparse_moe_expert_fp32_amd import configs, inputs  # noqa: E402

PEAK_BF16 = 2.5e15      # dense bf16 matrix-core FLOP/s of MI355X
PEAK_HBM = 8.0e12       # HBM3E bytes/s
METRIC = "TQP MoE-layer tokens/s, E=460 top-12, T=8192; % of MFMA/HBM roofline"
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gateup_flops(cfg) -> float:
    """Algorithmic FLOPs of the gate/up stage per step: for every routed slot,
    the int4-base product of both matrices (2*d*2f) and the adapter product
    (X A) B's second factor (2*r*2f); X A itself runs in its own kernel."""
    S = cfg.T * cfg.k
    return 2.0 * S * 2 * cfg.f * (cfg.d + cfg.r)


def layer_flops(cfg, train: bool) -> float:
    S = cfg.T * cfg.k
    fwd = S * (6.0 * cfg.d * cfg.f + 6.0 * cfg.r * (cfg.d + cfg.f))
    if not train:
        return fwd
    return fwd + S * (6.0 * cfg.d * cfg.f + 12.0 * cfg.r * (cfg.d + cfg.f))


def kernel_sources_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_moe_expert_fp32_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; None otherwise."""
    path = os.path.join(PROFILES, f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("sources_hash") != kernel_sources_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(cfg, inp, target_s: float):
    """The fp64 oracle (as it stands) on the first Ts tokens of the workload:
    whole-layer forward and, for a training step, the adapter backward."""
    import oracle
    from threadpoolctl import threadpool_limits
    cores = len(os.sched_getaffinity(0))
    lam = cfg.lora_scale

    def run(Ts):
        sub = dict(inp)
        sub["x"], sub["dy"] = inp["x"][:Ts], inp["dy"][:Ts]
        t0 = time.perf_counter()
        fwd = oracle.forward(sub, cfg.k, cfg.group, lam, keep=cfg.train)
        if cfg.train:
            oracle.backward(sub, fwd, cfg.k, cfg.group, lam)
        return time.perf_counter() - t0

    with threadpool_limits(cores):
        Ts = 8
        dt = run(Ts)
        # grow the sample until it takes a few seconds, stay inside the budget
        while dt < target_s / 4 and Ts < cfg.T:
            Ts = min(cfg.T, Ts * 4)
            dt = run(Ts)
    return {"value": Ts / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {Ts} of {cfg.T} tokens, fp64 whole-layer forward"
                      f"{' + adapter backward' if cfg.train else ''} in {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=configs.C5.name, choices=sorted(configs.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the reversible-replay and growth measurements (kernel "
                         "profiles of the layer step alone)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (a kernel of "
                         "known traffic that calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer is "
              "built and measured on a single MI355X and has no multi-GPU path.", flush=True)
        sys.exit(2)

    import torch
    from sparse_moe_expert_fp32_amd import binding as B
    from sparse_moe_expert_fp32_amd.layer import DeviceLayer, grow_inputs, to_numpy

    cfg = configs.CONFIGS[args.workload]
    t0 = time.perf_counter()
    inp = inputs.generate(cfg, args.seed)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    L = DeviceLayer(cfg, inp, device="cuda:0")
    step = L.train_step if cfg.train else L.forward
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")

    # timed region: K steps between two events; the gate/up GEMM's launches
    # are bracketed by their own events on the same stream
    B.moe_timer_start("gateup")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    k_ms, k_launches = B.moe_timer_stop()
    ms = total_ms / args.steps
    tokens_per_s = cfg.T / (ms / 1e3)
    log(f"{ms:.3f} ms/step, {tokens_per_s:.4g} tokens/s; gate/up {k_ms / max(1, k_launches):.3f} "
        f"ms x {k_launches / args.steps:.0f}/step")

    # forward-only rate of the same inputs (context)
    ev0.record(stream)
    for _ in range(args.steps):
        L.forward()
    ev1.record(stream)
    torch.cuda.synchronize()
    fwd_ms = ev0.elapsed_time(ev1) / args.steps

    # adapter optimizer step (AdamW over the six adapters through
    # moe_adamw_step), timed on its own after the layer steps
    adamw = None
    if cfg.train:
        L.init_optimizer()
        for _ in range(2):
            L.optimizer_step()
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            L.optimizer_step()
        ev1.record(stream)
        torch.cuda.synchronize()
        opt_ms = ev0.elapsed_time(ev1) / args.steps
        n_par = sum(t[0].numel() for t in L.opt.values())
        nbytes = n_par * (16 + 12 + 2)   # read p, g, m, v; write p, m, v and the bf16 copy
        adamw = {"ms": opt_ms, "params": n_par, "bytes": nbytes,
                 "GB_s": nbytes / (opt_ms / 1e3) / 1e9, "frac_hbm": nbytes / (opt_ms / 1e3) / PEAK_HBM}
        log(f"adamw {opt_ms:.3f} ms for {n_par} adapter parameters")

    # reversible residual block around the layer: the backward's replay
    # x2 = y2 - MoE(y1), i.e. the layer forward recomputed from y1 and the
    # coupling (moe_rev_couple), timed on its own; the reconstruction error
    # is against the x2 the forward coupling started from
    reversible = growth = None
    if not args.no_extras:
        act = torch.bfloat16 if cfg.act == "bf16" else torch.float32
        gen = torch.Generator().manual_seed(7)
        x2 = torch.randn(cfg.T, cfg.d, generator=gen).to(L.dev).to(act)
        y2, back = torch.empty_like(x2), torch.empty_like(x2)
        L.rev_forward(x2, y2)
        L.rev_inverse(y2, back)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            L.rev_inverse(y2, back)
        ev1.record(stream)
        torch.cuda.synchronize()
        rev_ms = ev0.elapsed_time(ev1) / args.steps
        rerr = (back.float() - x2.float()).abs()
        reversible = {"replay_ms": rev_ms, "x2_max_abs_err": float(rerr.max()),
                      "x2_exact_fraction": float((rerr == 0).float().mean())}
        log(f"reversible replay {rev_ms:.3f} ms, x2 max abs error {float(rerr.max()):.3e}")

        # few -> many growth (moe_grow_copy, moe_grow_router): the transform of
        # this layer to twice the experts, timed, and the grown layer's forward
        # (twice k, unperturbed router) against the original output
        ev0.record(stream)
        cfg2, g2 = grow_inputs(L.t, cfg, 2)
        ev1.record(stream)
        torch.cuda.synchronize()
        grow_ms = ev0.elapsed_time(ev1)
        y_orig = L.y.float().clone()
        L2 = DeviceLayer(cfg2, g2, device=L.dev, with_backward=False)
        L2.forward()
        torch.cuda.synchronize()
        growth = {"factor": 2, "experts": cfg2.E, "top_k": cfg2.k, "transform_ms": grow_ms,
                  "forward_rel_l2_vs_original": float((L2.y.float() - y_orig).norm() / y_orig.norm())}
        log(f"growth x2: {grow_ms:.3f} ms, grown forward rel L2 vs original "
            f"{growth['forward_rel_l2_vs_original']:.2e}")
        del L2, g2

    per_launch_ms = k_ms / max(1, k_launches)
    launches_per_step = k_launches / args.steps
    flops_launch = gateup_flops(cfg) / launches_per_step
    achieved = flops_launch / (per_launch_ms / 1e3)
    traffic = measured_traffic("gateup")
    counts = to_numpy(L.counts)
    rec = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.act == "bf16" else "f32",
        "data": "synthetic (seeded; int4 base quantised from N(0,1/fan_in) weights)",
        "config": {"workload": cfg.name + (" (forward + adapter-only backward)" if cfg.train
                                           else " (forward)"),
                   "T": cfg.T, "d_model": cfg.d, "experts": cfg.E, "top_k": cfg.k,
                   "d_ff": cfg.f, "rank": cfg.r, "group": cfg.group, "act": cfg.act,
                   "router_bias_var": cfg.router_bias_var},
        "roofline": {"bound": "mfma", "achieved": achieved / 1e12, "peak": PEAK_BF16 / 1e12,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16,
                     "traffic": traffic,
                     "kernel": "gate/up expert GEMM (one launch per tile class: 128/96/64/32 rows)",
                     "kernel_ms": per_launch_ms, "launches_per_step": launches_per_step,
                     "flops_per_launch": flops_launch},
        "layer_tflops": layer_flops(cfg, cfg.train) / (ms / 1e3) / 1e12,
        "layer_frac_of_bf16_peak": layer_flops(cfg, cfg.train) / (ms / 1e3) / PEAK_BF16,
        "forward_ms": fwd_ms,
        # the frozen int4 base is re-laid out once at setup (moe_pack_base_f
        # for the forward, moe_pack_base_t for the backward), like its
        # quantisation; the timed steps run every per-step kernel
        "base_packed_for_forward": bool(getattr(L, "packed_f", None)),
        "base_packed_for_backward": bool(getattr(L, "packed", None)),
        "adamw": adamw,
        "reversible": reversible,
        "growth": growth,
        "forward_tokens_per_s": cfg.T / (fwd_ms / 1e3),
        "load": {"max": int(counts.max()), "mean": float(counts.mean()),
                 "empty_experts": int((counts == 0).sum())},
    }
    if args.copy_probe_mb:
        n = args.copy_probe_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_probe_bytes"] = n
        del src, dst
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        rec["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
        log(f"cpu baseline took {time.perf_counter() - t0:.1f} s")
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
